// Seeded synthetic weights, generated on the device straight into the
// canonical layouts.  Each element is a pure function of (key, index), where
// key = mix(seed ^ (tid << 32)) and mix is the SplitMix64 output function
// (Steele, Lea & Flood, OOPSLA 2014), so any element can be drawn alone.
#include "common.h"

namespace dfssm {

static constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__host__ __device__ __forceinline__ uint64_t mix64(uint64_t x) {
  uint64_t z = x + kGamma;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

uint64_t host_mix64(uint64_t x) { return mix64(x); }

// 24-bit uniform in [0, 1), exact in fp32 and fp64
__device__ __forceinline__ double u24(uint64_t d) { return (double)(d >> 40) * 0x1p-24; }

__global__ void gen_kernel(void* dst, size_t n, int mode, uint64_t key, double a, double bma, float cval) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    switch (mode) {
      case GEN_WORDS:
        ((uint32_t*)dst)[i] = (uint32_t)(mix64(key + i) >> 32);
        break;
      case GEN_UNIFORM: {
        // fp64 multiply then fp64 add, each rounded (no fused multiply-add), then one rounding to fp32
        double v = __dadd_rn(a, __dmul_rn(bma, u24(mix64(key + i))));
        ((float*)dst)[i] = __double2float_rn(v);
        break;
      }
      case GEN_INT8:
        ((int8_t*)dst)[i] = (int8_t)((int)(mix64(key + i) % 255ull) - 127);
        break;
      case GEN_NORMAL: {
        double acc = 0.0;
        for (int k = 0; k < 12; ++k) acc = __dadd_rn(acc, u24(mix64(key + 12ull * i + (uint64_t)k)));
        ((float*)dst)[i] = __double2float_rn(__dadd_rn(acc, -6.0));
        break;
      }
      default:
        ((float*)dst)[i] = cval;
        break;
    }
  }
}

hipError_t launch_gen(void* dst, size_t n, int mode, uint64_t key, double a, double bma, float cval,
                      hipStream_t st) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(gen_kernel, dim3((unsigned)blocks), dim3(256), 0, st, dst, n, mode, key, a, bma, cval);
  return hipGetLastError();
}

}  // namespace dfssm
