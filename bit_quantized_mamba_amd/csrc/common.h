// Internal declarations shared by the library's translation units (not installed).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dfssm {

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float silu_f(float v) { return v / (1.0f + __expf(-v)); }

// softplus with the usual linear branch above 20 (log1p(e^a) - a < 2.1e-9 there)
__device__ __forceinline__ float softplus_f(float a) { return a > 20.0f ? a : log1pf(__expf(a)); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ---------------------------------------------------------------------------
// kernel argument bundles
// ---------------------------------------------------------------------------

// Prepared int8 activation rows: q, its 8 two's-complement bit planes
// ([row][d_in/32][8] words: word w plane b holds bit b of q[32w .. 32w+31]),
// the row sum of q, the scale s and the LoRA-down vector t = A q * sA * s.
struct QPrep {
  const int8_t* q;
  const uint32_t* planes;
  const int32_t* qsum;
  const float* s;
  const float* t;
};

enum ProjEpilogue : int {
  EPI_STORE = 0,   // y[b][o] (and acc[b][o] when non-null)
  EPI_IN_PROJ = 1, // z / dt_raw -> zx; x,B,C channels -> conv shift register -> xc
  EPI_OUT_PROJ = 2 // h[b][o] += y
};

struct ProjArgs {
  const uint32_t* bits;  // [d_out][d_in/32]
  const float* sw;       // [d_out]
  const int8_t* Bm;      // [d_out][r]
  const float* sB;       // [d_out]
  QPrep in;
  int d_in, d_out, r, B;
  // EPI_STORE
  int32_t* acc;
  float* y;
  // EPI_IN_PROJ
  float* zx;             // [B][d_out]
  float* xc;             // [B][conv_dim]
  float* conv_state;     // layer base; [b][K-1][conv_dim] with batch stride conv_bstride
  size_t conv_bstride;
  const float* conv_w;   // [conv_dim][K]
  const float* conv_b;   // [conv_dim]
  int d_inner, conv_dim, K;
  // EPI_OUT_PROJ
  float* h;              // [B][d_out]
};

// ---------------------------------------------------------------------------
// launchers (kernels.hip, gen.hip)
// ---------------------------------------------------------------------------

enum GenMode : int { GEN_WORDS = 0, GEN_UNIFORM = 1, GEN_INT8 = 2, GEN_NORMAL = 3, GEN_CONST = 4 };

uint64_t host_mix64(uint64_t x);
hipError_t launch_gen(void* dst, size_t n, int mode, uint64_t key, double a, double bma, float cval,
                      hipStream_t st);

hipError_t launch_embed(const int32_t* tok, int tok_stride, const int8_t* E, const float* sE, int dm, int V,
                        int B, float* h, int* err, hipStream_t st);

// RMSNorm (weight w) + per-row int8 quantisation + bit planes + row sum + LoRA-down.
// A may be null (r ignored, t untouched).
hipError_t launch_norm_quant(const float* x, const float* w, int n, int B, float eps, const int8_t* A,
                             const float* sA, int r, int8_t* q, uint32_t* planes, int32_t* qsum, float* s,
                             float* t, hipStream_t st);

// bit planes + row sum + LoRA-down of given int8 rows
hipError_t launch_qprep(const int8_t* q, const float* s, int n, int B, const int8_t* A, const float* sA, int r,
                        uint32_t* planes, int32_t* qsum, float* t, hipStream_t st);

hipError_t launch_proj(const ProjArgs& a, int epi, hipStream_t st);

hipError_t launch_ssm(const float* xc, const float* zx, int ld_zx, const float* A_log, const float* dt_bias,
                      const float* D, float* ssm_layer, size_t ssm_bstride, float* g, int B, int H, int P, int N,
                      int d_inner, int conv_dim, hipStream_t st);

hipError_t launch_lm_head(const int8_t* E, const float* sE, const int8_t* qf, const float* sf, int V, int dm,
                          int B, float* logits, hipStream_t st);

// argmax per row (lowest index on ties); writes next[b], and when out != null
// also out[(*counter) * B + b] and lets block 0 advance *counter.
hipError_t launch_argmax(const float* logits, int V, int B, int32_t* next, int32_t* out, int32_t* counter,
                         hipStream_t st);

hipError_t launch_quant_rows(const float* u, int rows, int n, int8_t* q, float* s, hipStream_t st);

hipError_t launch_zero(void* p, size_t bytes, hipStream_t st);

}  // namespace dfssm
