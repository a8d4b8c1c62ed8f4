// Density-field representation of the SSM state (gist.science technical
// summary §2.D: a binary field with K^2 about 4 d_state cells, built by
// normalisation, sigma-delta injection with error feedback and binarisation,
// read back by popcount, applied at chunk boundaries).
//
// One field per state row -- the d_state values of one head channel -- with 4
// cells per value: scale = max |x|, density d = (x / scale + 1) / 2, a
// first-order sigma-delta modulator walks the 4 n cells in order carrying its
// error across cells and values (a = d + e; cell = a >= 1/2; e = a - cell),
// and the readout of value i is scale * (popcount of its 4 cells - 2) / 2.
// Each step is one rounded fp32 operation in a fixed order, so the cells are
// a pure function of the row's fp32 values.  Cell c is bit c % 32 of word
// c / 32: a row of 128 values is 16 words and a scale, 7.5 times smaller than
// the fp32 row.
//
// The modulator is sequential along a row, so a thread owns a row.  In the
// engine's state layout ([H][P/16][N][16] per layer and sequence) the 16
// channels of a block are contiguous for each state index, so 16 threads
// reading value n of their rows read one 64-byte segment.
#include "common.h"

namespace dfssm {

// Encode one row held in registers: cells into w[0 .. N/8), returns the scale.
template <int N>
__device__ __forceinline__ float density_encode_row(const float (&v)[N], uint32_t (&w)[N / 8]) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < N; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
  for (int k = 0; k < N / 8; ++k) w[k] = 0u;
  if (!(amax > 0.0f)) return 0.0f;
  float e = 0.0f;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float d = (__fdiv_rn(v[i], amax) + 1.0f) * 0.5f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float a = d + e;
      const uint32_t bit = a >= 0.5f ? 1u : 0u;
      e = a - (float)bit;
      const int c = 4 * i + k;
      w[c >> 5] |= bit << (c & 31);
    }
  }
  return amax;
}

__device__ __forceinline__ float density_value(const uint32_t* w, int i, float scale) {
  const int p = __builtin_popcount((w[i >> 3] >> (4 * (i & 7))) & 0xFu);
  return scale * ((float)(p - 2) * 0.5f);
}

// ---------------------------------------------------------------------------
// stateless row-major form: x [rows][N] <-> field [rows][N / 8], scale [rows]
// ---------------------------------------------------------------------------
template <int N>
__global__ __launch_bounds__(256) void density_encode_rows_kernel(const float* __restrict__ x, int rows,
                                                                  uint32_t* __restrict__ field,
                                                                  float* __restrict__ scale) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= rows) return;
  float v[N];
  const float4* x4 = (const float4*)(x + (size_t)r * N);
#pragma unroll
  for (int q = 0; q < N / 4; ++q) {
    const float4 t = x4[q];
    v[4 * q] = t.x;
    v[4 * q + 1] = t.y;
    v[4 * q + 2] = t.z;
    v[4 * q + 3] = t.w;
  }
  uint32_t w[N / 8];
  const float sc = density_encode_row<N>(v, w);
  uint32_t* f = field + (size_t)r * (N / 8);
#pragma unroll
  for (int k = 0; k < N / 8; ++k) f[k] = w[k];
  scale[r] = sc;
}

// one thread per value
__global__ __launch_bounds__(256) void density_decode_rows_kernel(const uint32_t* __restrict__ field,
                                                                  const float* __restrict__ scale, int rows, int n,
                                                                  float* __restrict__ x) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)rows * n) return;
  const size_t r = idx / n;
  const int i = (int)(idx % n);
  x[idx] = density_value(field + r * (n / 8), i, scale[r]);
}

template <int N>
static hipError_t launch_encode_rows(const float* x, int rows, uint32_t* field, float* scale, hipStream_t st) {
  hipLaunchKernelGGL(density_encode_rows_kernel<N>, dim3((rows + 255) / 256), dim3(256), 0, st, x, rows, field,
                     scale);
  return hipGetLastError();
}

bool density_supported(int n) { return n == 16 || n == 32 || n == 64 || n == 128; }

hipError_t launch_density_encode_rows(const float* x, int rows, int n, uint32_t* field, float* scale,
                                      hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  switch (n) {
    case 16: return launch_encode_rows<16>(x, rows, field, scale, st);
    case 32: return launch_encode_rows<32>(x, rows, field, scale, st);
    case 64: return launch_encode_rows<64>(x, rows, field, scale, st);
    case 128: return launch_encode_rows<128>(x, rows, field, scale, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_density_decode_rows(const uint32_t* field, const float* scale, int rows, int n, float* x,
                                      hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  const size_t total = (size_t)rows * n;
  hipLaunchKernelGGL(density_decode_rows_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, field,
                     scale, rows, n, x);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// the engine's state: sequences [s0, s0 + ns) of layout [L][H][P/16][N][16],
// batch stride bstride floats.  Row r = ((s * L + l) * H + h) * P + p in
// canonical order; thread r owns it.
// MODE 0: pack (field, scale out); 1: unpack (field, scale in, state out);
// 2: round trip in place (state -> field -> state, no field stored).
// ---------------------------------------------------------------------------
template <int N, int MODE>
__global__ __launch_bounds__(256) void density_state_kernel(float* __restrict__ ssm, size_t bstride, int rows_per_seq,
                                                            int P, int total_rows, uint32_t* __restrict__ field,
                                                            float* __restrict__ scale) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= total_rows) return;
  const int s = r / rows_per_seq, rr = r % rows_per_seq;  // rr = (l * H + h) * P + p
  const int p = rr % P, lh = rr / P;
  float* base = ssm + (size_t)s * bstride + (size_t)lh * P * N + ((size_t)(p >> 4) * N) * 16 + (p & 15);
  if (MODE == 1) {
    uint32_t w[N / 8];
    const uint32_t* f = field + (size_t)r * (N / 8);
#pragma unroll
    for (int k = 0; k < N / 8; ++k) w[k] = f[k];
    const float sc = scale[r];
#pragma unroll
    for (int i = 0; i < N; ++i) base[(size_t)i * 16] = density_value(w, i, sc);
    return;
  }
  float v[N];
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = base[(size_t)i * 16];
  uint32_t w[N / 8];
  const float sc = density_encode_row<N>(v, w);
  if (MODE == 0) {
    uint32_t* f = field + (size_t)r * (N / 8);
#pragma unroll
    for (int k = 0; k < N / 8; ++k) f[k] = w[k];
    scale[r] = sc;
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) base[(size_t)i * 16] = density_value(w, i, sc);
  }
}

template <int N>
static hipError_t launch_state_n(const DensityStateArgs& a, int mode, hipStream_t st) {
  const dim3 grid((a.total_rows + 255) / 256);
  switch (mode) {
    case 0:
      hipLaunchKernelGGL((density_state_kernel<N, 0>), grid, dim3(256), 0, st, a.ssm, a.bstride, a.rows_per_seq,
                         a.P, a.total_rows, a.field, a.scale);
      break;
    case 1:
      hipLaunchKernelGGL((density_state_kernel<N, 1>), grid, dim3(256), 0, st, a.ssm, a.bstride, a.rows_per_seq,
                         a.P, a.total_rows, a.field, a.scale);
      break;
    default:
      hipLaunchKernelGGL((density_state_kernel<N, 2>), grid, dim3(256), 0, st, a.ssm, a.bstride, a.rows_per_seq,
                         a.P, a.total_rows, a.field, a.scale);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_density_state(const DensityStateArgs& a, int n, int mode, hipStream_t st) {
  if (a.total_rows <= 0) return hipSuccess;
  switch (n) {
    case 16: return launch_state_n<16>(a, mode, st);
    case 32: return launch_state_n<32>(a, mode, st);
    case 64: return launch_state_n<64>(a, mode, st);
    case 128: return launch_state_n<128>(a, mode, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dfssm
