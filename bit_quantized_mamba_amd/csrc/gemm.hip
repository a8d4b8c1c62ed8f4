// Kernels of the batched path: many token rows per layer (batched decode, one
// row per sequence; prefill, B x T rows), gfx950.
//
//  * rows_quant: RMSNorm + per-token int8 quantisation of a row (one wave per
//    row, or one workgroup per row from K = 2048), plus the row sum of the
//    codes and the LoRA down-projection t = float(A q) * sA * s.
//  * bitgemm: the 1-bit scaffold GEMM on the int8 matrix cores.  The 0/1
//    bytes of the scaffold bits (bit 1 -> 1) multiply the int8 codes on
//    v_mfma_i32_32x32x32_i8, giving pos[m][n] = sum of q over the +1 weights;
//    the signed product is 2 pos - sum(q).  The scaffold bits are expanded to
//    bytes in LDS once per k-tile (first form) or in registers per operand
//    (second form).  The LoRA up-projection is a rank-16 product on
//    v_mfma_f32_32x32x16_bf16 over an exact three-way bf16 split of t, in the
//    epilogue, then row scales and either a plain store (in_proj) or the
//    residual add (out_proj).
//  * conv_seq / conv_state_update: the depthwise causal conv over T tokens of
//    each sequence, with the stored window as the history before t = 0.
//  * embed_rows: the embedding rows of a chunk of tokens.
//
// The SSM scans over T tokens are in scan.hip.
#include "common.h"

namespace dfssm {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// v = p1 + p2 + p3 exactly, each part a bf16: p1 keeps the top 8 significant
// bits of v (truncation), p2 the top 8 of the remainder, p3 the remaining at
// most 8 bits.  The remainders are exact fp32 differences.
__device__ __forceinline__ void bf16_split3(float v, __bf16& p1, __bf16& p2, __bf16& p3) {
  const uint32_t u1 = __float_as_uint(v) & 0xFFFF0000u;
  const float r1 = v - __uint_as_float(u1);
  const uint32_t u2 = __float_as_uint(r1) & 0xFFFF0000u;
  const float r2 = r1 - __uint_as_float(u2);
  p1 = __builtin_bit_cast(__bf16, (unsigned short)(u1 >> 16));
  p2 = __builtin_bit_cast(__bf16, (unsigned short)(u2 >> 16));
  p3 = __builtin_bit_cast(__bf16, (unsigned short)(__float_as_uint(r2) >> 16));
}


// ---------------------------------------------------------------------------
// rows_quant: one wave per row, four rows per workgroup.  Lane L holds the
// 16-element chunks j = L + 64 mm of the row (chunk j = elements 16 j ..
// 16 j + 15), so its codes form whole 16-byte words and each LoRA-down row
// is read as one 16-byte load per chunk.
// ---------------------------------------------------------------------------
template <int K>
__global__ __launch_bounds__(256) void rows_quant_kernel(RowsArgs a) {
  constexpr int NCH = K / 16, MM = (NCH + 63) / 64;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.M) return;  // whole wave leaves together
  const float4* x4 = (const float4*)(a.x + (size_t)row * a.ldx);
  const float4* w4 = (const float4*)a.w;
  float4 p[MM][4];
  float ss = 0.0f, pm = 0.0f;
#pragma unroll
  for (int mm = 0; mm < MM; ++mm) {
    const int j = lane + 64 * mm;
    const bool live = j < NCH;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 xv = live ? x4[4 * j + i] : make_float4(0.f, 0.f, 0.f, 0.f);
      const float4 wv = live ? w4[4 * j + i] : make_float4(0.f, 0.f, 0.f, 0.f);
      ss += xv.x * xv.x + xv.y * xv.y + xv.z * xv.z + xv.w * xv.w;
      p[mm][i] = make_float4(xv.x * wv.x, xv.y * wv.y, xv.z * wv.z, xv.w * wv.w);
      pm = fmaxf(pm, fmaxf(fmaxf(fabsf(p[mm][i].x), fabsf(p[mm][i].y)),
                           fmaxf(fabsf(p[mm][i].z), fabsf(p[mm][i].w))));
    }
  }
  ss = wave_sum(ss);
  pm = wave_max(pm);
  const float rstd = 1.0f / sqrtf(ss / (float)K + a.eps);
  const float amax = rstd * pm;
  const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
  const float s = amax > 0.0f ? amax / 127.0f : 0.0f;
  auto qz = [&](float v) -> uint32_t {
    float r = rintf(rstd * v * inv);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (uint32_t)(uint8_t)(int8_t)(int)r;
  };
  uint4 qd[MM];
  int qsum = 0;
#pragma unroll
  for (int mm = 0; mm < MM; ++mm) {
    uint32_t d[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t b0 = qz(p[mm][i].x), b1 = qz(p[mm][i].y), b2 = qz(p[mm][i].z), b3 = qz(p[mm][i].w);
      d[i] = b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
      qsum += (int)(int8_t)b0 + (int)(int8_t)b1 + (int)(int8_t)b2 + (int)(int8_t)b3;
    }
    qd[mm] = make_uint4(d[0], d[1], d[2], d[3]);
    const int j = lane + 64 * mm;
    if (j < NCH) *(uint4*)(a.q + (size_t)row * K + 16 * j) = qd[mm];
  }
  qsum = wave_sum_i(qsum);
  if (lane == 0) {
    a.s[row] = s;
    if (a.qsum) a.qsum[row] = qsum;
  }
  if (!a.A) return;
  // LoRA down: t[k] = float(sum_i A[k][i] q_i) * sA[k] * s, all 16 sums in flight
  int acc[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    int v = 0;
#pragma unroll
    for (int mm = 0; mm < MM; ++mm) {
      const int j = lane + 64 * mm;
      const uint4 av = j < NCH ? *(const uint4*)(a.A + (size_t)k * K + 16 * j) : make_uint4(0, 0, 0, 0);
      v = __builtin_amdgcn_sdot4((int)av.x, (int)qd[mm].x, v, false);
      v = __builtin_amdgcn_sdot4((int)av.y, (int)qd[mm].y, v, false);
      v = __builtin_amdgcn_sdot4((int)av.z, (int)qd[mm].z, v, false);
      v = __builtin_amdgcn_sdot4((int)av.w, (int)qd[mm].w, v, false);
    }
    acc[k] = v;
  }
#pragma unroll
  for (int k = 0; k < 16; ++k) acc[k] = wave_sum_i(acc[k]);
  if (lane < 16) {
    int v = acc[0];
#pragma unroll
    for (int k = 1; k < 16; ++k) v = lane == k ? acc[k] : v;
    a.t[(size_t)row * 16 + lane] = (float)v * a.sA[lane] * s;
  }
}

// rows_quant_row: the same operation with one workgroup per row (K >= 2048),
// thread i holding the E = K / 256 consecutive elements E i .. E i + E - 1:
// a few rows (batched decode) spread over as many CUs as there are rows, and
// each thread's LoRA-down operands (8 bytes per rank and pair of code words)
// are loaded together with its inputs.
template <int K>
__global__ __launch_bounds__(256) void rows_quant_row_kernel(RowsArgs a) {
  constexpr int E = K / 256, E4 = E / 4;
  static_assert(E % 8 == 0, "8, 16 or 32 elements per thread");
  __shared__ float red_f[2][4];
  __shared__ int red_i[4][17];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = blockIdx.x;
  const float4* x4 = (const float4*)(a.x + (size_t)row * a.ldx) + E4 * tid;
  const float4* w4 = (const float4*)a.w + E4 * tid;
  float4 xs[E4], ws[E4];
#pragma unroll
  for (int i = 0; i < E4; ++i) {
    xs[i] = x4[i];
    ws[i] = w4[i];
  }
  // the LoRA-down rows this thread needs, loaded with the row so that both
  // latencies overlap
  uint2 av[16][E4 / 2];
  if (a.A) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const uint2* ar = (const uint2*)(a.A + (size_t)k * K + E * tid);
#pragma unroll
      for (int i = 0; i < E4 / 2; ++i) av[k][i] = ar[i];
    }
  }
  float4 p[E4];
  float ss = 0.0f, pm = 0.0f;
#pragma unroll
  for (int i = 0; i < E4; ++i) {
    const float4 xv = xs[i], wv = ws[i];
    ss += xv.x * xv.x + xv.y * xv.y + xv.z * xv.z + xv.w * xv.w;
    p[i] = make_float4(xv.x * wv.x, xv.y * wv.y, xv.z * wv.z, xv.w * wv.w);
    pm = fmaxf(pm, fmaxf(fmaxf(fabsf(p[i].x), fabsf(p[i].y)), fmaxf(fabsf(p[i].z), fabsf(p[i].w))));
  }
  ss = wave_sum(ss);
  pm = wave_max(pm);
  if (lane == 0) {
    red_f[0][wave] = ss;
    red_f[1][wave] = pm;
  }
  __syncthreads();
  ss = (red_f[0][0] + red_f[0][1]) + (red_f[0][2] + red_f[0][3]);
  pm = fmaxf(fmaxf(red_f[1][0], red_f[1][1]), fmaxf(red_f[1][2], red_f[1][3]));
  const float rstd = 1.0f / sqrtf(ss / (float)K + a.eps);
  const float amax = rstd * pm;
  const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
  const float s = amax > 0.0f ? amax / 127.0f : 0.0f;
  auto qz = [&](float v) -> uint32_t {
    float r = rintf(rstd * v * inv);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (uint32_t)(uint8_t)(int8_t)(int)r;
  };
  uint32_t d[E4];
  int qsum = 0;
#pragma unroll
  for (int i = 0; i < E4; ++i) {
    const uint32_t b0 = qz(p[i].x), b1 = qz(p[i].y), b2 = qz(p[i].z), b3 = qz(p[i].w);
    d[i] = b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
    qsum += (int)(int8_t)b0 + (int)(int8_t)b1 + (int)(int8_t)b2 + (int)(int8_t)b3;
  }
  int8_t* qrow = a.q + (size_t)row * K + E * tid;
#pragma unroll
  for (int i = 0; i < E4; i += 2) *(uint2*)(qrow + 4 * i) = make_uint2(d[i], d[i + 1]);
  // LoRA down: t[k] = float(sum_i A[k][i] q_i) * sA[k] * s
  int acc[17];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    int v = 0;
#pragma unroll
    for (int i = 0; i < E4; i += 2) {
      v = __builtin_amdgcn_sdot4((int)av[k][i / 2].x, (int)d[i], v, false);
      v = __builtin_amdgcn_sdot4((int)av[k][i / 2].y, (int)d[i + 1], v, false);
    }
    acc[k] = a.A ? v : 0;
  }
  acc[16] = qsum;
#pragma unroll
  for (int k = 0; k < 17; ++k) acc[k] = wave_sum_i(acc[k]);
  if (lane == 0) {
#pragma unroll
    for (int k = 0; k < 17; ++k) red_i[wave][k] = acc[k];
  }
  __syncthreads();
  if (tid < 17) {
    const int v = red_i[0][tid] + red_i[1][tid] + red_i[2][tid] + red_i[3][tid];
    if (tid == 16) {
      a.s[row] = s;
      if (a.qsum) a.qsum[row] = v;
    } else if (a.A) {
      a.t[(size_t)row * 16 + tid] = (float)v * a.sA[tid] * s;
    }
  }
}

// LoRA down of many rows on the matrix cores: t[m][r] = float(sum_k A[r][k]
// q[m][k]) * sA[r] * s[m], the same products as the row quantiser's (the
// integer sum is exact, so either kernel gives the same t).  Workgroup = 32
// rows, the four waves take a quarter of K each and sum through LDS; the 16
// ranks are the first 16 of the 32 MFMA columns (the rest read rank 15 and are
// zeroed).  Operands go straight from memory into MFMA registers: lane l holds
// row / rank l % 32 and k-half l / 32 of each 32-wide k-step.
constexpr int kLoraUnroll = 8;

__global__ __launch_bounds__(256) void lora_down_kernel(RowsArgs a, int K) {
  __shared__ int red[3][16][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, kg = lane >> 5;
  const int m0 = blockIdx.x * 32;
  const int mc = min(m0 + col, a.M - 1), rc = min(col, 15);
  const int ks = K / 4, kbeg = wave * ks, kend = kbeg + ks;
  const int8_t* qrow = a.q + (size_t)mc * K + 16 * kg;
  const int8_t* arow = a.A + (size_t)rc * K + 16 * kg;
  v16i acc = (v16i){};
  for (int k0 = kbeg; k0 < kend; k0 += 32 * kLoraUnroll) {
    v4i af[kLoraUnroll], bf[kLoraUnroll];
#pragma unroll
    for (int u = 0; u < kLoraUnroll; ++u) {
      af[u] = *(const v4i*)(qrow + k0 + 32 * u);
      bf[u] = *(const v4i*)(arow + k0 + 32 * u);
    }
#pragma unroll
    for (int u = 0; u < kLoraUnroll; ++u) {
      if (col >= 16) bf[u] = (v4i){};
      acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[u], bf[u], acc, 0, 0, 0);
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) red[wave - 1][r][lane] = acc[r];
  }
  __syncthreads();
  if (wave > 0 || col >= 16) return;
  const float sa = a.sA[col];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int m = m0 + 8 * (r >> 2) + 4 * kg + (r & 3);
    const int v = acc[r] + red[0][r][lane] + red[1][r][lane] + red[2][r][lane];
    if (m < a.M) a.t[(size_t)m * 16 + col] = (float)v * sa * a.s[m];
  }
}

hipError_t launch_rows_quant(const RowsArgs& a, int K, hipStream_t st) {
  if (a.M <= 0) return hipSuccess;
  if (a.A && a.M >= 4096 && K % 1024 == 0 && K <= 8192) {
    // many rows: quantise without the LoRA down, then the LoRA down on the
    // matrix cores (the quantiser would re-read the 16 rows of A from L2 for
    // every row)
    RowsArgs r = a;
    r.A = nullptr;
    hipError_t e = launch_rows_quant(r, K, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(lora_down_kernel, dim3((a.M + 31) / 32), dim3(256), 0, st, a, K);
    return hipGetLastError();
  }
  const dim3 grid((a.M + 3) / 4), block(256);
  switch (K) {
    case 2048: hipLaunchKernelGGL(rows_quant_row_kernel<2048>, dim3(a.M), block, 0, st, a); return hipGetLastError();
    case 4096: hipLaunchKernelGGL(rows_quant_row_kernel<4096>, dim3(a.M), block, 0, st, a); return hipGetLastError();
    case 8192: hipLaunchKernelGGL(rows_quant_row_kernel<8192>, dim3(a.M), block, 0, st, a); return hipGetLastError();
    default: break;
  }
  switch (K) {
    case 256: hipLaunchKernelGGL(rows_quant_kernel<256>, grid, block, 0, st, a); break;
    case 512: hipLaunchKernelGGL(rows_quant_kernel<512>, grid, block, 0, st, a); break;
    case 1024: hipLaunchKernelGGL(rows_quant_kernel<1024>, grid, block, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// bitgemm
// ---------------------------------------------------------------------------

// 0/1 bytes of nibble x (bits 0..3): byte j = bit j.  The multiply copies
// bit i to positions i, i + 7, i + 14 and i + 21; those 16 positions are all
// distinct (so nothing carries) and bit j's copy at 7 j + j = 8 j is the one
// the mask keeps.
__device__ __forceinline__ uint32_t spread_nibble(uint32_t x) { return __umul24(x & 15u, 0x00204081u) & 0x01010101u; }

constexpr int kGemmKB = 64;       // k per LDS stage
constexpr int kGemmLdsRow = 80;   // bytes per LDS tile row (64 + 16 padding)

template <int TM, int TN>
struct GemmTile {
  static constexpr int WAVES_M = TM >= 128 ? 2 : 1, WAVES_N = 4 / WAVES_M;
  static constexpr int WM = TM / WAVES_M, WN = TN / WAVES_N;  // wave tile
  static constexpr int BM = WM / 32, BN = WN / 32;            // 32x32 blocks per wave
  static constexpr int A_BYTES = TM * kGemmLdsRow, B_BYTES = TN * kGemmLdsRow;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int A_CHUNKS = TM * kGemmKB / 16;  // 16-byte chunks of an A k-tile
  static constexpr int B_WORDS = TN * kGemmKB / 32;   // scaffold words of a B k-tile
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be whole 32x32 blocks");
};

// Epilogue of a batched scaffold GEMM tile: 2 acc - sum(q) gives the signed
// scaffold sum, scaled by the column and row scales; the LoRA-up term runs on
// the f32 matrix cores; store or residual add.  acc[i][j] is the 32 x 32 block
// at tile rows wm0 + 32 i, columns wn0 + 32 j.  gsm: at least TM * 120 bytes
// of LDS (reused after the first barrier here).  CONV: the tile may hold conv
// channels of decode tokens (a.xc set); without it no register is set aside
// for the conv windows.
template <int TM, int BM, int BN, int EPI, bool CONV = true>
__device__ __forceinline__ void gemm_tile_epilogue(const GemmArgs& a, const v16i (&acc)[BM][BN], int m0, int n0,
                                                   int wm0, int wn0, unsigned char* gsm) {
  const int lane = threadIdx.x & 63;
  // row data of the tile into LDS: the row scale, the code sum and the
  // LoRA-down vector t.  The plain store form splits t once per row into its
  // three bf16 parts (every wave of the tile multiplies the same rows), as
  // [row][part][16 ranks] with rows 112 bytes apart; the residual and conv
  // forms keep t as fp32 rows 20 floats apart and split it per lane (measured
  // faster there).  Either row stride puts the 16-byte reads of 8 consecutive
  // lanes on 8 different groups of 4 banks.
  constexpr bool kPreSplit = EPI == GEMM_EPI_STORE && !CONV;
  constexpr int kTbRow = 112;
  __syncthreads();
  float* s_s = (float*)gsm;              // [TM]
  int* s_qs = (int*)(s_s + TM);          // [TM]
  unsigned char* s_tb = (unsigned char*)(s_qs + TM);  // [TM][kTbRow] (pre-split) or [TM][20] floats
  float* s_t = (float*)s_tb;
  for (int i = threadIdx.x; i < TM; i += 256) {
    const int m = m0 + i;
    s_s[i] = m < a.M ? a.s[m] : 0.0f;
    s_qs[i] = m < a.M ? a.qsum[m] : 0;
  }
  if constexpr (kPreSplit) {
    for (int i = threadIdx.x; i < TM * 2; i += 256) {  // row i / 2, ranks 8 (i & 1) .. + 7
      const int m = m0 + i / 2;
      float4 u = make_float4(0.f, 0.f, 0.f, 0.f), w = u;
      if (m < a.M) {
        const float4* tp = (const float4*)(a.t + (size_t)m * 16 + 8 * (i & 1));
        u = tp[0];
        w = tp[1];
      }
      const float tv[8] = {u.x, u.y, u.z, u.w, w.x, w.y, w.z, w.w};
      v8bf p1, p2, p3;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        __bf16 b1, b2, b3;
        bf16_split3(tv[e], b1, b2, b3);
        p1[e] = b1;
        p2[e] = b2;
        p3[e] = b3;
      }
      unsigned char* dst = s_tb + (i / 2) * kTbRow + 16 * (i & 1);
      *(v8bf*)dst = p1;
      *(v8bf*)(dst + 32) = p2;
      *(v8bf*)(dst + 64) = p3;
    }
  } else {
    for (int i = threadIdx.x; i < TM * 16; i += 256) {
      const int m = m0 + i / 16;
      s_t[(i >> 4) * 20 + (i & 15)] = m < a.M ? a.t[(size_t)m * 16 + (i & 15)] : 0.0f;
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < BN; ++j) {
    const int n = n0 + wn0 + 32 * j + (lane & 31);
    const bool nok = n < a.N;
    const float sw = nok ? a.sw[n] : 0.0f, sb = nok ? a.sB[n] : 0.0f;
    // LoRA up operand of this column: B[n][8 h + e], h = lane / 32 (int8, exact in bf16)
    const uint4 bq = nok ? *(const uint4*)(a.Bm + (size_t)n * 16) : make_uint4(0, 0, 0, 0);
    const uint32_t bw2[2] = {(lane >> 5) ? bq.z : bq.x, (lane >> 5) ? bq.w : bq.y};
    v8bf bB;
#pragma unroll
    for (int e = 0; e < 8; ++e) bB[e] = (__bf16)(float)(int8_t)(bw2[e >> 2] >> (8 * (e & 3)));
    // residual values of the column block's BM row blocks, all loaded before
    // any of them is used (one memory round trip per column block, and before
    // any store of the block: see the skinny kernel)
    float prev[BM][16];
#pragma unroll
    for (int i = 0; i < BM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm0 + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        prev[i][r] = (EPI == GEMM_EPI_RESIDUAL && m < a.M && nok) ? a.y[(size_t)m * a.ldy + n] : 0.0f;
      }
    // conv shift register of this column (one decode token per row), or none
    const bool conv_col = CONV && EPI == GEMM_EPI_STORE && a.xc && nok && n >= a.x_off && n < a.x_off + a.cdim;
    const int cc = min(max(n - a.x_off, 0), a.cdim - 1);
    float4 cw = make_float4(0.f, 0.f, 0.f, 0.f);
    float cb = 0.0f;
    if (CONV && EPI == GEMM_EPI_STORE && a.xc) {
      cw = *(const float4*)(a.conv_w + (size_t)cc * 4);
      cb = a.conv_b[cc];
    }
#pragma unroll
    for (int i = 0; i < BM; ++i) {
      const int rb = wm0 + 32 * i;  // tile-local first row of the block
      // t of row rb + lane % 32, ranks 8 h .. 8 h + 7, split exactly into three
      // bf16 parts (each part is the top 8 significant bits of what is left), so
      // the rank-16 product is three bf16 matrix-core steps with exact products
      v8bf t1, t2, t3;
      if constexpr (kPreSplit) {
        const unsigned char* tb = s_tb + (rb + (lane & 31)) * kTbRow + 16 * (lane >> 5);
        t1 = *(const v8bf*)tb;
        t2 = *(const v8bf*)(tb + 32);
        t3 = *(const v8bf*)(tb + 64);
      } else {
        const float4* tr4 = (const float4*)(s_t + (rb + (lane & 31)) * 20 + 8 * (lane >> 5));
        const float4 ta = tr4[0], tb = tr4[1];
        const float tr[8] = {ta.x, ta.y, ta.z, ta.w, tb.x, tb.y, tb.z, tb.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          __bf16 p1, p2, p3;
          bf16_split3(tr[e], p1, p2, p3);
          t1[e] = p1;
          t2[e] = p2;
          t3[e] = p3;
        }
      }
      v16f lo = (v16f){};
      lo = __builtin_amdgcn_mfma_f32_32x32x16_bf16(t1, bB, lo, 0, 0, 0);
      lo = __builtin_amdgcn_mfma_f32_32x32x16_bf16(t2, bB, lo, 0, 0, 0);
      lo = __builtin_amdgcn_mfma_f32_32x32x16_bf16(t3, bB, lo, 0, 0, 0);
      // the block's conv windows, loaded before any of its stores (rows past
      // the end read the last one)
      float w0[16], w1[16], w2[16];
      if (CONV && EPI == GEMM_EPI_STORE && a.xc) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = min(m0 + rb + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3), a.M - 1);
          const float* st = a.conv_state + (size_t)m * a.conv_bstride + cc;
          w0[r] = st[0];
          w1[r] = st[a.cdim];
          w2[r] = st[2 * a.cdim];
        }
      }
      // a block inside the matrix stores without a test per element
      const bool full = nok && m0 + rb + 32 <= a.M;
      // row scales and code sums of this lane's rows: four consecutive rows a
      // read (the residual and conv forms, which hold the block's residual
      // values or conv windows, read them one at a time and keep fewer
      // registers live)
      float4 sv = make_float4(0.f, 0.f, 0.f, 0.f);
      int4 qv = make_int4(0, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ml = rb + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int m = m0 + ml;
        float rs;
        int rq;
        if constexpr (kPreSplit) {
          if ((r & 3) == 0) {
            sv = *(const float4*)(s_s + ml);
            qv = *(const int4*)(s_qs + ml);
          }
          rs = (r & 3) == 0 ? sv.x : (r & 3) == 1 ? sv.y : (r & 3) == 2 ? sv.z : sv.w;
          rq = (r & 3) == 0 ? qv.x : (r & 3) == 1 ? qv.y : (r & 3) == 2 ? qv.z : qv.w;
        } else {
          rs = s_s[ml];
          rq = s_qs[ml];
        }
        if (full || (m < a.M && nok)) {
          const int sacc = 2 * acc[i][j][r] - rq;
          const float y = proj_out(sacc, sw, rs, sb, lo[r]);
          // non-temporal: the output streams past the caches (prefill 8 x 2048:
          // 54.7-54.8 vs 56.1-56.3 ms)
          __builtin_nontemporal_store(prev[i][r] + y, &a.y[(size_t)m * a.ldy + n]);
          if (a.acc) a.acc[(size_t)m * a.N + n] = sacc;
          if (conv_col) {  // one decode token: the conv shift register of channel cc
            float* st = a.conv_state + (size_t)m * a.conv_bstride + cc;
            a.xc[(size_t)m * a.cdim + cc] = silu_f(conv4(cb, cw.x, w0[r], cw.y, w1[r], cw.z, w2[r], cw.w, y));
            st[0] = w1[r];
            st[a.cdim] = w2[r];
            st[2 * a.cdim] = y;
          }
        }
      }
    }
  }
}

template <int TM, int TN, int EPI>
__global__ __launch_bounds__(256) void bitgemm_kernel(GemmArgs a) {
  using T = GemmTile<TM, TN>;
  extern __shared__ __attribute__((aligned(16))) unsigned char gsm[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = blockIdx.x * TN, m0 = blockIdx.y * TM;
  const int wm0 = (wave / T::WAVES_N) * T::WM, wn0 = (wave % T::WAVES_N) * T::WN;
  const int K = a.K, KW = K / 32;
  const int nk = K / kGemmKB;

  // global -> registers for one k-tile
  constexpr int AC = (T::A_CHUNKS + 255) / 256, BW = (T::B_WORDS + 255) / 256;
  uint4 ar[AC];
  uint32_t br[BW];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int i = 0; i < AC; ++i) {
      const int c = threadIdx.x + 256 * i;
      const int r = c >> 2, ch = c & 3;
      const int m = m0 + r;
      ar[i] = (c < T::A_CHUNKS && m < a.M)
                  ? *(const uint4*)(a.q + (size_t)m * K + (size_t)kt * kGemmKB + ch * 16)
                  : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < BW; ++i) {
      const int c = threadIdx.x + 256 * i;
      const int r = c >> 1, hw = c & 1;
      const int n = n0 + r;
      br[i] = (c < T::B_WORDS && n < a.N) ? a.bits[(size_t)n * KW + kt * 2 + hw] : 0u;
    }
  };
  // registers -> LDS stage (scaffold words expanded to 0/1 bytes)
  auto store_tile = [&](int stg) {
    unsigned char* As = gsm + stg * T::STAGE;
    unsigned char* Bs = As + T::A_BYTES;
#pragma unroll
    for (int i = 0; i < AC; ++i) {
      const int c = threadIdx.x + 256 * i;
      if (c < T::A_CHUNKS) *(uint4*)(As + (c >> 2) * kGemmLdsRow + (c & 3) * 16) = ar[i];
    }
#pragma unroll
    for (int i = 0; i < BW; ++i) {
      const int c = threadIdx.x + 256 * i;
      if (c < T::B_WORDS) {
        const uint32_t wv = br[i];
        uint4 lo, hi;
        lo.x = spread_nibble(wv);
        lo.y = spread_nibble(wv >> 4);
        lo.z = spread_nibble(wv >> 8);
        lo.w = spread_nibble(wv >> 12);
        hi.x = spread_nibble(wv >> 16);
        hi.y = spread_nibble(wv >> 20);
        hi.z = spread_nibble(wv >> 24);
        hi.w = spread_nibble(wv >> 28);
        unsigned char* dst = Bs + (c >> 1) * kGemmLdsRow + (c & 1) * 32;
        *(uint4*)dst = lo;
        *(uint4*)(dst + 16) = hi;
      }
    }
  };

  v16i acc[T::BM][T::BN];
#pragma unroll
  for (int i = 0; i < T::BM; ++i)
#pragma unroll
    for (int j = 0; j < T::BN; ++j) acc[i][j] = (v16i){};

  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int stg = kt & 1;
    if (kt + 1 < nk) load_tile(kt + 1);
    const unsigned char* As = gsm + stg * T::STAGE;
    const unsigned char* Bs = As + T::A_BYTES;
#pragma unroll
    for (int kk = 0; kk < kGemmKB / 32; ++kk) {
      const int koff = kk * 32 + 16 * (lane >> 5);
      v4i af[T::BM], bf[T::BN];
#pragma unroll
      for (int i = 0; i < T::BM; ++i) af[i] = *(const v4i*)(As + (wm0 + 32 * i + (lane & 31)) * kGemmLdsRow + koff);
#pragma unroll
      for (int j = 0; j < T::BN; ++j) bf[j] = *(const v4i*)(Bs + (wn0 + 32 * j + (lane & 31)) * kGemmLdsRow + koff);
#pragma unroll
      for (int i = 0; i < T::BM; ++i)
#pragma unroll
        for (int j = 0; j < T::BN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) {
      store_tile(stg ^ 1);  // the other stage: last read before the previous barrier
      __syncthreads();
    }
  }

  gemm_tile_epilogue<TM, T::BM, T::BN, EPI>(a, acc, m0, n0, wm0, wn0, gsm);
}

// The scaffold GEMM for many rows (prefill), second form.  Tile 128 x TN,
// k-tiles of 128; four waves in a WR x (4 / WR) grid, each (128 / WR) rows x
// (TN / (4 / WR)) columns of v_mfma_i32_32x32x32_i8 blocks, so a wave expands
// only its own column blocks.  LDS holds the A tile (int8 codes) and the
// scaffold *bits* of the B tile (TN x 16 bytes a stage instead of TN x 128 of
// expanded bytes); each lane expands the 16 bits of its B operand to 0/1
// bytes in registers right before the multiply.  Global loads run two k-tiles
// ahead in two register sets, LDS is double buffered: one barrier per k-tile,
// and each tile's loads have two tiles of matrix work to land.  OCC
// workgroups share a CU (the accumulators then live in VGPRs).
constexpr int kG2TM = 128, kG2KB = 128, kG2ARow = kG2KB + 16;
constexpr int kG2CW = kG2KB / 32;  // scaffold words per column of a k-tile
constexpr int kG2AC = kG2KB / 16;  // 16-byte A chunks per row of a k-tile
constexpr int kG2A = kG2TM * kG2ARow;
constexpr int kG2PT = kG2TM * kG2AC / 256;  // A chunks per thread and k-tile
template <int TN>
struct G2 {
  static constexpr int B = TN * kG2CW * 4, STAGE = kG2A + B;
  static constexpr int PB = TN * kG2CW / 256;  // B words per thread and k-tile
};

__device__ __forceinline__ v4i expand16(uint32_t b) {
  return (v4i){(int)spread_nibble(b), (int)spread_nibble(b >> 4), (int)spread_nibble(b >> 8),
               (int)spread_nibble(b >> 12)};
}

template <int EPI, int TN, int WR, int OCC, bool CONV>
__global__ __launch_bounds__(256, OCC) void bitgemm2_kernel(GemmArgs a) {
  constexpr int TM = kG2TM, KB = kG2KB, WC = 4 / WR;
  constexpr int BM = TM / WR / 32, BN = TN / WC / 32;
  constexpr int PB = G2<TN>::PB, STAGE = G2<TN>::STAGE;
  extern __shared__ __attribute__((aligned(16))) unsigned char gsm[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // XCD-aware tile order: workgroups are dealt to the 8 XCDs round-robin, so
  // workgroup g runs on XCD g % 8; XCD x takes a contiguous run of tiles in
  // row-block-major order, and the tiles that share a row block of A (and
  // every column block of B) share that XCD's L2.
  int n0, m0;
  {
    const int ntn = gridDim.x, T = gridDim.x * gridDim.y;
    const int g = blockIdx.x + ntn * blockIdx.y;
    const int q = T / 8, r = T % 8, x = g % 8;
    const int tile = x * q + min(x, r) + g / 8;
    n0 = (tile % ntn) * TN;
    m0 = (tile / ntn) * TM;
  }
  const int wm0 = WR == 1 ? 0 : (wave / WC) * (TM / WR), wn0 = (WC == 4 ? wave : wave % WC) * (TN / WC);
  const int K = a.K, KW = K / 32, nk = K / KB;
  // a thread's share of a k-tile: A chunks c = t + 256 i (row c / 8, 16-byte
  // chunk c % 8), B words c = t + 256 i (column c / 4, word c % 4)
  struct Tile {
    uint4 a[kG2PT];
    uint32_t b[PB];
  };
  // branch-free loads: rows and columns past the end read the last one, so
  // the compiler can count the loads in flight exactly (a branch around a
  // load makes it wait for all of them).  Those copies are stored as they
  // are: accumulator element (m, n) depends only on A row m and B column n,
  // and the epilogue stores no row past M and no column past N.
  auto load = [&](int kt, Tile& R) {
#pragma unroll
    for (int i = 0; i < kG2PT; ++i) {
      const int c = threadIdx.x + 256 * i;
      const int m = m0 + c / kG2AC;
      R.a[i] = *(const uint4*)(a.q + (size_t)min(m, a.M - 1) * K + (size_t)kt * KB + (c % kG2AC) * 16);
    }
#pragma unroll
    for (int i = 0; i < PB; ++i) {
      const int c = threadIdx.x + 256 * i;
      const int n = n0 + c / kG2CW;
      R.b[i] = a.bits[(size_t)min(n, a.N - 1) * KW + kt * kG2CW + c % kG2CW];
    }
  };
  auto store = [&](int stg, const Tile& R) {
    unsigned char* As = gsm + stg * STAGE;
    uint32_t* Bw = (uint32_t*)(As + kG2A);
#pragma unroll
    for (int i = 0; i < kG2PT; ++i) {
      const int c = threadIdx.x + 256 * i;
      // (stored component by component: a whole-struct copy keeps the
      // register sets in scratch memory)
      const uint4 v = R.a[i];
      *(uint4*)(As + (c / kG2AC) * kG2ARow + (c % kG2AC) * 16) = make_uint4(v.x, v.y, v.z, v.w);
    }
#pragma unroll
    for (int i = 0; i < PB; ++i) Bw[threadIdx.x + 256 * i] = R.b[i];
  };
  v16i acc[BM][BN];
#pragma unroll
  for (int i = 0; i < BM; ++i)
#pragma unroll
    for (int j = 0; j < BN; ++j) acc[i][j] = (v16i){};
  auto compute = [&](int stg) {
    const unsigned char* As = gsm + stg * STAGE;
    const unsigned char* Bb = As + kG2A;
#pragma unroll
    for (int kk = 0; kk < KB / 32; ++kk) {
      const int koff = kk * 32 + 16 * (lane >> 5);
      v4i af[BM], bf[BN];
#pragma unroll
      for (int j = 0; j < BN; ++j) {
        const int col = wn0 + 32 * j + (lane & 31);
        bf[j] = expand16(*(const uint16_t*)(Bb + col * (kG2CW * 4) + kk * 4 + 2 * (lane >> 5)));
      }
#pragma unroll
      for (int i = 0; i < BM; ++i) af[i] = *(const v4i*)(As + (wm0 + 32 * i + (lane & 31)) * kG2ARow + koff);
#pragma unroll
      for (int i = 0; i < BM; ++i)
#pragma unroll
        for (int j = 0; j < BN; ++j) acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  };

  // nk is even (K % 256 == 0), so the loop runs whole pairs of k-tiles with
  // no exit in between, and the loads are unconditional (indexes clamped to
  // the last tile): the compiler keeps one accumulator set and waits only
  // for the tile being stored, not for the one still in flight.
  Tile R0, R1;
  load(0, R0);
  load(1, R1);
  store(0, R0);
  load(min(2, nk - 1), R0);
  __syncthreads();
  // at step kt: LDS stage kt % 2 holds k-tile kt; the register set of parity
  // (kt + 1) % 2 holds tile kt + 1 and the other one tile kt + 2
  for (int kt = 0; kt < nk; kt += 2) {
    compute(0);
    store(1, R1);
    __syncthreads();
    load(min(kt + 3, nk - 1), R1);
    compute(1);
    store(0, R0);  // after the last pair: a copy of the last tile nobody reads
    __syncthreads();
    load(min(kt + 4, nk - 1), R0);
  }
  gemm_tile_epilogue<TM, BM, BN, EPI, CONV>(a, acc, m0, n0, wm0, wn0, gsm);
}

// tile width, wave rows and workgroups per CU of the many-row scaffold GEMM
constexpr int kG2TN = 128, kG2WR = 1, kG2OCC = 3;

template <int TM, int TN>
static hipError_t launch_bitgemm_t(const GemmArgs& a, int epi, hipStream_t st) {
  using T = GemmTile<TM, TN>;
  const dim3 grid((a.N + TN - 1) / TN, (a.M + TM - 1) / TM), block(256);
  size_t lds = 2 * (size_t)T::STAGE;
  const size_t epi_lds = (size_t)TM * (4 + 4 + 112);
  if (epi_lds > lds) lds = epi_lds;
  if (epi == GEMM_EPI_RESIDUAL)
    hipLaunchKernelGGL((bitgemm_kernel<TM, TN, GEMM_EPI_RESIDUAL>), grid, block, lds, st, a);
  else
    hipLaunchKernelGGL((bitgemm_kernel<TM, TN, GEMM_EPI_STORE>), grid, block, lds, st, a);
  return hipGetLastError();
}

hipError_t launch_bitgemm(const GemmArgs& a, int epi, hipStream_t st) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (a.K % kGemmKB) return hipErrorInvalidValue;
  if (a.M <= 32) return launch_bitgemm_t<32, 128>(a, epi, st);
  if (a.K % (2 * kG2KB) == 0) {
    const dim3 grid((a.N + kG2TN - 1) / kG2TN, (a.M + kG2TM - 1) / kG2TM), block(256);
    const size_t lds = 2 * (size_t)G2<kG2TN>::STAGE;
    if ((size_t)grid.x * grid.y <= 512) {
      // few tiles (a batch of decode tokens): half-width tiles of 2 x 2 waves
      // give the launch twice the workgroups
      const dim3 g64((a.N + 63) / 64, grid.y);
      const size_t lds64 = 2 * (size_t)G2<64>::STAGE;
      if (epi == GEMM_EPI_RESIDUAL)
        hipLaunchKernelGGL((bitgemm2_kernel<GEMM_EPI_RESIDUAL, 64, 2, kG2OCC, false>), g64, block, lds64, st, a);
      else if (a.xc)
        hipLaunchKernelGGL((bitgemm2_kernel<GEMM_EPI_STORE, 64, 2, kG2OCC, true>), g64, block, lds64, st, a);
      else
        hipLaunchKernelGGL((bitgemm2_kernel<GEMM_EPI_STORE, 64, 2, kG2OCC, false>), g64, block, lds64, st, a);
      return hipGetLastError();
    }
    if (epi == GEMM_EPI_RESIDUAL)
      hipLaunchKernelGGL((bitgemm2_kernel<GEMM_EPI_RESIDUAL, kG2TN, kG2WR, kG2OCC, false>), grid, block, lds, st, a);
    else if (a.xc)
      hipLaunchKernelGGL((bitgemm2_kernel<GEMM_EPI_STORE, kG2TN, kG2WR, kG2OCC, true>), grid, block, lds, st, a);
    else
      hipLaunchKernelGGL((bitgemm2_kernel<GEMM_EPI_STORE, kG2TN, kG2WR, kG2OCC, false>), grid, block, lds, st, a);
    return hipGetLastError();
  }
  return launch_bitgemm_t<128, 256>(a, epi, st);
}

// ---------------------------------------------------------------------------
// skinny GEMM (a few rows: batched decode, the LM head of its sequences).
// One 32 x 32 output block per workgroup; the four waves take a quarter of K
// each and sum their accumulators through LDS.  Operands go straight from
// global memory (the weights streamed once, the codes from L2) into MFMA
// registers: lane l holds row / column l % 32 and k-half l / 32 of each
// 32-wide k-step, and 16 scaffold bits become 16 0/1 bytes in registers.
// More than 32 rows take several 32-row blocks; workgroups are dealt to the
// 8 XCDs in contiguous runs of tiles with the row block fastest, so the row
// blocks of a column block read its weights on one XCD (from its L2 after
// the first).
// ---------------------------------------------------------------------------
constexpr int kSkinnyUnroll = 16;  // k-steps whose loads are issued together

// VEC: K is a multiple of 4 x 32 x kSkinnyUnroll, so every wave's k slice is
// whole groups of k-steps (the loads need neither clamps nor branches)
template <int KIND, bool VEC>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(SkinnyArgs a0, int nrb) {
  __shared__ int red[3][16][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int n0, r0;
  {
    const int T = gridDim.x, g = blockIdx.x;  // T = nrb x column blocks
    const int q = T / 8, r = T % 8, x = g % 8;
    const int tile = x * q + min(x, r) + g / 8;
    n0 = (tile / nrb) * 32;
    r0 = (tile % nrb) * 32;
  }
  // this workgroup's row block as a GEMM of its own (at most 32 rows)
  SkinnyArgs a = a0;
  a.M = min(32, a0.M - r0);
  a.q += (size_t)r0 * a0.K;
  a.s += r0;
  if (a.qsum) a.qsum += r0;
  if (a.t) a.t += (size_t)r0 * 16;
  a.y += (size_t)r0 * a0.ldy;
  if (a.acc) a.acc += (size_t)r0 * a0.N;
  if (a.xc) a.xc += (size_t)r0 * a0.cdim;
  if (a.conv_state) a.conv_state += (size_t)r0 * a0.conv_bstride;
  const int col = lane & 31, kg = lane >> 5;
  const int n = n0 + col;
  const bool nok = n < a.N, mok = col < a.M;  // this lane's B column and A row
  // Out-of-range rows and columns read a valid row and are zeroed by a
  // select: no load sits behind a branch, so none of them serialises.
  const int nc = nok ? n : a.N - 1, mc = mok ? col : a.M - 1;
  const int K = a.K, ks = K / 4;              // k slice of this wave
  const int kbeg = wave * ks, kend = kbeg + ks;
  // whole groups of scaffold words load 16 bytes at a time where every group start is 16-byte aligned
  const bool wvec = K % (4 * 32 * 4) == 0;
  const int8_t* qrow = a.q + (size_t)mc * K + 16 * kg;

  // Operands of the epilogue (wave 0), loaded before the main loop so that
  // their latency hides under it.
  const bool conv_col = KIND == SK_IN && a.xc && n >= a.x_off && n < a.x_off + a.cdim;
  const int c = min(max(n - a.x_off, 0), a.cdim - 1);
  float sm[16], prev[16], w0[16], w1[16], w2[16], tj[8];
  int qm[16];
  float sw = 0.f, sb = 0.f, cw0 = 0.f, cw1 = 0.f, cw2 = 0.f, cw3 = 0.f, cb = 0.f;
  uint4 bq = make_uint4(0, 0, 0, 0);
  if (wave == 0) {
    sw = a.sw[nc];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = min(8 * (r >> 2) + 4 * kg + (r & 3), a.M - 1);
      sm[r] = a.s[m];
      qm[r] = KIND != SK_HEAD ? a.qsum[m] : 0;
      prev[r] = KIND == SK_OUT ? a.y[(size_t)m * a.ldy + nc] : 0.0f;
      if (KIND == SK_IN && a.xc) {
        const float* st = a.conv_state + (size_t)m * a.conv_bstride + c;
        w0[r] = st[0];
        w1[r] = st[a.cdim];
        w2[r] = st[2 * a.cdim];
      } else {
        w0[r] = w1[r] = w2[r] = 0.0f;
      }
    }
    if (KIND != SK_HEAD) {
      sb = a.sB[nc];
      bq = *(const uint4*)(a.Bm + (size_t)nc * 16);
#pragma unroll
      for (int e = 0; e < 8; ++e) tj[e] = a.t[(size_t)mc * 16 + 8 * kg + e];
    }
    if (KIND == SK_IN && a.xc) {
      const float4 wv = *(const float4*)(a.conv_w + (size_t)c * 4);
      cw0 = wv.x; cw1 = wv.y; cw2 = wv.z; cw3 = wv.w;
      cb = a.conv_b[c];
    }
  }

  v16i acc = (v16i){};
  for (int k0 = kbeg; k0 < kend; k0 += 32 * kSkinnyUnroll) {
    v4i af[kSkinnyUnroll], bf[kSkinnyUnroll];
    uint32_t bw[kSkinnyUnroll];
    if constexpr (VEC) {
      // every wave's k slice is whole groups: no clamp, no per-step word
      // loads, and no branch, so no load waits for another one to land
#pragma unroll
      for (int u = 0; u < kSkinnyUnroll; ++u) {
        af[u] = *(const v4i*)(qrow + k0 + 32 * u);
        if (KIND == SK_HEAD) bf[u] = *(const v4i*)((const int8_t*)a.w + (size_t)nc * K + k0 + 32 * u + 16 * kg);
      }
      if (KIND != SK_HEAD) {
        const uint4* wp = (const uint4*)((const uint32_t*)a.w + (size_t)nc * (K / 32) + k0 / 32);
#pragma unroll
        for (int v = 0; v < kSkinnyUnroll / 4; ++v) {
          const uint4 w4 = wp[v];
          bw[4 * v] = w4.x;
          bw[4 * v + 1] = w4.y;
          bw[4 * v + 2] = w4.z;
          bw[4 * v + 3] = w4.w;
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < kSkinnyUnroll; ++u) {
        const int k = min(k0 + 32 * u, kend - 32);  // a partial last group re-reads valid data, zeroed below
        af[u] = *(const v4i*)(qrow + k);
        if (KIND == SK_HEAD)
          bf[u] = *(const v4i*)((const int8_t*)a.w + (size_t)nc * K + k + 16 * kg);
        else if (!wvec || k0 + 32 * kSkinnyUnroll > kend)  // one word per k-step
          bw[u] = ((const uint32_t*)a.w)[(size_t)nc * (K / 32) + k / 32];
      }
      if (KIND != SK_HEAD && wvec && k0 + 32 * kSkinnyUnroll <= kend) {
        // a whole group: the column's kSkinnyUnroll words are contiguous, four per 16-byte load
        const uint4* wp = (const uint4*)((const uint32_t*)a.w + (size_t)nc * (K / 32) + k0 / 32);
#pragma unroll
        for (int v = 0; v < kSkinnyUnroll / 4; ++v) {
          const uint4 w4 = wp[v];
          bw[4 * v] = w4.x;
          bw[4 * v + 1] = w4.y;
          bw[4 * v + 2] = w4.z;
          bw[4 * v + 3] = w4.w;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kSkinnyUnroll; ++u) {
      const bool live = mok && (VEC || k0 + 32 * u < kend);
      if (!live) af[u] = (v4i){};
      if (KIND != SK_HEAD) {
        const uint32_t h = nok ? bw[u] >> (16 * kg) : 0u;
        bf[u] = (v4i){(int)spread_nibble(h), (int)spread_nibble(h >> 4), (int)spread_nibble(h >> 8),
                      (int)spread_nibble(h >> 12)};
      } else if (!nok) {
        bf[u] = (v4i){};
      }
      acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[u], bf[u], acc, 0, 0, 0);
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) red[wave - 1][r][lane] = acc[r];
  }
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] += red[0][r][lane] + red[1][r][lane] + red[2][r][lane];

  if (KIND == SK_HEAD) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = 8 * (r >> 2) + 4 * kg + (r & 3);
      if (m < a.M && nok) a.y[(size_t)m * a.ldy + n] = (float)acc[r] * sw * sm[r];
    }
    return;
  }
  // LoRA up, lo[m][n] = sum_j t[m][j] B[n][j]: three bf16 matrix-core steps on
  // the exact three-way split of t (the arithmetic of gemm_tile_epilogue, so a
  // row gets the same value on either GEMM)
  const uint32_t bw2[2] = {kg ? bq.z : bq.x, kg ? bq.w : bq.y};
  v8bf bB, t1, t2, t3;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    bB[e] = (__bf16)(nok ? (float)(int8_t)(bw2[e >> 2] >> (8 * (e & 3))) : 0.0f);
    __bf16 p1, p2, p3;
    bf16_split3(mok ? tj[e] : 0.0f, p1, p2, p3);
    t1[e] = p1;
    t2[e] = p2;
    t3[e] = p3;
  }
  v16f lo = (v16f){};
  lo = __builtin_amdgcn_mfma_f32_32x32x16_bf16(t1, bB, lo, 0, 0, 0);
  lo = __builtin_amdgcn_mfma_f32_32x32x16_bf16(t2, bB, lo, 0, 0, 0);
  lo = __builtin_amdgcn_mfma_f32_32x32x16_bf16(t3, bB, lo, 0, 0, 0);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int m = 8 * (r >> 2) + 4 * kg + (r & 3);
    if (m >= a.M || !nok) continue;
    const int sacc = 2 * acc[r] - qm[r];
    const float y = proj_out(sacc, sw, sm[r], sb, lo[r]);
    if (a.acc) a.acc[(size_t)m * a.N + n] = sacc;
    float* yp = a.y + (size_t)m * a.ldy + n;
    if (KIND == SK_OUT) {
      *yp = prev[r] + y;
    } else {
      *yp = y;
      if (conv_col) {  // one decode token: the conv shift register of channel c
        float* st = a.conv_state + (size_t)m * a.conv_bstride + c;
        const float v = conv4(cb, cw0, w0[r], cw1, w1[r], cw2, w2[r], cw3, y);
        a.xc[(size_t)m * a.cdim + c] = silu_f(v);
        st[0] = w1[r];
        st[a.cdim] = w2[r];
        st[2 * a.cdim] = y;
      }
    }
  }
}

hipError_t launch_gemm_skinny(const SkinnyArgs& a, int kind, hipStream_t st) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (a.K % 128) return hipErrorInvalidValue;
  const int nrb = (a.M + 31) / 32;
  const long tiles = (long)nrb * ((a.N + 31) / 32);
  if (tiles > 0x7fffffffL) return hipErrorInvalidValue;
  const dim3 grid((unsigned)tiles), block(256);
  const bool vec = a.K % (4 * 32 * kSkinnyUnroll) == 0;
  switch (kind * 2 + (vec ? 1 : 0)) {
    case SK_IN * 2: hipLaunchKernelGGL((gemm_skinny_kernel<SK_IN, false>), grid, block, 0, st, a, nrb); break;
    case SK_IN * 2 + 1: hipLaunchKernelGGL((gemm_skinny_kernel<SK_IN, true>), grid, block, 0, st, a, nrb); break;
    case SK_OUT * 2: hipLaunchKernelGGL((gemm_skinny_kernel<SK_OUT, false>), grid, block, 0, st, a, nrb); break;
    case SK_OUT * 2 + 1: hipLaunchKernelGGL((gemm_skinny_kernel<SK_OUT, true>), grid, block, 0, st, a, nrb); break;
    case SK_HEAD * 2: hipLaunchKernelGGL((gemm_skinny_kernel<SK_HEAD, false>), grid, block, 0, st, a, nrb); break;
    case SK_HEAD * 2 + 1: hipLaunchKernelGGL((gemm_skinny_kernel<SK_HEAD, true>), grid, block, 0, st, a, nrb); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// causal conv over T (depthwise, width 4) + SiLU
// ---------------------------------------------------------------------------
constexpr int kConvChunk = 16;  // tokens per thread

// Thread = four consecutive channels (float4) and kConvChunk tokens: the
// inputs of its tokens and the three before them are all loaded first (the
// stored window stands in before t = 0), then the outputs are computed.
__global__ __launch_bounds__(256) void conv_seq_kernel(ConvSeqArgs a) {
  const int c = 4 * (blockIdx.x * 256 + threadIdx.x);
  const int b = blockIdx.z;
  if (c >= a.cdim) return;
  const int t0 = blockIdx.y * kConvChunk;
  const int nt = min(a.T - t0, kConvChunk);
  const float* st = a.state + (size_t)b * a.state_bstride + c;  // [3][cdim], oldest first
  const float* xin = a.zx + (size_t)b * a.T * a.ldzx + a.x_off + c;
  float4 x[kConvChunk + 3];
#pragma unroll
  for (int j = 0; j < kConvChunk + 3; ++j) {
    const int t = min(t0 - 3 + j, a.T - 1);
    const float* src = t >= 0 ? xin + (size_t)t * a.ldzx : st + (size_t)(t + 3) * a.cdim;
    x[j] = *(const float4*)src;
  }
  float4 w[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) w[k] = *(const float4*)(a.w + (size_t)(c + k) * 4);
  const float4 bias = *(const float4*)(a.bias + c);
  float* out = a.xc + ((size_t)b * a.T + t0) * a.cdim + c;
#pragma unroll
  for (int j = 0; j < kConvChunk; ++j) {
    if (j < nt) {
      float4 o;
      o.x = silu_f(conv4(bias.x, w[0].x, x[j].x, w[0].y, x[j + 1].x, w[0].z, x[j + 2].x, w[0].w, x[j + 3].x));
      o.y = silu_f(conv4(bias.y, w[1].x, x[j].y, w[1].y, x[j + 1].y, w[1].z, x[j + 2].y, w[1].w, x[j + 3].y));
      o.z = silu_f(conv4(bias.z, w[2].x, x[j].z, w[2].y, x[j + 1].z, w[2].z, x[j + 2].z, w[2].w, x[j + 3].z));
      o.w = silu_f(conv4(bias.w, w[3].x, x[j].w, w[3].y, x[j + 1].w, w[3].z, x[j + 2].w, w[3].w, x[j + 3].w));
      *(float4*)(out + (size_t)j * a.cdim) = o;
    }
  }
}

// window after the T tokens: the last three raw inputs (older ones from the
// previous window when T < 3)
__global__ __launch_bounds__(256) void conv_state_update_kernel(ConvSeqArgs a) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int b = blockIdx.y;
  if (c >= a.cdim) return;
  float* st = a.state + (size_t)b * a.state_bstride;
  const float* xin = a.zx + a.x_off + c;
  float nv[3];
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int t = a.T - 3 + j;
    nv[j] = t >= 0 ? xin[(size_t)((size_t)b * a.T + t) * a.ldzx] : st[(size_t)(j + a.T) * a.cdim + c];
  }
#pragma unroll
  for (int j = 0; j < 3; ++j) st[(size_t)j * a.cdim + c] = nv[j];
}

hipError_t launch_conv_state_update(const ConvSeqArgs& a, hipStream_t st) {
  if (a.B <= 0 || a.T <= 0) return hipSuccess;
  const dim3 g2((a.cdim + 255) / 256, a.B);
  hipLaunchKernelGGL(conv_state_update_kernel, g2, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_conv_seq(const ConvSeqArgs& a, hipStream_t st) {
  if (a.B <= 0 || a.T <= 0) return hipSuccess;
  if (a.cdim % 4 || a.x_off % 4 || a.ldzx % 4) return hipErrorInvalidValue;
  const dim3 g1((a.cdim / 4 + 255) / 256, (a.T + kConvChunk - 1) / kConvChunk, a.B);
  hipLaunchKernelGGL(conv_seq_kernel, g1, dim3(256), 0, st, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_conv_state_update(a, st);
}

// ---------------------------------------------------------------------------
// embedding of a chunk of tokens: row m = b * T + t reads tok[b * tok_stride + t0 + t]
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void embed_rows_kernel(const int32_t* __restrict__ tok, int tok_stride, int t0, int T,
                                                         const int8_t* __restrict__ E, const float* __restrict__ sE,
                                                         int dm, int V, float* __restrict__ h, int* err) {
  const int m = blockIdx.x;
  const int b = m / T, t = m % T;
  int tk = tok[(size_t)b * tok_stride + t0 + t];
  if (tk < 0 || tk >= V) {
    if (threadIdx.x == 0) atomicOr(err, 1);
    tk = 0;
  }
  const float sc = sE[tk];
  const int8_t* er = E + (size_t)tk * dm;
  for (int i = threadIdx.x; i < dm; i += 256) h[(size_t)m * dm + i] = (float)er[i] * sc;
}

hipError_t launch_embed_rows(const int32_t* tok, int tok_stride, int t0, int B, int T, const int8_t* E,
                             const float* sE, int dm, int V, float* h, int* err, hipStream_t st) {
  if (B * T <= 0) return hipSuccess;
  hipLaunchKernelGGL(embed_rows_kernel, dim3(B * T), dim3(256), 0, st, tok, tok_stride, t0, T, E, sE, dm, V, h, err);
  return hipGetLastError();
}

}  // namespace dfssm
