// Decode-path kernels for gfx950 (wave64).
//
//  * norm_quant: RMSNorm + per-token int8 quantisation of one activation row
//    per workgroup, then the operand preparation the 1-bit GEMV needs: the
//    eight two's-complement bit planes of q, the row sum of q, and the LoRA
//    down-projection t = A q (rank r) -- so the GEMV itself never touches q.
//  * proj_gemv: the fused 1-bit scaffold GEMV.  With q split into bit planes
//    P_b, the sum of q over the +1 weights of a 32-weight word w is
//    sum_{b<7} 2^b popcount(w & P_b) - 128 popcount(w & P_7), so one packed
//    weight word costs 8 AND + 8 bit-count-and-add instructions and the
//    scaffold dot product is acc = 2 * (that sum) - sum(q).  Weights stream
//    from HBM as 128-bit loads, one row per U = d_in/128 lanes.  The epilogue
//    applies the row scale, the LoRA up-projection, and (for in_proj) the conv
//    shift register or (for out_proj) the residual add.
//  * ssm: one workgroup per (sequence, head, 16 head channels): state update
//    S <- dA S + dt x B^T and y = S C + D x over the whole state dimension,
//    then the SiLU(z) gate.
//  * lm_head: int8 GEMV over the tied embedding with 4-way int8 dot products.
//  * argmax, embed, row quantiser, zero fill.
#include "common.h"

namespace dfssm {

// ---------------------------------------------------------------------------
// block reductions (blockDim.x a multiple of 64, <= 1024)
// ---------------------------------------------------------------------------

__device__ float block_sum(float v, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float r = 0.0f;
  for (int i = 0; i < nw; ++i) r += red[i];
  return r;
}

__device__ float block_max(float v, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_max(v);
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < nw; ++i) r = fmaxf(r, red[i]);
  return r;
}

__device__ int block_sum_i(int v, int* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_sum_i(v);
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  int r = 0;
  for (int i = 0; i < nw; ++i) r += red[i];
  return r;
}

// ---------------------------------------------------------------------------
// operand preparation from an int8 row held in LDS
// ---------------------------------------------------------------------------

// planes: word w (32 inputs), plane b: bit k = bit b of (uint8)q[32 w + k].
// A wave covers 64 inputs (two words) per ballot.
__device__ void write_planes(const int8_t* qs, int n, uint32_t* planes) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  for (int i0 = wave * 64; i0 < n; i0 += nw * 64) {
    const int i = i0 + lane;
    const uint32_t qi = (i < n) ? (uint32_t)(uint8_t)qs[i] : 0u;
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const uint64_t m = __ballot((qi >> b) & 1u);
      if (lane == 0) {
        planes[(i0 >> 5) * 8 + b] = (uint32_t)m;
        if (i0 + 32 < n) planes[((i0 >> 5) + 1) * 8 + b] = (uint32_t)(m >> 32);
      }
    }
  }
}

// t[k] = float(sum_i A[k][i] q_i) * sA[k] * s ; one wave per k.  n % 4 == 0.
__device__ void lora_down(const int8_t* qs, int n, const int8_t* A, const float* sA, int r, float s, float* t) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int nw4 = n >> 2;
  for (int k = wave; k < r; k += nw) {
    const int* arow = (const int*)(A + (size_t)k * n);
    const int* q4 = (const int*)qs;
    int acc = 0;
    for (int j = lane; j < nw4; j += 64) acc = __builtin_amdgcn_sdot4(arow[j], q4[j], acc, false);
    acc = wave_sum_i(acc);
    if (lane == 0) t[k] = (float)acc * sA[k] * s;
  }
}

// ---------------------------------------------------------------------------
// norm + quant + prep.  One workgroup (1024 threads) per row.
// dynamic LDS: n floats + n int8
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(1024) void norm_quant_kernel(const float* __restrict__ x, const float* __restrict__ w,
                                                          int n, float eps, const int8_t* __restrict__ A,
                                                          const float* __restrict__ sA, int r,
                                                          int8_t* __restrict__ q, uint32_t* __restrict__ planes,
                                                          int32_t* __restrict__ qsum, float* __restrict__ s_out,
                                                          float* __restrict__ t) {
  extern __shared__ unsigned char smem[];
  float* us = (float*)smem;
  int8_t* qs = (int8_t*)(us + n);
  __shared__ float red[16];
  __shared__ int redi[16];
  const int b = blockIdx.x;
  const float* xr = x + (size_t)b * n;

  float ss = 0.0f;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const float v = xr[i];
    ss += v * v;
  }
  ss = block_sum(ss, red);
  const float rstd = 1.0f / sqrtf(ss / (float)n + eps);
  float amax = 0.0f;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const float u = xr[i] * rstd * w[i];
    us[i] = u;
    amax = fmaxf(amax, fabsf(u));
  }
  amax = block_max(amax, red);
  const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
  const float s = amax > 0.0f ? amax / 127.0f : 0.0f;
  int qsum_p = 0;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    float rq = rintf(us[i] * inv);
    rq = fminf(fmaxf(rq, -127.0f), 127.0f);
    const int8_t qi = (int8_t)(int)rq;
    qs[i] = qi;
    q[(size_t)b * n + i] = qi;
    qsum_p += qi;
  }
  const int tot = block_sum_i(qsum_p, redi);  // includes the barrier that publishes qs
  if (threadIdx.x == 0) {
    qsum[b] = tot;
    s_out[b] = s;
  }
  write_planes(qs, n, planes + (size_t)b * (n / 32) * 8);
  if (A) lora_down(qs, n, A, sA, r, s, t + (size_t)b * r);
}

hipError_t launch_norm_quant(const float* x, const float* w, int n, int B, float eps, const int8_t* A,
                             const float* sA, int r, int8_t* q, uint32_t* planes, int32_t* qsum, float* s,
                             float* t, hipStream_t st) {
  const size_t sm = (size_t)n * 5;
  hipLaunchKernelGGL(norm_quant_kernel, dim3(B), dim3(1024), sm, st, x, w, n, eps, A, sA, r, q, planes, qsum, s,
                     t);
  return hipGetLastError();
}

__global__ __launch_bounds__(1024) void qprep_kernel(const int8_t* __restrict__ q, const float* __restrict__ s,
                                                     int n, const int8_t* __restrict__ A,
                                                     const float* __restrict__ sA, int r,
                                                     uint32_t* __restrict__ planes, int32_t* __restrict__ qsum,
                                                     float* __restrict__ t) {
  extern __shared__ unsigned char smem[];
  int8_t* qs = (int8_t*)smem;
  __shared__ int redi[16];
  const int b = blockIdx.x;
  int p = 0;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int8_t qi = q[(size_t)b * n + i];
    qs[i] = qi;
    p += qi;
  }
  const int tot = block_sum_i(p, redi);
  if (threadIdx.x == 0) qsum[b] = tot;
  write_planes(qs, n, planes + (size_t)b * (n / 32) * 8);
  if (A) lora_down(qs, n, A, sA, r, s[b], t + (size_t)b * r);
}

hipError_t launch_qprep(const int8_t* q, const float* s, int n, int B, const int8_t* A, const float* sA, int r,
                        uint32_t* planes, int32_t* qsum, float* t, hipStream_t st) {
  hipLaunchKernelGGL(qprep_kernel, dim3(B), dim3(1024), (size_t)n, st, q, s, n, A, sA, r, planes, qsum, t);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// 1-bit scaffold GEMV + LoRA + epilogue.
// Block: 256 threads (4 waves).  Lane layout: U = d_in/128 lanes per row, lane
// j of a row owns 128-bit chunk j (words 4j..4j+3) of every row it visits and
// keeps those words' 32 plane words in registers.  Each wave visits NP passes
// of 64/U rows with all NP weight loads issued before any arithmetic.
// ---------------------------------------------------------------------------

constexpr int kProjWaves = 4;
constexpr int kProjNP = 2;

__device__ __forceinline__ int plane_dot(const uint4 w, const uint32_t (&P)[4][8]) {
  uint32_t c[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    uint32_t v = __builtin_popcount(w.x & P[0][b]);
    v += __builtin_popcount(w.y & P[1][b]);
    v += __builtin_popcount(w.z & P[2][b]);
    v += __builtin_popcount(w.w & P[3][b]);
    c[b] = v;
  }
  int pos = 0;
#pragma unroll
  for (int b = 0; b < 7; ++b) pos += (int)(c[b] << b);
  pos -= (int)(c[7] << 7);
  return pos;
}

template <int EPI>
__global__ __launch_bounds__(256) void proj_gemv_kernel(ProjArgs a) {
  const int U = a.d_in >> 7;  // lanes per row (power of two, <= 64)
  const int W = a.d_in >> 5;  // words per row
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & (U - 1);
  const int sub = lane / U;
  const int rpp = 64 / U;  // rows per pass
  const int b = blockIdx.y;

  // weights first: they do not depend on the activations
  const int row0 = (blockIdx.x * kProjWaves + wave) * rpp * kProjNP;
  uint4 wv[kProjNP];
  const uint4* bits4 = (const uint4*)a.bits;
#pragma unroll
  for (int p = 0; p < kProjNP; ++p) {
    const int row = row0 + p * rpp + sub;
    wv[p] = row < a.d_out ? bits4[(size_t)row * (W >> 2) + j] : make_uint4(0, 0, 0, 0);
  }
  uint32_t P[4][8];
  {
    const uint4* pl = (const uint4*)(a.in.planes + (size_t)b * W * 8 + (size_t)j * 32);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint4 v = pl[k];
      P[k >> 1][(k & 1) * 4 + 0] = v.x;
      P[k >> 1][(k & 1) * 4 + 1] = v.y;
      P[k >> 1][(k & 1) * 4 + 2] = v.z;
      P[k >> 1][(k & 1) * 4 + 3] = v.w;
    }
  }
  const int qsum = a.in.qsum[b];
  const float s = a.in.s[b];
  const float* t = a.in.t + (size_t)b * a.r;

#pragma unroll
  for (int p = 0; p < kProjNP; ++p) {
    int pos = plane_dot(wv[p], P);
    for (int o = U >> 1; o > 0; o >>= 1) pos += __shfl_xor(pos, o, 64);
    const int row = row0 + p * rpp + sub;
    if (j == 0 && row < a.d_out) {
      const int acc = 2 * pos - qsum;
      float lo = 0.0f;
      const int8_t* brow = a.Bm + (size_t)row * a.r;
      for (int k = 0; k < a.r; ++k) lo += (float)brow[k] * t[k];
      const float y = (float)acc * a.sw[row] * s + a.sB[row] * lo;
      const size_t bo = (size_t)b * a.d_out + row;
      if (a.acc) a.acc[bo] = acc;
      if (EPI == EPI_STORE) {
        a.y[bo] = y;
      } else if (EPI == EPI_OUT_PROJ) {
        a.h[bo] += y;
      } else {
        const int c = row - a.d_inner;
        if (c >= 0 && c < a.conv_dim) {
          float* cs = a.conv_state + (size_t)b * a.conv_bstride;
          const float* wc = a.conv_w + (size_t)c * a.K;
          float v = a.conv_b[c];
          for (int k = 0; k < a.K - 1; ++k) v += wc[k] * cs[(size_t)k * a.conv_dim + c];
          v += wc[a.K - 1] * y;
          for (int k = 0; k < a.K - 2; ++k) cs[(size_t)k * a.conv_dim + c] = cs[(size_t)(k + 1) * a.conv_dim + c];
          cs[(size_t)(a.K - 2) * a.conv_dim + c] = y;
          a.xc[(size_t)b * a.conv_dim + c] = silu_f(v);
        } else {
          a.zx[bo] = y;
        }
      }
    }
  }
}

hipError_t launch_proj(const ProjArgs& a, int epi, hipStream_t st) {
  const int U = a.d_in >> 7;
  const int rows_per_block = kProjWaves * (64 / U) * kProjNP;
  dim3 grid((a.d_out + rows_per_block - 1) / rows_per_block, a.B);
  switch (epi) {
    case EPI_STORE: hipLaunchKernelGGL(proj_gemv_kernel<EPI_STORE>, grid, dim3(256), 0, st, a); break;
    case EPI_IN_PROJ: hipLaunchKernelGGL(proj_gemv_kernel<EPI_IN_PROJ>, grid, dim3(256), 0, st, a); break;
    default: hipLaunchKernelGGL(proj_gemv_kernel<EPI_OUT_PROJ>, grid, dim3(256), 0, st, a); break;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// SSM state update + gate.  State block of (b, h, 16-channel group pg) is
// [N][16] fp32, contiguous; thread t owns float4 (n = f/4, channels 4(f%4)..)
// for f = t, t + 256, ...
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void ssm_kernel(const float* __restrict__ xc, const float* __restrict__ zx,
                                                  int ld_zx, const float* __restrict__ A_log,
                                                  const float* __restrict__ dt_bias, const float* __restrict__ D,
                                                  float* __restrict__ ssm_layer, size_t ssm_bstride,
                                                  float* __restrict__ g, int H, int P, int N, int d_inner,
                                                  int conv_dim) {
  __shared__ float4 red[4][4];
  const int b = blockIdx.y;
  const int groups = P >> 4;
  const int hp = blockIdx.x;
  const int h = hp / groups, pg = hp - h * groups;
  const float* xcb = xc + (size_t)b * conv_dim;
  const float* zxb = zx + (size_t)b * ld_zx;
  const float dt = softplus_f(zxb[d_inner + conv_dim + h] + dt_bias[h]);
  const float dA = __expf(-dt * __expf(A_log[h]));
  const int pq = threadIdx.x & 3;
  const int c0 = h * P + pg * 16 + pq * 4;
  const float4 x4 = *(const float4*)(xcb + c0);
  const float4 dx = make_float4(dt * x4.x, dt * x4.y, dt * x4.z, dt * x4.w);
  float4* st = (float4*)(ssm_layer + (size_t)b * ssm_bstride + (size_t)hp * N * 16);
  const float* Bv = xcb + d_inner;
  const float* Cv = xcb + d_inner + N;
  float4 yp = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int f = threadIdx.x; f < N * 4; f += 256) {
    const int n = f >> 2;
    float4 S = st[f];
    const float bn = Bv[n], cn = Cv[n];
    S.x = S.x * dA + dx.x * bn;
    S.y = S.y * dA + dx.y * bn;
    S.z = S.z * dA + dx.z * bn;
    S.w = S.w * dA + dx.w * bn;
    st[f] = S;
    yp.x += S.x * cn;
    yp.y += S.y * cn;
    yp.z += S.z * cn;
    yp.w += S.w * cn;
  }
  // reduce over lanes with the same pq (lane bits 2..5), then over the 4 waves
#pragma unroll
  for (int o = 4; o < 64; o <<= 1) {
    yp.x += __shfl_xor(yp.x, o, 64);
    yp.y += __shfl_xor(yp.y, o, 64);
    yp.z += __shfl_xor(yp.z, o, 64);
    yp.w += __shfl_xor(yp.w, o, 64);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane < 4) red[wave][lane] = yp;
  __syncthreads();
  if (threadIdx.x < 16) {
    const int q = threadIdx.x >> 2, e = threadIdx.x & 3;
    float y = 0.0f;
    for (int wv = 0; wv < 4; ++wv) {
      const float4 v = red[wv][q];
      y += e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
    }
    const int c = h * P + pg * 16 + threadIdx.x;
    const float xv = xcb[c];
    y += D[h] * xv;
    const float z = zxb[c];
    g[(size_t)b * d_inner + c] = y * silu_f(z);
  }
}

hipError_t launch_ssm(const float* xc, const float* zx, int ld_zx, const float* A_log, const float* dt_bias,
                      const float* D, float* ssm_layer, size_t ssm_bstride, float* g, int B, int H, int P, int N,
                      int d_inner, int conv_dim, hipStream_t st) {
  dim3 grid(H * (P / 16), B);
  hipLaunchKernelGGL(ssm_kernel, grid, dim3(256), 0, st, xc, zx, ld_zx, A_log, dt_bias, D, ssm_layer, ssm_bstride,
                     g, H, P, N, d_inner, conv_dim);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// LM head: logits[b][v] = float(sum_i E[v][i] qf[b][i]) * sE[v] * sf[b]
// L = min(64, dm/16) lanes per row, M = dm/16/L 128-bit chunks per lane.
// ---------------------------------------------------------------------------

constexpr int kHeadWaves = 4;
constexpr int kHeadNP = 4;

__global__ __launch_bounds__(256) void lm_head_kernel(const int8_t* __restrict__ E, const float* __restrict__ sE,
                                                      const int8_t* __restrict__ qf, const float* __restrict__ sf,
                                                      int V, int dm, float* __restrict__ logits) {
  const int C = dm >> 4;  // 128-bit chunks per row
  const int L = C < 64 ? C : 64;
  const int M = C / L;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & (L - 1);
  const int sub = lane / L;
  const int rpp = 64 / L;
  const int b = blockIdx.y;
  const int row0 = (blockIdx.x * kHeadWaves + wave) * rpp * kHeadNP;
  const uint4* E4 = (const uint4*)E;
  const uint4* q4 = (const uint4*)(qf + (size_t)b * dm);
  const float sfb = sf[b];
  for (int p = 0; p < kHeadNP; ++p) {
    const int row = row0 + p * rpp + sub;
    int acc = 0;
    if (row < V) {
      for (int m = 0; m < M; ++m) {
        const uint4 e = E4[(size_t)row * C + j + m * L];
        const uint4 q = q4[j + m * L];
        acc = __builtin_amdgcn_sdot4((int)e.x, (int)q.x, acc, false);
        acc = __builtin_amdgcn_sdot4((int)e.y, (int)q.y, acc, false);
        acc = __builtin_amdgcn_sdot4((int)e.z, (int)q.z, acc, false);
        acc = __builtin_amdgcn_sdot4((int)e.w, (int)q.w, acc, false);
      }
    }
    for (int o = L >> 1; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
    if (j == 0 && row < V) logits[(size_t)b * V + row] = (float)acc * sE[row] * sfb;
  }
}

hipError_t launch_lm_head(const int8_t* E, const float* sE, const int8_t* qf, const float* sf, int V, int dm,
                          int B, float* logits, hipStream_t st) {
  const int C = dm >> 4;
  const int L = C < 64 ? C : 64;
  const int rows_per_block = kHeadWaves * (64 / L) * kHeadNP;
  dim3 grid((V + rows_per_block - 1) / rows_per_block, B);
  hipLaunchKernelGGL(lm_head_kernel, grid, dim3(256), 0, st, E, sE, qf, sf, V, dm, logits);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// argmax (lowest index on ties), one workgroup per row
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(1024) void argmax_kernel(const float* __restrict__ logits, int V, int B,
                                                      int32_t* __restrict__ next, int32_t* __restrict__ out,
                                                      int32_t* __restrict__ counter) {
  __shared__ float bv[16];
  __shared__ int bi[16];
  const int b = blockIdx.x;
  const float* lr = logits + (size_t)b * V;
  float best = -__builtin_huge_valf();
  int idx = 0x7fffffff;
  // Rows of a multiple of 4 logits from a 16-byte aligned base are read as float4, four
  // loads in flight per thread (indexes clamped, not branched around, so the
  // loads issue together); a thread meets its indexes in increasing order, so
  // the strict compare keeps the lowest index of equal values.
  const int V4 = V % 4 == 0 && ((uintptr_t)logits & 15) == 0 ? V / 4 : 0;
  const float4* l4 = (const float4*)lr;
  for (int base = threadIdx.x; base < V4; base += 4 * (int)blockDim.x) {
    float4 x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) x[u] = l4[min(base + u * (int)blockDim.x, V4 - 1)];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = base + u * (int)blockDim.x;
      if (i < V4) {
        if (x[u].x > best) { best = x[u].x; idx = 4 * i; }
        if (x[u].y > best) { best = x[u].y; idx = 4 * i + 1; }
        if (x[u].z > best) { best = x[u].z; idx = 4 * i + 2; }
        if (x[u].w > best) { best = x[u].w; idx = 4 * i + 3; }
      }
    }
  }
  for (int v = 4 * V4 + threadIdx.x; v < V; v += blockDim.x) {
    const float x = lr[v];
    if (x > best) { best = x; idx = v; }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ob = __shfl_xor(best, o, 64);
    const int oi = __shfl_xor(idx, o, 64);
    if (ob > best || (ob == best && oi < idx)) { best = ob; idx = oi; }
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) { bv[wave] = best; bi[wave] = idx; }
  __syncthreads();
  if (threadIdx.x == 0) {
    const int nw = blockDim.x >> 6;
    for (int w = 1; w < nw; ++w)
      if (bv[w] > best || (bv[w] == best && bi[w] < idx)) { best = bv[w]; idx = bi[w]; }
    if (idx == 0x7fffffff) idx = 0;  // all -inf / NaN row
    if (out) out[(size_t)(*counter) * B + b] = idx;
    next[b] = idx;
  }
}

// advance the generation counter once every row has read it
__global__ void counter_advance_kernel(int32_t* counter) {
  if (threadIdx.x == 0) *counter += 1;
}

hipError_t launch_argmax(const float* logits, int V, int B, int32_t* next, int32_t* out, int32_t* counter,
                         hipStream_t st) {
  hipLaunchKernelGGL(argmax_kernel, dim3(B), dim3(1024), 0, st, logits, V, B, next, out, counter);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !out) return e;
  hipLaunchKernelGGL(counter_advance_kernel, dim3(1), dim3(64), 0, st, counter);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// embedding
// ---------------------------------------------------------------------------

__global__ void embed_kernel(const int32_t* __restrict__ tok, int tok_stride, const int8_t* __restrict__ E,
                             const float* __restrict__ sE, int dm, int V, float* __restrict__ h,
                             int* __restrict__ err) {
  const int b = blockIdx.x;
  int t = tok[(size_t)b * tok_stride];
  if (t < 0 || t >= V) {
    if (threadIdx.x == 0) atomicOr(err, 1);
    t = 0;
  }
  const float sc = sE[t];
  for (int i = threadIdx.x; i < dm; i += blockDim.x) h[(size_t)b * dm + i] = (float)E[(size_t)t * dm + i] * sc;
}

hipError_t launch_embed(const int32_t* tok, int tok_stride, const int8_t* E, const float* sE, int dm, int V,
                        int B, float* h, int* err, hipStream_t st) {
  hipLaunchKernelGGL(embed_kernel, dim3(B), dim3(256), 0, st, tok, tok_stride, E, sE, dm, V, h, err);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// plain per-row quantiser (two passes over global memory)
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(1024) void quant_rows_kernel(const float* __restrict__ u, int n, int8_t* __restrict__ q,
                                                          float* __restrict__ s) {
  __shared__ float red[16];
  const int b = blockIdx.x;
  const float* ur = u + (size_t)b * n;
  float amax = 0.0f;
  for (int i = threadIdx.x; i < n; i += blockDim.x) amax = fmaxf(amax, fabsf(ur[i]));
  amax = block_max(amax, red);
  const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    float rq = rintf(ur[i] * inv);
    rq = fminf(fmaxf(rq, -127.0f), 127.0f);
    q[(size_t)b * n + i] = (int8_t)(int)rq;
  }
  if (threadIdx.x == 0) s[b] = amax > 0.0f ? amax / 127.0f : 0.0f;
}

hipError_t launch_quant_rows(const float* u, int rows, int n, int8_t* q, float* s, hipStream_t st) {
  hipLaunchKernelGGL(quant_rows_kernel, dim3(rows), dim3(1024), 0, st, u, n, q, s);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// zero fill (used instead of memset so the same call can live inside graphs)
// ---------------------------------------------------------------------------

__global__ void zero_kernel(uint32_t* p, size_t nwords) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < nwords; i += stride) p[i] = 0u;
}

// fp16 -> fp32, exact (every binary16 value is a binary32 value)
__global__ void f16_to_f32_kernel(const _Float16* __restrict__ src, float* __restrict__ dst, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) dst[i] = (float)src[i];
}

hipError_t launch_f16_to_f32(const void* src, float* dst, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(f16_to_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (const _Float16*)src, dst, n);
  return hipGetLastError();
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t st) {
  const size_t nw = bytes / 4;
  if (nw == 0) return hipSuccess;
  size_t blocks = (nw + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (uint32_t*)p, nw);
  return hipGetLastError();
}

}  // namespace dfssm
