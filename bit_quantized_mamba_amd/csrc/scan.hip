// SSM scans of the batched path over T tokens per sequence, gfx950.
//
//  * scan_kernel: the recurrence token by token, one workgroup per
//    (sequence, head), state in registers, B and C staged through LDS; gated
//    output.
//  * scan1_kernel: one decode token per sequence (headdim 64, d_state 128).
//  * ssd_gram_kernel / ssd_scan_kernel: the same recurrence for headdim 64,
//    d_state 128 unrolled over chunks of 64 tokens into matrix products on
//    the fp32 matrix cores (prefill).
//
// The recurrence (the Mamba-2 block, per head h and sequence):
//   dt = softplus(dt_raw + dt_bias), dA = exp(-dt exp(A_log)),
//   S <- dA S + dt x B^T, y = S C + D x, g = y * silu(z).
#include "common.h"

namespace dfssm {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// SSM scan over T tokens.  Workgroup (head h, sequence b) of 4 P threads:
// thread (p = tid / 4, seg = tid % 4) holds S[p][seg N/4 .. +N/4) in
// registers.  B, C, x, z and dt of kScanChunk tokens are staged in LDS; y[p]
// is the sum over the four threads of a quad (DPP).
// ---------------------------------------------------------------------------
constexpr int kScanChunk = 16;

template <int P, int N>
__global__ __launch_bounds__(4 * P) void scan_kernel(ScanArgs a) {
  constexpr int NPT = N / 4;
  constexpr int NT = 4 * P;
  __shared__ float sB[kScanChunk][N], sC[kScanChunk][N], sx[kScanChunk][P], sz[kScanChunk][P], sdt[kScanChunk];
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  const int p = tid >> 2, seg = tid & 3;
  float* stb = a.ssm + (size_t)b * a.ssm_bstride + (size_t)h * P * N;  // [P/16][N][16]
  float S[NPT];
#pragma unroll
  for (int j = 0; j < NPT; ++j) {
    const int n = seg * NPT + j;
    S[j] = stb[((size_t)(p >> 4) * N + n) * 16 + (p & 15)];
  }
  const float dtb = a.dt_bias[h], ea = __expf(a.A_log[h]), Dh = a.D[h];
  const size_t row0 = (size_t)b * a.T;
  for (int t0 = 0; t0 < a.T; t0 += kScanChunk) {
    const int tc = min(kScanChunk, a.T - t0);
    __syncthreads();  // previous chunk fully consumed
    for (int i = tid; i < tc * N; i += NT) {
      const int tt = i / N, n = i % N;
      const float* xr = a.xc + (row0 + t0 + tt) * a.cdim;
      sB[tt][n] = xr[a.d_inner + n];
      sC[tt][n] = xr[a.d_inner + N + n];
    }
    for (int i = tid; i < tc * P; i += NT) {
      const int tt = i / P, pp = i % P;
      sx[tt][pp] = a.xc[(row0 + t0 + tt) * a.cdim + (size_t)h * P + pp];
      sz[tt][pp] = a.zx[(row0 + t0 + tt) * a.ldzx + (size_t)h * P + pp];
    }
    for (int i = tid; i < tc; i += NT) sdt[i] = a.zx[(row0 + t0 + i) * a.ldzx + a.dt_off + h];
    __syncthreads();
    for (int tt = 0; tt < tc; ++tt) {
      const float dt = softplus_f(sdt[tt] + dtb);
      const float dA = __expf(-dt * ea);
      const float x = sx[tt][p];
      const float dtx = dt * x;
      float y = 0.0f;
#pragma unroll
      for (int j = 0; j < NPT; ++j) {
        const int n = seg * NPT + j;
        S[j] = S[j] * dA + dtx * sB[tt][n];
        y += S[j] * sC[tt][n];
      }
      y += dpp_f<kDppQuadSwap1>(y);
      y += dpp_f<kDppQuadSwap2>(y);
      if (seg == 0) {
        const float yy = y + Dh * x;
        a.g[(row0 + t0 + tt) * a.d_inner + (size_t)h * P + p] = yy * silu_f(sz[tt][p]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < NPT; ++j) {
    const int n = seg * NPT + j;
    stb[((size_t)(p >> 4) * N + n) * 16 + (p & 15)] = S[j];
  }
}

// One decode token per sequence (T = 1), headdim 64, d_state 128.  Workgroup
// (four heads, sequence) of 1024 threads, 256 per head (four heads a workgroup
// measured 3.5 % faster per batch-512 step than one, two 2 %); within a head, wave w
// takes the channel block pb = w (channels 16 w .. 16 w + 15, one [N][16]
// slab of the [P/16][N][16] state layout, 8 KB), lane l the channels
// 16 w + 4 (l & 3) + 0..3 of states n = 16 i + (l >> 2), i = 0..7.  So for
// each i the 64 lanes of a wave read (and later write) one contiguous 1 KB of
// state, whole cache lines.  B and C (shared by the heads of a sequence) are
// staged in LDS once per workgroup; the sum over states crosses the 16 state
// groups once, through LDS.  When the head count is not a multiple of 4,
// the last workgroup's quarters without a head only take part in the
// barriers.
__global__ __launch_bounds__(1024) void scan1_kernel(ScanArgs a) {
  constexpr int P = 64, N = 128, NPT = 8;
  __shared__ __attribute__((aligned(16))) float red4[4][16][P];
  __shared__ float sBC[2 * N];
  const int quarter = threadIdx.x >> 8, t = threadIdx.x & 255;
  // items (four heads of one sequence) blockIdx.x, blockIdx.x + gridDim.x, ...
  const int ngrp = (a.H + 3) / 4, nitems = ngrp * a.B;
  for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
  const int h = 4 * (item % ngrp) + quarter, b = item / ngrp;
  const bool live = h < a.H;
  float (*red)[P] = red4[quarter];
  const int lane = t & 63, pb = t >> 6, pq = lane & 3, ns = lane >> 2;
  const int p0 = pb * 16 + pq * 4;
  const int hc = live ? h : a.H - 1;  // a head without work reads valid memory and stores nothing
  float* stb = a.ssm + (size_t)b * a.ssm_bstride + (size_t)hc * P * N;
  const float* xr = a.xc + (size_t)b * a.cdim;
  float4 S[NPT];
  // the state is streamed (read once and written once per step): non-temporal accesses
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    const v4f v = __builtin_nontemporal_load((const v4f*)(stb + ((size_t)(pb * N + 16 * i + ns) * 16 + pq * 4)));
    S[i] = make_float4(v.x, v.y, v.z, v.w);
  }
  if (quarter == 0) sBC[t] = xr[a.d_inner + t];  // B then C (2 N = 256 values)
  const float4 xv = *(const float4*)(xr + hc * P + p0);
  const float dt = softplus_f(a.zx[(size_t)b * a.ldzx + a.dt_off + hc] + a.dt_bias[hc]);
  const float dA = __expf(-dt * __expf(a.A_log[hc]));
  const float dx0 = dt * xv.x, dx1 = dt * xv.y, dx2 = dt * xv.z, dx3 = dt * xv.w;
  __syncthreads();
  float y0 = 0.f, y1 = 0.f, y2 = 0.f, y3 = 0.f;
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    const float bn = sBC[16 * i + ns], cn = sBC[N + 16 * i + ns];
    float4 v = S[i];
    v.x = v.x * dA + dx0 * bn;
    v.y = v.y * dA + dx1 * bn;
    v.z = v.z * dA + dx2 * bn;
    v.w = v.w * dA + dx3 * bn;
    S[i] = v;
    y0 += v.x * cn;
    y1 += v.y * cn;
    y2 += v.z * cn;
    y3 += v.w * cn;
  }
  if (live) {
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const v4f v = {S[i].x, S[i].y, S[i].z, S[i].w};
      __builtin_nontemporal_store(v, (v4f*)(stb + ((size_t)(pb * N + 16 * i + ns) * 16 + pq * 4)));
    }
  }
  *(float4*)&red[ns][p0] = make_float4(y0, y1, y2, y3);
  __syncthreads();
  if (live && t < P) {
    float yy = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) yy += red[k][t];
    const float x = xr[h * P + t];
    const float z = a.zx[(size_t)b * a.ldzx + h * P + t];
    a.g[(size_t)b * a.d_inner + h * P + t] = (yy + a.D[h] * x) * silu_f(z);
  }
  __syncthreads();  // sBC and red are the next item's
  }
}

// ---------------------------------------------------------------------------
// Chunked scan on the matrix cores (headdim P = 64, d_state N = 128).
//
// Within a chunk of L = 64 tokens, with a_t = -dt_t exp(A_log) and the
// running sums A_i = a_0 + ... + a_i (positions i, j in the chunk), the
// recurrence unrolls to
//   S_i = exp(A_i) S_in + sum_{j<=i} exp(A_i - A_j) dt_j x_j B_j^T
//   y_i = exp(A_i) S_in C_i + sum_{j<=i} exp(A_i - A_j) dt_j (C_i . B_j) x_j.
// With G = C B^T (shared by all heads of a sequence) and
// M[i][j] = G[i][j] exp(A_i - A_j) dt_j for j <= i (0 above the diagonal):
//   Y     = diag(exp(A)) C S_in^T + M X                        [L][P]
//   S_out = exp(A_{L-1}) S_in + X^T diag(w) B,  w_j = exp(A_{L-1} - A_j) dt_j
// The ragged tail of a sequence is padded with tokens of dt = 0 (no decay, no
// input), which leave the state as it is.  Every product is fp32 on
// v_mfma_f32_32x32x2f32 (exact products, fp32 sums).
//
// ssd_gram_kernel writes G for every chunk; ssd_scan_kernel walks the chunks
// of one sequence in order for two heads, with the state in registers.
// ---------------------------------------------------------------------------
static_assert(kSsdL == 64, "the chunked scan is written for chunks of 64 tokens");
constexpr int kSsdRow = kSsdL + 4;             // LDS row of 64 floats (+4 against bank conflicts)
constexpr int kSsdCRow = 128 + 8;              // LDS row of 128 floats (+8: rows 4 apart fall on other banks)
constexpr int kSsdOC = 0;                      // C       [64 i][kSsdCRow]
constexpr int kSsdOB = kSsdOC + 64 * kSsdCRow;   // B     [64 j][kSsdCRow]
constexpr int kSsdOX = kSsdOB + 64 * kSsdCRow;   // x of both heads [64 j][kSsdCRow]
constexpr int kSsdOG = kSsdOX + 64 * kSsdCRow;   // G     [64 i][kSsdRow]
constexpr int kSsdOPar = kSsdOG + 64 * kSsdRow;  // per head: A_i, dt_j, w_j, exp(A_i)  [2][4][64]
constexpr int kSsdOZ = kSsdOPar + 2 * 4 * 64;     // z of both heads [64 i][kSsdCRow]
constexpr int kSsdOCW = kSsdOZ + 64 * kSsdCRow;  // conv weights of both heads' x channels [128][4]
constexpr int kSsdOCB = kSsdOCW + 128 * 4;        // conv biases [128]
constexpr int kSsdFloats = kSsdOCB + 128;
constexpr size_t kSsdLds = sizeof(float) * kSsdFloats;
static_assert(8 * 16 * 64 <= 64 * kSsdCRow, "the partial-sum exchange fits in the C buffer");

// Workgroup barrier that orders LDS only: __syncthreads() would also wait for
// every global load and store in flight (the next chunk's operands, the
// outputs just written).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ v16f mfma_f32(float a, float b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// G[b][c][i][j] = C_{t0+i} . B_{t0+j} for chunk c of sequence b, where B and
// C are the causal conv outputs of the chunk's tokens: computed here from the
// in_proj output (the three inputs before the chunk from the previous rows or
// the stored window) and written to the chunk's record for the scan.  Rows
// past the end of the sequence count as zero.  Then the chunk parameters of
// every head.  Workgroup (chunk, sequence), wave w computes the 32 x 32 tile
// (w >> 1, w & 1) of G; the tile above the diagonal is never read and not
// written.
__global__ __launch_bounds__(256) void ssd_gram_kernel(ScanArgs a) {
  constexpr int N = 128;
  __shared__ __attribute__((aligned(16))) float sC[64 * kSsdRow], sB[64 * kSsdRow];
  const int c = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, col = lane & 31, half = lane >> 5;
  const int ti = wave >> 1, tj = wave & 1;
  const int t0 = c * kSsdL, Lc = min(kSsdL, a.T - t0);
  const size_t row0 = (size_t)b * a.T + t0, rowb = (size_t)b * a.T;
  float* const recB = a.gram + ((size_t)b * gridDim.x + c) * ssd_record_floats(a.H) + kSsdL * kSsdL +
                      (size_t)a.H * 4 * kSsdL;
  float* const recC = recB + kSsdL * N;
  // conv: thread = channel ch of this half (0..63 of B, 64..127 of C), tokens 32 rh .. 32 rh + 31
  const int ch = tid & 127, rh = tid >> 7;
  v16f acc = (v16f){};
  for (int nh = 0; nh < 2; ++nh) {  // two halves of d_state
    if (nh) __syncthreads();
    {
      const int n = nh * 64 + (ch & 63);
      const int cc = a.d_inner + (ch < 64 ? 0 : N) + n;  // conv channel
      const float4 cw = *(const float4*)(a.conv_w + (size_t)cc * 4);
      const float cb = a.conv_b[cc];
      const float* zcol = a.zx + a.x_off + cc;
      const float* wst = a.conv_state + (size_t)b * a.conv_bstride + cc;
      float v[32 + 3];  // inputs of tokens t0 + 32 rh - 3 ..
#pragma unroll
      for (int k = 0; k < 35; ++k) {
        const int t = t0 + 32 * rh - 3 + k;
        const float* src = t >= 0 ? zcol + (rowb + min(t, a.T - 1)) * a.ldzx : wst + (size_t)(t + 3) * a.cdim;
        v[k] = *src;
      }
      float* dst = (ch < 64 ? sB : sC) + (ch & 63);
      float* rdst = (ch < 64 ? recB : recC) + n;
#pragma unroll
      for (int r = 0; r < 32; ++r) {
        const int j = 32 * rh + r;
        const float o = j < Lc ? silu_f(conv4(cb, cw.x, v[r], cw.y, v[r + 1], cw.z, v[r + 2], cw.w, v[r + 3])) : 0.0f;
        dst[j * kSsdRow] = o;
        rdst[(size_t)j * N] = o;
      }
    }
    __syncthreads();
    if (wave != 1) {
      const float* ar = sC + (32 * ti + col) * kSsdRow + 4 * half;
      const float* br = sB + (32 * tj + col) * kSsdRow + 4 * half;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float4 av = *(const float4*)(ar + 8 * q), bv = *(const float4*)(br + 8 * q);
        acc = mfma_f32(av.x, bv.x, acc);
        acc = mfma_f32(av.y, bv.y, acc);
        acc = mfma_f32(av.z, bv.z, acc);
        acc = mfma_f32(av.w, bv.w, acc);
      }
    }
  }
  float* rec = a.gram + ((size_t)b * gridDim.x + c) * ssd_record_floats(a.H);
  if (wave != 1) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = 32 * ti + 8 * (r >> 2) + 4 * half + (r & 3);
      rec[i * kSsdL + 32 * tj + col] = acc[r];
    }
  }
  // chunk parameters of every head (wave w: heads w, w + 4, ...; lane = position j):
  // A_j (running sum of -dt exp(A_log)), dt_j, w_j = exp(A_{L-1} - A_j) dt_j, exp(A_j)
  float* par = rec + kSsdL * kSsdL;
  const size_t rj = row0 + min(lane, Lc - 1);
  // the inputs of kHB heads are loaded together (one memory latency per
  // batch instead of one per head); heads past H read head H - 1, unused
  constexpr int kHB = 8;
  for (int h0 = wave; h0 < a.H; h0 += 4 * kHB) {
    float raw[kHB], bias[kHB], alog[kHB];
#pragma unroll
    for (int i = 0; i < kHB; ++i) {
      const int h = min(h0 + 4 * i, a.H - 1);
      raw[i] = a.zx[rj * a.ldzx + a.dt_off + h];
      bias[i] = a.dt_bias[h];
      alog[i] = a.A_log[h];
    }
#pragma unroll
    for (int i = 0; i < kHB; ++i) {
      const int h = h0 + 4 * i;
      if (h >= a.H) break;
      const float dt = lane < Lc ? softplus_f(raw[i] + bias[i]) : 0.0f;
      float cum = -dt * __expf(alog[i]);
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const float o = __shfl_up(cum, d);
        if (lane >= d) cum += o;
      }
      // A_{L-1} is the last real token's running sum, and padding lanes (dt
      // = 0) take exactly that value: the lanes' scan trees round
      // differently, and when |A| is huge the difference between two trees'
      // sums of the same terms is far from 0
      const float end = __shfl(cum, Lc - 1);
      if (lane >= Lc) cum = end;
      float* ph = par + h * 256;
      ph[lane] = cum;
      ph[64 + lane] = dt;
      // A_{L-1} - A_j <= 0 (the running sums never increase); with huge |A|
      // the trees' rounding can make it positive, where exp may overflow:
      // the clamp keeps the exact bound
      ph[128 + lane] = __expf(fminf(end - cum, 0.0f)) * dt;
      ph[192 + lane] = __expf(cum);
    }
  }
}

// One chunk's operands in registers: per thread the in_proj outputs x of
// channels 4 q .. 4 q + 3 of both heads (q = tid % 32) for tokens 4 rg - 3 ..
// 4 rg + 3 (rg = tid / 32; before the sequence start the stored conv window),
// four float4 of the conv outputs B and C (from the chunk's record) and of z
// (rows j = idx / 32, float4 q = idx % 32 of idx = tid + 512 k), two of G
// and (threads < 128) one of the two heads' parameters.  Tokens past the
// sequence end read the last one; their values are zeroed or unused.
struct SsdStage {
  float4 x[7], b[4], c[4], z[4], g[2], par;
};

__device__ __forceinline__ void ssd_stage_load(const ScanArgs& a, int hp, int tid, int b, int t0, const float* rec,
                                               SsdStage& st) {
  const size_t rowb = (size_t)b * a.T;
  {
    const int q = tid & 31, rg = tid >> 5;
    const float* xz = a.zx + a.x_off + (size_t)(2 * hp) * 64 + 4 * q;
    const float* xw = a.conv_state + (size_t)b * a.conv_bstride + (size_t)(2 * hp) * 64 + 4 * q;
#pragma unroll
    for (int k = 0; k < 7; ++k) {
      const int t = t0 + 4 * rg - 3 + k;
      const float* src = t >= 0 ? xz + (rowb + min(t, a.T - 1)) * a.ldzx : xw + (size_t)(t + 3) * a.cdim;
      st.x[k] = *(const float4*)src;
    }
  }
  const float* recB = rec + kSsdL * kSsdL + (size_t)a.H * 4 * kSsdL;
  const float* recC = recB + kSsdL * 128;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int idx = tid + 512 * k;
    const int j = idx >> 5, q = idx & 31;
    st.b[k] = *(const float4*)(recB + j * 128 + 4 * q);
    st.c[k] = *(const float4*)(recC + j * 128 + 4 * q);
    // z is read once: non-temporal (54.70-54.74 vs 54.90-55.16 ms per 8 x 2048 prefill)
    const v4f zv = __builtin_nontemporal_load(
        (const v4f*)(a.zx + (rowb + min(t0 + j, a.T - 1)) * a.ldzx + (size_t)(2 * hp) * 64 + 4 * q));
    st.z[k] = make_float4(zv.x, zv.y, zv.z, zv.w);
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int idx = tid + 512 * k;
    st.g[k] = *(const float4*)(rec + (idx >> 4) * kSsdL + 4 * (idx & 15));
  }
  st.par = *(const float4*)(rec + kSsdL * kSsdL + (size_t)(2 * hp) * 256 + 4 * (tid & 127));
}

// Workgroup (head pair, sequence) of 8 waves; wave w serves head 2 hp + (w >> 2),
// channel block pb = (w >> 1) & 1 (channels 32 pb .. 32 pb + 31) and half
// h2 = (w & 1) ^ (w >> 2) (waves w and w + 4 share a SIMD; with opposite halves
// each SIMD gets one wave of either half, and the halves differ in work: the
// first position block's M X needs only j < 32): it holds the state tiles
// S^T[n][p] of states 64 h2 .. 64 h2 + 63
// (two 32 x 32 accumulator tiles: lane = channel, register = state) and
// produces the outputs of chunk positions 32 h2 .. 32 h2 + 31.  Per chunk:
//  (a) partial C S_in^T over its 64 states for both position blocks (its own
//      state tiles are the A operand as they sit in the accumulators), the
//      partial of the other block handed to the partner wave through LDS;
//  (b) + M X for its positions;
//  (c) S <- exp(A_{L-1}) S + X^T diag(w) B for its state tiles.
// The k index of every product runs over 4-element runs: k-step s of half hf
// is element 8 (s / 4) + 4 hf + s % 4, the order in which the accumulator
// registers hold the states, so that C and G come from LDS as one 16-byte
// read per four steps (x and B, stored as rows, are read along them).
__global__ __launch_bounds__(512, 1) void ssd_scan_kernel(ScanArgs a) {
  constexpr int P = 64, N = 128;
  extern __shared__ __attribute__((aligned(16))) float sm[];
  const int hp = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, col = lane & 31, half = lane >> 5;
  const int hh = wave >> 2, pb = (wave >> 1) & 1, h2 = (wave & 1) ^ hh;
  const int h = 2 * hp + hh;
  const int p = 32 * pb + col;  // this lane's channel in (b), (c) and the state tiles
  const int nch = (a.T + kSsdL - 1) / kSsdL;
  const size_t rowb = (size_t)b * a.T;
  float* sPar = sm + kSsdOPar + hh * 256;  // [0] A_i  [64] dt_j  [128] w_j  [192] exp(A_i)
  const float* sXh = sm + kSsdOX + hh * 64;  // x of this head: [j][kSsdCRow]

  float* stb = a.ssm + (size_t)b * a.ssm_bstride + (size_t)h * P * N;  // [P/16][N][16]
  // state element (p, n) of tile t, register r: n = 64 h2 + 32 t + 8 (r / 4) + 4 half + r % 4;
  // relative to this lane's first element the offsets are compile-time constants
  float* sp = stb + ((size_t)(p >> 4) * N + 64 * h2 + 4 * half) * 16 + (p & 15);
  v16f S[2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) S[t][r] = sp[(32 * t + 8 * (r >> 2) + (r & 3)) * 16];
  const float Dh = a.D[h];
  const int iy = 32 * h2 + col;  // this lane's output position
  const size_t recf = ssd_record_floats(a.H);

  // conv weights and biases of both heads' x channels, for the whole launch
  if (tid < 128) {
    const int cch = 2 * hp * 64 + tid;
    *(float4*)(sm + kSsdOCW + 4 * tid) = *(const float4*)(a.conv_w + (size_t)cch * 4);
    sm[kSsdOCB + tid] = a.conv_b[cch];
  }
  SsdStage st;
  ssd_stage_load(a, hp, tid, b, 0, a.gram + (size_t)b * nch * recf, st);
  // gated outputs of the previous chunk, stored once the next chunk's loads
  // have been waited for (a store issued after those loads would hold them up)
  float4 go[4];
  float* gprev = nullptr;

  for (int c = 0; c < nch; ++c) {
    const int t0 = c * kSsdL, Lc = min(kSsdL, a.T - t0);
    const size_t row0 = rowb + t0;
    lds_barrier();  // the previous chunk is done with LDS
    // ---- the chunk's operands into LDS: x of both heads, B, C, G, z, parameters
    {
      // x: the causal conv of this thread's 4 channels, tokens 4 rg .. 4 rg + 3
      {
        const int q = tid & 31, rg = tid >> 5;
        const float4* cw = (const float4*)(sm + kSsdOCW) + 4 * q;
        const float4 cw0 = cw[0], cw1 = cw[1], cw2 = cw[2], cw3 = cw[3];
        const float4 cb = *(const float4*)(sm + kSsdOCB + 4 * q);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = 4 * rg + r;
          const float4 x0 = st.x[r], x1 = st.x[r + 1], x2 = st.x[r + 2], x3 = st.x[r + 3];
          float4 o;
          o.x = silu_f(conv4(cb.x, cw0.x, x0.x, cw0.y, x1.x, cw0.z, x2.x, cw0.w, x3.x));
          o.y = silu_f(conv4(cb.y, cw1.x, x0.y, cw1.y, x1.y, cw1.z, x2.y, cw1.w, x3.y));
          o.z = silu_f(conv4(cb.z, cw2.x, x0.z, cw2.y, x1.z, cw2.z, x2.z, cw2.w, x3.z));
          o.w = silu_f(conv4(cb.w, cw3.x, x0.w, cw3.y, x1.w, cw3.z, x2.w, cw3.w, x3.w));
          if (j >= Lc) o = make_float4(0.f, 0.f, 0.f, 0.f);
          *(float4*)(sm + kSsdOX + j * kSsdCRow + 4 * q) = o;
        }
      }
      // B and C (conv outputs from the chunk's record, zero past the end), z
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int idx = tid + 512 * k;
        const int j = idx >> 5, q = idx & 31;
        *(float4*)(sm + kSsdOB + j * kSsdCRow + 4 * q) = st.b[k];
        *(float4*)(sm + kSsdOC + j * kSsdCRow + 4 * q) = st.c[k];
        *(float4*)(sm + kSsdOZ + j * kSsdCRow + 4 * q) = st.z[k];
      }
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int idx = tid + 512 * k;
        *(float4*)(sm + kSsdOG + (idx >> 4) * kSsdRow + 4 * (idx & 15)) = st.g[k];
      }
      if (tid < 128) *(float4*)(sm + kSsdOPar + 4 * tid) = st.par;
    }
    if (gprev) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) *(float4*)(gprev + 32 * pb + 8 * r4 + 4 * half) = go[r4];
    }
    lds_barrier();
    if (c + 1 < nch)  // loaded while this chunk is computed
      ssd_stage_load(a, hp, tid, b, t0 + kSsdL, a.gram + ((size_t)b * nch + c + 1) * recf, st);

    // ---- (a) Y_inter^T[p][i] = exp(A_i) sum_n S_in[p][n] C[i][n], partial over this wave's 64 states, both position blocks
    v16f Y0 = (v16f){}, Y1 = (v16f){};
    {
      const float e0 = sPar[192 + col], e1 = sPar[192 + 32 + col];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int nb = 2 * h2 + t;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const float4 c0 = *(const float4*)(sm + kSsdOC + col * kSsdCRow + 32 * nb + 8 * r4 + 4 * half);
          const float4 c1 = *(const float4*)(sm + kSsdOC + (32 + col) * kSsdCRow + 32 * nb + 8 * r4 + 4 * half);
          Y0 = mfma_f32(S[t][4 * r4 + 0], c0.x, Y0);
          Y1 = mfma_f32(S[t][4 * r4 + 0], c1.x, Y1);
          Y0 = mfma_f32(S[t][4 * r4 + 1], c0.y, Y0);
          Y1 = mfma_f32(S[t][4 * r4 + 1], c1.y, Y1);
          Y0 = mfma_f32(S[t][4 * r4 + 2], c0.z, Y0);
          Y1 = mfma_f32(S[t][4 * r4 + 2], c1.z, Y1);
          Y0 = mfma_f32(S[t][4 * r4 + 3], c0.w, Y0);
          Y1 = mfma_f32(S[t][4 * r4 + 3], c1.w, Y1);
        }
      }
      // exp(A_i) scales output column i (lane % 32 of either block)
      Y0 *= e0;
      Y1 *= e1;
    }
    lds_barrier();  // C is no longer read: its space takes the partial sums
    float* xch = sm + kSsdOC;
    {
      const v16f& give = h2 ? Y0 : Y1;
#pragma unroll
      for (int r = 0; r < 16; ++r) xch[(wave * 16 + r) * 64 + lane] = give[r];
    }
    lds_barrier();
    v16f Yo = h2 ? Y1 : Y0;
#pragma unroll
    for (int r = 0; r < 16; ++r) Yo[r] += xch[((wave ^ 1) * 16 + r) * 64 + lane];

    // ---- (b) + M X for positions 32 h2 .. 32 h2 + 31 (positions j <= i only) and
    // (c) S <- exp(A_{L-1}) S + X^T diag(w) B for this wave's state tiles, one
    // group of four k-steps at a time (both take the same x operands)
    {
      const float cumi = sPar[iy];
      const float dec = __expf(sPar[63]);
      S[0] *= dec;
      S[1] *= dec;
      const float* bt0 = sm + kSsdOB + 64 * h2 + col;  // B[j][n] of this lane's states n = 64 h2 + col (+ 32)
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int j0 = 8 * q + 4 * half;
        float xq[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) xq[e] = sXh[(j0 + e) * kSsdCRow + p];
        if (q < 4 || h2) {  // positions < 32 need j < 32 only
          const float4 gv = *(const float4*)(sm + kSsdOG + iy * kSsdRow + j0);
          const float4 cj = *(const float4*)(sPar + j0);
          const float4 dj = *(const float4*)(sPar + 64 + j0);
          const float gq[4] = {gv.x, gv.y, gv.z, gv.w}, cq[4] = {cj.x, cj.y, cj.z, cj.w},
                      dq[4] = {dj.x, dj.y, dj.z, dj.w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            Yo = mfma_f32(xq[e], j0 + e <= iy ? gq[e] * __expf(fminf(cumi - cq[e], 0.0f)) * dq[e] : 0.0f, Yo);
        }
        const float4 wv = *(const float4*)(sPar + 128 + j0);
        const float wq[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float b0 = bt0[(j0 + e) * kSsdCRow], b1 = bt0[(j0 + e) * kSsdCRow + 32];
          S[0] = mfma_f32(b0 * wq[e], xq[e], S[0]);
          S[1] = mfma_f32(b1 * wq[e], xq[e], S[1]);
        }
      }
    }

    // ---- gated output of position iy: lane register r is channel 32 pb + 8 (r / 4) + 4 half + r % 4
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int p0 = 32 * pb + 8 * r4 + 4 * half;
      const float4 xq = *(const float4*)(sXh + iy * kSsdCRow + p0);
      const float4 zq = *(const float4*)(sm + kSsdOZ + iy * kSsdCRow + hh * 64 + p0);
      go[r4].x = (Yo[4 * r4 + 0] + Dh * xq.x) * silu_f(zq.x);
      go[r4].y = (Yo[4 * r4 + 1] + Dh * xq.y) * silu_f(zq.y);
      go[r4].z = (Yo[4 * r4 + 2] + Dh * xq.z) * silu_f(zq.z);
      go[r4].w = (Yo[4 * r4 + 3] + Dh * xq.w) * silu_f(zq.w);
    }
    gprev = iy < Lc ? a.g + (row0 + iy) * a.d_inner + (size_t)h * P : nullptr;
  }
  if (gprev) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) *(float4*)(gprev + 32 * pb + 8 * r4 + 4 * half) = go[r4];
  }
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) sp[(32 * t + 8 * (r >> 2) + (r & 3)) * 16] = S[t][r];
}

hipError_t launch_scan(const ScanArgs& a, int P, int N, hipStream_t st) {
  if (a.B <= 0 || a.T <= 0) return hipSuccess;
  const dim3 grid(a.H, a.B);
  if (a.T == 1 && P == 64 && N == 128) {
    // Two items per workgroup once there are many more items than the 512
    // workgroups that fit the chip at once (batch 512 as two chains of 256:
    // 20.64-20.69 vs 20.88-20.92 ms per step over 32 steps on one box, the
    // same over 8); with fewer items that would leave CUs idle (batch 32:
    // 2.69 vs 2.55 ms), and four or more per workgroup measured no better.
    const int nitems = (a.H + 3) / 4 * a.B;
    const int per = nitems >= 2048 ? 2 : 1;
    hipLaunchKernelGGL(scan1_kernel, dim3((nitems + per - 1) / per), dim3(1024), 0, st, a);
    return hipGetLastError();
  }
  if (P == 64 && N == 128) {
    if (!a.gram || !a.conv_w || !a.conv_b || !a.conv_state || a.H % 2) return hipErrorInvalidValue;
    if (a.x_off % 4 || a.ldzx % 4 || a.cdim % 4 || a.conv_bstride % 4) return hipErrorInvalidValue;
    // set on every call: the limit is per device, and the call is a host-side table update
    const hipError_t e = hipFuncSetAttribute((const void*)ssd_scan_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)kSsdLds);
    if (e != hipSuccess) return e;
    const int nch = (a.T + kSsdL - 1) / kSsdL;
    hipLaunchKernelGGL(ssd_gram_kernel, dim3(nch, a.B), dim3(256), 0, st, a);
    hipLaunchKernelGGL(ssd_scan_kernel, dim3(a.H / 2, a.B), dim3(512), kSsdLds, st, a);
    return hipGetLastError();
  }
  if (P == 32 && N == 16) hipLaunchKernelGGL((scan_kernel<32, 16>), grid, dim3(128), 0, st, a);
  else if (P == 64 && N == 64) hipLaunchKernelGGL((scan_kernel<64, 64>), grid, dim3(256), 0, st, a);
  else if (P == 32 && N == 128) hipLaunchKernelGGL((scan_kernel<32, 128>), grid, dim3(128), 0, st, a);
  else if (P == 64 && N == 16) hipLaunchKernelGGL((scan_kernel<64, 16>), grid, dim3(256), 0, st, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

bool scan_takes_conv_inputs(int P, int N) { return P == 64 && N == 128; }

bool scan_supported(int P, int N) {
  return (P == 64 && (N == 128 || N == 64 || N == 16)) || (P == 32 && (N == 16 || N == 128));
}

}  // namespace dfssm
