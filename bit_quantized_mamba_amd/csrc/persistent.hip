// Batch-1 decode as one persistent kernel.
//
// Why: at batch 1 a layer is a chain of three all-to-all dependencies (the
// residual stream h feeds every in_proj row; the SSM of every head needs the
// shared B and C channels; every out_proj row needs the whole gated SSM
// output).  On MI355X a kernel boundary costs ~1.6 us and so does a software
// all-to-all among 256 workgroups, while a layer's weights and state stream
// in ~1.3 us, so the step is bound by these dependency hops, not by HBM.  One
// launch keeps every workgroup resident across all layers and tokens, so the
// weights and state a workgroup will need next are already in flight (they
// do not depend on the token) while it waits on a hop, and no launch gap is
// paid at all.
//
// Work split: workgroup w = (head hd, 16-channel slice j) owns
//   in_proj rows z[hd, j*16 .. +16) and x[hd, j*16 .. +16), the dt row of its
//   head (computed by the head's slices redundantly), and B/C rows i with
//   i % G == w; their conv channels; the SSM state block [hd][j*16..+16][:];
//   out_proj rows [w * d_model/G, +d_model/G).
// Hops: each value crossing workgroups is published as a 64-bit word
// {fp32 bits, epoch} with a relaxed device-scope atomic store into R = 8
// replicas (replica r read by the workgroups with w % 8 == r, which spreads
// the readers of a line); readers poll with relaxed device-scope atomic
// loads until the epoch matches.  A value and its epoch travel in one
// single-copy-atomic word, so no fence or flag ordering is involved, and
// every instance of a hop has its own epoch.  Each box is reused once per
// layer; a writer can only reach its next use after every reader has passed
// the hop that follows this one, so one buffer per box suffices.
// Every wait is bounded: a workgroup that polls too long sets a device abort
// flag, which all waits check, so a fault ends the kernel instead of hanging.
#include "common.h"
#include "persistent.h"

namespace dfssm {

constexpr int kPT = 256;  // threads per workgroup: one wave per SIMD, so each wave has the full register file
constexpr int kPW = kPT / 64;
constexpr int kR = 8;     // replicas of each published word
constexpr long kSpinLimit = 1 << 21;

__device__ __forceinline__ uint64_t ld64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t pack(float v, unsigned e) { return ((uint64_t)e << 32) | __float_as_uint(v); }

__device__ __forceinline__ bool aborted(const int* flag) {
  return __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
}

// publish value `v` as word `i` of a box of n words (all replicas)
__device__ __forceinline__ void publish(uint64_t* box, int n, int i, float v, unsigned e) {
  const uint64_t w = pack(v, e);
#pragma unroll 1
  for (int r = 0; r < kR; ++r) st64(box + (size_t)r * n + i, w);
}

// Read words [0, n) of this workgroup's replica into LDS.  All loads of a
// thread are issued before any is checked; in the common case every word is
// already current and the check is a handful of compares.  Stale words are
// re-polled one by one in a compact loop (kept rolled: the layer loop must fit
// the instruction cache).  Returns false (for every thread of the workgroup)
// on abort.
__device__ __noinline__ bool gather_slow(const uint64_t* src, int n, unsigned e, float* dst, int* abort_flag,
                                         int maxw) {
  for (int m = 0; m < maxw; ++m) {
    const int i = threadIdx.x + m * kPT;
    if (i >= n) break;
    uint64_t v = ld64(src + i);
    long spins = 0;
    while ((unsigned)(v >> 32) != e) {
      if (++spins > kSpinLimit) {
        __hip_atomic_store(abort_flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return false;
      }
      if ((spins & 63) == 0 && aborted(abort_flag)) return false;
      v = ld64(src + i);
    }
    dst[i] = __uint_as_float((unsigned)v);
  }
  return true;
}

template <int MAXW>
__device__ bool gather(const uint64_t* box, int n, unsigned e, float* dst, int* abort_flag, int* s_stop) {
  const uint64_t* src = box + (size_t)(blockIdx.x % kR) * n;
  uint64_t w[MAXW];
#pragma unroll
  for (int m = 0; m < MAXW; ++m) {
    const int i = threadIdx.x + m * kPT;
    w[m] = i < n ? ld64(src + i) : pack(0.0f, e);
  }
  bool fresh = true;
#pragma unroll
  for (int m = 0; m < MAXW; ++m) fresh &= (unsigned)(w[m] >> 32) == e;
  bool ok = true;
  if (fresh) {
#pragma unroll
    for (int m = 0; m < MAXW; ++m) {
      const int i = threadIdx.x + m * kPT;
      if (i < n) dst[i] = __uint_as_float((unsigned)w[m]);
    }
  } else {
    ok = gather_slow(src, n, e, dst, abort_flag, MAXW);
  }
  if (!ok) *s_stop = 1;
  __syncthreads();
  const bool stop = *s_stop != 0;
  return !stop;
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glob_void_t;

// Asynchronous copy of nchunks 16-byte chunks (nchunks % 64 == 0) from global
// memory into LDS, chunk f -> lds[f], without passing through registers.  The
// data is in LDS once this thread's earlier loads have completed (vmcnt) and
// the workgroup has synchronised.
__device__ __forceinline__ void lds_prefetch(const uint4* src, uint4* lds, int nchunks) {
  const int lane = threadIdx.x & 63;
  for (int m = 0; m * kPT < nchunks; ++m) {
    const int f0 = (threadIdx.x - lane) + m * kPT;  // first chunk of this wave's batch
    if (f0 < nchunks)
      __builtin_amdgcn_global_load_lds((glob_void_t*)(src + f0 + lane), (lds_void_t*)(lds + f0), 16, 0, 0);
  }
}

// ---------------------------------------------------------------------------
// compute phases.  One wave per SIMD: nothing hides latency, so every
// cross-lane step uses DPP, every reduction crosses waves at most once, and
// every operand that does not depend on the token is already in registers or
// LDS when its phase starts.
// ---------------------------------------------------------------------------

// v_writelane (put the wave-uniform v into lane L of r) through the compiler's
// intrinsic rather than inline asm, so that the wait states gfx950 needs
// between a VALU write of an SGPR (the ballot's compare) and a VALU read of
// it are inserted by the compiler
extern "C" __device__ int dfssm_writelane_i32(int v, int lane_sel, int old) __asm("llvm.amdgcn.writelane.i32");
template <int L>
__device__ __forceinline__ void write_lane(uint32_t& r, uint32_t v) {
  r = (uint32_t)dfssm_writelane_i32((int)v, L, (int)r);
}

// plane words b of the two 32-input halves covered by one wave-wide ballot,
// placed in lanes b and 8 + b of pw
template <int B>
__device__ __forceinline__ void put_plane_pair(uint32_t& pw, int qi) {
  const uint64_t mk = __ballot((qi >> B) & 1);
  write_lane<B>(pw, (uint32_t)mk);
  write_lane<8 + B>(pw, (uint32_t)(mk >> 32));
}

// RMSNorm of x[0..n) (LDS) with the norm weight in registers (thread t holds
// w[t + kPT*m]), then per-token int8 quantisation: q to qs (LDS bytes) and its
// 8 two's-complement bit planes to planes (LDS, [n/32][8] words).  With
// p = x*w and u = rstd*p, max|u| = rstd*max|p| exactly (rounding is monotone),
// so the sum of squares and max|p| share one cross-wave round.  Returns s.
template <int MW>
__device__ float p_norm_quant(const float* xs, const float (&wr)[MW], int n, float eps, int8_t* qs,
                              uint32_t* planes, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float p[MW];
  float ss = 0.0f, pm = 0.0f;
#pragma unroll
  for (int m = 0; m < MW; ++m) {
    const int i = threadIdx.x + m * kPT;
    const float x = i < n ? xs[i] : 0.0f;
    p[m] = x * wr[m];
    ss += x * x;
    pm = fmaxf(pm, fabsf(p[m]));
  }
  ss = wave_sum(ss);
  pm = wave_max(pm);
  if (lane == 0) {
    red[wave] = ss;
    red[kPW + wave] = pm;
  }
  __syncthreads();
  float tss = 0.0f, tpm = 0.0f;
#pragma unroll
  for (int v = 0; v < kPW; ++v) {
    tss += red[v];
    tpm = fmaxf(tpm, red[kPW + v]);
  }
  const float rstd = 1.0f / sqrtf(tss / (float)n + eps);
  const float amax = rstd * tpm;
  const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
#pragma unroll
  for (int m = 0; m < MW; ++m) {
    const int i0 = m * kPT + wave * 64;  // this wave's 64 consecutive inputs for this m
    if (i0 < n) {                        // uniform per wave
      const float u = rstd * p[m];
      float rq = rintf(u * inv);
      rq = fminf(fmaxf(rq, -127.0f), 127.0f);
      const int qi = (int)rq;
      qs[i0 + lane] = (int8_t)qi;
      // the 16 plane words of these 64 inputs (word i0/32 planes 0..7, word i0/32 + 1 planes 0..7)
      // collected into lanes 0..15 of one register, then stored by those lanes at once
      uint32_t pw = 0;
      put_plane_pair<0>(pw, qi);
      put_plane_pair<1>(pw, qi);
      put_plane_pair<2>(pw, qi);
      put_plane_pair<3>(pw, qi);
      put_plane_pair<4>(pw, qi);
      put_plane_pair<5>(pw, qi);
      put_plane_pair<6>(pw, qi);
      put_plane_pair<7>(pw, qi);
      if (lane < 16) planes[(i0 >> 5) * 8 + lane] = pw;
    }
  }
  __syncthreads();
  return amax > 0.0f ? amax / 127.0f : 0.0f;
}

// LoRA down-projection, rank 16, A staged in LDS as 16-byte chunks (C = n/16
// per row).  16 lanes per row: thread t takes row k = t/16 and chunks
// c = t%16 + 16*m, sums them locally, then a 16-lane DPP reduction.
// tout[k] = float(sum_i A[k][i] q_i) * sA[k] * s;  sA_row = sA[t/16].
template <int MC>
__device__ void p_lora_down(const uint4* alds, int n, const int8_t* qs, float sA_row, float s, float* tout) {
  const int k = threadIdx.x >> 4, c0 = threadIdx.x & 15;
  const int C = n >> 4;
  const uint4* q4 = (const uint4*)qs;
  const uint4* ar = alds + (size_t)k * C;
  int acc = 0;
#pragma unroll
  for (int m = 0; m < MC; ++m) {
    const int c = c0 + 16 * m;
    if (c < C) {
      const uint4 av = ar[c], q = q4[c];
      acc = __builtin_amdgcn_sdot4((int)av.x, (int)q.x, acc, false);
      acc = __builtin_amdgcn_sdot4((int)av.y, (int)q.y, acc, false);
      acc = __builtin_amdgcn_sdot4((int)av.z, (int)q.z, acc, false);
      acc = __builtin_amdgcn_sdot4((int)av.w, (int)q.w, acc, false);
    }
  }
  acc = group_sum_i(acc, 16);
  if (c0 == 0) tout[k] = (float)acc * sA_row * s;
  __syncthreads();
}

// sum of q over the +1 weights of four packed words (w), from the 32 plane
// words of those inputs (pl: [4 words][8 planes])
__device__ __forceinline__ int p_plane_dot(const uint4 w, const uint32_t (&pl)[32]) {
  int pos = 0;
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    uint32_t v = __builtin_popcount(w.x & pl[b]);
    v += __builtin_popcount(w.y & pl[8 + b]);
    v += __builtin_popcount(w.z & pl[16 + b]);
    v += __builtin_popcount(w.w & pl[24 + b]);
    pos += b < 7 ? (int)(v << b) : -(int)(v << 7);
  }
  return pos;
}

// sum of q over the 128 inputs whose planes are pl
__device__ __forceinline__ int p_plane_sum(const uint32_t (&pl)[32]) {
  int q = 0;
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const uint32_t v = __builtin_popcount(pl[b]) + __builtin_popcount(pl[8 + b]) + __builtin_popcount(pl[16 + b]) +
                       __builtin_popcount(pl[24 + b]);
    q += b < 7 ? (int)(v << b) : -(int)(v << 7);
  }
  return q;
}

__device__ __forceinline__ void load_planes(const uint32_t* planes, int j, uint32_t (&pl)[32]) {
  const uint4* p4 = (const uint4*)(planes + j * 32);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint4 v = p4[k];
    pl[4 * k + 0] = v.x;
    pl[4 * k + 1] = v.y;
    pl[4 * k + 2] = v.z;
    pl[4 * k + 3] = v.w;
  }
}

__device__ __forceinline__ float lora_up(const uint4 b, const float* t) {
  // sum_k B[k] t[k] over the 16 int8 of one LoRA up row, k in order
  const uint32_t wv[4] = {b.x, b.y, b.z, b.w};
  float lo = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) lo += (float)(int8_t)(wv[k >> 2] >> (8 * (k & 3))) * t[k];
  return lo;
}

// (value, index) argmax over the wave, larger value first, then lower index
__device__ __forceinline__ void argmax_step(float& best, int& idx, float ob, int oi) {
  if (ob > best || (ob == best && oi < idx)) {
    best = ob;
    idx = oi;
  }
}
template <int CTRL>
__device__ __forceinline__ void argmax_dpp(float& best, int& idx) {
  const float ob = dpp_f<CTRL>(best);
  const int oi = dpp_i<CTRL>(idx);
  argmax_step(best, idx, ob, oi);
}
__device__ __forceinline__ void wave_argmax(float& best, int& idx) {
  argmax_dpp<kDppQuadSwap1>(best, idx);
  argmax_dpp<kDppQuadSwap2>(best, idx);
  argmax_dpp<kDppRowHalfMirror>(best, idx);
  argmax_dpp<kDppRowMirror>(best, idx);
  float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(best), 0));
  int ix = __builtin_amdgcn_readlane(idx, 0);
#pragma unroll
  for (int r = 16; r < 64; r += 16)
    argmax_step(b, ix, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(best), r)),
                __builtin_amdgcn_readlane(idx, r));
  best = b;
  idx = ix;
}

// ---------------------------------------------------------------------------
// the kernel, compiled for each supported model shape so that lane layouts,
// row counts and weight offsets are constants (no per-layer pointer tables,
// little index arithmetic, few scalar registers)
// ---------------------------------------------------------------------------

constexpr int kMaxInRows = 40;  // in_proj rows per workgroup (z 16, x 16, dt, B/C)

template <int DM_, int DI_, int NS_, int HP_>
struct PShape {
  static constexpr int DM = DM_, DI = DI_, NS = NS_, HP = HP_;
  static constexpr int H = DI / HP, G = H * (HP / 16), CDIM = DI + 2 * NS, DPROJ = 2 * DI + 2 * NS + H;
  static constexpr int NBC = 2 * NS / G;  // B/C rows per workgroup
  static constexpr int NROWS = 33 + NBC;  // z 16, x 16, dt 1, B/C
  static constexpr int OUT_PER = DM / G;
  static constexpr int UI = DM / 128, RPPI = 64 / UI, NGI_T = (NROWS + RPPI - 1) / RPPI, NGI = (NGI_T + kPW - 1) / kPW;
  static constexpr int UO = DI / 128, RPPO = 64 / UO, NGO_T = (OUT_PER + RPPO - 1) / RPPO,
                       NGO = (NGO_T + kPW - 1) / kPW;
  static constexpr int MW1 = DM / kPT, MW2 = DI / kPT;
  static constexpr int MC1 = (DM / 16 + 15) / 16, MC2 = (DI / 16 + 15) / 16;
  static constexpr int NST = (NS + 63) / 64;
  static constexpr int CH = DM / 16, LH = CH < 64 ? CH : 64, MH = CH / LH, RPPH = 64 / LH, STEPH = kPW * RPPH;
  // one layer's tensors in kind order, each 256-byte aligned (the runtime's weight layout)
  static constexpr size_t SZ(int k) {
    return k == 0 ? (size_t)DPROJ * DM / 8 : k == 1 ? (size_t)DPROJ * 4 : k == 2 ? (size_t)16 * DM : k == 3 ? 64
         : k == 4 ? (size_t)DPROJ * 16 : k == 5 ? (size_t)DPROJ * 4 : k == 6 ? (size_t)DM * DI / 8
         : k == 7 ? (size_t)DM * 4 : k == 8 ? (size_t)16 * DI : k == 9 ? 64 : k == 10 ? (size_t)DM * 16
         : k == 11 ? (size_t)DM * 4 : k == 12 ? (size_t)CDIM * 16 : k == 13 ? (size_t)CDIM * 4
         : k <= 16 ? (size_t)H * 4 : k == 17 ? (size_t)DM * 4 : (size_t)DI * 4;
  }
  static constexpr size_t OFF(int k) {
    size_t o = 0;
    for (int i = 0; i < k; ++i) o += (SZ(i) + 255) / 256 * 256;
    return o;
  }
  static constexpr size_t LSTRIDE = OFF(19);
  static_assert(2 * NS % G == 0 && DM % G == 0 && DM % kPT == 0 && DI % kPT == 0, "unsupported shape");
  static_assert(NROWS <= kMaxInRows, "too many in_proj rows per workgroup");
};

constexpr int kHeadDepth = 8;  // LM-head rows in flight per wave
static_assert(kPT == 256 && kPW == 4, "one wave per 4 state channels and 16 lanes per LoRA rank row");

template <class S>
__global__ __launch_bounds__(kPT, 1) void decode_persistent_kernel(PersistArgs a) {
  extern __shared__ unsigned char smem[];
  constexpr int DM = S::DM, DI = S::DI, NS = S::NS, HP = S::HP, G = S::G, CDIM = S::CDIM;
  constexpr int MX = DM > DI ? DM : DI;
  const int w = blockIdx.x;
  const int hd = w / (HP / 16), j = w % (HP / 16);

  // LDS carve-up
  float* hs = (float*)smem;                     // [DM] residual stream
  float* gs = hs + DM;                          // [DI] gated SSM output (all heads); also argmax candidates
  int8_t* qs = (int8_t*)(gs + DI);              // [MX] int8 codes
  uint32_t* pl = (uint32_t*)(qs + MX);          // [MX/32][8] bit planes
  float* bcs = (float*)(pl + (MX / 32) * 8);    // [2NS] B, C
  float* tls = bcs + 2 * NS;                    // [16] LoRA down vector
  float* rowv = tls + 16;                       // [kMaxInRows] outputs of own in_proj rows
  float* red = rowv + kMaxInRows;               // [2*kPW]
  int* s_stop = (int*)(red + 2 * kPW);          // [1]
  int* s_tok = s_stop + 1;                      // [1]
  float* s_arg = (float*)(s_tok + 2);           // [2*kPW]
  uint4* ains = (uint4*)(((uintptr_t)(s_arg + 2 * kPW) + 15) & ~(uintptr_t)15);  // [16 * DM/16] LoRA-down A, in_proj
  uint4* aouts = ains + 16 * (DM / 16);         // [16 * DI/16] LoRA-down A, out_proj
  if (threadIdx.x == 0) *s_stop = 0;
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  unsigned e = a.epoch0;  // same value in every workgroup
  int tok = a.tok_in[0];
  const char* wb = a.wbase;

  auto in_row = [&](int k) -> int {
    if (k < 16) return hd * HP + j * 16 + k;                 // z
    if (k < 32) return DI + hd * HP + j * 16 + (k - 16);     // x
    if (k == 32) return 2 * DI + 2 * NS + hd;                // dt
    return 2 * DI + (w + (k - 33) * G);                      // B/C
  };

  const int ji = lane & (S::UI - 1), subi = lane / S::UI;
  const bool lead_i = lane == group_sum_lane(subi * S::UI, S::UI);
  const int jo = lane & (S::UO - 1), subo = lane / S::UO;
  const bool lead_o = lane == group_sum_lane(subo * S::UO, S::UO);
  const bool conv_thread = threadIdx.x < 16 + S::NBC;
  const int conv_k = threadIdx.x < 16 ? 16 + threadIdx.x : 33 + (threadIdx.x - 16);
  const int conv_c = conv_thread ? in_row(conv_k) - DI : 0;

  // ---- registers prefetched for phase A (in_proj) of a layer
  uint4 win[S::NGI];
  float nw[S::MW1];
  float isw[S::NGI], isb[S::NGI];
  uint4 ib[S::NGI];
  float cw[4], cb, cst[3];
  float sAi;
  // ---- registers prefetched for phases S and B (SSM, out_proj) of a layer
  uint4 wout[S::NGO];
  float gw[S::MW2];
  float osw[S::NGO], osb[S::NGO];
  uint4 ob[S::NGO];
  float4 st[S::NST];  // state float4 (n = lane + 64 m, channels 4*wave ..) of the block [NS][16]
  float dtb, alog, dval;
  float sAo;

  auto lp = [&](int l, int k) -> const char* { return wb + (size_t)l * S::LSTRIDE + S::OFF(k); };

  auto load_A = [&](int l) {
    const uint4* b4 = (const uint4*)lp(l, DFSSM_PK_IN_BITS);
    const float* sw = (const float*)lp(l, DFSSM_PK_IN_SW);
    const float* sb = (const float*)lp(l, DFSSM_PK_IN_SB);
    const int8_t* bm = (const int8_t*)lp(l, DFSSM_PK_IN_B);
#pragma unroll
    for (int m = 0; m < S::NGI; ++m) {
      const int g = wave + m * kPW;
      const int k = g * S::RPPI + subi;
      const bool live = g < S::NGI_T && k < S::NROWS;
      const int row = live ? in_row(k) : 0;
      win[m] = live ? b4[(size_t)row * S::UI + ji] : make_uint4(0, 0, 0, 0);
      const bool lead = live && lead_i;
      isw[m] = lead ? sw[row] : 0.0f;
      isb[m] = lead ? sb[row] : 0.0f;
      ib[m] = lead ? *(const uint4*)(bm + (size_t)row * 16) : make_uint4(0, 0, 0, 0);
    }
    const float* nwp = (const float*)lp(l, DFSSM_PK_NORM_W);
#pragma unroll
    for (int m = 0; m < S::MW1; ++m) nw[m] = nwp[threadIdx.x + m * kPT];
    lds_prefetch((const uint4*)lp(l, DFSSM_PK_IN_A), ains, 16 * (DM / 16));
    sAi = ((const float*)lp(l, DFSSM_PK_IN_SA))[threadIdx.x >> 4];
    if (conv_thread) {
      const float* wc = (const float*)lp(l, DFSSM_PK_CONV_W) + (size_t)conv_c * 4;
      cw[0] = wc[0]; cw[1] = wc[1]; cw[2] = wc[2]; cw[3] = wc[3];
      cb = ((const float*)lp(l, DFSSM_PK_CONV_B))[conv_c];
      const float* cs = a.conv + (size_t)l * 3 * CDIM;
      cst[0] = cs[conv_c]; cst[1] = cs[CDIM + conv_c]; cst[2] = cs[2 * CDIM + conv_c];
    }
  };
  auto load_B = [&](int l) {
    const uint4* b4 = (const uint4*)lp(l, DFSSM_PK_OUT_BITS);
    const float* sw = (const float*)lp(l, DFSSM_PK_OUT_SW);
    const float* sb = (const float*)lp(l, DFSSM_PK_OUT_SB);
    const int8_t* bm = (const int8_t*)lp(l, DFSSM_PK_OUT_B);
#pragma unroll
    for (int m = 0; m < S::NGO; ++m) {
      const int g = wave + m * kPW;
      const int k = g * S::RPPO + subo;
      const bool live = g < S::NGO_T && k < S::OUT_PER;
      const int row = w * S::OUT_PER + k;
      wout[m] = live ? b4[(size_t)row * S::UO + jo] : make_uint4(0, 0, 0, 0);
      const bool lead = live && lead_o;
      osw[m] = lead ? sw[row] : 0.0f;
      osb[m] = lead ? sb[row] : 0.0f;
      ob[m] = lead ? *(const uint4*)(bm + (size_t)row * 16) : make_uint4(0, 0, 0, 0);
    }
    const float* gwp = (const float*)lp(l, DFSSM_PK_GNORM_W);
#pragma unroll
    for (int m = 0; m < S::MW2; ++m) gw[m] = gwp[threadIdx.x + m * kPT];
    lds_prefetch((const uint4*)lp(l, DFSSM_PK_OUT_A), aouts, 16 * (DI / 16));
    sAo = ((const float*)lp(l, DFSSM_PK_OUT_SA))[threadIdx.x >> 4];
    const float4* s4 = (const float4*)(a.ssm + (size_t)l * S::H * HP * NS + (size_t)w * NS * 16);
#pragma unroll
    for (int m = 0; m < S::NST; ++m) {
      const int n = lane + 64 * m;
      st[m] = n < NS ? s4[n * 4 + wave] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    dtb = ((const float*)lp(l, DFSSM_PK_DT_BIAS))[hd];
    alog = ((const float*)lp(l, DFSSM_PK_A_LOG))[hd];
    dval = ((const float*)lp(l, DFSSM_PK_D))[hd];
  };

  // phase timestamps (100 MHz device clock) for performance analysis
  auto prof = [&](int t, int l, int ev) {
    if (a.prof && t < a.prof_tokens && threadIdx.x == 0)
      a.prof[(((size_t)t * (a.n_layer + 1) + l) * G + w) * kProfEvents + ev] = wall_clock64();
  };

  load_A(0);
  load_B(0);
  const int T = a.n_tokens;
  const int Lm = a.n_layer;
  bool ok = true;
  for (int t = 0; t < T && ok; ++t) {
    // ---- embedding (every workgroup, no hop)
    {
      int tk = tok;
      if (tk < 0 || tk >= a.vocab) {
        if (threadIdx.x == 0 && w == 0) atomicOr(a.err, 1);
        tk = 0;
      }
      const float sc = a.sE[tk];
#pragma unroll
      for (int m = 0; m < S::MW1; ++m) {
        const int i = threadIdx.x + m * kPT;
        hs[i] = (float)a.E[(size_t)tk * DM + i] * sc;
      }
      __syncthreads();
    }
    for (int l = 0; l < Lm && ok; ++l) {
      prof(t, l, 0);
      if (l > 0) {
        ok = gather<S::MW1>(a.hbox, DM, e, hs, a.abort_flag, s_stop);
        ++e;
        if (!ok) break;
      }
      prof(t, l, 1);
      if (a.trace_h && w == 0)
        for (int i = threadIdx.x; i < DM; i += kPT) a.trace_h[(size_t)l * DM + i] = hs[i];
      // ---- phase A: norm, quantise, LoRA down, 1-bit GEMV of own rows, conv
      const float s1 = p_norm_quant<S::MW1>(hs, nw, DM, a.eps, qs, pl, red);
      prof(t, l, 2);
      if (a.trace_q1 && w == 0)
        for (int i = threadIdx.x; i < DM; i += kPT) a.trace_q1[(size_t)l * DM + i] = qs[i];
      p_lora_down<S::MC1>(ains, DM, qs, sAi, s1, tls);
      prof(t, l, 3);
      {
        uint32_t plw[32];
        load_planes(pl, ji, plw);
        const int qpart = p_plane_sum(plw);
#pragma unroll
        for (int m = 0; m < S::NGI; ++m) {
          const int g = wave + m * kPW;
          if (g < S::NGI_T) {  // uniform per wave
            const int acc = group_sum_i(2 * p_plane_dot(win[m], plw) - qpart, S::UI);
            const int k = g * S::RPPI + subi;
            if (lead_i && k < S::NROWS) rowv[k] = (float)acc * isw[m] * s1 + isb[m] * lora_up(ib[m], tls);
          }
        }
      }
      __syncthreads();
      prof(t, l, 4);
      if (conv_thread) {
        const float y = rowv[conv_k];
        const float v = cb + cw[0] * cst[0] + cw[1] * cst[1] + cw[2] * cst[2] + cw[3] * y;
        const float xv = silu_f(v);
        rowv[conv_k] = xv;
        if (conv_k >= 33) publish(a.bcbox, 2 * NS, conv_c - DI, xv, e);
        cst[0] = cst[1];  // shifted window, written back after the next hop
        cst[1] = cst[2];
        cst[2] = y;
      }
      prof(t, l, 5);
      // keep this layer's new conv window: load_A below refills cst for the next layer
      float cst_prev[3] = {cst[0], cst[1], cst[2]};
      // the next layer's phase-A operands stream in during the two hops below
      // (after the last layer: layer 0 of the next token)
      load_A(l + 1 < Lm ? l + 1 : 0);
      ok = gather<(2 * NS + kPT - 1) / kPT>(a.bcbox, 2 * NS, e, bcs, a.abort_flag, s_stop);
      ++e;
      if (!ok) break;
      prof(t, l, 6);
      // stores go out after the hop: a hop's polling load waits for every earlier memory operation
      if (conv_thread) {
        float* cs = a.conv + (size_t)l * 3 * CDIM;
        cs[conv_c] = cst_prev[0];
        cs[CDIM + conv_c] = cst_prev[1];
        cs[2 * CDIM + conv_c] = cst_prev[2];
      }
      // ---- phase S: SSM on the state block [hd][j*16 .. +16][0 .. NS), gate.
      // Wave v owns channels 4v .. 4v+3, its lanes the state rows n = lane + 64 m.
      {
        const float dt = softplus_f(rowv[32] + dtb);
        const float dA = __expf(-dt * __expf(alog));
        const float* xr = rowv + 16 + wave * 4;
        const float x0 = dt * xr[0], x1 = dt * xr[1], x2 = dt * xr[2], x3 = dt * xr[3];
        float y0 = 0.f, y1 = 0.f, y2 = 0.f, y3 = 0.f;
#pragma unroll
        for (int m = 0; m < S::NST; ++m) {
          const int n = lane + 64 * m;
          if (n < NS) {
            const float bn = bcs[n], cn = bcs[NS + n];
            float4 v = st[m];
            v.x = v.x * dA + x0 * bn;
            v.y = v.y * dA + x1 * bn;
            v.z = v.z * dA + x2 * bn;
            v.w = v.w * dA + x3 * bn;
            st[m] = v;
            y0 += v.x * cn;
            y1 += v.y * cn;
            y2 += v.z * cn;
            y3 += v.w * cn;
          }
        }
        y0 = wave_sum(y0);
        y1 = wave_sum(y1);
        y2 = wave_sum(y2);
        y3 = wave_sum(y3);
        if (lane < 4) {
          const int c = wave * 4 + lane;  // channel within the slice
          const float y = (lane == 0 ? y0 : lane == 1 ? y1 : lane == 2 ? y2 : y3) + dval * rowv[16 + c];
          const float g = y * silu_f(rowv[c]);
          publish(a.gbox, DI, hd * HP + j * 16 + c, g, e);
        }
      }
      prof(t, l, 7);
      ok = gather<S::MW2>(a.gbox, DI, e, gs, a.abort_flag, s_stop);
      ++e;
      if (!ok) break;
      prof(t, l, 8);
      {
        float4* s4 = (float4*)(a.ssm + (size_t)l * S::H * HP * NS + (size_t)w * NS * 16);
#pragma unroll
        for (int m = 0; m < S::NST; ++m) {
          const int n = lane + 64 * m;
          if (n < NS) s4[n * 4 + wave] = st[m];
        }
      }
      // ---- phase B: gated norm, quantise, LoRA down, 1-bit GEMV of own rows, residual
      {
        const float s2 = p_norm_quant<S::MW2>(gs, gw, DI, a.eps, qs, pl, red);
        if (a.trace_q2 && w == 0)
          for (int i = threadIdx.x; i < DI; i += kPT) a.trace_q2[(size_t)l * DI + i] = qs[i];
        p_lora_down<S::MC2>(aouts, DI, qs, sAo, s2, tls);
        uint32_t plw[32];
        load_planes(pl, jo, plw);
        const int qpart = p_plane_sum(plw);
#pragma unroll
        for (int m = 0; m < S::NGO; ++m) {
          const int g = wave + m * kPW;
          if (g < S::NGO_T) {
            const int acc = group_sum_i(2 * p_plane_dot(wout[m], plw) - qpart, S::UO);
            const int k = g * S::RPPO + subo;
            if (lead_o && k < S::OUT_PER) {
              const int row = w * S::OUT_PER + k;
              const float y = (float)acc * osw[m] * s2 + osb[m] * lora_up(ob[m], tls);
              publish(a.hbox, DM, row, hs[row] + y, e);
            }
          }
        }
      }
      prof(t, l, 9);
      load_B(l + 1 < Lm ? l + 1 : 0);
      __syncthreads();
    }
    if (!ok) break;
    // ---- final norm + LM head + argmax
    prof(t, Lm, 0);
    constexpr int LH = S::LH, MH = S::MH, RPPH = S::RPPH, STEPH = S::STEPH;
    const int rows_per = (a.vocab + G - 1) / G;
    const int r0 = w * rows_per;
    const int r1 = min(a.vocab, r0 + rows_per);
    const int jh = lane & (LH - 1), subh = lane / LH;
    const bool lead_h = lane == group_sum_lane(subh * LH, LH);
    float fn[S::MW1];
#pragma unroll
    for (int m = 0; m < S::MW1; ++m) fn[m] = a.final_norm[threadIdx.x + m * kPT];
    uint4 eb[kHeadDepth][MH];
    int erow[kHeadDepth];
#pragma unroll
    for (int d = 0; d < kHeadDepth; ++d) {
      const int row = r0 + wave * RPPH + d * STEPH + subh;
      erow[d] = row;
      const uint4* e4 = (const uint4*)(a.E + (size_t)(row < r1 ? row : 0) * DM);
#pragma unroll
      for (int c = 0; c < MH; ++c) eb[d][c] = row < r1 ? e4[jh + c * LH] : make_uint4(0, 0, 0, 0);
    }
    ok = gather<S::MW1>(a.hbox, DM, e, hs, a.abort_flag, s_stop);
    ++e;
    if (!ok) break;
    prof(t, Lm, 1);
    if (a.trace_h && w == 0)
      for (int i = threadIdx.x; i < DM; i += kPT) a.trace_h[(size_t)Lm * DM + i] = hs[i];
    const float sf = p_norm_quant<S::MW1>(hs, fn, DM, a.eps, qs, pl, red);
    prof(t, Lm, 2);
    if (a.trace_qf && w == 0)
      for (int i = threadIdx.x; i < DM; i += kPT) a.trace_qf[i] = qs[i];
    {
      const uint4* q4 = (const uint4*)qs;
      uint4 qv[MH];
#pragma unroll
      for (int c = 0; c < MH; ++c) qv[c] = q4[jh + c * LH];
      float best = -__builtin_huge_valf();
      int bidx = 0x7fffffff;
      for (int base = 0; base < rows_per; base += kHeadDepth * STEPH) {
#pragma unroll
        for (int d = 0; d < kHeadDepth; ++d) {
          const int row = erow[d];
          int acc = 0;
#pragma unroll
          for (int c = 0; c < MH; ++c) {
            acc = __builtin_amdgcn_sdot4((int)eb[d][c].x, (int)qv[c].x, acc, false);
            acc = __builtin_amdgcn_sdot4((int)eb[d][c].y, (int)qv[c].y, acc, false);
            acc = __builtin_amdgcn_sdot4((int)eb[d][c].z, (int)qv[c].z, acc, false);
            acc = __builtin_amdgcn_sdot4((int)eb[d][c].w, (int)qv[c].w, acc, false);
          }
          acc = group_sum_i(acc, LH);
          if (lead_h && row < r1) {
            const float lg = (float)acc * a.sE[row] * sf;
            a.logits[row] = lg;
            argmax_step(best, bidx, lg, row);
          }
          // refill this slot with the row kHeadDepth iterations ahead
          const int nrow = row + kHeadDepth * STEPH;
          erow[d] = nrow;
          const uint4* e4 = (const uint4*)(a.E + (size_t)(nrow < r1 ? nrow : 0) * DM);
#pragma unroll
          for (int c = 0; c < MH; ++c) eb[d][c] = nrow < r1 ? e4[jh + c * LH] : make_uint4(0, 0, 0, 0);
        }
      }
      wave_argmax(best, bidx);
      if (lane == 0) {
        s_arg[wave] = best;
        ((int*)s_arg)[kPW + wave] = bidx;
      }
      __syncthreads();
      if (threadIdx.x == 0) {
        for (int wv = 1; wv < kPW; ++wv) argmax_step(best, bidx, s_arg[wv], ((int*)s_arg)[kPW + wv]);
        // argmax candidates: value word and index word per workgroup
        publish(a.abox, 2 * G, w, best, e);
        publish(a.abox, 2 * G, G + w, __int_as_float(bidx), e);
      }
    }
    prof(t, Lm, 3);
    // every workgroup reduces the G candidates itself
    {
      float* cand = gs;
      ok = gather<(2 * G + kPT - 1) / kPT>(a.abox, 2 * G, e, cand, a.abort_flag, s_stop);
      ++e;
      if (!ok) break;
      if (wave == 0) {
        float best = -__builtin_huge_valf();
        int bidx = 0x7fffffff;
        for (int q = lane; q < G; q += 64) argmax_step(best, bidx, cand[q], __float_as_int(cand[G + q]));
        wave_argmax(best, bidx);
        if (lane == 0) {
          if (bidx == 0x7fffffff) bidx = 0;
          *s_tok = bidx;
          if (w == 0 && a.tok_out) a.tok_out[t] = bidx;
        }
      }
      __syncthreads();
      tok = *s_tok;
      prof(t, Lm, 4);
    }
  }
  if (w == 0 && threadIdx.x == 0) {
    if (ok) {
      if (a.tok_last) a.tok_last[0] = tok;
    } else {
      atomicOr(a.err, 2);
    }
  }
}

// the shapes this kernel is compiled for: the 2-layer test stack and the 1.3B shape
using ShapeTiny = PShape<256, 512, 16, 32>;
using Shape1p3b = PShape<2048, 4096, 128, 64>;

static size_t lds_bytes(int dm, int di, int ns) {
  const int mx = dm > di ? dm : di;
  return (size_t)dm * 4 + (size_t)di * 4 + (size_t)mx + (size_t)(mx / 32) * 8 * 4 + (size_t)2 * ns * 4 + 16 * 4 +
         kMaxInRows * 4 + 2 * kPW * 4 + 16 + 2 * kPW * 4 + 16 + (size_t)16 * (dm + di);
}

template <class S>
static const void* kernel_of() { return (const void*)decode_persistent_kernel<S>; }

template <class S>
static bool shape_is(int dm, int di, int ns, int hp) {
  return dm == S::DM && di == S::DI && ns == S::NS && hp == S::HP;
}

static const void* select_kernel(int dm, int di, int ns, int hp, size_t* stride, const size_t** /*unused*/) {
  if (shape_is<Shape1p3b>(dm, di, ns, hp)) { *stride = Shape1p3b::LSTRIDE; return kernel_of<Shape1p3b>(); }
  if (shape_is<ShapeTiny>(dm, di, ns, hp)) { *stride = ShapeTiny::LSTRIDE; return kernel_of<ShapeTiny>(); }
  return nullptr;
}

template <class S>
static size_t off_of(int k) { return S::OFF(k); }

bool persistent_layout(int d_model, int d_inner, int d_state, int headdim, size_t* stride, size_t* offsets) {
  size_t st = 0;
  if (!select_kernel(d_model, d_inner, d_state, headdim, &st, nullptr)) return false;
  *stride = st;
  for (int k = 0; k < 19; ++k)
    offsets[k] = shape_is<Shape1p3b>(d_model, d_inner, d_state, headdim) ? off_of<Shape1p3b>(k) : off_of<ShapeTiny>(k);
  return true;
}

hipError_t launch_decode_persistent(const PersistArgs& a, int grid, hipStream_t st) {
  size_t stride = 0;
  const void* k = select_kernel(a.d_model, a.d_inner, a.d_state, a.headdim, &stride, nullptr);
  if (!k) return hipErrorInvalidValue;
  PersistArgs args = a;
  void* params[] = {&args};
  return hipLaunchCooperativeKernel(k, dim3(grid), dim3(kPT), params,
                                    (unsigned)lds_bytes(a.d_model, a.d_inner, a.d_state), st);
}

// Whether the persistent kernel can run for these dimensions with `grid`
// co-resident workgroups on this device.  Fills *why on refusal.
bool persistent_supported(int d_model, int d_inner, int d_state, int headdim, int n_heads, int rank, int grid,
                          const char** why) {
  auto no = [&](const char* m) { *why = m; return false; };
  size_t stride = 0;
  const void* k = select_kernel(d_model, d_inner, d_state, headdim, &stride, nullptr);
  if (!k) return no("the persistent kernel is compiled for d_model/d_inner/d_state/headdim 2048/4096/128/64 and 256/512/16/32");
  if (grid != n_heads * (headdim / 16)) return no("grid mismatch");
  if (rank != 16) return no("the persistent path needs LoRA rank 16");
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return no("no device");
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return no("no CU count");
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, kPT, lds_bytes(d_model, d_inner, d_state)) != hipSuccess)
    return no("occupancy query failed");
  if ((long)per_cu * cus < grid) return no("grid does not fit co-resident on this device");
  return true;
}

size_t persistent_box_words(int d_model, int d_inner, int d_state, int grid) {
  return (size_t)kR * ((size_t)d_model + (size_t)d_inner + 2 * (size_t)d_state + 2 * (size_t)grid);
}

}  // namespace dfssm
