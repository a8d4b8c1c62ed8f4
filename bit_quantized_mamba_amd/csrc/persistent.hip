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
// Waves: a workgroup has 4 compute waves and 4 loader waves (one of each per
// SIMD).  The loader waves bring in every weight and state a layer needs
// (staged in LDS for the compute waves, or kept in their own registers for
// the LoRA down-projections they compute), so the compute waves' instruction
// streams and polls never wait behind weight traffic.
// Hops: values crossing workgroups travel in 64-bit words written with a
// relaxed device-scope atomic store into R = 4 replicas (replica r read by
// the workgroups with w % 4 == r, which spreads the readers of a line; 4
// measured faster per token than 1, 2, 8 or 16); readers poll with relaxed
// device-scope atomic loads until the word is fresh.  The small boxes (B/C,
// argmax) carry {fp32 bits, epoch}, every hop instance with its own epoch.
// The residual and gated-output boxes carry two values per word with a
// 2-bit write-count tag in their lowest mantissa bits (pack2; readers clear
// them), which halves the bytes every workgroup reads at those hops.  Freshness travels in the
// same single-copy-atomic word as the data, so no fence or flag ordering is
// involved.  Each box is reused once per layer; a writer can only reach its
// next use after every reader has passed the hop that follows this one, so
// one buffer per box suffices.
// Every wait is bounded: a workgroup that polls too long sets a device abort
// flag, which all waits check, so a fault ends the kernel instead of hanging.
#include "common.h"
#include "persistent.h"

#include <type_traits>

namespace dfssm {

constexpr int kPT = 256;  // compute threads per workgroup: one compute wave per SIMD
constexpr int kPW = kPT / 64;
constexpr int kLT = 256;  // loader threads (waves 4..7): the LoRA down-projections
constexpr int kBlock = kPT + kLT;
constexpr int kR = 4;     // replicas of each published word
constexpr long kSpinLimit = 1 << 21;
constexpr int kLutCopies = 16;

__device__ __forceinline__ uint64_t ld64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t pack(float v, unsigned e) { return ((uint64_t)e << 32) | __float_as_uint(v); }

// Paired words (the residual and gated-output boxes, whose per-hop volume is
// large): two fp32 values in one 64-bit word, the lowest mantissa bit of each
// carrying one bit of a 2-bit tag, the count of that box's writes mod 4.
// Every reader reads every word of its replica at every write, so by
// per-location coherence it can only see the current write or the one before,
// whose tag differs.  The host keeps the count across launches and clears the
// boxes when it cannot vouch for it.  Readers clear the tag bits (unpack2):
// every value crosses a hop with its lowest mantissa bit set to 0 (truncated
// toward zero by at most 1 ulp), the same whatever the write count, so
// results do not depend on how many tokens were decoded before, and zeros
// stay exactly zero.
constexpr uint64_t kTagMask = 0x0000000100000001ull;
__device__ __forceinline__ uint64_t tag_bits(unsigned c) {
  return (uint64_t)(c & 1u) | ((uint64_t)((c >> 1) & 1u) << 32);
}
__device__ __forceinline__ uint64_t pack2(float v0, float v1, unsigned c) {
  return ((((uint64_t)__float_as_uint(v1) << 32) | __float_as_uint(v0)) & ~kTagMask) | tag_bits(c);
}
__device__ __forceinline__ float2 unpack2(uint64_t w) {
  w &= ~kTagMask;
  return make_float2(__uint_as_float((unsigned)w), __uint_as_float((unsigned)(w >> 32)));
}

// The launch's arguments re-read from the kernel-argument segment at the point
// of use.  The pointer passes through an empty asm so the compiler cannot keep
// the loaded values live in scalar registers across the token loop: fields used
// once per token (LM head, token I/O, tracing) cost a scalar load there instead
// of occupying registers that the layer loop needs.
typedef __attribute__((address_space(4))) const PersistArgs* KArgs;
__device__ __forceinline__ KArgs kargs() {
  uint64_t v = (uint64_t)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(v));
  return (KArgs)v;
}

// Workgroup barrier that orders LDS only.  __syncthreads() also fences
// global memory, which on this target waits for every outstanding vector
// memory operation -- every prefetch in flight -- at every barrier.  No
// barrier here publishes global memory to the workgroup: values that cross
// threads go through LDS, and global data (weights, state) is prefetched into
// the registers of the thread that uses it.
__device__ __forceinline__ void wg_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ bool aborted(const int* flag) {
  return __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
}

// publish value `v` as word `i` of a box of n words (all replicas)
__device__ __forceinline__ void publish(uint64_t* box, int n, int i, float v, unsigned e) {
  const uint64_t w = pack(v, e);
#pragma unroll 1
  for (int r = 0; r < kR; ++r) st64(box + (size_t)r * n + i, w);
}

// publish values v0, v1 (entries 2i, 2i + 1) as paired word i of a box of n
// words (all replicas), write count c
__device__ __forceinline__ void publish2(uint64_t* box, int n, int i, float v0, float v1, unsigned c) {
  const uint64_t w = pack2(v0, v1, c);
#pragma unroll 1
  for (int r = 0; r < kR; ++r) st64(box + (size_t)r * n + i, w);
}

// Read words [0, n) of this workgroup's replica into LDS.  A thread issues
// all of its loads before checking any.  While some are stale it waits on the
// first stale one alone (a single poll in flight per thread keeps the polling
// traffic low while the publishers are still working), then re-issues every
// word that is still stale at once: publishers finish at nearly the same
// time, so the words missing when the first one lands arrive together and one
// parallel round picks them up.  Returns false (for every thread of the
// workgroup) on abort.
// PAIRED: paired words, fresh when their tag is tag_bits(key), two floats each
// to dst; else {value, epoch} words, fresh when the epoch is key.
template <int MAXW, bool PAIRED>
__device__ bool poll_words(const uint64_t* box, int n, unsigned key, uint64_t (&w)[MAXW], int* abort_flag) {
  const uint64_t* src = box + (size_t)(blockIdx.x % kR) * n;
  const uint64_t tb = tag_bits(key);
  auto fresh = [&](uint64_t v) { return PAIRED ? (v & kTagMask) == tb : (unsigned)(v >> 32) == key; };
#pragma unroll
  for (int m = 0; m < MAXW; ++m) {
    const int i = threadIdx.x + m * kPT;
    w[m] = i < n ? ld64(src + i) : (PAIRED ? tb : pack(0.0f, key));
  }
  bool ok = true;
  long spins = 0;
  for (;;) {
    int first = -1;
#pragma unroll
    for (int m = MAXW - 1; m >= 0; --m)
      if (!fresh(w[m])) first = m;
    if (first < 0) break;
    // wait on the first stale word
    const uint64_t* p = src + threadIdx.x + first * kPT;
    uint64_t v = ld64(p);
    while (!fresh(v)) {
      if (++spins > kSpinLimit) {
        __hip_atomic_store(abort_flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ok = false;
        break;
      }
      if ((spins & 63) == 0 && aborted(abort_flag)) {
        ok = false;
        break;
      }
      v = ld64(p);
    }
    if (!ok) break;
    // then one parallel round over every word still stale (including that one)
#pragma unroll
    for (int m = 0; m < MAXW; ++m)
      if (!fresh(w[m])) w[m] = ld64(src + threadIdx.x + m * kPT);
  }
  return ok;
}
template <int MAXW, bool PAIRED>
__device__ bool gather_words(const uint64_t* box, int n, unsigned key, float* dst, int* abort_flag, int* s_stop) {
  uint64_t w[MAXW];
  const bool ok = poll_words<MAXW, PAIRED>(box, n, key, w, abort_flag);
  if (ok) {
#pragma unroll
    for (int m = 0; m < MAXW; ++m) {
      const int i = threadIdx.x + m * kPT;
      if (i < n) {
        if (PAIRED)
          ((float2*)dst)[i] = unpack2(w[m]);
        else
          dst[i] = __uint_as_float((unsigned)w[m]);
      }
    }
  } else {
    *s_stop = 1;
  }
  wg_barrier();
  const bool stop = *s_stop != 0;
  return !stop;
}
template <int MAXW>
__device__ bool gather(const uint64_t* box, int n, unsigned e, float* dst, int* abort_flag, int* s_stop) {
  return gather_words<MAXW, false>(box, n, e, dst, abort_flag, s_stop);
}
// paired box of n words (2 n floats), write count c
template <int MAXW>
__device__ bool gather2(const uint64_t* box, int n, unsigned c, float* dst, int* abort_flag, int* s_stop) {
  return gather_words<MAXW, true>(box, n, c, dst, abort_flag, s_stop);
}

// ---------------------------------------------------------------------------
// compute phases.  One compute wave per SIMD: nothing hides latency, so every
// cross-lane step uses DPP, every reduction crosses waves at most once, and
// every operand that does not depend on the token is already in registers or
// LDS when its phase starts.
// ---------------------------------------------------------------------------

// The int8 codes sit in LDS in 16-byte chunks, chunk c at slot qchunk(c): the
// low four bits of c are XORed with bits 3..6 (a bijection that keeps every
// 16-chunk block in place).  A GEMV lane reads the 8 chunks of its 128
// inputs, so the 16 lanes of a row read chunks 8 apart; unswizzled those all
// fall in the same 2 of the 16 bank groups a 256-byte LDS row has, swizzled
// they hit 16 different ones (and 16 consecutive chunks stay conflict-free).
__device__ __forceinline__ int qchunk(int c) { return c ^ ((c >> 3) & 15); }
__device__ __forceinline__ int qbyte(int i) { return qchunk(i >> 4) * 16 + (i & 15); }
// Inputs of a thread in the norm phases: element m of thread t is input
// norm_idx(m).  With MW a multiple of 4 a thread holds runs of 4 consecutive
// inputs (one 16-byte load each, one 4-byte code store), else inputs t + 256 m.
template <int MW>
__device__ __forceinline__ int norm_idx(int m) {
  constexpr int V = MW % 4 == 0 ? 4 : 1;
  return V * ((int)threadIdx.x + kPT * (m / V)) + m % V;
}
template <int MW>
__device__ __forceinline__ void load_norm_w(float (&dst)[MW], const float* src) {
  if constexpr (MW % 4 == 0) {
#pragma unroll
    for (int m = 0; m < MW / 4; ++m) {
      const float4 v = ((const float4*)src)[threadIdx.x + kPT * m];
      dst[4 * m] = v.x;
      dst[4 * m + 1] = v.y;
      dst[4 * m + 2] = v.z;
      dst[4 * m + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int m = 0; m < MW; ++m) dst[m] = src[threadIdx.x + kPT * m];
  }
}

// RMSNorm with weight w fused with the per-token int8 quantiser over
// n = 256 MW inputs (thread layout: norm_idx).  Sum of squares and max |x w|
// cross the waves in one LDS round; since rstd > 0 scales every
// |u| = rstd |x w| alike, the absmax of u is rstd * max |x w|.  Codes go to qs
// (LDS, swizzled by qbyte); returns the scale amax / 127.
template <int MW>
__device__ float p_norm_quant(const float* xs, const float (&wr)[MW], int n, float eps, int8_t* qs, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float x[MW], p[MW];
  if constexpr (MW % 4 == 0) {
#pragma unroll
    for (int m = 0; m < MW / 4; ++m) {
      const float4 v = ((const float4*)xs)[threadIdx.x + kPT * m];
      x[4 * m] = v.x;
      x[4 * m + 1] = v.y;
      x[4 * m + 2] = v.z;
      x[4 * m + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int m = 0; m < MW; ++m) x[m] = xs[norm_idx<MW>(m)];
  }
  float ss = 0.0f, pm = 0.0f;
#pragma unroll
  for (int m = 0; m < MW; ++m) {
    p[m] = x[m] * wr[m];
    ss += x[m] * x[m];
    pm = fmaxf(pm, fabsf(p[m]));
  }
  ss = wave_sum(ss);
  pm = wave_max(pm);
  if (lane == 0) {
    red[wave] = ss;
    red[kPW + wave] = pm;
  }
  wg_barrier();
  float tss = 0.0f, tpm = 0.0f;
#pragma unroll
  for (int v = 0; v < kPW; ++v) {
    tss += red[v];
    tpm = fmaxf(tpm, red[kPW + v]);
  }
  const float rstd = 1.0f / sqrtf(tss / (float)n + eps);
  const float amax = rstd * tpm;
  const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
  auto code = [&](int m) -> int {
    const float u = rstd * p[m];
    const float rq = rintf(u * inv);
    return (int)fminf(fmaxf(rq, -127.0f), 127.0f);
  };
  if constexpr (MW % 4 == 0) {
#pragma unroll
    for (int m = 0; m < MW / 4; ++m) {
      const uint32_t pk = ((uint32_t)code(4 * m) & 0xFFu) | (((uint32_t)code(4 * m + 1) & 0xFFu) << 8) |
                          (((uint32_t)code(4 * m + 2) & 0xFFu) << 16) | ((uint32_t)code(4 * m + 3) << 24);
      *(uint32_t*)(qs + qbyte(norm_idx<MW>(4 * m))) = pk;
    }
  } else {
#pragma unroll
    for (int m = 0; m < MW; ++m) qs[qbyte(norm_idx<MW>(m))] = (int8_t)code(m);
  }
  wg_barrier();
  return amax > 0.0f ? amax / 127.0f : 0.0f;
}

// The residual and gated-output hops fused with the first half of their
// RMSNorm + quantiser: the thread that polled paired words i = t + 256 m
// keeps their values (inputs 2i, 2i+1, held in x) and forms p = x w, the
// partial sum of squares and max |p| (wave totals into red), so the hop's
// closing barrier is also the norm's statistics barrier and the values never
// take an LDS round trip.  np = number of pairs.
template <int MP>
__device__ __forceinline__ void pair_stats(const float (&x)[2 * MP], const float* wts, int np, float (&p)[2 * MP],
                                           float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float ss = 0.0f, pm = 0.0f;
#pragma unroll
  for (int m = 0; m < MP; ++m) {
    const int i = threadIdx.x + m * kPT;
    const float2 w2 = i < np ? ((const float2*)wts)[i] : make_float2(0.0f, 0.0f);
    p[2 * m] = x[2 * m] * w2.x;
    p[2 * m + 1] = x[2 * m + 1] * w2.y;
    ss += x[2 * m] * x[2 * m];
    ss += x[2 * m + 1] * x[2 * m + 1];
    pm = fmaxf(pm, fmaxf(fabsf(p[2 * m]), fabsf(p[2 * m + 1])));
  }
  ss = wave_sum(ss);
  pm = wave_max(pm);
  if (lane == 0) {
    red[wave] = ss;
    red[kPW + wave] = pm;
  }
}
// Second half (after the statistics barrier): the scale, then the codes of
// the held pairs into qs (swizzled), then the codes barrier.  n = 2 np
// inputs; returns amax / 127 as p_norm_quant does.
template <int MP>
__device__ float pair_quant(const float (&p)[2 * MP], int np, float eps, const float* red, int8_t* qs) {
  float tss = 0.0f, tpm = 0.0f;
#pragma unroll
  for (int v = 0; v < kPW; ++v) {
    tss += red[v];
    tpm = fmaxf(tpm, red[kPW + v]);
  }
  const float rstd = 1.0f / sqrtf(tss / (float)(2 * np) + eps);
  const float amax = rstd * tpm;
  const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
  auto code = [&](float pv) -> uint32_t {
    const float rq = rintf((rstd * pv) * inv);
    return (uint32_t)(int)fminf(fmaxf(rq, -127.0f), 127.0f) & 0xFFu;
  };
#pragma unroll
  for (int m = 0; m < MP; ++m) {
    const int i = threadIdx.x + m * kPT;
    if (i < np) *(uint16_t*)(qs + qbyte(2 * i)) = (uint16_t)(code(p[2 * m]) | (code(p[2 * m + 1]) << 8));
  }
  wg_barrier();
  return amax > 0.0f ? amax / 127.0f : 0.0f;
}

// LoRA down-projection, rank 16, by the loader waves: loader wave v computes
// rows 4v .. 4v+3.  Lane l takes the 16-byte input chunks l + 64 j (C = n/16
// chunks) and holds A[4v + r][chunk l + 64 j] in av[r J + j], so every code
// chunk is read from LDS once per wave and feeds 4 independent accumulators;
// four wave reductions follow.  tout[k] = float(sum_i A[k][i] q_i) * sA[k]
// (the code scale s is applied by the reader); sA_lane = sA[4v + (l & 3)].
template <int J>
__device__ void p_lora_down(const uint4 (&av)[4 * J], int n, const int8_t* qs, float sA_lane, float* tout, int lane,
                            int wave) {
  const int C = n >> 4;
  const uint4* q4 = (const uint4*)qs;
  uint4 qv[J];
#pragma unroll
  for (int j = 0; j < J; ++j) qv[j] = lane + 64 * j < C ? q4[qchunk(lane + 64 * j)] : make_uint4(0, 0, 0, 0);
  int acc[4] = {0, 0, 0, 0};
#pragma unroll
  for (int j = 0; j < J; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint4 a = av[r * J + j];
      acc[r] = __builtin_amdgcn_sdot4((int)a.x, (int)qv[j].x, acc[r], false);
      acc[r] = __builtin_amdgcn_sdot4((int)a.y, (int)qv[j].y, acc[r], false);
      acc[r] = __builtin_amdgcn_sdot4((int)a.z, (int)qv[j].z, acc[r], false);
      acc[r] = __builtin_amdgcn_sdot4((int)a.w, (int)qv[j].w, acc[r], false);
    }
  int tot[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) tot[r] = wave_sum_i(acc[r]);
  if (lane < 4) {
    const int t = lane == 0 ? tot[0] : lane == 1 ? tot[1] : lane == 2 ? tot[2] : tot[3];
    tout[4 * wave + lane] = (float)t * sA_lane;
  }
}

// Sign table: entry v (one byte of scaffold bits, input k at bit k) holds the
// eight signs +1 / -1 of those inputs as int8, inputs 0..3 in .x and 4..7 in
// .y, so that the 1-bit x int8 dot product runs on the packed int8 dot unit
// with no bit-plane transpose of the activations.  The table is stored
// kLutCopies times interleaved (entry v of copy c at [v][c]) and lane l reads
// copy l % kLutCopies: the 16 lanes an LDS cycle serves for 8-byte reads then
// hit 16 distinct bank pairs whatever bytes they look up.
__device__ __forceinline__ uint2 sign_entry(uint32_t v) {
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    lo |= (((v >> k) & 1u) ? 0x01u : 0xFFu) << (8 * k);
    hi |= (((v >> (k + 4)) & 1u) ? 0x01u : 0xFFu) << (8 * k);
  }
  return make_uint2(lo, hi);
}

// sum_i s_i q_i over the 128 inputs of one 16-byte chunk of scaffold bits w
// (word x = inputs 0..31, bit i of a word = input i), s_i = +1 where the bit is
// set and -1 where it is clear; qd holds the 128 int8 codes as 32 words.
// lut: this lane's copy of the sign table (table + lane % kLutCopies).
__device__ __forceinline__ int p_sign_dot(const uint4 w, const uint32_t (&qd)[32], const uint2* lut) {
  const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
  uint2 sg[16];  // all 16 lookups in flight before the first is used
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int b = 0; b < 4; ++b) sg[4 * c + b] = lut[((wv[c] >> (8 * b)) & 0xFFu) * kLutCopies];
  int acc = 0;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      acc = __builtin_amdgcn_sdot4((int)sg[4 * c + b].x, (int)qd[8 * c + 2 * b], acc, false);
      acc = __builtin_amdgcn_sdot4((int)sg[4 * c + b].y, (int)qd[8 * c + 2 * b + 1], acc, false);
    }
  }
  return acc;
}
// the int8 codes of inputs [128 j, 128 j + 128) as 32 words
__device__ __forceinline__ void load_codes(const int8_t* qs, int j, uint32_t (&qd)[32]) {
  const uint4* q4 = (const uint4*)qs;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint4 v = q4[qchunk(8 * j + k)];
    qd[4 * k + 0] = v.x;
    qd[4 * k + 1] = v.y;
    qd[4 * k + 2] = v.z;
    qd[4 * k + 3] = v.w;
  }
}
// Marks a prefetched register value as used here: the compiler cannot move
// work on it (a conversion, say) up to the load, where it would make the
// prefetch wait for its own data.
__device__ __forceinline__ int at_use(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// float sum over aligned groups of U lanes, the same DPP pattern (and result
// lanes) as group_sum_i
__device__ __forceinline__ float group_sum_f(float v, int U) {
  if (U >= 2) v += dpp_f<kDppQuadSwap1>(v);
  if (U >= 4) v += dpp_f<kDppQuadSwap2>(v);
  if (U >= 8) v += dpp_f<kDppRowHalfMirror>(v);
  if (U >= 16) v += dpp_f<kDppRowMirror>(v);
  if (U >= 32) v += dpp_f<kDppRowBcast15, 0xA>(v);
  if (U >= 64) v += dpp_f<kDppRowBcast31, 0x8>(v);
  return v;
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
  static constexpr int KZ = NBC, KX = NBC + 16, KDT = NBC + 32;  // first z, x and the dt row among them
  static constexpr int OUT_PER = DM / G;
  static constexpr int UI = DM / 128, RPPI = 64 / UI, NGI_T = (NROWS + RPPI - 1) / RPPI, NGI = (NGI_T + kPW - 1) / kPW;
  static constexpr int UO = DI / 128, RPPO = 64 / UO, NGO_T = (OUT_PER + RPPO - 1) / RPPO,
                       NGO = (NGO_T + kPW - 1) / kPW;
  static constexpr int MW1 = DM / kPT, MW2 = DI / kPT;
  static constexpr int GW1 = (DM / 2 + kPT - 1) / kPT, GW2 = (DI / 2 + kPT - 1) / kPT;  // paired words per thread
  // LoRA-up ranks per lane of a row group (lane j takes ranks j, j + U, ...)
  static constexpr int RLI = (16 + UI - 1) / UI, RLO = (16 + UO - 1) / UO;
  // LoRA-down operands per thread: 4 rows x J chunks (J = chunks per lane)
  static constexpr int J1 = (DM / 16 + 63) / 64, J2 = (DI / 16 + 63) / 64, MC1 = 4 * J1, MC2 = 4 * J2;
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
  static_assert(NBC <= RPPI, "the B/C rows must sit in row group 0 of wave 0");
  static_assert(RPPO % 2 == 0 && OUT_PER % 2 == 0, "out_proj rows are published in pairs from one wave");
};

constexpr int kHeadDepth = 8;  // LM-head rows in flight per wave
static_assert(kPT == 256 && kPW == 4 && kLT == 256, "one compute wave per 4 state channels, one loader wave per 4 LoRA ranks");

// Where compute thread t (0 .. kPT) of workgroup w sits in the work split;
// the loader waves stage each compute thread's operands from the same map.
template <class S>
struct TMap {
  int wave, lane, hd, j, w;
  int ji, subi, jo, subo;
  bool lead_i, lead_o, bc_thread, x_thread, conv_thread;
  int conv_k, conv_c, conv_slot;
  __device__ TMap(int t, int w_) {
    w = w_;
    wave = t >> 6;
    lane = t & 63;
    hd = w / (S::HP / 16);
    j = w % (S::HP / 16);
    ji = lane & (S::UI - 1);
    subi = lane / S::UI;
    lead_i = lane == group_sum_lane(subi * S::UI, S::UI);
    jo = lane & (S::UO - 1);
    subo = lane / S::UO;
    lead_o = lane == group_sum_lane(subo * S::UO, S::UO);
    // conv threads: the lane that reduces B/C row k (< NBC, row group 0 of
    // wave 0) convolves and publishes it right away; lanes 0..15 of wave 1
    // convolve the 16 x channels after the GEMV
    bc_thread = wave == 0 && lead_i && subi < S::NBC;
    x_thread = wave == 1 && lane < 16;
    conv_thread = bc_thread || x_thread;
    conv_k = bc_thread ? subi : S::KX + (lane & 15);
    conv_c = conv_thread ? in_row(conv_k) - S::DI : 0;
    conv_slot = bc_thread ? 16 + subi : (lane & 15);
  }
  // own in_proj rows, B/C first: their conv outputs are published while the
  // other rows are still being computed
  __device__ int in_row(int k) const {
    if (k < S::KZ) return 2 * S::DI + (w + k * S::G);                       // B/C
    if (k < S::KX) return hd * S::HP + j * 16 + (k - S::KZ);                // z
    if (k < S::KDT) return S::DI + hd * S::HP + j * 16 + (k - S::KX);       // x
    return 2 * S::DI + 2 * S::NS + hd;                                      // dt
  }
};

// LDS carve-up.  The operand images (a layer's weights, scales and state as
// the compute threads use them, [item][thread]) are written by the loader
// waves and read by the compute waves.
template <class S>
struct Lds {
  static constexpr int DM = S::DM, DI = S::DI, NS = S::NS, MX = DM > DI ? DM : DI;
  static constexpr size_t O_WIN = 0;                                          // uint4 [NGI][kPT]
  static constexpr size_t O_WOUT = O_WIN + (size_t)S::NGI * kPT * 16;         // uint4 [NGO][kPT]
  static constexpr size_t O_ST = O_WOUT + (size_t)S::NGO * kPT * 16;          // float4 [NST][kPT]
  static constexpr size_t O_HS = O_ST + (size_t)S::NST * kPT * 16;            // float [DM] residual stream
  static constexpr size_t O_GS = O_HS + (size_t)DM * 4;                       // float [DI] gated SSM output
  static constexpr size_t O_NW = O_GS + (size_t)DI * 4;                       // float [DM] norm weight
  static constexpr size_t O_GW = O_NW + (size_t)DM * 4;                       // float [DI] gated norm weight
  static constexpr size_t O_LUT = O_GW + (size_t)DI * 4;                      // uint2 [256][kLutCopies]
  static constexpr size_t O_QS = O_LUT + (size_t)256 * kLutCopies * 8;        // int8 [MX] codes
  static constexpr size_t O_ISW = O_QS + ((size_t)MX + 15) / 16 * 16;         // float [NGI][kPT]
  static constexpr size_t O_ISB = O_ISW + (size_t)S::NGI * kPT * 4;           // float [NGI][kPT]
  static constexpr size_t O_IB = O_ISB + (size_t)S::NGI * kPT * 4;            // int [NGI * RLI][kPT]
  static constexpr size_t O_OSW = O_IB + (size_t)S::NGI * S::RLI * kPT * 4;   // float [NGO][kPT]
  static constexpr size_t O_OSB = O_OSW + (size_t)S::NGO * kPT * 4;           // float [NGO][kPT]
  static constexpr size_t O_OB = O_OSB + (size_t)S::NGO * kPT * 4;            // int [NGO * RLO][kPT]
  static constexpr size_t O_CONV = O_OB + (size_t)S::NGO * S::RLO * kPT * 4;  // float [8][32] conv w, b, window
  static constexpr size_t O_HP = O_CONV + 8 * 32 * 4;                         // float [4] dt bias, A_log, D
  static constexpr size_t O_BCS = O_HP + 16;                                  // float [2 NS] B, C
  static constexpr size_t O_TLS = O_BCS + (size_t)2 * NS * 4;                 // float [16] LoRA-down vector
  static constexpr size_t O_ROWV = O_TLS + 16 * 4;                            // float [kMaxInRows] own in_proj rows
  static constexpr size_t O_RED = O_ROWV + kMaxInRows * 4;                    // float [2 kPW]
  static constexpr size_t O_STOP = O_RED + 2 * kPW * 4;                       // int [1], token int [1] (+ pad)
  static constexpr size_t O_ARG = O_STOP + 16;                                // float [2 kPW]
  static constexpr size_t BYTES = O_ARG + 2 * kPW * 4;

  uint4 *win, *wout;
  float4* st;
  float *hs, *gs, *nw, *gw, *isw, *isb, *osw, *osb, *conv, *hp, *bcs, *tls, *rowv, *red, *arg;
  int *ib, *ob, *stop, *tok;
  uint2* lut;
  int8_t* qs;
  __device__ explicit Lds(unsigned char* m) {
    win = (uint4*)(m + O_WIN);
    wout = (uint4*)(m + O_WOUT);
    st = (float4*)(m + O_ST);
    hs = (float*)(m + O_HS);
    gs = (float*)(m + O_GS);
    nw = (float*)(m + O_NW);
    gw = (float*)(m + O_GW);
    lut = (uint2*)(m + O_LUT);
    qs = (int8_t*)(m + O_QS);
    isw = (float*)(m + O_ISW);
    isb = (float*)(m + O_ISB);
    ib = (int*)(m + O_IB);
    osw = (float*)(m + O_OSW);
    osb = (float*)(m + O_OSB);
    ob = (int*)(m + O_OB);
    conv = (float*)(m + O_CONV);
    hp = (float*)(m + O_HP);
    bcs = (float*)(m + O_BCS);
    tls = (float*)(m + O_TLS);
    rowv = (float*)(m + O_ROWV);
    red = (float*)(m + O_RED);
    stop = (int*)(m + O_STOP);
    tok = stop + 1;
    arg = (float*)(m + O_ARG);
  }
};

// The loader waves (threads kPT .. kPT + kLT).  Loader thread lt stages the
// operands of compute thread lt: per layer, the in_proj image (scaffold bits
// of its rows, scales, LoRA-up weights, conv weights and window, the norm
// weight) and the out_proj / SSM image (scaffold bits, scales, LoRA-up
// weights, the SSM state block, the gated norm weight, the head's dt bias,
// A_log and D).  It also holds the LoRA-down matrices (96 KB per layer at the
// 1.3B shape, the bulk of what a workgroup reads) in registers and forms
// t = A q while the compute waves run the scaffold GEMV.  So the compute
// waves issue no weight or state loads at all: their instruction stream never
// stalls behind a full memory queue, and their polls wait for nothing but the
// hop (the vector memory counter is per wave).  Global loads are issued a
// phase or more before their LDS writes, so the data has landed by then.
// The loaders take no part in the hops: they pass the workgroup barriers in
// the same sequence as the compute waves (listed at the kernel) and stop
// where a hop reports an abort.
//
// Image timing (layer l): the compute waves read the in_proj image at the
// start of the layer and the out_proj image after the B/C hop.  The loaders
// issue the in_proj and out_proj loads of layer l+1 after the B/C hop (the
// SSM phase) and write the in_proj image between the gated-output hop and the
// gated norm, the out_proj image in layer l+1 between "in_proj rows done" and
// the B/C hop; the out_proj LoRA-down matrix of layer l goes out in the norm
// phase of layer l, the in_proj one of layer l+1 after the in_proj
// LoRA-down.  Both images
// are single-buffered: each write lands after the compute waves' last read
// of the previous layer's image and before their first read of the new one.  Conv and SSM state written back by the
// compute waves in layer l is re-read for layer l of the next token, at
// least one layer later (n_layer >= 2), after the compute waves' polls have
// completed those stores.
template <int V>
using I = std::integral_constant<int, V>;

template <class S>
__device__ void loader_waves(const PersistArgs& a, const Lds<S>& L) {
  constexpr int DM = S::DM, DI = S::DI, NS = S::NS, HP = S::HP, CDIM = S::CDIM;
  constexpr int NV1 = (DM / 4 + kLT - 1) / kLT, NV2 = (DI / 4 + kLT - 1) / kLT;  // float4 of a norm weight per thread
  const int lt = (int)threadIdx.x - kPT, lane = lt & 63, lw = lt >> 6;
  const TMap<S> tm(lt, blockIdx.x);
  const int w = tm.w;
  const char* wb = a.wbase;
  auto lp = [&](int l, int k) -> const char* { return wb + (size_t)l * S::LSTRIDE + S::OFF(k); };

  // in flight: in_proj image, out_proj image, LoRA-down matrices
  uint4 r_win[S::NGI];
  float r_isw[S::NGI], r_isb[S::NGI];
  int r_ib[S::NGI][S::RLI];
  float r_conv[8];
  float4 r_nw[NV1];
  uint4 r_wout[S::NGO];
  float r_osw[S::NGO], r_osb[S::NGO];
  int r_ob[S::NGO][S::RLO];
  float4 r_st[S::NST];
  float4 r_gw[NV2];
  float r_hp[3];
  uint4 ain[S::MC1], aout[S::MC2];
  float sAi, sAo;

  auto load_in = [&](int l) {
    const uint4* b4 = (const uint4*)lp(l, DFSSM_PK_IN_BITS);
    const float* sw = (const float*)lp(l, DFSSM_PK_IN_SW);
    const float* sb = (const float*)lp(l, DFSSM_PK_IN_SB);
    const int8_t* bm = (const int8_t*)lp(l, DFSSM_PK_IN_B);
#pragma unroll
    for (int m = 0; m < S::NGI; ++m) {
      const int g = tm.wave + m * kPW;
      const int k = g * S::RPPI + tm.subi;
      const bool live = g < S::NGI_T && k < S::NROWS;
      const int row = live ? tm.in_row(k) : 0;
      r_win[m] = live ? b4[(size_t)row * S::UI + tm.ji] : make_uint4(0, 0, 0, 0);
      r_isw[m] = live ? sw[row] : 0.0f;
      r_isb[m] = live ? sb[row] : 0.0f;
#pragma unroll
      for (int r = 0; r < S::RLI; ++r) {
        const int kk = tm.ji + S::UI * r;
        r_ib[m][r] = live && kk < 16 ? (int)bm[(size_t)row * 16 + kk] : 0;
      }
    }
    if (tm.conv_thread) {
      const float* wc = (const float*)lp(l, DFSSM_PK_CONV_W) + (size_t)tm.conv_c * 4;
      const float* cs = a.conv + (size_t)l * 3 * CDIM;
      r_conv[0] = wc[0]; r_conv[1] = wc[1]; r_conv[2] = wc[2]; r_conv[3] = wc[3];
      r_conv[4] = ((const float*)lp(l, DFSSM_PK_CONV_B))[tm.conv_c];
      r_conv[5] = cs[tm.conv_c]; r_conv[6] = cs[CDIM + tm.conv_c]; r_conv[7] = cs[2 * CDIM + tm.conv_c];
    }
    const float4* n4 = (const float4*)lp(l, DFSSM_PK_NORM_W);
#pragma unroll
    for (int m = 0; m < NV1; ++m) {
      const int q = lt + kLT * m;
      r_nw[m] = q < DM / 4 ? n4[q] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto write_in = [&]() {
#pragma unroll
    for (int m = 0; m < S::NGI; ++m) {
      L.win[m * kPT + lt] = r_win[m];
      L.isw[m * kPT + lt] = r_isw[m];
      L.isb[m * kPT + lt] = r_isb[m];
#pragma unroll
      for (int r = 0; r < S::RLI; ++r) L.ib[(m * S::RLI + r) * kPT + lt] = r_ib[m][r];
    }
    if (tm.conv_thread)
#pragma unroll
      for (int e = 0; e < 8; ++e) L.conv[e * 32 + tm.conv_slot] = r_conv[e];
#pragma unroll
    for (int m = 0; m < NV1; ++m) {
      const int q = lt + kLT * m;
      if (q < DM / 4) ((float4*)L.nw)[q] = r_nw[m];
    }
  };
  auto load_out = [&](int l) {
    const uint4* b4 = (const uint4*)lp(l, DFSSM_PK_OUT_BITS);
    const float* sw = (const float*)lp(l, DFSSM_PK_OUT_SW);
    const float* sb = (const float*)lp(l, DFSSM_PK_OUT_SB);
    const int8_t* bm = (const int8_t*)lp(l, DFSSM_PK_OUT_B);
#pragma unroll
    for (int m = 0; m < S::NGO; ++m) {
      const int g = tm.wave + m * kPW;
      const int k = g * S::RPPO + tm.subo;
      const bool live = g < S::NGO_T && k < S::OUT_PER;
      const int row = w * S::OUT_PER + (live ? k : 0);
      r_wout[m] = live ? b4[(size_t)row * S::UO + tm.jo] : make_uint4(0, 0, 0, 0);
      r_osw[m] = live ? sw[row] : 0.0f;
      r_osb[m] = live ? sb[row] : 0.0f;
#pragma unroll
      for (int r = 0; r < S::RLO; ++r) {
        const int kk = tm.jo + S::UO * r;
        r_ob[m][r] = live && kk < 16 ? (int)bm[(size_t)row * 16 + kk] : 0;
      }
    }
    const float4* s4 = (const float4*)(a.ssm + (size_t)l * S::H * HP * NS + (size_t)w * NS * 16);
#pragma unroll
    for (int m = 0; m < S::NST; ++m) {
      const int n = tm.lane + 64 * m;
      r_st[m] = n < NS ? s4[n * 4 + tm.wave] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const float4* g4 = (const float4*)lp(l, DFSSM_PK_GNORM_W);
#pragma unroll
    for (int m = 0; m < NV2; ++m) {
      const int q = lt + kLT * m;
      r_gw[m] = q < DI / 4 ? g4[q] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (lt == 0) {
      r_hp[0] = ((const float*)lp(l, DFSSM_PK_DT_BIAS))[tm.hd];
      r_hp[1] = ((const float*)lp(l, DFSSM_PK_A_LOG))[tm.hd];
      r_hp[2] = ((const float*)lp(l, DFSSM_PK_D))[tm.hd];
    }
  };
  auto write_out = [&]() {
#pragma unroll
    for (int m = 0; m < S::NGO; ++m) {
      L.wout[m * kPT + lt] = r_wout[m];
      L.osw[m * kPT + lt] = r_osw[m];
      L.osb[m * kPT + lt] = r_osb[m];
#pragma unroll
      for (int r = 0; r < S::RLO; ++r) L.ob[(m * S::RLO + r) * kPT + lt] = r_ob[m][r];
    }
#pragma unroll
    for (int m = 0; m < S::NST; ++m) L.st[m * kPT + lt] = r_st[m];
#pragma unroll
    for (int m = 0; m < NV2; ++m) {
      const int q = lt + kLT * m;
      if (q < DI / 4) ((float4*)L.gw)[q] = r_gw[m];
    }
    if (lt == 0) {
      L.hp[0] = r_hp[0];
      L.hp[1] = r_hp[1];
      L.hp[2] = r_hp[2];
    }
  };
  // LoRA-down matrices: rows 4 lw + r, chunks lane + 64 j (the p_lora_down layout)
  auto load_ain = [&](int l) {
    const uint4* A4 = (const uint4*)lp(l, DFSSM_PK_IN_A);
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int jj = 0; jj < S::J1; ++jj) {
        const int c = lane + 64 * jj;
        ain[r * S::J1 + jj] = c < DM / 16 ? A4[(size_t)(4 * lw + r) * (DM / 16) + c] : make_uint4(0, 0, 0, 0);
      }
    sAi = ((const float*)lp(l, DFSSM_PK_IN_SA))[4 * lw + (lane & 3)];
  };
  // rows 4 lw + r for r in [R0, R1) (compile-time bounds: no branches around the loads)
  auto load_aout = [&](int l, auto r0c, auto r1c) {
    constexpr int R0 = decltype(r0c)::value, R1 = decltype(r1c)::value;
    const uint4* A4 = (const uint4*)lp(l, DFSSM_PK_OUT_A);
#pragma unroll
    for (int r = R0; r < R1; ++r)
#pragma unroll
      for (int jj = 0; jj < S::J2; ++jj) {
        const int c = lane + 64 * jj;
        aout[r * S::J2 + jj] = c < DI / 16 ? A4[(size_t)(4 * lw + r) * (DI / 16) + c] : make_uint4(0, 0, 0, 0);
      }
    if constexpr (R0 == 0) sAo = ((const float*)lp(l, DFSSM_PK_OUT_SA))[4 * lw + (lane & 3)];
  };
  auto stopped = [&]() { return *L.stop != 0; };

  const int T = a.n_tokens, Lm = a.n_layer;
  // A workgroup's loads share one memory pipeline, so a compute wave's poll
  // queues behind any loader bytes issued just before it; and a loader wave
  // that is still issuing loads when the compute waves reach a barrier holds
  // them there.  So the loads go out in pieces that each fit the compute
  // phase between two barriers, in the phases without a poll at their end.
  load_in(0);
  load_ain(0);
  load_out(0);
  load_aout(0, I<0>{}, I<2>{});
  write_in();
  for (int t = 0; t < T; ++t) {
    wg_barrier();  // embedding row in LDS
    for (int l = 0; l < Lm; ++l) {
      const int ln = l + 1 < Lm ? l + 1 : 0;  // after the last layer: layer 0 of the next token
      wg_barrier();  // residual hop (layers > 0) and norm statistics
      if (stopped()) return;
      load_aout(l, I<2>{}, I<4>{});
      wg_barrier();  // in_proj codes in LDS
      p_lora_down<S::J1>(ain, DM, L.qs, sAi, L.tls, lane, lw);
      wg_barrier();  // LoRA-down vector ready
      load_in(ln);
      load_ain(ln);
      wg_barrier();  // in_proj rows done
      write_out();   // this layer's out_proj image
      wg_barrier();  // B/C hop
      if (stopped()) return;
      wg_barrier();  // gated-output hop and gated norm statistics
      if (stopped()) return;
      write_in();    // the next layer's in_proj image
      wg_barrier();  // out_proj codes in LDS
      p_lora_down<S::J2>(aout, DI, L.qs, sAo, L.tls, lane, lw);
      wg_barrier();  // LoRA-down vector ready
      load_out(ln);
      load_aout(ln, I<0>{}, I<2>{});
      wg_barrier();  // end of layer
    }
    wg_barrier();  // final residual hop
    if (stopped()) return;
    wg_barrier();  // final norm statistics
    wg_barrier();  // final codes
    wg_barrier();  // per-wave argmax candidates
    wg_barrier();  // argmax hop
    if (stopped()) return;
    wg_barrier();  // next token chosen
  }
}

// MODE 0: the plain kernel.  MODE 1: also writes phase timestamps (profiling;
// nothing else added, so the phases keep close to the plain kernel's timing).
// MODE 2: also writes the traces of intermediate values (tests) and the
// timestamps.
//
// Workgroup barriers per token, the same sequence in the compute and loader
// waves: embedding; per layer residual hop (layers > 0) with the norm
// statistics, codes, LoRA-down vector ready, in_proj rows done, B/C hop,
// gated-output hop with the gated norm statistics, codes, LoRA-down vector
// ready, end of layer; then final residual hop, final norm statistics, codes,
// per-wave argmax candidates, argmax hop, next token chosen.
template <class S, int MODE>
__global__ __launch_bounds__(kBlock, 1) void decode_persistent_kernel(PersistArgs a) {
  constexpr bool TR = MODE == 2;
  extern __shared__ unsigned char smem[];
  constexpr int DM = S::DM, DI = S::DI, NS = S::NS, HP = S::HP, G = S::G, CDIM = S::CDIM;
  constexpr int KZ = S::KZ, KX = S::KX, KDT = S::KDT;
  const Lds<S> L(smem);
  float* const hs = L.hs;
  float* const gs = L.gs;
  int8_t* const qs = L.qs;
  float* const bcs = L.bcs;
  float* const tls = L.tls;
  float* const rowv = L.rowv;
  float* const red = L.red;
  int* const s_stop = L.stop;
  int* const s_tok = L.tok;
  float* const s_arg = L.arg;
  if (threadIdx.x == 0) *s_stop = 0;
  for (int f = threadIdx.x; f < 256 * kLutCopies; f += kBlock) L.lut[f] = sign_entry((uint32_t)(f / kLutCopies));
  wg_barrier();
  if (threadIdx.x >= kPT) {
    loader_waves<S>(a, L);
    return;
  }

  const int w = blockIdx.x;
  const TMap<S> tm(threadIdx.x, w);
  const int lane = tm.lane, wave = tm.wave, hd = tm.hd, j = tm.j;
  const int ji = tm.ji, subi = tm.subi, jo = tm.jo, subo = tm.subo;
  const bool lead_i = tm.lead_i, lead_o = tm.lead_o, bc_thread = tm.bc_thread, x_thread = tm.x_thread;
  const bool conv_thread = tm.conv_thread;
  const int conv_k = tm.conv_k, conv_c = tm.conv_c;
  const uint2* lut_l = L.lut + (lane % kLutCopies);
  unsigned e = a.epoch0;  // same value in every workgroup
  int tok = kargs()->tok_in[0];
  unsigned pc = a.pair0;  // write count of the paired boxes (one write per layer)
  uint64_t* const hbox = a.boxes;            // paired, DM / 2 words
  uint64_t* const bcbox = hbox + kR * DM / 2;
  uint64_t* const gbox = bcbox + kR * 2 * NS;  // paired, DI / 2 words
  uint64_t* const abox = gbox + kR * DI / 2;

  // conv weights and window of this thread's channel (conv threads)
  float cw[4], cb, cst[3];
  auto conv_step = [&](float y) -> float {
    const float v = cb + cw[0] * cst[0] + cw[1] * cst[1] + cw[2] * cst[2] + cw[3] * y;
    cst[0] = cst[1];
    cst[1] = cst[2];
    cst[2] = y;
    return silu_f(v);
  };

  // phase timestamps (100 MHz device clock) for performance analysis
  auto prof = [&](int t, int l, int ev) {
    if constexpr (MODE >= 1) {
      const KArgs k = kargs();
      if (k->prof && t < k->prof_tokens && threadIdx.x == 0)
        k->prof[(((size_t)t * (k->n_layer + 1) + l) * G + w) * kProfEvents + ev] = wall_clock64();
    }
  };

  const int T = a.n_tokens;
  const int Lm = a.n_layer;
  bool ok = true;
  for (int t = 0; t < T && ok; ++t) {
    // ---- embedding (every workgroup, no hop)
    {
      const KArgs k = kargs();
      int tk = tok;
      if (tk < 0 || tk >= k->vocab) {
        if (threadIdx.x == 0 && w == 0) atomicOr(k->err, 1);
        tk = 0;
      }
      const float sc = k->sE[tk];
      const int8_t* er = k->E + (size_t)tk * DM;
#pragma unroll
      for (int m = 0; m < S::MW1; ++m) {
        const int i = threadIdx.x + m * kPT;
        hs[i] = (float)er[i] * sc;
      }
      wg_barrier();
    }
    for (int l = 0; l < Lm && ok; ++l) {
      prof(t, l, 0);
      float s1;
      // this layer's in_proj image (staged by the loader waves)
      uint4 win[S::NGI];
      float isw[S::NGI], isb[S::NGI];
      int ib[S::NGI][S::RLI];
#pragma unroll
      for (int m = 0; m < S::NGI; ++m) {
        win[m] = L.win[m * kPT + threadIdx.x];
        isw[m] = L.isw[m * kPT + threadIdx.x];
        isb[m] = L.isb[m * kPT + threadIdx.x];
#pragma unroll
        for (int r = 0; r < S::RLI; ++r) ib[m][r] = L.ib[(m * S::RLI + r) * kPT + threadIdx.x];
      }
      if (conv_thread) {
        const float* cv = L.conv + tm.conv_slot;
        cw[0] = cv[0]; cw[1] = cv[32]; cw[2] = cv[64]; cw[3] = cv[96];
        cb = cv[128];
        cst[0] = cv[160]; cst[1] = cv[192]; cst[2] = cv[224];
      }
      // ---- residual hop (layers > 0; layer 0 starts from the embedding row) fused
      // with the norm statistics
      {
        float xa[2 * S::GW1], pa[2 * S::GW1];
        bool got = true;
        if (l > 0) {
          uint64_t wv[S::GW1];
          got = poll_words<S::GW1, true>(hbox, DM / 2, pc - 1, wv, a.abort_flag);
#pragma unroll
          for (int m = 0; m < S::GW1; ++m) {
            const int i = threadIdx.x + m * kPT;
            const float2 v = unpack2(wv[m]);
            xa[2 * m] = v.x;
            xa[2 * m + 1] = v.y;
            if (i < DM / 2) ((float2*)hs)[i] = make_float2(xa[2 * m], xa[2 * m + 1]);
          }
          ++e;
        } else {
#pragma unroll
          for (int m = 0; m < S::GW1; ++m) {
            const int i = threadIdx.x + m * kPT;
            const float2 v = i < DM / 2 ? ((const float2*)hs)[i] : make_float2(0.0f, 0.0f);
            xa[2 * m] = v.x;
            xa[2 * m + 1] = v.y;
          }
        }
        pair_stats<S::GW1>(xa, L.nw, DM / 2, pa, red);
        if (!got) *s_stop = 1;
        wg_barrier();  // residual hop and norm statistics
        if (*s_stop) {
          ok = false;
          break;
        }
        prof(t, l, 1);
        if constexpr (TR) {
          float* th = kargs()->trace_h;
          if (th && w == 0)
            for (int i = threadIdx.x; i < DM; i += kPT) th[(size_t)l * DM + i] = hs[i];
        }
        s1 = pair_quant<S::GW1>(pa, DM / 2, a.eps, red, qs);
      }
      // ---- phase A: 1-bit GEMV of own rows (LoRA down by the loaders), conv
      prof(t, l, 2);
      if constexpr (TR) {
        int8_t* tq = kargs()->trace_q1;
        if (tq && w == 0)
          for (int i = threadIdx.x; i < DM; i += kPT) tq[(size_t)l * DM + i] = qs[qbyte(i)];
      }
      {
        // Every row group is computed (a wave's unused group has zero weights
        // and is not stored), so the table lookups of all groups are in flight
        // together; the loader waves form the LoRA-down vector meanwhile.  The
        // LoRA-up term is spread over the row's lanes.
        uint32_t qd[32];
        load_codes(qs, ji, qd);
        int part[S::NGI];
#pragma unroll
        for (int m = 0; m < S::NGI; ++m) part[m] = p_sign_dot(win[m], qd, lut_l);
        wg_barrier();  // LoRA-down vector ready
        prof(t, l, 3);
        float tl[S::RLI];
#pragma unroll
        for (int r = 0; r < S::RLI; ++r) tl[r] = ji + S::UI * r < 16 ? tls[ji + S::UI * r] * s1 : 0.0f;
        auto row_out = [&](int m, int part) -> float {
          const int acc = group_sum_i(part, S::UI);
          if constexpr (TR) {
            int32_t* ta = kargs()->trace_acc1;
            const int g = wave + m * kPW, k = g * S::RPPI + subi;
            if (ta && lead_i && g < S::NGI_T && k < S::NROWS) ta[(size_t)l * S::DPROJ + tm.in_row(k)] = acc;
          }
          float lo = 0.0f;
#pragma unroll
          for (int r = 0; r < S::RLI; ++r) lo += (float)ib[m][r] * tl[r];
          lo = group_sum_f(lo, S::UI);
          return (float)acc * isw[m] * s1 + isb[m] * lo;
        };
        // row group 0 first: it holds the B/C row, whose conv output is
        // published before the remaining groups are finished
        {
          const float y = row_out(0, part[0]);
          const int k = wave * S::RPPI + subi;
          if (lead_i && wave < S::NGI_T && k < S::NROWS) rowv[k] = y;
          if (bc_thread) publish(bcbox, 2 * NS, conv_c - DI, conv_step(y), e);
        }
#pragma unroll
        for (int m = 1; m < S::NGI; ++m) {
          const float y = row_out(m, part[m]);
          const int g = wave + m * kPW;
          const int k = g * S::RPPI + subi;
          if (lead_i && g < S::NGI_T && k < S::NROWS) rowv[k] = y;
        }
      }
      wg_barrier();  // in_proj rows done
      prof(t, l, 4);
      if (x_thread) rowv[conv_k] = conv_step(rowv[conv_k]);
      prof(t, l, 5);
      ok = gather<(2 * NS + kPT - 1) / kPT>(bcbox, 2 * NS, e, bcs, a.abort_flag, s_stop);
      ++e;
      if (!ok) break;
      prof(t, l, 6);
      if (conv_thread) {
        float* cs = a.conv + (size_t)l * 3 * CDIM;
        cs[conv_c] = cst[0];
        cs[CDIM + conv_c] = cst[1];
        cs[2 * CDIM + conv_c] = cst[2];
      }
      // this layer's out_proj image (staged by the loader waves)
      uint4 wout[S::NGO];
      float osw[S::NGO], osb[S::NGO];
      int ob[S::NGO][S::RLO];
      float4 st[S::NST];  // state float4 (n = lane + 64 m, channels 4*wave ..) of the block [NS][16]
#pragma unroll
      for (int m = 0; m < S::NGO; ++m) {
        wout[m] = L.wout[m * kPT + threadIdx.x];
        osw[m] = L.osw[m * kPT + threadIdx.x];
        osb[m] = L.osb[m * kPT + threadIdx.x];
#pragma unroll
        for (int r = 0; r < S::RLO; ++r) ob[m][r] = L.ob[(m * S::RLO + r) * kPT + threadIdx.x];
      }
#pragma unroll
      for (int m = 0; m < S::NST; ++m) st[m] = L.st[m * kPT + threadIdx.x];
      // ---- phase S: SSM on the state block [hd][j*16 .. +16][0 .. NS), gate.
      // Wave v owns channels 4v .. 4v+3, its lanes the state rows n = lane + 64 m.
      {
        const float dtb = L.hp[0], alog = L.hp[1], dval = L.hp[2];
        const float dt = softplus_f(rowv[KDT] + dtb);
        const float dA = __expf(-dt * __expf(alog));
        const float* xr = rowv + KX + wave * 4;
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
        // (one store instruction per replica: writing all replicas with one
        // instruction from 32 lanes measured ~5 % slower per token)
        // lanes 0..3 hold channels 4 wave + lane; lanes 0 and 2 publish pairs
        {
          const int c = wave * 4 + (lane & 3);  // channel within the slice
          const float y = ((lane & 3) == 0 ? y0 : (lane & 3) == 1 ? y1 : (lane & 3) == 2 ? y2 : y3) + dval * rowv[KX + c];
          const float g = y * silu_f(rowv[KZ + c]);
          const float gn = dpp_f<kDppQuadSwap1>(g);
          if (lane == 0 || lane == 2) publish2(gbox, DI / 2, (hd * HP + j * 16 + c) / 2, g, gn, pc);
        }
      }
      prof(t, l, 7);
      // ---- gated-output hop fused with the gated norm statistics
      float pg[2 * S::GW2];
      {
        float xg[2 * S::GW2];
        uint64_t wv[S::GW2];
        const bool got = poll_words<S::GW2, true>(gbox, DI / 2, pc, wv, a.abort_flag);
#pragma unroll
        for (int m = 0; m < S::GW2; ++m) {
          const float2 v = unpack2(wv[m]);
          xg[2 * m] = v.x;
          xg[2 * m + 1] = v.y;
        }
        pair_stats<S::GW2>(xg, L.gw, DI / 2, pg, red);
        if (!got) *s_stop = 1;
        wg_barrier();  // gated-output hop and gated norm statistics
        ++e;
        if (*s_stop) {
          ok = false;
          break;
        }
      }
      prof(t, l, 8);
      {
        float4* s4 = (float4*)(a.ssm + (size_t)l * S::H * HP * NS + (size_t)w * NS * 16);
#pragma unroll
        for (int m = 0; m < S::NST; ++m) {
          const int n = lane + 64 * m;
          if (n < NS) s4[n * 4 + wave] = st[m];
        }
      }

      // ---- phase B: gated norm, quantise, 1-bit GEMV of own rows (LoRA down by the loaders), residual
      {
        const float s2 = pair_quant<S::GW2>(pg, DI / 2, a.eps, red, qs);
        if constexpr (TR) {
          int8_t* tq = kargs()->trace_q2;
          if (tq && w == 0)
            for (int i = threadIdx.x; i < DI; i += kPT) tq[(size_t)l * DI + i] = qs[qbyte(i)];
        }
        uint32_t qd[32];
        load_codes(qs, jo, qd);
        int part[S::NGO];
#pragma unroll
        for (int m = 0; m < S::NGO; ++m) part[m] = p_sign_dot(wout[m], qd, lut_l);
        wg_barrier();  // LoRA-down vector ready
        float tl[S::RLO];
#pragma unroll
        for (int r = 0; r < S::RLO; ++r) tl[r] = jo + S::UO * r < 16 ? tls[jo + S::UO * r] * s2 : 0.0f;
#pragma unroll
        for (int m = 0; m < S::NGO; ++m) {
          const int acc = group_sum_i(part[m], S::UO);
          float lo = 0.0f;
#pragma unroll
          for (int r = 0; r < S::RLO; ++r) lo += (float)ob[m][r] * tl[r];
          lo = group_sum_f(lo, S::UO);
          const int g = wave + m * kPW;
          const int k = g * S::RPPO + subo;
          const bool live = g < S::NGO_T && k < S::OUT_PER;
          const int row = w * S::OUT_PER + (live ? k : 0);
          if constexpr (TR) {
            int32_t* ta = kargs()->trace_acc2;
            if (ta && lead_o && live) ta[(size_t)l * DM + row] = acc;
          }
          const float hv = hs[row] + ((float)acc * osw[m] * s2 + osb[m] * lo);
          // rows k, k + 1 (k even) sit in one group, row k + 1 lead UO lanes up
          const float hn = __int_as_float(__builtin_amdgcn_ds_bpermute(((lane + S::UO) & 63) * 4, __float_as_int(hv)));
          if (lead_o && live && (k & 1) == 0) publish2(hbox, DM / 2, row / 2, hv, hn, pc);
        }
      }
      prof(t, l, 9);
      ++pc;
      wg_barrier();  // end of layer
    }
    if (!ok) break;
    // ---- final norm + LM head + argmax
    prof(t, Lm, 0);
    constexpr int LH = S::LH, MH = S::MH, RPPH = S::RPPH, STEPH = S::STEPH;
    const int8_t* const E = kargs()->E;
    const float* const sE = kargs()->sE;
    const int vocab = kargs()->vocab;
    // logits are an output for the last token of the launch only
    float* const logits = t == T - 1 ? kargs()->logits : nullptr;
    const int rows_per = (vocab + G - 1) / G;
    const int r0 = w * rows_per;
    const int r1 = min(vocab, r0 + rows_per);
    const int jh = lane & (LH - 1), subh = lane / LH;
    const bool lead_h = lane == group_sum_lane(subh * LH, LH);
    float fn[S::MW1];
    {
      const float* fnp = kargs()->final_norm;
      load_norm_w<S::MW1>(fn, fnp);
    }
    // kHeadDepth rows per wave in flight: their bytes and their scales
    uint4 eb[kHeadDepth][MH];
    float es[kHeadDepth];
    int erow[kHeadDepth];
#pragma unroll
    for (int d = 0; d < kHeadDepth; ++d) {
      const int row = r0 + wave * RPPH + d * STEPH + subh;
      erow[d] = row;
      const bool live = row < r1;
      const uint4* e4 = (const uint4*)(E + (size_t)(live ? row : 0) * DM);
#pragma unroll
      for (int c = 0; c < MH; ++c) eb[d][c] = live ? e4[jh + c * LH] : make_uint4(0, 0, 0, 0);
      es[d] = live ? sE[row] : 0.0f;
    }
    ok = gather2<S::GW1>(hbox, DM / 2, pc - 1, hs, a.abort_flag, s_stop);
    ++e;
    if (!ok) break;
    prof(t, Lm, 1);
    if constexpr (TR) {
      float* th = kargs()->trace_h;
      if (th && w == 0)
        for (int i = threadIdx.x; i < DM; i += kPT) th[(size_t)Lm * DM + i] = hs[i];
    }
    const float sf = p_norm_quant<S::MW1>(hs, fn, DM, a.eps, qs, red);
    prof(t, Lm, 2);
    if constexpr (TR) {
      int8_t* tq = kargs()->trace_qf;
      if (tq && w == 0)
        for (int i = threadIdx.x; i < DM; i += kPT) tq[i] = qs[qbyte(i)];
    }
    {
      const uint4* q4 = (const uint4*)qs;
      uint4 qv[MH];
#pragma unroll
      for (int c = 0; c < MH; ++c) qv[c] = q4[qchunk(jh + c * LH)];
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
            const float lg = (float)acc * es[d] * sf;
            if (logits) logits[row] = lg;
            argmax_step(best, bidx, lg, row);
          }
          // refill this slot with the row kHeadDepth iterations ahead
          const int nrow = row + kHeadDepth * STEPH;
          erow[d] = nrow;
          const bool live = nrow < r1;
          const uint4* e4 = (const uint4*)(E + (size_t)(live ? nrow : 0) * DM);
#pragma unroll
          for (int c = 0; c < MH; ++c) eb[d][c] = live ? e4[jh + c * LH] : make_uint4(0, 0, 0, 0);
          es[d] = live ? sE[nrow] : 0.0f;
        }
      }
      wave_argmax(best, bidx);
      if (lane == 0) {
        s_arg[wave] = best;
        ((int*)s_arg)[kPW + wave] = bidx;
      }
      wg_barrier();
      if (threadIdx.x == 0) {
        for (int wv = 1; wv < kPW; ++wv) argmax_step(best, bidx, s_arg[wv], ((int*)s_arg)[kPW + wv]);
        // argmax candidates: value word and index word per workgroup
        publish(abox, 2 * G, w, best, e);
        publish(abox, 2 * G, G + w, __int_as_float(bidx), e);
      }
    }
    prof(t, Lm, 3);
    // every workgroup reduces the G candidates itself
    {
      float* cand = gs;
      ok = gather<(2 * G + kPT - 1) / kPT>(abox, 2 * G, e, cand, a.abort_flag, s_stop);
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
          int32_t* to = kargs()->tok_out;
          if (w == 0 && to) to[t] = bidx;
        }
      }
      wg_barrier();
      tok = *s_tok;
      prof(t, Lm, 4);
    }
  }
  if (w == 0 && threadIdx.x == 0) {
    const KArgs k = kargs();
    if (ok) {
      if (k->tok_last) k->tok_last[0] = tok;
    } else {
      atomicOr(k->err, 2);
    }
  }
}

// the shapes this kernel is compiled for: the 2-layer test stack and the 1.3B shape
using ShapeTiny = PShape<256, 512, 16, 32>;
using Shape1p3b = PShape<2048, 4096, 128, 64>;

template <class S>
static const void* kernel_of(int mode) {
  return mode == 2 ? (const void*)decode_persistent_kernel<S, 2>
         : mode == 1 ? (const void*)decode_persistent_kernel<S, 1>
                     : (const void*)decode_persistent_kernel<S, 0>;
}

template <class S>
static bool shape_is(int dm, int di, int ns, int hp) {
  return dm == S::DM && di == S::DI && ns == S::NS && hp == S::HP;
}

static size_t lds_bytes(int dm, int di, int ns, int hp) {
  if (shape_is<Shape1p3b>(dm, di, ns, hp)) return Lds<Shape1p3b>::BYTES;
  if (shape_is<ShapeTiny>(dm, di, ns, hp)) return Lds<ShapeTiny>::BYTES;
  return 0;
}

static const void* select_kernel(int dm, int di, int ns, int hp, size_t* stride, int mode = 0) {
  if (shape_is<Shape1p3b>(dm, di, ns, hp)) { *stride = Shape1p3b::LSTRIDE; return kernel_of<Shape1p3b>(mode); }
  if (shape_is<ShapeTiny>(dm, di, ns, hp)) { *stride = ShapeTiny::LSTRIDE; return kernel_of<ShapeTiny>(mode); }
  return nullptr;
}

template <class S>
static size_t off_of(int k) { return S::OFF(k); }

bool persistent_layout(int d_model, int d_inner, int d_state, int headdim, size_t* stride, size_t* offsets) {
  size_t st = 0;
  if (!select_kernel(d_model, d_inner, d_state, headdim, &st)) return false;
  *stride = st;
  for (int k = 0; k < 19; ++k)
    offsets[k] = shape_is<Shape1p3b>(d_model, d_inner, d_state, headdim) ? off_of<Shape1p3b>(k) : off_of<ShapeTiny>(k);
  return true;
}

hipError_t launch_decode_persistent(const PersistArgs& a, int grid, hipStream_t st) {
  size_t stride = 0;
  const bool tr = a.trace_h || a.trace_q1 || a.trace_q2 || a.trace_qf || a.trace_acc1 || a.trace_acc2;
  const int mode = tr ? 2 : a.prof ? 1 : 0;
  const void* k = select_kernel(a.d_model, a.d_inner, a.d_state, a.headdim, &stride, mode);
  if (!k) return hipErrorInvalidValue;
  PersistArgs args = a;
  void* params[] = {&args};
  return hipLaunchCooperativeKernel(k, dim3(grid), dim3(kBlock), params,
                                    (unsigned)lds_bytes(a.d_model, a.d_inner, a.d_state, a.headdim), st);
}

// Whether the persistent kernel can run for these dimensions with `grid`
// co-resident workgroups on this device.  Fills *why on refusal.
bool persistent_supported(int d_model, int d_inner, int d_state, int headdim, int n_heads, int rank, int grid,
                          const char** why) {
  auto no = [&](const char* m) { *why = m; return false; };
  size_t stride = 0;
  const void* k = select_kernel(d_model, d_inner, d_state, headdim, &stride);
  if (!k) return no("the persistent kernel is compiled for d_model/d_inner/d_state/headdim 2048/4096/128/64 and 256/512/16/32");
  if (grid != n_heads * (headdim / 16)) return no("grid mismatch");
  if (rank != 16) return no("the persistent path needs LoRA rank 16");
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return no("no device");
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return no("no CU count");
  for (int mode = 0; mode < 3; ++mode) {  // every variant (plain, timestamps, traces) must fit
    k = select_kernel(d_model, d_inner, d_state, headdim, &stride, mode);
    const size_t lds = lds_bytes(d_model, d_inner, d_state, headdim);
    if (hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
      return no("the kernel's LDS carve-up does not fit a workgroup on this device");
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, kBlock, lds) !=
        hipSuccess)
      return no("occupancy query failed");
    if ((long)per_cu * cus < grid) return no("grid does not fit co-resident on this device");
  }
  return true;
}

size_t persistent_box_words(int d_model, int d_inner, int d_state, int grid) {
  return (size_t)kR * ((size_t)d_model / 2 + (size_t)d_inner / 2 + 2 * (size_t)d_state + 2 * (size_t)grid);
}

}  // namespace dfssm
