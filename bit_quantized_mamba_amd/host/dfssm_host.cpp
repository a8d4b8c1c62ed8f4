// Host CPU backend of the DF-SSM decode step.
//
// gist.science technical summary §2.C, CPU (AVX-512): the packed 1-bit
// scaffold is expanded to int8 in registers and multiplied on the VNNI byte
// dot product, so the weights stream from memory at one bit each; §3: the
// CPU speed-up this buys.  The model and its arithmetic are those of the
// device library (include/dfssm.h): int8 activation codes (per token,
// symmetric absmax), exact int32 scaffold sums 2 pos - sum(q), the LoRA
// correction sB * B (float(A q) sA s), the depthwise causal conv with SiLU,
// the Mamba-2 recurrence in fp32, the gated RMSNorm, the tied int8 LM head
// and the greedy argmax (lowest index on ties).
//
// Layout of the work: one OpenMP parallel region per call; each phase of a
// layer is a work-shared loop over independent outputs (weight rows, conv
// channels, heads), so every output element is computed by one thread in a
// fixed order and the results do not depend on the thread count.  Row
// reductions (the norms) sum fixed blocks of a row in parallel and combine
// the blocks in order.  Only the integer products differ between the two
// instruction paths, and integers are exact, so both paths give the same
// bits.
#include <immintrin.h>
#include <omp.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/dfssm_host.h"

namespace {

thread_local std::string g_err;

dfssm_status fail(dfssm_status s, std::string m) {
  g_err = std::move(m);
  return s;
}

// ---------------------------------------------------------------------------
// integer products (the only code that differs between the two paths)
// ---------------------------------------------------------------------------

// sum of q[i] over the set bits of a K-bit scaffold row (K % 64 == 0);
// weight i is bit i % 32 of word i / 32
int pos_portable(const uint32_t* w, const int8_t* q, int K) {
  int pos = 0;
  for (int j = 0; j < K / 32; ++j) {
    const uint32_t b = w[j];
    const int8_t* qq = q + 32 * j;
    int s = 0;
    for (int k = 0; k < 32; ++k) s += (int)((b >> k) & 1u) * (int)qq[k];
    pos += s;
  }
  return pos;
}

void pos_rows_portable(const uint32_t* bits, int o0, int o1, const int8_t* q, int K, int32_t* out) {
  for (int o = o0; o < o1; ++o) out[o - o0] = pos_portable(bits + (size_t)o * (K / 32), q, K);
}

// sum of qu[i] * a[i] with qu unsigned bytes (K % 64 == 0)
int dotu_portable(const uint8_t* qu, const int8_t* a, int K) {
  int s = 0;
  for (int i = 0; i < K; ++i) s += (int)qu[i] * (int)a[i];
  return s;
}

// The bits of 64 weights become a 0/1 byte vector (the 64-bit mask loaded
// straight into a mask register, then a masked move of a vector of ones);
// dpbusd multiplies it by 64 int8 codes and sums groups of 4 into 16 int32
// lanes.  Four accumulators keep four dot products in flight (the
// instruction's latency is several cycles).
__attribute__((target("avx512f,avx512bw,avx512vnni"), always_inline)) inline int pos_vnni(const uint32_t* w, const int8_t* q, int K) {
  const __m512i ones = _mm512_set1_epi8(1);
  auto mask = [w](int j) -> __mmask64 {
    uint64_t v;
    std::memcpy(&v, w + 2 * j, 8);
    return (__mmask64)v;
  };
  __m512i a0 = _mm512_setzero_si512(), a1 = a0, a2 = a0, a3 = a0;
  const int n = K / 64;
  int j = 0;
  for (; j + 3 < n; j += 4) {
    a0 = _mm512_dpbusd_epi32(a0, _mm512_maskz_mov_epi8(mask(j), ones), _mm512_loadu_si512(q + 64 * j));
    a1 = _mm512_dpbusd_epi32(a1, _mm512_maskz_mov_epi8(mask(j + 1), ones),
                             _mm512_loadu_si512(q + 64 * j + 64));
    a2 = _mm512_dpbusd_epi32(a2, _mm512_maskz_mov_epi8(mask(j + 2), ones),
                             _mm512_loadu_si512(q + 64 * j + 128));
    a3 = _mm512_dpbusd_epi32(a3, _mm512_maskz_mov_epi8(mask(j + 3), ones),
                             _mm512_loadu_si512(q + 64 * j + 192));
  }
  for (; j < n; ++j)
    a0 = _mm512_dpbusd_epi32(a0, _mm512_maskz_mov_epi8(mask(j), ones), _mm512_loadu_si512(q + 64 * j));
  return _mm512_reduce_add_epi32(_mm512_add_epi32(_mm512_add_epi32(a0, a1), _mm512_add_epi32(a2, a3)));
}

// rows [o0, o1) of a scaffold matrix (K / 32 words per row) against one code row
__attribute__((target("avx512f,avx512bw,avx512vnni"))) void pos_rows_vnni(const uint32_t* bits, int o0, int o1,
                                                                          const int8_t* q, int K, int32_t* out) {
  for (int o = o0; o < o1; ++o) out[o - o0] = pos_vnni(bits + (size_t)o * (K / 32), q, K);
}

__attribute__((target("avx512f,avx512bw,avx512vnni"))) int dotu_vnni(const uint8_t* qu, const int8_t* a, int K) {
  __m512i a0 = _mm512_setzero_si512(), a1 = a0, a2 = a0, a3 = a0;
  const int n = K / 64;
  int j = 0;
  for (; j + 3 < n; j += 4) {
    a0 = _mm512_dpbusd_epi32(a0, _mm512_loadu_si512(qu + 64 * j), _mm512_loadu_si512(a + 64 * j));
    a1 = _mm512_dpbusd_epi32(a1, _mm512_loadu_si512(qu + 64 * j + 64), _mm512_loadu_si512(a + 64 * j + 64));
    a2 = _mm512_dpbusd_epi32(a2, _mm512_loadu_si512(qu + 64 * j + 128), _mm512_loadu_si512(a + 64 * j + 128));
    a3 = _mm512_dpbusd_epi32(a3, _mm512_loadu_si512(qu + 64 * j + 192), _mm512_loadu_si512(a + 64 * j + 192));
  }
  for (; j < n; ++j) a0 = _mm512_dpbusd_epi32(a0, _mm512_loadu_si512(qu + 64 * j), _mm512_loadu_si512(a + 64 * j));
  return _mm512_reduce_add_epi32(_mm512_add_epi32(_mm512_add_epi32(a0, a1), _mm512_add_epi32(a2, a3)));
}

bool cpu_has_vnni() {
  __builtin_cpu_init();
  return __builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw") &&
         __builtin_cpu_supports("avx512vnni");
}

struct IntOps {
  void (*pos_rows)(const uint32_t*, int, int, const int8_t*, int, int32_t*);
  int (*dotu)(const uint8_t*, const int8_t*, int);
};

// ---------------------------------------------------------------------------
// the seeded synthetic generator (its definition is in dfssm.h)
// ---------------------------------------------------------------------------

inline uint64_t mix64(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
inline uint64_t stream_key(uint64_t seed, uint64_t tid) { return mix64(seed ^ (tid << 32)); }
inline double unit24(uint64_t d) { return (double)(d >> 40) * 0x1p-24; }

enum Dist { D_WORDS, D_INT8, D_UNIFORM, D_CONST, D_NORMAL };

void gen_fill(void* dst, size_t n, Dist dist, uint64_t key, double a, double b) {
#pragma omp parallel for schedule(static)
  for (size_t i = 0; i < n; ++i) {
    switch (dist) {
      case D_WORDS: ((uint32_t*)dst)[i] = (uint32_t)(mix64(key + i) >> 32); break;
      case D_INT8: ((int8_t*)dst)[i] = (int8_t)((int)(mix64(key + i) % 255u) - 127); break;
      case D_UNIFORM: ((float*)dst)[i] = (float)(a + (b - a) * unit24(mix64(key + i))); break;
      case D_CONST: ((float*)dst)[i] = (float)a; break;
      case D_NORMAL: {
        double s = 0.0;  // Irwin-Hall: 12 uniforms in order, exact in fp64
        for (int k = 0; k < 12; ++k) s = s + unit24(mix64(key + 12 * i + k));
        ((float*)dst)[i] = (float)(s - 6.0);
        break;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// shared floating-point pieces
// ---------------------------------------------------------------------------

inline float silu(float v) { return v / (1.0f + std::exp(-v)); }
inline float softplus(float v) { return v > 20.0f ? v : std::log1p(std::exp(v)); }


}  // namespace

// ---------------------------------------------------------------------------
// the context
// ---------------------------------------------------------------------------

struct dfssm_host {
  dfssm_config cfg{};
  int L = 0, dm = 0, di = 0, N = 0, P = 0, V = 0, Kc = 0, r = 0, H = 0, cd = 0, dp = 0, maxB = 0;
  float eps = 1e-5f;
  int threads = 1;
  int isa = DFSSM_HOST_ISA_PORTABLE;

  struct Tensor {
    std::vector<unsigned char> buf;
    size_t elem = 0, count = 0;
    template <class T> T* p() { return (T*)buf.data(); }
    template <class T> const T* p() const { return (const T*)buf.data(); }
  };
  std::vector<std::vector<Tensor>> lt;  // [layer][kind]
  std::vector<Tensor> gt;               // model-wide
  std::vector<std::vector<int32_t>> asum_in, asum_out;  // row sums of the LoRA-down matrices
  std::vector<std::vector<int8_t>> bt_in, bt_out;        // LoRA-up matrices transposed: [r][d_out]
  std::vector<int32_t> esum;                            // row sums of the embedding

  std::vector<float> conv, ssm;  // state
  // workspace
  std::vector<float> h, zx, xc, g, s, stats, lg;
  std::vector<int32_t> part;                 // [B][chunks][33]: per-chunk LoRA-down dots and code sum
  std::vector<int32_t> tl_qsum;              // per thread [B]: code sums
  std::vector<float> tl_t;                   // per thread [B][32]: LoRA-down vectors
  std::vector<int8_t> q;
  std::vector<uint8_t> qu;
  std::vector<float> best_v;
  std::vector<int32_t> best_i;

  size_t conv_per_seq() const { return (size_t)L * cd * (Kc - 1); }
  size_t ssm_per_seq() const { return (size_t)L * H * P * N; }
};

namespace {

struct Spec {
  size_t elem, count;
};

Spec layer_spec(const dfssm_host* c, int kind) {
  const size_t dm = c->dm, di = c->di, dp = c->dp, r = c->r, cd = c->cd, H = c->H, K = c->Kc;
  switch (kind) {
    case DFSSM_T_IN_BITS: return {4, dp * (dm / 32)};
    case DFSSM_T_IN_SW: return {4, dp};
    case DFSSM_T_IN_A: return {1, r * dm};
    case DFSSM_T_IN_SA: return {4, r};
    case DFSSM_T_IN_B: return {1, dp * r};
    case DFSSM_T_IN_SB: return {4, dp};
    case DFSSM_T_OUT_BITS: return {4, dm * (di / 32)};
    case DFSSM_T_OUT_SW: return {4, dm};
    case DFSSM_T_OUT_A: return {1, r * di};
    case DFSSM_T_OUT_SA: return {4, r};
    case DFSSM_T_OUT_B: return {1, dm * r};
    case DFSSM_T_OUT_SB: return {4, dm};
    case DFSSM_T_CONV_W: return {4, cd * K};
    case DFSSM_T_CONV_B: return {4, cd};
    case DFSSM_T_A_LOG: return {4, H};
    case DFSSM_T_DT_BIAS: return {4, H};
    case DFSSM_T_D: return {4, H};
    case DFSSM_T_NORM_W: return {4, dm};
    case DFSSM_T_GNORM_W: return {4, di};
    default: return {0, 0};
  }
}

Spec global_spec(const dfssm_host* c, int kind) {
  switch (kind) {
    case DFSSM_G_EMBED: return {1, (size_t)c->V * c->dm};
    case DFSSM_G_EMBED_SCALE: return {4, (size_t)c->V};
    case DFSSM_G_FINAL_NORM: return {4, (size_t)c->dm};
    default: return {0, 0};
  }
}

dfssm_host::Tensor* tensor(dfssm_host* c, int layer, int kind) {
  if (layer == -1) return kind >= 0 && kind < 3 ? &c->gt[kind] : nullptr;
  if (layer < 0 || layer >= c->L || kind < 0 || kind >= DFSSM_T_PER_LAYER) return nullptr;
  return &c->lt[layer][kind];
}

// derived sums that the offset trick of the int8 x int8 products needs
void refresh_sums(dfssm_host* c, int layer, int kind) {
  auto rows = [](const int8_t* m, int nr, int nc, std::vector<int32_t>& out) {
    out.assign(nr, 0);
    for (int i = 0; i < nr; ++i) {
      int s = 0;
      for (int k = 0; k < nc; ++k) s += m[(size_t)i * nc + k];
      out[i] = s;
    }
  };
  if (layer == -1 && kind == DFSSM_G_EMBED) {
    c->esum.assign(c->V, 0);
    const int8_t* E = c->gt[DFSSM_G_EMBED].p<int8_t>();
#pragma omp parallel for schedule(static) num_threads(c->threads)
    for (int v = 0; v < c->V; ++v) {
      int s = 0;
      for (int k = 0; k < c->dm; ++k) s += E[(size_t)v * c->dm + k];
      c->esum[v] = s;
    }
  } else if (layer >= 0 && kind == DFSSM_T_IN_A) {
    rows(c->lt[layer][kind].p<int8_t>(), c->r, c->dm, c->asum_in[layer]);
  } else if (layer >= 0 && kind == DFSSM_T_OUT_A) {
    rows(c->lt[layer][kind].p<int8_t>(), c->r, c->di, c->asum_out[layer]);
  } else if (layer >= 0 && (kind == DFSSM_T_IN_B || kind == DFSSM_T_OUT_B)) {
    const int n = kind == DFSSM_T_IN_B ? c->dp : c->dm;
    const int8_t* Bm = c->lt[layer][kind].p<int8_t>();
    std::vector<int8_t>& t = kind == DFSSM_T_IN_B ? c->bt_in[layer] : c->bt_out[layer];
    t.resize((size_t)c->r * n);
    for (int o = 0; o < n; ++o)
      for (int k = 0; k < c->r; ++k) t[(size_t)k * n + o] = Bm[(size_t)o * c->r + k];
  }
}

// Per-layer tensor distributions of the synthetic generator.
struct GenSpec {
  Dist d;
  double a, b;
};
GenSpec layer_gen(int kind) {
  const double ln16 = 2.772588722239781;
  switch (kind) {
    case DFSSM_T_IN_BITS:
    case DFSSM_T_OUT_BITS: return {D_WORDS, 0, 0};
    case DFSSM_T_IN_SW:
    case DFSSM_T_OUT_SW: return {D_UNIFORM, 0.01, 0.05};
    case DFSSM_T_IN_A:
    case DFSSM_T_IN_B:
    case DFSSM_T_OUT_A:
    case DFSSM_T_OUT_B: return {D_INT8, 0, 0};
    case DFSSM_T_IN_SA:
    case DFSSM_T_IN_SB:
    case DFSSM_T_OUT_SA:
    case DFSSM_T_OUT_SB: return {D_CONST, (double)1e-3f, 0};
    case DFSSM_T_CONV_W:
    case DFSSM_T_CONV_B: return {D_UNIFORM, -0.5, 0.5};
    case DFSSM_T_A_LOG: return {D_UNIFORM, 0.0, ln16};
    case DFSSM_T_DT_BIAS: return {D_UNIFORM, -4.0, -1.0};
    case DFSSM_T_D: return {D_NORMAL, 0, 0};
    default: return {D_UNIFORM, 0.5, 1.5};  // norm weights
  }
}

// ---------------------------------------------------------------------------
// one decode step of B sequences
// ---------------------------------------------------------------------------

struct Trace {
  float* h = nullptr;
  int8_t *q1 = nullptr, *q2 = nullptr, *qf = nullptr;
  int32_t *acc1 = nullptr, *acc2 = nullptr;
};

constexpr int kChunk = 256;  // codes per work item of the quantiser

// Sum of squares and max |x w| of one fixed block of a row, written where
// the row's quantiser finds them (stats [B][nb][2]).  Producers of a row
// call it for their blocks as they finish them, so the statistics cost no
// extra pass and no extra barrier.
inline void block_stats(const float* x, const float* w, int n, float* out) {
  float ss = 0.0f, pm = 0.0f;
  for (int k = 0; k < n; ++k) {
    ss += x[k] * x[k];
    pm = std::max(pm, std::fabs(x[k] * w[k]));
  }
  out[0] = ss;
  out[1] = pm;
}

// Inside the parallel region: RMSNorm + int8 quantisation of B rows x[b]
// (length K, weight w) whose nb block statistics are in stats [B][nb][2]
// (summed here in block order): codes into c->q (row stride K), the unsigned
// copy q + 128 into c->qu, scales into c->s.  u = rstd (x w) with
// rstd = 1 / sqrt(mean(x^2) + eps); amax = rstd max |x w|;
// q = clamp(rint(u (127 / amax)), -127, 127), s = amax / 127 (zero row: 0).
// Each chunk of kChunk codes also leaves its code sum and, with A (the LoRA
// down matrix, r rows of K), its r integer dot products with the codes (in
// the unsigned-offset form) in c->part [B][nchunk][33]; row_terms adds the
// chunks up.  One barrier.
void quant_rows(dfssm_host* c, const IntOps& ops, const float* x, const float* w, int K, int B, const int8_t* A,
                const float* stats, int nb) {
  const int r = c->r;
  const int nchunk = (K + kChunk - 1) / kChunk;
#pragma omp for schedule(static)
  for (int i = 0; i < B * nchunk; ++i) {
    const int b = i / nchunk, ci = i % nchunk, k0 = ci * kChunk, k1 = std::min(K, k0 + kChunk);
    float ss = 0.0f, pm = 0.0f;
    for (int j = 0; j < nb; ++j) {
      ss += stats[2 * (b * nb + j)];
      pm = std::max(pm, stats[2 * (b * nb + j) + 1]);
    }
    const float rstd = 1.0f / std::sqrt(ss / (float)K + c->eps);
    const float amax = rstd * pm;
    const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
    const float* xr = x + (size_t)b * K;
    int8_t* qr = c->q.data() + (size_t)b * K;
    uint8_t* ur = c->qu.data() + (size_t)b * K;
    int sq = 0;
    for (int k = k0; k < k1; ++k) {
      float v = std::rint(rstd * (xr[k] * w[k]) * inv);
      v = std::min(std::max(v, -127.0f), 127.0f);
      qr[k] = (int8_t)(int)v;
      ur[k] = (uint8_t)((int)qr[k] + 128);
      sq += qr[k];
    }
    int32_t* part = c->part.data() + ((size_t)b * nchunk + ci) * 33;
    part[32] = sq;
    if (A)
      for (int k = 0; k < r; ++k) part[k] = ops.dotu(ur + k0, A + (size_t)k * K + k0, k1 - k0);
    if (ci == 0) c->s[b] = amax > 0.0f ? amax / 127.0f : 0.0f;
  }
  // (implicit barrier)
}

// Per thread, after quant_rows: the code sums and the LoRA-down vectors of
// the B rows, t[b][k] = float(sum_i A[k][i] q_b[i]) sA[k] s_b (the chunks'
// integers added, the offset's 128 sum_i A[k][i] taken off: exact).
void row_terms(dfssm_host* c, int K, int B, const int32_t* asum, const float* sA, int32_t* qsum, float* t) {
  const int nchunk = (K + kChunk - 1) / kChunk, r = c->r;
  for (int b = 0; b < B; ++b) {
    int sq = 0;
    int acc[32] = {};
    for (int ci = 0; ci < nchunk; ++ci) {
      const int32_t* part = c->part.data() + ((size_t)b * nchunk + ci) * 33;
      sq += part[32];
      for (int k = 0; k < r; ++k) acc[k] += part[k];
    }
    qsum[b] = sq;
    for (int k = 0; k < r; ++k) t[(size_t)b * 32 + k] = (float)(acc[k] - 128 * asum[k]) * sA[k] * c->s[b];
  }
}

constexpr int kRowBlock = 16;  // scaffold rows per integer call

// scaffold + LoRA projection of B code rows (length K) to rows [0, n):
// y = float(2 pos - sum q) sw s + sB sum_k B[o][k] t_k (k in order, from the
// transposed copy Bt [r][n] so that a block of rows is one vector), then
// `out(b, o, y, acc)` per row and `done(b, block, o0, count)` per block of
// kRowBlock rows
template <class Out, class Done>
void project(dfssm_host* c, const IntOps& ops, const uint32_t* bits, const float* sw, const int8_t* Bt,
             const float* sB, const int32_t* asum, const float* sA, int K, int n, int B, Out out, Done done) {
  const int r = c->r;
  const int nblk = (n + kRowBlock - 1) / kRowBlock;
  const size_t me = (size_t)omp_get_thread_num();
  int32_t* qsum = c->tl_qsum.data() + me * c->maxB;
  float* tt = c->tl_t.data() + me * c->maxB * 32;
  row_terms(c, K, B, asum, sA, qsum, tt);
#pragma omp for schedule(static)
  for (int blk = 0; blk < nblk; ++blk) {
    const int o0 = blk * kRowBlock, cnt = std::min(n, o0 + kRowBlock) - o0;
    for (int b = 0; b < B; ++b) {
      int32_t pos[kRowBlock];
      ops.pos_rows(bits, o0, o0 + cnt, c->q.data() + (size_t)b * K, K, pos);
      const float* tb = tt + (size_t)b * 32;
      float lo[kRowBlock] = {};
      for (int k = 0; k < r; ++k) {
        const int8_t* bk = Bt + (size_t)k * n + o0;
        const float tk = tb[k];
        for (int i = 0; i < cnt; ++i) lo[i] += (float)bk[i] * tk;
      }
      for (int i = 0; i < cnt; ++i) {
        const int o = o0 + i, acc = 2 * pos[i] - qsum[b];
        out(b, o, (float)acc * sw[o] * c->s[b] + sB[o] * lo[i], acc);
      }
      done(b, blk, o0, cnt);
    }
  }
}

// head: the final norm, LM head and argmax run (a prefill skips them for all
// but its last position)
void step(dfssm_host* c, const IntOps& ops, const int32_t* tok, int B, const Trace* tr, float* logits,
          int32_t* next, bool head = true) {
  const int dm = c->dm, di = c->di, N = c->N, P = c->P, H = c->H, cd = c->cd, dp = c->dp, V = c->V, Lm = c->L;
  const int8_t* E = c->gt[DFSSM_G_EMBED].p<int8_t>();
  const float* sE = c->gt[DFSSM_G_EMBED_SCALE].p<float>();
  float* hb = c->h.data();
  float* lg = logits ? logits : c->lg.data();
  const int nthr = c->threads;
  // norm statistics of the residual rows by blocks of kRowBlock, of the gated rows by heads
  float* st1 = c->stats.data();
  float* st2 = c->stats.data() + (size_t)B * (dm / kRowBlock) * 2;
  const int nb1 = dm / kRowBlock, nb2 = H;
#pragma omp parallel num_threads(nthr)
  {
    const float* w0 = Lm > 0 ? c->lt[0][DFSSM_T_NORM_W].p<float>() : c->gt[DFSSM_G_FINAL_NORM].p<float>();
#pragma omp for schedule(static)
    for (int i = 0; i < B * nb1; ++i) {
      const int b = i / nb1, o0 = (i % nb1) * kRowBlock, tk = tok[b];
      float* hr = hb + (size_t)b * dm + o0;
      for (int k = 0; k < kRowBlock; ++k) hr[k] = (float)E[(size_t)tk * dm + o0 + k] * sE[tk];
      block_stats(hr, w0 + o0, kRowBlock, st1 + 2 * (size_t)i);
    }
    for (int l = 0; l < Lm; ++l) {
      auto& T = c->lt[l];
      if (tr && tr->h) {
#pragma omp for schedule(static)
        for (int b = 0; b < B; ++b) std::memcpy(tr->h + ((size_t)l * B + b) * dm, hb + (size_t)b * dm, 4 * dm);
      }
      // ---- pre-norm, quantise, LoRA down, in_proj
      quant_rows(c, ops, hb, T[DFSSM_T_NORM_W].p<float>(), dm, B, T[DFSSM_T_IN_A].p<int8_t>(), st1, nb1);
      if (tr && tr->q1) {
#pragma omp for schedule(static)
        for (int b = 0; b < B; ++b) std::memcpy(tr->q1 + ((size_t)l * B + b) * dm, c->q.data() + (size_t)b * dm, dm);
      }
      float* zx = c->zx.data();
      float* xc = c->xc.data();
      const float* cw = T[DFSSM_T_CONV_W].p<float>();
      const float* cb = T[DFSSM_T_CONV_B].p<float>();
      int32_t* a1 = tr && tr->acc1 ? tr->acc1 + (size_t)l * B * dp : nullptr;
      // in_proj rows, and for rows di .. di + cd ([x, B, C]) the conv shift
      // register + SiLU of that channel, by the thread that made the row
      project(c, ops, T[DFSSM_T_IN_BITS].p<uint32_t>(), T[DFSSM_T_IN_SW].p<float>(), c->bt_in[l].data(),
              T[DFSSM_T_IN_SB].p<float>(), c->asum_in[l].data(), T[DFSSM_T_IN_SA].p<float>(), dm, dp, B,
              [&](int b, int o, float y, int acc) {
                zx[(size_t)b * dp + o] = y;
                if (a1) a1[(size_t)b * dp + o] = acc;
                const int ch = o - di;
                if (ch >= 0 && ch < cd) {
                  float* win = c->conv.data() + (size_t)b * c->conv_per_seq() + ((size_t)l * cd + ch) * 3;
                  const float* wc = cw + (size_t)ch * 4;
                  const float a = cb[ch] + wc[0] * win[0] + wc[1] * win[1] + wc[2] * win[2] + wc[3] * y;
                  win[0] = win[1];
                  win[1] = win[2];
                  win[2] = y;
                  xc[(size_t)b * cd + ch] = silu(a);
                }
              },
              [](int, int, int, int) {});
      // ---- SSM recurrence and gate, one (sequence, head) per iteration
      const float* alog = T[DFSSM_T_A_LOG].p<float>();
      const float* dtb = T[DFSSM_T_DT_BIAS].p<float>();
      const float* Dv = T[DFSSM_T_D].p<float>();
      const float* gw = T[DFSSM_T_GNORM_W].p<float>();
      float* g = c->g.data();
#pragma omp for schedule(static)
      for (int i = 0; i < B * H; ++i) {
        const int b = i / H, hd = i % H;
        const float dt = softplus(zx[(size_t)b * dp + di + cd + hd] + dtb[hd]);
        const float dA = std::exp(-dt * std::exp(alog[hd]));
        const float* xr = xc + (size_t)b * cd;
        const float* Bv = xr + di;
        const float* Cv = xr + di + N;
        float* S = c->ssm.data() + (size_t)b * c->ssm_per_seq() + (((size_t)l * H + hd) * P) * N;
        for (int p = 0; p < P; ++p) {
          const int ch = hd * P + p;
          const float x = xr[ch];
          const float xdt = dt * x;
          float* Sr = S + (size_t)p * N;
          float part[16] = {};
          for (int n0 = 0; n0 < N; n0 += 16)
            for (int j = 0; j < 16; ++j) {
              const float sv = dA * Sr[n0 + j] + xdt * Bv[n0 + j];
              Sr[n0 + j] = sv;
              part[j] += sv * Cv[n0 + j];
            }
          for (int w = 8; w > 0; w >>= 1)
            for (int j = 0; j < w; ++j) part[j] += part[j + w];
          const float y = part[0] + Dv[hd] * x;
          g[(size_t)b * di + ch] = y * silu(zx[(size_t)b * dp + ch]);
        }
        block_stats(g + (size_t)b * di + hd * P, gw + hd * P, P, st2 + 2 * (size_t)i);
      }
      // ---- gated RMSNorm, quantise, LoRA down, out_proj + residual
      quant_rows(c, ops, g, gw, di, B, T[DFSSM_T_OUT_A].p<int8_t>(), st2, nb2);
      if (tr && tr->q2) {
#pragma omp for schedule(static)
        for (int b = 0; b < B; ++b) std::memcpy(tr->q2 + ((size_t)l * B + b) * di, c->q.data() + (size_t)b * di, di);
      }
      int32_t* a2 = tr && tr->acc2 ? tr->acc2 + (size_t)l * B * dm : nullptr;
      const float* wn = l + 1 < Lm ? c->lt[l + 1][DFSSM_T_NORM_W].p<float>() : c->gt[DFSSM_G_FINAL_NORM].p<float>();
      project(c, ops, T[DFSSM_T_OUT_BITS].p<uint32_t>(), T[DFSSM_T_OUT_SW].p<float>(), c->bt_out[l].data(),
              T[DFSSM_T_OUT_SB].p<float>(), c->asum_out[l].data(), T[DFSSM_T_OUT_SA].p<float>(), di, dm, B,
              [&](int b, int o, float y, int acc) {
                hb[(size_t)b * dm + o] += y;
                if (a2) a2[(size_t)b * dm + o] = acc;
              },
              [&](int b, int blk, int o0, int cnt) {  // statistics for the next norm
                block_stats(hb + (size_t)b * dm + o0, wn + o0, cnt, st1 + 2 * ((size_t)b * nb1 + blk));
              });
    }
    if (tr && tr->h) {
#pragma omp for schedule(static)
      for (int b = 0; b < B; ++b) std::memcpy(tr->h + ((size_t)Lm * B + b) * dm, hb + (size_t)b * dm, 4 * dm);
    }
    if (head) {
      // ---- final norm, quantise, tied int8 LM head, greedy argmax
      quant_rows(c, ops, hb, c->gt[DFSSM_G_FINAL_NORM].p<float>(), dm, B, nullptr, st1, nb1);
      if (tr && tr->qf) {
#pragma omp for schedule(static)
        for (int b = 0; b < B; ++b) std::memcpy(tr->qf + (size_t)b * dm, c->q.data() + (size_t)b * dm, dm);
      }
#pragma omp for schedule(static)
      for (int v = 0; v < V; ++v) {
        const int8_t* er = E + (size_t)v * dm;
        for (int b = 0; b < B; ++b) {
          const int dot = ops.dotu(c->qu.data() + (size_t)b * dm, er, dm) - 128 * c->esum[v];
          lg[(size_t)b * V + v] = (float)dot * sE[v] * c->s[b];
        }
      }
      if (next) {
        // per thread the first maximum of its static share, then the threads'
        // candidates in thread order (ties keep the lower index)
        const int nt = omp_get_num_threads(), me = omp_get_thread_num();
        const int per = (V + nt - 1) / nt, v0 = std::min(V, me * per), v1 = std::min(V, v0 + per);
        for (int b = 0; b < B; ++b) {
          float bv = -INFINITY;
          int bi = -1;
          for (int v = v0; v < v1; ++v) {
            const float x = lg[(size_t)b * V + v];
            if (x > bv) {
              bv = x;
              bi = v;
            }
          }
          c->best_v[(size_t)b * nt + me] = bv;
          c->best_i[(size_t)b * nt + me] = bi;
        }
#pragma omp barrier
#pragma omp for schedule(static)
        for (int b = 0; b < B; ++b) {
          float bv = -INFINITY;
          int bi = -1;
          for (int j = 0; j < nt; ++j) {
            const int ci = c->best_i[(size_t)b * nt + j];
            if (ci >= 0 && (bi < 0 || c->best_v[(size_t)b * nt + j] > bv)) {
              bv = c->best_v[(size_t)b * nt + j];
              bi = ci;
            }
          }
          next[b] = bi < 0 ? 0 : bi;
        }
      }
    }  // head
  }
}

dfssm_status check_step(dfssm_host* c, const int32_t* tok, int B) {
  if (!c) return fail(DFSSM_E_INVALID, "null context");
  if (!tok) return fail(DFSSM_E_INVALID, "null token pointer");
  if (B < 1 || B > c->maxB) return fail(DFSSM_E_INVALID, "batch must be in [1, max_batch]");
  for (int b = 0; b < B; ++b)
    if (tok[b] < 0 || tok[b] >= c->V) return fail(DFSSM_E_INVALID, "token id outside [0, vocab)");
  return DFSSM_OK;
}

IntOps ops_of(const dfssm_host* c) {
  if (c->isa == DFSSM_HOST_ISA_AVX512VNNI) return {pos_rows_vnni, dotu_vnni};
  return {pos_rows_portable, dotu_portable};
}

// workspace for B rows (grown on demand; logits only when the caller passes none)
void ensure_ws(dfssm_host* c, int B, bool need_logits) {
  const int nt = c->threads;
  if (need_logits && c->lg.size() < (size_t)B * c->V) c->lg.resize((size_t)B * c->V);
  if (c->best_v.size() < (size_t)B * nt) {
    c->best_v.resize((size_t)B * nt);
    c->best_i.resize((size_t)B * nt);
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------

extern "C" {

const char* dfssm_host_last_error(void) { return g_err.c_str(); }

dfssm_status dfssm_host_create(const dfssm_config* cfg, int32_t n_threads, dfssm_host** out) {
  if (!cfg || !out) return fail(DFSSM_E_INVALID, "null argument");
  *out = nullptr;
  const dfssm_config& k = *cfg;
  // (d_model, d_inner <= 32768 keeps every offset int8 dot product, 255 * 127 * K, inside int32)
  if (k.n_layer < 1 || k.d_model < 64 || k.d_model % 64 || k.d_model > 32768 || k.d_inner < 64 || k.d_inner % 64 ||
      k.d_inner > 32768 || k.d_state < 16 ||
      k.d_state % 16 || k.headdim < 1 || k.d_inner % k.headdim || k.vocab < 1 || k.d_conv != 4 || k.lora_rank < 1 ||
      k.lora_rank > 32 || k.max_batch < 1 || k.max_batch > 1024)
    return fail(DFSSM_E_UNSUPPORTED, "shape outside the host backend's support (see dfssm_host.h)");
  if (n_threads < 0 || n_threads > 1024) return fail(DFSSM_E_INVALID, "n_threads must be in [0, 1024]");
  dfssm_host* c = nullptr;
  try {
    c = new dfssm_host();
    c->cfg = k;
    c->L = k.n_layer;
    c->dm = k.d_model;
    c->di = k.d_inner;
    c->N = k.d_state;
    c->P = k.headdim;
    c->V = k.vocab;
    c->Kc = k.d_conv;
    c->r = k.lora_rank;
    c->H = k.d_inner / k.headdim;
    c->cd = k.d_inner + 2 * k.d_state;
    c->dp = 2 * k.d_inner + 2 * k.d_state + c->H;
    c->maxB = k.max_batch;
    c->eps = k.norm_eps > 0.0f ? k.norm_eps : 1e-5f;
    c->threads = n_threads > 0 ? n_threads : omp_get_max_threads();
    c->isa = cpu_has_vnni() ? DFSSM_HOST_ISA_AVX512VNNI : DFSSM_HOST_ISA_PORTABLE;
    c->lt.resize(c->L);
    for (int l = 0; l < c->L; ++l) {
      c->lt[l].resize(DFSSM_T_PER_LAYER);
      for (int kind = 0; kind < DFSSM_T_PER_LAYER; ++kind) {
        const Spec s = layer_spec(c, kind);
        c->lt[l][kind].elem = s.elem;
        c->lt[l][kind].count = s.count;
        c->lt[l][kind].buf.assign(s.elem * s.count, 0);
      }
    }
    c->gt.resize(3);
    for (int kind = 0; kind < 3; ++kind) {
      const Spec s = global_spec(c, kind);
      c->gt[kind].elem = s.elem;
      c->gt[kind].count = s.count;
      c->gt[kind].buf.assign(s.elem * s.count, 0);
    }
    c->asum_in.assign(c->L, std::vector<int32_t>(c->r, 0));
    c->asum_out.assign(c->L, std::vector<int32_t>(c->r, 0));
    c->bt_in.assign(c->L, std::vector<int8_t>((size_t)c->r * c->dp, 0));
    c->bt_out.assign(c->L, std::vector<int8_t>((size_t)c->r * c->dm, 0));
    c->esum.assign(c->V, 0);
    c->conv.assign((size_t)c->maxB * c->conv_per_seq(), 0.0f);
    c->ssm.assign((size_t)c->maxB * c->ssm_per_seq(), 0.0f);
    const size_t B = c->maxB, wide = std::max(c->dm, c->di);
    c->h.assign(B * c->dm, 0.0f);
    c->zx.assign(B * c->dp, 0.0f);
    c->xc.assign(B * c->cd, 0.0f);
    c->g.assign(B * c->di, 0.0f);
    c->s.assign(B, 0.0f);
    c->stats.assign(B * ((size_t)c->dm / kRowBlock + c->H) * 2, 0.0f);
    c->part.assign(B * ((wide + kChunk - 1) / kChunk) * 33, 0);
    c->tl_qsum.assign((size_t)c->threads * B, 0);
    c->tl_t.assign((size_t)c->threads * B * 32, 0.0f);
    c->q.assign(B * wide, 0);
    c->qu.assign(B * wide, 0);
  } catch (const std::bad_alloc&) {
    delete c;
    return fail(DFSSM_E_OOM, "host allocation failed");
  }
  *out = c;
  return DFSSM_OK;
}

void dfssm_host_destroy(dfssm_host* h) { delete h; }

dfssm_status dfssm_host_set_isa(dfssm_host* h, int32_t isa) {
  if (!h) return fail(DFSSM_E_INVALID, "null context");
  if (isa == DFSSM_HOST_ISA_AUTO) {
    h->isa = cpu_has_vnni() ? DFSSM_HOST_ISA_AVX512VNNI : DFSSM_HOST_ISA_PORTABLE;
    return DFSSM_OK;
  }
  if (isa == DFSSM_HOST_ISA_PORTABLE) {
    h->isa = isa;
    return DFSSM_OK;
  }
  if (isa == DFSSM_HOST_ISA_AVX512VNNI) {
    if (!cpu_has_vnni()) return fail(DFSSM_E_UNSUPPORTED, "this CPU has no AVX-512 VNNI");
    h->isa = isa;
    return DFSSM_OK;
  }
  return fail(DFSSM_E_INVALID, "unknown instruction path");
}

dfssm_status dfssm_host_get_isa(const dfssm_host* h, int32_t* isa) {
  if (!h || !isa) return fail(DFSSM_E_INVALID, "null argument");
  *isa = h->isa;
  return DFSSM_OK;
}

dfssm_status dfssm_host_load_synthetic(dfssm_host* h, uint64_t seed) {
  if (!h) return fail(DFSSM_E_INVALID, "null context");
  for (int l = 0; l < h->L; ++l)
    for (int kind = 0; kind < DFSSM_T_PER_LAYER; ++kind) {
      const GenSpec g = layer_gen(kind);
      auto& T = h->lt[l][kind];
      gen_fill(T.buf.data(), T.count, g.d, stream_key(seed, (uint64_t)(64 * l + kind)), g.a, g.b);
      refresh_sums(h, l, kind);
    }
  const GenSpec gg[3] = {{D_INT8, 0, 0}, {D_UNIFORM, 0.01, 0.02}, {D_UNIFORM, 0.5, 1.5}};
  for (int kind = 0; kind < 3; ++kind) {
    auto& T = h->gt[kind];
    gen_fill(T.buf.data(), T.count, gg[kind].d, stream_key(seed, (uint64_t)(4096 + kind)), gg[kind].a, gg[kind].b);
    refresh_sums(h, -1, kind);
  }
  std::fill(h->conv.begin(), h->conv.end(), 0.0f);
  std::fill(h->ssm.begin(), h->ssm.end(), 0.0f);
  return DFSSM_OK;
}

dfssm_status dfssm_host_set_tensor(dfssm_host* h, int32_t layer, int32_t kind, const void* src, size_t bytes) {
  if (!h || !src) return fail(DFSSM_E_INVALID, "null argument");
  dfssm_host::Tensor* T = tensor(h, layer, kind);
  if (!T) return fail(DFSSM_E_INVALID, "unknown tensor");
  if (bytes != T->buf.size()) return fail(DFSSM_E_INVALID, "tensor size mismatch");
  std::memcpy(T->buf.data(), src, bytes);
  refresh_sums(h, layer, kind);
  return DFSSM_OK;
}

dfssm_status dfssm_host_get_tensor(const dfssm_host* h, int32_t layer, int32_t kind, void* dst, size_t bytes) {
  if (!h || !dst) return fail(DFSSM_E_INVALID, "null argument");
  const dfssm_host::Tensor* T = tensor(const_cast<dfssm_host*>(h), layer, kind);
  if (!T) return fail(DFSSM_E_INVALID, "unknown tensor");
  if (bytes != T->buf.size()) return fail(DFSSM_E_INVALID, "tensor size mismatch");
  std::memcpy(dst, T->buf.data(), bytes);
  return DFSSM_OK;
}

dfssm_status dfssm_host_reset_state(dfssm_host* h, int32_t batch) {
  if (!h) return fail(DFSSM_E_INVALID, "null context");
  if (batch < 0 || batch > h->maxB) return fail(DFSSM_E_INVALID, "batch must be in [0, max_batch]");
  std::fill(h->conv.begin(), h->conv.begin() + (size_t)batch * h->conv_per_seq(), 0.0f);
  std::fill(h->ssm.begin(), h->ssm.begin() + (size_t)batch * h->ssm_per_seq(), 0.0f);
  return DFSSM_OK;
}

dfssm_status dfssm_host_get_state(const dfssm_host* h, int32_t seq, float* conv, float* ssm) {
  if (!h) return fail(DFSSM_E_INVALID, "null context");
  if (seq < 0 || seq >= h->maxB) return fail(DFSSM_E_INVALID, "sequence slot out of range");
  if (conv) std::memcpy(conv, h->conv.data() + (size_t)seq * h->conv_per_seq(), 4 * h->conv_per_seq());
  if (ssm) std::memcpy(ssm, h->ssm.data() + (size_t)seq * h->ssm_per_seq(), 4 * h->ssm_per_seq());
  return DFSSM_OK;
}

dfssm_status dfssm_host_set_state(dfssm_host* h, int32_t seq, const float* conv, const float* ssm) {
  if (!h) return fail(DFSSM_E_INVALID, "null context");
  if (seq < 0 || seq >= h->maxB) return fail(DFSSM_E_INVALID, "sequence slot out of range");
  if (conv) std::memcpy(h->conv.data() + (size_t)seq * h->conv_per_seq(), conv, 4 * h->conv_per_seq());
  if (ssm) std::memcpy(h->ssm.data() + (size_t)seq * h->ssm_per_seq(), ssm, 4 * h->ssm_per_seq());
  return DFSSM_OK;
}

dfssm_status dfssm_host_trace_step(dfssm_host* h, const int32_t* tok, int32_t B, float* h_trace, int8_t* q1,
                                   int8_t* q2, int8_t* qf, float* logits, int32_t* acc1, int32_t* acc2) {
  dfssm_status v = check_step(h, tok, B);
  if (v != DFSSM_OK) return v;
  try {
    ensure_ws(h, B, !logits);
  } catch (const std::bad_alloc&) {
    return fail(DFSSM_E_OOM, "host allocation failed");
  }
  Trace tr;
  tr.h = h_trace;
  tr.q1 = q1;
  tr.q2 = q2;
  tr.qf = qf;
  tr.acc1 = acc1;
  tr.acc2 = acc2;
  step(h, ops_of(h), tok, B, &tr, logits, nullptr);
  return DFSSM_OK;
}

dfssm_status dfssm_host_decode_step(dfssm_host* h, const int32_t* tok, int32_t B, float* logits, int32_t* next) {
  dfssm_status v = check_step(h, tok, B);
  if (v != DFSSM_OK) return v;
  try {
    ensure_ws(h, B, !logits);
  } catch (const std::bad_alloc&) {
    return fail(DFSSM_E_OOM, "host allocation failed");
  }
  step(h, ops_of(h), tok, B, nullptr, logits, next);
  return DFSSM_OK;
}

dfssm_status dfssm_host_generate(dfssm_host* h, int32_t* tok, int32_t B, int32_t n_steps, int32_t* out) {
  dfssm_status v = check_step(h, tok, B);
  if (v != DFSSM_OK) return v;
  if (n_steps < 0) return fail(DFSSM_E_INVALID, "negative step count");
  try {
    ensure_ws(h, B, true);
  } catch (const std::bad_alloc&) {
    return fail(DFSSM_E_OOM, "host allocation failed");
  }
  const IntOps ops = ops_of(h);
  for (int i = 0; i < n_steps; ++i) {
    step(h, ops, tok, B, nullptr, nullptr, tok);
    if (out) std::memcpy(out + (size_t)i * B, tok, 4 * (size_t)B);
  }
  return DFSSM_OK;
}

dfssm_status dfssm_host_prefill(dfssm_host* h, const int32_t* tok, int32_t B, int32_t T, float* last_logits,
                                int32_t* next) {
  if (!h) return fail(DFSSM_E_INVALID, "null context");
  if (!tok) return fail(DFSSM_E_INVALID, "null token pointer");
  if (B < 1 || B > h->maxB) return fail(DFSSM_E_INVALID, "batch must be in [1, max_batch]");
  if (T < 1) return fail(DFSSM_E_INVALID, "prompt length must be >= 1");
  for (size_t i = 0; i < (size_t)B * T; ++i)
    if (tok[i] < 0 || tok[i] >= h->V) return fail(DFSSM_E_INVALID, "token id outside [0, vocab)");
  std::vector<int32_t> col;
  try {
    col.resize(B);
    ensure_ws(h, B, !last_logits);
  } catch (const std::bad_alloc&) {
    return fail(DFSSM_E_OOM, "host allocation failed");
  }
  const IntOps ops = ops_of(h);
  for (int t = 0; t < T; ++t) {
    for (int b = 0; b < B; ++b) col[b] = tok[(size_t)b * T + t];
    const bool last = t == T - 1;
    step(h, ops, col.data(), B, nullptr, last ? last_logits : nullptr, last ? next : nullptr, last);
  }
  return DFSSM_OK;
}

dfssm_status dfssm_host_copy_rate(dfssm_host* h, size_t bytes, int32_t iters, double* gbs) {
  if (!h || !gbs) return fail(DFSSM_E_INVALID, "null argument");
  if (bytes < 64 * (size_t)h->threads || iters < 1) return fail(DFSSM_E_INVALID, "buffer too small or no iterations");
  bytes &= ~(size_t)63;
  std::vector<unsigned char> a, b;
  try {
    a.assign(bytes, 1);
    b.assign(bytes, 0);
  } catch (const std::bad_alloc&) {
    return fail(DFSSM_E_OOM, "host allocation failed");
  }
  const int nt = h->threads;
  const size_t per = (bytes / nt) & ~(size_t)63;
  auto run = [&]() {
#pragma omp parallel num_threads(nt)
    {
      const int me = omp_get_thread_num();
      const size_t o = (size_t)me * per, n = me == nt - 1 ? bytes - o : per;
      std::memcpy(b.data() + o, a.data() + o, n);
    }
  };
  run();  // first touch
  const auto t0 = std::chrono::steady_clock::now();
  for (int i = 0; i < iters; ++i) run();
  const double s = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
  *gbs = 2.0 * (double)bytes * iters / s / 1e9;
  return DFSSM_OK;
}

}  // extern "C"
