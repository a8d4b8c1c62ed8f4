// Host runtime behind include/dfssm.h: context, device memory, synthetic
// load, state I/O, the decode / prefill / layer step orchestration and the
// graph cache.  Every step of the model runs in the kernels of kernels.hip.
#include <algorithm>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "../../include/dfssm.h"
#include "common.h"
#include "persistent.h"

using namespace dfssm;

// Scratch of dfssm_k_gemm_noalloc: a file-scope device array, one copy per
// GPU for the life of the process.  In host code the array's name stands for
// no device address (a kernel given it would fault); host code uses only the
// address hipGetSymbolAddress returns for the current device.
constexpr size_t kNoAllocScratchBytes = (size_t)8 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

thread_local std::string g_err;

dfssm_status fail(dfssm_status st, const std::string& msg) {
  g_err = msg;
  return st;
}

#define HIP_TRY(expr)                                                                          \
  do {                                                                                         \
    hipError_t _e = (expr);                                                                    \
    if (_e != hipSuccess)                                                                      \
      return fail(DFSSM_E_HIP, std::string(#expr) + ": " + hipGetErrorString(_e));             \
  } while (0)

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct TensorInfo {
  size_t offset = 0;  // into the weight block
  size_t bytes = 0;
  size_t count = 0;
  int elem = 4;
};

}  // namespace

struct dfssm_ctx {
  dfssm_config cfg{};
  int device = 0;
  int H = 0, P = 0, N = 0, dm = 0, di = 0, cdim = 0, dproj = 0, K = 0, r = 0, V = 0, L = 0, maxB = 0;
  float eps = 1e-5f;

  // weights
  std::vector<TensorInfo> layer_t;  // L * 19
  std::vector<TensorInfo> global_t; // 3
  char* wbuf = nullptr;
  size_t wbytes = 0;
  bool loaded = false;

  // state
  float* conv = nullptr;  // [maxB][L][K-1][cdim]
  float* ssm = nullptr;   // [maxB][L][H][P/16][N][16]
  size_t conv_bstride = 0, ssm_bstride = 0;

  // workspace (all [maxB][...])
  float *h = nullptr, *zx = nullptr, *xc = nullptr, *g = nullptr, *logits = nullptr;
  int8_t *q1 = nullptr, *q2 = nullptr;
  uint32_t *pl1 = nullptr, *pl2 = nullptr;
  int32_t *qs1 = nullptr, *qs2 = nullptr;
  float *s1 = nullptr, *s2 = nullptr, *t1 = nullptr, *t2 = nullptr;
  int32_t* next = nullptr;
  int32_t* counter = nullptr;
  int* err = nullptr;
  char* ws = nullptr;
  size_t wsbytes = 0, sbytes = 0;
  char* sbuf = nullptr;

  // graphs keyed by (B, d_tok, d_out)
  std::map<std::tuple<int, const void*, const void*>, hipGraphExec_t> graphs;

  // the two halves of a small batched decode step run as concurrent chains
  // on these streams (created on first use): fork and join events
  hipStream_t split_st[4] = {};
  hipEvent_t split_ev[5] = {};

  // memory: one block for weights, state, workspace and mailboxes (the
  // caller's arena, or a library allocation); the batched-path workspace is
  // part of the caller's arena, or grows on demand in its own allocation
  char* arena = nullptr;
  size_t arena_bytes = 0;
  bool own_arena = false;
  size_t chunk_rows = 16384;  // token rows per prefill chunk
  size_t o_w = 0, o_s = 0, o_ws = 0, o_box = 0, o_abort = 0, o_gw = 0;
  struct WsOff {
    size_t h, zx, xc, g, lg, q1, q2, p1, p2, qs1, qs2, s1, s2, t1, t2, nx, ct, er;
  } wo{};

  // batched path (decode with B > 1, prefill): rows of tokens per layer
  struct GemmWs {
    size_t rows = 0;  // capacity in token rows
    size_t bytes = 0;
    char* buf = nullptr;
    float *h = nullptr, *s = nullptr, *t = nullptr, *zx = nullptr, *xc = nullptr, *g = nullptr;
    int8_t* q = nullptr;
    int32_t* qsum = nullptr;
    float* gram = nullptr;  // chunked-scan workspace
    bool fixed = false;     // carved from the caller's arena: never moves or grows
  } gw;

  // persistent batch-1 path
  int path = DFSSM_PATH_AUTO;
  bool persist_ok = false;
  std::string persist_why;
  int persist_grid = 0;
  uint64_t* boxes = nullptr;
  size_t box_words = 0;
  int* abort_flag = nullptr;
  unsigned host_epoch = 1;
  unsigned pair_count = 1;  // writes of the paired boxes so far + 1 (boxes zeroed: every tag is 0)

  void* tensor_ptr(int layer, int kind) const {
    const TensorInfo& t = layer >= 0 ? layer_t[(size_t)layer * DFSSM_T_PER_LAYER + kind] : global_t[kind];
    return wbuf + t.offset;
  }
  template <typename T>
  T* lt(int layer, int kind) const { return (T*)tensor_ptr(layer, kind); }
};

namespace {

dfssm_status validate(const dfssm_config* c) {
  if (!c) return fail(DFSSM_E_INVALID, "null config");
  if (c->n_layer < 1 || c->d_model < 1 || c->d_inner < 1 || c->d_state < 1 || c->headdim < 1 || c->vocab < 1 ||
      c->lora_rank < 1 || c->max_batch < 1)
    return fail(DFSSM_E_INVALID, "config dimensions must be positive");
  auto pow2le64 = [](int x) { return x >= 1 && x <= 64 && (x & (x - 1)) == 0; };
  if (c->d_model % 128 || !pow2le64(c->d_model / 128))
    return fail(DFSSM_E_UNSUPPORTED, "d_model must be 128 * 2^k <= 8192");
  if (c->d_inner % 128 || !pow2le64(c->d_inner / 128))
    return fail(DFSSM_E_UNSUPPORTED, "d_inner must be 128 * 2^k <= 8192");
  if (c->headdim % 16 || c->d_inner % c->headdim) return fail(DFSSM_E_UNSUPPORTED, "headdim must be a multiple of 16 dividing d_inner");
  if ((c->d_inner / c->headdim) % 4) return fail(DFSSM_E_UNSUPPORTED, "the head count must be a multiple of 4");
  if (c->d_state % 2) return fail(DFSSM_E_UNSUPPORTED, "d_state must be even");
  if (c->d_conv != 4) return fail(DFSSM_E_UNSUPPORTED, "d_conv must be 4");
  if (c->lora_rank > 32) return fail(DFSSM_E_UNSUPPORTED, "lora_rank must be <= 32");
  if (c->max_batch > 1024) return fail(DFSSM_E_UNSUPPORTED, "max_batch must be <= 1024");
  if (!(c->norm_eps >= 0.0f)) return fail(DFSSM_E_INVALID, "norm_eps must be >= 0");
  if (c->max_chunk_rows < 0 || c->max_chunk_rows > (1 << 20))
    return fail(DFSSM_E_INVALID, "max_chunk_rows must be in [0, 2^20]");
  return DFSSM_OK;
}

struct Spec {
  size_t count;
  int elem;
};

Spec layer_spec(const dfssm_ctx* c, int kind) {
  const size_t dm = c->dm, di = c->di, dp = c->dproj, r = c->r, cd = c->cdim, H = c->H;
  switch (kind) {
    case DFSSM_T_IN_BITS: return {dp * (dm / 32), 4};
    case DFSSM_T_IN_SW: return {dp, 4};
    case DFSSM_T_IN_A: return {r * dm, 1};
    case DFSSM_T_IN_SA: return {r, 4};
    case DFSSM_T_IN_B: return {dp * r, 1};
    case DFSSM_T_IN_SB: return {dp, 4};
    case DFSSM_T_OUT_BITS: return {dm * (di / 32), 4};
    case DFSSM_T_OUT_SW: return {dm, 4};
    case DFSSM_T_OUT_A: return {r * di, 1};
    case DFSSM_T_OUT_SA: return {r, 4};
    case DFSSM_T_OUT_B: return {dm * r, 1};
    case DFSSM_T_OUT_SB: return {dm, 4};
    case DFSSM_T_CONV_W: return {cd * (size_t)c->K, 4};
    case DFSSM_T_CONV_B: return {cd, 4};
    case DFSSM_T_A_LOG: case DFSSM_T_DT_BIAS: case DFSSM_T_D: return {H, 4};
    case DFSSM_T_NORM_W: return {dm, 4};
    default: return {di, 4};  // GNORM_W
  }
}

Spec global_spec(const dfssm_ctx* c, int kind) {
  if (kind == DFSSM_G_EMBED) return {(size_t)c->V * c->dm, 1};
  if (kind == DFSSM_G_EMBED_SCALE) return {(size_t)c->V, 4};
  return {(size_t)c->dm, 4};
}

// synthetic generator parameters per kind
struct GenParam {
  int mode;
  double a, b;
  float cval;
};

GenParam layer_gen(int kind) {
  switch (kind) {
    case DFSSM_T_IN_BITS: case DFSSM_T_OUT_BITS: return {GEN_WORDS, 0, 0, 0};
    case DFSSM_T_IN_SW: case DFSSM_T_OUT_SW: return {GEN_UNIFORM, 0.01, 0.05, 0};
    case DFSSM_T_IN_A: case DFSSM_T_IN_B: case DFSSM_T_OUT_A: case DFSSM_T_OUT_B: return {GEN_INT8, 0, 0, 0};
    case DFSSM_T_IN_SA: case DFSSM_T_IN_SB: case DFSSM_T_OUT_SA: case DFSSM_T_OUT_SB:
      return {GEN_CONST, 0, 0, (float)1e-3};
    case DFSSM_T_CONV_W: case DFSSM_T_CONV_B: return {GEN_UNIFORM, -0.5, 0.5, 0};
    case DFSSM_T_A_LOG: return {GEN_UNIFORM, 0.0, 2.772588722239781, 0};
    case DFSSM_T_DT_BIAS: return {GEN_UNIFORM, -4.0, -1.0, 0};
    case DFSSM_T_D: return {GEN_NORMAL, 0, 0, 0};
    default: return {GEN_UNIFORM, 0.5, 1.5, 0};  // norm weights
  }
}

GenParam global_gen(int kind) {
  if (kind == DFSSM_G_EMBED) return {GEN_INT8, 0, 0, 0};
  if (kind == DFSSM_G_EMBED_SCALE) return {GEN_UNIFORM, 0.01, 0.02, 0};
  return {GEN_UNIFORM, 0.5, 1.5, 0};
}

hipStream_t S(void* s) { return (hipStream_t)s; }

// ---------------------------------------------------------------------------
// one layer on the context's workspace h[0..B)
// ---------------------------------------------------------------------------
hipError_t norm_quant_in(dfssm_ctx* c, int l, int B, hipStream_t st) {
  return launch_norm_quant(c->h, c->lt<float>(l, DFSSM_T_NORM_W), c->dm, B, c->eps, c->lt<int8_t>(l, DFSSM_T_IN_A),
                           c->lt<float>(l, DFSSM_T_IN_SA), c->r, c->q1, c->pl1, c->qs1, c->s1, c->t1, st);
}

hipError_t in_proj(dfssm_ctx* c, int l, int B, hipStream_t st, int32_t* acc = nullptr) {
  ProjArgs a{};
  a.acc = acc;
  a.bits = c->lt<uint32_t>(l, DFSSM_T_IN_BITS);
  a.sw = c->lt<float>(l, DFSSM_T_IN_SW);
  a.Bm = c->lt<int8_t>(l, DFSSM_T_IN_B);
  a.sB = c->lt<float>(l, DFSSM_T_IN_SB);
  a.in = QPrep{c->q1, c->pl1, c->qs1, c->s1, c->t1};
  a.d_in = c->dm;
  a.d_out = c->dproj;
  a.r = c->r;
  a.B = B;
  a.zx = c->zx;
  a.xc = c->xc;
  a.conv_state = c->conv + (size_t)l * (c->K - 1) * c->cdim;
  a.conv_bstride = c->conv_bstride;
  a.conv_w = c->lt<float>(l, DFSSM_T_CONV_W);
  a.conv_b = c->lt<float>(l, DFSSM_T_CONV_B);
  a.d_inner = c->di;
  a.conv_dim = c->cdim;
  a.K = c->K;
  return launch_proj(a, EPI_IN_PROJ, st);
}

hipError_t ssm_step(dfssm_ctx* c, int l, int B, hipStream_t st) {
  return launch_ssm(c->xc, c->zx, c->dproj, c->lt<float>(l, DFSSM_T_A_LOG), c->lt<float>(l, DFSSM_T_DT_BIAS),
                    c->lt<float>(l, DFSSM_T_D), c->ssm + (size_t)l * c->H * c->P * c->N, c->ssm_bstride, c->g, B,
                    c->H, c->P, c->N, c->di, c->cdim, st);
}

hipError_t norm_quant_out(dfssm_ctx* c, int l, int B, hipStream_t st) {
  return launch_norm_quant(c->g, c->lt<float>(l, DFSSM_T_GNORM_W), c->di, B, c->eps, c->lt<int8_t>(l, DFSSM_T_OUT_A),
                           c->lt<float>(l, DFSSM_T_OUT_SA), c->r, c->q2, c->pl2, c->qs2, c->s2, c->t2, st);
}

hipError_t out_proj(dfssm_ctx* c, int l, int B, hipStream_t st, int32_t* acc = nullptr) {
  ProjArgs o{};
  o.acc = acc;
  o.bits = c->lt<uint32_t>(l, DFSSM_T_OUT_BITS);
  o.sw = c->lt<float>(l, DFSSM_T_OUT_SW);
  o.Bm = c->lt<int8_t>(l, DFSSM_T_OUT_B);
  o.sB = c->lt<float>(l, DFSSM_T_OUT_SB);
  o.in = QPrep{c->q2, c->pl2, c->qs2, c->s2, c->t2};
  o.d_in = c->di;
  o.d_out = c->dm;
  o.r = c->r;
  o.B = B;
  o.h = c->h;
  return launch_proj(o, EPI_OUT_PROJ, st);
}

hipError_t lm_head(dfssm_ctx* c, int B, float* logits, hipStream_t st) {
  return launch_lm_head(c->lt<int8_t>(-1, DFSSM_G_EMBED), c->lt<float>(-1, DFSSM_G_EMBED_SCALE), c->q1, c->s1, c->V,
                        c->dm, B, logits, st);
}

dfssm_status enqueue_layer(dfssm_ctx* c, int l, int B, hipStream_t st, int8_t* q1_out = nullptr,
                           int8_t* q2_out = nullptr, int32_t* acc1_out = nullptr, int32_t* acc2_out = nullptr) {
  HIP_TRY(norm_quant_in(c, l, B, st));
  if (q1_out) HIP_TRY(hipMemcpyAsync(q1_out, c->q1, (size_t)B * c->dm, hipMemcpyDeviceToDevice, st));
  HIP_TRY(in_proj(c, l, B, st, acc1_out));
  HIP_TRY(ssm_step(c, l, B, st));
  HIP_TRY(norm_quant_out(c, l, B, st));
  if (q2_out) HIP_TRY(hipMemcpyAsync(q2_out, c->q2, (size_t)B * c->di, hipMemcpyDeviceToDevice, st));
  HIP_TRY(out_proj(c, l, B, st, acc2_out));
  return DFSSM_OK;
}

// full step: embed -> layers -> (final norm, LM head, argmax)
struct Trace {
  float* h = nullptr;
  int8_t* q1 = nullptr;
  int8_t* q2 = nullptr;
  int8_t* qf = nullptr;
  int32_t* acc1 = nullptr;  // [L][rows][d_in_proj]
  int32_t* acc2 = nullptr;  // [L][rows][d_model]
};

dfssm_status enqueue_step(dfssm_ctx* c, const int32_t* tok, int tok_stride, int B, float* logits, int32_t* next,
                          int32_t* out, const Trace* tr, bool head, hipStream_t st) {
  float* trace = tr ? tr->h : nullptr;
  HIP_TRY(launch_embed(tok, tok_stride, c->lt<int8_t>(-1, DFSSM_G_EMBED), c->lt<float>(-1, DFSSM_G_EMBED_SCALE), c->dm,
                       c->V, B, c->h, c->err, st));
  for (int l = 0; l < c->L; ++l) {
    if (trace)
      HIP_TRY(hipMemcpyAsync(trace + (size_t)l * B * c->dm, c->h, sizeof(float) * B * c->dm,
                             hipMemcpyDeviceToDevice, st));
    dfssm_status r = enqueue_layer(c, l, B, st, tr && tr->q1 ? tr->q1 + (size_t)l * B * c->dm : nullptr,
                                   tr && tr->q2 ? tr->q2 + (size_t)l * B * c->di : nullptr,
                                   tr && tr->acc1 ? tr->acc1 + (size_t)l * B * c->dproj : nullptr,
                                   tr && tr->acc2 ? tr->acc2 + (size_t)l * B * c->dm : nullptr);
    if (r != DFSSM_OK) return r;
  }
  if (trace)
    HIP_TRY(hipMemcpyAsync(trace + (size_t)c->L * B * c->dm, c->h, sizeof(float) * B * c->dm,
                           hipMemcpyDeviceToDevice, st));
  if (!head) return DFSSM_OK;
  HIP_TRY(launch_norm_quant(c->h, c->lt<float>(-1, DFSSM_G_FINAL_NORM), c->dm, B, c->eps, nullptr, nullptr, 0, c->q1,
                            c->pl1, c->qs1, c->s1, c->t1, st));
  if (tr && tr->qf) HIP_TRY(hipMemcpyAsync(tr->qf, c->q1, (size_t)B * c->dm, hipMemcpyDeviceToDevice, st));
  float* lg = logits ? logits : c->logits;
  HIP_TRY(lm_head(c, B, lg, st));
  if (next || out) HIP_TRY(launch_argmax(lg, c->V, B, next ? next : c->next, out, c->counter, st));
  return DFSSM_OK;
}

// ---------------------------------------------------------------------------
// batched path: every layer on all B * T token rows at once
// ---------------------------------------------------------------------------
constexpr size_t kPrefillChunkRows = 16384;  // default token rows per prefill chunk (bounds the workspace)

struct GemmLayout {
  size_t h, s, t, zx, xc, g, q, qs, gram, bytes;
};

// The batched-path workspace for `rows` token rows.
GemmLayout gemm_layout(const dfssm_ctx* c, size_t rows) {
  GemmLayout L{};
  const size_t mx = (size_t)std::max(c->dm, c->di);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align_up(bytes); return o; };
  L.h = take(4 * rows * c->dm);
  L.s = take(4 * rows);
  L.t = take(4 * rows * 16);
  L.zx = take(4 * rows * c->dproj);
  L.xc = take(4 * rows * c->cdim);
  L.g = take(4 * rows * c->di);
  L.q = take(rows * mx);
  L.qs = take(4 * rows);
  L.gram = take(4 * (rows / kSsdL + (size_t)c->maxB) * ssd_record_floats(c->H));
  L.bytes = off;
  return L;
}

void assign_gemm_ws(dfssm_ctx* c, char* buf, size_t rows, const GemmLayout& L) {
  c->gw.rows = rows;
  c->gw.bytes = L.bytes;
  c->gw.buf = buf;
  c->gw.h = (float*)(buf + L.h);
  c->gw.s = (float*)(buf + L.s);
  c->gw.t = (float*)(buf + L.t);
  c->gw.zx = (float*)(buf + L.zx);
  c->gw.xc = (float*)(buf + L.xc);
  c->gw.g = (float*)(buf + L.g);
  c->gw.q = (int8_t*)(buf + L.q);
  c->gw.qsum = (int32_t*)(buf + L.qs);
  c->gw.gram = (float*)(buf + L.gram);
}

// Token rows the caller's arena gives the batched path.
size_t fixed_gemm_rows(const dfssm_ctx* c) { return std::max(c->chunk_rows, (size_t)c->maxB); }

// Grow the batched-path workspace to at least `rows` token rows.  Cached
// graphs hold pointers into it, so they are dropped when it moves.  In the
// caller's arena the workspace is fixed: a request beyond it is an error.
dfssm_status ensure_gemm_ws(dfssm_ctx* c, size_t rows) {
  if (rows <= c->gw.rows) return DFSSM_OK;
  if (c->gw.fixed)
    return fail(DFSSM_E_INVALID, "the arena's batched-path workspace holds " + std::to_string(c->gw.rows) +
                                     " token rows; " + std::to_string(rows) + " requested");
  rows = std::max(rows, (size_t)c->maxB);
  const GemmLayout L = gemm_layout(c, rows);
  char* buf = nullptr;
  if (hipMalloc(&buf, L.bytes) != hipSuccess) {
    (void)hipGetLastError();
    return fail(DFSSM_E_OOM, "batched-path workspace allocation failed");
  }
  if (c->gw.buf) {
    HIP_TRY(hipDeviceSynchronize());
    (void)hipFree(c->gw.buf);
  }
  for (auto& kv : c->graphs) (void)hipGraphExecDestroy(kv.second);
  c->graphs.clear();
  assign_gemm_ws(c, buf, rows, L);
  return DFSSM_OK;
}

// One layer on rows m = b * T + t of the batched workspace (B sequences in
// state slots 0..B-1, T tokens each, in order).
// Decode (one token per sequence) of at most kSkinnyDecodeRows sequences
// uses the skinny GEMM (32-row blocks), with the conv shift register in the
// in_proj epilogue; more rows use the tiled GEMM.
constexpr int kSkinnyDecodeRows = 32;
bool skinny_decode(int B, int T) { return T == 1 && B <= kSkinnyDecodeRows; }

hipError_t b_rows_in(dfssm_ctx* c, int l, int M, hipStream_t st) {
  auto& w = c->gw;
  RowsArgs ra{w.h, c->dm, c->lt<float>(l, DFSSM_T_NORM_W), M, c->eps, c->lt<int8_t>(l, DFSSM_T_IN_A),
              c->lt<float>(l, DFSSM_T_IN_SA), w.q, w.s, w.qsum, w.t};
  return launch_rows_quant(ra, c->dm, st);
}

hipError_t b_in_proj(dfssm_ctx* c, int l, int B, int T, hipStream_t st, int32_t* acc = nullptr) {
  auto& w = c->gw;
  const int M = B * T;
  float* conv_l = c->conv + (size_t)l * (c->K - 1) * c->cdim;
  if (skinny_decode(B, T)) {
    SkinnyArgs si{};
    si.q = w.q; si.s = w.s; si.qsum = w.qsum; si.t = w.t;
    si.w = c->lt<uint32_t>(l, DFSSM_T_IN_BITS);
    si.sw = c->lt<float>(l, DFSSM_T_IN_SW);
    si.Bm = c->lt<int8_t>(l, DFSSM_T_IN_B);
    si.sB = c->lt<float>(l, DFSSM_T_IN_SB);
    si.M = M; si.N = c->dproj; si.K = c->dm;
    si.y = w.zx; si.ldy = c->dproj;
    si.xc = w.xc; si.conv_state = conv_l; si.conv_bstride = c->conv_bstride;
    si.conv_w = c->lt<float>(l, DFSSM_T_CONV_W); si.conv_b = c->lt<float>(l, DFSSM_T_CONV_B);
    si.x_off = c->di; si.cdim = c->cdim;
    si.acc = acc;
    return launch_gemm_skinny(si, SK_IN, st);
  }
  GemmArgs gi{w.q, w.s, w.qsum, w.t, c->lt<uint32_t>(l, DFSSM_T_IN_BITS), c->lt<float>(l, DFSSM_T_IN_SW),
              c->lt<int8_t>(l, DFSSM_T_IN_B), c->lt<float>(l, DFSSM_T_IN_SB), M, c->dproj, c->dm, w.zx, c->dproj,
              acc};
  if (T == 1) {  // one decode token per sequence: the conv shift register in the GEMM epilogue
    gi.xc = w.xc; gi.conv_state = conv_l; gi.conv_bstride = c->conv_bstride;
    gi.conv_w = c->lt<float>(l, DFSSM_T_CONV_W); gi.conv_b = c->lt<float>(l, DFSSM_T_CONV_B);
    gi.x_off = c->di; gi.cdim = c->cdim;
    return launch_bitgemm(gi, GEMM_EPI_STORE, st);
  }
  hipError_t e = launch_bitgemm(gi, GEMM_EPI_STORE, st);
  if (e != hipSuccess || scan_takes_conv_inputs(c->P, c->N)) return e;  // else the scan applies the conv
  ConvSeqArgs ca{w.zx, c->dproj, c->di, w.xc, conv_l, c->conv_bstride,
                 c->lt<float>(l, DFSSM_T_CONV_W), c->lt<float>(l, DFSSM_T_CONV_B), B, T, c->cdim};
  return launch_conv_seq(ca, st);
}

hipError_t b_scan(dfssm_ctx* c, int l, int B, int T, hipStream_t st) {
  auto& w = c->gw;
  ScanArgs sa{w.xc, w.zx, c->dproj, 2 * c->di + 2 * c->N, c->lt<float>(l, DFSSM_T_A_LOG),
              c->lt<float>(l, DFSSM_T_DT_BIAS), c->lt<float>(l, DFSSM_T_D),
              c->ssm + (size_t)l * c->H * c->P * c->N, c->ssm_bstride, w.g, B, T, c->H, c->di, c->cdim,
              w.gram};
  if (T == 1 || !scan_takes_conv_inputs(c->P, c->N)) return launch_scan(sa, c->P, c->N, st);
  // the scan convolves the in_proj output itself, reading the stored window;
  // the window moves on once the scan is done with it
  float* conv_l = c->conv + (size_t)l * (c->K - 1) * c->cdim;
  sa.x_off = c->di;
  sa.conv_w = c->lt<float>(l, DFSSM_T_CONV_W);
  sa.conv_b = c->lt<float>(l, DFSSM_T_CONV_B);
  sa.conv_state = conv_l;
  sa.conv_bstride = c->conv_bstride;
  hipError_t e = launch_scan(sa, c->P, c->N, st);
  if (e != hipSuccess) return e;
  ConvSeqArgs ca{w.zx, c->dproj, c->di, w.xc, conv_l, c->conv_bstride,
                 c->lt<float>(l, DFSSM_T_CONV_W), c->lt<float>(l, DFSSM_T_CONV_B), B, T, c->cdim};
  return launch_conv_state_update(ca, st);
}

hipError_t b_rows_out(dfssm_ctx* c, int l, int M, hipStream_t st) {
  auto& w = c->gw;
  RowsArgs rb{w.g, c->di, c->lt<float>(l, DFSSM_T_GNORM_W), M, c->eps, c->lt<int8_t>(l, DFSSM_T_OUT_A),
              c->lt<float>(l, DFSSM_T_OUT_SA), w.q, w.s, w.qsum, w.t};
  return launch_rows_quant(rb, c->di, st);
}

hipError_t b_out_proj(dfssm_ctx* c, int l, int B, int T, hipStream_t st, int32_t* acc = nullptr) {
  auto& w = c->gw;
  const int M = B * T;
  if (skinny_decode(B, T)) {
    SkinnyArgs so{};
    so.q = w.q; so.s = w.s; so.qsum = w.qsum; so.t = w.t;
    so.w = c->lt<uint32_t>(l, DFSSM_T_OUT_BITS);
    so.sw = c->lt<float>(l, DFSSM_T_OUT_SW);
    so.Bm = c->lt<int8_t>(l, DFSSM_T_OUT_B);
    so.sB = c->lt<float>(l, DFSSM_T_OUT_SB);
    so.M = M; so.N = c->dm; so.K = c->di;
    so.y = w.h; so.ldy = c->dm;
    so.acc = acc;
    return launch_gemm_skinny(so, SK_OUT, st);
  }
  GemmArgs go{w.q, w.s, w.qsum, w.t, c->lt<uint32_t>(l, DFSSM_T_OUT_BITS), c->lt<float>(l, DFSSM_T_OUT_SW),
              c->lt<int8_t>(l, DFSSM_T_OUT_B), c->lt<float>(l, DFSSM_T_OUT_SB), M, c->dm, c->di, w.h, c->dm, acc};
  return launch_bitgemm(go, GEMM_EPI_RESIDUAL, st);
}

// final norm + quantise of the last token row of each sequence, then the LM head
hipError_t b_head(dfssm_ctx* c, int B, int T, float* lg, int8_t* qf_out, hipStream_t st) {
  auto& w = c->gw;
  RowsArgs rf{w.h + (size_t)(T - 1) * c->dm, T * c->dm, c->lt<float>(-1, DFSSM_G_FINAL_NORM), B, c->eps, nullptr,
              nullptr, w.q, w.s, nullptr, nullptr};
  hipError_t e = launch_rows_quant(rf, c->dm, st);
  if (e == hipSuccess && qf_out) e = hipMemcpyAsync(qf_out, w.q, (size_t)B * c->dm, hipMemcpyDeviceToDevice, st);
  if (e != hipSuccess) return e;
  if (c->dm % 128 == 0) {
    // the int8 LM head on the matrix cores, one launch of 32-row blocks (the
    // row blocks of a column block share its embedding rows in one XCD's L2)
    SkinnyArgs sh{};
    sh.q = w.q; sh.s = w.s;
    sh.w = c->lt<int8_t>(-1, DFSSM_G_EMBED);
    sh.sw = c->lt<float>(-1, DFSSM_G_EMBED_SCALE);
    sh.M = B; sh.N = c->V; sh.K = c->dm;
    sh.y = lg; sh.ldy = c->V;
    return launch_gemm_skinny(sh, SK_HEAD, st);
  }
  return launch_lm_head(c->lt<int8_t>(-1, DFSSM_G_EMBED), c->lt<float>(-1, DFSSM_G_EMBED_SCALE), w.q, w.s, c->V,
                        c->dm, B, lg, st);
}

dfssm_status enqueue_layer_gemm(dfssm_ctx* c, int l, int B, int T, hipStream_t st, int8_t* q1_out,
                                int8_t* q2_out, int32_t* acc1_out = nullptr, int32_t* acc2_out = nullptr) {
  const int M = B * T;
  HIP_TRY(b_rows_in(c, l, M, st));
  if (q1_out) HIP_TRY(hipMemcpyAsync(q1_out, c->gw.q, (size_t)M * c->dm, hipMemcpyDeviceToDevice, st));
  HIP_TRY(b_in_proj(c, l, B, T, st, acc1_out));
  HIP_TRY(b_scan(c, l, B, T, st));
  HIP_TRY(b_rows_out(c, l, M, st));
  if (q2_out) HIP_TRY(hipMemcpyAsync(q2_out, c->gw.q, (size_t)M * c->di, hipMemcpyDeviceToDevice, st));
  HIP_TRY(b_out_proj(c, l, B, T, st, acc2_out));
  return DFSSM_OK;
}

// Tokens tok[b * tok_stride + t0 + t], t < T, of B sequences through every
// layer; with `head`, the last token of each sequence through the final norm,
// the LM head and the argmax.  Trace buffers (optional) are indexed by row
// m = b * T + t: h [L+1][B*T][d_model], q1 [L][B*T][d_model],
// q2 [L][B*T][d_inner], qf [B][d_model].
dfssm_status enqueue_step_gemm(dfssm_ctx* c, const int32_t* tok, int tok_stride, int t0, int B, int T, float* logits,
                               int32_t* next, int32_t* out, const Trace* tr, bool head, hipStream_t st) {
  auto& w = c->gw;
  const size_t M = (size_t)B * T;
  HIP_TRY(launch_embed_rows(tok, tok_stride, t0, B, T, c->lt<int8_t>(-1, DFSSM_G_EMBED),
                            c->lt<float>(-1, DFSSM_G_EMBED_SCALE), c->dm, c->V, w.h, c->err, st));
  for (int l = 0; l < c->L; ++l) {
    if (tr && tr->h)
      HIP_TRY(hipMemcpyAsync(tr->h + (size_t)l * M * c->dm, w.h, sizeof(float) * M * c->dm,
                             hipMemcpyDeviceToDevice, st));
    dfssm_status r = enqueue_layer_gemm(c, l, B, T, st, tr && tr->q1 ? tr->q1 + (size_t)l * M * c->dm : nullptr,
                                        tr && tr->q2 ? tr->q2 + (size_t)l * M * c->di : nullptr,
                                        tr && tr->acc1 ? tr->acc1 + (size_t)l * M * c->dproj : nullptr,
                                        tr && tr->acc2 ? tr->acc2 + (size_t)l * M * c->dm : nullptr);
    if (r != DFSSM_OK) return r;
  }
  if (tr && tr->h)
    HIP_TRY(hipMemcpyAsync(tr->h + (size_t)c->L * M * c->dm, w.h, sizeof(float) * M * c->dm,
                           hipMemcpyDeviceToDevice, st));
  if (!head) return DFSSM_OK;
  float* lg = logits ? logits : c->logits;
  HIP_TRY(b_head(c, B, T, lg, tr ? tr->qf : nullptr, st));
  if (next || out) HIP_TRY(launch_argmax(lg, c->V, B, next ? next : c->next, out, c->counter, st));
  return DFSSM_OK;
}

// Whether decode of batch B runs on the batched (GEMM) path.
bool use_gemm(const dfssm_ctx* c, int B) {
  if (c->path == DFSSM_PATH_KERNELS) return false;
  if (c->path == DFSSM_PATH_GEMM) return true;
  return B > 1;
}

// The batched workspace and state seen from sequence r0 on: every row-indexed
// workspace buffer and both state arrays shifted by r0 rows (the code buffer
// by r0 rows of its widest row, so either row width stays inside the shifted
// region), restored on destruction.  Kernels take the pointers when they are
// enqueued, so two row ranges can be enqueued one after the other.
struct RowShift {
  dfssm_ctx* c;
  dfssm_ctx::GemmWs gw;
  float *ssm, *conv;
  RowShift(dfssm_ctx* c_, int r0) : c(c_), gw(c_->gw), ssm(c_->ssm), conv(c_->conv) {
    auto& w = c->gw;
    const size_t r = (size_t)r0;
    w.h += r * c->dm;
    w.s += r;
    w.t += r * 16;
    w.zx += r * c->dproj;
    w.xc += r * c->cdim;
    w.g += r * c->di;
    w.q += r * (size_t)std::max(c->dm, c->di);
    w.qsum += r;
    c->ssm += r * c->ssm_bstride;
    c->conv += r * c->conv_bstride;
  }
  ~RowShift() {
    c->gw = gw;
    c->ssm = ssm;
    c->conv = conv;
  }
};

// Decode steps of two or more sequences split the layers into kSplitChains
// concurrent chains of consecutive sequences.  At small batches every kernel
// is a chain of memory latency using a fraction of the chip, so the chains
// overlap; at large batches one chain's projections overlap the other's
// state-bound scan (measured per step: batch 32 2.79 -> 2.57 ms, 128 7.69 ->
// 6.97, 256 12.74 -> 11.64, 512 22.6 -> 20.9; batch 64 unchanged).
// Sequences are independent and every kernel's result for a row depends on
// that row alone, so the split changes no value.  The embedding runs before
// the fork, the final norm, LM head and argmax after the join.
constexpr int kSplitChains = 2;
bool split_decode(int B) { return B >= 2; }

dfssm_status enqueue_decode_split(dfssm_ctx* c, const int32_t* tok, int B, float* logits, int32_t* next,
                                  int32_t* out, hipStream_t st) {
  const int n = std::min(kSplitChains, B);
  for (int k = 0; k < n; ++k)
    if (!c->split_st[k]) HIP_TRY(hipStreamCreateWithFlags(&c->split_st[k], hipStreamNonBlocking));
  for (int k = 0; k <= n; ++k)
    if (!c->split_ev[k]) HIP_TRY(hipEventCreateWithFlags(&c->split_ev[k], hipEventDisableTiming));
  auto& w = c->gw;
  HIP_TRY(launch_embed_rows(tok, 1, 0, B, 1, c->lt<int8_t>(-1, DFSSM_G_EMBED), c->lt<float>(-1, DFSSM_G_EMBED_SCALE),
                            c->dm, c->V, w.h, c->err, st));
  HIP_TRY(hipEventRecord(c->split_ev[0], st));
  int r0 = 0;
  for (int k = 0; k < n; ++k) {
    const int rows = B / n + (k < B % n ? 1 : 0);
    hipStream_t sk = c->split_st[k];
    HIP_TRY(hipStreamWaitEvent(sk, c->split_ev[0], 0));
    {
      RowShift shift(c, r0);
      for (int l = 0; l < c->L; ++l) {
        const dfssm_status r = enqueue_layer_gemm(c, l, rows, 1, sk, nullptr, nullptr);
        if (r != DFSSM_OK) return r;
      }
    }
    HIP_TRY(hipEventRecord(c->split_ev[1 + k], sk));
    r0 += rows;
  }
  for (int k = 0; k < n; ++k) HIP_TRY(hipStreamWaitEvent(st, c->split_ev[1 + k], 0));
  float* lg = logits ? logits : c->logits;
  HIP_TRY(b_head(c, B, 1, lg, nullptr, st));
  if (next || out) HIP_TRY(launch_argmax(lg, c->V, B, next ? next : c->next, out, c->counter, st));
  return DFSSM_OK;
}

// one decode step of B sequences on whichever path serves batch B (not the persistent one)
dfssm_status enqueue_decode(dfssm_ctx* c, const int32_t* tok, int B, float* logits, int32_t* next, int32_t* out,
                            const Trace* tr, hipStream_t st) {
  if (use_gemm(c, B)) {
    if (!tr && split_decode(B)) return enqueue_decode_split(c, tok, B, logits, next, out, st);
    return enqueue_step_gemm(c, tok, 1, 0, B, 1, logits, next, out, tr, true, st);
  }
  return enqueue_step(c, tok, 1, B, logits, next, out, tr, true, st);
}

// Whether batch-B work runs on the persistent kernel; fails when it is required but cannot run.
dfssm_status use_persistent(const dfssm_ctx* c, int B, bool* yes) {
  *yes = false;
  if (B != 1 || c->path == DFSSM_PATH_KERNELS || c->path == DFSSM_PATH_GEMM) return DFSSM_OK;
  if (!c->persist_ok) {
    if (c->path == DFSSM_PATH_PERSISTENT)
      return fail(DFSSM_E_UNSUPPORTED, "persistent decode unavailable: " + c->persist_why);
    return DFSSM_OK;
  }
  *yes = true;
  return DFSSM_OK;
}

dfssm_status run_persistent(dfssm_ctx* c, const int32_t* tok_in, int32_t* tok_last, int32_t* tok_out, int n_tokens,
                            float* logits, const Trace* tr, hipStream_t st, unsigned long long* prof = nullptr,
                            int prof_tokens = 0) {
  const unsigned need = (unsigned)n_tokens * persistent_exchanges_per_token(c->L) + 1;
  if ((unsigned long long)c->host_epoch + need >= 0x7fffffffull) {
    // epochs are never reused: clear the boxes and start over
    HIP_TRY(launch_zero(c->boxes, sizeof(uint64_t) * c->box_words, st));
    c->host_epoch = 1;
    c->pair_count = 1;
  }
  PersistArgs a{};
  a.wbase = c->wbuf;
  a.n_layer = c->L;
  a.d_model = c->dm;
  a.d_inner = c->di;
  a.d_state = c->N;
  a.headdim = c->P;
  a.n_heads = c->H;
  a.vocab = c->V;
  a.d_conv = c->K;
  a.rank = c->r;
  a.eps = c->eps;
  a.E = c->lt<int8_t>(-1, DFSSM_G_EMBED);
  a.sE = c->lt<float>(-1, DFSSM_G_EMBED_SCALE);
  a.final_norm = c->lt<float>(-1, DFSSM_G_FINAL_NORM);
  a.conv = c->conv;
  a.ssm = c->ssm;
  a.boxes = c->boxes;
  a.epoch0 = c->host_epoch;
  a.pair0 = c->pair_count;
  a.abort_flag = c->abort_flag;
  a.err = c->err;
  a.tok_in = tok_in;
  a.tok_last = tok_last;
  a.tok_out = tok_out;
  a.n_tokens = n_tokens;
  a.logits = logits ? logits : c->logits;
  if (tr) {
    a.trace_h = tr->h;
    a.trace_q1 = tr->q1;
    a.trace_q2 = tr->q2;
    a.trace_qf = tr->qf;
    a.trace_acc1 = tr->acc1;
    a.trace_acc2 = tr->acc2;
  }
  a.prof = prof;
  a.prof_tokens = prof_tokens;
  c->host_epoch += need;
  c->pair_count += (unsigned)n_tokens * (unsigned)c->L;
  HIP_TRY(launch_decode_persistent(a, c->persist_grid, st));
  return DFSSM_OK;
}

dfssm_status check_ctx(const dfssm_ctx* c, bool need_loaded = true) {
  if (!c) return fail(DFSSM_E_INVALID, "null context");
  if (need_loaded && !c->loaded) return fail(DFSSM_E_STATE, "weights not loaded");
  return DFSSM_OK;
}

dfssm_status check_B(const dfssm_ctx* c, int B) {
  if (B < 1 || B > c->maxB)
    return fail(DFSSM_E_INVALID, "batch " + std::to_string(B) + " outside [1, " + std::to_string(c->maxB) + "]");
  return DFSSM_OK;
}

}  // namespace

// ===========================================================================
// C ABI
// ===========================================================================

extern "C" {

const char* dfssm_version(void) { return "dfssm-mi355x 0.1 (gfx950)"; }

const char* dfssm_last_error(const dfssm_ctx*) { return g_err.c_str(); }

}  // extern "C"

namespace {

// Dimensions and the memory plan of a context: weights | state | decode
// workspace | mailboxes | abort flag | batched-path workspace (the last only
// when the caller provides the arena).  Pure host arithmetic.
void plan_memory(dfssm_ctx* c, const dfssm_config* cfg) {
  c->cfg = *cfg;
  c->L = cfg->n_layer;
  c->dm = cfg->d_model;
  c->di = cfg->d_inner;
  c->N = cfg->d_state;
  c->P = cfg->headdim;
  c->H = cfg->d_inner / cfg->headdim;
  c->V = cfg->vocab;
  c->K = cfg->d_conv;
  c->r = cfg->lora_rank;
  c->maxB = cfg->max_batch;
  c->cdim = c->di + 2 * c->N;
  c->dproj = 2 * c->di + 2 * c->N + c->H;
  c->eps = cfg->norm_eps > 0.0f ? cfg->norm_eps : 1e-5f;
  c->chunk_rows = cfg->max_chunk_rows > 0 ? (size_t)cfg->max_chunk_rows : kPrefillChunkRows;

  // weights
  size_t off = 0;
  c->layer_t.assign((size_t)c->L * DFSSM_T_PER_LAYER, TensorInfo{});
  for (int l = 0; l < c->L; ++l)
    for (int k = 0; k < DFSSM_T_PER_LAYER; ++k) {
      Spec sp = layer_spec(c, k);
      TensorInfo& t = c->layer_t[(size_t)l * DFSSM_T_PER_LAYER + k];
      t.offset = off;
      t.count = sp.count;
      t.elem = sp.elem;
      t.bytes = sp.count * sp.elem;
      off += align_up(t.bytes);
    }
  c->global_t.assign(3, TensorInfo{});
  for (int k = 0; k < 3; ++k) {
    Spec sp = global_spec(c, k);
    TensorInfo& t = c->global_t[k];
    t.offset = off;
    t.count = sp.count;
    t.elem = sp.elem;
    t.bytes = sp.count * sp.elem;
    off += align_up(t.bytes);
  }
  c->wbytes = off;

  // state
  c->conv_bstride = (size_t)c->L * (c->K - 1) * c->cdim;
  c->ssm_bstride = (size_t)c->L * c->H * c->P * c->N;
  const size_t conv_bytes = align_up(sizeof(float) * c->conv_bstride * c->maxB);
  const size_t ssm_bytes = align_up(sizeof(float) * c->ssm_bstride * c->maxB);
  c->sbytes = conv_bytes + ssm_bytes;

  // decode workspace (all [max_batch][...])
  const size_t B = c->maxB;
  size_t wo = 0;
  auto take = [&](size_t bytes) { size_t o = wo; wo += align_up(bytes); return o; };
  auto& o = c->wo;
  o.h = take(sizeof(float) * B * c->dm);
  o.zx = take(sizeof(float) * B * c->dproj);
  o.xc = take(sizeof(float) * B * c->cdim);
  o.g = take(sizeof(float) * B * c->di);
  o.lg = take(sizeof(float) * B * c->V);
  o.q1 = take(B * c->dm);
  o.q2 = take(B * c->di);
  o.p1 = take(sizeof(uint32_t) * B * (c->dm / 32) * 8);
  o.p2 = take(sizeof(uint32_t) * B * (c->di / 32) * 8);
  o.qs1 = take(4 * B);
  o.qs2 = take(4 * B);
  o.s1 = take(4 * B);
  o.s2 = take(4 * B);
  o.t1 = take(4 * B * c->r);
  o.t2 = take(4 * B * c->r);
  o.nx = take(4 * B);
  o.ct = take(4);
  o.er = take(4);
  c->wsbytes = wo;

  // mailboxes of the persistent kernel (sized whenever the shape is one it is
  // compiled for; unused if the device cannot run it)
  c->persist_grid = c->H * (c->P / 16);
  size_t stride = 0, offs[DFSSM_T_PER_LAYER];
  c->box_words = persistent_layout(c->dm, c->di, c->N, c->P, &stride, offs)
                     ? persistent_box_words(c->dm, c->di, c->N, c->persist_grid) : 0;

  size_t a = 0;
  c->o_w = a; a += align_up(c->wbytes);
  c->o_s = a; a += align_up(c->sbytes);
  c->o_ws = a; a += align_up(c->wsbytes);
  c->o_box = a; a += align_up(sizeof(uint64_t) * c->box_words);
  c->o_abort = a; a += kAlign;
  c->o_gw = a;
  c->arena_bytes = a;  // without the batched-path workspace
}

// ---------------------------------------------------------------------------
// the stateless matrix-core projection (dfssm_k_gemm and its allocation-free twin)
// ---------------------------------------------------------------------------
dfssm_status check_k_gemm(const uint32_t* d_bits, const float* d_sw, const int8_t* d_A, const float* d_sA,
                          const int8_t* d_B, const float* d_sB, int32_t d_in, int32_t d_out, const int8_t* d_q,
                          const float* d_s, int32_t M, float* d_y) {
  if (!d_bits || !d_sw || !d_A || !d_sA || !d_B || !d_sB || !d_q || !d_s || !d_y)
    return fail(DFSSM_E_INVALID, "null pointer");
  if (d_in < 128 || d_in % 128 || (d_in / 128) > 64 || ((d_in / 128) & (d_in / 128 - 1)))
    return fail(DFSSM_E_UNSUPPORTED, "d_in must be 128 * 2^k <= 8192");
  if (d_out < 1 || M < 1 || M > 65535) return fail(DFSSM_E_INVALID, "bad d_out / M");
  return DFSSM_OK;
}

// operand scratch of one projection: the activations' bit planes (M d_in
// bytes), their row sums (4 M) and LoRA-down vectors (64 M)
size_t k_gemm_scratch_bytes(int d_in, int M) {
  return align_up((size_t)M * d_in) + align_up(4 * (size_t)M) + align_up(4 * (size_t)M * 16);
}

hipError_t k_gemm_run(const uint32_t* d_bits, const float* d_sw, const int8_t* d_A, const float* d_sA,
                      const int8_t* d_B, const float* d_sB, int d_in, int d_out, const int8_t* d_q, const float* d_s,
                      int M, int32_t* d_acc, float* d_y, char* tmp, hipStream_t st) {
  uint32_t* planes = (uint32_t*)tmp;
  int32_t* qsum = (int32_t*)(tmp + align_up((size_t)M * d_in));
  float* t = (float*)(tmp + align_up((size_t)M * d_in) + align_up(4 * (size_t)M));
  hipError_t e = launch_qprep(d_q, d_s, d_in, M, d_A, d_sA, 16, planes, qsum, t, st);
  if (e != hipSuccess) return e;
  if (M <= kSkinnyDecodeRows) {  // the decode-sized kernel
    SkinnyArgs a{};
    a.q = d_q; a.s = d_s; a.qsum = qsum; a.t = t;
    a.w = d_bits; a.sw = d_sw; a.Bm = d_B; a.sB = d_sB;
    a.M = M; a.N = d_out; a.K = d_in;
    a.y = d_y; a.ldy = d_out; a.acc = d_acc;
    return launch_gemm_skinny(a, SK_IN, st);
  }
  GemmArgs a{d_q, d_s, qsum, t, d_bits, d_sw, d_B, d_sB, M, d_out, d_in, d_y, d_out, d_acc};
  return launch_bitgemm(a, GEMM_EPI_STORE, st);
}

// The allocation-free entry point's scratch (declared at file scope above)
// is reached only through the per-device address that hipGetSymbolAddress
// returns, taken once per device with that device current.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

dfssm_status noalloc_scratch(char** out) {
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(DFSSM_E_UNSUPPORTED, "device index beyond the scratch table");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(DFSSM_E_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = (char*)g_scratch_ptr[dev];
  return DFSSM_OK;
}

}  // namespace

extern "C" {

dfssm_status dfssm_arena_bytes(const dfssm_config* cfg, size_t* bytes) {
  if (!bytes) return fail(DFSSM_E_INVALID, "null output pointer");
  dfssm_status v = validate(cfg);
  if (v != DFSSM_OK) return v;
  dfssm_ctx tmp;
  plan_memory(&tmp, cfg);
  *bytes = tmp.o_gw + align_up(gemm_layout(&tmp, fixed_gemm_rows(&tmp)).bytes);
  return DFSSM_OK;
}

dfssm_status dfssm_create(const dfssm_config* cfg, int32_t device, void* arena, size_t arena_bytes,
                          dfssm_ctx** out) {
  if (!out) return fail(DFSSM_E_INVALID, "null output pointer");
  *out = nullptr;
  dfssm_status v = validate(cfg);
  if (v != DFSSM_OK) return v;
  if (arena && ((uintptr_t)arena % kAlign))
    return fail(DFSSM_E_INVALID, "the arena must be 256-byte aligned");
  int ndev = 0;
  HIP_TRY(hipGetDeviceCount(&ndev));
  if (device < 0 || device >= ndev) return fail(DFSSM_E_INVALID, "device index out of range");
  HIP_TRY(hipSetDevice(device));

  dfssm_ctx* c = new dfssm_ctx();
  c->device = device;
  plan_memory(c, cfg);
  const GemmLayout gl = gemm_layout(c, fixed_gemm_rows(c));
  const size_t need = c->o_gw + align_up(gl.bytes);
  if (arena) {
    if (arena_bytes < need) {
      delete c;
      return fail(DFSSM_E_INVALID, "arena too small: " + std::to_string(arena_bytes) + " bytes, need " +
                                       std::to_string(need) + " (dfssm_arena_bytes)");
    }
    c->arena = (char*)arena;
    c->own_arena = false;
    assign_gemm_ws(c, c->arena + c->o_gw, fixed_gemm_rows(c), gl);
    c->gw.fixed = true;
  } else {
    if (hipMalloc(&c->arena, c->arena_bytes) != hipSuccess) {
      (void)hipGetLastError();
      delete c;
      return fail(DFSSM_E_OOM, "device allocation failed");
    }
    c->own_arena = true;
  }
  c->wbuf = c->arena + c->o_w;
  c->sbuf = c->arena + c->o_s;
  c->ws = c->arena + c->o_ws;
  c->conv = (float*)c->sbuf;
  c->ssm = (float*)(c->sbuf + align_up(sizeof(float) * c->conv_bstride * c->maxB));
  char* w = c->ws;
  const auto& o = c->wo;
  c->h = (float*)(w + o.h);
  c->zx = (float*)(w + o.zx);
  c->xc = (float*)(w + o.xc);
  c->g = (float*)(w + o.g);
  c->logits = (float*)(w + o.lg);
  c->q1 = (int8_t*)(w + o.q1);
  c->q2 = (int8_t*)(w + o.q2);
  c->pl1 = (uint32_t*)(w + o.p1);
  c->pl2 = (uint32_t*)(w + o.p2);
  c->qs1 = (int32_t*)(w + o.qs1);
  c->qs2 = (int32_t*)(w + o.qs2);
  c->s1 = (float*)(w + o.s1);
  c->s2 = (float*)(w + o.s2);
  c->t1 = (float*)(w + o.t1);
  c->t2 = (float*)(w + o.t2);
  c->next = (int32_t*)(w + o.nx);
  c->counter = (int32_t*)(w + o.ct);
  c->err = (int*)(w + o.er);
  c->boxes = c->box_words ? (uint64_t*)(c->arena + c->o_box) : nullptr;
  c->abort_flag = (int*)(c->arena + c->o_abort);
  // state, workspace, mailboxes and the abort flag start at zero
  if (launch_zero(c->arena + c->o_s, c->o_gw - c->o_s, nullptr) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
    dfssm_destroy(c);
    return fail(DFSSM_E_HIP, "initial clear failed");
  }
  // persistent batch-1 path: supported on this device, and the weight layout the kernel assumes
  const char* why = "";
  c->persist_ok = c->box_words > 0 &&
                  persistent_supported(c->dm, c->di, c->N, c->P, c->H, c->r, c->persist_grid, &why);
  c->persist_why = why;
  if (c->persist_ok && c->L < 2) {
    // the kernel re-reads a layer's conv and SSM state one layer after writing it back
    c->persist_ok = false;
    c->persist_why = "the persistent kernel needs at least 2 layers";
  }
  if (c->persist_ok) {
    // the kernel addresses layer l, kind k as base + l * stride + offset(k): check that this is our layout
    size_t stride = 0, offs[DFSSM_T_PER_LAYER];
    bool same = persistent_layout(c->dm, c->di, c->N, c->P, &stride, offs);
    for (int l = 0; same && l < c->L; ++l)
      for (int k = 0; same && k < DFSSM_T_PER_LAYER; ++k)
        same = c->layer_t[(size_t)l * DFSSM_T_PER_LAYER + k].offset == (size_t)l * stride + offs[k];
    if (!same) {
      c->persist_ok = false;
      c->persist_why = "weight layout differs from the persistent kernel's";
    }
  }
  *out = c;
  return DFSSM_OK;
}

void dfssm_destroy(dfssm_ctx* c) {
  if (!c) return;
  (void)hipSetDevice(c->device);
  (void)hipDeviceSynchronize();
  for (auto& kv : c->graphs) (void)hipGraphExecDestroy(kv.second);
  for (hipStream_t s : c->split_st)
    if (s) (void)hipStreamDestroy(s);
  for (hipEvent_t e : c->split_ev)
    if (e) (void)hipEventDestroy(e);
  if (c->gw.buf && !c->gw.fixed) (void)hipFree(c->gw.buf);
  if (c->arena && c->own_arena) (void)hipFree(c->arena);
  delete c;
}

dfssm_status dfssm_device_bytes(const dfssm_ctx* c, size_t* bytes) {
  if (!c || !bytes) return fail(DFSSM_E_INVALID, "null argument");
  *bytes = c->arena_bytes + c->gw.bytes;
  return DFSSM_OK;
}

dfssm_status dfssm_load_synthetic(dfssm_ctx* c, uint64_t seed, void* stream) {
  dfssm_status v = check_ctx(c, false);
  if (v != DFSSM_OK) return v;
  HIP_TRY(hipSetDevice(c->device));
  for (int l = 0; l < c->L; ++l)
    for (int k = 0; k < DFSSM_T_PER_LAYER; ++k) {
      const TensorInfo& t = c->layer_t[(size_t)l * DFSSM_T_PER_LAYER + k];
      const GenParam gp = layer_gen(k);
      const uint64_t tid = (uint64_t)(64 * l + k);
      const uint64_t key = host_mix64(seed ^ (tid << 32));
      HIP_TRY(launch_gen(c->wbuf + t.offset, t.count, gp.mode, key, gp.a, gp.b - gp.a, gp.cval, S(stream)));
    }
  for (int k = 0; k < 3; ++k) {
    const TensorInfo& t = c->global_t[k];
    const GenParam gp = global_gen(k);
    const uint64_t tid = (uint64_t)(4096 + k);
    const uint64_t key = host_mix64(seed ^ (tid << 32));
    HIP_TRY(launch_gen(c->wbuf + t.offset, t.count, gp.mode, key, gp.a, gp.b - gp.a, gp.cval, S(stream)));
  }
  HIP_TRY(launch_zero(c->sbuf, c->sbytes, S(stream)));
  c->loaded = true;
  return DFSSM_OK;
}

static dfssm_status tensor_lookup(dfssm_ctx* c, int32_t layer, int32_t kind, size_t bytes, const TensorInfo** ti) {
  if (!c) return fail(DFSSM_E_INVALID, "null context");
  if (layer >= c->L || layer < -1) return fail(DFSSM_E_INVALID, "layer out of range");
  if (layer >= 0 && (kind < 0 || kind >= DFSSM_T_PER_LAYER)) return fail(DFSSM_E_INVALID, "tensor kind out of range");
  if (layer < 0 && (kind < 0 || kind > 2)) return fail(DFSSM_E_INVALID, "global tensor kind out of range");
  const TensorInfo& t = layer >= 0 ? c->layer_t[(size_t)layer * DFSSM_T_PER_LAYER + kind] : c->global_t[kind];
  if (bytes != t.bytes)
    return fail(DFSSM_E_INVALID, "tensor size mismatch: got " + std::to_string(bytes) + ", need " + std::to_string(t.bytes));
  *ti = &t;
  return DFSSM_OK;
}

dfssm_status dfssm_set_tensor(dfssm_ctx* c, int32_t layer, int32_t kind, const void* host, size_t bytes) {
  const TensorInfo* t = nullptr;
  dfssm_status v = tensor_lookup(c, layer, kind, bytes, &t);
  if (v != DFSSM_OK) return v;
  if (!host) return fail(DFSSM_E_INVALID, "null host pointer");
  HIP_TRY(hipSetDevice(c->device));
  HIP_TRY(hipDeviceSynchronize());
  HIP_TRY(hipMemcpy(c->wbuf + t->offset, host, bytes, hipMemcpyHostToDevice));
  c->loaded = true;
  return DFSSM_OK;
}

dfssm_status dfssm_get_tensor(dfssm_ctx* c, int32_t layer, int32_t kind, void* host, size_t bytes) {
  const TensorInfo* t = nullptr;
  dfssm_status v = tensor_lookup(c, layer, kind, bytes, &t);
  if (v != DFSSM_OK) return v;
  if (!host) return fail(DFSSM_E_INVALID, "null host pointer");
  HIP_TRY(hipSetDevice(c->device));
  HIP_TRY(hipDeviceSynchronize());
  HIP_TRY(hipMemcpy(host, c->wbuf + t->offset, bytes, hipMemcpyDeviceToHost));
  return DFSSM_OK;
}

dfssm_status dfssm_reset_state(dfssm_ctx* c, int32_t batch, void* stream) {
  dfssm_status v = check_ctx(c, false);
  if (v != DFSSM_OK) return v;
  if ((v = check_B(c, batch)) != DFSSM_OK) return v;
  HIP_TRY(launch_zero(c->conv, sizeof(float) * c->conv_bstride * batch, S(stream)));
  HIP_TRY(launch_zero(c->ssm, sizeof(float) * c->ssm_bstride * batch, S(stream)));
  return DFSSM_OK;
}

dfssm_status dfssm_get_state(dfssm_ctx* c, int32_t seq, float* host_conv, float* host_ssm) {
  dfssm_status v = check_ctx(c, false);
  if (v != DFSSM_OK) return v;
  if (seq < 0 || seq >= c->maxB) return fail(DFSSM_E_INVALID, "sequence slot out of range");
  HIP_TRY(hipSetDevice(c->device));
  HIP_TRY(hipDeviceSynchronize());
  const int K1 = c->K - 1;
  if (host_conv) {
    std::vector<float> tmp(c->conv_bstride);
    HIP_TRY(hipMemcpy(tmp.data(), c->conv + (size_t)seq * c->conv_bstride, sizeof(float) * tmp.size(),
                      hipMemcpyDeviceToHost));
    for (int l = 0; l < c->L; ++l)
      for (int k = 0; k < K1; ++k)
        for (int ch = 0; ch < c->cdim; ++ch)
          host_conv[((size_t)l * c->cdim + ch) * K1 + k] = tmp[((size_t)l * K1 + k) * c->cdim + ch];
  }
  if (host_ssm) {
    std::vector<float> tmp(c->ssm_bstride);
    HIP_TRY(hipMemcpy(tmp.data(), c->ssm + (size_t)seq * c->ssm_bstride, sizeof(float) * tmp.size(),
                      hipMemcpyDeviceToHost));
    const int G = c->P / 16;
    for (int l = 0; l < c->L; ++l)
      for (int h = 0; h < c->H; ++h)
        for (int p = 0; p < c->P; ++p)
          for (int n = 0; n < c->N; ++n) {
            const size_t src = ((((size_t)l * c->H + h) * G + p / 16) * c->N + n) * 16 + (p % 16);
            host_ssm[(((size_t)l * c->H + h) * c->P + p) * c->N + n] = tmp[src];
          }
  }
  return DFSSM_OK;
}

dfssm_status dfssm_set_state(dfssm_ctx* c, int32_t seq, const float* host_conv, const float* host_ssm) {
  dfssm_status v = check_ctx(c, false);
  if (v != DFSSM_OK) return v;
  if (seq < 0 || seq >= c->maxB) return fail(DFSSM_E_INVALID, "sequence slot out of range");
  HIP_TRY(hipSetDevice(c->device));
  HIP_TRY(hipDeviceSynchronize());
  const int K1 = c->K - 1;
  if (host_conv) {
    std::vector<float> tmp(c->conv_bstride);
    for (int l = 0; l < c->L; ++l)
      for (int k = 0; k < K1; ++k)
        for (int ch = 0; ch < c->cdim; ++ch)
          tmp[((size_t)l * K1 + k) * c->cdim + ch] = host_conv[((size_t)l * c->cdim + ch) * K1 + k];
    HIP_TRY(hipMemcpy(c->conv + (size_t)seq * c->conv_bstride, tmp.data(), sizeof(float) * tmp.size(),
                      hipMemcpyHostToDevice));
  }
  if (host_ssm) {
    std::vector<float> tmp(c->ssm_bstride);
    const int G = c->P / 16;
    for (int l = 0; l < c->L; ++l)
      for (int h = 0; h < c->H; ++h)
        for (int p = 0; p < c->P; ++p)
          for (int n = 0; n < c->N; ++n) {
            const size_t dst = ((((size_t)l * c->H + h) * G + p / 16) * c->N + n) * 16 + (p % 16);
            tmp[dst] = host_ssm[(((size_t)l * c->H + h) * c->P + p) * c->N + n];
          }
    HIP_TRY(hipMemcpy(c->ssm + (size_t)seq * c->ssm_bstride, tmp.data(), sizeof(float) * tmp.size(),
                      hipMemcpyHostToDevice));
  }
  return DFSSM_OK;
}

dfssm_status dfssm_decode_step(dfssm_ctx* c, const int32_t* d_tok, int32_t B, float* d_logits, int32_t* d_next,
                               void* stream) {
  dfssm_status v = check_ctx(c);
  if (v != DFSSM_OK) return v;
  if ((v = check_B(c, B)) != DFSSM_OK) return v;
  if (!d_tok) return fail(DFSSM_E_INVALID, "null token pointer");
  bool pers = false;
  if ((v = use_persistent(c, B, &pers)) != DFSSM_OK) return v;
  if (pers) return run_persistent(c, d_tok, nullptr, d_next, 1, d_logits, nullptr, S(stream));
  if (use_gemm(c, B) && (v = ensure_gemm_ws(c, B)) != DFSSM_OK) return v;
  return enqueue_decode(c, d_tok, B, d_logits, d_next, nullptr, nullptr, S(stream));
}

dfssm_status dfssm_generate(dfssm_ctx* c, int32_t* d_tok, int32_t B, int32_t n_steps, int32_t* d_out,
                            int32_t use_graph, void* stream) {
  dfssm_status v = check_ctx(c);
  if (v != DFSSM_OK) return v;
  if ((v = check_B(c, B)) != DFSSM_OK) return v;
  if (!d_tok) return fail(DFSSM_E_INVALID, "null token pointer");
  if (n_steps < 0) return fail(DFSSM_E_INVALID, "negative step count");
  if (n_steps == 0) return DFSSM_OK;
  hipStream_t st = S(stream);
  bool pers = false;
  if ((v = use_persistent(c, B, &pers)) != DFSSM_OK) return v;
  if (pers) return run_persistent(c, d_tok, d_tok, d_out, n_steps, nullptr, nullptr, st);
  if (use_gemm(c, B) && (v = ensure_gemm_ws(c, B)) != DFSSM_OK) return v;
  if (d_out) HIP_TRY(launch_zero(c->counter, 4, st));
  if (!use_graph) {
    for (int i = 0; i < n_steps; ++i) {
      v = enqueue_decode(c, d_tok, B, nullptr, d_tok, d_out, nullptr, st);
      if (v != DFSSM_OK) return v;
    }
    return DFSSM_OK;
  }
  auto key = std::make_tuple((int)B * 4 + (use_gemm(c, B) ? 1 : 0), (const void*)d_tok, (const void*)d_out);
  auto it = c->graphs.find(key);
  hipGraphExec_t exec = nullptr;
  if (it == c->graphs.end()) {
    hipStream_t cap = nullptr;
    HIP_TRY(hipStreamCreateWithFlags(&cap, hipStreamNonBlocking));
    hipGraph_t graph = nullptr;
    hipError_t e = hipStreamBeginCapture(cap, hipStreamCaptureModeThreadLocal);
    if (e == hipSuccess) {
      v = enqueue_decode(c, d_tok, B, nullptr, d_tok, d_out, nullptr, cap);
      hipError_t e2 = hipStreamEndCapture(cap, &graph);
      if (v == DFSSM_OK && e2 != hipSuccess) v = fail(DFSSM_E_HIP, std::string("graph capture: ") + hipGetErrorString(e2));
    } else {
      v = fail(DFSSM_E_HIP, std::string("begin capture: ") + hipGetErrorString(e));
    }
    if (v == DFSSM_OK) {
      e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
      if (e != hipSuccess) v = fail(DFSSM_E_HIP, std::string("graph instantiate: ") + hipGetErrorString(e));
    }
    if (graph) (void)hipGraphDestroy(graph);
    (void)hipStreamDestroy(cap);
    if (v != DFSSM_OK) return v;
    c->graphs[key] = exec;
  } else {
    exec = it->second;
  }
  for (int i = 0; i < n_steps; ++i) HIP_TRY(hipGraphLaunch(exec, st));
  return DFSSM_OK;
}

dfssm_status dfssm_prefill(dfssm_ctx* c, const int32_t* d_tok, int32_t B, int32_t T, float* d_last_logits,
                           int32_t* d_next, void* stream) {
  dfssm_status v = check_ctx(c);
  if (v != DFSSM_OK) return v;
  if ((v = check_B(c, B)) != DFSSM_OK) return v;
  if (!d_tok) return fail(DFSSM_E_INVALID, "null token pointer");
  if (T < 1) return fail(DFSSM_E_INVALID, "prompt length must be >= 1");
  if (c->path != DFSSM_PATH_KERNELS) {
    // batched path, in chunks of whole token rows across the B sequences
    const int tc = (int)std::max<size_t>(1, std::min<size_t>((size_t)T, c->chunk_rows / (size_t)B));
    if ((v = ensure_gemm_ws(c, (size_t)B * tc)) != DFSSM_OK) return v;
    for (int t0 = 0; t0 < T; t0 += tc) {
      const int n = std::min(tc, T - t0);
      const bool last = t0 + n == T;
      v = enqueue_step_gemm(c, d_tok, T, t0, B, n, last ? d_last_logits : nullptr, last ? d_next : nullptr, nullptr,
                            nullptr, last && (d_last_logits || d_next), S(stream));
      if (v != DFSSM_OK) return v;
    }
    return DFSSM_OK;
  }
  for (int t = 0; t < T; ++t) {
    const bool last = t == T - 1;
    v = enqueue_step(c, d_tok + t, T, B, last ? d_last_logits : nullptr, last ? d_next : nullptr, nullptr, nullptr,
                     last && (d_last_logits || d_next), S(stream));
    if (v != DFSSM_OK) return v;
  }
  return DFSSM_OK;
}

dfssm_status dfssm_layer_step(dfssm_ctx* c, int32_t layer, const float* d_h_in, float* d_h_out, int32_t B,
                              int8_t* d_q1, int8_t* d_q2, void* stream) {
  dfssm_status v = check_ctx(c);
  if (v != DFSSM_OK) return v;
  if ((v = check_B(c, B)) != DFSSM_OK) return v;
  if (layer < 0 || layer >= c->L) return fail(DFSSM_E_INVALID, "layer out of range");
  if (!d_h_in || !d_h_out) return fail(DFSSM_E_INVALID, "null activation pointer");
  hipStream_t st = S(stream);
  HIP_TRY(hipMemcpyAsync(c->h, d_h_in, sizeof(float) * B * c->dm, hipMemcpyDeviceToDevice, st));
  v = enqueue_layer(c, layer, B, st, d_q1, d_q2);
  if (v != DFSSM_OK) return v;
  HIP_TRY(hipMemcpyAsync(d_h_out, c->h, sizeof(float) * B * c->dm, hipMemcpyDeviceToDevice, st));
  return DFSSM_OK;
}

dfssm_status dfssm_layer_step_f16(dfssm_ctx* c, int32_t layer, const uint16_t* d_h_f16, float* d_h_out, int32_t B,
                                  int8_t* d_q1, int8_t* d_q2, void* stream) {
  dfssm_status v = check_ctx(c);
  if (v != DFSSM_OK) return v;
  if ((v = check_B(c, B)) != DFSSM_OK) return v;
  if (layer < 0 || layer >= c->L) return fail(DFSSM_E_INVALID, "layer out of range");
  if (!d_h_f16 || !d_h_out) return fail(DFSSM_E_INVALID, "null activation pointer");
  hipStream_t st = S(stream);
  HIP_TRY(launch_f16_to_f32(d_h_f16, c->h, (size_t)B * c->dm, st));
  v = enqueue_layer(c, layer, B, st, d_q1, d_q2);
  if (v != DFSSM_OK) return v;
  HIP_TRY(hipMemcpyAsync(d_h_out, c->h, sizeof(float) * B * c->dm, hipMemcpyDeviceToDevice, st));
  return DFSSM_OK;
}

dfssm_status dfssm_trace_step(dfssm_ctx* c, const int32_t* d_tok, int32_t B, float* d_h_trace, int8_t* d_q1_trace,
                              int8_t* d_q2_trace, int8_t* d_qf, float* d_logits, int32_t* d_acc1_trace,
                              int32_t* d_acc2_trace, void* stream) {
  dfssm_status v = check_ctx(c);
  if (v != DFSSM_OK) return v;
  if ((v = check_B(c, B)) != DFSSM_OK) return v;
  if (!d_tok || !d_h_trace) return fail(DFSSM_E_INVALID, "null pointer");
  Trace tr;
  tr.h = d_h_trace;
  tr.q1 = d_q1_trace;
  tr.q2 = d_q2_trace;
  tr.qf = d_qf;
  tr.acc1 = d_acc1_trace;
  tr.acc2 = d_acc2_trace;
  bool pers = false;
  if ((v = use_persistent(c, B, &pers)) != DFSSM_OK) return v;
  if (pers) return run_persistent(c, d_tok, nullptr, nullptr, 1, d_logits, &tr, S(stream));
  if (use_gemm(c, B) && (v = ensure_gemm_ws(c, B)) != DFSSM_OK) return v;
  return enqueue_decode(c, d_tok, B, d_logits, nullptr, nullptr, &tr, S(stream));
}

dfssm_status dfssm_trace_prefill(dfssm_ctx* c, const int32_t* d_tok, int32_t B, int32_t T, float* d_h_trace,
                                 int8_t* d_q1_trace, int8_t* d_q2_trace, int8_t* d_qf, float* d_logits,
                                 int32_t* d_acc1_trace, int32_t* d_acc2_trace, void* stream) {
  dfssm_status v = check_ctx(c);
  if (v != DFSSM_OK) return v;
  if ((v = check_B(c, B)) != DFSSM_OK) return v;
  if (!d_tok || !d_h_trace) return fail(DFSSM_E_INVALID, "null pointer");
  if (T < 1 || (size_t)B * T > c->chunk_rows)
    return fail(DFSSM_E_INVALID, "traced prefill takes 1 <= B * T <= " + std::to_string(c->chunk_rows) + " rows");
  if ((v = ensure_gemm_ws(c, (size_t)B * T)) != DFSSM_OK) return v;
  Trace tr;
  tr.h = d_h_trace;
  tr.q1 = d_q1_trace;
  tr.q2 = d_q2_trace;
  tr.qf = d_qf;
  tr.acc1 = d_acc1_trace;
  tr.acc2 = d_acc2_trace;
  return enqueue_step_gemm(c, d_tok, T, 0, B, T, d_logits, nullptr, nullptr, &tr, true, S(stream));
}

dfssm_status dfssm_time_kernel(dfssm_ctx* c, int32_t kernel, int32_t B, int32_t iters, float* avg_us, void* stream) {
  dfssm_status v = check_ctx(c);
  if (v != DFSSM_OK) return v;
  if ((v = check_B(c, B)) != DFSSM_OK) return v;
  if (iters < 1 || !avg_us) return fail(DFSSM_E_INVALID, "iters must be >= 1 and avg_us non-null");
  if (kernel < DFSSM_K_IN_PROJ || kernel > DFSSM_K_B_LM_HEAD) return fail(DFSSM_E_INVALID, "unknown kernel id");
  const bool batched = kernel >= DFSSM_K_B_ROWS_IN;
  if (batched && (v = ensure_gemm_ws(c, B)) != DFSSM_OK) return v;
  hipStream_t st = S(stream);
  auto launch = [&](int i) -> hipError_t {
    const int l = i % c->L;
    switch (kernel) {
      case DFSSM_K_IN_PROJ: return in_proj(c, l, B, st);
      case DFSSM_K_SSM: return ssm_step(c, l, B, st);
      case DFSSM_K_OUT_PROJ: return out_proj(c, l, B, st);
      case DFSSM_K_LM_HEAD: return lm_head(c, B, c->logits, st);
      case DFSSM_K_NORM_QUANT: return norm_quant_in(c, l, B, st);
      case DFSSM_K_B_ROWS_IN: return b_rows_in(c, l, B, st);
      case DFSSM_K_B_IN_PROJ: return b_in_proj(c, l, B, 1, st);
      case DFSSM_K_B_SCAN: return b_scan(c, l, B, 1, st);
      case DFSSM_K_B_ROWS_OUT: return b_rows_out(c, l, B, st);
      case DFSSM_K_B_OUT_PROJ: return b_out_proj(c, l, B, 1, st);
      default: return b_head(c, B, 1, c->logits, nullptr, st);
    }
  };
  // operands of the projection / LM head kernels come from the norm kernels
  if (batched) {
    HIP_TRY(b_rows_in(c, 0, B, st));
    HIP_TRY(b_in_proj(c, 0, B, 1, st));
    HIP_TRY(b_scan(c, 0, B, 1, st));
    HIP_TRY(b_rows_out(c, 0, B, st));
  } else {
    HIP_TRY(norm_quant_in(c, 0, B, st));
  }
  for (int i = 0; i < 3; ++i) HIP_TRY(launch(i));
  hipEvent_t e0, e1;
  HIP_TRY(hipEventCreate(&e0));
  HIP_TRY(hipEventCreate(&e1));
  hipError_t e = hipEventRecord(e0, st);
  for (int i = 0; i < iters && e == hipSuccess; ++i) e = launch(i);
  if (e == hipSuccess) e = hipEventRecord(e1, st);
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  float ms = 0.0f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (e != hipSuccess) return fail(DFSSM_E_HIP, std::string("time_kernel: ") + hipGetErrorString(e));
  *avg_us = ms * 1000.0f / (float)iters;
  return DFSSM_OK;
}

dfssm_status dfssm_check_device(dfssm_ctx* c, void* stream) {
  dfssm_status v = check_ctx(c, false);
  if (v != DFSSM_OK) return v;
  HIP_TRY(hipStreamSynchronize(S(stream)));
  int flag = 0;
  HIP_TRY(hipMemcpy(&flag, c->err, sizeof(int), hipMemcpyDeviceToHost));
  if (flag) {
    HIP_TRY(launch_zero(c->err, 4, nullptr));
    if (c->abort_flag) HIP_TRY(launch_zero(c->abort_flag, 4, nullptr));
    if (flag & 2) {
      // an aborted launch leaves the paired boxes with unknown write counts
      HIP_TRY(launch_zero(c->boxes, sizeof(uint64_t) * c->box_words, nullptr));
      c->pair_count = 1;
    }
    HIP_TRY(hipDeviceSynchronize());
    std::string msg;
    if (flag & 1) msg += "a kernel flagged an out-of-range token id; ";
    if (flag & 2) msg += "the persistent decode kernel gave up waiting on another workgroup and aborted; ";
    return fail(DFSSM_E_DEVICE, msg);
  }
  return DFSSM_OK;
}

dfssm_status dfssm_profile_persistent(dfssm_ctx* c, int32_t* d_tok, int32_t n_tokens, uint64_t* d_prof,
                                      int32_t prof_tokens, void* stream) {
  dfssm_status v = check_ctx(c);
  if (v != DFSSM_OK) return v;
  if (!c->persist_ok) return fail(DFSSM_E_UNSUPPORTED, "persistent decode unavailable: " + c->persist_why);
  if (!d_tok || !d_prof || n_tokens < 1 || prof_tokens < 1 || prof_tokens > n_tokens)
    return fail(DFSSM_E_INVALID, "bad profile arguments");
  return run_persistent(c, d_tok, d_tok, nullptr, n_tokens, nullptr, nullptr, S(stream),
                        (unsigned long long*)d_prof, prof_tokens);
}

dfssm_status dfssm_set_path(dfssm_ctx* c, int32_t path) {
  if (!c) return fail(DFSSM_E_INVALID, "null context");
  if (path < DFSSM_PATH_AUTO || path > DFSSM_PATH_GEMM) return fail(DFSSM_E_INVALID, "unknown path");
  if (path == DFSSM_PATH_GEMM && !scan_supported(c->P, c->N))
    return fail(DFSSM_E_UNSUPPORTED, "the batched path is not compiled for this headdim / d_state");
  if (path == DFSSM_PATH_PERSISTENT && !c->persist_ok)
    return fail(DFSSM_E_UNSUPPORTED, "persistent decode unavailable: " + c->persist_why);
  c->path = path;
  return DFSSM_OK;
}

dfssm_status dfssm_k_quant(const float* d_u, int32_t rows, int32_t n, int8_t* d_q, float* d_s, void* stream) {
  if (!d_u || !d_q || !d_s) return fail(DFSSM_E_INVALID, "null pointer");
  if (rows < 1 || n < 1 || n > 65536) return fail(DFSSM_E_INVALID, "rows must be >= 1 and 1 <= n <= 65536");
  HIP_TRY(launch_quant_rows(d_u, rows, n, d_q, d_s, S(stream)));
  return DFSSM_OK;
}

dfssm_status dfssm_k_proj(const uint32_t* d_bits, const float* d_sw, const int8_t* d_A, const float* d_sA,
                          const int8_t* d_B, const float* d_sB, int32_t d_in, int32_t d_out, int32_t r,
                          const int8_t* d_q, const float* d_s, int32_t B, int32_t* d_acc, float* d_y, void* stream) {
  if (!d_bits || !d_sw || !d_A || !d_sA || !d_B || !d_sB || !d_q || !d_s || !d_y)
    return fail(DFSSM_E_INVALID, "null pointer");
  if (d_in < 128 || d_in % 128 || (d_in / 128) > 64 || ((d_in / 128) & (d_in / 128 - 1)))
    return fail(DFSSM_E_UNSUPPORTED, "d_in must be 128 * 2^k <= 8192");
  if (d_out < 1 || r < 1 || r > 32 || B < 1 || B > 65535) return fail(DFSSM_E_INVALID, "bad d_out / r / B");
  hipStream_t st = S(stream);
  const size_t pl_bytes = sizeof(uint32_t) * (size_t)B * (d_in / 32) * 8;
  char* tmp = nullptr;
  const size_t tbytes = align_up(pl_bytes) + align_up(4 * (size_t)B) + align_up(4 * (size_t)B * r);
  HIP_TRY(hipMallocAsync((void**)&tmp, tbytes, st));
  uint32_t* planes = (uint32_t*)tmp;
  int32_t* qsum = (int32_t*)(tmp + align_up(pl_bytes));
  float* t = (float*)(tmp + align_up(pl_bytes) + align_up(4 * (size_t)B));
  hipError_t e = launch_qprep(d_q, d_s, d_in, B, d_A, d_sA, r, planes, qsum, t, st);
  if (e == hipSuccess) {
    ProjArgs a{};
    a.bits = d_bits;
    a.sw = d_sw;
    a.Bm = d_B;
    a.sB = d_sB;
    a.in = QPrep{d_q, planes, qsum, d_s, t};
    a.d_in = d_in;
    a.d_out = d_out;
    a.r = r;
    a.B = B;
    a.acc = d_acc;
    a.y = d_y;
    e = launch_proj(a, EPI_STORE, st);
  }
  hipError_t e2 = hipFreeAsync(tmp, st);
  if (e != hipSuccess) return fail(DFSSM_E_HIP, std::string("k_proj: ") + hipGetErrorString(e));
  if (e2 != hipSuccess) return fail(DFSSM_E_HIP, std::string("k_proj free: ") + hipGetErrorString(e2));
  return DFSSM_OK;
}

dfssm_status dfssm_k_density_encode(const float* d_x, int32_t rows, int32_t n, uint32_t* d_field, float* d_scale,
                                   void* stream) {
  if (!d_x || !d_field || !d_scale) return fail(DFSSM_E_INVALID, "null pointer");
  if (rows < 1) return fail(DFSSM_E_INVALID, "rows must be >= 1");
  if (!density_supported(n)) return fail(DFSSM_E_UNSUPPORTED, "n must be 16, 32, 64 or 128");
  HIP_TRY(launch_density_encode_rows(d_x, rows, n, d_field, d_scale, S(stream)));
  return DFSSM_OK;
}

dfssm_status dfssm_k_density_decode(const uint32_t* d_field, const float* d_scale, int32_t rows, int32_t n, float* d_x,
                                   void* stream) {
  if (!d_x || !d_field || !d_scale) return fail(DFSSM_E_INVALID, "null pointer");
  if (rows < 1) return fail(DFSSM_E_INVALID, "rows must be >= 1");
  if (!density_supported(n)) return fail(DFSSM_E_UNSUPPORTED, "n must be 16, 32, 64 or 128");
  HIP_TRY(launch_density_decode_rows(d_field, d_scale, rows, n, d_x, S(stream)));
  return DFSSM_OK;
}

static dfssm_status density_state(dfssm_ctx* c, int32_t seq0, int32_t nseq, uint32_t* field, float* scale, int mode,
                                  void* stream) {
  dfssm_status v = check_ctx(c, false);
  if (v != DFSSM_OK) return v;
  if (seq0 < 0 || nseq < 1 || seq0 + nseq > c->maxB) return fail(DFSSM_E_INVALID, "sequence slots out of range");
  if (!density_supported(c->N)) return fail(DFSSM_E_UNSUPPORTED, "the density codec needs d_state 16, 32, 64 or 128");
  if (mode != 2 && (!field || !scale)) return fail(DFSSM_E_INVALID, "null field or scale pointer");
  DensityStateArgs a{};
  a.ssm = c->ssm + (size_t)seq0 * c->ssm_bstride;
  a.bstride = c->ssm_bstride;
  a.rows_per_seq = c->L * c->H * c->P;
  a.P = c->P;
  a.total_rows = a.rows_per_seq * nseq;
  a.field = field;
  a.scale = scale;
  HIP_TRY(launch_density_state(a, c->N, mode, S(stream)));
  return DFSSM_OK;
}

dfssm_status dfssm_state_pack(dfssm_ctx* c, int32_t seq0, int32_t nseq, uint32_t* d_field, float* d_scale,
                              void* stream) {
  return density_state(c, seq0, nseq, d_field, d_scale, 0, stream);
}

dfssm_status dfssm_state_unpack(dfssm_ctx* c, int32_t seq0, int32_t nseq, const uint32_t* d_field,
                                const float* d_scale, void* stream) {
  return density_state(c, seq0, nseq, (uint32_t*)d_field, (float*)d_scale, 1, stream);
}

dfssm_status dfssm_state_roundtrip(dfssm_ctx* c, int32_t seq0, int32_t nseq, void* stream) {
  return density_state(c, seq0, nseq, nullptr, nullptr, 2, stream);
}

dfssm_status dfssm_k_gemm(const uint32_t* d_bits, const float* d_sw, const int8_t* d_A, const float* d_sA,
                          const int8_t* d_B, const float* d_sB, int32_t d_in, int32_t d_out, const int8_t* d_q,
                          const float* d_s, int32_t M, int32_t* d_acc, float* d_y, void* stream) {
  dfssm_status v = check_k_gemm(d_bits, d_sw, d_A, d_sA, d_B, d_sB, d_in, d_out, d_q, d_s, M, d_y);
  if (v != DFSSM_OK) return v;
  hipStream_t st = S(stream);
  char* tmp = nullptr;
  HIP_TRY(hipMallocAsync((void**)&tmp, k_gemm_scratch_bytes(d_in, M), st));
  const hipError_t e = k_gemm_run(d_bits, d_sw, d_A, d_sA, d_B, d_sB, d_in, d_out, d_q, d_s, M, d_acc, d_y, tmp, st);
  const hipError_t e2 = hipFreeAsync(tmp, st);
  if (e != hipSuccess) return fail(DFSSM_E_HIP, std::string("k_gemm: ") + hipGetErrorString(e));
  if (e2 != hipSuccess) return fail(DFSSM_E_HIP, std::string("k_gemm free: ") + hipGetErrorString(e2));
  return DFSSM_OK;
}

dfssm_status dfssm_k_gemm_noalloc(const uint32_t* d_bits, const float* d_sw, const int8_t* d_A, const float* d_sA,
                                  const int8_t* d_B, const float* d_sB, int32_t d_in, int32_t d_out,
                                  const int8_t* d_q, const float* d_s, int32_t M, int32_t* d_acc, float* d_y,
                                  void* stream) {
  dfssm_status v = check_k_gemm(d_bits, d_sw, d_A, d_sA, d_B, d_sB, d_in, d_out, d_q, d_s, M, d_y);
  if (v != DFSSM_OK) return v;
  const size_t need = k_gemm_scratch_bytes(d_in, M);
  if (need > kNoAllocScratchBytes)
    return fail(DFSSM_E_INVALID, "k_gemm_noalloc: M * d_in + 68 M = " + std::to_string(need) +
                                     " bytes of operand scratch exceed the static " +
                                     std::to_string(kNoAllocScratchBytes) + "-byte buffer");
  char* tmp = nullptr;
  if ((v = noalloc_scratch(&tmp)) != DFSSM_OK) return v;
  const hipError_t e = k_gemm_run(d_bits, d_sw, d_A, d_sA, d_B, d_sB, d_in, d_out, d_q, d_s, M, d_acc, d_y, tmp,
                                  S(stream));
  if (e != hipSuccess) return fail(DFSSM_E_HIP, std::string("k_gemm_noalloc: ") + hipGetErrorString(e));
  return DFSSM_OK;
}

}  // extern "C"
