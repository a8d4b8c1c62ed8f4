// Internal declarations shared by the library's translation units (not installed).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dfssm {

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------

// SiLU v / (1 + exp(-v)) as v times the hardware reciprocal (1 ulp) of
// 1 + exp(-v): an IEEE division expands to about ten instructions, a quarter
// of the vector instructions of a chunk of the matrix-core scan.  Both limits
// hold: exp(-v) = inf gives v * 0, exp(-v) = 0 gives v.
__device__ __forceinline__ float silu_f(float v) { return v * __builtin_amdgcn_rcpf(1.0f + __expf(-v)); }

// log(1 + x) for x >= 0 from the natural log of u = fl(1 + x): log(u) * x / (u - 1)
// corrects the rounding of 1 + x (D. Goldberg, "What every computer scientist
// should know about floating-point arithmetic", 1991, Theorem 4).
__device__ __forceinline__ float log1p_pos(float x) {
  const float u = 1.0f + x;
  return u == 1.0f ? x : __logf(u) * __fdividef(x, u - 1.0f);
}

// softplus with the usual linear branch above 20 (log1p(e^a) - a < 2.1e-9 there)
__device__ __forceinline__ float softplus_f(float a) { return a > 20.0f ? a : log1p_pos(__expf(a)); }

// ---------------------------------------------------------------------------
// cross-lane reductions on DPP (data movement inside the VALU; no LDS round
// trip).  Lanes form rows of 16.  quad_perm swaps within 4 lanes, the row
// half-mirror pairs the two quads of each half row, the row mirror pairs the
// two halves of a row, and row_bcast:15 / :31 carry a row's last lane into
// the next row(s).  All lanes must be active.
// ---------------------------------------------------------------------------
enum : int {
  kDppQuadSwap1 = 0xB1,  // quad_perm [1,0,3,2]
  kDppQuadSwap2 = 0x4E,  // quad_perm [2,3,0,1]
  kDppRowHalfMirror = 0x141,
  kDppRowMirror = 0x140,
  kDppRowBcast15 = 0x142,
  kDppRowBcast31 = 0x143
};

template <int CTRL, int ROWMASK = 0xF>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWMASK, 0xF, false);
}
template <int CTRL, int ROWMASK = 0xF>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWMASK, 0xF, false));
}

// Sum over aligned groups of U lanes (U a power of two, 1..64).  For U <= 16
// every lane of a group ends with the group sum; for U = 32 the sum is valid
// in lanes 16..31 and 48..63 (rows 1 and 3); for U = 64 in lanes 48..63.
__device__ __forceinline__ int group_sum_i(int v, int U) {
  if (U >= 2) v += dpp_i<kDppQuadSwap1>(v);
  if (U >= 4) v += dpp_i<kDppQuadSwap2>(v);
  if (U >= 8) v += dpp_i<kDppRowHalfMirror>(v);
  if (U >= 16) v += dpp_i<kDppRowMirror>(v);
  if (U >= 32) v += dpp_i<kDppRowBcast15, 0xA>(v);
  if (U >= 64) v += dpp_i<kDppRowBcast31, 0x8>(v);
  return v;
}
// lane holding the sum of the group that starts at lane g0 (see group_sum_i)
__device__ __forceinline__ int group_sum_lane(int g0, int U) {
  return U <= 16 ? g0 : (U == 32 ? g0 + 16 : 48);
}

// sum over each row of 16 lanes, in every lane of the row
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_f<kDppQuadSwap1>(v);
  v += dpp_f<kDppQuadSwap2>(v);
  v += dpp_f<kDppRowHalfMirror>(v);
  v += dpp_f<kDppRowMirror>(v);
  return v;
}

// row (16-lane) all-reduce, then the four rows combined through readlane:
// the result is uniform across the wave.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<kDppQuadSwap1>(v);
  v += dpp_f<kDppQuadSwap2>(v);
  v += dpp_f<kDppRowHalfMirror>(v);
  v += dpp_f<kDppRowMirror>(v);
  const int b = __float_as_int(v);
  return (__int_as_float(__builtin_amdgcn_readlane(b, 0)) + __int_as_float(__builtin_amdgcn_readlane(b, 16))) +
         (__int_as_float(__builtin_amdgcn_readlane(b, 32)) + __int_as_float(__builtin_amdgcn_readlane(b, 48)));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<kDppQuadSwap1>(v));
  v = fmaxf(v, dpp_f<kDppQuadSwap2>(v));
  v = fmaxf(v, dpp_f<kDppRowHalfMirror>(v));
  v = fmaxf(v, dpp_f<kDppRowMirror>(v));
  const int b = __float_as_int(v);
  return fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 0)), __int_as_float(__builtin_amdgcn_readlane(b, 16))),
               fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 32)), __int_as_float(__builtin_amdgcn_readlane(b, 48))));
}
__device__ __forceinline__ int wave_sum_i(int v) {
  v = group_sum_i(v, 16);
  return (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
         (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
}

// The projection output float(sacc) * sw * s + sB * lo and the causal conv
// sum, each rounded in one fixed order (two products, then a fused
// multiply-add; a chain of fused multiply-adds) whatever the compiler would
// contract: every kernel that produces them gives a row the same value.
__device__ __forceinline__ float proj_out(int sacc, float sw, float s, float sb, float lo) {
#pragma clang fp contract(off)
  return __builtin_fmaf(sb, lo, ((float)sacc * sw) * s);
}
__device__ __forceinline__ float conv4(float bias, float w0, float x0, float w1, float x1, float w2, float x2,
                                       float w3, float x3) {
  return __builtin_fmaf(w3, x3, __builtin_fmaf(w2, x2, __builtin_fmaf(w1, x1, __builtin_fmaf(w0, x0, bias))));
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
  int32_t* acc;          // [B][d_out] signed scaffold sums (any epilogue), or null
  // EPI_STORE
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
// batched path (gemm.hip)
// ---------------------------------------------------------------------------

// rows x [M][ldx] (fp32) -> codes q [M][K], scale s [M], code sum qsum [M]
// (may be null) and, when A is non-null, the LoRA-down vectors t [M][16].
struct RowsArgs {
  const float* x;
  int ldx;
  const float* w;   // norm weight [K]
  int M;
  float eps;
  const int8_t* A;  // [16][K] or null
  const float* sA;  // [16]
  int8_t* q;
  float* s;
  int32_t* qsum;
  float* t;
};

enum GemmEpilogue : int { GEMM_EPI_STORE = 0, GEMM_EPI_RESIDUAL = 1 };

// y[m][n] (=, or += for the residual) float(sum_k q[m][k] sign(n, k)) * sw[n] * s[m]
//                                      + sB[n] * sum_j B[n][j] t[m][j]
struct GemmArgs {
  const int8_t* q;      // [M][K]
  const float* s;       // [M]
  const int32_t* qsum;  // [M]
  const float* t;       // [M][16]
  const uint32_t* bits; // [N][K/32]
  const float* sw;      // [N]
  const int8_t* Bm;     // [N][16]
  const float* sB;      // [N]
  int M, N, K;
  float* y;             // [M][ldy]
  int ldy;
  int32_t* acc;         // [M][N] signed scaffold sums, or null
  // one decode token per sequence (row m = sequence m): the conv shift
  // register of columns [x_off, x_off + cdim) in the epilogue, or xc null
  float* xc;            // [M][cdim]
  float* conv_state;    // sequence 0's window [3][cdim]; sequence m at + m * conv_bstride
  size_t conv_bstride;
  const float* conv_w;  // [cdim][4]
  const float* conv_b;
  int x_off, cdim;
};

// M <= 32 rows against N weight rows, one 32 x 32 block per workgroup
enum SkinnyKind : int {
  SK_IN = 0,   // scaffold + LoRA -> y (stored); with xc set, columns [x_off, x_off + cdim) also go
               // through the conv shift register of one decode token (state updated, SiLU output to xc)
  SK_OUT = 1,  // scaffold + LoRA, residual: y += ...
  SK_HEAD = 2  // int8 weight rows (the tied LM head): y = float(sum w q) * sw[n] * s[m]
};
struct SkinnyArgs {
  const int8_t* q;      // [M][K]
  const float* s;       // [M]
  const int32_t* qsum;  // [M] (scaffold kinds)
  const float* t;       // [M][16] (scaffold kinds)
  const void* w;        // scaffold bits uint32 [N][K/32], or int8 [N][K] for SK_HEAD
  const float* sw;      // [N] row scale
  const int8_t* Bm;     // [N][16] LoRA up (scaffold kinds)
  const float* sB;      // [N]
  int M, N, K;
  float* y;
  int ldy;
  int32_t* acc;         // [M][N] signed scaffold sums, or null
  float* xc;            // [M][cdim] or null
  float* conv_state;    // sequence 0's window [3][cdim]; sequence m at + m * conv_bstride
  size_t conv_bstride;
  const float* conv_w;  // [cdim][4]
  const float* conv_b;
  int x_off, cdim;
};

// causal depthwise conv over T tokens of B sequences (rows b * T + t)
struct ConvSeqArgs {
  const float* zx;  // in_proj output rows [B*T][ldzx]; conv inputs at columns x_off + c
  int ldzx, x_off;
  float* xc;        // [B*T][cdim]
  float* state;     // sequence 0's window [3][cdim] (oldest first); sequence b at + b * state_bstride
  size_t state_bstride;
  const float* w;   // [cdim][4]
  const float* bias;
  int B, T, cdim;
};

struct ScanArgs {
  const float* xc;  // [B*T][cdim]: x at [0, d_inner), B at d_inner, C at d_inner + N
  const float* zx;  // [B*T][ldzx]: z at [0, d_inner), dt_raw at dt_off
  int ldzx, dt_off;
  const float* A_log;
  const float* dt_bias;
  const float* D;
  float* ssm;       // this layer, sequence 0: [H][P/16][N][16]; sequence b at + b * ssm_bstride
  size_t ssm_bstride;
  float* g;         // [B*T][d_inner]
  int B, T, H, d_inner, cdim;
  float* gram;      // chunked scan workspace: B * ceil(T / kSsdL) records of ssd_record_floats(H), or null
  // The chunked scan takes the conv inputs (the in_proj output x, B, C at
  // zx columns x_off + c) and applies the causal conv itself, with the stored
  // window as the history before t = 0; xc is then not read.
  int x_off;
  const float* conv_w;      // [cdim][4]
  const float* conv_b;      // [cdim]
  const float* conv_state;  // sequence 0's window [3][cdim] (oldest first); sequence b at + b * conv_bstride
  size_t conv_bstride;
};

// The chunked scan (headdim 64, d_state 128) works on chunks of kSsdL tokens;
// its workspace record per chunk is G [kSsdL][kSsdL], per head the chunk
// parameters A_j, dt_j, w_j, exp(A_j) [H][4][kSsdL], then the chunk's conv
// outputs B [kSsdL][128] and C [kSsdL][128].
constexpr int kSsdL = 64;
__host__ __device__ constexpr size_t ssd_record_floats(int H) {
  return (size_t)kSsdL * kSsdL + (size_t)H * 4 * kSsdL + 2 * (size_t)kSsdL * 128;
}

hipError_t launch_rows_quant(const RowsArgs& a, int K, hipStream_t st);
hipError_t launch_bitgemm(const GemmArgs& a, int epi, hipStream_t st);
hipError_t launch_gemm_skinny(const SkinnyArgs& a, int kind, hipStream_t st);
hipError_t launch_conv_seq(const ConvSeqArgs& a, hipStream_t st);  // conv, then the window update
hipError_t launch_conv_state_update(const ConvSeqArgs& a, hipStream_t st);
bool scan_takes_conv_inputs(int P, int N);  // the scan applies the conv itself (then run the window update after it)
hipError_t launch_scan(const ScanArgs& a, int P, int N, hipStream_t st);
bool scan_supported(int P, int N);
hipError_t launch_embed_rows(const int32_t* tok, int tok_stride, int t0, int B, int T, const int8_t* E,
                             const float* sE, int dm, int V, float* h, int* err, hipStream_t st);

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

// density-field state codec (codec.hip)
struct DensityStateArgs {
  float* ssm;         // sequence s0's state, layout [L][H][P/16][N][16]
  size_t bstride;     // floats between sequences
  int rows_per_seq;   // L * H * P
  int P;
  int total_rows;     // rows_per_seq * sequences
  uint32_t* field;    // [total_rows][N / 8] (modes 0, 1)
  float* scale;       // [total_rows]
};
bool density_supported(int n);
hipError_t launch_density_encode_rows(const float* x, int rows, int n, uint32_t* field, float* scale,
                                      hipStream_t st);
hipError_t launch_density_decode_rows(const uint32_t* field, const float* scale, int rows, int n, float* x,
                                      hipStream_t st);
// mode 0 pack, 1 unpack, 2 round trip in place
hipError_t launch_density_state(const DensityStateArgs& a, int n, int mode, hipStream_t st);
hipError_t launch_f16_to_f32(const void* src, float* dst, size_t n, hipStream_t st);

}  // namespace dfssm
