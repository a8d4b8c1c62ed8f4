/*
 * dfssm_oracle.c -- plain CPU oracle of the DF-SSM decode step.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU library never
 * links, calls or includes it, and it shares no source with the GPU path.
 *
 * What it computes.  The pages ("Density Field State Space Models: 1-Bit
 * Distillation, Efficient Inference, and Knowledge Organization in Mamba-2",
 * gist.science technical summary and arxivdaily abstract) describe a Mamba-2
 * 1.3B stack whose in_proj/out_proj weights are a frozen 1-bit sign scaffold
 * with an int8 rank-16 LoRA correction, int8 per-row-scaled LoRA and
 * embedding / LM head, a stateful conv shift register and the SSM recurrence
 * (gist.science summary §2.B, §2.C; arxivdaily English abstract).  The pages
 * do not print the Mamba-2 block; it is taken from its published definition
 * (Dao & Gu 2024, "Transformers are SSMs", Mamba-2 block), and every step the
 * pages leave open is read as stated next to the code below.
 *
 * Precision.  Every floating-point quantity is carried in fp64.  The one place
 * where a float decides an integer -- the int8 activation quantiser -- takes
 * its decision in fp32 (the value is rounded once to fp32 first), the
 * precision of the GPU kernels, so that both sides quantise identical fp32
 * inputs identically.  Integer dot products are exact (int64).
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fno-fast-math (no contraction,
 * IEEE semantics).  OpenMP only splits independent output rows / heads.
 *
 * Parity pins: every function here is checked by the CPU test suite against
 * closed forms, special cases and library routines (one-hot and all-sign
 * scaffold probes, numpy integer matmuls of the unpacked matrix, quantiser
 * rounding cases, conv impulse response, SSM dt = 0 / memoryless / C = 0
 * cases and the unrolled (quadratic) form of the recurrence, head/channel
 * permutation invariance of a layer, zero-path cases of the layer, and the
 * pages' storage figures).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_EPS 1e-5 /* RMSNorm epsilon: pages silent; Mamba-2 default */

/* shape vector, same order as synth.Shape.as_ints() */
enum { SH_NL = 0, SH_DM, SH_DI, SH_DS, SH_HD, SH_V, SH_K, SH_R, SH_N };

/* per-layer tensor order */
enum {
  T_IN_BITS = 0, T_IN_SW, T_IN_A, T_IN_SA, T_IN_B, T_IN_SB,
  T_OUT_BITS, T_OUT_SW, T_OUT_A, T_OUT_SA, T_OUT_B, T_OUT_SB,
  T_CONV_W, T_CONV_B, T_A_LOG, T_DT_BIAS, T_D, T_NORM_W, T_GNORM_W, T_PER_LAYER
};
/* A layer's pointer array: the T_PER_LAYER tensors above, then two optional
 * (nullable) pre-unpacked sign matrices of the scaffolds (or_unpack_signs),
 * int8 [d_in_proj][d_model] and [d_model][d_inner].  When present, the
 * scaffold sums read the signs from them instead of from the bits; the sums
 * are the same integers either way.                                         */
enum { T_IN_SIGNS = T_PER_LAYER, T_OUT_SIGNS, LW_STRIDE };
/* global tensors follow the n_layer * LW_STRIDE layer pointers */
enum { G_E = 0, G_SE, G_FNORM };

static double silu(double v) { return v / (1.0 + exp(-v)); }

/* softplus(a) = log(1 + e^a), evaluated without overflow. */
static double softplus(double a) { return a > 0.0 ? a + log1p(exp(-a)) : log1p(exp(a)); }

/* ------------------------------------------------------------------------ */
/* Activation quantiser (pages: int8 operands on both sides of the scaffold
 * matmul, gist.science summary §2.C; granularity unstated -> per token,
 * symmetric absmax, [-127, 127], round half to even).  Decision in fp32.     */
void or_quant_f32(const float* u, int n, int8_t* q, float* s_out) {
  float amax = 0.0f;
  for (int i = 0; i < n; ++i) {
    float a = fabsf(u[i]);
    if (a > amax) amax = a;
  }
  if (!(amax > 0.0f)) {
    for (int i = 0; i < n; ++i) q[i] = 0;
    *s_out = 0.0f;
    return;
  }
  float inv = 127.0f / amax;
  for (int i = 0; i < n; ++i) {
    float r = rintf(u[i] * inv);
    if (r > 127.0f) r = 127.0f;
    if (r < -127.0f) r = -127.0f;
    q[i] = (int8_t)r;
  }
  *s_out = amax / 127.0f;
}

void or_quant(const double* u, int n, int8_t* q, float* s_out) {
  float* uf = (float*)malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
  for (int i = 0; i < n; ++i) uf[i] = (float)u[i];
  or_quant_f32(uf, n, q, s_out);
  free(uf);
}

/* Several roundings are correct near a tie.  An implementation that computes
 * u in fp32 may land on the other side of a rounding tie than this oracle
 * when u * 127/amax lies within its own rounding error of k + 1/2.  Such a
 * code is accepted here: `force` (nullable) proposes codes; a proposed code
 * is taken only if it equals the oracle's own code, or differs from it by
 * one with the oracle's scaled value within `delta` of the tie between the
 * two.  Returns the number of proposed codes that were rejected (then q holds
 * the oracle's own codes).  *flipped (nullable) receives the number of
 * proposed codes that were taken although they differ from the oracle's own
 * (0 when any proposal was rejected).                                        */
int or_quant_forced(const double* u, int n, const int8_t* force, double delta, int8_t* q, float* s_out,
                    int* flipped) {
  float* uf = (float*)malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
  for (int i = 0; i < n; ++i) uf[i] = (float)u[i];
  or_quant_f32(uf, n, q, s_out);
  int bad = 0, flips = 0;
  if (force && *s_out > 0.0f) {
    float amax = 0.0f;
    for (int i = 0; i < n; ++i) if (fabsf(uf[i]) > amax) amax = fabsf(uf[i]);
    const float inv = 127.0f / amax;
    for (int i = 0; i < n; ++i) {
      if (force[i] == q[i]) continue;
      const int d = (int)force[i] - (int)q[i];
      const double x = (double)(uf[i] * inv);
      const double tie = (double)q[i] + 0.5 * d;
      if ((d == 1 || d == -1) && fabs(x - tie) <= delta) {
        q[i] = force[i];
        ++flips;
      } else {
        ++bad;
      }
    }
    if (bad) {
      or_quant_f32(uf, n, q, s_out);
      flips = 0;
    }
  } else if (force) {
    for (int i = 0; i < n; ++i) bad += force[i] != 0;
  }
  free(uf);
  if (flipped) *flipped = flips;
  return bad;
}

/* ------------------------------------------------------------------------ */
/* RMSNorm: u = x / sqrt(mean(x^2) + eps) * w. */
void or_rmsnorm(const double* x, const float* w, int n, double* u) {
  double ss = 0.0;
  for (int i = 0; i < n; ++i) ss += x[i] * x[i];
  double r = 1.0 / sqrt(ss / (double)n + OR_EPS);
  for (int i = 0; i < n; ++i) u[i] = x[i] * r * (double)w[i];
}

/* ------------------------------------------------------------------------ */
/* 1-bit scaffold dot products (gist.science summary §2.B: scaffold frozen at
 * its rounded values; §2.C and the arxivdaily abstract: 1-bit packed weights
 * used as int8).  Weight (o, i) is +1 if bit (i mod 32) of word
 * bits[o * (d_in/32) + i/32] is set, -1 otherwise.  acc[o] = sum_i w(o,i) q_i. */
int or_scaffold_acc(const uint32_t* bits, int d_out, int d_in, const int8_t* q, int32_t* acc) {
  const int words = d_in / 32;
  int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
  for (int o = 0; o < d_out; ++o) {
    int64_t a = 0;
    const uint32_t* row = bits + (size_t)o * words;
    for (int i = 0; i < d_in; ++i) {
      int sign = ((row[i >> 5] >> (i & 31)) & 1u) ? 1 : -1;
      a += (int64_t)sign * q[i];
    }
    if (a > INT32_MAX || a < INT32_MIN) bad = 1;
    acc[o] = (int32_t)a;
  }
  return bad ? -1 : 0;
}

/* The scaffold as a dense sign matrix: signs[o][i] = +1 where bit (i mod 32)
 * of word bits[o][i/32] is set, -1 otherwise (the layout read above). */
void or_unpack_signs(const uint32_t* bits, int d_out, int d_in, int8_t* signs) {
  const int words = d_in / 32;
#pragma omp parallel for schedule(static)
  for (int o = 0; o < d_out; ++o)
    for (int i = 0; i < d_in; ++i)
      signs[(size_t)o * d_in + i] = ((bits[(size_t)o * words + (i >> 5)] >> (i & 31)) & 1u) ? 1 : -1;
}

/* acc[o] = sum_i signs[o][i] q_i, the same integer as or_scaffold_acc on the
 * bits the signs came from.  Row sums fit int32 for d_in <= 131072
 * (131072 * 127 < 2^31), which is checked.                                   */
int or_sign_acc(const int8_t* signs, int d_out, int d_in, const int8_t* q, int32_t* acc) {
  if (d_in > 131072) return -1;
#pragma omp parallel for schedule(static)
  for (int o = 0; o < d_out; ++o) {
    const int8_t* row = signs + (size_t)o * d_in;
    int32_t a = 0;
    for (int i = 0; i < d_in; ++i) a += (int32_t)row[i] * (int32_t)q[i];
    acc[o] = a;
  }
  return 0;
}

/* int8 matrix-vector product: out[r] = sum_c M[r][c] v[c] (exact). */
static void int8_matvec(const int8_t* M, int rows, int cols, const int8_t* v, int64_t* out) {
#pragma omp parallel for schedule(static) if (rows >= 4096)
  for (int r = 0; r < rows; ++r) {
    int64_t a = 0;
    const int8_t* m = M + (size_t)r * cols;
    for (int c = 0; c < cols; ++c) a += (int64_t)m[c] * v[c];
    out[r] = a;
  }
}

/* Projection = scaffold + LoRA (gist.science summary §2.B: rank-16 int8 LoRA
 * on in_proj and out_proj of every layer; int8 with per-row scales).
 *   ys[o] = acc[o] * sw[o] * s
 *   t[k]  = (sum_i A[k][i] q_i) * sA[k] * s          (A: r x d_in)
 *   yl[o] = sB[o] * sum_k B[o][k] t[k]                 (B: d_out x r)
 *   y[o]  = ys[o] + yl[o]
 * acc_out / ta_out (nullable) receive the exact integer sums.              */
int or_proj_signs(const uint32_t* bits, const int8_t* signs, const float* sw, const int8_t* A, const float* sA,
                  const int8_t* B, const float* sB, int d_in, int d_out, int r,
                  const int8_t* q, float s, double* y, int32_t* acc_out, int64_t* ta_out);
int or_proj(const uint32_t* bits, const float* sw, const int8_t* A, const float* sA,
            const int8_t* B, const float* sB, int d_in, int d_out, int r,
            const int8_t* q, float s, double* y, int32_t* acc_out, int64_t* ta_out) {
  return or_proj_signs(bits, NULL, sw, A, sA, B, sB, d_in, d_out, r, q, s, y, acc_out, ta_out);
}

/* or_proj with the scaffold optionally given as its unpacked sign matrix
 * (signs nullable; the bits are used when it is NULL).                      */
int or_proj_signs(const uint32_t* bits, const int8_t* signs, const float* sw, const int8_t* A, const float* sA,
                  const int8_t* B, const float* sB, int d_in, int d_out, int r,
                  const int8_t* q, float s, double* y, int32_t* acc_out, int64_t* ta_out) {
  int32_t* acc = (int32_t*)malloc(sizeof(int32_t) * (size_t)d_out);
  int64_t* ta = (int64_t*)malloc(sizeof(int64_t) * (size_t)r);
  double* t = (double*)malloc(sizeof(double) * (size_t)r);
  int rc = signs ? or_sign_acc(signs, d_out, d_in, q, acc) : or_scaffold_acc(bits, d_out, d_in, q, acc);
  int8_matvec(A, r, d_in, q, ta);
  for (int k = 0; k < r; ++k) t[k] = (double)ta[k] * (double)sA[k] * (double)s;
#pragma omp parallel for schedule(static) if (d_out >= 4096)
  for (int o = 0; o < d_out; ++o) {
    double ys = (double)acc[o] * (double)sw[o] * (double)s;
    double l = 0.0;
    for (int k = 0; k < r; ++k) l += (double)B[(size_t)o * r + k] * t[k];
    y[o] = ys + (double)sB[o] * l;
  }
  if (acc_out) memcpy(acc_out, acc, sizeof(int32_t) * (size_t)d_out);
  if (ta_out) memcpy(ta_out, ta, sizeof(int64_t) * (size_t)r);
  free(acc); free(ta); free(t);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Conv shift register (gist.science summary §2.C: stateful shift-register
 * kernel; Mamba-2 definition: depthwise causal conv of width K over the
 * x, B, C channels, bias, then SiLU).  state[c] holds the previous K-1 inputs,
 * oldest first; tap K-1 multiplies the newest input.                         */
void or_conv_step(const double* xin, const float* w, const float* b, int C, int K,
                  double* state, double* out) {
  for (int c = 0; c < C; ++c) {
    double* st = state + (size_t)c * (K - 1);
    double v = (double)b[c];
    for (int k = 0; k < K - 1; ++k) v += (double)w[(size_t)c * K + k] * st[k];
    v += (double)w[(size_t)c * K + (K - 1)] * xin[c];
    out[c] = silu(v);
    for (int k = 0; k < K - 2; ++k) st[k] = st[k + 1];
    if (K >= 2) st[K - 2] = xin[c];
  }
}

/* ------------------------------------------------------------------------ */
/* SSM recurrence, one token (gist.science summary §2.C: SSM recurrence kernel;
 * fixed-size state, §1; Mamba-2 definition with ngroups = 1):
 *   dt_h = softplus(dt_raw_h + dt_bias_h)
 *   dA_h = exp(-dt_h * exp(A_log_h))
 *   S[h][p][n] <- dA_h * S[h][p][n] + dt_h * x[h][p] * B[n]
 *   y[h][p]    =  sum_n S[h][p][n] * C[n] + D_h * x[h][p]                     */
void or_ssm_step(const double* x, const double* Bv, const double* Cv, const double* dt_raw,
                 const float* A_log, const float* dt_bias, const float* D,
                 int H, int P, int N, double* S, double* y, double* dt_out) {
#pragma omp parallel for schedule(static) if (H * P * N >= 65536)
  for (int h = 0; h < H; ++h) {
    double dt = softplus(dt_raw[h] + (double)dt_bias[h]);
    double dA = exp(-dt * exp((double)A_log[h]));
    if (dt_out) dt_out[h] = dt;
    for (int p = 0; p < P; ++p) {
      double xv = x[(size_t)h * P + p];
      double* s = S + ((size_t)h * P + p) * N;
      double acc = 0.0;
      for (int n = 0; n < N; ++n) {
        s[n] = s[n] * dA + dt * xv * Bv[n];
        acc += s[n] * Cv[n];
      }
      y[(size_t)h * P + p] = acc + (double)D[h] * xv;
    }
  }
}

/* Gated RMSNorm (Mamba-2 definition, norm after gate): u = RMSNorm(y * silu(z)) * w. */
void or_gated_rmsnorm(const double* y, const double* z, const float* w, int n, double* u) {
  double* g = (double*)malloc(sizeof(double) * (size_t)n);
  for (int i = 0; i < n; ++i) g[i] = y[i] * silu(z[i]);
  or_rmsnorm(g, w, n, u);
  free(g);
}

/* ------------------------------------------------------------------------ */
/* One layer, one token: h_out = h_in + out_proj(gated_norm(SSM(conv(in_proj(
 * quant(RMSNorm(h_in))))))).  in_proj output order (Mamba-2): z | x | B | C | dt.
 * dbg (nullable, fp64): zxbcdt[d_in_proj] | xc[conv_dim] | dt[H] | y[d_inner]
 *   | u2[d_inner] | out[d_model].
 * q1/s1, q2/s2 (nullable): the int8 activations and scales fed to in_proj and
 * out_proj.                                                                   */
int or_layer_step_forced(const int* sh, const void* const* lw, const double* h_in,
                         double* conv_state, double* ssm_state, double* h_out, double* dbg,
                         int8_t* q1_out, float* s1_out, int8_t* q2_out, float* s2_out,
                         const int8_t* q1_force, const int8_t* q2_force, double delta, int* rejected,
                         int* flipped) {
  const int dm = sh[SH_DM], di = sh[SH_DI], ds = sh[SH_DS], hd = sh[SH_HD], K = sh[SH_K], r = sh[SH_R];
  const int H = di / hd, cdim = di + 2 * ds, dproj = 2 * di + 2 * ds + H;
  double* u = (double*)malloc(sizeof(double) * (size_t)dm);
  int8_t* q1 = (int8_t*)malloc((size_t)dm);
  double* zx = (double*)malloc(sizeof(double) * (size_t)dproj);
  double* xc = (double*)malloc(sizeof(double) * (size_t)cdim);
  double* y = (double*)malloc(sizeof(double) * (size_t)di);
  double* u2 = (double*)malloc(sizeof(double) * (size_t)di);
  int8_t* q2 = (int8_t*)malloc((size_t)di);
  double* out = (double*)malloc(sizeof(double) * (size_t)dm);
  double* dt = (double*)malloc(sizeof(double) * (size_t)H);
  float s1, s2;
  int rc = 0;

  int rej = 0, fl1 = 0, fl2 = 0;
  or_rmsnorm(h_in, (const float*)lw[T_NORM_W], dm, u);
  rej += or_quant_forced(u, dm, q1_force, delta, q1, &s1, &fl1);
  rc |= or_proj_signs((const uint32_t*)lw[T_IN_BITS], (const int8_t*)lw[T_IN_SIGNS], (const float*)lw[T_IN_SW],
                (const int8_t*)lw[T_IN_A],
                (const float*)lw[T_IN_SA], (const int8_t*)lw[T_IN_B], (const float*)lw[T_IN_SB],
                dm, dproj, r, q1, s1, zx, NULL, NULL);
  const double* z = zx;
  const double* xBC = zx + di;
  const double* dt_raw = zx + di + cdim;
  or_conv_step(xBC, (const float*)lw[T_CONV_W], (const float*)lw[T_CONV_B], cdim, K, conv_state, xc);
  or_ssm_step(xc, xc + di, xc + di + ds, dt_raw, (const float*)lw[T_A_LOG], (const float*)lw[T_DT_BIAS],
              (const float*)lw[T_D], H, hd, ds, ssm_state, y, dt);
  or_gated_rmsnorm(y, z, (const float*)lw[T_GNORM_W], di, u2);
  rej += or_quant_forced(u2, di, q2_force, delta, q2, &s2, &fl2);
  if (rejected) *rejected = rej;
  if (flipped) *flipped = fl1 + fl2;
  rc |= or_proj_signs((const uint32_t*)lw[T_OUT_BITS], (const int8_t*)lw[T_OUT_SIGNS], (const float*)lw[T_OUT_SW],
                (const int8_t*)lw[T_OUT_A],
                (const float*)lw[T_OUT_SA], (const int8_t*)lw[T_OUT_B], (const float*)lw[T_OUT_SB],
                di, dm, r, q2, s2, out, NULL, NULL);
  for (int i = 0; i < dm; ++i) h_out[i] = h_in[i] + out[i];

  if (dbg) {
    double* d = dbg;
    memcpy(d, zx, sizeof(double) * (size_t)dproj); d += dproj;
    memcpy(d, xc, sizeof(double) * (size_t)cdim); d += cdim;
    memcpy(d, dt, sizeof(double) * (size_t)H); d += H;
    memcpy(d, y, sizeof(double) * (size_t)di); d += di;
    memcpy(d, u2, sizeof(double) * (size_t)di); d += di;
    memcpy(d, out, sizeof(double) * (size_t)dm);
  }
  if (q1_out) memcpy(q1_out, q1, (size_t)dm);
  if (s1_out) *s1_out = s1;
  if (q2_out) memcpy(q2_out, q2, (size_t)di);
  if (s2_out) *s2_out = s2;
  free(u); free(q1); free(zx); free(xc); free(y); free(u2); free(q2); free(out); free(dt);
  return rc;
}

int or_layer_step(const int* sh, const void* const* lw, const double* h_in,
                  double* conv_state, double* ssm_state, double* h_out, double* dbg,
                  int8_t* q1_out, float* s1_out, int8_t* q2_out, float* s2_out) {
  return or_layer_step_forced(sh, lw, h_in, conv_state, ssm_state, h_out, dbg, q1_out, s1_out, q2_out, s2_out,
                              NULL, NULL, 0.0, NULL, NULL);
}

/* ------------------------------------------------------------------------ */
/* Tied int8 LM head (gist.science summary §2.B: embedding / LM head int8 with
 * per-row scales; §3 size composition: one int8 copy):
 *   logits[v] = (sum_i E[v][i] qf_i) * sE[v] * sf.  Returns argmax, lowest
 *   index on ties.                                                          */
int or_lm_head_forced(const int* sh, const int8_t* E, const float* sE, const float* fnorm,
                      const double* h, double* logits, int8_t* qf_out, float* sf_out,
                      const int8_t* qf_force, double delta, int* rejected, int* flipped) {
  const int dm = sh[SH_DM], V = sh[SH_V];
  double* u = (double*)malloc(sizeof(double) * (size_t)dm);
  int8_t* qf = (int8_t*)malloc((size_t)dm);
  int64_t* acc = (int64_t*)malloc(sizeof(int64_t) * (size_t)V);
  float sf;
  or_rmsnorm(h, fnorm, dm, u);
  int rej = or_quant_forced(u, dm, qf_force, delta, qf, &sf, flipped);
  if (rejected) *rejected = rej;
  int8_matvec(E, V, dm, qf, acc);
  int best = 0;
  for (int v = 0; v < V; ++v) {
    logits[v] = (double)acc[v] * (double)sE[v] * (double)sf;
    if (logits[v] > logits[best]) best = v;
  }
  if (qf_out) memcpy(qf_out, qf, (size_t)dm);
  if (sf_out) *sf_out = sf;
  free(u); free(qf); free(acc);
  return best;
}

int or_lm_head(const int* sh, const int8_t* E, const float* sE, const float* fnorm,
               const double* h, double* logits, int8_t* qf_out, float* sf_out) {
  return or_lm_head_forced(sh, E, sE, fnorm, h, logits, qf_out, sf_out, NULL, 0.0, NULL, NULL);
}

/* Embedding lookup with the tied table: h[i] = E[tok][i] * sE[tok]. */
void or_embed(const int* sh, const int8_t* E, const float* sE, int tok, double* h) {
  const int dm = sh[SH_DM];
  for (int i = 0; i < dm; ++i) h[i] = (double)E[(size_t)tok * dm + i] * (double)sE[tok];
}

/* One decode step of one sequence through the whole stack.
 * w: n_layer * LW_STRIDE layer pointers (19 tensors, 2 optional sign
 * matrices), then E, sE, final_norm.
 * conv: [n_layer][conv_dim][K-1], ssm: [n_layer][H][P][N] (fp64, updated).
 * logits (nullable): [V]; h_trace (nullable): [(n_layer + 1)][d_model], the
 * residual stream entering each layer and after the last one.
 * Returns the greedy next token (argmax, lowest index on ties), or -1 when
 * logits is NULL, or -2 on an out-of-range token / integer overflow.        */
int or_decode_step(const int* sh, const void* const* w, double* conv, double* ssm, int tok,
                   double* logits, double* h_trace) {
  const int nl = sh[SH_NL], dm = sh[SH_DM], di = sh[SH_DI], ds = sh[SH_DS], hd = sh[SH_HD];
  const int K = sh[SH_K], V = sh[SH_V];
  const int H = di / hd, cdim = di + 2 * ds;
  if (tok < 0 || tok >= V) return -2;
  const void* const* g = w + (size_t)nl * LW_STRIDE;
  double* h = (double*)malloc(sizeof(double) * (size_t)dm);
  double* h2 = (double*)malloc(sizeof(double) * (size_t)dm);
  int rc = 0;
  or_embed(sh, (const int8_t*)g[G_E], (const float*)g[G_SE], tok, h);
  for (int l = 0; l < nl; ++l) {
    if (h_trace) memcpy(h_trace + (size_t)l * dm, h, sizeof(double) * (size_t)dm);
    rc |= or_layer_step(sh, w + (size_t)l * LW_STRIDE, h,
                        conv + (size_t)l * cdim * (K - 1), ssm + (size_t)l * H * hd * ds,
                        h2, NULL, NULL, NULL, NULL, NULL);
    double* t = h; h = h2; h2 = t;
  }
  if (h_trace) memcpy(h_trace + (size_t)nl * dm, h, sizeof(double) * (size_t)dm);
  int next = -1;
  if (logits)
    next = or_lm_head(sh, (const int8_t*)g[G_E], (const float*)g[G_SE], (const float*)g[G_FNORM], h, logits,
                      NULL, NULL);
  free(h); free(h2);
  return rc ? -2 : next;
}

/* Prefill of one sequence = the decode step applied to each prompt token in
 * turn (the recurrence is sequential); logits of the last position only.    */
int or_prefill(const int* sh, const void* const* w, double* conv, double* ssm, const int* toks, int T,
               double* last_logits) {
  int next = -1;
  for (int t = 0; t < T; ++t) {
    next = or_decode_step(sh, w, conv, ssm, toks[t], (t == T - 1) ? last_logits : NULL, NULL);
    if (next == -2) return -2;
  }
  return next;
}

/* ------------------------------------------------------------------------ */
/* Density-field representation of the SSM state (gist.science summary §2.D:
 * a binary field per state element with K^2 about 4 d_state cells, built by
 * normalisation, sigma-delta injection with error feedback and binarisation,
 * read back by popcount; applied at chunk boundaries).  Reading taken: one
 * field per state ROW -- the d_state values S[h][p][:] of one head channel
 * -- with 4 cells per element (4 d_state cells, K = sqrt(4 d_state)), since a
 * field of 4 d_state bits per single element would be 16 times larger than
 * the fp32 value it replaces.  For a row x[0..n):
 *   normalisation: scale = max |x_i| (0 for an all-zero row);
 *                  density d_i = (x_i / scale + 1) / 2 in [0, 1];
 *   sigma-delta:   e = 0; for cell c = 0 .. 4n-1 (element i = c / 4):
 *                  a = d_i + e; bit_c = (a >= 1/2); e = a - bit_c;
 *   readout:       p_i = popcount of element i's 4 cells;
 *                  x_i' = scale * ((p_i - 2) / 2).
 * The encoder's decisions are taken in fp32 (the precision of the device
 * kernels; each step one rounded fp32 operation), the readout is exact
 * (p_i - 2 is a small integer, halving and the product are one rounding).
 * Field layout: cell c is bit (c % 32) of word c / 32.                     */
void or_density_encode(const float* x, int n, uint32_t* field, float* scale_out) {
  float amax = 0.0f;
  for (int i = 0; i < n; ++i) {
    const float a = fabsf(x[i]);
    if (a > amax) amax = a;
  }
  const int words = (4 * n + 31) / 32;
  for (int w = 0; w < words; ++w) field[w] = 0u;
  *scale_out = amax;
  if (!(amax > 0.0f)) return;
  float e = 0.0f;
  for (int i = 0; i < n; ++i) {
    const float d = (x[i] / amax + 1.0f) * 0.5f;
    for (int k = 0; k < 4; ++k) {
      const float a = d + e;
      const int bit = a >= 0.5f;
      e = a - (float)bit;
      const int c = 4 * i + k;
      if (bit) field[c >> 5] |= 1u << (c & 31);
    }
  }
}

void or_density_decode(const uint32_t* field, float scale, int n, float* x) {
  for (int i = 0; i < n; ++i) {
    int p = 0;
    for (int k = 0; k < 4; ++k) {
      const int c = 4 * i + k;
      p += (int)((field[c >> 5] >> (c & 31)) & 1u);
    }
    x[i] = scale * ((float)(p - 2) * 0.5f);
  }
}

/* Threads the OpenMP loops above use (1 when built without OpenMP). */
#ifdef _OPENMP
#include <omp.h>
int or_num_threads(void) { return omp_get_max_threads(); }
#else
int or_num_threads(void) { return 1; }
#endif
