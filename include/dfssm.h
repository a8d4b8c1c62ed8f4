/*
 * dfssm.h -- C ABI of the DF-SSM decode library for AMD Instinct MI355X (gfx950).
 *
 * The model: a Mamba-2 stack whose in_proj / out_proj weights are a frozen
 * 1-bit sign scaffold (with an fp32 per-row scale) plus an int8 rank-r LoRA
 * correction, a depthwise causal conv shift register, the Mamba-2 SSM
 * recurrence, and an int8 per-row-scaled embedding tied to the LM head.
 * Sources: "Density Field State Space Models: 1-Bit Distillation, Efficient
 * Inference, and Knowledge Organization in Mamba-2" -- gist.science technical
 * summary §2.B (frozen scaffold, LoRA r = 16 on in_proj and out_proj of all
 * layers, int8 LoRA and embedding / LM head with per-row scales), §2.C
 * (1-bit weights used as int8 operands, custom conv shift-register and SSM
 * recurrence kernels, whole forward captured as one graph), §3 (size
 * composition: one tied int8 embedding copy) and the arxivdaily English
 * abstract.  The Mamba-2 block itself is its published definition.
 *
 * Conventions shared by every entry point
 *  - Pointers named d_* are device pointers (hipMalloc'd or torch CUDA tensor
 *    storage) owned by the caller; they must stay valid until the work
 *    enqueued on `stream` has finished.  Pointers named host* are host memory.
 *  - `stream` is a hipStream_t passed as void*; NULL is the null stream.
 *  - Compute entry points only enqueue work and return; they never block the
 *    host, so they may be captured into a graph.  Entry points documented as
 *    synchronous wait for the device.
 *  - Every function returns a dfssm_status.  On any error nothing has been
 *    enqueued, outputs are untouched, and dfssm_last_error() describes it.
 *    No C++ exception crosses this boundary.
 *  - A context is not thread-safe: use one per host thread.
 *  - Layouts are row-major ("canonical") unless stated.  A 1-bit scaffold
 *    matrix of shape d_out x d_in is stored as uint32 words
 *    [d_out][d_in / 32]; weight (o, i) is +1 when bit (i % 32) of word
 *    [o][i / 32] is set and -1 when it is clear.
 *  - Activation quantisation (unstated on the pages; read here as per token,
 *    symmetric absmax int8): q_i = clamp(rint(u_i * (127 / amax)), -127, 127)
 *    with the division and product in fp32 and ties to even, s = amax / 127;
 *    an all-zero vector gives q = 0, s = 0.
 */
#ifndef DFSSM_H
#define DFSSM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DFSSM_OK = 0,
  DFSSM_E_INVALID = -1,     /* bad argument: shape, pointer, size, index */
  DFSSM_E_OOM = -2,         /* device allocation failed */
  DFSSM_E_HIP = -3,         /* a HIP runtime call failed */
  DFSSM_E_STATE = -4,       /* call out of order (e.g. decode before weights are loaded) */
  DFSSM_E_UNSUPPORTED = -5, /* shape outside what the kernels implement */
  DFSSM_E_DEVICE = -6       /* error flagged by a kernel (e.g. token id >= vocab) */
} dfssm_status;

/* Model dimensions (ngroups = 1).  Derived: n_heads = d_inner / headdim,
 * conv_dim = d_inner + 2 d_state, d_in_proj = 2 d_inner + 2 d_state + n_heads.
 * Supported: d_model and d_inner multiples of 128 with d/128 a power of two
 * <= 64; headdim a multiple of 16 and n_heads a multiple of 4; d_state
 * even; d_conv = 4; 1 <= lora_rank <= 32;
 * 1 <= max_batch <= 1024.  norm_eps is the RMSNorm epsilon (1e-5 if 0).
 * max_chunk_rows: token rows (summed over the batch) that one prefill chunk
 * of the batched path holds, 0 for the default 16384; it sizes the
 * batched-path workspace (0 <= max_chunk_rows <= 2^20).                     */
typedef struct {
  int32_t n_layer, d_model, d_inner, d_state, headdim, vocab, d_conv, lora_rank;
  int32_t max_batch;
  float norm_eps;
  int32_t max_chunk_rows;
} dfssm_config;

/* Per-layer tensor kinds (dfssm_set_tensor / dfssm_get_tensor with layer >= 0). */
enum {
  DFSSM_T_IN_BITS = 0,  /* uint32 [d_in_proj][d_model/32] scaffold signs            */
  DFSSM_T_IN_SW = 1,    /* fp32 [d_in_proj] scaffold row scale                     */
  DFSSM_T_IN_A = 2,     /* int8 [r][d_model]  LoRA down projection                 */
  DFSSM_T_IN_SA = 3,    /* fp32 [r]                                                */
  DFSSM_T_IN_B = 4,     /* int8 [d_in_proj][r] LoRA up projection                  */
  DFSSM_T_IN_SB = 5,    /* fp32 [d_in_proj]                                        */
  DFSSM_T_OUT_BITS = 6, /* uint32 [d_model][d_inner/32]                            */
  DFSSM_T_OUT_SW = 7,   /* fp32 [d_model]                                          */
  DFSSM_T_OUT_A = 8,    /* int8 [r][d_inner]                                       */
  DFSSM_T_OUT_SA = 9,   /* fp32 [r]                                                */
  DFSSM_T_OUT_B = 10,   /* int8 [d_model][r]                                       */
  DFSSM_T_OUT_SB = 11,  /* fp32 [d_model]                                          */
  DFSSM_T_CONV_W = 12,  /* fp32 [conv_dim][d_conv], tap d_conv-1 meets the newest input */
  DFSSM_T_CONV_B = 13,  /* fp32 [conv_dim]                                         */
  DFSSM_T_A_LOG = 14,   /* fp32 [n_heads], A = -exp(A_log)                          */
  DFSSM_T_DT_BIAS = 15, /* fp32 [n_heads]                                          */
  DFSSM_T_D = 16,       /* fp32 [n_heads]                                          */
  DFSSM_T_NORM_W = 17,  /* fp32 [d_model] pre-norm weight                          */
  DFSSM_T_GNORM_W = 18, /* fp32 [d_inner] gated-norm weight                         */
  DFSSM_T_PER_LAYER = 19
};
/* Model-wide tensor kinds (layer = -1). */
enum {
  DFSSM_G_EMBED = 0,       /* int8 [vocab][d_model], tied with the LM head */
  DFSSM_G_EMBED_SCALE = 1, /* fp32 [vocab]                                 */
  DFSSM_G_FINAL_NORM = 2   /* fp32 [d_model]                               */
};

typedef struct dfssm_ctx dfssm_ctx;

/* Library version string (static storage). */
const char* dfssm_version(void);

/* Message of the last error on this host thread (ctx may be NULL). */
const char* dfssm_last_error(const dfssm_ctx* ctx);

/* Device bytes a context of this configuration needs when the caller
 * provides its memory (dfssm_create with an arena): the weights, the
 * recurrent state of max_batch sequences, the decode workspace, the
 * persistent kernel's mailboxes and the batched-path workspace of
 * max(max_chunk_rows, max_batch) token rows.  Host arithmetic only: touches
 * no device.                                                                */
dfssm_status dfssm_arena_bytes(const dfssm_config* cfg, size_t* bytes);

/* Create a context on `device`: validates cfg and lays out the weights, the
 * recurrent state of max_batch sequences, the workspace and the mailboxes in
 * device memory.  arena: NULL, and the library allocates that memory (freed
 * by dfssm_destroy; the batched-path workspace then grows on first use), or
 * a 256-byte-aligned device buffer of at least dfssm_arena_bytes(cfg) bytes
 * owned by the caller, who must keep it alive until dfssm_destroy returns and
 * free it afterwards; the context then makes no device allocation of its own
 * (prefill chunks and traced prefills are bounded by the arena's workspace).
 * Zeroes the state.  Synchronous.                                          */
dfssm_status dfssm_create(const dfssm_config* cfg, int32_t device, void* arena, size_t arena_bytes,
                          dfssm_ctx** out);
void dfssm_destroy(dfssm_ctx* ctx);

/* Execution path.  DFSSM_PATH_AUTO (default) runs batch-1 decode_step /
 * generate / trace_step as one persistent kernel (every workgroup resident
 * across all layers and tokens, hops between workgroups through device
 * memory) when the shape and device allow it, decode of B > 1 sequences and
 * every prefill on the batched path (each layer on all token rows at once:
 * int8 matrix-core GEMMs for the projections; the SSM over a prompt as
 * 64-token chunks of fp32 matrix products with the causal conv inside for
 * headdim 64 / d_state 128, else a causal conv pass and a sequential scan;
 * prefill in chunks of at most max_chunk_rows token rows across the batch).
 * DFSSM_PATH_KERNELS runs everything as per-layer GEMV kernels, one token at
 * a time.  DFSSM_PATH_PERSISTENT is AUTO but fails with DFSSM_E_UNSUPPORTED
 * where batch 1 cannot use the persistent kernel.  DFSSM_PATH_GEMM runs
 * every decode (batch 1 included) and prefill on the batched path.          */
enum { DFSSM_PATH_AUTO = 0, DFSSM_PATH_KERNELS = 1, DFSSM_PATH_PERSISTENT = 2, DFSSM_PATH_GEMM = 3 };
dfssm_status dfssm_set_path(dfssm_ctx* ctx, int32_t path);

/* Device bytes the context uses (its arena plus a grown batched-path workspace). */
dfssm_status dfssm_device_bytes(const dfssm_ctx* ctx, size_t* bytes);

/* Fill every weight with the seeded synthetic generator, on the device, in
 * the canonical layouts above.  Value of element i of tensor (layer, kind):
 * draw = mix(mix(seed ^ (tid << 32)) + i) with mix the SplitMix64 output
 * function and tid = 64 layer + kind (4096 + kind for model-wide tensors);
 * sign words = draw >> 32; int8 = draw % 255 - 127; uniforms
 * fp32(a + (b - a) (draw >> 40) 2^-24) in fp64; "N(0,1)" = sum of 12 such
 * uniforms minus 6.  Distributions: scaffold row scales U(0.01, 0.05); LoRA
 * int8 with row scales 1e-3; conv weight and bias U(-0.5, 0.5); A_log
 * U(0, ln 16); dt_bias U(-4, -1); D "N(0,1)"; norm weights U(0.5, 1.5);
 * embedding int8 with row scales U(0.01, 0.02).  Also zeroes the state.
 * Enqueued on `stream`.                                                      */
dfssm_status dfssm_load_synthetic(dfssm_ctx* ctx, uint64_t seed, void* stream);

/* Copy one weight tensor in or out (host memory, canonical layout, `bytes`
 * must equal the tensor size).  layer = -1 selects a model-wide tensor.
 * Synchronous.  dfssm_set_tensor marks the weights as loaded.               */
dfssm_status dfssm_set_tensor(dfssm_ctx* ctx, int32_t layer, int32_t kind, const void* host, size_t bytes);
dfssm_status dfssm_get_tensor(dfssm_ctx* ctx, int32_t layer, int32_t kind, void* host, size_t bytes);

/* Zero the conv and SSM state of sequences [0, batch).  Enqueued. */
dfssm_status dfssm_reset_state(dfssm_ctx* ctx, int32_t batch, void* stream);

/* Read / write the recurrent state of one sequence slot, synchronously.
 * host_conv: fp32 [n_layer][conv_dim][d_conv - 1], the previous inputs of
 * each conv channel, oldest first.  host_ssm: fp32 [n_layer][n_heads]
 * [headdim][d_state].  Either pointer may be NULL to skip that part.       */
dfssm_status dfssm_get_state(dfssm_ctx* ctx, int32_t seq, float* host_conv, float* host_ssm);
dfssm_status dfssm_set_state(dfssm_ctx* ctx, int32_t seq, const float* host_conv, const float* host_ssm);

/* One decode step for sequences [0, B) (gist.science summary §2.C: the
 * decode pipeline of bit-packed scaffold products on int8 operands, the
 * stateful conv shift register and the SSM recurrence; arxivdaily abstract:
 * batch-1 decode speed): token d_tok[b] goes through the whole stack,
 * updating the state of slot b.  d_logits: fp32 [B][vocab] or NULL;
 * d_next: int32 [B] greedy next token (argmax, lowest index on ties) or NULL;
 * d_next may alias d_tok.  A token id outside [0, vocab) is read as 0 and
 * flagged; the flag surfaces as DFSSM_E_DEVICE from dfssm_check_device.     */
dfssm_status dfssm_decode_step(dfssm_ctx* ctx, const int32_t* d_tok, int32_t B, float* d_logits,
                               int32_t* d_next, void* stream);

/* n_steps greedy decode steps for sequences [0, B) (gist.science summary
 * §2.C: the whole forward replayed as one graph against launch overhead at
 * batch 1; here one persistent launch at batch 1, a HIP graph otherwise).  d_tok [B] holds the
 * first input tokens and receives the last generated ones; d_out (int32
 * [n_steps][B], may be NULL) receives every generated token.  The argmax is
 * fed back on the device.  With use_graph != 0 one step is captured into a
 * HIP graph (cached per B and pointer set) and replayed n_steps times.      */
dfssm_status dfssm_generate(dfssm_ctx* ctx, int32_t* d_tok, int32_t B, int32_t n_steps, int32_t* d_out,
                            int32_t use_graph, void* stream);

/* Prefill sequences [0, B) with the prompt d_tok (int32 [B][T], row-major)
 * starting from their current state (gist.science summary §2.C: the same
 * stateful conv and SSM recurrence run over the prompt; here the SSM over 64-
 * token chunks, the pages mentioning chunk boundaries of the state in §2.D);
 * the result equals T decode steps up to fp32 summation order.  Leaves the
 * state after the last token.
 * d_last_logits: fp32 [B][vocab] of the last position, or NULL; d_next: int32
 * [B] greedy next token, or NULL.                                           */
dfssm_status dfssm_prefill(dfssm_ctx* ctx, const int32_t* d_tok, int32_t B, int32_t T, float* d_last_logits,
                           int32_t* d_next, void* stream);

/* One layer for sequences [0, B) (gist.science summary §2.B/§2.C: one
 * Mamba-2 block with its scaffold + LoRA projections, conv shift register and
 * SSM recurrence): d_h_out = d_h_in + mixer(d_h_in), both fp32 [B][d_model],
 * using and updating layer `layer` of slots [0, B), on the per-layer GEMV
 * kernels.  d_q1 (int8 [B][d_model]) and d_q2 (int8 [B][d_inner]), when
 * non-NULL, receive the quantised activations fed to in_proj and out_proj.  */
dfssm_status dfssm_layer_step(dfssm_ctx* ctx, int32_t layer, const float* d_h_in, float* d_h_out, int32_t B,
                              int8_t* d_q1, int8_t* d_q2, void* stream);

/* dfssm_layer_step with fp16 input activations: d_h_f16 holds IEEE binary16
 * values [B][d_model] (upcast exactly to fp32 on the device).              */
dfssm_status dfssm_layer_step_f16(dfssm_ctx* ctx, int32_t layer, const uint16_t* d_h_f16, float* d_h_out,
                                  int32_t B, int8_t* d_q1, int8_t* d_q2, void* stream);

/* A decode step that also records its intermediate results: d_h_trace fp32
 * [n_layer + 1][B][d_model] is the residual stream entering every layer and
 * after the last; d_q1_trace int8 [n_layer][B][d_model], d_q2_trace int8
 * [n_layer][B][d_inner] and d_qf int8 [B][d_model] (each may be NULL) are the
 * quantised inputs of every in_proj, out_proj and of the LM head;
 * d_acc1_trace int32 [n_layer][B][d_in_proj] and d_acc2_trace int32
 * [n_layer][B][d_model] (each may be NULL) receive the exact scaffold sums
 * sum_i w(o,i) q_i of every in_proj and out_proj row (gist.science summary
 * §2.C: the 1-bit scaffold used as int8 operands of an integer product).
 * Runs on the same path as dfssm_decode_step for this B; at batch 1 on the
 * persistent path it is the kernel's tracing instantiation, one token per
 * launch.                                                                   */
dfssm_status dfssm_trace_step(dfssm_ctx* ctx, const int32_t* d_tok, int32_t B, float* d_h_trace,
                              int8_t* d_q1_trace, int8_t* d_q2_trace, int8_t* d_qf, float* d_logits,
                              int32_t* d_acc1_trace, int32_t* d_acc2_trace, void* stream);

/* Prefill of sequences [0, B) on the batched path in one chunk (1 <= B T <=
 * 16384 token rows, the prefill chunk size) that also records its
 * intermediate results, row m = b T + t: d_h_trace fp32
 * [n_layer + 1][B T][d_model], d_q1_trace int8 [n_layer][B T][d_model],
 * d_q2_trace int8 [n_layer][B T][d_inner] (each may be NULL but d_h_trace),
 * d_qf int8 [B][d_model] (LM-head input of the last position), d_logits fp32
 * [B][vocab] (last position), d_acc1_trace int32 [n_layer][B T][d_in_proj]
 * and d_acc2_trace int32 [n_layer][B T][d_model] (scaffold sums as for
 * dfssm_trace_step), each may be NULL.  Same kernels and launch shapes as
 * dfssm_prefill of that chunk.  Leaves the state after the last token.
 * Enqueued.                                                                */
dfssm_status dfssm_trace_prefill(dfssm_ctx* ctx, const int32_t* d_tok, int32_t B, int32_t T, float* d_h_trace,
                                 int8_t* d_q1_trace, int8_t* d_q2_trace, int8_t* d_qf, float* d_logits,
                                 int32_t* d_acc1_trace, int32_t* d_acc2_trace, void* stream);

/* Kernel timing for roofline reports.  Launches one kernel of the batch-B
 * decode step `iters` times back to back on `stream` (layer i % n_layer on
 * launch i, same arguments as inside the step) between two HIP events and
 * writes the mean time per launch in microseconds to *avg_us.  Synchronous.
 * Leaves the recurrent state and the workspace undefined: reset the state
 * before decoding again.                                                   */
enum {
  /* per-layer GEMV path */
  DFSSM_K_IN_PROJ = 0,    /* norm-quantised input -> 1-bit GEMV + LoRA + conv epilogue */
  DFSSM_K_SSM = 1,        /* SSM state update + gate                                  */
  DFSSM_K_OUT_PROJ = 2,   /* 1-bit GEMV + LoRA + residual                             */
  DFSSM_K_LM_HEAD = 3,    /* tied int8 LM head GEMV                                   */
  DFSSM_K_NORM_QUANT = 4, /* RMSNorm + quantise + operand prep of the in_proj input    */
  /* batched path, one decode token for each of B sequences */
  DFSSM_K_B_ROWS_IN = 5,   /* RMSNorm + quantise + LoRA down of the residual rows       */
  DFSSM_K_B_IN_PROJ = 6,   /* scaffold + LoRA GEMM of in_proj (+ conv)                  */
  DFSSM_K_B_SCAN = 7,      /* SSM state update + gate                                   */
  DFSSM_K_B_ROWS_OUT = 8,  /* gated RMSNorm + quantise + LoRA down                      */
  DFSSM_K_B_OUT_PROJ = 9,  /* scaffold + LoRA GEMM of out_proj + residual               */
  DFSSM_K_B_LM_HEAD = 10   /* final norm + int8 LM head                                 */
};
dfssm_status dfssm_time_kernel(dfssm_ctx* ctx, int32_t kernel, int32_t B, int32_t iters, float* avg_us,
                               void* stream);

/* Phase timestamps of the persistent batch-1 decode kernel, for performance
 * analysis: greedy-decodes n_tokens from d_tok[0] (updated in place like
 * dfssm_generate) and writes, for the first prof_tokens tokens, the device
 * clock (100 MHz counter, uint64) at 10 points of every layer (index n_layer
 * covers the LM head) of every workgroup into d_prof: uint64
 * [prof_tokens][n_layer + 1][n_heads * headdim / 16][10].  Points per layer:
 * 0 start, 1 residual stream received, 2 normalised and quantised, 3 LoRA
 * down done, 4 in_proj rows done, 5 conv done and B/C published, 6 B/C
 * received, 7 SSM done and output published, 8 SSM outputs received,
 * 9 out_proj rows done and published.  LM head: 0 start, 1 residual
 * received, 2 quantised, 3 logits and local argmax done, 4 token chosen.
 * Requires the persistent path.  Enqueued.                                 */
dfssm_status dfssm_profile_persistent(dfssm_ctx* ctx, int32_t* d_tok, int32_t n_tokens, uint64_t* d_prof,
                                      int32_t prof_tokens, void* stream);

/* Density-field representation of the SSM state (gist.science summary §2.D:
 * a binary field with about 4 d_state cells, built by normalisation,
 * sigma-delta injection with error feedback and binarisation, read back by
 * popcount, applied at chunk boundaries).  One field per state row (the
 * d_state values of one head channel), 4 cells per value: scale = max |x|,
 * density d = (x / scale + 1) / 2, a first-order sigma-delta modulator over
 * the row's 4 d_state cells in order (a = d + e; cell = (a >= 1/2); e = a -
 * cell; e starts at 0), readout x' = scale * (popcount of the value's 4 cells
 * - 2) / 2; every step one fp32 operation.  Cell c of a row is bit c % 32 of
 * word c / 32: d_state / 8 uint32 words and one fp32 scale per row (7.5 times
 * smaller than the fp32 row at d_state 128).
 *
 * dfssm_state_pack writes the fields of sequence slots [seq0, seq0 + nseq):
 * d_field uint32 [nseq][n_layer][n_heads][headdim][d_state / 8], d_scale fp32
 * [nseq][n_layer][n_heads][headdim]; dfssm_state_unpack replaces those slots'
 * SSM state by the fields' readout; dfssm_state_roundtrip does both in place
 * (the state passes through the codec, as at a chunk boundary, without
 * storing the field).  The conv state is untouched.  Requires d_state 16, 32,
 * 64 or 128.  Enqueued.                                                    */
dfssm_status dfssm_state_pack(dfssm_ctx* ctx, int32_t seq0, int32_t nseq, uint32_t* d_field, float* d_scale,
                              void* stream);
dfssm_status dfssm_state_unpack(dfssm_ctx* ctx, int32_t seq0, int32_t nseq, const uint32_t* d_field,
                                const float* d_scale, void* stream);
dfssm_status dfssm_state_roundtrip(dfssm_ctx* ctx, int32_t seq0, int32_t nseq, void* stream);

/* Wait for `stream` and report (then clear) any error flagged by a kernel. */
dfssm_status dfssm_check_device(dfssm_ctx* ctx, void* stream);

/* ---- stateless kernel entry points (tests) ---------------------------- */

/* Per-row int8 quantiser (see the conventions above; the pages imply int8
 * activations by the int8 x int8 product of gist.science summary §2.C):
 * d_u fp32 [rows][n] -> d_q int8 [rows][n], d_s fp32 [rows].
 * 1 <= n <= 65536.                                                          */
dfssm_status dfssm_k_quant(const float* d_u, int32_t rows, int32_t n, int8_t* d_q, float* d_s, void* stream);

/* The density-field codec on row-major rows (see dfssm_state_pack): d_x
 * fp32 [rows][n] -> d_field uint32 [rows][n / 8], d_scale fp32 [rows], and
 * back.  n is 16, 32, 64 or 128.  Enqueued.                               */
dfssm_status dfssm_k_density_encode(const float* d_x, int32_t rows, int32_t n, uint32_t* d_field, float* d_scale,
                                   void* stream);
dfssm_status dfssm_k_density_decode(const uint32_t* d_field, const float* d_scale, int32_t rows, int32_t n, float* d_x,
                                   void* stream);

/* Scaffold + LoRA projection of B int8 activation rows (gist.science summary
 * §2.B/§2.C):  acc[b][o] = sum_i w(o,i) q[b][i] exactly (int32);
 * t[b][k] = float(sum_i A[k][i] q[b][i]) * sA[k] * s[b];
 * y[b][o] = float(acc) * sw[o] * s[b] + sB[o] * sum_k B[o][k] t[b][k].
 * d_bits uint32 [d_out][d_in/32], d_A int8 [r][d_in], d_B int8 [d_out][r],
 * d_q int8 [B][d_in], d_s fp32 [B]; outputs d_acc int32 [B][d_out] (or NULL)
 * and d_y fp32 [B][d_out].  Runs the per-layer path's bit-plane GEMV for
 * any B (the int8 matrix-core GEMM is dfssm_k_gemm).  Enqueued; uses
 * stream-ordered temporary memory.                                          */
dfssm_status dfssm_k_proj(const uint32_t* d_bits, const float* d_sw, const int8_t* d_A, const float* d_sA,
                          const int8_t* d_B, const float* d_sB, int32_t d_in, int32_t d_out, int32_t r,
                          const int8_t* d_q, const float* d_s, int32_t B, int32_t* d_acc, float* d_y,
                          void* stream);

/* The same projection on the batched path's matrix-core GEMM, M rows
 * (gist.science summary §2.B/§2.C): r is 16; d_A int8 [16][d_in], d_B int8
 * [d_out][16]; d_q int8 [M][d_in], d_s fp32 [M]; outputs d_acc int32
 * [M][d_out] (or NULL) and d_y fp32 [M][d_out], as for dfssm_k_proj.
 * d_in is 128 * 2^k <= 8192.  M <= 32 runs the decode-sized kernel (one
 * 32 x 32 block per workgroup, K split over its waves), larger M the tiled
 * one.  Enqueued; uses stream-ordered temporary memory.                    */
dfssm_status dfssm_k_gemm(const uint32_t* d_bits, const float* d_sw, const int8_t* d_A, const float* d_sA,
                          const int8_t* d_B, const float* d_sB, int32_t d_in, int32_t d_out, const int8_t* d_q,
                          const float* d_s, int32_t M, int32_t* d_acc, float* d_y, void* stream);

/* dfssm_k_gemm for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * same arguments, same kernels and results, no hipMalloc / hipFree / stream-
 * ordered allocation.  The operand scratch (M * d_in + 68 M bytes, each part
 * rounded up to 256) lives in a static 8 MiB device buffer that each GPU the
 * library runs on holds until the process ends; larger requests fail with
 * DFSSM_E_INVALID before any work.  Every call on one GPU shares that buffer:
 * calls that overlap on one GPU (different streams or threads) race and must
 * be serialised by the caller.  Enqueued.                                   */
dfssm_status dfssm_k_gemm_noalloc(const uint32_t* d_bits, const float* d_sw, const int8_t* d_A, const float* d_sA,
                                  const int8_t* d_B, const float* d_sB, int32_t d_in, int32_t d_out,
                                  const int8_t* d_q, const float* d_s, int32_t M, int32_t* d_acc, float* d_y,
                                  void* stream);

#ifdef __cplusplus
}
#endif
#endif /* DFSSM_H */
