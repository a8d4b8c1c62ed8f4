/*
 * dfssm_host.h -- C ABI of the host CPU backend of the DF-SSM decode step.
 *
 * The same model and the same arithmetic as the device library (dfssm.h):
 * 1-bit sign scaffold with an fp32 row scale plus an int8 rank-r LoRA on
 * in_proj / out_proj, the depthwise causal conv shift register, the Mamba-2
 * SSM recurrence, the int8 tied embedding / LM head, int8 activation codes.
 * Source: "Density Field State Space Models: 1-Bit Distillation, Efficient
 * Inference, and Knowledge Organization in Mamba-2" -- gist.science
 * technical summary §2.C, CPU (AVX-512): the packed sign bits are expanded
 * to int8 in registers and fed to the VNNI byte dot product
 * (_mm512_dpbusd_epi32), so the weights stream from memory at one bit each;
 * §3 reports the resulting CPU speed-up (2.9x on an Intel Xeon, baseline
 * unstated).
 *
 * Here 64 bits of a weight row become a 0/1 byte vector (one mask load and
 * one masked move of a vector of ones), dpbusd sums the int8 codes where a
 * bit is set (pos), and the scaffold sum is 2 pos - sum(q): an exact int32.  The LM
 * head and the LoRA down products are int8 x int8 dot products on the same
 * instruction (one operand offset by 128, the offset's exact contribution
 * subtracted).  Every floating-point operation is shared by both integer
 * paths and fixed in order, so the AVX-512 VNNI path and the portable one
 * give bit-identical results.
 *
 * Conventions
 *  - All pointers are host memory owned by the caller; every call is
 *    synchronous and returns when its results are written.
 *  - Shapes, tensor kinds, layouts, quantisation and the synthetic generator
 *    are those of dfssm.h (dfssm_config, DFSSM_T_*, DFSSM_G_*).  max_chunk_rows
 *    is ignored.  Supported: d_model and d_inner multiples of 64 up to 32768;
 *    d_state a multiple of 16; d_conv = 4; 1 <= lora_rank <= 32;
 *    1 <= max_batch <= 1024.
 *  - Every function returns a dfssm_status; on error outputs and state are
 *    untouched and dfssm_host_last_error() describes it.  No C++ exception
 *    crosses this boundary.  A context is not thread-safe; each call runs
 *    its own worker threads (OpenMP).
 *  - Test infrastructure (the CPU oracle) is not part of this library.
 */
#ifndef DFSSM_HOST_H
#define DFSSM_HOST_H

#include <stddef.h>
#include <stdint.h>

#include "dfssm.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct dfssm_host dfssm_host;

/* Integer-product paths. */
enum {
  DFSSM_HOST_ISA_AUTO = 0,        /* AVX-512 VNNI where the CPU has it, else portable */
  DFSSM_HOST_ISA_PORTABLE = 1,    /* plain C++ loops (any x86-64-v3 CPU)              */
  DFSSM_HOST_ISA_AVX512VNNI = 2   /* AVX-512 F/BW + VNNI dpbusd                      */
};

/* Message of the last error on this host thread. */
const char* dfssm_host_last_error(void);

/* Create a host context: validates cfg, allocates the weights (zero) and
 * the state of max_batch sequences (zero).  n_threads: worker threads per
 * call (0 = the OpenMP default).                                            */
dfssm_status dfssm_host_create(const dfssm_config* cfg, int32_t n_threads, dfssm_host** out);
void dfssm_host_destroy(dfssm_host* h);

/* Select the integer-product path; DFSSM_E_UNSUPPORTED if this CPU lacks it.
 * dfssm_host_get_isa reports the path in use (never AUTO).                 */
dfssm_status dfssm_host_set_isa(dfssm_host* h, int32_t isa);
dfssm_status dfssm_host_get_isa(const dfssm_host* h, int32_t* isa);

/* Fill every weight with the seeded synthetic generator of dfssm.h
 * (dfssm_load_synthetic: same values, element for element) and zero the
 * state.                                                                    */
dfssm_status dfssm_host_load_synthetic(dfssm_host* h, uint64_t seed);

/* Copy one weight tensor in or out (canonical layout of dfssm.h; `bytes`
 * must equal the tensor size; layer = -1 selects a model-wide tensor).     */
dfssm_status dfssm_host_set_tensor(dfssm_host* h, int32_t layer, int32_t kind, const void* src, size_t bytes);
dfssm_status dfssm_host_get_tensor(const dfssm_host* h, int32_t layer, int32_t kind, void* dst, size_t bytes);

/* Zero the conv and SSM state of sequences [0, batch). */
dfssm_status dfssm_host_reset_state(dfssm_host* h, int32_t batch);

/* Read / write the state of one sequence slot: conv fp32 [n_layer][conv_dim]
 * [d_conv - 1] (oldest input first), ssm fp32 [n_layer][n_heads][headdim]
 * [d_state]; either pointer may be NULL.                                    */
dfssm_status dfssm_host_get_state(const dfssm_host* h, int32_t seq, float* conv, float* ssm);
dfssm_status dfssm_host_set_state(dfssm_host* h, int32_t seq, const float* conv, const float* ssm);

/* One decode step of sequences [0, B) (gist.science summary §2.C): token
 * tok[b] through every layer, updating slot b.  logits fp32 [B][vocab] or
 * NULL; next int32 [B] (argmax, lowest index on ties) or NULL.  A token id
 * outside [0, vocab) is DFSSM_E_INVALID (nothing runs).                    */
dfssm_status dfssm_host_decode_step(dfssm_host* h, const int32_t* tok, int32_t B, float* logits, int32_t* next);

/* The decode step recording its intermediate results, in the layouts of
 * dfssm_trace_step: h_trace fp32 [n_layer + 1][B][d_model], q1 int8
 * [n_layer][B][d_model], q2 int8 [n_layer][B][d_inner], qf int8 [B][d_model],
 * logits fp32 [B][vocab], acc1 int32 [n_layer][B][d_in_proj], acc2 int32
 * [n_layer][B][d_model] (the exact scaffold sums); each may be NULL.        */
dfssm_status dfssm_host_trace_step(dfssm_host* h, const int32_t* tok, int32_t B, float* h_trace, int8_t* q1,
                                   int8_t* q2, int8_t* qf, float* logits, int32_t* acc1, int32_t* acc2);

/* n_steps greedy steps: tok [B] holds the first inputs and receives the last
 * generated tokens; out int32 [n_steps][B] (or NULL) every generated token. */
dfssm_status dfssm_host_generate(dfssm_host* h, int32_t* tok, int32_t B, int32_t n_steps, int32_t* out);

/* Prefill of sequences [0, B) with the prompt tok int32 [B][T] from their
 * current state, as T decode steps (the recurrence in token order, so the
 * result is that of the decode loop bit for bit); last_logits fp32
 * [B][vocab] and next int32 [B] of the last position, each may be NULL.    */
dfssm_status dfssm_host_prefill(dfssm_host* h, const int32_t* tok, int32_t B, int32_t T, float* last_logits,
                                int32_t* next);

/* Measured memory rate of this host with the context's threads: copies a
 * buffer of `bytes` (rounded down to 64) `iters` times and reports read +
 * written bytes per second, in GB/s (the ceiling a memory-bound step meets
 * on this machine; no published peak is assumed).                         */
dfssm_status dfssm_host_copy_rate(dfssm_host* h, size_t bytes, int32_t iters, double* gbs);

#ifdef __cplusplus
}
#endif

#endif /* DFSSM_HOST_H */
