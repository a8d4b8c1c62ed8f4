// Internal: arguments of the persistent batch-1 decode kernel.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dfssm {


// tensor kinds of a layer, in storage order
enum : int {
  DFSSM_PK_IN_BITS = 0, DFSSM_PK_IN_SW, DFSSM_PK_IN_A, DFSSM_PK_IN_SA, DFSSM_PK_IN_B, DFSSM_PK_IN_SB,
  DFSSM_PK_OUT_BITS, DFSSM_PK_OUT_SW, DFSSM_PK_OUT_A, DFSSM_PK_OUT_SA, DFSSM_PK_OUT_B, DFSSM_PK_OUT_SB,
  DFSSM_PK_CONV_W, DFSSM_PK_CONV_B, DFSSM_PK_A_LOG, DFSSM_PK_DT_BIAS, DFSSM_PK_D, DFSSM_PK_NORM_W, DFSSM_PK_GNORM_W
};

struct PersistArgs {
  const char* wbase;  // layer l, kind k at wbase + l * stride + offset(k) (checked by the runtime)
  int n_layer, d_model, d_inner, d_state, headdim, n_heads, vocab, d_conv, rank;
  float eps;
  const int8_t* E;
  const float* sE;
  const float* final_norm;
  float* conv;  // sequence slot 0: [n_layer][d_conv-1][conv_dim]
  float* ssm;   // sequence slot 0: [n_layer][H][P/16][N][16]
  // mailboxes, one block (R replicas each): h [R][d_model / 2] (paired) | B,C [R][2 d_state] |
  // g [R][d_inner / 2] (paired) | argmax [R][2 grid]
  uint64_t* boxes;
  unsigned epoch0;  // first epoch of this launch (host-assigned, never reused)
  unsigned pair0;   // write count of the paired boxes at the first write of this launch (mod 4 differs
                    // from the tag every paired word holds when the launch starts)
  int* abort_flag;
  int* err;
  const int32_t* tok_in;  // [1] first input token
  int32_t* tok_last;      // [1] or null: receives the last generated token
  int32_t* tok_out;       // [n_tokens] or null
  int n_tokens;
  float* logits;          // [vocab], logits of the last token
  float* trace_h;         // [n_layer + 1][d_model] or null (n_tokens == 1)
  int8_t* trace_q1;       // [n_layer][d_model] or null
  int8_t* trace_q2;       // [n_layer][d_inner] or null
  int8_t* trace_qf;       // [d_model] or null
  int32_t* trace_acc1;    // [n_layer][d_in_proj] in_proj scaffold sums, or null
  int32_t* trace_acc2;    // [n_layer][d_model] out_proj scaffold sums, or null
  unsigned long long* prof;  // or null: phase timestamps [prof_tokens][n_layer + 1][grid][kProfEvents]
  int prof_tokens;
};

constexpr int kProfEvents = 10;

// exchanges one token uses (the launch needs epochs [epoch0, epoch0 + n_tokens * this))
inline unsigned persistent_exchanges_per_token(int n_layer) { return (unsigned)(3 * n_layer + 1); }

hipError_t launch_decode_persistent(const PersistArgs& a, int grid, hipStream_t st);
bool persistent_supported(int d_model, int d_inner, int d_state, int headdim, int n_heads, int rank, int grid,
                          const char** why);
size_t persistent_box_words(int d_model, int d_inner, int d_state, int grid);
// layer stride and per-kind offsets the kernel assumes for this shape (false: shape not compiled)
bool persistent_layout(int d_model, int d_inner, int d_state, int headdim, size_t* stride, size_t* offsets);

}  // namespace dfssm
