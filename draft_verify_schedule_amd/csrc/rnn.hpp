// RNN head of the sequential draft stage (DSpark paper, section 3.1, RNN
// head): host-side parameters and launchers shared by the draft driver.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace dspark {

struct RnnParams {
  int B, K, V, r, d;
  const uint16_t* H;   // [B, K, d] bf16 backbone hidden states (h_k at [b, k-1])
  const uint16_t* W;   // [3r, 2r + d] bf16: gate rows, candidate rows, output rows
  const uint16_t* W1;  // [V, r] bf16 Markov embedding
  const int32_t* x0;   // [B] anchors
  const int32_t* x;    // [B, K] drafted tokens (x_{k-1} is read at position k)
  float* Hp;           // workspace [hp_split, B * K, 3r]: partial sums of W[:, 2r:] h for every
                       // (request, position), one per slice of the d-wide contraction
  int hp_split;        // contraction slices of the projection GEMM (set by rnn_bind_workspace)
  float* s[2];         // workspace [B, r] x 2: state of the odd / even positions
  float* O;            // [B, K, r] output parts o_k (the caller's buffer)
  uint16_t* W2h;       // fp16 copy of W2 in MFMA fragment order (caller's, or in the workspace)
  bool w2h_ready;      // W2h was made by the caller: the call does not rebuild it
  const uint16_t* W2;  // [V, r] bf16 column-major W2
};

// with_w2h: room for the fp16 copy of W2 (absent when the caller made it)
size_t rnn_workspace_bytes(int B, int K, int V, int r, int d, bool with_w2h = true);
// Carves Hp, the two state buffers and W2h out of a workspace of
// rnn_workspace_bytes; a caller-made copy (p.w2h_ready) is kept.
void rnn_bind_workspace(RnnParams& p, void* workspace);
// fp16 copy of the column-major bf16 W2 in MFMA fragment order (the layout
// W2SwzFrags reads): the operand the split output parts meet on the MFMA.
int run_w2_to_f16(const uint16_t* W2, uint16_t* out, int V, int r, hipStream_t stream);
size_t w2_f16_bytes(int V, int r);
// Hp = h W[:, 2r:]^T for all B * K rows: one MFMA GEMM per call, its
// contraction split in hp_split slices whose partials rnn_step adds in order.
int run_rnn_hproj(const RnnParams& p, hipStream_t stream);
// The gated update of position k (1-based) for every request: writes s_k and o_k.
int run_rnn_step(const RnnParams& p, int k, hipStream_t stream);

}  // namespace dspark
