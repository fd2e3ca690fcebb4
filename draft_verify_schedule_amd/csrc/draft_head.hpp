// Host-side parameters of the confidence head evaluated inside the Markov
// draft (DSpark paper, section 3.2.1, Confidence Head): shared by the C ABI
// and the draft driver.
#pragma once

#include <cstdint>

namespace dspark {

struct DraftHead {
  const void* H;      // [B, K, d] hidden states (h_k at [b, k-1]), bf16 or f32
  bool h_bf16;
  int d;
  const float* w_h;   // [d]
  const float* w_e;   // [r] (unused when r == 0)
  float bias;
  const float* T;     // [K] calibration temperatures, or null (T = 1)
  float* c_out;       // [B, K]
  float* logit_out;   // [B, K] or null
};

}  // namespace dspark
