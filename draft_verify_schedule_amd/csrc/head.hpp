// Arithmetic of the confidence head (DSpark paper, section 3.2.1, Confidence
// Head: a linear projection of the hidden state and the previous token's
// Markov embedding, then a sigmoid), shared by the standalone head kernel and
// the draft's locate pass, which evaluates the head of each position as soon
// as the previous token is known.  Both take every product in the same lane
// and the same order and sum the lanes with the same xor tree, so they give
// bit-identical confidences:
//   lane l accumulates w_h . h over its elements (16-byte vector steps of 8
//   bf16 / 4 f32 elements at l * 8 + 512 t / l * 4 + 256 t, or single
//   elements l + 64 t), then w_e . W1[x_{k-1}] over elements l + 64 t, in
//   fp32 with fused multiply-adds; the wave sums the lanes pairwise at
//   distances 32, 16, ..., 1.
#pragma once

#include <math.h>

#include "common.hpp"

namespace dspark {

// One vector step over 8 bf16 hidden-state elements (v: the lane's 16 bytes
// of the row, w0 / w1: w_h of elements 0..3 / 4..7), in the fixed order
// 0, 1, 4, 5, 2, 3, 6, 7.
__device__ __forceinline__ float head_step_bf16(float s, u32x4 v, f32x4 w0, f32x4 w1) {
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    s = fmaf(w0[2 * e], __uint_as_float(v[e] << 16), s);
    s = fmaf(w0[2 * e + 1], __uint_as_float(v[e] & 0xFFFF0000u), s);
    s = fmaf(w1[2 * e], __uint_as_float(v[e + 2] << 16), s);
    s = fmaf(w1[2 * e + 1], __uint_as_float(v[e + 2] & 0xFFFF0000u), s);
  }
  return s;
}

// One vector step over 4 f32 hidden-state elements.
__device__ __forceinline__ float head_step_f32(float s, u32x4 v, f32x4 w0) {
#pragma unroll
  for (int e = 0; e < 4; ++e) s = fmaf(w0[e], __uint_as_float(v[e]), s);
  return s;
}

// The lane's part of w_h . h for a row h of d elements.  VEC: 16-byte steps
// (h and w_h 16-byte aligned, d a multiple of 8 for bf16 / 4 for f32).
template <typename HT, bool VEC>
__device__ __forceinline__ float head_hidden_part(const HT* h, const float* w_h, int d, int lane) {
  float s = 0.f;
  if constexpr (VEC) {
    constexpr int E = 16 / sizeof(HT);
    for (int j = lane * E; j < d; j += 64 * E) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(h + j);
      const f32x4 w0 = *reinterpret_cast<const f32x4*>(w_h + j);
      if constexpr (sizeof(HT) == 2) s = head_step_bf16(s, v, w0, *reinterpret_cast<const f32x4*>(w_h + j + 4));
      else s = head_step_f32(s, v, w0);
    }
  } else {
    for (int j = lane; j < d; j += 64) {
      float hv;
      if constexpr (sizeof(HT) == 2) hv = bf16_bits_to_f32(h[j]);
      else hv = h[j];
      s = fmaf(w_h[j], hv, s);
    }
  }
  return s;
}

// The lane's Markov part, added after its hidden-state part: w_e[j] (from
// we(t)) times element j of the previous token's W1 row (bf16 bits from
// elem(j)) for j = lane + 64 t < r, t = 0, 1, 2, 3 (r <= 256).
constexpr int kHeadMarkovSteps = 4;
template <typename WE, typename Elem>
__device__ __forceinline__ float head_markov_part(float s, int r, int lane, WE we, Elem elem) {
#pragma unroll
  for (int t = 0; t < kHeadMarkovSteps; ++t) {
    const int j = lane + 64 * t;
    if (j < r) s = fmaf(we(t), bf16_bits_to_f32(elem(j)), s);
  }
  return s;
}

// The wave's sum of the lanes' parts (every lane ends with it).
__device__ __forceinline__ float head_wave_sum(float s) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
  return s;
}

// c = sigmoid(z / T), T the position's calibration temperature (1 before
// calibration).
__device__ __forceinline__ float head_sigmoid(float z, float t) { return 1.f / (1.f + expf(-z / t)); }

}  // namespace dspark
