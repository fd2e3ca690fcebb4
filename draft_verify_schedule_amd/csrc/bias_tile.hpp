// The rank-r Markov bias as an MFMA tile: for a stage of 64 rows (requests)
// and one wave's 64 vocabulary columns, bias[m, n] = sum_i W1[prev_m, i] * W2[i, n]
// on v_mfma_f32_16x16x32_bf16 (bf16 in, fp32 accumulate).  This is the one
// dense contraction of the draft: B x r times r x V (DSpark paper, section
// 3.1, Markov head; "Speculative decoding, from zero to DSpark", Appendix A4).
//
// Operand placement (16x16x32 MFMA, wave64):
//   A (16 x 32): lane l supplies row l%16, k = 8*(l/16) .. +7   -> a W2 column
//   B (32 x 16): lane l supplies column l%16, same k range      -> an E row
//   D (16 x 16): lane l holds rows 4*(l/16) + i (i = 0..3), column l%16.
// The 64 columns of a wave are split over four MFMAs ("blocks" b = 0..3) and
// A-row a of block b is mapped to column n0 + 16*(a/4) + 4*b + a%4, so that
// after the four MFMAs lane l holds 16 CONSECUTIVE columns
// n0 + 16*(l/16) .. +15 of row l%16: the epilogue then reads its 16 base
// logits with two 16-byte loads (bf16) and no shuffles.
#pragma once

#include "common.hpp"

namespace dspark {

constexpr int kStageRows = 64;   // rows (requests) per LDS stage
constexpr int kWaveCols = 64;    // vocabulary columns per wave (= one partial slice)
constexpr int kTileCols = 256;   // columns per workgroup (4 waves)

// LDS row pitch in bf16 elements for the E stage: 16 bytes of padding breaks
// the power-of-two stride between the 16 rows a b128 read touches.
template <int KC>
struct EStage {
  static constexpr int kPitch = 32 * KC + 8;
  uint16_t e[kStageRows][kPitch];
};

// Workgroup -> (column tile, row stage), XCD-aware: workgroups are dealt to
// the 8 XCDs round-robin by linear id, so the stages of one column tile are
// given consecutive slots on the same XCD and share its W2 tile in that L2.
__device__ __forceinline__ bool xcd_tile(int linear, int ncol_tiles, int nstages, int& col_tile,
                                         int& stage) {
  const int xcd = linear & 7;
  const int slot = linear >> 3;
  stage = slot % nstages;
  col_tile = (slot / nstages) * 8 + xcd;
  return col_tile < ncol_tiles;
}

__host__ __device__ inline int xcd_grid(int ncol_tiles, int nstages) {
  return 8 * nstages * ((ncol_tiles + 7) / 8);
}

// A-operand fragments of one wave's 64 columns (all r, in KC chunks of 32).
template <int KC>
__device__ __forceinline__ void load_w2_frags(const uint16_t* __restrict__ W2t, int r, int V,
                                              int n0, int lane, bf16x8 (&fr)[4][KC]) {
  const int a = lane & 15;
  const int kq = (lane >> 4) * 8;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int col = n0 + 16 * (a >> 2) + 4 * b + (a & 3);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const int k = 32 * kc + kq;
      if (col < V && k < r) {
        fr[b][kc] = *reinterpret_cast<const bf16x8*>(W2t + (size_t)col * r + k);
      } else {
        fr[b][kc] = bf16x8{};
      }
    }
  }
}

// Stage E rows W1[prev(row)] of rows [row0, row0 + 64) into LDS (zeros for
// rows past nrows, invalid previous tokens, or k >= r).  prev_of(row) returns
// the previous token of that row or -1.  All 256 threads take part.
template <int KC, typename PrevFn>
__device__ __forceinline__ void stage_e(EStage<KC>& st, const uint16_t* __restrict__ W1, int r,
                                        int V, int row0, int nrows, PrevFn prev_of) {
  constexpr int kVecPerRow = 4 * KC;  // 16-byte vectors per padded row
  for (int v = threadIdx.x; v < kStageRows * kVecPerRow; v += 256) {
    const int row = v / kVecPerRow;
    const int k = 8 * (v % kVecPerRow);
    const int g = row0 + row;
    u32x4 val = u32x4{0u, 0u, 0u, 0u};
    if (g < nrows && k < r) {
      const int prev = prev_of(g);
      if (prev >= 0 && prev < V)
        val = *reinterpret_cast<const u32x4*>(W1 + (size_t)prev * r + k);
    }
    *reinterpret_cast<u32x4*>(&st.e[row][k]) = val;
  }
}

// bias for 16 rows (group g of the stage) x the wave's 64 columns.
// acc[b][i] = bias[row 16g + l%16, column n0 + 16*(l/16) + 4b + i].
template <int KC>
__device__ __forceinline__ void mfma_group(const EStage<KC>& st, int g, int lane,
                                           const bf16x8 (&w2)[4][KC], f32x4 (&acc)[4]) {
  bf16x8 e[KC];
  const int row = 16 * g + (lane & 15);
  const int kq = (lane >> 4) * 8;
#pragma unroll
  for (int kc = 0; kc < KC; ++kc)
    e[kc] = *reinterpret_cast<const bf16x8*>(&st.e[row][32 * kc + kq]);
#pragma unroll
  for (int b = 0; b < 4; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
#pragma unroll
    for (int b = 0; b < 4; ++b)
      acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w2[b][kc], e[kc], acc[b], 0, 0, 0);
  }
}

// One bias value on the vector ALU (fp32 FMA in index order), used when a
// single column of a single row is re-evaluated (the sampling re-scan).
__device__ __forceinline__ float valu_bias(const uint16_t* __restrict__ w1row,
                                           const uint16_t* __restrict__ w2col, int r) {
  float s = 0.f;
  for (int k = 0; k < r; k += 8) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(w1row + k);
    const u32x4 b = *reinterpret_cast<const u32x4*>(w2col + k);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s = fmaf(__uint_as_float(a[e] << 16), __uint_as_float(b[e] << 16), s);
      s = fmaf(__uint_as_float(a[e] & 0xFFFF0000u), __uint_as_float(b[e] & 0xFFFF0000u), s);
    }
  }
  return s;
}

}  // namespace dspark
