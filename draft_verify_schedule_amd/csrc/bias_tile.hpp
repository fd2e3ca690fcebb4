// The rank-r Markov bias as an MFMA tile: for a stage of 128 rows (requests)
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

constexpr int kGroupsPerWG = 8;                  // 16-row MFMA groups per workgroup
constexpr int kStageRows = 16 * kGroupsPerWG;     // rows (requests) per workgroup / LDS stage
constexpr int kWaveCols = 64;    // vocabulary columns per wave (= one partial slice)
constexpr int kTileCols = 256;   // columns per workgroup (4 waves)

// LDS row pitch in bf16 elements for the E stage: 16 bytes of padding breaks
// the power-of-two stride between the 16 rows a b128 read touches.
// SPLIT: rows staged from fp32 values v (the RNN head's output parts) hold
// hi = fp16(v) in columns [0, 32 KC) and lo = fp16(v - hi) in [32 KC, 64 KC);
// both meet the same W2 fragment (converted to fp16, which holds every bf16
// weight of magnitude 2^-14 .. 2^15 exactly), on the fp16 MFMA.  hi + lo
// carries v to 2^-22 relative (plus 2^-25 absolute where lo is subnormal),
// where one bf16 operand would keep 2^-8 and a bf16 pair 2^-16.
// NR: rows of the stage (128, or 256 for the draft's two-stage sweep).
template <int KC, bool SPLIT = false, int NR = kStageRows>
struct EStage {
  static constexpr int kLo = 32 * KC;  // column of the lo half (SPLIT)
  static constexpr int kPitch = (SPLIT ? 64 : 32) * KC + 8;
  static constexpr int kRows = NR;
  uint16_t e[NR][kPitch];
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

// A-operand fragments of one wave's 64 columns (all r, in KC chunks of 32),
// through a buffer resource over W2 (column-major, V * r bf16): the per-lane
// part of the address is one VGPR, the block / chunk part is scalar.  Columns
// past V read as zero.  For k >= r the fragment holds the next column's
// weights; they meet zeros in E (staged as zero for k >= r) and add nothing.
struct W2Frags {
  rsrc_t rsrc;
  uint32_t lane_off;   // bytes: lane's column within a block and its k group
  uint32_t col_bytes;  // bytes per column (r * 2)
  uint32_t bytes;      // resource size
  __device__ __forceinline__ void setup(const uint16_t* W2t, int r, int V, int lane) {
    bytes = (uint32_t)V * (uint32_t)r * 2u;
    rsrc = make_rsrc(W2t, bytes);
    const int a = lane & 15;
    col_bytes = (uint32_t)r * 2u;
    lane_off = (uint32_t)(16 * (a >> 2) + (a & 3)) * col_bytes + (uint32_t)((lane >> 4) * 8) * 2u;
  }
  // FT: bf16x8 (W2 as given) or f16x8 (its fp16 copy, for SPLIT stages)
  template <int KC, typename FT>
  __device__ __forceinline__ void load(int n0, FT (&fr)[4][KC]) const {
    load_from<KC>((uint32_t)n0 * col_bytes, fr);
  }
  // valid = false: every offset is past the resource, the registers read as
  // zero and no memory is touched (wave-uniform select, no branch)
  template <int KC, typename FT>
  __device__ __forceinline__ void load_if(int n0, bool valid, FT (&fr)[4][KC]) const {
    load_from<KC>(valid ? (uint32_t)n0 * col_bytes : bytes, fr);
  }
  template <int KC, int K0 = 0, int K1 = KC, typename FT>
  __device__ __forceinline__ void load_from(uint32_t base, FT (&fr)[4][KC]) const {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
#pragma unroll
      for (int kc = K0; kc < K1; ++kc) {
        const uint32_t soff = base + (uint32_t)(4 * b) * col_bytes + (uint32_t)(64 * kc);
        fr[b][kc] = __builtin_bit_cast(FT, buffer_load16(rsrc, lane_off, soff));
      }
    }
  }
  // k chunks [K0, K1) only (valid = false: zeros, no memory access)
  template <int KC, int K0, int K1, typename FT>
  __device__ __forceinline__ void load_range_if(int n0, bool valid, FT (&fr)[4][KC]) const {
    load_from<KC, K0, K1>(valid ? (uint32_t)n0 * col_bytes : bytes, fr);
  }
};

// The same A-operand fragments from a copy of W2 rearranged once per call
// (w2_swizzle_kernel): for 64-column block blk, fragment f = b * KC + kc is
// 1 KB holding lane l's 16 bytes at 16 l, in the order the MFMA reads them.
// A wave's fragment load is then one contiguous kilobyte (8 cache lines)
// where the column-major W2 puts each lane's 16 bytes 16 lanes away from its
// neighbours in the same line (every lane a separate cache access).
struct W2SwzFrags {
  rsrc_t rsrc;
  uint32_t lane_off;   // 16 * lane
  uint32_t blk_bytes;  // 4 * KC * 1024
  uint32_t bytes;      // resource size
  __device__ __forceinline__ void setup(const uint16_t* W2s, int kc_count, int V, int lane) {
    blk_bytes = (uint32_t)(4 * kc_count) * 1024u;
    bytes = (uint32_t)((V + 63) / 64) * blk_bytes;
    rsrc = make_rsrc(W2s, bytes);
    lane_off = (uint32_t)lane * 16u;
  }
  template <int KC, int K0 = 0, int K1 = KC, typename FT>
  __device__ __forceinline__ void load_from(uint32_t base, FT (&fr)[4][KC]) const {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
#pragma unroll
      for (int kc = K0; kc < K1; ++kc)
        fr[b][kc] = __builtin_bit_cast(FT, buffer_load16(rsrc, lane_off, base + (uint32_t)(b * KC + kc) * 1024u));
    }
  }
  // n0: first column of the block (a multiple of 64)
  template <int KC, typename FT>
  __device__ __forceinline__ void load(int n0, FT (&fr)[4][KC]) const {
    load_from<KC>((uint32_t)(n0 / 64) * blk_bytes, fr);
  }
  template <int KC, typename FT>
  __device__ __forceinline__ void load_if(int n0, bool valid, FT (&fr)[4][KC]) const {
    load_from<KC>(valid ? (uint32_t)(n0 / 64) * blk_bytes : bytes, fr);
  }
  template <int KC, int K0, int K1, typename FT>
  __device__ __forceinline__ void load_range_if(int n0, bool valid, FT (&fr)[4][KC]) const {
    load_from<KC, K0, K1>(valid ? (uint32_t)(n0 / 64) * blk_bytes : bytes, fr);
  }
};

// Either layout chosen at run time: the fragment-ordered copy when the
// caller supplied one, else the column-major W2.  Both place fragment
// (b, kc) of the block starting at column n0 at a per-lane offset plus a
// wave-uniform offset linear in (n0 / 64, b, kc); only the strides differ.
struct W2AnyFrags {
  rsrc_t rsrc;
  uint32_t lane_off, blk_stride, b_stride, kc_stride, bytes;
  __device__ __forceinline__ void setup(const uint16_t* W2t, const uint16_t* W2s, int r, int V, int lane) {
    const int kc_count = (r + 31) / 32;
    if (W2s) {
      blk_stride = (uint32_t)(4 * kc_count) * 1024u;
      bytes = (uint32_t)((V + 63) / 64) * blk_stride;
      rsrc = make_rsrc(W2s, bytes);
      lane_off = (uint32_t)lane * 16u;
      b_stride = (uint32_t)kc_count * 1024u;
      kc_stride = 1024u;
    } else {
      const uint32_t col_bytes = (uint32_t)r * 2u;
      bytes = (uint32_t)V * col_bytes;
      rsrc = make_rsrc(W2t, bytes);
      const int a = lane & 15;
      lane_off = (uint32_t)(16 * (a >> 2) + (a & 3)) * col_bytes + (uint32_t)((lane >> 4) * 8) * 2u;
      blk_stride = 64u * col_bytes;
      b_stride = 4u * col_bytes;
      kc_stride = 64u;
    }
  }
  template <int KC, int K0 = 0, int K1 = KC, typename FT>
  __device__ __forceinline__ void load_from(uint32_t base, FT (&fr)[4][KC]) const {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
#pragma unroll
      for (int kc = K0; kc < K1; ++kc)
        fr[b][kc] = __builtin_bit_cast(FT, buffer_load16(rsrc, lane_off, base + (uint32_t)b * b_stride +
                                                                             (uint32_t)kc * kc_stride));
    }
  }
  // n0: first column of the block (a multiple of 64)
  template <int KC, typename FT>
  __device__ __forceinline__ void load(int n0, FT (&fr)[4][KC]) const {
    load_from<KC>((uint32_t)(n0 / 64) * blk_stride, fr);
  }
  template <int KC, int K0, int K1, typename FT>
  __device__ __forceinline__ void load_range_if(int n0, bool valid, FT (&fr)[4][KC]) const {
    load_from<KC, K0, K1>(valid ? (uint32_t)(n0 / 64) * blk_stride : bytes, fr);
  }
};

// Stage E rows W1[prev(row)] of rows [row0, row0 + 32 * waves) into LDS (zeros
// for rows past nrows, invalid previous tokens, or k >= r).  prev_of(row)
// returns the previous token of that row or -1.  Waves 0, 1, .. take 32 rows
// each (4 waves for a 128-row stage, 8 for a 256-row one); each load instruction covers two whole rows, 32
// lanes x 16 contiguous bytes per row, so one instruction touches 8 cache
// lines instead of 64.  Lane j reads the previous token of row j of its
// wave's 32 once; the token of each loaded row comes by a lane shuffle.
//
// Split in two so that a kernel can request other data (its first base
// logits and W2 fragments) between the W1 loads and the LDS stores: loads
// complete in order, so the stores then wait for the W1 rows only.
template <int KC>
struct EStageLoad {
  static constexpr int kChunks = 4 * KC;  // 16-byte vectors per padded row, <= 32
  static constexpr int kLoads = 16;       // two rows per load instruction
  u32x4 vals[kLoads];
  uint32_t valid;  // bit i: the row of load i has a valid token

  template <typename PrevFn>
  __device__ __forceinline__ void load(const uint16_t* __restrict__ W1, int r, int V, int row0, int nrows,
                                       PrevFn prev_of) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int c = lane & 31;
    const int g = row0 + 32 * wave + c;
    const int my_prev = (g < nrows) ? prev_of(g) : -1;
    const int k = 8 * c;
    const bool k_ok = c < kChunks && k < r;
    valid = 0;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int prev = __shfl(my_prev, 2 * i + (lane >> 5), 64);
      const bool ok = prev >= 0 && prev < V;
      valid |= (ok && k_ok) ? (1u << i) : 0u;
      vals[i] = *reinterpret_cast<const u32x4*>(W1 + (size_t)(ok ? prev : 0) * r + (k_ok ? k : 0));
    }
  }
  template <int NR>
  __device__ __forceinline__ void store(EStage<KC, false, NR>& st, int r) const {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int c = lane & 31;
    if (c < kChunks) {
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        const int row = 32 * wave + 2 * i + (lane >> 5);
        *reinterpret_cast<u32x4*>(&st.e[row][8 * c]) = ((valid >> i) & 1u) ? vals[i] : u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
};

template <int KC, typename PrevFn, int NR>
__device__ __forceinline__ void stage_e(EStage<KC, false, NR>& st, const uint16_t* __restrict__ W1, int r,
                                        int V, int row0, int nrows, PrevFn prev_of) {
  EStageLoad<KC> ld;
  ld.load(W1, r, V, row0, nrows, prev_of);
  ld.store(st, r);
}

// Round to nearest even, as raw bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// fp16 of f (round to nearest even) as raw bits.
__device__ __forceinline__ uint32_t f16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// Stage fp32 rows (width r, row stride r; 16-byte aligned, r % 4 == 0) as
// split hi/lo fp16 rows.  row_of(row) gives the source row or -1 (zeros);
// columns past r are zero.  Each wave takes 32 rows, 8 at a time: one
// 16-byte load per lane and row, 64 lanes per row.
template <int KC, typename RowFn>
__device__ __forceinline__ void stage_rows(EStage<KC, true>& st, const float* __restrict__ src, int r, int row0,
                                           int nrows, RowFn row_of) {
  static_assert(KC <= 8, "64 lanes x 4 values per row");
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c = 4 * lane;
  const bool c_ok = c < r && c < 32 * KC;
#pragma unroll
  for (int i0 = 0; i0 < 32; i0 += 8) {
    f32x4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int g = row0 + 32 * wave + i0 + i;
      const int src_row = g < nrows ? row_of(g) : -1;
      v[i] = (src_row >= 0 && c_ok) ? *reinterpret_cast<const f32x4*>(src + (size_t)src_row * r + c)
                                    : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = 32 * wave + i0 + i;
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const _Float16 h = (_Float16)v[i][e];
        hi[e] = (uint32_t)__builtin_bit_cast(uint16_t, h);
        lo[e] = f16_bits(v[i][e] - (float)h);
      }
      if (c < 32 * KC) {
        *reinterpret_cast<uint2*>(&st.e[row][c]) = make_uint2(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16));
        *reinterpret_cast<uint2*>(&st.e[row][EStage<KC, true>::kLo + c]) =
            make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
      }
    }
  }
}

// Byte offset of this lane's E fragment row within the stage (group 0,
// chunk 0).  Callers that loop over column blocks pass it through
// launder() once per block so that the compiler cannot hoist the (loop
// invariant) LDS reads of all groups out of the loop and keep them live.
template <int KC, bool SPLIT = false>
__device__ __forceinline__ int e_lane_offset(int lane) {
  return ((lane & 15) * EStage<KC, SPLIT>::kPitch + (lane >> 4) * 8) * 2;  // the pitch does not depend on NR
}

__device__ __forceinline__ int launder(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// bias for 16 rows (group g of the stage) x the wave's 64 columns.
// acc[b][i] = bias[row 16g + l%16, column n0 + 16*(l/16) + 4b + i].
// With ZERO = false the accumulators arrive holding the base logits of the
// same 16 x 64 tile, so the MFMAs leave base + bias in them directly.
// Only the k chunks [K0, K1) (K0 = 0, K1 = KC: the whole contraction); ZERO
// clears the accumulators first.
// SPLIT stages (fp16 W2 fragments, w2 of type f16x8) add the lo half of each
// chunk right after its hi half on the fp16 MFMA.
template <int KC, bool ZERO = true, int K0 = 0, int K1 = KC, bool SPLIT, int NR, typename FT>
__device__ __forceinline__ void mfma_group(const EStage<KC, SPLIT, NR>& st, int g, int lane,
                                           const FT (&w2)[4][KC], f32x4 (&acc)[4],
                                           int e_off = -1) {
  FT e[KC];
  FT el[SPLIT ? KC : 1];
  if (e_off < 0) e_off = e_lane_offset<KC, SPLIT>(lane);
  const char* base =
      reinterpret_cast<const char*>(&st.e[0][0]) + e_off + g * 16 * EStage<KC, SPLIT, NR>::kPitch * 2;
#pragma unroll
  for (int kc = K0; kc < K1; ++kc) {
    e[kc] = *reinterpret_cast<const FT*>(base + 64 * kc);
    if constexpr (SPLIT) el[kc] = *reinterpret_cast<const FT*>(base + 2 * EStage<KC, true>::kLo + 64 * kc);
  }
  if constexpr (ZERO) {
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int kc = K0; kc < K1; ++kc) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      if constexpr (SPLIT) {
        static_assert(sizeof(FT) == sizeof(f16x8), "fp16 fragments");
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(w2[b][kc], e[kc], acc[b], 0, 0, 0);
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(w2[b][kc], el[kc], acc[b], 0, 0, 0);
      } else {
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w2[b][kc], e[kc], acc[b], 0, 0, 0);
      }
    }
  }
}

// The 16 logits a lane needs for one group (16 consecutive columns n.. of one
// row), requested ahead of use.  Loads are unconditional (a masked vector is
// read from column 0 of a valid row instead) so that no branch or register
// copy sits between the request and its use; masking to -inf happens at
// unpack time.  bf16 vectors stay packed (8 registers).
template <typename T, bool VEC>
struct GroupLogits {
  float f[16];
  __device__ __forceinline__ void load(const T* __restrict__ row, int n, int V) {
#pragma unroll
    for (int e = 0; e < 16; ++e) f[e] = load_logit(row, (n + e < V) ? n + e : 0);
  }
  __device__ __forceinline__ void unpack(float out[16], int n, int V, bool live) const {
#pragma unroll
    for (int e = 0; e < 16; ++e) out[e] = (live && n + e < V) ? f[e] : -INFINITY;
  }
};

template <>
struct GroupLogits<float, true> {
  f32x4 w[4];
  __device__ __forceinline__ void load(const float* __restrict__ row, int n, int V) {
#pragma unroll
    for (int h = 0; h < 4; ++h) w[h] = *reinterpret_cast<const f32x4*>(row + ((n + 4 * h < V) ? n + 4 * h : 0));
  }
  __device__ __forceinline__ void unpack(float out[16], int n, int V, bool live) const {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const bool ok = live && n + 4 * h < V;
#pragma unroll
      for (int e = 0; e < 4; ++e) out[4 * h + e] = ok ? w[h][e] : -INFINITY;
    }
  }
};

template <>
struct GroupLogits<uint16_t, true> {
  u32x4 w[2];
  __device__ __forceinline__ void load(const uint16_t* __restrict__ row, int n, int V) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
      w[h] = *reinterpret_cast<const u32x4*>(row + ((n + 8 * h < V) ? n + 8 * h : 0));
  }
  __device__ __forceinline__ void unpack(float out[16], int n, int V, bool live) const {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const bool ok = live && n + 8 * h < V;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        out[8 * h + 2 * e] = ok ? __uint_as_float(w[h][e] << 16) : -INFINITY;
        out[8 * h + 2 * e + 1] = ok ? __uint_as_float(w[h][e] & 0xFFFF0000u) : -INFINITY;
      }
    }
  }
};

// Group logits through a buffer resource (16-byte aligned rows): per-lane
// offset in a VGPR, group / block offset scalar.
template <typename T>
struct GroupLogitsBuf;

template <>
struct GroupLogitsBuf<uint16_t> {
  u32x4 w[2];
  __device__ __forceinline__ void load(rsrc_t r, uint32_t voff, uint32_t soff) {
    w[0] = buffer_load16(r, voff, soff);
    w[1] = buffer_load16(r, voff, soff + 16u);
  }
  __device__ __forceinline__ void unpack(float out[16], int n, int V, bool live) const {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const bool ok = live && n + 8 * h < V;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        out[8 * h + 2 * e] = ok ? __uint_as_float(w[h][e] << 16) : -INFINITY;
        out[8 * h + 2 * e + 1] = ok ? __uint_as_float(w[h][e] & 0xFFFF0000u) : -INFINITY;
      }
    }
  }
  // all 16 columns in range and the row live
  __device__ __forceinline__ void unpack(float out[16]) const {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        out[8 * h + 2 * e] = __uint_as_float(w[h][e] << 16);
        out[8 * h + 2 * e + 1] = __uint_as_float(w[h][e] & 0xFFFF0000u);
      }
    }
  }
};

template <>
struct GroupLogitsBuf<float> {
  u32x4 w[4];
  __device__ __forceinline__ void load(rsrc_t r, uint32_t voff, uint32_t soff) {
#pragma unroll
    for (int h = 0; h < 4; ++h) w[h] = buffer_load16(r, voff, soff + 16u * h);
  }
  __device__ __forceinline__ void unpack(float out[16], int n, int V, bool live) const {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const bool ok = live && n + 4 * h < V;
#pragma unroll
      for (int e = 0; e < 4; ++e) out[4 * h + e] = ok ? __uint_as_float(w[h][e]) : -INFINITY;
    }
  }
  __device__ __forceinline__ void unpack(float out[16]) const {
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e) out[4 * h + e] = __uint_as_float(w[h][e]);
  }
};

// Bias values on the vector ALU, used when the 64 columns of one slice of one
// row are re-evaluated (the sampling re-scans): lane l owns column col and
// accumulates sum_k W1[prev, k] * W2[k, col] over k in [k0, k0 + 64) in fp32
// FMAs in index order.  All sixteen 16-byte loads of a chunk are requested
// before the first FMA, so a chunk costs one memory round trip.  Requires
// r % 8 == 0; k >= r contributes nothing.
__device__ __forceinline__ float bias_chunk64(const uint16_t* __restrict__ w1row,
                                             const uint16_t* __restrict__ w2col, int k0, int r) {
  u32x4 av[8], bv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int k = k0 + 8 * i;
    const bool ok = k < r;  // uniform; the load is unconditional (address clamped) so that
    const int kk = ok ? k : 0;  // every load of the chunk stays in one basic block
    const u32x4 x = *reinterpret_cast<const u32x4*>(w1row + kk);
    const u32x4 y = *reinterpret_cast<const u32x4*>(w2col + kk);
    av[i] = ok ? x : u32x4{0u, 0u, 0u, 0u};
    bv[i] = ok ? y : u32x4{0u, 0u, 0u, 0u};
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s = fmaf(__uint_as_float(av[i][e] << 16), __uint_as_float(bv[i][e] << 16), s);
      s = fmaf(__uint_as_float(av[i][e] & 0xFFFF0000u), __uint_as_float(bv[i][e] & 0xFFFF0000u), s);
    }
  }
  return s;
}

// bias_chunk64 with W2 read from its fragment-ordered copy (W2SwzFrags
// layout): w2blk is the slice's 64-column block, c the lane's column in it
// (0..63).  Same products in the same order; for a wave the loads of one k
// step are four runs of 16 consecutive 16-byte entries instead of 64
// scattered ones.
__device__ __forceinline__ float bias_chunk64_swz(const uint16_t* __restrict__ w1row, const char* __restrict__ w2blk,
                                                 int c, int k0, int r, int kc_count) {
  const int a = 4 * (c >> 4) + (c & 3);  // MFMA A-row of column c ...
  const int b = (c >> 2) & 3;            // ... in block b
  u32x4 av[8], bv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int k = k0 + 8 * i;
    const bool ok = k < r;
    const int kk = ok ? k : 0;
    const int f = b * kc_count + (kk >> 5);
    const u32x4 x = *reinterpret_cast<const u32x4*>(w1row + kk);
    const u32x4 y = *reinterpret_cast<const u32x4*>(w2blk + (size_t)f * 1024 + (16 * ((kk >> 3) & 3) + a) * 16);
    av[i] = ok ? x : u32x4{0u, 0u, 0u, 0u};
    bv[i] = ok ? y : u32x4{0u, 0u, 0u, 0u};
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s = fmaf(__uint_as_float(av[i][e] << 16), __uint_as_float(bv[i][e] << 16), s);
      s = fmaf(__uint_as_float(av[i][e] & 0xFFFF0000u), __uint_as_float(bv[i][e] & 0xFFFF0000u), s);
    }
  }
  return s;
}

// The same over an fp32 row (the RNN head's output part o): lane l owns
// column col and accumulates sum_k o[k] * W2[k, col] over k in [k0, k0 + 64)
// in fp32 FMAs in index order.  Requires r % 8 == 0.
__device__ __forceinline__ float bias_chunk64_rows(const float* __restrict__ orow,
                                                  const uint16_t* __restrict__ w2col, int k0, int r) {
  f32x4 av[16];
  u32x4 bv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int k = k0 + 8 * i;
    const bool ok = k < r;
    const int kk = ok ? k : 0;
    const f32x4 x0 = *reinterpret_cast<const f32x4*>(orow + kk);
    const f32x4 x1 = *reinterpret_cast<const f32x4*>(orow + kk + 4);
    const u32x4 y = *reinterpret_cast<const u32x4*>(w2col + kk);
    av[2 * i] = ok ? x0 : f32x4{0.f, 0.f, 0.f, 0.f};
    av[2 * i + 1] = ok ? x1 : f32x4{0.f, 0.f, 0.f, 0.f};
    bv[i] = ok ? y : u32x4{0u, 0u, 0u, 0u};
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a0 = av[2 * i + e / 2][2 * (e % 2)];
      const float a1 = av[2 * i + e / 2][2 * (e % 2) + 1];
      s = fmaf(a0, __uint_as_float(bv[i][e] << 16), s);
      s = fmaf(a1, __uint_as_float(bv[i][e] & 0xFFFF0000u), s);
    }
  }
  return s;
}

// One wave: the chunks of 64 in order, summed left to right.
__device__ __forceinline__ float valu_bias(const uint16_t* __restrict__ w1row,
                                           const uint16_t* __restrict__ w2col, int r) {
  float s = 0.f;
  for (int k0 = 0; k0 < r; k0 += 64) s += bias_chunk64(w1row, w2col, k0, r);
  return s;
}

__device__ __forceinline__ float valu_bias_rows(const float* __restrict__ orow,
                                                const uint16_t* __restrict__ w2col, int r) {
  float s = 0.f;
  for (int k0 = 0; k0 < r; k0 += 64) s += bias_chunk64_rows(orow, w2col, k0, r);
  return s;
}

// Four waves of a workgroup (r <= 256): wave w takes the chunk starting at
// 64 w; the four chunk sums are combined in chunk order through LDS
// (part[256], all waves must call it).  Returns the bias on every wave.
// With orow set, the bias input is that fp32 row instead of w1row.
// w2blk (Markov head only): the slice's block of the fragment-ordered W2,
// read instead of w2col.
__device__ __forceinline__ float valu_bias_4waves(const uint16_t* __restrict__ w1row, const float* __restrict__ orow,
                                                  const uint16_t* __restrict__ w2col, int r, bool ok,
                                                  int wave, int lane, float* part,
                                                  const char* __restrict__ w2blk = nullptr) {
  float v = 0.f;
  if (ok) {
    if (orow) v = bias_chunk64_rows(orow, w2col, 64 * wave, r);
    else if (w2blk) v = bias_chunk64_swz(w1row, w2blk, lane, 64 * wave, r, (r + 31) / 32);
    else v = bias_chunk64(w1row, w2col, 64 * wave, r);
  }
  part[wave * 64 + lane] = v;
  __syncthreads();
  return ((part[lane] + part[64 + lane]) + part[128 + lane]) + part[192 + lane];
}

// Bias of one column per lane, all of r <= 256 (r % 8 == 0), for the draft's
// one-wave re-scan.  The bias input row is the same for the whole wave and has
// been staged in LDS by the caller, zero-filled to 256 values (row: 32 entries
// of 8 bf16 W1 weights, or with ROWS 64 entries of 4 fp32 values of the RNN
// head's output part).  Each lane streams its column of W2 through the buffer
// resource w2 (column-major: the column's r weights at byte offset off0; swz:
// the lane's entries of the slice's fragment-ordered block at off0); every
// load is issued before the first product, and a load past r (or with !ok)
// gets an offset past the resource and reads zeros.  Chunks of 64 in k
// order, the chunk sums added left to right; within a chunk the W1 bias takes
// packed bf16 dot products of the pairs (k, k + 1) in index order
// (v_dot2c_f32_bf16, fp32 accumulation), the RNN head's fp32 row fp32 FMAs in
// index order.  Zero terms past r leave the sums unchanged.  !ok gives 0.
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;

constexpr int kMaxRankRow = 64;  // 16-byte entries of a staged bias row: r <= 256 fp32 values

template <bool ROWS>
__device__ __forceinline__ float lane_bias_staged(const u32x4* row, rsrc_t w2, uint32_t w2_bytes, uint32_t off0,
                                                  bool swz, int r, bool ok, int lane) {
  u32x4 bv[32];
  const int a = 4 * (lane >> 4) + (lane & 3);  // swz: MFMA A-row of the lane's column ...
  const int b = (lane >> 2) & 3;               // ... in block b
  const int kc_count = (r + 31) / 32;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int k = 8 * i;
    const uint32_t off = swz ? off0 + (uint32_t)(b * kc_count + (k >> 5)) * 1024u + (uint32_t)(16 * ((k >> 3) & 3) + a) * 16u
                             : off0 + (uint32_t)k * 2u;
    bv[i] = buffer_load16(w2, (ok && k < r) ? off : w2_bytes, 0u);
  }
  __builtin_amdgcn_sched_barrier(0);  // every load requested before the first product
  float c[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float s = 0.f;
#pragma unroll
    for (int i = 8 * j; i < 8 * j + 8; ++i) {
      if constexpr (ROWS) {
        const u32x4 p0 = row[2 * i];
        const u32x4 p1 = row[2 * i + 1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const u32x4& pa = e < 2 ? p0 : p1;
          s = fmaf(__uint_as_float(pa[2 * (e % 2)]), __uint_as_float(bv[i][e] << 16), s);
          s = fmaf(__uint_as_float(pa[2 * (e % 2) + 1]), __uint_as_float(bv[i][e] & 0xFFFF0000u), s);
        }
      } else {
        // bf16 pairs straight into the packed dot product (k, k + 1 per dword)
        const u32x4 av = row[i];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // the dwords go through scalars: a bit cast of a vector element
          // expression is not reliable here
          const uint32_t x = av[e], y = bv[i][e];
          s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, x), __builtin_bit_cast(bf16x2_t, y), s, false);
        }
      }
    }
    c[j] = s;
  }
  return ok ? ((c[0] + c[1]) + c[2]) + c[3] : 0.f;
}

}  // namespace dspark
