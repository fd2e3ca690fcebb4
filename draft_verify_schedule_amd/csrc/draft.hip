// Sequential Markov-head draft (DSpark paper, section 3.1: parallel stage
// gives base logits U_k; the sequential stage adds the first-order transition
// bias W1[x_{k-1}] W2 and samples left to right; "Speculative decoding, from
// zero to DSpark", section 6).
//
// Per position k (sequential: x_k feeds the next gather) two launches:
//   draft_partials  one HBM pass over U_k fused with the bias MFMA tile:
//                   per (request, 64-column slice) the softmax partial
//                   (max, sum exp2(z - max)) of z = (U_k + bias) * log2(e)/T,
//                   or (max, first argmax) when greedy.  The bias is never
//                   written to memory.
//   draft_locate    one wave per request: merges the slice partials into the
//                   normaliser, finds the slice where the CDF crosses u * S,
//                   re-evaluates that slice's 64 logits and picks the token.
// With the RNN head (same paper, section 3.1, RNN head) a third launch comes
// first at each position, rnn_step, which leaves the head's output part o_k
// for every request; the bias is then o_k W2 (o_k staged as split bf16 rows)
// instead of W1[x_{k-1}] W2.
#include <algorithm>
#include <type_traits>

#include "bias_tile.hpp"
#include "launch.hpp"
#include "rnn.hpp"

namespace dspark {

constexpr int kPersistentWGs = 256;  // one per CU on 256 CUs
constexpr int kDraftWaves = 8;       // waves per draft workgroup: two per SIMD, one E stage per CU

struct DraftArgs {
  const void* U;           // [B, K, V]
  const uint16_t* W1;      // [V, r] bf16
  const uint16_t* W2t;     // column-major W2: [V, r] bf16
  const int32_t* prev;     // previous token of request b at prev[b * prev_stride]
  int prev_stride;
  int B, K, V, r, k;       // k: 1-based position
  float c2;                // log2(e) / T (1 when greedy)
  float2* part;            // [B, nslices]
  int nslices;             // ceil(V / 64)
  int ncol_tiles, nstages;
  uint64_t seed, step;
  int32_t* x_out;
  float* q_out;
  float* lse_out;
  const float* O;          // RNN head: output parts [B, K, r] fp32, row b * K + k - 1 (else null)
  const uint16_t* W2h;     // RNN head: fp16 copy of W2t
  const uint16_t* W2s;     // Markov head: W2t rearranged into MFMA fragment order (w2_swizzle_kernel)
};

// Epilogue of one group: z = base logits + bias for 16 consecutive columns of
// one row per lane; the four lanes sharing a row (l, l^16, l^32, l^48) cover the
// wave's 64-column slice.  Returns, on all four lanes, the slice's (scaled
// max, sum exp2) or (max, first argmax as int bits).  MASKED: columns >= V
// are excluded; without it every column of the slice is in range.
template <bool GREEDY, bool MASKED>
__device__ __forceinline__ float2 slice_values(const float (&z)[16], int cbase, int V, float c2) {
  if constexpr (GREEDY) {
    float m = -INFINITY;
    int idx = -1;
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if ((!MASKED || cbase + e < V) && (idx < 0 || z[e] > m)) {
        m = z[e];
        idx = cbase + e;
      }
    {
      float ma, mb;
      int ia, ib;
      row_pair16(m, ma, mb);
      row_pair16(idx, ia, ib);
      merge_argmax(ma, ia, mb, ib);
      row_pair32(ma, m, mb);
      row_pair32(ia, idx, ib);
      merge_argmax(m, idx, mb, ib);
    }
    return make_float2(m, __int_as_float(idx));
  } else {
    float m = z[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) m = fmaxf(m, z[e]);
    m = rows_max(m);
    const float mc = m * c2;
    // branch-free: a slice with no finite logit (mc = -inf) subtracts
    // -FLT_MAX instead, so its terms are exp2(-inf) = 0 and it reports
    // (-inf, 0); any other slice subtracts its own scaled maximum
    const float base = max_arith(mc, -FLT_MAX);
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) s += fast_exp2(fmaf(z[e], c2, -base));
    s = rows_sum(s);
    return make_float2(mc, s);
  }
}

// Base-logit access of the fused pass.  Aligned rows (VEC) go through a
// buffer resource: the lane's row-within-group and column offset is one VGPR,
// the group and block offsets are scalar.  Rows past B read as zero (past the
// resource) and are masked at unpack.  Unaligned rows use plain loads.
template <typename UT, bool VEC>
struct UAccess;

template <typename UT>
struct UAccess<UT, true> {
  using Buf = GroupLogitsBuf<UT>;
  rsrc_t rsrc;
  uint32_t lane_off;
  uint32_t bytes;      // resource size
  uint64_t row_bytes;  // K * V * sizeof(UT): request stride
  __device__ __forceinline__ void setup(const DraftArgs& a, int lane) {
    const UT* base = reinterpret_cast<const UT*>(a.U) + (size_t)(a.k - 1) * a.V;
    const uint64_t total = ((uint64_t)a.B * a.K * a.V - (uint64_t)(a.k - 1) * a.V) * sizeof(UT);
    bytes = (uint32_t)total;
    rsrc = make_rsrc(base, bytes);
    row_bytes = (uint64_t)a.K * a.V * sizeof(UT);
    lane_off = (uint32_t)((uint64_t)(lane & 15) * row_bytes + (uint64_t)(16 * (lane >> 4)) * sizeof(UT));
  }
  __device__ __forceinline__ uint32_t offset(int row, int blk) const {
    return (uint32_t)((uint64_t)row * row_bytes + (uint64_t)blk * kWaveCols * sizeof(UT));
  }
  __device__ __forceinline__ void load(Buf& b, int row, int blk) const { b.load(rsrc, lane_off, offset(row, blk)); }
  // valid = false: offset past the resource, zeros, no memory access
  __device__ __forceinline__ void load_if(Buf& b, int row, int blk, bool valid) const {
    b.load(rsrc, lane_off, valid ? offset(row, blk) : bytes);
  }
};

template <typename UT>
struct UAccess<UT, false> {
  using Buf = GroupLogits<UT, false>;
  const UT* U;
  int B, K, V, k, lane;
  __device__ __forceinline__ void setup(const DraftArgs& a, int lane_) {
    U = reinterpret_cast<const UT*>(a.U);
    B = a.B;
    K = a.K;
    V = a.V;
    k = a.k;
    lane = lane_;
  }
  __device__ __forceinline__ void load(Buf& b, int row, int blk) const {
    const int rr = row + (lane & 15);
    const UT* p = U + ((size_t)(rr < B ? rr : 0) * K + (k - 1)) * V;
    b.load(p, blk * kWaveCols + 16 * (lane >> 4), V);
  }
};

// bf16 base logits of one 16-row group read coalesced: lane l takes the 16
// bytes at 16 (l % 8) of row l / 8 (w[0], rows 0..7 of the group) and of row
// 8 + l / 8 (w[1]), so each load instruction covers 8 whole 128-byte row
// segments.  The MFMA layout instead wants lane l to hold 32 bytes of row
// l % 16, which puts a row segment's four pieces 16 lanes apart and makes
// every lane a separate cache access; the sweep moves the data between the
// two layouts through LDS.  Offsets past the resource read as zero.
struct UCoal {
  rsrc_t rsrc;
  uint32_t lane_off;
  uint32_t bytes;
  uint64_t row_bytes;
  __device__ __forceinline__ void setup(const DraftArgs& a, int lane) {
    const uint16_t* base = reinterpret_cast<const uint16_t*>(a.U) + (size_t)(a.k - 1) * a.V;
    bytes = (uint32_t)(((uint64_t)a.B * a.K * a.V - (uint64_t)(a.k - 1) * a.V) * 2u);
    rsrc = make_rsrc(base, bytes);
    row_bytes = (uint64_t)a.K * a.V * 2u;
    lane_off = (uint32_t)((uint64_t)(lane >> 3) * row_bytes + (uint64_t)(lane & 7) * 16u);
  }
  __device__ __forceinline__ void load_if(GroupLogitsBuf<uint16_t>& b, int row, int blk, bool valid) const {
    const uint32_t off = (uint32_t)((uint64_t)row * row_bytes + (uint64_t)blk * kWaveCols * 2u);
    const uint32_t off8 = (uint32_t)((uint64_t)(row + 8) * row_bytes + (uint64_t)blk * kWaveCols * 2u);
    // each base logit is read once per call: non-temporal, so that the
    // stream does not displace W2, which the next position reads again
    b.w[0] = buffer_load16_nt(rsrc, lane_off, valid ? off : bytes);
    b.w[1] = buffer_load16_nt(rsrc, lane_off, valid ? off8 : bytes);
  }
};

// Persistent workgroups, one per CU: 8 waves (two per SIMD), 128 rows (8
// MFMA groups of 16), and a contiguous range of 64-column blocks.  The W1
// rows of the 128 requests are staged in LDS once (by waves 0..3) and shared
// by all 8 waves; each wave sweeps blocks of the range (its first by index,
// the rest claimed in order), holding one block's W2 fragments in registers
// for all 8 groups.  One workgroup per CU rather than two of 4 waves: the CU
// holds one E stage, so the split stages of the RNN head (133 KB) also run
// two waves per SIMD.
//
// FULL (a stage of 128 live rows, 16-byte aligned rows): the complete blocks
// are swept by a software pipeline with no branches: several groups of base
// logits are in flight (also across block boundaries), group g+1's MFMAs are
// issued before group g's epilogue, and the next block's W2 fragments are
// requested as soon as the last MFMA of the current block has issued.  Loads
// that have no block to read and the stores of lanes 16..63 get offsets past
// their buffer resource (no memory access).  The block holding the column
// tail (V not a multiple of 64) and partial stages take the plain path.
// ROWS: the bias inputs are the fp32 rows a.O (RNN head) instead of gathered
// W1 rows.
// G: 16-row groups per stage (8, or 16 for the bf16 Markov sweep of full
// stage pairs: 256 rows share each W2 block loaded into a wave's registers,
// halving the W2 reloads per base logit; the E stage then takes 135 KB of
// LDS and the wave's base-logit tile is single-buffered).
template <typename UT, bool VEC, int KC, bool GREEDY, bool FULL, bool ROWS, int G = kGroupsPerWG>
__global__ __launch_bounds__(kDraftWaves * 64) __attribute__((amdgpu_waves_per_eu(2)))
void draft_partials_kernel(DraftArgs a, int stage0, int nstages) {
  static_assert(!FULL || VEC, "the pipelined sweep reads through buffer resources");
  static_assert(G == kGroupsPerWG || (FULL && !ROWS && KC > 0), "256-row stages: full bf16 Markov stages only");
  constexpr int KCs = KC > 0 ? KC : 1;
  constexpr int kRows = 16 * G;
  int split, stage;
  if (!xcd_tile(blockIdx.x, a.ncol_tiles, nstages, split, stage)) return;
  stage += stage0;
  const int lane = threadIdx.x & 63;
  const int wave = wave_index();
  const int row0 = stage * kRows;
  const int ngroups = min(G, (a.B - row0 + 15) / 16);
  const int nblocks = (a.V + kWaveCols - 1) / kWaveCols;
  const int blk_begin = (int)((int64_t)split * nblocks / a.ncol_tiles);
  const int blk_end = (int)((int64_t)(split + 1) * nblocks / a.ncol_tiles);
  auto row_of = [&](int g) { return row0 + 16 * g + (lane & 15); };
  auto row_live = [&](int g) { return row_of(g) < a.B; };
  const int lane_col = 16 * (lane >> 4);
  // blocks [blk_begin, blk_stop) of a full stage are swept by the pipeline
  const int blk_stop = FULL ? min(blk_end, a.V / kWaveCols) : blk_begin;
  int blk = blk_begin + wave;

  // Prologue, in request order: the previous tokens and their W1 rows (they
  // gate the first MFMA through the LDS stage), then the first groups of
  // base logits and the first block's W2 fragments; the LDS stores of the E
  // stage wait for the W1 rows only.
  __shared__ EStage<KCs, ROWS, kRows> st;
  // Blocks of the pipelined sweep after each wave's first are handed out in
  // order from this counter, so the eight waves of the workgroup finish
  // within a block of each other (a static split gives some waves one block
  // more than others).
  __shared__ int blk_next;
  if constexpr (FULL) {
    if (threadIdx.x == 0) blk_next = blk_begin + kDraftWaves;
  }
  EStageLoad<KCs> eld;
  constexpr int kStageWaves = kRows / 32;  // 32 rows gathered per wave
  if constexpr (KC > 0 && !ROWS) {
    const int32_t* prev = a.prev;
    const int stride = a.prev_stride;
    if (wave < kStageWaves) eld.load(a.W1, a.r, a.V, row0, a.B, [&](int g) { return prev[(size_t)g * stride]; });
  }

  UAccess<UT, VEC> ua;
  ua.setup(a, lane);
  // groups of base logits in flight per wave: 8 registers per packed bf16 group, 16 per fp32
  constexpr int kPrefetch = (FULL && sizeof(UT) == 2) ? 4 : 1;
  typename UAccess<UT, VEC>::Buf buf[kPrefetch];
  // UX: full bf16 stages of the Markov head load their base logits coalesced
  // (UCoal) and pass each group through this wave's LDS tile (row pitch 144
  // bytes, conflict-free for the MFMA-layout reads): two tiles, two groups
  // ahead of use (128-row stages), or one tile, one group ahead (256-row
  // stages, whose E stage leaves room for one)
  constexpr bool UX = FULL && !ROWS && std::is_same_v<UT, uint16_t>;
  constexpr int NT = G == kGroupsPerWG ? 2 : 1;
  static_assert(UX || NT == 2, "single-tile pipeline: coalesced bf16 loads only");
  __shared__ u32x4 utile[UX ? kDraftWaves : 1][NT][16 * 9];
  UCoal uc;
  if constexpr (FULL) {
    if constexpr (UX) uc.setup(a, lane);
#pragma unroll
    for (int g = 0; g < kPrefetch; ++g) {
      if constexpr (UX) uc.load_if(buf[g], row0 + 16 * g, blk, blk < blk_stop);
      else ua.load_if(buf[g], row0 + 16 * g, blk, blk < blk_stop);
    }
  }

  std::conditional_t<ROWS, f16x8, bf16x8> w2[4][KCs];
  // fragment-ordered W2: its fp16 copy for the RNN head's split stages
  W2SwzFrags wf;
  if constexpr (KC > 0) {
    wf.setup(ROWS ? a.W2h : a.W2s, KC, a.V, lane);
    if constexpr (FULL) wf.template load_if<KC>(blk * kWaveCols, blk < blk_stop, w2);
    if constexpr (ROWS) {
      const int K = a.K, k = a.k;
      if (wave < 4) stage_rows<KC>(st, a.O, a.r, row0, a.B, [&](int g) { return g * K + k - 1; });
    } else {
      if (wave < kStageWaves) eld.store(st, a.r);
    }
    __syncthreads();
  }

  if constexpr (FULL && KC == 0) __syncthreads();  // blk_next

  if constexpr (FULL) {
    const uint32_t part_bytes = (uint32_t)((uint64_t)a.B * a.nslices * sizeof(float2));
    const int4v prs = raw_rsrc_words(a.part, part_bytes);
    const uint32_t row_bytes = (uint32_t)a.nslices * (uint32_t)sizeof(float2);
    const uint32_t st_voff = lane < 16 ? (uint32_t)lane * row_bytes : part_bytes;
    // Group h's base logits sit in buf[h % kPrefetch] until they seed h's
    // accumulators (one step before h's epilogue); the freed slot is refilled
    // kPrefetch groups ahead.
    static_assert(G % kPrefetch == 0, "ring");
    // the next block is claimed at the start of the current one: its base
    // logits and W2 fragments are requested during the current block
    auto claim = [&]() {
      int v = 0;
      if (lane == 0) v = atomicAdd(&blk_next, 1);
      return __builtin_amdgcn_readfirstlane(v);
    };
    // UX: group h (of the block, h >= G: of the next one) goes from ring slot
    // h % kPrefetch into tile h % NT before its MFMAs (xwrite), and comes back
    // in the MFMA layout one step before them (xread); the slot is refilled
    // with group h + kPrefetch as soon as it is written out.  LDS operations
    // of one wave complete in order, so no barrier is needed, and with one
    // tile a group is written only after the previous one has been read.
    auto xwrite = [&](int h) {
      if constexpr (UX) {
        utile[wave][h % NT][(lane >> 3) * 9 + (lane & 7)] = buf[h % kPrefetch].w[0];
        utile[wave][h % NT][(8 + (lane >> 3)) * 9 + (lane & 7)] = buf[h % kPrefetch].w[1];
      }
    };
    auto xread = [&](int h, float (&u)[16]) {
      if constexpr (UX) {
        GroupLogitsBuf<uint16_t> t;
        t.w[0] = utile[wave][h % NT][(lane & 15) * 9 + 2 * (lane >> 4)];
        t.w[1] = utile[wave][h % NT][(lane & 15) * 9 + 2 * (lane >> 4) + 1];
        t.unpack(u);
      }
    };
    if constexpr (UX) {
      xwrite(0);
      uc.load_if(buf[0], row0 + 16 * kPrefetch, blk, blk < blk_stop);
      if constexpr (NT == 2) {
        xwrite(1);
        uc.load_if(buf[1], row0 + 16 * (kPrefetch + 1), blk, blk < blk_stop);
      }
    }
    while (blk < blk_stop) {
      const int cbase = blk * kWaveCols + lane_col;
      const int nxt = claim();
      const bool has_next = nxt < blk_stop;
      const int e_off = launder(e_lane_offset<KCs, ROWS>(lane));
      auto refill = [&](int h) {  // slot h % kPrefetch now takes group h (maybe of the next block)
        if constexpr (UX) {
          if (h < G) uc.load_if(buf[h % kPrefetch], row0 + 16 * h, blk, true);
          else uc.load_if(buf[h % kPrefetch], row0 + 16 * (h - G), nxt, has_next);
        } else {
          if (h < G) ua.load(buf[h % kPrefetch], row0 + 16 * h, blk);
          else ua.load_if(buf[h % kPrefetch], row0 + 16 * (h - G), nxt, has_next);
        }
      };
      f32x4 acc[4];
      {
        float u[16];
        if constexpr (UX) {
          xread(0, u);
          if constexpr (NT == 1) {  // one tile: group 1 goes in once group 0 is out
            xwrite(1);
            refill(1 + kPrefetch);
          }
        } else {
          buf[0].unpack(u);
          refill(kPrefetch);
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[b] = f32x4{u[4 * b], u[4 * b + 1], u[4 * b + 2], u[4 * b + 3]};
        if constexpr (KC > 0) mfma_group<KC, false>(st, 0, lane, w2, acc, e_off);
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float z[16];
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i) z[4 * b + i] = acc[b][i];
        if (g + 1 < G) {
          float u[16];
          if constexpr (UX) {
            xread(g + 1, u);
          } else {
            buf[(g + 1) % kPrefetch].unpack(u);
            refill(g + 1 + kPrefetch);
          }
#pragma unroll
          for (int b = 0; b < 4; ++b) acc[b] = f32x4{u[4 * b], u[4 * b + 1], u[4 * b + 2], u[4 * b + 3]};
          if constexpr (KC > 0) {
            if (g + 2 < G) {
              mfma_group<KC, false>(st, g + 1, lane, w2, acc, e_off);
            } else {
              // last group of the block: the first half of the next block's W2
              // fragments is requested as soon as the MFMAs reading those
              // registers have issued, the second half after the rest
              constexpr int KH = KC / 2;
              mfma_group<KC, false, 0, KH>(st, g + 1, lane, w2, acc, e_off);
              __builtin_amdgcn_sched_barrier(0);
              wf.template load_range_if<KC, 0, KH>(nxt * kWaveCols, has_next, w2);
              __builtin_amdgcn_sched_barrier(0);
              mfma_group<KC, false, KH, KC>(st, g + 1, lane, w2, acc, e_off);
            }
          }
        } else if constexpr (KC > 0) {
          wf.template load_range_if<KC, KC / 2, KC>(nxt * kWaveCols, has_next, w2);
        }
        if constexpr (UX) {
          if (NT == 2 || g + 2 <= G) {  // one tile: the next block's group 1 waits for its group 0's read
            xwrite(g + 2);
            refill(g + 2 + kPrefetch);
          }
        }
        const float2 v = slice_values<GREEDY, false>(z, cbase, a.V, a.c2);
        buffer_store8_untracked(prs, v, st_voff, (uint32_t)(row0 + 16 * g) * row_bytes + (uint32_t)blk * 8u);
      }
      blk = nxt;
    }
  }

  // plain path: partial stages, and the column-tail block of a full stage
  // (claimed by exactly one wave: blk_stop is the only block of the range
  // past the pipelined ones)
  for (; blk < blk_end; blk += kDraftWaves) {
    const int cbase = blk * kWaveCols + lane_col;
    float2* part = a.part + blk;
    if constexpr (KC > 0) wf.template load<KC>(blk * kWaveCols, w2);
    for (int g = 0; g < ngroups; ++g) {
      typename UAccess<UT, VEC>::Buf one;
      ua.load(one, row0 + 16 * g, blk);
      float z[16];
      one.unpack(z, cbase, a.V, row_live(g));
      if constexpr (KC > 0) {
        f32x4 acc[4];
        mfma_group<KC>(st, g, lane, w2, acc, launder(e_lane_offset<KC, ROWS>(lane)));
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i) z[4 * b + i] += acc[b][i];
      }
      const float2 v = slice_values<GREEDY, true>(z, cbase, a.V, a.c2);
      if (row_live(g) && lane < 16) part[(size_t)row_of(g) * a.nslices] = v;
    }
  }
}

// One wave per request.  Lane l owns the contiguous run of slices
// [l * per, (l + 1) * per), per = ceil(nslices / 64), read once into
// registers (rows of more than 64 * kLocRun slices re-read their runs).  Wave
// reductions give M = max of the slices' scaled maxima and each run's mass in
// fp64; an fp64 wave scan of the run masses finds the lane whose run holds
// the crossing of u * S; every lane walks its own run and the owner's
// crossing is broadcast; then each lane re-evaluates one of the chosen
// slice's 64 logits and a wave scan of their masses picks the token.  No
// barrier and two dependent memory round trips (the partials, then the
// slice's base logits and W2 block).
constexpr int kLocRun = 40;

template <typename UT, bool GREEDY>
__global__ __launch_bounds__(64) void draft_locate_kernel(DraftArgs a) {
  const int lane = threadIdx.x;
  const int b = blockIdx.x;
  const size_t out = (size_t)b * a.K + (a.k - 1);
  const int prev = a.prev[(size_t)b * a.prev_stride];
  const float2* part = a.part + (size_t)b * a.nslices;
  const int ns = a.nslices;
  const int per = (ns + 63) / 64;
  const int s0 = min(ns, lane * per);
  const int s1 = min(ns, s0 + per);
  const bool in_regs = per <= kLocRun;
  // the bias input row of the re-scan (W1[prev], or the RNN head's output
  // part), the same for the whole wave, is staged in LDS while the partials
  // are in flight
  __shared__ u32x4 sh_row[kMaxRankRow];
  const bool prev_ok = prev >= 0 && prev < a.V;
  float2 p[kLocRun];
  if (in_regs) {
    // every load is issued (no branch): slots past the lane's run read zeros
    // from past the end of the row's resource, a slice with no mass
    const rsrc_t prow = make_rsrc(part, (uint32_t)ns * (uint32_t)sizeof(float2));
#pragma unroll
    for (int i = 0; i < kLocRun; ++i)
      p[i] = buffer_load8(prow, (s0 + i < s1) ? (uint32_t)(s0 + i) * 8u : (uint32_t)ns * 8u, 0u);
  }
  // the bias input row, requested after the partials (its address waits for
  // prev; no branch: a lane past r, or a request without a bias row, reads
  // zeros) and written to LDS once needed
  u32x4 row_in = u32x4{0u, 0u, 0u, 0u};
  if constexpr (!GREEDY) {
    const bool has_row = a.r > 0 && prev_ok;
    const int n = a.O ? a.r / 4 : a.r / 8;
    const rsrc_t rr = a.O ? make_rsrc(a.O + out * a.r, (uint32_t)a.r * 4u)
                          : make_rsrc(a.W1 + (size_t)(prev_ok ? prev : 0) * a.r, (uint32_t)a.r * 2u);
    row_in = buffer_load16(rr, (has_row && lane < n) ? (uint32_t)lane * 16u : 0xFFFFFFF0u, 0u);
  }
  __builtin_amdgcn_sched_barrier(0);
  if (in_regs) {
#pragma unroll
    for (int i = 0; i < kLocRun; ++i)
      if (s0 + i >= s1) p[i].x = -INFINITY;  // past the run (read as zeros): no maximum
  }
  if (!prev_ok) {
    if (lane == 0) {
      a.x_out[out] = -1;
      a.q_out[out] = NAN;
      a.lse_out[out] = NAN;
    }
    return;
  }
  // the decision uniform, computed while the loads are in flight
  const float u = GREEDY ? 0.f : decision_uniform(a.seed, a.step, (uint32_t)b, (uint32_t)a.k, kPurposeDraft);

  if constexpr (GREEDY) {
    float m = -INFINITY;
    int idx = -1;
    if (in_regs) {
#pragma unroll
      for (int i = 0; i < kLocRun; ++i)
        if (s0 + i < s1) merge_argmax(m, idx, p[i].x, __float_as_int(p[i].y));  // (no load in the branch)
    } else {
      for (int s = s0; s < s1; ++s) merge_argmax(m, idx, part[s].x, __float_as_int(part[s].y));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float m2 = __shfl_xor(m, off, 64);
      const int i2 = __shfl_xor(idx, off, 64);
      merge_argmax(m, idx, m2, i2);
    }
    if (lane == 0) {
      a.x_out[out] = idx;
      a.q_out[out] = 1.0f;
      a.lse_out[out] = m;
    }
    return;
  }

  float M = -INFINITY;
  if (in_regs) {
#pragma unroll
    for (int i = 0; i < kLocRun; ++i) M = fmaxf(M, p[i].x);
  } else {
    for (int s = s0; s < s1; ++s) M = fmaxf(M, part[s].x);
  }
  M = wave_max(M);
  // slice masses in fp32, their CDF in fp64
  auto weight = [&](float2 q) { return (q.x == -INFINITY) ? 0.0 : (double)(q.y * fast_exp2(q.x - M)); };
  double local = 0.0;
  if (in_regs) {
    double l4[4] = {0.0, 0.0, 0.0, 0.0};  // four chains in flight
#pragma unroll
    for (int i = 0; i < kLocRun; ++i) l4[i & 3] += weight(p[i]);
    local = (l4[0] + l4[1]) + (l4[2] + l4[3]);
  } else {
    for (int s = s0; s < s1; ++s) local += weight(part[s]);
  }
  const double incl = wave_inclusive_scan_dpp(local);
  const double S = __shfl(incl, 63, 64);
  const double target = (double)u * S;
  // owner: first lane whose inclusive sum passes the target, else the last with mass
  int owner = wave_first_lane(incl > target);
  if (owner < 0) {
    const unsigned long long mm = __ballot(local > 0.0);
    owner = mm ? 63 - __clzll((long long)mm) : 0;
  }
  // the owner's run: its first slice with mass whose cumulative sum passes
  // the target, else its last slice with mass
  int s_star;
  double before;
  float m_s;
  if (in_regs) {
    // the owner lane puts its run in LDS (in-order LDS access within the
    // wave: no barrier), lane i takes its slice i and an fp64 wave scan of
    // the masses finds the crossing
    __shared__ float2 sh_run[kLocRun];
    sh_row[lane] = row_in;  // the bias row, zero-filled past r
    if (lane == owner) {
#pragma unroll
      for (int i = 0; i < kLocRun; ++i) sh_run[i] = p[i];
    }
    const double acc0 = __shfl(incl - local, owner, 64);
    const int os0 = __shfl(s0, owner, 64);
    const float2 q = lane < kLocRun ? sh_run[lane] : make_float2(-INFINITY, 0.f);
    const double w = weight(q);
    const double cum = acc0 + wave_inclusive_scan_dpp(w);
    int pick = wave_first_lane(cum > target && w > 0.0);
    if (pick < 0) {  // rounding: the last slice with mass
      const unsigned long long mm = __ballot(w > 0.0);
      pick = mm ? 63 - __clzll((long long)mm) : -1;
    }
    if (pick < 0) {  // no mass at all (non-finite logits): stay in range
      s_star = 0;
      before = acc0;
      m_s = __shfl(p[0].x, 0, 64);
    } else {
      s_star = os0 + pick;
      before = __shfl(cum - w, pick, 64);
      m_s = __shfl(q.x, pick, 64);
    }
  } else {
    sh_row[lane] = row_in;
    double acc = incl - local;
    int hit = -1, last = -1;
    double hit_before = 0.0, last_before = acc;
    float hit_m = 0.f, last_m = 0.f;
    for (int s = s0; s < s1; ++s) {
      const float2 q = part[s];
      const double w = weight(q);
      if (w > 0.0) {
        if (hit < 0 && acc + w > target) {
          hit = s;
          hit_before = acc;
          hit_m = q.x;
        }
        last = s;
        last_before = acc;
        last_m = q.x;
      }
      acc += w;
    }
    if (hit < 0) {
      hit = last;
      hit_before = last_before;
      hit_m = last_m;
    }
    if (hit < 0) {  // no mass at all (non-finite logits): stay in range
      hit = 0;
      hit_before = incl - local;
      hit_m = part[0].x;
    }
    s_star = __shfl(hit, owner, 64);
    before = __shfl(hit_before, owner, 64);
    m_s = __shfl(hit_m, owner, 64);
  }

  // re-evaluate the 64 logits of slice s_star, one column per lane
  const int col = s_star * kWaveCols + lane;
  const bool col_ok = col < a.V;
  const UT* urow = reinterpret_cast<const UT*>(a.U) + ((size_t)b * a.K + (a.k - 1)) * a.V;
  // the base logit and the W2 weights are requested together (buffer loads:
  // a column past V reads zero, no branch)
  const rsrc_t ur = make_rsrc(urow, (uint32_t)a.V * (uint32_t)sizeof(UT));
  const uint32_t uoff = col_ok ? (uint32_t)col * (uint32_t)sizeof(UT) : 0xFFFFFFF0u;
  float base;
  if constexpr (sizeof(UT) == 2)
    base = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(ur, (int)uoff, 0, 0) << 16);
  else
    base = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ur, (int)uoff, 0, 0));
  float bias = 0.f;
  if (a.r > 0) {
    const int kc_count = (a.r + 31) / 32;
    const bool swz = a.W2s != nullptr && a.O == nullptr;
    const uint32_t w2_bytes = swz ? (uint32_t)((size_t)((a.V + kWaveCols - 1) / kWaveCols) * 4 * kc_count * 1024)
                                  : (uint32_t)((size_t)a.V * a.r * 2);
    const rsrc_t w2 = make_rsrc(swz ? static_cast<const void*>(a.W2s) : static_cast<const void*>(a.W2t), w2_bytes);
    const uint32_t off0 = swz ? (uint32_t)s_star * 4u * (uint32_t)kc_count * 1024u
                              : (uint32_t)(col_ok ? col : 0) * (uint32_t)a.r * 2u;
    bias = a.O ? lane_bias_staged<true>(sh_row, w2, w2_bytes, off0, false, a.r, col_ok, lane)
               : lane_bias_staged<false>(sh_row, w2, w2_bytes, off0, swz, a.r, col_ok, lane);
  }
  const float t_in = (float)((target - before) / (double)fast_exp2(m_s - M));
  const float z = col_ok ? base + bias : -INFINITY;
  const float e = col_ok ? fast_exp2(fmaf(z, a.c2, -m_s)) : 0.f;
  const float cum = wave_inclusive_scan_dpp(e);
  int pick = wave_first_lane(cum > t_in && e > 0.f);
  if (pick < 0) {
    const unsigned long long mm = __ballot(e > 0.f);
    pick = mm ? 63 - __clzll((long long)mm) : 0;
  }
  const float zx = __shfl(z, pick, 64);
  if (lane == 0) {
    a.x_out[out] = s_star * kWaveCols + pick;
    a.q_out[out] = fast_exp2(fmaf(zx, a.c2, -M)) / (float)S;
    a.lse_out[out] = (M + fast_log2((float)S)) * kLn2;
  }
}

// Full 128-row stages and the trailing partial stage (B not a multiple of
// 128) are separate launches of separately register-allocated variants.
// bf16 base logits with a Markov head sweep pairs of full stages as 256-row
// stages (each pair one stage of the 256-row variant, over the whole grid).
template <typename UT, bool VEC, int KC, bool GREEDY, bool ROWS = false>
static int launch_partials(const DraftArgs& a, hipStream_t stream) {
  const int full = VEC ? a.B / kStageRows : 0;  // unaligned rows: the plain variant throughout
  const int partial = a.nstages - full;
  if constexpr (VEC) {
    int done = 0;
    if constexpr (!ROWS && KC > 0 && std::is_same_v<UT, uint16_t>) {
      const int pairs = full / 2;
      if (pairs > 0) {
        DraftArgs b = a;
        b.ncol_tiles = std::max(1, std::min(a.nslices, kPersistentWGs / pairs));
        const int rc = launch_kernel("draft_partials",
                                     draft_partials_kernel<UT, VEC, KC, GREEDY, true, false, 2 * kGroupsPerWG>,
                                     dim3(xcd_grid(b.ncol_tiles, pairs)), dim3(kDraftWaves * 64), stream, b, 0,
                                     pairs);
        if (rc) return rc;
        done = 2 * pairs;
      }
    }
    if (full > done) {
      const int rc = launch_kernel("draft_partials", draft_partials_kernel<UT, VEC, KC, GREEDY, true, ROWS>,
                                   dim3(xcd_grid(a.ncol_tiles, full - done)), dim3(kDraftWaves * 64), stream, a,
                                   done, full - done);
      if (rc) return rc;
    }
  }
  if (partial > 0) {
    return launch_kernel("draft_partials", draft_partials_kernel<UT, VEC, KC, GREEDY, false, ROWS>,
                         dim3(xcd_grid(a.ncol_tiles, partial)), dim3(kDraftWaves * 64), stream, a, full, partial);
  }
  return 0;
}

template <typename UT, bool VEC, bool GREEDY>
static int dispatch_kc(const DraftArgs& a, hipStream_t stream) {
  // RNN head: one variant, r <= 256 zero-padded to eight chunks
  if (a.O) return launch_partials<UT, VEC, 8, GREEDY, true>(a, stream);
  switch ((a.r + 31) / 32) {
    case 0: return launch_partials<UT, VEC, 0, GREEDY>(a, stream);
    case 1: return launch_partials<UT, VEC, 1, GREEDY>(a, stream);
    case 2: return launch_partials<UT, VEC, 2, GREEDY>(a, stream);
    case 3: return launch_partials<UT, VEC, 3, GREEDY>(a, stream);
    case 4: return launch_partials<UT, VEC, 4, GREEDY>(a, stream);
    case 5: return launch_partials<UT, VEC, 5, GREEDY>(a, stream);
    case 6: return launch_partials<UT, VEC, 6, GREEDY>(a, stream);
    case 7: return launch_partials<UT, VEC, 7, GREEDY>(a, stream);
    case 8: return launch_partials<UT, VEC, 8, GREEDY>(a, stream);
    default: return -1;
  }
}

// W2 (column-major, V x r bf16) into fragment order for KC = ceil(r / 32)
// chunks: entry (blk, f = b * KC + kc, lane l) holds the 8 weights of column
// 64 blk + 16 (a / 4) + a % 4 + 4 b (a = l % 16) at k = 32 kc + 8 (l / 16) ..
// +7, or zeros past V or past r.  F16: the weights converted to fp16 (the
// RNN head's split stages; exact for bf16 magnitudes 2^-14 .. 2^15).  One
// thread per 16-byte entry; the writes are contiguous.
template <bool F16>
__global__ __launch_bounds__(256) void w2_swizzle_kernel(const uint16_t* __restrict__ W2, u32x4* __restrict__ out,
                                                         int V, int r, int KC, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const int lane = (int)(i & 63);
    const size_t fi = i >> 6;
    const int f = (int)(fi % (size_t)(4 * KC));
    const size_t blk = fi / (size_t)(4 * KC);
    const int b = f / KC, kc = f % KC;
    const int a = lane & 15;
    const size_t col = blk * 64 + (size_t)(16 * (a >> 2) + (a & 3) + 4 * b);
    const int k = 32 * kc + 8 * (lane >> 4);
    u32x4 v = (col < (size_t)V && k < r) ? *reinterpret_cast<const u32x4*>(W2 + col * r + k) : u32x4{0u, 0u, 0u, 0u};
    if constexpr (F16) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        v[e] = f16_bits(__uint_as_float(v[e] << 16)) | (f16_bits(__uint_as_float(v[e] & 0xFFFF0000u)) << 16);
    }
    out[i] = v;
  }
}

size_t w2_swizzle_bytes(int V, int r) {
  if (r <= 0) return 0;
  const size_t kc = (size_t)(r + 31) / 32;
  return (size_t)(((int64_t)V + kWaveCols - 1) / kWaveCols) * 4 * kc * 1024;
}

// W2 (column-major) into fragment order for kc chunks of 32 (zeros past r)
// at out, ceil(V / 64) * 4 * kc KB; f16: as fp16 values.
int run_w2_swizzle(const uint16_t* W2, void* out, int V, int r, int kc, bool f16, hipStream_t stream) {
  const size_t n = (size_t)(((int64_t)V + kWaveCols - 1) / kWaveCols) * 4 * kc * 64;
  const dim3 grid((unsigned)std::max<size_t>(std::min<size_t>((n + 255) / 256, 8192), 1));
  u32x4* o = reinterpret_cast<u32x4*>(out);
  return f16 ? launch_kernel("w2_to_f16", w2_swizzle_kernel<true>, grid, dim3(256), stream, W2, o, V, r, kc, n)
             : launch_kernel("w2_swizzle", w2_swizzle_kernel<false>, grid, dim3(256), stream, W2, o, V, r, kc, n);
}

template <typename UT, bool GREEDY>
static int run_draft_typed(DraftArgs a, bool vec, bool make_w2s, const RnnParams* rnn, hipStream_t stream) {
  if (make_w2s) {
    const int rc = run_w2_swizzle(a.W2t, const_cast<uint16_t*>(a.W2s), a.V, a.r, (a.r + 31) / 32, false, stream);
    if (rc) return rc;
  }
  if (rnn) {
    int rc = rnn->w2h_ready ? 0 : run_w2_to_f16(rnn->W2, rnn->W2h, a.V, a.r, stream);
    if (rc) return rc;
    rc = run_rnn_hproj(*rnn, stream);
    if (rc) return rc;
  }
  for (int k = 1; k <= a.K; ++k) {
    a.k = k;
    if (k == 1) {
      // prev set by the caller to the anchors
    } else {
      a.prev = a.x_out + (k - 2);
      a.prev_stride = a.K;
    }
    if (rnn) {
      const int rc = run_rnn_step(*rnn, k, stream);
      if (rc) return rc;
    }
    int rc = vec ? dispatch_kc<UT, true, GREEDY>(a, stream) : dispatch_kc<UT, false, GREEDY>(a, stream);
    if (rc) return rc;
    rc = launch_kernel("draft_locate", draft_locate_kernel<UT, GREEDY>, dim3(a.B), dim3(64), stream, a);
    if (rc) return rc;
  }
  return 0;
}

// Log-normaliser of every request's draft row at position a.k from its
// slice partials (one wave per request): lse = (M + log2 S) ln 2 with
// M = max of the slices' scaled maxima, S = sum_s s_s 2^(m_s - M).
__global__ __launch_bounds__(256) void draft_lse_kernel(DraftArgs a) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x * 4 + wave_index();
  if (b >= a.B) return;
  const float2* part = a.part + (size_t)b * a.nslices;
  float m = -INFINITY, s = 0.f;
  for (int i = lane; i < a.nslices; i += 64) {
    const float2 p = part[i];
    merge_ms(m, s, p.x, p.y);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float m2 = __shfl_xor(m, off, 64);
    const float s2 = __shfl_xor(s, off, 64);
    merge_ms(m, s, m2, s2);
  }
  if (lane == 0) a.lse_out[(size_t)b * a.K + (a.k - 1)] = (m + fast_log2(s)) * kLn2;
}

// The draft rows' log-normalisers lse[r, k-1] = log sum_v exp((D[r, k-1, v] +
// W1[x_{k-1}] W2[:, v]) / T), x_0 = x0, for every request and position (T > 0):
// the draft's fused bias pass at each position, then the merge above.
// W2s: the fragment-ordered copy of W2 (required when r > 0); part: slice
// partials [R, ceil(V / 64)] (draft_workspace_bytes(R, K, V)).
int run_markov_lse(int R, int K, int V, int r, float temperature, const void* D, bool d_bf16, const void* W1,
                   const void* W2, const void* W2s, const int32_t* x0, const int32_t* x, float* lse_out,
                   void* part, hipStream_t stream) {
  DraftArgs a{};
  a.U = D;
  a.W1 = reinterpret_cast<const uint16_t*>(W1);
  a.W2t = reinterpret_cast<const uint16_t*>(W2);
  a.W2s = reinterpret_cast<const uint16_t*>(W2s);
  a.B = R;
  a.K = K;
  a.V = V;
  a.r = r;
  a.nslices = (V + kWaveCols - 1) / kWaveCols;
  a.nstages = (R + kStageRows - 1) / kStageRows;
  a.ncol_tiles = std::max(1, std::min(a.nslices, kPersistentWGs / a.nstages));
  a.part = reinterpret_cast<float2*>(part);
  a.c2 = kLog2e / temperature;
  a.lse_out = lse_out;
  // prev of position k: the anchors at k = 1, then x[:, k-2]
  const uintptr_t base = reinterpret_cast<uintptr_t>(D);
  const bool vec = (base % 16 == 0) && (V % (d_bf16 ? 8 : 4) == 0);
  auto run = [&](auto tag) -> int {
    using UT = decltype(tag);
    for (int k = 1; k <= K; ++k) {
      a.k = k;
      a.prev = k == 1 ? x0 : x + (k - 2);
      a.prev_stride = k == 1 ? 1 : K;
      int rc = vec ? dispatch_kc<UT, true, false>(a, stream) : dispatch_kc<UT, false, false>(a, stream);
      if (rc) return rc;
      rc = launch_kernel("draft_lse", draft_lse_kernel, dim3((R + 3) / 4), dim3(256), stream, a);
      if (rc) return rc;
    }
    return 0;
  };
  return d_bf16 ? run(uint16_t{}) : run(float{});
}

size_t draft_workspace_bytes(int B, int K, int V) {
  (void)K;
  const size_t ns = (size_t)(((int64_t)V + kWaveCols - 1) / kWaveCols);
  return ((size_t)B * ns * sizeof(float2) + 255) / 256 * 256;
}

int run_draft(int B, int K, int V, int r, float temperature, const void* U, bool u_bf16,
              const void* W1, const void* W2, const void* W2f, const int32_t* x0, uint64_t seed, uint64_t step,
              int32_t* x_out, float* q_out, float* lse_out, void* workspace, const RnnParams* rnn,
              hipStream_t stream) {
  DraftArgs a{};
  a.U = U;
  a.W1 = reinterpret_cast<const uint16_t*>(W1);
  a.W2t = reinterpret_cast<const uint16_t*>(W2);
  a.prev = x0;
  a.prev_stride = 1;
  a.B = B;
  a.K = K;
  a.V = V;
  a.r = r;
  a.nslices = (V + kWaveCols - 1) / kWaveCols;
  // persistent grid: one 8-wave workgroup per CU; column ranges split the
  // 64-column blocks evenly, row stages of 128 requests
  a.nstages = (B + kStageRows - 1) / kStageRows;
  a.ncol_tiles = std::max(1, std::min(a.nslices, kPersistentWGs / a.nstages));
  a.part = reinterpret_cast<float2*>(workspace);
  // Markov head: the caller's fragment-ordered W2, else a copy made here
  // after the slice partials
  const bool make_w2s = !rnn && r > 0 && !W2f;
  a.W2s = (!rnn && r > 0) ? (W2f ? reinterpret_cast<const uint16_t*>(W2f)
                                 : reinterpret_cast<const uint16_t*>(reinterpret_cast<char*>(workspace) +
                                                                     draft_workspace_bytes(B, K, V)))
                          : nullptr;
  a.seed = seed;
  a.step = step;
  a.x_out = x_out;
  a.q_out = q_out;
  a.lse_out = lse_out;
  a.O = rnn ? rnn->O : nullptr;
  a.W2h = rnn ? rnn->W2h : nullptr;
  const bool greedy = temperature == 0.f;
  a.c2 = greedy ? 1.f : kLog2e / temperature;
  const uintptr_t base = reinterpret_cast<uintptr_t>(U);
  if (u_bf16) {
    const bool vec = (V % 8 == 0) && (base % 16 == 0);
    return greedy ? run_draft_typed<uint16_t, true>(a, vec, make_w2s, rnn, stream)
                  : run_draft_typed<uint16_t, false>(a, vec, make_w2s, rnn, stream);
  }
  const bool vec = (V % 4 == 0) && (base % 16 == 0);
  return greedy ? run_draft_typed<float, true>(a, vec, make_w2s, rnn, stream)
                : run_draft_typed<float, false>(a, vec, make_w2s, rnn, stream);
}

}  // namespace dspark
