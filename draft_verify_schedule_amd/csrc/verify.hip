// Rejection-sampling verification over the flattened variable-length batch
// (DSpark paper, section 2.1 and section 5.3; "Speculative decoding, from zero
// to DSpark", section 2 and Appendix A1; the glean.smartcoder article's
// five-step verification routine).
//
// Request r owns flat target rows cu[r] .. cu[r+1]-1 (its l_r drafts, then the
// bonus row).  Launches:
//   verify_rowstats   one HBM pass over every flat target row: per 2048-column
//                     slice the softmax partial (max, sum exp2) of t * log2(e)/T,
//                     or (max, first argmax) when greedy;
//   verify_accept     one wave per flat row: merges its partials into the
//                     row normaliser and runs the min(1, p/q) test of the
//                     draft token the row judges;
//   verify_decide     one thread per request: first rejection -> n_acc and
//                     which row needs a correction (residual) or bonus sample;
//   verify_residual   (T > 0) for rejecting requests, one pass over the
//                     rejected position's target and draft rows, the draft
//                     row's Markov bias rebuilt on MFMA: per 64-column slice
//                     the mass of max(0, p - q);
//   verify_sample     (T > 0) one wave per request: inverse-CDF draw of the
//                     correction (residual partials, 64-column re-scan) or the
//                     bonus (target partials, 2048-column re-scan).
// Drafts of the RNN head (DSpark paper, section 3.1, RNN head) pass their
// output parts O [R, K, r] fp32: the draft row of position j then carries the
// bias O[r, j-1] W2, staged as split hi/lo bf16 rows for the MFMA.
#include <algorithm>
#include <type_traits>

#include "bias_tile.hpp"
#include "launch.hpp"

namespace dspark {

constexpr int kRowChunk = 8192;   // columns per rowstats workgroup (2048 per wave)
// columns per target-row partial: one per wave of the row-statistics pass
// (fewer, coarser partials: the pass's writes cost far more than their bytes
// inside its read stream)
constexpr int kRowSlice = 2048;
constexpr int kRowstatsWGs = 1024;  // persistent rowstats grid: 4 workgroups per CU (measured faster than 8)
constexpr int kMaxPositions = 16;   // draft positions per request (the ABI's limit on K)

struct VerifyArgs {
  int R, K, V, N, r;
  float c2;                 // log2(e) / T, or 1 when greedy
  const void* P;            // [N, V]
  const int32_t* cu;        // [R + 1]
  const void* D;            // [R, K, V]
  const uint16_t* W1;
  const uint16_t* W2t;
  const int32_t* x0;        // [R]
  const int32_t* x;         // [R, K]
  const float* q_tok;       // [R, K]
  const float* lse_d;       // [R, K]
  const float* O;           // RNN head: output parts [R, K, r] fp32 (else null)
  const uint16_t* W2h;      // RNN head: fp16 copy of W2t
  const uint16_t* W2s;      // acceptance label, Markov head: W2t in MFMA fragment order
  uint64_t seed, step;
  int32_t* n_acc_out;
  int32_t* tok_out;
  // workspace
  float2* ppart;            // [N, nsP]
  float2* rowms;            // [N]  (max, sum) or (max, argmax bits)
  int32_t* flag;            // [N]  1 accept, 0 reject, 2 bad row, 3 bonus row
  int4* info;               // [R]  (mode, sample row, position, n_acc)
  float* rpart;             // [R, ns64]
  int32_t* rej_list;        // [R]  correcting requests, compacted (any order)
  int32_t* rej_count;       // [1]
  int nsP, ns64, nchunks;
  int ncol_tiles, nstages;
  // rows of a rowstats pass over the draft rows D [R * K, V]: row r * K + j is
  // streamed only when j < l_r (cu_seqlens of the verify layout); else null
  const int32_t* row_cu;
  int row_K;
  float* ppart2;            // greedy: runner-up value per slice [N, nsP] (else null)
  float* margin;            // [N]  decision margin of each flat row (else null)
  float* rmin;              // [R]  smallest accept margin of each request (T > 0)
  float* min_margin_out;    // [R]  or null
  // acceptance label, streamed residual pass: per (job, item) fp64 sums of the
  // residual masses a job (one wave of one workgroup) swept for that item
  double* lpart;            // [njobs, N]
  int njobs;
};

// Whether row q of a pass over the draft rows is judged by the layout
// (request q / K, position q % K < l_r); every row when no filter is set.
__device__ __forceinline__ bool drow_judged(const VerifyArgs& a, int q) {
  if (!a.row_cu) return true;
  const int r = q / a.row_K;
  const int j = q - r * a.row_K;
  return j < a.row_cu[r + 1] - a.row_cu[r] - 1;
}

// ---------------------------------------------------------------- rowstats --
template <typename PT, bool VEC, bool GREEDY>
__global__ __launch_bounds__(256) void verify_rowstats_kernel(VerifyArgs a) {
  const int row = blockIdx.x / a.nchunks;
  const int chunk = blockIdx.x - row * a.nchunks;
  const int lane = threadIdx.x & 63;
  const int wave = wave_index();
  const int wbase = chunk * kRowChunk + wave * (kRowChunk / 4);
  if (wbase >= a.V || !drow_judged(a, row)) return;
  const PT* prow = reinterpret_cast<const PT*>(a.P) + (size_t)row * a.V;
  float2* out = a.ppart + (size_t)row * a.nsP;
  float* out2 = a.ppart2 ? a.ppart2 + (size_t)row * a.nsP : nullptr;

  if constexpr (VEC) {
    constexpr int EPL = 16 / sizeof(PT);          // elements per 16-byte load
    constexpr int COLS = 64 * EPL;                // columns per load instruction
    constexpr int ITERS = (kRowChunk / 4) / COLS; // loads per wave
    static_assert(kRowSlice == kRowChunk / 4, "one slice per wave");
    float v[ITERS][EPL];
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int c = wbase + it * COLS + lane * EPL;
      if (c < a.V) {
        if constexpr (sizeof(PT) == 2) {
          const u32x4 w = *reinterpret_cast<const u32x4*>(prow + c);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[it][2 * e] = __uint_as_float(w[e] << 16);
            v[it][2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
          }
        } else {
          const f32x4 w = *reinterpret_cast<const f32x4*>(prow + c);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[it][e] = w[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) v[it][e] = -INFINITY;
      }
    }
    // one slice per wave: the lane's ITERS x EPL values in column order
    const int slice = wbase / kRowSlice;
    if constexpr (GREEDY) {
      float m = -INFINITY, m2 = -INFINITY;
      int idx = -1;
#pragma unroll
      for (int it = 0; it < ITERS; ++it) {
        const int c = wbase + it * COLS + lane * EPL;
#pragma unroll
        for (int e = 0; e < EPL; ++e)
          if (c + e < a.V) merge_top2(m, idx, m2, v[it][e], c + e, -INFINITY);
      }
      wave_merge_top2(m, idx, m2);
      if (lane == 0 && slice < a.nsP && idx >= 0) {
        out[slice] = make_float2(m, __int_as_float(idx));
        if (out2) out2[slice] = m2;
      }
    } else {
      float m = -INFINITY;
#pragma unroll
      for (int it = 0; it < ITERS; ++it)
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          v[it][e] *= a.c2;  // past V: -inf
          m = fmaxf(m, v[it][e]);
        }
      m = wave_max_dpp(m);
      float s = 0.f;
      if (m != -INFINITY) {
#pragma unroll
        for (int it = 0; it < ITERS; ++it)
#pragma unroll
          for (int e = 0; e < EPL; ++e) s += exp2f(v[it][e] - m);
      }
      s = wave_sum_dpp(s);
      if (lane == 0 && slice < a.nsP) out[slice] = make_float2(m, s);
    }
  } else {
    // any alignment: lane-strided scalar loads, the wave's 2048 columns (one
    // slice) held as 32 values per lane, lane l taking columns l, l + 64, ...
    constexpr int T = kRowSlice / 64;
    float v[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int c = wbase + 64 * t + lane;
      v[t] = (c < a.V) ? load_logit(prow, c) : -INFINITY;
    }
    const int slice = wbase / kRowSlice;
    if constexpr (GREEDY) {
      float m = -INFINITY, m2 = -INFINITY;
      int idx = -1;
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const int c = wbase + 64 * t + lane;
        if (c < a.V) merge_top2(m, idx, m2, v[t], c, -INFINITY);
      }
      wave_merge_top2(m, idx, m2);
      if (lane == 0 && idx >= 0) {
        out[slice] = make_float2(m, __int_as_float(idx));
        if (out2) out2[slice] = m2;
      }
    } else {
      float m = -INFINITY;
#pragma unroll
      for (int t = 0; t < T; ++t) {
        v[t] *= a.c2;
        m = fmaxf(m, v[t]);
      }
      m = wave_max_dpp(m);
      float s = 0.f;
      if (m != -INFINITY) {
#pragma unroll
        for (int t = 0; t < T; ++t) s += exp2f(v[t] - m);
      }
      s = wave_sum_dpp(s);
      if (lane == 0) out[slice] = make_float2(m, s);
    }
  }
}

// Aligned-row variant: persistent grid-stride over (row, 8192-column chunk)
// items.  Wave w covers columns [2048 w, 2048 w + 2048) of the chunk, one
// slice.  Load l of lane l' reads the 16 bytes at 1024 l + 16 l' of the
// wave's columns, so each load instruction covers whole 128-byte lines (a
// lane holding 32 contiguous columns would read each line in four
// instructions of two lanes each, four times the cache accesses), and the
// loads are non-temporal (each row is read once); each lane reduces its 32
// values, then DPP steps and the row swaps finish the slice, and lane 0
// writes its partial.  The next item's loads (buffer resource, per-lane VGPR
// offset, scalar row offset) are issued before the current item is reduced;
// the loop body has no branches: loads past the last item and stores of the
// other lanes get offsets past their buffer resource.
template <typename PT, bool GREEDY>
__global__ __launch_bounds__(256) void verify_rowstats_stream_kernel(VerifyArgs a) {
  constexpr int kWaveColsR = kRowChunk / 4;     // 2048
  constexpr int CPL = kWaveColsR / 64;          // columns per lane per item
  constexpr int EPL = 16 / sizeof(PT);          // elements per 16-byte load
  constexpr int LOADS = CPL / EPL;
  static_assert(kRowSlice == kWaveColsR, "one slice per wave");
  const int lane = threadIdx.x & 63;
  const int wave = wave_index();
  const int items = a.N * a.nchunks;
  const uint32_t pbytes = (uint32_t)((uint64_t)a.N * a.V * sizeof(PT));
  const rsrc_t rs = make_rsrc(a.P, pbytes);
  const uint32_t lane_off = (uint32_t)lane * 16u;
  const uint32_t obytes = (uint32_t)((uint64_t)a.N * a.nsP * sizeof(float2));
  const int4v ors = raw_rsrc_words(a.ppart, obytes);
  const bool leader = lane == 0;

  const uint32_t o2bytes = a.ppart2 ? obytes / 2u : 0u;
  const int4v o2rs = raw_rsrc_words(a.ppart2, o2bytes);
  auto issue = [&](int item, u32x4 (&w)[LOADS]) {
    const bool live = item < items && drow_judged(a, item / a.nchunks);
    const int row = live ? item / a.nchunks : 0;
    const int chunk = live ? item - row * a.nchunks : 0;
    const int wbase = chunk * kRowChunk + wave * kWaveColsR;
    const uint32_t soff = live ? (uint32_t)(((uint64_t)row * a.V + wbase) * sizeof(PT)) : pbytes;
#pragma unroll
    for (int l = 0; l < LOADS; ++l) w[l] = buffer_load16_nt(rs, lane_off + (uint32_t)(1024 * l), soff);
  };
  // one item's statistics; MASK: the wave's 2048 columns pass the end of the
  // row (only then are values masked: V is a multiple of EPL, so whole
  // vectors are in or out)
  auto reduce_as = [&](auto mask_tag, int row, int wbase, const u32x4 (&w)[LOADS]) {
    constexpr bool MASK = decltype(mask_tag)::value;
    // value e = l * EPL + j of the lane is column col(e): increasing in e
    const int c0 = wbase + lane * EPL;
    auto col = [&](int e) { return c0 + (e / EPL) * (64 * EPL) + e % EPL; };
    float v[CPL];
#pragma unroll
    for (int l = 0; l < LOADS; ++l) {
      const bool ok = !MASK || col(l * EPL) < a.V;
      if constexpr (sizeof(PT) == 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[l * EPL + 2 * e] = ok ? __uint_as_float(w[l][e] << 16) : -INFINITY;
          v[l * EPL + 2 * e + 1] = ok ? __uint_as_float(w[l][e] & 0xFFFF0000u) : -INFINITY;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[l * EPL + e] = ok ? __uint_as_float(w[l][e]) : -INFINITY;
      }
    }
    float2 res;
    float runner_up = 0.f;
    if constexpr (GREEDY) {
      float m = -INFINITY, m2 = -INFINITY;
      int idx = -1;
      if constexpr (MASK) {
#pragma unroll
        for (int e = 0; e < CPL; ++e)
          if (col(e) < a.V) merge_top2(m, idx, m2, v[e], col(e), -INFINITY);
      } else {
        // every column valid: the max, its first index, and the largest value
        // at any other index (a tie gives the max itself)
        m = v[0];
#pragma unroll
        for (int e = 1; e < CPL; ++e) m = fmaxf(m, v[e]);
        int first = CPL - 1;
#pragma unroll
        for (int e = CPL - 2; e >= 0; --e) first = (v[e] == m) ? e : first;
        if (a.ppart2) {  // runner-up only when decision margins are asked for (wave-uniform)
#pragma unroll
          for (int e = 0; e < CPL; ++e) m2 = fmaxf(m2, e == first ? -INFINITY : v[e]);
        }
        idx = col(first);
      }
      // the slice is the whole wave
      if (a.ppart2) wave_merge_top2(m, idx, m2);
      else wave_merge_argmax(m, idx);
      res = make_float2(m, __int_as_float(idx));
      runner_up = m2;
    } else {
      float m = v[0];
#pragma unroll
      for (int e = 1; e < CPL; ++e) m = fmaxf(m, v[e]);
      m = wave_max_dpp(m);
      const bool empty = m == -INFINITY;
      const float mc = empty ? 0.f : m * a.c2;
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < CPL; ++e) s += fast_exp2(fmaf(v[e], a.c2, -mc));
      s = wave_sum_dpp(s);
      res = make_float2(empty ? -INFINITY : mc, s);
    }
    const int slice = wbase / kRowSlice;
    const uint32_t voff = (leader && slice < a.nsP) ? (uint32_t)(((uint64_t)row * a.nsP + slice) * sizeof(float2))
                                                    : obytes;
    buffer_store8_untracked(ors, res, voff, 0u);
    if constexpr (GREEDY) {
      if (a.ppart2) buffer_store4_untracked(o2rs, runner_up, voff / 2u, 0u);  // offsets past the resource drop
    }
  };
  auto reduce = [&](int item, const u32x4 (&w)[LOADS]) {
    const int row = item / a.nchunks;
    const int chunk = item - row * a.nchunks;
    const int wbase = chunk * kRowChunk + wave * kWaveColsR;
    if (wbase + kWaveColsR > a.V) reduce_as(std::true_type{}, row, wbase, w);  // wave-uniform branch
    else reduce_as(std::false_type{}, row, wbase, w);
  };

  int item = blockIdx.x;
  u32x4 cur[LOADS], nxt[LOADS];
  issue(item, cur);
  for (; item < items; item += gridDim.x) {
    issue(item + gridDim.x, nxt);
    __builtin_amdgcn_sched_barrier(0);  // keep the next item's loads ahead of this item's waits
    reduce(item, cur);
#pragma unroll
    for (int l = 0; l < LOADS; ++l) cur[l] = nxt[l];
  }
}

// ------------------------------------------------------------------ accept --
// Request owning flat row i: the largest r with cu[r] <= i (cu is validated by
// the caller of the result, never trusted for indexing beyond [0, R]).
__device__ __forceinline__ int owner_of(const int32_t* cu, int R, int i) {
  int lo = 0, hi = R - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= i) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// The same search by a whole wave in two rounds of loads (R <= 4096): 64
// probes at stride ceil(R / 64) bracket i, then up to 64 probes inside the
// bracket.  For non-decreasing cu it returns what owner_of returns.
__device__ __forceinline__ int owner_of_wave(const int32_t* cu, int R, int i) {
  if (R > 64 * 64) return owner_of(cu, R, i);
  const int lane = threadIdx.x & 63;
  const int step = (R + 63) / 64;
  const int p1 = lane * step;
  const bool in1 = p1 < R && cu[min(p1, R - 1)] <= i;
  const unsigned long long m1 = __ballot(in1);
  const int lo = m1 ? (63 - __clzll((long long)m1)) * step : 0;
  const int p2 = lo + lane;
  const bool in2 = lane < step && p2 < R && cu[min(p2, R - 1)] <= i;
  const unsigned long long m2 = __ballot(in2);
  return m2 ? lo + 63 - __clzll((long long)m2) : lo;
}

// Merge of one row's slice partials by a wave: lane l takes slices l, l + 64,
// ... in that order (all loads requested together when the row has at most
// 64 * kMergePer slices), then a butterfly over the lanes.
constexpr int kMergePer = 16;
template <bool GREEDY>
__device__ __forceinline__ void merge_row(const float2* __restrict__ part, int ns, float& m, float& s, int& idx) {
  const int lane = threadIdx.x & 63;
  m = -INFINITY;
  s = 0.f;
  idx = -1;
  if (ns <= 64 * kMergePer) {
    float2 pv[kMergePer];
#pragma unroll
    for (int j = 0; j < kMergePer; ++j) pv[j] = (lane + 64 * j < ns) ? part[lane + 64 * j] : make_float2(0.f, 0.f);
#pragma unroll
    for (int j = 0; j < kMergePer; ++j) {
      if (lane + 64 * j < ns) {
        if constexpr (GREEDY) merge_argmax(m, idx, pv[j].x, __float_as_int(pv[j].y));
        else merge_ms(m, s, pv[j].x, pv[j].y);
      }
    }
  } else {
    for (int k = lane; k < ns; k += 64) {
      const float2 p = part[k];
      if constexpr (GREEDY) merge_argmax(m, idx, p.x, __float_as_int(p.y));
      else merge_ms(m, s, p.x, p.y);
    }
  }
}

// The draft logit z_q(x) = D[r, j, x] + W1[prev] . W2[:, x] of one column
// by a whole wave (lane l takes the weights k = 8 l .. 8 l + 7, fp32
// products, wave sum); used when the caller gives no q_tok.
template <typename DT>
__device__ __forceinline__ float draft_logit_wave(const VerifyArgs& a, int r, int j, int xcol) {
  const int lane = threadIdx.x & 63;
  const DT* drow = reinterpret_cast<const DT*>(a.D) + ((size_t)r * a.K + j) * a.V;
  float bias = 0.f;
  if (a.r > 0) {
    const int prev = j == 0 ? a.x0[r] : a.x[(size_t)r * a.K + j - 1];
    const int pv = (prev >= 0 && prev < a.V) ? prev : 0;  // an invalid token flags the request elsewhere
    const int k = 8 * lane;
    if (k < a.r) {
      const u32x4 e = *reinterpret_cast<const u32x4*>(a.W1 + (size_t)pv * a.r + k);
      const u32x4 w = *reinterpret_cast<const u32x4*>(a.W2t + (size_t)xcol * a.r + k);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bias = fmaf(__uint_as_float(e[i] << 16), __uint_as_float(w[i] << 16), bias);
        bias = fmaf(__uint_as_float(e[i] & 0xFFFF0000u), __uint_as_float(w[i] & 0xFFFF0000u), bias);
      }
    }
    bias = wave_sum(bias);
  }
  return load_logit(drow, xcol) + bias;
}

template <typename PT, typename DT, bool GREEDY>
__global__ __launch_bounds__(256) void verify_accept_kernel(VerifyArgs a) {
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + wave_index();
  if (blockIdx.x == 0 && threadIdx.x == 0) *a.rej_count = 0;  // filled by the decide kernel
  if (i >= a.N) return;
  const float2* part = a.ppart + (size_t)i * a.nsP;
  float m, s = 0.f, m2 = -INFINITY;
  int idx;
  if constexpr (GREEDY) {
    // (max, first argmax, runner-up): lane l merges slices l, l + 64, ...
    m = -INFINITY;
    idx = -1;
    const float* part2 = a.ppart2 ? a.ppart2 + (size_t)i * a.nsP : nullptr;
    for (int k0 = 0; k0 < a.nsP; k0 += 64 * kMergePer) {
      float2 pv[kMergePer];
      float p2[kMergePer];
#pragma unroll
      for (int t = 0; t < kMergePer; ++t) {
        const int k = k0 + lane + 64 * t;
        pv[t] = k < a.nsP ? part[k] : make_float2(-INFINITY, __int_as_float(-1));
        p2[t] = (part2 && k < a.nsP) ? part2[k] : -INFINITY;
      }
#pragma unroll
      for (int t = 0; t < kMergePer; ++t) merge_top2(m, idx, m2, pv[t].x, __float_as_int(pv[t].y), p2[t]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float om = __shfl_xor(m, off, 64);
      const int oi = __shfl_xor(idx, off, 64);
      const float om2 = __shfl_xor(m2, off, 64);
      merge_top2(m, idx, m2, om, oi, om2);
    }
  } else {
    merge_row<false>(part, a.nsP, m, s, idx);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float om = __shfl_xor(m, off, 64);
      const float os = __shfl_xor(s, off, 64);
      merge_ms(m, s, om, os);
    }
  }
  const int r = owner_of_wave(a.cu, a.R, i);
  if (lane == 0) a.rowms[i] = GREEDY ? make_float2(m, __int_as_float(idx)) : make_float2(m, s);

  const int c0 = a.cu[r], c1 = a.cu[r + 1];
  const int j = i - c0;             // this row judges draft position j + 1
  int state;                        // 2 bad row, 3 bonus row, else a draft to judge
  int xj = 0;
  if (!(c0 >= 0 && c0 <= i && i < c1 && c1 <= a.N && c1 - c0 <= a.K + 1)) {
    state = 2;
  } else if (j >= c1 - c0 - 1) {
    state = 3;
  } else {
    xj = a.x[(size_t)r * a.K + j];
    state = (xj < 0 || xj >= a.V) ? 2 : 0;
  }
  // the decision margin: the target's top-2 gap (greedy), else |u - ratio|
  const float gap = m - m2;
  if (state != 0) {
    if (lane == 0) {
      a.flag[i] = state;
      if (a.margin) a.margin[i] = (state == 3 && GREEDY) ? gap : NAN;
    }
    return;
  }
  if constexpr (GREEDY) {
    if (lane == 0) {
      a.flag[i] = (idx == xj) ? 1 : 0;
      if (a.margin) a.margin[i] = gap;
    }
  } else {
    float q;
    if (a.q_tok) {
      q = a.q_tok[(size_t)r * a.K + j];
    } else {
      // q_j(x_j) = exp((z_q(x_j) - lse) / T), lse from the caller or the pass over the draft rows
      const float zq = draft_logit_wave<DT>(a, r, j, xj);
      q = fast_exp2(fmaf(zq, a.c2, -a.lse_d[(size_t)r * a.K + j] * kLog2e));
    }
    if (lane == 0) {
      const PT* prow = reinterpret_cast<const PT*>(a.P) + (size_t)i * a.V;
      const float t = load_logit(prow, xj) * a.c2;
      const float p = exp2f(t - m) / s;
      const float ratio = (q > 0.f) ? p / q : INFINITY;
      const float u = decision_uniform(a.seed, a.step, (uint32_t)r, (uint32_t)(j + 1), kPurposeAccept);
      a.flag[i] = (u < ratio) ? 1 : 0;
      if (a.margin) a.margin[i] = fabsf(u - ratio);
    }
  }
}

// ------------------------------------------------------------------ decide --
template <bool GREEDY>
__global__ __launch_bounds__(256) void verify_decide_kernel(VerifyArgs a) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= a.R) return;
  const int c0 = a.cu[r], c1 = a.cu[r + 1];
  bool ok = c0 >= 0 && c1 > c0 && c1 <= a.N && c1 - c0 <= a.K + 1;
  int n = 0, L = 0;
  if (ok) {
    L = c1 - c0 - 1;  // <= K <= kMaxPositions
    // the request's flags, loaded together
    int f[kMaxPositions + 1];
#pragma unroll
    for (int j = 0; j <= kMaxPositions; ++j) f[j] = (j <= L) ? a.flag[c0 + j] : 1;
    bool run = true;  // still in the leading run of accepted drafts
#pragma unroll
    for (int j = 0; j <= kMaxPositions; ++j) {
      if (f[j] == 2) ok = false;
      if (j < L && run && f[j] == 1) ++n;
      else run = false;
    }
    if (!GREEDY && a.r > 0 && (a.x0[r] < 0 || a.x0[r] >= a.V)) ok = false;
  }
  if (!ok) {
    a.info[r] = make_int4(-1, 0, 0, 0);
    a.n_acc_out[r] = -1;
    a.tok_out[r] = -1;
    if (a.min_margin_out) a.min_margin_out[r] = NAN;
    return;
  }
  const int mode = (n < L) ? 1 : 0;  // 1: correction from the residual, 0: bonus
  a.info[r] = make_int4(mode, c0 + n, n + 1, n);
  if (!GREEDY && mode == 1) a.rej_list[atomicAdd(a.rej_count, 1)] = r;
  a.n_acc_out[r] = n;
  if constexpr (GREEDY) a.tok_out[r] = __float_as_int(a.rowms[c0 + n].y);
  if (a.min_margin_out) {
    // rows examined: the accept tests j = 0 .. min(n, L - 1); when greedy
    // also the row whose argmax is emitted (row n: the rejected or the bonus row)
    const int last = GREEDY ? n : min(n, L - 1);
    float mg[kMaxPositions + 1];
#pragma unroll
    for (int j = 0; j <= kMaxPositions; ++j) mg[j] = (j <= last) ? a.margin[c0 + j] : INFINITY;
    float mm = INFINITY;
#pragma unroll
    for (int j = 0; j <= kMaxPositions; ++j) mm = fminf(mm, mg[j]);
    if constexpr (GREEDY) a.min_margin_out[r] = mm;
    else a.rmin[r] = mm;  // the draw's own margin is added by the sample kernel
  }
}

// ---------------------------------------------------------------- residual --
// max(0, p - q) over the rejected position, 64-column slice masses.  Same
// tiling and software pipeline as the draft's fused pass: 4 waves x 64
// columns, 128 requests (8 MFMA groups) per workgroup, W2 fragments held in
// registers, the target and draft rows of group g+2 requested before the
// epilogue of group g.  Requests that are not correcting take no loads.
template <typename PT, typename DT, bool VEC_P, bool VEC_D, int KC, bool LABEL = false, bool ROWS = false>
__global__ __launch_bounds__(256) void verify_residual_kernel(VerifyArgs a) {
  int col_tile, stage;
  if (!xcd_tile(blockIdx.x, a.ncol_tiles, a.nstages, col_tile, stage)) return;
  const int lane = threadIdx.x & 63;
  const int wave = wave_index();
  const int n0 = col_tile * kTileCols + wave * kWaveCols;
  const int row0 = stage * kStageRows;
  // LABEL: one item per (request, position) pair, item i = r * K + k; its
  // target row is P row i, its draft row D row i
  const int nrow = LABEL ? a.R * a.K : a.R;
  const int ngroups = min(kGroupsPerWG, (nrow - row0 + 15) / 16);
  const bool col_live = n0 < a.V;
  const int cbase = n0 + 16 * (lane >> 4);
  const int slice = n0 / kWaveCols;
  auto req = [&](int g) { return row0 + 16 * g + (lane & 15); };
  // requests that do not correct (or lie past R) read row 0 and are masked
  auto info_of = [&](int g) {
    if constexpr (LABEL) return req(g) < nrow ? make_int4(1, req(g), 0, 0) : make_int4(-1, 0, 0, 0);
    else return req(g) < a.R ? a.info[req(g)] : make_int4(-1, 0, 0, 0);
  };
  auto prow = [&](const int4& in) {
    return reinterpret_cast<const PT*>(a.P) + (size_t)(in.x == 1 ? in.y : 0) * a.V;
  };
  auto drow = [&](int g, const int4& in) {
    const size_t row = LABEL ? (size_t)req(g) : (size_t)req(g) * a.K + in.w;
    return reinterpret_cast<const DT*>(a.D) + (in.x == 1 ? row * a.V : 0);
  };

  GroupLogits<PT, VEC_P> pb0, pb1;
  GroupLogits<DT, VEC_D> db0, db1;
  int4 in0 = info_of(0), in1 = make_int4(-1, 0, 0, 0);
  pb0.load(prow(in0), cbase, a.V);
  db0.load(drow(0, in0), cbase, a.V);
  if (ngroups > 1) {
    in1 = info_of(1);
    pb1.load(prow(in1), cbase, a.V);
    db1.load(drow(1, in1), cbase, a.V);
  }

  __shared__ EStage<(KC > 0 ? KC : 1), ROWS> st;
  std::conditional_t<ROWS, f16x8, bf16x8> w2[4][(KC > 0 ? KC : 1)];
  if constexpr (KC > 0) {
    const int4* info = a.info;
    const int32_t* x0 = a.x0;
    const int32_t* x = a.x;
    const int K = a.K;
    if constexpr (ROWS) {
      stage_rows<KC>(st, a.O, a.r, row0, nrow, [&](int g) {
        if constexpr (LABEL) return g;
        const int4 in = info[g];
        return in.x == 1 ? g * K + in.w : -1;
      });
    } else {
      stage_e<KC>(st, a.W1, a.r, a.V, row0, nrow, [&](int g) {
        if constexpr (LABEL) return (g % K == 0) ? x0[g / K] : x[g - 1];
        const int4 in = info[g];
        if (in.x != 1) return -1;
        return in.w == 0 ? x0[g] : x[(size_t)g * K + in.w - 1];
      });
    }
    if (col_live) {
      // the RNN head's fp16 copy of W2 is in fragment order
      std::conditional_t<ROWS, W2SwzFrags, W2Frags> wf;
      if constexpr (ROWS) wf.setup(a.W2h, KC, a.V, lane);
      else wf.setup(a.W2t, a.r, a.V, lane);
      wf.template load<KC>(n0, w2);
    }
    __syncthreads();
  }
  if (!col_live) return;

  f32x4 acc[4], nxt[4];
  if constexpr (KC > 0) mfma_group<KC>(st, 0, lane, w2, acc);
#pragma unroll
  for (int g = 0; g < kGroupsPerWG; ++g) {
    if (g >= ngroups) break;
    if constexpr (KC > 0) {
      if (g + 1 < ngroups) mfma_group<KC>(st, g + 1, lane, w2, nxt);
    }
    float t[16], z[16];
    int4 in;
    if (g & 1) {
      in = in1;
      pb1.unpack(t, cbase, a.V, in.x == 1);
      db1.unpack(z, cbase, a.V, in.x == 1);
      if (g + 2 < ngroups) {
        in1 = info_of(g + 2);
        pb1.load(prow(in1), cbase, a.V);
        db1.load(drow(g + 2, in1), cbase, a.V);
      }
    } else {
      in = in0;
      pb0.unpack(t, cbase, a.V, in.x == 1);
      db0.unpack(z, cbase, a.V, in.x == 1);
      if (g + 2 < ngroups) {
        in0 = info_of(g + 2);
        pb0.load(prow(in0), cbase, a.V);
        db0.load(drow(g + 2, in0), cbase, a.V);
      }
    }
    if constexpr (KC > 0) {
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) z[4 * b + i] += acc[b][i];
      if (g + 1 < ngroups) {
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[b] = nxt[b];
      }
    }
    const bool live = in.x == 1;
    float s = 0.f;
    if (live) {
      const float2 ms = a.rowms[in.y];
      const float lp = ms.x + fast_log2(ms.y);
      const float lq = a.lse_d[LABEL ? (size_t)req(g) : (size_t)req(g) * a.K + in.w] * kLog2e;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = fast_exp2(fmaf(t[e], a.c2, -lp));
        const float q = fast_exp2(fmaf(z[e], a.c2, -lq));
        s += fmaxf(p - q, 0.f);
      }
    }
    s += __shfl_xor(s, 16, 64);
    s += __shfl_xor(s, 32, 64);
    if (live && lane < 16) a.rpart[(size_t)req(g) * a.ns64 + slice] = s;
  }
}

// Aligned-row variant: only the compacted correcting requests stream.
// Persistent workgroups (about two per CU) pick a 128-request stage of the
// list and a range of 64-column blocks at run time, from the list length the
// decide kernel left on the device.  G = 16 (bf16 Markov verification with
// more than 128 requests): 256-request stages swept by one 8-wave workgroup
// per CU, so each W2 block a wave loads serves up to twice the rows and the
// stage's W1 rows are gathered by half as many workgroups.  Per request, the row offsets and the
// two log-normalisers sit in LDS; target and draft rows go through buffer
// resources; each draft row seeds the MFMA accumulators, so the MFMAs leave
// z = D + bias directly.
struct ResidualRow {
  uint32_t p_off, d_off;  // byte offsets of the target and draft rows
  float lp, lq;           // log2-normalisers of p and q
};

template <typename PT, typename DT, int KC, bool LABEL = false, bool ROWS = false, int G = kGroupsPerWG>
__global__ __launch_bounds__(G * 32) __attribute__((amdgpu_waves_per_eu(2)))
void verify_residual_stream_kernel(VerifyArgs a) {
  constexpr int kRows = 16 * G;  // requests per stage
  constexpr int kWaves = G / 2;  // waves per workgroup
  static_assert(G == kGroupsPerWG || (G == 2 * kGroupsPerWG && !ROWS && KC > 0 && std::is_same_v<PT, uint16_t> &&
                                      std::is_same_v<DT, uint16_t>),
                "256-request stages: bf16 rows of the Markov head only");
  // LABEL: one item per (request, position) pair, item i = r * K + k, with
  // target row i and draft row i; otherwise the compacted correcting requests
  const int count = LABEL ? a.R * a.K : *a.rej_count;
  if (count <= 0) return;
  const int active = (count + kRows - 1) / kRows;
  const int slots = gridDim.x / 8;
  const int per_stage = slots / active;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int stage = slot % active, sp = slot / active;
  if (sp >= per_stage) return;
  const int nsplit = per_stage * 8, split = sp * 8 + xcd;
  const int lane = threadIdx.x & 63;
  const int wave = wave_index();
  const int row0 = stage * kRows;
  const int nrows = min(kRows, count - row0);
  const int ngroups = (nrows + 15) / 16;
  const int nblocks = (a.V + kWaveCols - 1) / kWaveCols;
  const int blk_begin = (int)((int64_t)split * nblocks / nsplit);
  const int blk_end = (int)((int64_t)(split + 1) * nblocks / nsplit);

  __shared__ ResidualRow rows[kRows];
  __shared__ EStage<(KC > 0 ? KC : 1), ROWS, kRows> st;
  if (threadIdx.x < kRows) {
    ResidualRow rr{0u, 0u, 0.f, 0.f};
    if ((int)threadIdx.x < nrows) {
      const int item = row0 + threadIdx.x;
      const int r = LABEL ? item : a.rej_list[item];
      const int4 in = LABEL ? make_int4(1, item, 0, 0) : a.info[r];
      const uint64_t drow = LABEL ? (uint64_t)item : (uint64_t)r * a.K + in.w;
      const float2 ms = a.rowms[in.y];
      rr.p_off = (uint32_t)((uint64_t)in.y * a.V * sizeof(PT));
      rr.d_off = (uint32_t)(drow * a.V * sizeof(DT));
      rr.lp = ms.x + fast_log2(ms.y);
      rr.lq = a.lse_d[drow] * kLog2e;
    }
    rows[threadIdx.x] = rr;
  }
  std::conditional_t<ROWS, f16x8, bf16x8> w2[4][(KC > 0 ? KC : 1)];
  // fragment-ordered W2 (one contiguous KB per fragment load): the label's
  // Markov pass and the RNN head's fp16 copy; Markov verification reads the
  // caller's fragment-ordered copy when given, else the column-major W2
  constexpr bool SWZ = LABEL || ROWS;
  std::conditional_t<SWZ, W2SwzFrags, W2AnyFrags> wf;
  if constexpr (KC > 0) {
    // the wave's first W2 block is requested before the stage's gather (it
    // does not depend on it), so the two latencies overlap
    if constexpr (SWZ) wf.setup(ROWS ? a.W2h : a.W2s, KC, a.V, lane);
    else wf.setup(a.W2t, a.W2s, a.r, a.V, lane);
    if (blk_begin + wave < blk_end) wf.template load<KC>((blk_begin + wave) * kWaveCols, w2);
    const int32_t* list = a.rej_list;
    const int4* info = a.info;
    const int32_t* x0 = a.x0;
    const int32_t* x = a.x;
    const int K = a.K;
    if constexpr (ROWS) {
      stage_rows<KC>(st, a.O, a.r, row0, count, [&](int g) {
        if constexpr (LABEL) return g;
        const int r = list[g];
        return r * K + info[r].w;
      });
    } else {
      stage_e<KC>(st, a.W1, a.r, a.V, row0, count, [&](int g) {
        if constexpr (LABEL) return (g % K == 0) ? x0[g / K] : x[g - 1];
        const int r = list[g];
        const int4 in = info[r];
        return in.w == 0 ? x0[r] : x[(size_t)r * K + in.w - 1];
      });
    }
  }
  __syncthreads();

  const rsrc_t prs = make_rsrc(a.P, (uint32_t)((uint64_t)a.N * a.V * sizeof(PT)));
  const rsrc_t drs = make_rsrc(a.D, (uint32_t)((uint64_t)a.R * a.K * a.V * sizeof(DT)));
  const uint32_t lane_col = (uint32_t)(16 * (lane >> 4));
  auto row_info = [&](int g) { return rows[16 * g + (lane & 15)]; };
  auto live = [&](int g) { return 16 * g + (lane & 15) < nrows; };
  // CX: bf16 target and draft rows are read coalesced: lane l takes the 16
  // bytes at 16 (l % 8) of the block's 128-byte segment of rows l / 8 (w[0])
  // and 8 + l / 8 (w[1]) of the group, so one load instruction covers eight
  // whole segments, and the group goes into the MFMA layout (lane l: 32
  // bytes of row l % 16) through this wave's LDS tile (row pitch 144 bytes).
  // The lanes end up with the bytes the MFMA-layout loads would have read.
  // One tile serves both rows: LDS operations of a wave complete in order.
  constexpr bool CX = std::is_same_v<PT, uint16_t> && std::is_same_v<DT, uint16_t>;
  __shared__ u32x4 xtile[CX ? kWaves : 1][16 * 9];
  auto cload = [&](GroupLogitsBuf<PT>& pb, GroupLogitsBuf<DT>& db, int g, int blk) {
    if constexpr (CX) {
      const ResidualRow r0 = rows[16 * g + (lane >> 3)], r1 = rows[16 * g + 8 + (lane >> 3)];
      const uint32_t c = (uint32_t)blk * kWaveCols * 2u + 16u * (uint32_t)(lane & 7);
      // target and draft rows are read once here: non-temporal, so that
      // they do not displace W2, which every block of the pass reads again
      pb.w[0] = buffer_load16_nt(prs, r0.p_off + c, 0u);
      pb.w[1] = buffer_load16_nt(prs, r1.p_off + c, 0u);
      db.w[0] = buffer_load16_nt(drs, r0.d_off + c, 0u);
      db.w[1] = buffer_load16_nt(drs, r1.d_off + c, 0u);
    }
  };
  auto xpose = [&](auto& b) {
    if constexpr (CX) {
      xtile[wave][(lane >> 3) * 9 + (lane & 7)] = b.w[0];
      xtile[wave][(8 + (lane >> 3)) * 9 + (lane & 7)] = b.w[1];
      b.w[0] = xtile[wave][(lane & 15) * 9 + 2 * (lane >> 4)];
      b.w[1] = xtile[wave][(lane & 15) * 9 + 2 * (lane >> 4) + 1];
    }
  };

  // CX: two groups in flight (group g + 2 is requested into g's buffers).
  // PF (the label, whose waves sweep tens of blocks; verification's sweep a
  // few and measured slower with it): also across blocks when the group
  // count is even (group 0 / 1 of the next block go into the buffers of the
  // last two), and the next block's W2 fragments are requested during the
  // last group's MFMAs
  constexpr bool PF = CX && LABEL;
  GroupLogitsBuf<PT> pb0, pb1;
  GroupLogitsBuf<DT> db0, db1;
  const bool xpf = PF && ngroups % 2 == 0;
  bool first = true;
  // LABEL: this wave's sums for rows lane, 64 + lane, ... of the stage (named
  // registers: an array indexed by the group stayed in scratch memory)
  double lacc0 = 0.0, lacc1 = 0.0, lacc2 = 0.0, lacc3 = 0.0;
  for (int blk = blk_begin + wave; blk < blk_end; blk += kWaves) {
    const int nxt = blk + kWaves;
    const bool has_next = nxt < blk_end;
    const int cbase = blk * kWaveCols + (int)lane_col;
    const uint32_t pcol = (uint32_t)cbase * sizeof(PT), dcol = (uint32_t)cbase * sizeof(DT);
    if constexpr (KC > 0) {
      if (!PF && !first) wf.template load<KC>(blk * kWaveCols, w2);  // the first block's was requested above
    }
    const int e_off = launder(e_lane_offset<(KC > 0 ? KC : 1), ROWS>(lane));
    // one group in the MFMA layout: the draft rows seed the accumulators, the
    // MFMAs add the bias, and the residual mass of the 64 columns is stored;
    // refill requests a later group's rows into the freed buffers before the
    // epilogue; pf: the block's last group, whose MFMAs are split in two
    // halves so that each half's W2 registers take the next block's
    // fragments as soon as the MFMAs reading them have issued
    auto group = [&](int g, const ResidualRow& cur, GroupLogitsBuf<PT>& pb, GroupLogitsBuf<DT>& db, auto refill,
                     bool pf) {
      const bool lv = live(g);
      float u[16];
      db.unpack(u, cbase, a.V, lv);
      f32x4 acc[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[b] = f32x4{u[4 * b], u[4 * b + 1], u[4 * b + 2], u[4 * b + 3]};
      if constexpr (KC > 0) {
        if (!pf) {
          mfma_group<KC, false>(st, g, lane, w2, acc, e_off);
        } else {
          constexpr int KH = KC / 2;
          mfma_group<KC, false, 0, KH>(st, g, lane, w2, acc, e_off);
          __builtin_amdgcn_sched_barrier(0);
          wf.template load_range_if<KC, 0, KH>(nxt * kWaveCols, has_next, w2);
          __builtin_amdgcn_sched_barrier(0);
          mfma_group<KC, false, KH, KC>(st, g, lane, w2, acc, e_off);
          __builtin_amdgcn_sched_barrier(0);
          wf.template load_range_if<KC, KH, KC>(nxt * kWaveCols, has_next, w2);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      float t[16];
      pb.unpack(t, cbase, a.V, lv);
      refill(pb, db);
      float s = 0.f;
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = 4 * b + i;
          const float p = fast_exp2(fmaf(t[e], a.c2, -cur.lp));
          const float q = fast_exp2(fmaf(acc[b][i], a.c2, -cur.lq));
          s += fmaxf(p - q, 0.f);
        }
      s = rows_sum(s);
      if constexpr (LABEL) {
        // the label needs each item's total only: group g's row sums are kept
        // by the lanes of quarter g % 4 (lane l ends with rows l, 64 + l, ...
        // of the stage), added in block order in fp64
        const double ds = (lane >> 4) == (g & 3) ? (double)s : 0.0;
        // rows 64 q + lane come from groups 4 q .. 4 q + 3 (the sums are >= 0,
        // so adding 0.0 to the other accumulators leaves them unchanged)
        const int q = g >> 2;
        lacc0 += q == 0 ? ds : 0.0;
        lacc1 += q == 1 ? ds : 0.0;
        if constexpr (G > 8) {
          lacc2 += q == 2 ? ds : 0.0;
          lacc3 += q == 3 ? ds : 0.0;
        }
      } else if (lv && lane < 16) {
        a.rpart[(size_t)a.rej_list[row0 + 16 * g + lane] * a.ns64 + blk] = s;
      }
    };
    if constexpr (CX) {
      if (first || !xpf) {
        cload(pb0, db0, 0, blk);
        if (ngroups > 1) cload(pb1, db1, 1, blk);
      }
      auto step = [&](int g, GroupLogitsBuf<PT>& pb, GroupLogitsBuf<DT>& db) {
        xpose(db);
        xpose(pb);
        group(g, row_info(g), pb, db, [&](GroupLogitsBuf<PT>& np, GroupLogitsBuf<DT>& nd) {
          if (g + 2 < ngroups) cload(np, nd, g + 2, blk);
          else if (xpf && has_next) cload(np, nd, g + 2 - ngroups, nxt);
        }, PF && g + 1 == ngroups);
      };
      for (int g = 0; g < ngroups; g += 2) {
        step(g, pb0, db0);
        if (g + 1 < ngroups) step(g + 1, pb1, db1);
      }
    } else {
      ResidualRow ri = row_info(0);
      pb0.load(prs, ri.p_off + pcol, 0u);
      db0.load(drs, ri.d_off + dcol, 0u);
      for (int g = 0; g < ngroups; ++g) {
        const ResidualRow cur = ri;
        group(g, cur, pb0, db0, [&](GroupLogitsBuf<PT>& np, GroupLogitsBuf<DT>& nd) {
          if (g + 1 < ngroups) {  // the next group's rows
            ri = row_info(g + 1);
            np.load(prs, ri.p_off + pcol, 0u);
            nd.load(drs, ri.d_off + dcol, 0u);
          }
        }, false);
      }
    }
    first = false;
  }
  if constexpr (LABEL) {
    // one partial per (job, item), jobs = (split, wave); written even when the
    // wave had no block (zeros), so every partial the reduction reads is set
    const size_t job = (size_t)split * kWaves + wave;
    const double sums[4] = {lacc0, lacc1, lacc2, lacc3};
#pragma unroll
    for (int q = 0; q < G / 4; ++q)
      if (64 * q + lane < nrows) a.lpart[job * count + row0 + 64 * q + lane] = sums[q];
  }
}

// ------------------------------------------------------------------ sample --
// Inverse-CDF over slice masses w_s (fp64 running sums: thousands of slices
// per row): the slice where the running sum first exceeds target and the mass
// before it.  Lanes own contiguous slice chunks.
struct SliceHit {
  int slice;
  double before;
};

constexpr int kSamPer = 40;  // slices per lane held in registers by the sample kernel

template <typename WeightFn>
__device__ __forceinline__ SliceHit find_slice(int ns, double target, double incl, double local, int s_begin,
                                               int s_end, WeightFn weight) {
  const int lane = threadIdx.x & 63;
  int owner = wave_first_lane(incl > target);
  if (owner < 0) {
    const unsigned long long m = __ballot(local > 0.0);
    owner = m ? 63 - __clzll((long long)m) : 0;
  }
  int s_star = -1;
  double before = 0.0;
  if (lane == owner) {
    double acc = incl - local;
    int last = -1;
    double last_before = acc;
    for (int s = s_begin; s < s_end; ++s) {
      const double w = weight(s);
      if (w > 0.0) {
        last = s;
        last_before = acc;
        if (acc + w > target) {
          s_star = s;
          before = acc;
          break;
        }
      }
      acc += w;
    }
    if (s_star < 0) {
      s_star = last;
      before = last_before;
    }
  }
  SliceHit h;
  h.slice = __shfl(s_star, owner, 64);
  h.before = __shfl(before, owner, 64);
  if (h.slice < 0 || h.slice >= ns) h.slice = 0;
  return h;
}

// The crossing of `target` over slice weights held in registers (lane l's
// contiguous run w[0..N) of slices s0.., fp32 values whose running sum is
// kept in fp64): the owner lane (the first whose inclusive sum passes the
// target, else the last with mass) puts its run in this wave's LDS slots
// `run`, lane i takes entry i, and an fp64 wave scan finds the first entry
// with mass whose running sum passes the target, else the last with mass.
// Returns the slice (0 when nothing has mass) and the mass before it; `pick`
// is the entry's index in the owner's run (-1 when nothing has mass).  LDS
// accesses of one wave complete in order: no barrier.
template <int N, typename T>
__device__ __forceinline__ SliceHit cross_in_run(double target, double incl, double local, int s0, int ns,
                                                 const T (&run_regs)[N], T* run, float (*weight)(T, float),
                                                 float M, int lane, int& pick) {
  int owner = wave_first_lane(incl > target);
  if (owner < 0) {
    const unsigned long long m = __ballot(local > 0.0);
    owner = m ? 63 - __clzll((long long)m) : 0;
  }
  if (lane == owner) {
#pragma unroll
    for (int i = 0; i < N; ++i) run[i] = run_regs[i];
  }
  const double acc0 = __shfl(incl - local, owner, 64);
  const int os0 = __shfl(s0, owner, 64);
  const double w = lane < N ? (double)weight(run[lane < N ? lane : 0], M) : 0.0;
  const double cum = acc0 + wave_inclusive_scan_dpp(w);
  pick = wave_first_lane(cum > target && w > 0.0);
  if (pick < 0) {  // rounding: the last entry with mass
    const unsigned long long m = __ballot(w > 0.0);
    pick = m ? 63 - __clzll((long long)m) : -1;
  }
  SliceHit h;
  if (pick < 0) {
    h.slice = 0;
    h.before = acc0;
  } else {
    h.slice = os0 + pick;
    h.before = __shfl(cum - w, pick, 64);
  }
  if (h.slice >= ns) h.slice = 0;
  return h;
}

__device__ __forceinline__ float mass_of(float w, float) { return w; }
__device__ __forceinline__ float mass_of_part(float2 q, float M) {
  return q.x == -INFINITY ? 0.f : q.y * fast_exp2(q.x - M);
}

// One wave per request.  Correction: the residual slice masses of the
// request are requested together with its decision (branch-free buffer
// loads, all in flight), the bias input row (W1[x_{j-1}] or the RNN output
// part) while they are reduced, and the crossing slice's 64 columns are
// re-evaluated (draft base logit + bias from the staged row and the slice's
// W2 block, target logit) with every load requested together.  Bonus (or a
// correction with no residual mass): the target row's 2048-column partials,
// then the crossing slice's 2048 logits.
template <typename PT, typename DT>
__global__ __launch_bounds__(256) void verify_sample_kernel(VerifyArgs a) {
  const int lane = threadIdx.x & 63;
  const int wv = wave_index();
  const int r = blockIdx.x * 4 + wv;
  if (r >= a.R) return;
  __shared__ u32x4 sh_row[4][kMaxRankRow];
  __shared__ float sh_run[4][kSamPer];
  __shared__ float2 sh_prun[4][kSamPer];
  __shared__ float sh_bonus[4][kRowSlice / 64];

  // correction weights: requested before the decision is known (a request
  // that takes the bonus leaves them unused)
  const int ns64 = a.ns64;
  const int per64 = (ns64 + 63) / 64;
  const int c0 = min(ns64, lane * per64), c1 = min(ns64, c0 + per64);
  const bool cregs = per64 <= kSamPer;
  float cw[kSamPer];
  if (cregs) {
    const rsrc_t rr = make_rsrc(a.rpart + (size_t)r * ns64, (uint32_t)ns64 * 4u);
#pragma unroll
    for (int i = 0; i < kSamPer; ++i)
      cw[i] = __uint_as_float(
          __builtin_amdgcn_raw_buffer_load_b32(rr, (int)((c0 + i < c1) ? (uint32_t)(c0 + i) * 4u : (uint32_t)ns64 * 4u), 0, 0));
  }
  const int4 in = a.info[r];
  __builtin_amdgcn_sched_barrier(0);
  if (in.x < 0) return;  // decide already wrote -1
  const float u = decision_uniform(a.seed, a.step, (uint32_t)r, (uint32_t)in.z, kPurposeResample);
  const PT* prow = reinterpret_cast<const PT*>(a.P) + (size_t)in.y * a.V;
  const float2 ms = a.rowms[in.y];
  const float lp = ms.x + fast_log2(ms.y);
  bool use_p = in.x == 0;

  if (!use_p) {
    // the bias input row (its address waits for the previous token), staged
    // in LDS once the crossing is known; lanes past r read zeros
    const size_t drow = (size_t)r * a.K + in.w;
    const int prev = in.w == 0 ? a.x0[r] : a.x[drow - 1];
    const bool prev_ok = prev >= 0 && prev < a.V;
    u32x4 row_in = u32x4{0u, 0u, 0u, 0u};
    if (a.r > 0) {
      const int n = a.O ? a.r / 4 : a.r / 8;
      const rsrc_t rr = a.O ? make_rsrc(a.O + drow * a.r, (uint32_t)a.r * 4u)
                            : make_rsrc(a.W1 + (size_t)(prev_ok ? prev : 0) * a.r, (uint32_t)a.r * 2u);
      row_in = buffer_load16(rr, ((a.O || prev_ok) && lane < n) ? (uint32_t)lane * 16u : 0xFFFFFFF0u, 0u);
    }
    double local = 0.0;
    if (cregs) {
      double l4[4] = {0.0, 0.0, 0.0, 0.0};  // four chains in flight
#pragma unroll
      for (int i = 0; i < kSamPer; ++i) l4[i & 3] += (double)cw[i];  // past the run: read as zero
      local = (l4[0] + l4[1]) + (l4[2] + l4[3]);
    } else {
      const float* rp = a.rpart + (size_t)r * ns64;
      for (int s = c0; s < c1; ++s) local += (double)rp[s];
    }
    const double incl = wave_inclusive_scan_dpp(local);
    const double Z = __shfl(incl, 63, 64);
    if (Z > 0.0 && Z <= 2.0) {
      const double target = (double)u * Z;
      SliceHit h;
      if (cregs) {
        int pk;
        h = cross_in_run<kSamPer, float>(target, incl, local, c0, ns64, cw, sh_run[wv], mass_of, 0.f, lane, pk);
      } else {
        const float* rp = a.rpart + (size_t)r * ns64;
        h = find_slice(ns64, target, incl, local, c0, c1, [&](int s) { return (double)rp[s]; });
      }
      sh_row[wv][lane] = row_in;
      // the slice's 64 columns, one per lane: draft and target logits and the
      // W2 block requested together (a column past V reads zero, no branch)
      const int col = h.slice * kWaveCols + lane;
      const bool col_ok = col < a.V;
      const rsrc_t dr = make_rsrc(reinterpret_cast<const DT*>(a.D) + drow * a.V, (uint32_t)a.V * (uint32_t)sizeof(DT));
      const rsrc_t pr = make_rsrc(prow, (uint32_t)a.V * (uint32_t)sizeof(PT));
      const uint32_t doff = col_ok ? (uint32_t)col * (uint32_t)sizeof(DT) : 0xFFFFFFF0u;
      const uint32_t poff = col_ok ? (uint32_t)col * (uint32_t)sizeof(PT) : 0xFFFFFFF0u;
      float zq, zp;
      if constexpr (sizeof(DT) == 2)
        zq = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(dr, (int)doff, 0, 0) << 16);
      else
        zq = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(dr, (int)doff, 0, 0));
      if constexpr (sizeof(PT) == 2)
        zp = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(pr, (int)poff, 0, 0) << 16);
      else
        zp = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(pr, (int)poff, 0, 0));
      if (a.r > 0 && (a.O || prev_ok)) {
        const int kc_count = (a.r + 31) / 32;
        const bool swz = a.W2s != nullptr && a.O == nullptr;
        const uint32_t w2_bytes = swz ? (uint32_t)((size_t)((a.V + kWaveCols - 1) / kWaveCols) * 4 * kc_count * 1024)
                                      : (uint32_t)((size_t)a.V * a.r * 2);
        const rsrc_t w2 = make_rsrc(swz ? static_cast<const void*>(a.W2s) : static_cast<const void*>(a.W2t), w2_bytes);
        const uint32_t off0 = swz ? (uint32_t)h.slice * 4u * (uint32_t)kc_count * 1024u
                                  : (uint32_t)(col_ok ? col : 0) * (uint32_t)a.r * 2u;
        zq += a.O ? lane_bias_staged<true>(sh_row[wv], w2, w2_bytes, off0, false, a.r, col_ok, lane)
                  : lane_bias_staged<false>(sh_row[wv], w2, w2_bytes, off0, swz, a.r, col_ok, lane);
      }
      const float lq = a.lse_d[drow] * kLog2e;
      float rho = 0.f;
      if (col_ok) {
        const float p = fast_exp2(fmaf(zp, a.c2, -lp));
        const float q = fast_exp2(fmaf(zq, a.c2, -lq));
        rho = fmaxf(p - q, 0.f);
      }
      const float t_in = (float)(target - h.before);
      const float cum = wave_inclusive_scan_dpp(rho);
      int pick = wave_first_lane(cum > t_in && rho > 0.f);
      // the draw's margin: distance of the target from the nearer CDF edge of
      // the drawn column, over the total mass (0 when rounding picked it)
      float edge = INFINITY;
      if (pick >= 0) {
        const float hi = __shfl(cum, pick, 64), w = __shfl(rho, pick, 64);
        edge = fminf(hi - t_in, t_in - (hi - w));
      } else {
        const unsigned long long m = __ballot(rho > 0.f);
        pick = m ? 63 - __clzll((long long)m) : 0;
        edge = 0.f;
      }
      if (lane == 0) {
        a.tok_out[r] = h.slice * kWaveCols + pick;
        if (a.min_margin_out) a.min_margin_out[r] = fminf(a.rmin[r], (float)((double)edge / Z));
      }
      return;
    }
    use_p = true;  // zero residual mass (rounding only): draw from p
  }

  // bonus (or fallback): target partials per 2048-column slice
  const float2* pp = a.ppart + (size_t)in.y * a.nsP;
  const int ns = a.nsP;
  const int per = (ns + 63) / 64;
  const int s_begin = min(ns, lane * per), s_end = min(ns, s_begin + per);
  const bool regs = per <= kSamPer;
  float2 pv[kSamPer];
  float M = -INFINITY;
  if (regs) {
    const rsrc_t prr = make_rsrc(pp, (uint32_t)ns * 8u);
#pragma unroll
    for (int i = 0; i < kSamPer; ++i)
      pv[i] = buffer_load8(prr, (s_begin + i < s_end) ? (uint32_t)(s_begin + i) * 8u : (uint32_t)ns * 8u, 0u);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kSamPer; ++i)
      if (s_begin + i >= s_end) pv[i].x = -INFINITY;  // past the run (read as zeros): no mass
#pragma unroll
    for (int i = 0; i < kSamPer; ++i) M = fmaxf(M, pv[i].x);
  } else {
    for (int s = lane; s < ns; s += 64) M = fmaxf(M, pp[s].x);
  }
  M = wave_max(M);
  auto weight = [&](int s) {
    const float2 p = pp[s];
    return (p.x == -INFINITY) ? 0.0 : (double)(p.y * fast_exp2(p.x - M));
  };
  double local = 0.0;
  if (regs) {
    double l4[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int i = 0; i < kSamPer; ++i) l4[i & 3] += (double)mass_of_part(pv[i], M);
    local = (l4[0] + l4[1]) + (l4[2] + l4[3]);
  } else {
    for (int s = s_begin; s < s_end; ++s) local += weight(s);
  }
  const double incl = wave_inclusive_scan_dpp(local);
  const double S = __shfl(incl, 63, 64);
  const double target = (double)u * S;
  SliceHit h;
  float m_s;
  if (regs) {
    int pk;
    h = cross_in_run<kSamPer, float2>(target, incl, local, s_begin, ns, pv, sh_prun[wv], mass_of_part, M, lane, pk);
    m_s = pk >= 0 ? sh_prun[wv][pk].x : pp[h.slice].x;
  } else {
    h = find_slice(ns, target, incl, local, s_begin, s_end, weight);
    m_s = pp[h.slice].x;
  }
  // the target inside the slice, in the slice's own scale (fp64: 2048 terms)
  const double t_in = (target - h.before) / (double)fast_exp2(m_s - M);
  // the slice's columns, kBonusPer consecutive per lane (16-byte loads when
  // whole vectors lie inside the row, past V reading zero)
  constexpr int kBonusPer = kRowSlice / 64;
  float e[kBonusPer];
  double lsum = 0.0;
  {
    const int col0 = h.slice * kRowSlice + kBonusPer * lane;
    const rsrc_t pr = make_rsrc(prow, (uint32_t)a.V * (uint32_t)sizeof(PT));
    constexpr int EPL = 16 / sizeof(PT);
    float v[kBonusPer];
    if (a.V % EPL == 0) {
#pragma unroll
      for (int q = 0; q < kBonusPer / EPL; ++q) {
        const int c = col0 + EPL * q;
        const u32x4 d = buffer_load16(pr, c < a.V ? (uint32_t)c * (uint32_t)sizeof(PT) : 0xFFFFFFF0u, 0u);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if constexpr (sizeof(PT) == 2) {
            v[EPL * q + 2 * k] = __uint_as_float(d[k] << 16);
            v[EPL * q + 2 * k + 1] = __uint_as_float(d[k] & 0xFFFF0000u);
          } else {
            v[EPL * q + k] = __uint_as_float(d[k]);
          }
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < kBonusPer; ++k) v[k] = (col0 + k < a.V) ? load_logit(prow, col0 + k) : 0.f;
    }
    double l4[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int k = 0; k < kBonusPer; ++k) {
      e[k] = (col0 + k < a.V) ? fast_exp2(v[k] * a.c2 - m_s) : 0.f;
      l4[k & 3] += (double)e[k];
    }
    lsum = (l4[0] + l4[1]) + (l4[2] + l4[3]);
  }
  const double incl2 = wave_inclusive_scan_dpp(lsum);
  int owner = wave_first_lane(incl2 > t_in && lsum > 0.0);
  if (owner < 0) {
    const unsigned long long m = __ballot(lsum > 0.0);
    owner = m ? 63 - __clzll((long long)m) : 0;
  }
  // the owner's kBonusPer values through LDS (in-order LDS access within the
  // wave: no barrier), lane i takes value i, and an fp64 wave scan finds the
  // first column with mass whose running sum passes the target, else the
  // last column with mass
  if (lane == owner) {
#pragma unroll
    for (int k = 0; k < kBonusPer; ++k) sh_bonus[wv][k] = e[k];
  }
  const double acc0 = __shfl(incl2 - lsum, owner, 64);
  const double w = lane < kBonusPer ? (double)sh_bonus[wv][lane < kBonusPer ? lane : 0] : 0.0;
  const double cum = acc0 + wave_inclusive_scan_dpp(w);
  int pick = wave_first_lane(cum > t_in && w > 0.0);
  double edge = 0.0;  // distance of the target from the drawn column's CDF edges (0: picked by rounding)
  if (pick >= 0) {
    const double hi = __shfl(cum, pick, 64), wp = __shfl(w, pick, 64);
    edge = fmin(hi - t_in, t_in - (hi - wp));
  } else {
    const unsigned long long m = __ballot(w > 0.0);
    pick = m ? 63 - __clzll((long long)m) : 0;
  }
  if (lane == 0) {
    a.tok_out[r] = h.slice * kRowSlice + kBonusPer * owner + pick;
    if (a.min_margin_out) {
      // the slice's values are scaled by 2^(M - m_s) against the masses summing to S
      const float mg = S > 0.0 ? (float)(edge * (double)fast_exp2(m_s - M) / S) : 0.f;
      a.min_margin_out[r] = fminf(a.rmin[r], mg);
    }
  }
}

// ------------------------------------------------------------------ host ---
static size_t align256(size_t n) { return (n + 255) / 256 * 256; }

struct VerifyLayout {
  size_t ppart, rowms, flag, info, rpart, rej, margin, rmin, ppart2, lse, dpart, w2s, total;
};

size_t draft_workspace_bytes(int B, int K, int V);
size_t w2_swizzle_bytes(int V, int r);
int run_w2_swizzle(const uint16_t* W2, void* out, int V, int r, int kc, bool f16, hipStream_t stream);

// lse_pass: room to recompute the draft rows' log-normalisers (r == 0: the
// rowstats partials of the R * K draft rows; r > 0: the draft's slice
// partials of one position, plus the fragment-ordered W2 when make_w2s).
// margins: the per-row decision margins and the greedy runner-ups.
static VerifyLayout verify_layout(int R, int K, int V, int N, int r, bool lse_pass, bool make_w2s, bool margins) {
  VerifyLayout l{};
  const size_t nsP = (size_t)(((int64_t)V + kRowSlice - 1) / kRowSlice);
  const size_t ns64 = (size_t)(((int64_t)V + kWaveCols - 1) / kWaveCols);
  size_t off = 0;
  auto take = [&](size_t& at, size_t bytes) {
    at = off;
    off += align256(bytes);
  };
  take(l.ppart, (size_t)N * nsP * sizeof(float2));
  take(l.rowms, (size_t)N * sizeof(float2));
  take(l.flag, (size_t)N * sizeof(int32_t));
  take(l.info, (size_t)R * sizeof(int4));
  take(l.rpart, (size_t)R * ns64 * sizeof(float));
  take(l.rej, (size_t)(R + 1) * sizeof(int32_t));
  take(l.margin, margins ? (size_t)N * sizeof(float) : 0);
  take(l.rmin, margins ? (size_t)R * sizeof(float) : 0);
  take(l.ppart2, margins ? (size_t)N * nsP * sizeof(float) : 0);
  take(l.lse, lse_pass ? (size_t)R * K * sizeof(float) : 0);
  take(l.dpart, !lse_pass ? 0 : r == 0 ? (size_t)R * K * nsP * sizeof(float2) : draft_workspace_bytes(R, K, V));
  take(l.w2s, (lse_pass && r > 0 && make_w2s) ? w2_swizzle_bytes(V, r) : 0);
  l.total = off;
  return l;
}

// The query: enough for every combination of optional inputs and outputs.
size_t verify_workspace_bytes(int R, int K, int V, int r, int N) {
  return verify_layout(R, K, V, N, r, true, true, true).total;
}
size_t verify_workspace_need(int R, int K, int V, int r, int N, bool lse_given, bool w2f_given, bool margins,
                             float temperature) {
  const bool lse_pass = !lse_given && temperature > 0.f;
  return verify_layout(R, K, V, N, r, lse_pass, !w2f_given, margins).total;
}

// Log-normaliser of each row from its 2048-column rowstats partials (one wave
// per row): lse = (M + log2 S) ln 2, the draft's convention.
__global__ __launch_bounds__(256) void row_lse_kernel(const float2* __restrict__ part, int nrows, int ns,
                                                      float* __restrict__ lse) {
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + wave_index();
  if (i >= nrows) return;
  float m, s;
  int idx;
  merge_row<false>(part + (size_t)i * ns, ns, m, s, idx);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float om = __shfl_xor(m, off, 64);
    const float os = __shfl_xor(s, off, 64);
    merge_ms(m, s, om, os);
  }
  if (lane == 0) lse[i] = (m + fast_log2(s)) * kLn2;
}

// ------------------------------------------------------- acceptance label --
// c*_i = 1 - 1/2 ||q_i - p_i||_1 for every (request, position) item
// i = r * K + k (DSpark paper, section 3.2.1: the confidence head's label is
// the per-step acceptance rate fixed by the total variation distance between
// the draft and target distributions; "Speculative decoding, from zero to
// DSpark", section 2).  The passes of verification are reused: row
// statistics of the target rows, their merge into the normaliser below, the
// residual mass sum_v max(0, p - q) per 64-column slice (the LABEL mapping of
// the residual kernels), and 1 minus its fp64 total here.  Greedy: c* is 1
// where the target row's first argmax is the drafted token.
template <bool GREEDY>
__global__ __launch_bounds__(256) void label_merge_kernel(VerifyArgs a) {
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + wave_index();
  if (i >= a.N) return;
  const float2* part = a.ppart + (size_t)i * a.nsP;
  float m, s;
  int idx;
  merge_row<GREEDY>(part, a.nsP, m, s, idx);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float m2 = __shfl_xor(m, off, 64);
    if constexpr (GREEDY) {
      const int i2 = __shfl_xor(idx, off, 64);
      merge_argmax(m, idx, m2, i2);
    } else {
      const float s2 = __shfl_xor(s, off, 64);
      merge_ms(m, s, m2, s2);
    }
  }
  if (lane == 0) a.rowms[i] = GREEDY ? make_float2(m, __int_as_float(idx)) : make_float2(m, s);
}

template <bool GREEDY>
__global__ __launch_bounds__(256) void label_reduce_kernel(VerifyArgs a, float* __restrict__ c_out) {
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + wave_index();
  if (i >= a.N) return;
  const int k = i % a.K;
  const int prev = k == 0 ? a.x0[i / a.K] : a.x[i - 1];
  const int xi = a.x[i];
  const bool ok = prev >= 0 && prev < a.V && xi >= 0 && xi < a.V;
  if constexpr (GREEDY) {
    if (lane == 0) c_out[i] = ok ? ((__float_as_int(a.rowms[i].y) == xi) ? 1.f : 0.f) : NAN;
    return;
  }
  const float* rp = a.rpart + (size_t)i * a.ns64;
  double z = 0.0;
  for (int s = lane; s < a.ns64; s += 64) z += (double)rp[s];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) z += __shfl_xor(z, off, 64);
  if (lane == 0) c_out[i] = ok ? (float)fmin(1.0, fmax(0.0, 1.0 - z)) : NAN;
}

// The label from the streamed residual pass: c = 1 - (sum over jobs, in job
// order, of the item's fp64 partial sums), one thread per item.
__global__ __launch_bounds__(256) void label_reduce_jobs_kernel(VerifyArgs a, float* __restrict__ c_out) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= a.N) return;
  const int k = i % a.K;
  const int prev = k == 0 ? a.x0[i / a.K] : a.x[i - 1];
  const int xi = a.x[i];
  const bool ok = prev >= 0 && prev < a.V && xi >= 0 && xi < a.V;
  double z = 0.0;
#pragma unroll 8
  for (int j = 0; j < a.njobs; ++j) z += a.lpart[(size_t)j * a.N + i];
  c_out[i] = ok ? (float)fmin(1.0, fmax(0.0, 1.0 - z)) : NAN;
}

template <typename PT, typename DT, bool VEC_P, bool VEC_D, int KC, bool LABEL, bool ROWS = false>
static int launch_residual(const VerifyArgs& a, hipStream_t stream) {
  return launch_kernel(LABEL ? "label_residual" : "verify_residual",
                       verify_residual_kernel<PT, DT, VEC_P, VEC_D, KC, LABEL, ROWS>,
                       dim3(xcd_grid(a.ncol_tiles, a.nstages)), dim3(256), stream, a);
}

template <typename PT, typename DT, bool VEC_P, bool VEC_D, bool LABEL = false>
static int dispatch_residual(const VerifyArgs& a, hipStream_t stream) {
  // RNN head: one variant, r <= 256 zero-padded to eight chunks
  if (a.O) return launch_residual<PT, DT, VEC_P, VEC_D, 8, LABEL, true>(a, stream);
  switch ((a.r + 31) / 32) {
    case 0: return launch_residual<PT, DT, VEC_P, VEC_D, 0, LABEL>(a, stream);
    case 1: return launch_residual<PT, DT, VEC_P, VEC_D, 1, LABEL>(a, stream);
    case 2: return launch_residual<PT, DT, VEC_P, VEC_D, 2, LABEL>(a, stream);
    case 3: return launch_residual<PT, DT, VEC_P, VEC_D, 3, LABEL>(a, stream);
    case 4: return launch_residual<PT, DT, VEC_P, VEC_D, 4, LABEL>(a, stream);
    case 5: return launch_residual<PT, DT, VEC_P, VEC_D, 5, LABEL>(a, stream);
    case 6: return launch_residual<PT, DT, VEC_P, VEC_D, 6, LABEL>(a, stream);
    case 7: return launch_residual<PT, DT, VEC_P, VEC_D, 7, LABEL>(a, stream);
    case 8: return launch_residual<PT, DT, VEC_P, VEC_D, 8, LABEL>(a, stream);
    default: return -1;
  }
}

// Grid of the streamed residual pass over `rows` items: about two workgroups
// per CU (one for 256-row stages), and enough 8-slot rows for every stage.
static int residual_stream_slots(int rows, int stage_rows = kStageRows) {
  return std::max(stage_rows == kStageRows ? 64 : 32, (rows + stage_rows - 1) / stage_rows);
}

// Rows per stage of the streamed residual pass over `rows` items: 256 for
// bf16 rows of the Markov head (big) when there are more than 128, else 128.
static int residual_stage_rows(int rows, bool big) { return big && rows > kStageRows ? 2 * kStageRows : kStageRows; }

// Jobs (workgroup split x wave) of one stage in that grid, each writing one
// partial per item of the acceptance label: the kernel's own split arithmetic
// (stage_rows / 32 waves per workgroup).
static int label_jobs(int N, int stage_rows) {
  const int active = (N + stage_rows - 1) / stage_rows;
  return residual_stream_slots(N, stage_rows) / active * 8 * (stage_rows / 32);
}
// room for either stage size (the workspace query does not see the dtypes)
static int label_jobs_max(int N) {
  return std::max(label_jobs(N, kStageRows), label_jobs(N, residual_stage_rows(N, true)));
}

template <typename PT, typename DT, int KC, bool LABEL, bool ROWS = false>
static int launch_residual_stream(const VerifyArgs& a, hipStream_t stream) {
  const int rows = LABEL ? a.R * a.K : a.R;
  if constexpr (!ROWS && KC > 0 && std::is_same_v<PT, uint16_t> && std::is_same_v<DT, uint16_t>) {
    if (residual_stage_rows(rows, true) != kStageRows) {  // more items than one 128-row stage
      constexpr int G = 2 * kGroupsPerWG;
      return launch_kernel(LABEL ? "label_residual" : "verify_residual",
                           verify_residual_stream_kernel<PT, DT, KC, LABEL, false, G>,
                           dim3(8 * residual_stream_slots(rows, 16 * G)), dim3(32 * G), stream, a);
    }
  }
  const int slots = residual_stream_slots(rows);
  return launch_kernel(LABEL ? "label_residual" : "verify_residual",
                       verify_residual_stream_kernel<PT, DT, KC, LABEL, ROWS>, dim3(8 * slots), dim3(256), stream, a);
}

template <typename PT, typename DT, bool LABEL = false>
static int dispatch_residual_stream(const VerifyArgs& a, hipStream_t stream) {
  if (a.O) return launch_residual_stream<PT, DT, 8, LABEL, true>(a, stream);
  switch ((a.r + 31) / 32) {
    case 0: return launch_residual_stream<PT, DT, 0, LABEL>(a, stream);
    case 1: return launch_residual_stream<PT, DT, 1, LABEL>(a, stream);
    case 2: return launch_residual_stream<PT, DT, 2, LABEL>(a, stream);
    case 3: return launch_residual_stream<PT, DT, 3, LABEL>(a, stream);
    case 4: return launch_residual_stream<PT, DT, 4, LABEL>(a, stream);
    case 5: return launch_residual_stream<PT, DT, 5, LABEL>(a, stream);
    case 6: return launch_residual_stream<PT, DT, 6, LABEL>(a, stream);
    case 7: return launch_residual_stream<PT, DT, 7, LABEL>(a, stream);
    case 8: return launch_residual_stream<PT, DT, 8, LABEL>(a, stream);
    default: return -1;
  }
}

int run_markov_lse(int R, int K, int V, int r, float temperature, const void* D, bool d_bf16, const void* W1,
                   const void* W2, const void* W2s, const int32_t* x0, const int32_t* x, float* lse_out,
                   void* part, hipStream_t stream);

template <typename PT, typename DT>
static int run_verify_typed(VerifyArgs& a, bool greedy, bool vec_p, bool vec_d, hipStream_t stream) {
  int rc;
  const dim3 b256(256);
  const dim3 stream_grid(std::min(a.N * a.nchunks, kRowstatsWGs));
  if (greedy) {
    rc = vec_p ? launch_kernel("verify_rowstats", verify_rowstats_stream_kernel<PT, true>, stream_grid, b256,
                               stream, a)
               : launch_kernel("verify_rowstats", verify_rowstats_kernel<PT, false, true>,
                               dim3(a.N * a.nchunks), b256, stream, a);
    if (rc) return rc;
    rc = launch_kernel("verify_accept", verify_accept_kernel<PT, DT, true>, dim3((a.N + 3) / 4), b256, stream, a);
    if (rc) return rc;
    return launch_kernel("verify_decide", verify_decide_kernel<true>, dim3((a.R + 255) / 256), b256, stream, a);
  }
  rc = vec_p ? launch_kernel("verify_rowstats", verify_rowstats_stream_kernel<PT, false>, stream_grid, b256,
                             stream, a)
             : launch_kernel("verify_rowstats", verify_rowstats_kernel<PT, false, false>,
                             dim3(a.N * a.nchunks), b256, stream, a);
  if (rc) return rc;
  rc = launch_kernel("verify_accept", verify_accept_kernel<PT, DT, false>, dim3((a.N + 3) / 4), b256, stream, a);
  if (rc) return rc;
  rc = launch_kernel("verify_decide", verify_decide_kernel<false>, dim3((a.R + 255) / 256), b256, stream, a);
  if (rc) return rc;
  if (vec_p && vec_d) rc = dispatch_residual_stream<PT, DT>(a, stream);
  else if (vec_p) rc = dispatch_residual<PT, DT, true, false>(a, stream);
  else if (vec_d) rc = dispatch_residual<PT, DT, false, true>(a, stream);
  else rc = dispatch_residual<PT, DT, false, false>(a, stream);
  if (rc) return rc;
  return launch_kernel("verify_sample", verify_sample_kernel<PT, DT>, dim3((a.R + 3) / 4), b256, stream, a);
}

// The draft rows' log-normalisers when the caller has none (T > 0), into
// lse [R * K]: r == 0 (no bias) one rowstats pass over the judged draft rows
// and a merge; with a Markov head the draft's fused bias pass per position.
template <typename DT>
static int run_draft_row_lse(const VerifyArgs& a, bool d_bf16, bool vec_d, float temperature, float* lse,
                             void* dpart, hipStream_t stream) {
  if (a.r > 0)
    return run_markov_lse(a.R, a.K, a.V, a.r, temperature, a.D, d_bf16, a.W1, a.W2t, a.W2s, a.x0, a.x, lse, dpart,
                          stream);
  VerifyArgs d = a;
  d.P = a.D;
  d.N = a.R * a.K;
  d.ppart = reinterpret_cast<float2*>(dpart);
  d.ppart2 = nullptr;
  d.row_cu = a.cu;
  d.row_K = a.K;
  int rc = vec_d ? launch_kernel("verify_rowstats", verify_rowstats_stream_kernel<DT, false>,
                                 dim3(std::min(d.N * d.nchunks, kRowstatsWGs)), dim3(256), stream, d)
                 : launch_kernel("verify_rowstats", verify_rowstats_kernel<DT, false, false>,
                                 dim3(d.N * d.nchunks), dim3(256), stream, d);
  if (rc) return rc;
  return launch_kernel("verify_row_lse", row_lse_kernel, dim3((d.N + 3) / 4), dim3(256), stream,
                       reinterpret_cast<const float2*>(dpart), d.N, d.nsP, lse);
}

int run_verify(int R, int K, int V, float temperature, const void* P, bool p_bf16, int N,
               const int32_t* cu, const void* D, bool d_bf16, const void* W1, const void* W2, const void* W2f,
               int r, const int32_t* x0, const int32_t* x, const float* q_tok, const float* lse_d,
               uint64_t seed, uint64_t step, int32_t* n_acc_out, int32_t* tok_out, float* min_margin_out,
               void* workspace, const float* O, const uint16_t* W2h, hipStream_t stream) {
  const bool greedy = temperature == 0.f;
  const bool lse_pass = !greedy && !lse_d;
  const bool margins = min_margin_out != nullptr;
  const VerifyLayout l = verify_layout(R, K, V, N, r, lse_pass, !W2f, margins);
  char* ws = reinterpret_cast<char*>(workspace);
  VerifyArgs a{};
  a.R = R;
  a.K = K;
  a.V = V;
  a.N = N;
  a.r = r;
  a.c2 = greedy ? 1.f : kLog2e / temperature;
  a.P = P;
  a.cu = cu;
  a.D = D;
  a.W1 = reinterpret_cast<const uint16_t*>(W1);
  a.W2t = reinterpret_cast<const uint16_t*>(W2);
  a.W2s = (!O && r > 0) ? reinterpret_cast<const uint16_t*>(W2f) : nullptr;
  a.x0 = x0;
  a.x = x;
  a.q_tok = q_tok;
  a.lse_d = lse_d;
  a.O = O;
  a.W2h = W2h;
  a.seed = seed;
  a.step = step;
  a.n_acc_out = n_acc_out;
  a.tok_out = tok_out;
  a.ppart = reinterpret_cast<float2*>(ws + l.ppart);
  a.rowms = reinterpret_cast<float2*>(ws + l.rowms);
  a.flag = reinterpret_cast<int32_t*>(ws + l.flag);
  a.info = reinterpret_cast<int4*>(ws + l.info);
  a.rpart = reinterpret_cast<float*>(ws + l.rpart);
  a.rej_count = reinterpret_cast<int32_t*>(ws + l.rej);
  a.rej_list = a.rej_count + 1;
  if (margins) {
    a.margin = reinterpret_cast<float*>(ws + l.margin);
    a.rmin = reinterpret_cast<float*>(ws + l.rmin);
    a.ppart2 = greedy ? reinterpret_cast<float*>(ws + l.ppart2) : nullptr;
    a.min_margin_out = min_margin_out;
  }
  a.nsP = (V + kRowSlice - 1) / kRowSlice;
  a.ns64 = (V + kWaveCols - 1) / kWaveCols;
  a.nchunks = (V + kRowChunk - 1) / kRowChunk;
  a.ncol_tiles = (V + kTileCols - 1) / kTileCols;
  a.nstages = (R + kStageRows - 1) / kStageRows;
  const uintptr_t pb = reinterpret_cast<uintptr_t>(P), db = reinterpret_cast<uintptr_t>(D);
  const bool vec_p = (pb % 16 == 0) && (V % (p_bf16 ? 8 : 4) == 0);
  const bool vec_d = (db % 16 == 0) && (V % (d_bf16 ? 8 : 4) == 0);
  if (lse_pass) {
    float* lse = reinterpret_cast<float*>(ws + l.lse);
    if (r > 0 && !W2f) {  // the fused bias pass reads the fragment-ordered W2
      const int rc = run_w2_swizzle(a.W2t, ws + l.w2s, V, r, (r + 31) / 32, false, stream);
      if (rc) return rc;
      a.W2s = reinterpret_cast<const uint16_t*>(ws + l.w2s);
    }
    const int rc = d_bf16 ? run_draft_row_lse<uint16_t>(a, true, vec_d, temperature, lse, ws + l.dpart, stream)
                          : run_draft_row_lse<float>(a, false, vec_d, temperature, lse, ws + l.dpart, stream);
    if (rc) return rc;
    a.lse_d = lse;
  }
  if (p_bf16 && d_bf16) return run_verify_typed<uint16_t, uint16_t>(a, greedy, vec_p, vec_d, stream);
  if (p_bf16) return run_verify_typed<uint16_t, float>(a, greedy, vec_p, vec_d, stream);
  if (d_bf16) return run_verify_typed<float, uint16_t>(a, greedy, vec_p, vec_d, stream);
  return run_verify_typed<float, float>(a, greedy, vec_p, vec_d, stream);
}

// r > 0 (Markov head): plus W2 in fragment order for the residual pass
size_t label_workspace_bytes(int B, int K, int V, int r) {
  const size_t N = (size_t)B * K;
  const size_t nsP = (size_t)(((int64_t)V + kRowSlice - 1) / kRowSlice), ns64 = (size_t)(((int64_t)V + kWaveCols - 1) / kWaveCols);
  // the residual region holds per-slice masses (unaligned rows) or the
  // streamed pass's per-(job, item) sums
  const size_t resid = std::max(N * ns64 * sizeof(float), (size_t)label_jobs_max((int)N) * N * sizeof(double));
  return align256(N * nsP * sizeof(float2)) + align256(N * sizeof(float2)) + align256(resid) + w2_swizzle_bytes(V, r);
}

template <typename PT, typename DT>
static int run_label_typed(VerifyArgs& a, float* c_out, bool greedy, bool vec_p, bool vec_d, hipStream_t stream) {
  int rc;
  const dim3 b256(256);
  const dim3 stream_grid(std::min(a.N * a.nchunks, kRowstatsWGs));
  const dim3 per_row((a.N + 3) / 4);
  if (greedy) {
    rc = vec_p ? launch_kernel("label_rowstats", verify_rowstats_stream_kernel<PT, true>, stream_grid, b256, stream, a)
               : launch_kernel("label_rowstats", verify_rowstats_kernel<PT, false, true>, dim3(a.N * a.nchunks), b256,
                               stream, a);
    if (rc) return rc;
    rc = launch_kernel("label_merge", label_merge_kernel<true>, per_row, b256, stream, a);
    if (rc) return rc;
    return launch_kernel("label_reduce", label_reduce_kernel<true>, per_row, b256, stream, a, c_out);
  }
  rc = vec_p ? launch_kernel("label_rowstats", verify_rowstats_stream_kernel<PT, false>, stream_grid, b256, stream, a)
             : launch_kernel("label_rowstats", verify_rowstats_kernel<PT, false, false>, dim3(a.N * a.nchunks), b256,
                             stream, a);
  if (rc) return rc;
  rc = launch_kernel("label_merge", label_merge_kernel<false>, per_row, b256, stream, a);
  if (rc) return rc;
  if (vec_p && vec_d) {
    // per-(job, item) sums instead of per-slice masses, in the same region
    a.lpart = reinterpret_cast<double*>(a.rpart);
    constexpr bool big = std::is_same_v<PT, uint16_t> && std::is_same_v<DT, uint16_t>;
    a.njobs = label_jobs(a.N, residual_stage_rows(a.N, big && a.r > 0 && !a.O));
    rc = dispatch_residual_stream<PT, DT, true>(a, stream);
    if (rc) return rc;
    return launch_kernel("label_reduce", label_reduce_jobs_kernel, dim3((a.N + 255) / 256), b256, stream, a, c_out);
  }
  if (vec_p) rc = dispatch_residual<PT, DT, true, false, true>(a, stream);
  else if (vec_d) rc = dispatch_residual<PT, DT, false, true, true>(a, stream);
  else rc = dispatch_residual<PT, DT, false, false, true>(a, stream);
  if (rc) return rc;
  return launch_kernel("label_reduce", label_reduce_kernel<false>, per_row, b256, stream, a, c_out);
}

int run_label(int B, int K, int V, float temperature, const void* P, bool p_bf16, const void* D, bool d_bf16,
              const void* W1, const void* W2, const void* W2f, int r, const int32_t* x0, const int32_t* x,
              const float* lse_d, float* c_out, void* workspace, const float* O, const uint16_t* W2h,
              hipStream_t stream) {
  const int N = B * K;
  char* ws = reinterpret_cast<char*>(workspace);
  VerifyArgs a{};
  a.R = B;
  a.K = K;
  a.V = V;
  a.N = N;
  a.r = r;
  const bool greedy = temperature == 0.f;
  a.c2 = greedy ? 1.f : kLog2e / temperature;
  a.P = P;
  a.D = D;
  a.W1 = reinterpret_cast<const uint16_t*>(W1);
  a.W2t = reinterpret_cast<const uint16_t*>(W2);
  a.x0 = x0;
  a.x = x;
  a.lse_d = lse_d;
  a.O = O;
  a.W2h = W2h;
  a.nsP = (V + kRowSlice - 1) / kRowSlice;
  a.ns64 = (V + kWaveCols - 1) / kWaveCols;
  a.nchunks = (V + kRowChunk - 1) / kRowChunk;
  a.ncol_tiles = (V + kTileCols - 1) / kTileCols;
  a.nstages = (N + kStageRows - 1) / kStageRows;
  size_t off = 0;
  a.ppart = reinterpret_cast<float2*>(ws + off);
  off += align256((size_t)N * a.nsP * sizeof(float2));
  a.rowms = reinterpret_cast<float2*>(ws + off);
  off += align256((size_t)N * sizeof(float2));
  a.rpart = reinterpret_cast<float*>(ws + off);
  off += align256(std::max((size_t)N * a.ns64 * sizeof(float), (size_t)label_jobs_max(N) * N * sizeof(double)));
  const uintptr_t pb = reinterpret_cast<uintptr_t>(P), db = reinterpret_cast<uintptr_t>(D);
  const bool vec_p = (pb % 16 == 0) && (V % (p_bf16 ? 8 : 4) == 0);
  const bool vec_d = (db % 16 == 0) && (V % (d_bf16 ? 8 : 4) == 0);
  if (!O && r > 0 && temperature != 0.f && vec_p && vec_d) {  // the streamed residual pass reads it
    if (W2f) {
      a.W2s = reinterpret_cast<const uint16_t*>(W2f);
    } else {
      a.W2s = reinterpret_cast<const uint16_t*>(ws + off);
      const int rc = run_w2_swizzle(a.W2t, ws + off, V, r, (r + 31) / 32, false, stream);
      if (rc) return rc;
    }
  }
  if (p_bf16 && d_bf16) return run_label_typed<uint16_t, uint16_t>(a, c_out, greedy, vec_p, vec_d, stream);
  if (p_bf16) return run_label_typed<uint16_t, float>(a, c_out, greedy, vec_p, vec_d, stream);
  if (d_bf16) return run_label_typed<float, uint16_t>(a, c_out, greedy, vec_p, vec_d, stream);
  return run_label_typed<float, float>(a, c_out, greedy, vec_p, vec_d, stream);
}

}  // namespace dspark
