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
#include "bias_tile.hpp"
#include "launch.hpp"

namespace dspark {

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
};

template <typename UT, bool VEC, int KC, bool GREEDY>
__global__ __launch_bounds__(256) void draft_partials_kernel(DraftArgs a) {
  int col_tile, stage;
  if (!xcd_tile(blockIdx.x, a.ncol_tiles, a.nstages, col_tile, stage)) return;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n0 = col_tile * kTileCols + wave * kWaveCols;
  const int row0 = stage * kStageRows;

  __shared__ EStage<(KC > 0 ? KC : 1)> st;
  bf16x8 w2[4][(KC > 0 ? KC : 1)];
  if constexpr (KC > 0) {
    const int32_t* prev = a.prev;
    const int stride = a.prev_stride;
    stage_e<KC>(st, a.W1, a.r, a.V, row0, a.B, [&](int g) { return prev[(size_t)g * stride]; });
    load_w2_frags<KC>(a.W2t, a.r, a.V, n0, lane, w2);
    __syncthreads();
  }
  if (n0 >= a.V) return;

  const UT* U = reinterpret_cast<const UT*>(a.U);
  const int cbase = n0 + 16 * (lane >> 4);
  const int slice = n0 / kWaveCols;
  for (int g = 0; g < kStageRows / 16; ++g) {
    const int row = row0 + 16 * g + (lane & 15);
    if (row0 + 16 * g >= a.B) break;
    float z[16];
    const bool live = row < a.B;
    if (live) {
      const UT* urow = U + ((size_t)row * a.K + (a.k - 1)) * a.V;
      Logits16<UT>::template load<VEC>(urow, cbase, a.V, z);
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) z[e] = -INFINITY;
    }
    if constexpr (KC > 0) {
      f32x4 acc[4];
      mfma_group<KC>(st, g, lane, w2, acc);
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) z[4 * b + i] += acc[b][i];
    }
    if constexpr (GREEDY) {
      float m = -INFINITY;
      int idx = -1;
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (cbase + e < a.V && (z[e] > m || idx < 0)) {
          m = z[e];
          idx = cbase + e;
        }
#pragma unroll
      for (int off = 16; off <= 32; off <<= 1) {
        const float m2 = __shfl_xor(m, off, 64);
        const int i2 = __shfl_xor(idx, off, 64);
        merge_argmax(m, idx, m2, i2);
      }
      if (live && lane < 16) a.part[(size_t)row * a.nslices + slice] = make_float2(m, __int_as_float(idx));
    } else {
      float m = -INFINITY;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        z[e] *= a.c2;
        m = fmaxf(m, z[e]);
      }
      float s = 0.f;
      if (m != -INFINITY) {
#pragma unroll
        for (int e = 0; e < 16; ++e) s += exp2f(z[e] - m);
      }
#pragma unroll
      for (int off = 16; off <= 32; off <<= 1) {
        const float m2 = __shfl_xor(m, off, 64);
        const float s2 = __shfl_xor(s, off, 64);
        merge_ms(m, s, m2, s2);
      }
      if (live && lane < 16) a.part[(size_t)row * a.nslices + slice] = make_float2(m, s);
    }
  }
}

// One wave per request.
template <typename UT, bool GREEDY>
__global__ __launch_bounds__(256) void draft_locate_kernel(DraftArgs a) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (b >= a.B) return;
  const size_t out = (size_t)b * a.K + (a.k - 1);
  const int prev = a.prev[(size_t)b * a.prev_stride];
  if (prev < 0 || prev >= a.V) {
    if (lane == 0) {
      a.x_out[out] = -1;
      a.q_out[out] = NAN;
      a.lse_out[out] = NAN;
    }
    return;
  }
  const float2* part = a.part + (size_t)b * a.nslices;
  const int ns = a.nslices;

  if constexpr (GREEDY) {
    float m = -INFINITY;
    int idx = -1;
    for (int s = lane; s < ns; s += 64) {
      const float2 p = part[s];
      merge_argmax(m, idx, p.x, __float_as_int(p.y));
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

  // global max and normaliser S = sum_s s_s * 2^(m_s - M)
  float M = -INFINITY;
  for (int s = lane; s < ns; s += 64) M = fmaxf(M, part[s].x);
  M = wave_max(M);
  const int per = (ns + 63) / 64;
  const int s_begin = min(ns, lane * per);
  const int s_end = min(ns, s_begin + per);
  float local = 0.f;
  for (int s = s_begin; s < s_end; ++s) {
    const float2 p = part[s];
    local += (p.x == -INFINITY) ? 0.f : p.y * exp2f(p.x - M);
  }
  const float incl = wave_inclusive_scan(local);
  const float S = __shfl(incl, 63, 64);
  const float u = decision_uniform(a.seed, a.step, (uint32_t)b, (uint32_t)a.k, kPurposeDraft);
  const float target = u * S;
  int owner = wave_first_lane(incl > target);
  if (owner < 0) {  // rounding put u*S at or past the total: last lane with mass
    const unsigned long long m = __ballot(local > 0.f);
    owner = m ? 63 - __clzll((long long)m) : 0;
  }
  // the owner walks its slices in order
  int s_star = -1;
  float before = 0.f;
  if (lane == owner) {
    float acc = incl - local;
    int last = -1;
    float last_before = acc;
    for (int s = s_begin; s < s_end; ++s) {
      const float2 p = part[s];
      const float w = (p.x == -INFINITY) ? 0.f : p.y * exp2f(p.x - M);
      if (w > 0.f) {
        last = s;
        last_before = acc;
      }
      if (acc + w > target && w > 0.f) {
        s_star = s;
        before = acc;
        break;
      }
      acc += w;
    }
    if (s_star < 0) {
      s_star = last;
      before = last_before;
    }
  }
  s_star = __shfl(s_star, owner, 64);
  before = __shfl(before, owner, 64);
  if (s_star < 0) s_star = 0;  // no mass at all (non-finite logits): keep indices in range
  const float m_s = part[s_star].x;
  const float f_s = exp2f(m_s - M);
  const float t_in = (target - before) / f_s;

  // re-evaluate the 64 logits of slice s_star, one column per lane
  const int col = s_star * kWaveCols + lane;
  float z2 = -INFINITY;
  if (col < a.V) {
    const UT* urow = reinterpret_cast<const UT*>(a.U) + ((size_t)b * a.K + (a.k - 1)) * a.V;
    float z = load_logit(urow, col);
    if (a.r > 0) z += valu_bias(a.W1 + (size_t)prev * a.r, a.W2t + (size_t)col * a.r, a.r);
    z2 = z * a.c2;
  }
  const float e = (col < a.V) ? exp2f(z2 - m_s) : 0.f;
  const float cum = wave_inclusive_scan(e);
  int pick = wave_first_lane(cum > t_in && e > 0.f);
  if (pick < 0) {
    const unsigned long long m = __ballot(e > 0.f);
    pick = m ? 63 - __clzll((long long)m) : 0;
  }
  const float z2x = __shfl(z2, pick, 64);
  if (lane == 0) {
    a.x_out[out] = s_star * kWaveCols + pick;
    a.q_out[out] = exp2f(z2x - M) / S;
    a.lse_out[out] = (M + log2f(S)) * kLn2;
  }
}

template <typename UT, bool VEC, int KC, bool GREEDY>
static int launch_partials(const DraftArgs& a, hipStream_t stream) {
  const int grid = xcd_grid(a.ncol_tiles, a.nstages);
  return launch_kernel("draft_partials", draft_partials_kernel<UT, VEC, KC, GREEDY>, dim3(grid),
                       dim3(256), stream, a);
}

template <typename UT, bool VEC, bool GREEDY>
static int dispatch_kc(const DraftArgs& a, hipStream_t stream) {
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

template <typename UT, bool GREEDY>
static int run_draft_typed(DraftArgs a, bool vec, hipStream_t stream) {
  for (int k = 1; k <= a.K; ++k) {
    a.k = k;
    if (k == 1) {
      // prev set by the caller to the anchors
    } else {
      a.prev = a.x_out + (k - 2);
      a.prev_stride = a.K;
    }
    int rc = vec ? dispatch_kc<UT, true, GREEDY>(a, stream) : dispatch_kc<UT, false, GREEDY>(a, stream);
    if (rc) return rc;
    rc = launch_kernel("draft_locate", draft_locate_kernel<UT, GREEDY>, dim3((a.B + 3) / 4), dim3(256),
                       stream, a);
    if (rc) return rc;
  }
  return 0;
}

size_t draft_workspace_bytes(int B, int V) {
  const size_t ns = (size_t)(V + kWaveCols - 1) / kWaveCols;
  return ((size_t)B * ns * sizeof(float2) + 255) / 256 * 256;
}

int run_draft(int B, int K, int V, int r, float temperature, const void* U, bool u_bf16,
              const void* W1, const void* W2, const int32_t* x0, uint64_t seed, uint64_t step,
              int32_t* x_out, float* q_out, float* lse_out, void* workspace, hipStream_t stream) {
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
  a.ncol_tiles = (V + kTileCols - 1) / kTileCols;
  a.nstages = (B + kStageRows - 1) / kStageRows;
  a.part = reinterpret_cast<float2*>(workspace);
  a.seed = seed;
  a.step = step;
  a.x_out = x_out;
  a.q_out = q_out;
  a.lse_out = lse_out;
  const bool greedy = temperature == 0.f;
  a.c2 = greedy ? 1.f : kLog2e / temperature;
  const uintptr_t base = reinterpret_cast<uintptr_t>(U);
  if (u_bf16) {
    const bool vec = (V % 8 == 0) && (base % 16 == 0);
    return greedy ? run_draft_typed<uint16_t, true>(a, vec, stream)
                  : run_draft_typed<uint16_t, false>(a, vec, stream);
  }
  const bool vec = (V % 4 == 0) && (base % 16 == 0);
  return greedy ? run_draft_typed<float, true>(a, vec, stream) : run_draft_typed<float, false>(a, vec, stream);
}

}  // namespace dspark
