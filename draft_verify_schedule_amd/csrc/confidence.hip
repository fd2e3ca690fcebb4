// Confidence head and Sequential Temperature Scaling (DSpark paper, section
// 3.2.1: Confidence Head and Post-hoc Calibration; "Speculative decoding,
// from zero to DSpark", section 8, The confidence head, and Appendix A5).
//
// confidence_head: one wave per (request, position) item i = r * K + k:
//   z_i = w_h . h_i + w_e . W1[x_{r,k-1}] + b   (x_{r,0} = anchor)
//   c_i = sigmoid(z_i / T_k)
// lanes take strided elements of both dot products (fp32), the wave sum is a
// fixed xor tree.
//
// sts_advance / sts_ece / sts_pick, for each position k in order (the
// temperatures of positions < k already fixed in T_out): sts_advance writes
// one 16-byte record per held-out sample (prefix = prod_{i<k} sigmoid(l_{n,i}
// / T_i) in fp64, left to right, advanced by one factor per position; this
// position's logit and label); sts_ece, one workgroup per (chunk of samples,
// 4 grid temperatures): pred = prefix * sigmoid(l_{n,k} / T_g), bin =
// floor(pred * n_bins) (last bin closed), per-thread bin slots in LDS (no
// atomics) added by a fixed pairwise tree into one partial per (T_g, chunk,
// bin); sts_pick merges the partials in chunk order, ECE_g = sum_b |labels_b
// - sum pred_b| / N, and the first grid value with the smallest ECE becomes
// T_k.  Every sum runs in a fixed order, so the result is deterministic.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace dspark {

struct HeadArgs {
  int B, K, d, r, V;
  const void* H;  // [B, K, d]
  const float* w_h;
  const float* w_e;
  float bias;
  const uint16_t* W1;  // [V, r] bf16
  const int32_t* x0;
  const int32_t* x;
  const float* T;  // [K] or null
  float* c_out;
  float* logit_out;  // or null
};

template <typename HT, bool VEC>
__global__ __launch_bounds__(256) void confidence_head_kernel(HeadArgs a) {
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + wave_index();
  if (i >= a.B * a.K) return;
  const int r = i / a.K, k = i - r * a.K;
  const int prev = k == 0 ? a.x0[r] : a.x[i - 1];
  const HT* h = reinterpret_cast<const HT*>(a.H) + (size_t)i * a.d;
  const bool ok = prev >= 0 && prev < a.V;
  float s = 0.f;
  if constexpr (VEC) {
    // 16-byte loads: lane takes 4 (f32) or 8 (bf16) consecutive elements per
    // step.  The first kPre steps, and the Markov part's elements (r <= 256:
    // at most 4 per lane), are all requested before the first product (one
    // memory round trip for rows up to 64 * kPre * E wide); wider rows loop
    // over the rest.  The products are taken in the same order either way.
    constexpr int E = 16 / sizeof(HT);
    constexpr int NW = sizeof(HT) == 2 ? 2 : 1;  // f32x4 of w_h per step
    constexpr int kPre = 8;
    u32x4 hv[kPre];
    f32x4 hw[kPre][NW];
#pragma unroll
    for (int t = 0; t < kPre; ++t) {
      const int j = lane * E + 64 * E * t;
      if (j < a.d) {
        hv[t] = *reinterpret_cast<const u32x4*>(h + j);
#pragma unroll
        for (int q = 0; q < NW; ++q) hw[t][q] = *reinterpret_cast<const f32x4*>(a.w_h + j + 4 * q);
      }
    }
    float we[4];
    uint32_t ev[4];
    const bool markov = a.r > 0 && ok;
    if (markov) {
      const uint16_t* e = a.W1 + (size_t)prev * a.r;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int j = lane + 64 * t;
        if (j < a.r) {
          we[t] = a.w_e[j];
          ev[t] = e[j];
        }
      }
    }
    auto step = [&](u32x4 v, const f32x4 (&w)[NW]) {
      if constexpr (sizeof(HT) == 2) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          s = fmaf(w[0][2 * e], __uint_as_float(v[e] << 16), s);
          s = fmaf(w[0][2 * e + 1], __uint_as_float(v[e] & 0xFFFF0000u), s);
          s = fmaf(w[NW - 1][2 * e], __uint_as_float(v[e + 2] << 16), s);
          s = fmaf(w[NW - 1][2 * e + 1], __uint_as_float(v[e + 2] & 0xFFFF0000u), s);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) s = fmaf(w[0][e], __uint_as_float(v[e]), s);
      }
    };
#pragma unroll
    for (int t = 0; t < kPre; ++t)
      if (lane * E + 64 * E * t < a.d) step(hv[t], hw[t]);
    for (int j = lane * E + 64 * E * kPre; j < a.d; j += 64 * E) {
      f32x4 w[NW];
#pragma unroll
      for (int q = 0; q < NW; ++q) w[q] = *reinterpret_cast<const f32x4*>(a.w_h + j + 4 * q);
      step(*reinterpret_cast<const u32x4*>(h + j), w);
    }
    if (markov) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (lane + 64 * t < a.r) s = fmaf(we[t], bf16_bits_to_f32(ev[t]), s);
    }
  } else {
    for (int j = lane; j < a.d; j += 64) {
      float hv;
      if constexpr (sizeof(HT) == 2) hv = bf16_bits_to_f32(h[j]);
      else hv = h[j];
      s = fmaf(a.w_h[j], hv, s);
    }
    if (a.r > 0 && ok) {
      const uint16_t* e = a.W1 + (size_t)prev * a.r;
      for (int j = lane; j < a.r; j += 64) s = fmaf(a.w_e[j], bf16_bits_to_f32(e[j]), s);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
  if (lane == 0) {
    const float z = s + a.bias;
    const float t = a.T ? a.T[k] : 1.f;
    a.c_out[i] = ok ? 1.f / (1.f + expf(-z / t)) : NAN;
    if (a.logit_out) a.logit_out[i] = ok ? z : NAN;
  }
}

int run_confidence_head(int B, int K, int d, int r, int V, const void* H, bool h_bf16, const float* w_h,
                        const float* w_e, float bias, const void* W1, const int32_t* x0, const int32_t* x,
                        const float* T, float* c_out, float* logit_out, hipStream_t stream) {
  HeadArgs a{B, K, d, r, V, H, w_h, w_e, bias, reinterpret_cast<const uint16_t*>(W1), x0, x, T, c_out, logit_out};
  const dim3 grid((B * K + 3) / 4);
  // vector path: rows and w_h 16-byte aligned
  const bool vec = d % (h_bf16 ? 8 : 4) == 0 && reinterpret_cast<uintptr_t>(H) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(w_h) % 16 == 0;
  if (h_bf16)
    return vec ? launch_kernel("confidence_head", confidence_head_kernel<uint16_t, true>, grid, dim3(256), stream, a)
               : launch_kernel("confidence_head", confidence_head_kernel<uint16_t, false>, grid, dim3(256), stream, a);
  return vec ? launch_kernel("confidence_head", confidence_head_kernel<float, true>, grid, dim3(256), stream, a)
             : launch_kernel("confidence_head", confidence_head_kernel<float, false>, grid, dim3(256), stream, a);
}

// ------------------------------------------------------------------- STS --
constexpr int kStsThreads = 256;
constexpr int kStsMaxBins = 32;
constexpr int kStsPerThread = 16;                          // samples per thread of an ECE workgroup
constexpr int kStsChunk = kStsPerThread * kStsThreads;     // samples per ECE workgroup
constexpr int kStsTemps = 4;                               // grid temperatures per ECE workgroup

// One held-out sample at the current position: the cumulative product of
// the earlier positions' calibrated sigmoids, this position's logit and label.
struct alignas(16) StsRec {
  double prefix;
  float logit;
  int32_t label;
};

struct StsArgs {
  int N, K, G, nbins, k, nchunks;
  const float* logits;     // [N, K]
  const uint8_t* survived; // [N, K]
  const float* grid;       // [G]
  float* T_out;            // [K]
  float* ece_out;          // [K] or null
  StsRec* rec;             // [N]
  double* psum;            // [G, nchunks, kStsMaxBins]: prediction sums per chunk and bin
  int32_t* pcnt;           // [G, nchunks, kStsMaxBins]: samples | labels << 16 per chunk and bin
};

// sigmoid in fp64 without forming exp of a large positive argument:
// e = exp(-|z|); 1 / (1 + e) for z >= 0, e / (1 + e) below (branch-free, so
// a wave with logits of both signs evaluates one exp and one division)
__device__ __forceinline__ double sigmoid_d(double z) {
  const double e = exp(-fabs(z));
  return (z >= 0.0 ? 1.0 : e) / (1.0 + e);
}

// The records of position k: at k = 0 the product is 1; after T_{k-1} is
// fixed, prefix <- prefix * sigmoid(l_{n,k-1} / T_{k-1}) (left to right, as
// the cumulative product is defined), then this position's logit and label.
__global__ __launch_bounds__(kStsThreads) void sts_advance_kernel(StsArgs a) {
  const int n = blockIdx.x * kStsThreads + threadIdx.x;
  if (n >= a.N) return;
  double pre = 1.0;
  if (a.k > 0) {
    const StsRec r = a.rec[n];
    pre = r.prefix * sigmoid_d((double)r.logit / (double)a.T_out[a.k - 1]);
  }
  StsRec out;
  out.prefix = pre;
  out.logit = a.logits[(size_t)n * a.K + a.k];
  out.label = a.survived[(size_t)n * a.K + a.k] ? 1 : 0;
  a.rec[n] = out;
}

// One workgroup per (chunk of kStsChunk samples, kStsTemps grid temperatures)
// at position k.  Each thread loads its kStsPerThread records once; for each
// temperature T_g: pred = prefix * sigmoid(l / T_g), bin = floor(pred *
// n_bins) clamped to the last bin, accumulated in the thread's own LDS slots
// (prediction sums in fp64, sample and label counts packed in one int: at
// most 16 samples per thread), so no atomics; a fixed pairwise tree over the
// threads then gives the chunk's partial per bin.  A sample with no
// prediction (NaN) is in no bin.
template <int NB>
__global__ __launch_bounds__(kStsThreads) void sts_ece_kernel(StsArgs a) {
  __shared__ double sp[NB * kStsThreads];
  __shared__ int32_t sc[NB * kStsThreads];
  const int t = threadIdx.x;
  const int c = blockIdx.x;
  const int n0 = c * kStsChunk + t;
  StsRec r[kStsPerThread];
#pragma unroll
  for (int i = 0; i < kStsPerThread; ++i) {
    const int n = n0 + i * kStsThreads;
    if (n < a.N) {
      r[i] = a.rec[n];
    } else {
      r[i].prefix = NAN;  // past the end: no prediction
      r[i].logit = 0.f;
      r[i].label = 0;
    }
  }
  for (int tg = 0; tg < kStsTemps; ++tg) {
    const int g = blockIdx.y * kStsTemps + tg;
    if (g >= a.G) break;  // uniform over the workgroup
    if (tg > 0) __syncthreads();  // the previous temperature's partials are read
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      sp[b * kStsThreads + t] = 0.0;
      sc[b * kStsThreads + t] = 0;
    }
    const double T = (double)a.grid[g];
#pragma unroll
    for (int i = 0; i < kStsPerThread; ++i) {
      const double pred = r[i].prefix * sigmoid_d((double)r[i].logit / T);
      const bool has = !isnan(pred);  // branch-free: a NaN adds zero to bin 0
      int b = has ? (int)(pred * a.nbins) : 0;
      b = b < 0 ? 0 : (b >= a.nbins ? a.nbins - 1 : b);
      sp[b * kStsThreads + t] += has ? pred : 0.0;
      sc[b * kStsThreads + t] += has ? 1 + (r[i].label << 16) : 0;
    }
    // at most kStsChunk samples per chunk: the packed halves never carry
    for (int h = kStsThreads / 2; h > 0; h >>= 1) {
      __syncthreads();
      if (t < h) {
        for (int b = 0; b < a.nbins; ++b) {
          sp[b * kStsThreads + t] += sp[b * kStsThreads + t + h];
          sc[b * kStsThreads + t] += sc[b * kStsThreads + t + h];
        }
      }
    }
    __syncthreads();
    if (t < a.nbins) {
      const size_t o = ((size_t)g * a.nchunks + c) * kStsMaxBins + t;
      a.psum[o] = sp[t * kStsThreads];
      a.pcnt[o] = sc[t * kStsThreads];
    }
  }
}

// One workgroup, in blocks of grid values: thread p of a block merges pair
// (T_g, bin b)'s chunk partials in chunk order into |labels - sum pred| (0 for
// an empty bin), then thread g adds its bins in order: ECE_g = sum / N.  The
// first grid value with the smallest ECE becomes T_k.
constexpr int kStsPickThreads = 1024;
constexpr int kStsPickTerms = 4096;

// (e2, i2) before (e1, i1) in the argmin order: a missing entry (index < 0)
// never wins, NaN comes first (as an argmin over values with NaN returns the
// first NaN), then the smaller value, then the lower index
__device__ __forceinline__ bool sts_before(double e2, int i2, double e1, int i1) {
  if (i2 < 0) return false;
  if (i1 < 0) return true;
  const bool n1 = isnan(e1), n2 = isnan(e2);
  if (n1 || n2) return n2 && (!n1 || i2 < i1);
  return e2 < e1 || (e2 == e1 && i2 < i1);
}

__global__ __launch_bounds__(kStsPickThreads) void sts_pick_kernel(StsArgs a) {
  __shared__ double term[kStsPickTerms];
  __shared__ double se[kStsPickThreads];
  __shared__ int si[kStsPickThreads];
  const int t = threadIdx.x;
  const int nb = a.nbins;
  const int per_block = kStsPickTerms / nb;  // grid values per block
  double best = INFINITY;
  int bi = -1;
  for (int g0 = 0; g0 < a.G; g0 += per_block) {
    const int ng = min(per_block, a.G - g0);
    for (int p = t; p < ng * nb; p += kStsPickThreads) {
      const int g = g0 + p / nb, b = p - (p / nb) * nb;
      const size_t o = (size_t)g * a.nchunks * kStsMaxBins + b;
      double s = 0.0;
      int64_t cnt = 0, lab = 0;
#pragma unroll 8
      for (int c = 0; c < a.nchunks; ++c) {
        s += a.psum[o + (size_t)c * kStsMaxBins];
        const int32_t cl = a.pcnt[o + (size_t)c * kStsMaxBins];
        cnt += cl & 0xFFFF;
        lab += (uint32_t)cl >> 16;
      }
      term[p] = cnt ? fabs((double)lab - s) : 0.0;
    }
    __syncthreads();
    if (t < ng) {
      double e = 0.0;
      for (int b = 0; b < nb; ++b) e += term[t * nb + b];
      e /= (double)a.N;
      if (sts_before(e, g0 + t, best, bi)) {
        best = e;
        bi = g0 + t;
      }
    }
    __syncthreads();
  }
  // argmin by a pairwise tree: the smaller ECE, the lower grid index on ties
  se[t] = best;
  si[t] = bi;
  for (int h = kStsPickThreads / 2; h > 0; h >>= 1) {
    __syncthreads();
    if (t < h) {
      const double e2 = se[t + h];
      const int i2 = si[t + h];
      if (sts_before(e2, i2, se[t], si[t])) {
        se[t] = e2;
        si[t] = i2;
      }
    }
  }
  __syncthreads();
  if (t == 0) {
    a.T_out[a.k] = a.grid[si[0]];
    if (a.ece_out) a.ece_out[a.k] = (float)se[0];
  }
}

static size_t align256(size_t b) { return (b + 255) / 256 * 256; }
static int sts_chunks(int N) { return (N + kStsChunk - 1) / kStsChunk; }

size_t sts_workspace_bytes(int N, int G) {
  const size_t parts = (size_t)G * sts_chunks(N) * kStsMaxBins;
  return align256((size_t)N * sizeof(StsRec)) + align256(parts * sizeof(double)) +
         align256(parts * sizeof(int32_t));
}

int run_sts_fit(int N, int K, const float* logits, const uint8_t* survived, int G, const float* grid, int nbins,
                float* T_out, float* ece_out, void* workspace, hipStream_t stream) {
  char* ws = reinterpret_cast<char*>(workspace);
  const int nchunks = sts_chunks(N);
  const size_t parts = (size_t)G * nchunks * kStsMaxBins;
  const size_t rec_bytes = align256((size_t)N * sizeof(StsRec));
  StsRec* rec = reinterpret_cast<StsRec*>(ws);
  double* psum = reinterpret_cast<double*>(ws + rec_bytes);
  int32_t* pcnt = reinterpret_cast<int32_t*>(ws + rec_bytes + align256(parts * sizeof(double)));
  StsArgs a{N, K, G, nbins, 0, nchunks, logits, survived, grid, T_out, ece_out, rec, psum, pcnt};
  const dim3 egrid(nchunks, (G + kStsTemps - 1) / kStsTemps);
  for (int k = 0; k < K; ++k) {
    a.k = k;
    int rc = launch_kernel("sts_advance", sts_advance_kernel, dim3((N + kStsThreads - 1) / kStsThreads),
                           dim3(kStsThreads), stream, a);
    if (rc) return rc;
    rc = nbins <= 16 ? launch_kernel("sts_ece", sts_ece_kernel<16>, egrid, dim3(kStsThreads), stream, a)
                     : launch_kernel("sts_ece", sts_ece_kernel<kStsMaxBins>, egrid, dim3(kStsThreads), stream, a);
    if (rc) return rc;
    rc = launch_kernel("sts_pick", sts_pick_kernel, dim3(1), dim3(kStsPickThreads), stream, a);
    if (rc) return rc;
  }
  return 0;
}

}  // namespace dspark
