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
// sts_ece: one workgroup per grid temperature T_g, at position k (the
// temperatures of positions < k already fixed in T_out): for every held-out
// sample n, pred = prod_{i<k} sigmoid(l_{n,i} / T_i) * sigmoid(l_{n,k} / T_g)
// (fp64, left to right), bin = floor(pred * n_bins) (last bin closed); each
// thread keeps its own bin counts, label counts and prediction sums in LDS
// (bin-major, no atomics), reduced in thread order, so the ECE
// sum_b |labels_b - sum pred_b| / N is deterministic.
// sts_pick: the first grid value with the smallest ECE becomes T_k.
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
  float s = 0.f;
  if constexpr (VEC) {
    // 16-byte loads: lane takes 4 (f32) or 8 (bf16) consecutive elements per step
    constexpr int E = 16 / sizeof(HT);
    for (int j = lane * E; j < a.d; j += 64 * E) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(h + j);
      const f32x4 w0 = *reinterpret_cast<const f32x4*>(a.w_h + j);
      if constexpr (sizeof(HT) == 2) {
        const f32x4 w1 = *reinterpret_cast<const f32x4*>(a.w_h + j + 4);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          s = fmaf(w0[2 * e], __uint_as_float(v[e] << 16), s);
          s = fmaf(w0[2 * e + 1], __uint_as_float(v[e] & 0xFFFF0000u), s);
          s = fmaf(w1[2 * e], __uint_as_float(v[e + 2] << 16), s);
          s = fmaf(w1[2 * e + 1], __uint_as_float(v[e + 2] & 0xFFFF0000u), s);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) s = fmaf(w0[e], __uint_as_float(v[e]), s);
      }
    }
  } else {
    for (int j = lane; j < a.d; j += 64) {
      float hv;
      if constexpr (sizeof(HT) == 2) hv = bf16_bits_to_f32(h[j]);
      else hv = h[j];
      s = fmaf(a.w_h[j], hv, s);
    }
  }
  const bool ok = prev >= 0 && prev < a.V;
  if (a.r > 0 && ok) {
    const uint16_t* e = a.W1 + (size_t)prev * a.r;
    for (int j = lane; j < a.r; j += 64) s = fmaf(a.w_e[j], bf16_bits_to_f32(e[j]), s);
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

struct StsArgs {
  int N, K, G, nbins, k;
  const float* logits;     // [N, K]
  const uint8_t* survived; // [N, K]
  const float* grid;       // [G]
  float* T_out;            // [K]
  float* ece_out;          // [K] or null
  double* ece_grid;        // [G] workspace
};

__device__ __forceinline__ double sigmoid_d(double z) { return 1.0 / (1.0 + exp(-z)); }

__global__ __launch_bounds__(kStsThreads) void sts_ece_kernel(StsArgs a) {
  __shared__ double sp[kStsMaxBins * kStsThreads];
  __shared__ int cnt[kStsMaxBins * kStsThreads];
  __shared__ int lab[kStsMaxBins * kStsThreads];
  const int t = threadIdx.x;
  const int g = blockIdx.x;
  for (int b = 0; b < a.nbins; ++b) {
    sp[b * kStsThreads + t] = 0.0;
    cnt[b * kStsThreads + t] = 0;
    lab[b * kStsThreads + t] = 0;
  }
  const double tg = (double)a.grid[g];
  for (int n = t; n < a.N; n += kStsThreads) {
    const float* l = a.logits + (size_t)n * a.K;
    double pred = 1.0;
    for (int i = 0; i < a.k; ++i) pred *= sigmoid_d((double)l[i] / (double)a.T_out[i]);
    pred *= sigmoid_d((double)l[a.k] / tg);
    int b = (int)(pred * a.nbins);
    b = b < 0 ? 0 : (b >= a.nbins ? a.nbins - 1 : b);
    sp[b * kStsThreads + t] += pred;
    cnt[b * kStsThreads + t] += 1;
    lab[b * kStsThreads + t] += a.survived[(size_t)n * a.K + a.k] ? 1 : 0;
  }
  __syncthreads();
  if (t < a.nbins) {  // thread b reduces bin b in thread order
    double s = 0.0;
    long long c = 0, y = 0;
    for (int u = 0; u < kStsThreads; ++u) {
      s += sp[t * kStsThreads + u];
      c += cnt[t * kStsThreads + u];
      y += lab[t * kStsThreads + u];
    }
    sp[t * kStsThreads] = c ? fabs((double)y - s) : 0.0;
  }
  __syncthreads();
  if (t == 0) {
    double e = 0.0;
    for (int b = 0; b < a.nbins; ++b) e += sp[b * kStsThreads];
    a.ece_grid[g] = e / (double)a.N;
  }
}

__global__ __launch_bounds__(64) void sts_pick_kernel(StsArgs a) {
  if (threadIdx.x != 0) return;
  int best = 0;
  for (int g = 1; g < a.G; ++g)
    if (a.ece_grid[g] < a.ece_grid[best]) best = g;  // the first minimum
  a.T_out[a.k] = a.grid[best];
  if (a.ece_out) a.ece_out[a.k] = (float)a.ece_grid[best];
}

size_t sts_workspace_bytes(int G) { return ((size_t)G * sizeof(double) + 255) / 256 * 256; }

int run_sts_fit(int N, int K, const float* logits, const uint8_t* survived, int G, const float* grid, int nbins,
                float* T_out, float* ece_out, void* workspace, hipStream_t stream) {
  StsArgs a{N, K, G, nbins, 0, logits, survived, grid, T_out, ece_out, reinterpret_cast<double*>(workspace)};
  for (int k = 0; k < K; ++k) {
    a.k = k;
    int rc = launch_kernel("sts_ece", sts_ece_kernel, dim3(G), dim3(kStsThreads), stream, a);
    if (rc) return rc;
    rc = launch_kernel("sts_pick", sts_pick_kernel, dim3(1), dim3(64), stream, a);
    if (rc) return rc;
  }
  return 0;
}

}  // namespace dspark
