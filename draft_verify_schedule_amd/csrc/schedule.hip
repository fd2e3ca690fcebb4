// Hardware-aware prefix scheduler (DSpark paper, section 3.2.2, Algorithm 1;
// modes of section 5.2; "Speculative decoding, from zero to DSpark", section 8).
//
// Two launches:
//   schedule_rank (one workgroup per 32 candidates): every workgroup builds
//     all candidate keys in LDS,
//       a[r,j] = c[r,1]*...*c[r,j] (float32, left to right), and for a > 0
//       key = ((0xFFFFFFFF - bits(a)) << 32) | ((j - 1) << 24) | r
//     so that ascending keys = a descending, then j ascending, then r
//     ascending (a is positive, so its bit pattern orders like its value);
//     keys are distinct, so the sorted position of a key is the number of
//     keys below it: 32 partial counts per key (1024 threads), summed, and the
//     key is written to that position of the workspace;
//   schedule (one workgroup of 1024 threads):
//     1. survival products again (a_out, the domain check, the candidate
//        count n_c), then thread t loads sorted keys t*E .. t*E+E-1
//        (E = candidates / 1024 rounded up to a power of two);
//     2. tau increments floor(a * 2^32) (exact int64 fixed point), block
//        prefix scan, Theta_n = double(tau_n) * 2^-32 * SPS[R + n] for every
//        admission count n; the cut n* is the first drop minus one
//        (EARLY_STOP), the earliest maximum (GLOBAL) or min(capacity, |E|)
//        (TOPK).  The fixed-point sum is exact, so this parallel evaluation
//        equals the sequential walk bit for bit;
//     3. l_r = number of r's candidates whose key lies below the n*-th sorted
//        key (a prefix of positions by construction), and cu_seqlens by a
//        block scan.
#include <mutex>

#include "common.hpp"
#include "launch.hpp"

namespace dspark {

constexpr int kSchedThreads = 1024;
constexpr int kSchedMaxKeys = 16384;

struct ScheduleArgs {
  int R, K;
  const float* __restrict__ c;
  const double* __restrict__ sps;
  int mode, capacity;
  float* __restrict__ a_out;
  int32_t* __restrict__ ell_out;
  int32_t* __restrict__ cu_out;
  int32_t* __restrict__ n_out;
  double* __restrict__ theta_out;
  const int32_t* __restrict__ capacity_dev;  // TOPK capacity read on the device, or null
};

constexpr int kSchedMaxK = 16;

// The K confidences of request r, all requested before the first is used
// (one memory round trip instead of K dependent ones).
__device__ __forceinline__ void load_confidences(const ScheduleArgs& a, int r, float (&cv)[kSchedMaxK]) {
#pragma unroll
  for (int j = 0; j < kSchedMaxK; ++j) cv[j] = (j < a.K) ? a.c[(size_t)r * a.K + j] : 1.0f;
}

__device__ __forceinline__ uint64_t make_key(float a, int j, int r) {
  return ((uint64_t)(0xFFFFFFFFu - __float_as_uint(a)) << 32) | ((uint64_t)j << 24) | (uint64_t)r;
}

__device__ __forceinline__ uint64_t key_increment(uint64_t key) {
  const float a = __uint_as_float(0xFFFFFFFFu - (uint32_t)(key >> 32));
  return (uint64_t)((double)a * 4294967296.0);  // a in (0, 1]: exact, truncation = floor
}

// Block-wide exclusive scan of one uint64 per thread (1024 threads = 16 waves).
__device__ __forceinline__ uint64_t block_exclusive_scan(uint64_t v, uint64_t* wave_sums,
                                                         uint64_t& total) {
  const int lane = threadIdx.x & 63;
  const int wave = wave_index();
  uint64_t incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint64_t o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wave_sums[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    uint64_t w = lane < kSchedThreads / 64 ? wave_sums[lane] : 0;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const uint64_t o = __shfl_up(w, off, 64);
      if (lane >= off) w += o;
    }
    if (lane < kSchedThreads / 64) wave_sums[lane] = w;  // inclusive wave totals
  }
  __syncthreads();
  const uint64_t before = wave ? wave_sums[wave - 1] : 0;
  total = wave_sums[kSchedThreads / 64 - 1];
  __syncthreads();
  return before + incl - v;
}

constexpr int kRankKeysPerWG = 32;
constexpr int kRankParts = kSchedThreads / kRankKeysPerWG;

__global__ __launch_bounds__(kSchedThreads) void schedule_rank_kernel(ScheduleArgs a, uint64_t* __restrict__ sorted) {
  __shared__ uint64_t keys[kSchedMaxKeys];
  __shared__ uint32_t part_cnt[kRankParts][kRankKeysPerWG];
  const int tid = threadIdx.x;
  const int R = a.R, K = a.K;
  const int n = R * K;
  for (int r = tid; r < R; r += kSchedThreads) {
    float cv[kSchedMaxK];
    load_confidences(a, r, cv);
    float acc = 1.0f;
#pragma unroll
    for (int j = 0; j < kSchedMaxK; ++j) {
      if (j < K) {
        acc = __fmul_rn(acc, cv[j]);
        keys[r * K + j] = (acc > 0.0f) ? make_key(acc, j, r) : ~0ull;
      }
    }
  }
  __syncthreads();
  // thread (part p, key slot q): keys of part p below key kk
  const int q = tid % kRankKeysPerWG;
  const int p = tid / kRankKeysPerWG;
  const int kk = blockIdx.x * kRankKeysPerWG + q;
  const uint64_t x = kk < n ? keys[kk] : ~0ull;
  const int y0 = (int)((int64_t)p * n / kRankParts);
  const int y1 = (int)((int64_t)(p + 1) * n / kRankParts);
  uint32_t cnt = 0;
  for (int y = y0; y < y1; ++y) cnt += keys[y] < x ? 1u : 0u;
  part_cnt[p][q] = cnt;
  __syncthreads();
  if (tid < kRankKeysPerWG && kk < n && x != ~0ull) {
    uint32_t rank = 0;
#pragma unroll
    for (int i = 0; i < kRankParts; ++i) rank += part_cnt[i][tid];
    sorted[rank] = x;  // rank < number of candidates with a > 0
  }
}

template <int E>
__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(ScheduleArgs a,
                                                                const uint64_t* __restrict__ sorted) {
  __shared__ uint64_t wave_sums[kSchedThreads / 64];
  __shared__ int bad;
  __shared__ int red_i[kSchedThreads / 64];
  __shared__ double red_d[kSchedThreads / 64];
  __shared__ uint64_t threshold_s;
  constexpr int P = kSchedThreads * E;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = wave_index();
  const int R = a.R, K = a.K;

  if (tid == 0) bad = 0;
  __syncthreads();

  // 1. survival products, the domain check and the number of candidates
  int cnt = 0;
  for (int r = tid; r < R; r += kSchedThreads) {
    float cv[kSchedMaxK];
    load_confidences(a, r, cv);
    float acc = 1.0f;
    bool ok = true;
#pragma unroll
    for (int j = 0; j < kSchedMaxK; ++j) {
      if (j < K) {
        ok = ok && (cv[j] >= 0.0f && cv[j] <= 1.0f);  // NaN fails both tests
        acc = __fmul_rn(acc, cv[j]);
        a.a_out[(size_t)r * K + j] = acc;
        cnt += acc > 0.0f;
      }
    }
    if (!ok) bad = 1;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) cnt += __shfl_xor(cnt, off, 64);
  if (lane == 0) red_i[wave] = cnt;
  __syncthreads();
  int n_c = 0;
  for (int w = 0; w < kSchedThreads / 64; ++w) n_c += red_i[w];
  __syncthreads();

  if (bad) {  // documented data error: a valid layout with no drafts
    for (int r = tid; r < R; r += kSchedThreads) {
      a.ell_out[r] = 0;
      a.cu_out[r + 1] = r + 1;
    }
    if (tid == 0) {
      a.cu_out[0] = 0;
      *a.n_out = -1;
      *a.theta_out = __longlong_as_double(0x7FF8000000000000ll);
    }
    return;
  }

  // thread tid holds sorted keys tid*E .. tid*E+E-1 (padding ~0)
  uint64_t v[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = tid * E + e;
    v[e] = (i < n_c) ? sorted[i] : ~0ull;
  }

  // 2. fixed-point tau over this thread's chunk, Theta per admission count
  const int i0 = tid * E;
  const int i1 = i0 + E;
  uint64_t local = 0;
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (i0 + e < n_c) local += key_increment(v[e]);
  uint64_t total;
  const uint64_t prefix = block_exclusive_scan(local, wave_sums, total);
  const uint64_t tau0 = (uint64_t)R << 32;
  const double theta0 = (double)tau0 * 0x1p-32 * a.sps[R];

  // candidate answer of this thread: EARLY_STOP -> first n with a drop;
  // GLOBAL -> best (Theta, smallest n)
  int first_drop = 0x7FFFFFFF;
  double best = (tid == 0) ? theta0 : -INFINITY;
  int best_n = (tid == 0) ? 0 : 0x7FFFFFFF;
  if (a.mode != 2 && i0 < n_c) {
    // SPS[R + i0 .. R + i1] of this thread's admission counts, requested together
    double spsv[E + 1];
#pragma unroll
    for (int e = 0; e <= E; ++e) spsv[e] = (i0 + e <= n_c) ? a.sps[R + i0 + e] : 0.0;
    uint64_t tau = tau0 + prefix;
    double prev_theta = (i0 == 0) ? theta0 : (double)tau * 0x1p-32 * spsv[0];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (i0 + e < n_c) {
        tau += key_increment(v[e]);
        const int n = i0 + e + 1;
        const double theta = (double)tau * 0x1p-32 * spsv[e + 1];
        if (theta <= prev_theta && n < first_drop) first_drop = n;
        if (theta > best) {
          best = theta;
          best_n = n;
        }
        prev_theta = theta;
      }
    }
  }
  // block reductions: min first_drop; max (best, -best_n)
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    first_drop = min(first_drop, __shfl_xor(first_drop, off, 64));
    const double b2 = __shfl_xor(best, off, 64);
    const int n2 = __shfl_xor(best_n, off, 64);
    if (b2 > best || (b2 == best && n2 < best_n)) {
      best = b2;
      best_n = n2;
    }
  }
  __shared__ int red_drop[kSchedThreads / 64];
  if (lane == 0) {
    red_drop[wave] = first_drop;
    red_i[wave] = best_n;
    red_d[wave] = best;
  }
  __syncthreads();
  __shared__ int n_star_s;
  if (tid == 0) {
    int fd = 0x7FFFFFFF, bn = 0x7FFFFFFF;
    double bv = -INFINITY;
    for (int w = 0; w < kSchedThreads / 64; ++w) {
      fd = min(fd, red_drop[w]);
      if (red_d[w] > bv || (red_d[w] == bv && red_i[w] < bn)) {
        bv = red_d[w];
        bn = red_i[w];
      }
    }
    int n_star;
    if (a.mode == 0) n_star = (fd == 0x7FFFFFFF) ? n_c : fd - 1;
    else if (a.mode == 1) n_star = bn;
    else n_star = min(max(a.capacity_dev ? *a.capacity_dev : a.capacity, 0), n_c);
    n_star_s = n_star;
    if (n_star >= P) threshold_s = ~0ull;
  }
  __syncthreads();
  const int n_star = n_star_s;
  // Theta of the chosen admission count and the threshold key (sorted index
  // n*), from the threads owning those indices
  if (n_star == 0) {
    if (tid == 0) *a.theta_out = theta0;
  } else if (n_star - 1 >= i0 && n_star - 1 < i1) {
    uint64_t tau = tau0 + prefix;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (i0 + e < n_star) tau += key_increment(v[e]);
    *a.theta_out = (double)tau * 0x1p-32 * a.sps[R + n_star];
  }
  if (n_star >= i0 && n_star < i1) {
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (i0 + e == n_star) threshold_s = v[e];
  }
  if (tid == 0) *a.n_out = n_star;
  __syncthreads();
  const uint64_t threshold = threshold_s;

  // 3. lengths and the flattened layout
  const int rper = (R + kSchedThreads - 1) / kSchedThreads;
  const int r0 = min(R, tid * rper);
  const int r1 = min(R, r0 + rper);
  uint64_t mine = 0;
  for (int r = r0; r < r1; ++r) {
    float cv[kSchedMaxK];
    load_confidences(a, r, cv);
    int ell = 0;
    float acc = 1.0f;
#pragma unroll
    for (int j = 0; j < kSchedMaxK; ++j) {
      if (j < K) {
        acc = __fmul_rn(acc, cv[j]);
        if (acc > 0.0f && make_key(acc, j, r) < threshold) ++ell;
      }
    }
    a.ell_out[r] = ell;
    mine += 1 + ell;
  }
  uint64_t all;
  uint64_t run = block_exclusive_scan(mine, wave_sums, all);
  if (tid == 0) a.cu_out[0] = 0;
  for (int r = r0; r < r1; ++r) {
    run += 1 + a.ell_out[r];
    a.cu_out[r + 1] = (int32_t)run;
  }
}

size_t schedule_workspace_bytes(int R, int K) {
  return (((size_t)R * K * sizeof(uint64_t)) + 255) & ~(size_t)255;
}

// An empty batch (R = 0): no candidates, B = tau = 0, so the layout is
// cu_seqlens = [0], nothing admitted, and Theta = 0 * SPS(0).
__global__ void schedule_empty_kernel(const double* __restrict__ sps, int32_t* __restrict__ cu_out,
                                      int32_t* __restrict__ n_out, double* __restrict__ theta_out) {
  if (threadIdx.x == 0) {
    cu_out[0] = 0;
    n_out[0] = 0;
    theta_out[0] = 0.0 * sps[0];
  }
}

int run_schedule(int R, int K, const float* c, const double* sps, int mode, int capacity,
                 const int32_t* capacity_dev, float* a_out, int32_t* ell_out, int32_t* cu_out, int32_t* n_out,
                 double* theta_out, void* workspace, hipStream_t stream) {
  if (R == 0)
    return launch_kernel("schedule", schedule_empty_kernel, dim3(1), dim3(64), stream, sps, cu_out, n_out, theta_out);
  ScheduleArgs a{R, K, c, sps, mode, capacity, a_out, ell_out, cu_out, n_out, theta_out, capacity_dev};
  uint64_t* sorted = reinterpret_cast<uint64_t*>(workspace);
  const int n = R * K;
  int rc = launch_kernel("schedule_rank", schedule_rank_kernel, dim3((n + kRankKeysPerWG - 1) / kRankKeysPerWG),
                         dim3(kSchedThreads), stream, a, sorted);
  if (rc) return rc;
  const uint64_t* cs = sorted;
  if (n <= kSchedThreads) return launch_kernel("schedule", schedule_kernel<1>, dim3(1), dim3(kSchedThreads), stream, a, cs);
  if (n <= 2 * kSchedThreads) return launch_kernel("schedule", schedule_kernel<2>, dim3(1), dim3(kSchedThreads), stream, a, cs);
  if (n <= 4 * kSchedThreads) return launch_kernel("schedule", schedule_kernel<4>, dim3(1), dim3(kSchedThreads), stream, a, cs);
  if (n <= 8 * kSchedThreads) return launch_kernel("schedule", schedule_kernel<8>, dim3(1), dim3(kSchedThreads), stream, a, cs);
  return launch_kernel("schedule", schedule_kernel<16>, dim3(1), dim3(kSchedThreads), stream, a, cs);
}

// ---- the schedule without a caller workspace --------------------------------
// The sorted candidate keys live in this library-owned device array instead
// of a workspace: every GPU the library runs on holds its own copy (128 KB)
// until the process ends, and every call on that GPU shares it.  In host
// code the name is a host-side stand-in, not a device address: kernels get
// the address hipGetSymbolAddress returns for the current device.
constexpr int kScratchKeys = kSchedMaxKeys;
static __device__ __align__(256) uint64_t scratch[kScratchKeys];

constexpr int kScratchMaxDevices = 64;
static std::mutex g_scratch_lock;
static void* g_scratch_ptr[kScratchMaxDevices] = {};

// The scratch array's device address on the current device, looked up once
// per device (with that device current); nullptr on failure.
static void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchMaxDevices) return nullptr;
  std::lock_guard<std::mutex> hold(g_scratch_lock);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

int schedule_scratch_keys() { return kScratchKeys; }

// dspark_schedule's launches with the sorted keys in the scratch array (no
// allocation, no workspace).  Returns -1 when R * K exceeds the array or its
// address cannot be had.  Nothing in the array needs to start at zero: the
// rank kernel writes every key the admission kernel reads.
int run_schedule_noalloc(int R, int K, const float* c, const double* sps, int mode, int capacity, float* a_out,
                         int32_t* ell_out, int32_t* cu_out, int32_t* n_out, double* theta_out, hipStream_t stream) {
  if ((int64_t)R * K > kScratchKeys) return -1;
  if (R == 0) return run_schedule(R, K, c, sps, mode, capacity, nullptr, a_out, ell_out, cu_out, n_out, theta_out,
                                  nullptr, stream);
  void* ptr = scratch_address();
  if (!ptr) return -1;
  return run_schedule(R, K, c, sps, mode, capacity, nullptr, a_out, ell_out, cu_out, n_out, theta_out, ptr, stream);
}

}  // namespace dspark
