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
//     keys below it (each wave ranks two keys, its lanes counting in
//     parallel); the key is written to that position of the workspace and
//     the position to the candidate's rank slot (no position for a = 0).
//     Workgroup 0 also
//     writes a_out, the domain check and the number of candidates n_c;
//   schedule (one workgroup of 1024 threads): every input it needs (n_c, the
//     domain flag, thread t's sorted keys t*E .. t*E+E-1 with
//     E = candidates / 1024 rounded up to a power of two, their SPS entries,
//     the ranks of thread t's requests' candidates) requested in one round
//     trip, then
//     1. tau increments floor(a * 2^32) (exact int64 fixed point), block
//        prefix scan, Theta_n = double(tau_n) * 2^-32 * SPS[R + n] for every
//        admission count n; the cut n* is the first drop minus one
//        (EARLY_STOP), the earliest maximum (GLOBAL) or min(capacity, |E|)
//        (TOPK).  The fixed-point sum is exact, so this parallel evaluation
//        equals the sequential walk bit for bit;
//     2. l_r = number of r's candidates ranked below n* (a prefix of
//        positions by construction), and cu_seqlens by a block scan.
#include <mutex>
#include <type_traits>

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

// uint64 lane exchanges on the DPP path: both halves moved with the same
// control; lanes without a source (or outside row_mask) receive `fill`.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ uint64_t dpp64(uint64_t v, uint64_t fill) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)fill, (int)(uint32_t)v, CTRL, ROWS, 0xF, false);
  const uint32_t hi =
      (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)(fill >> 32), (int)(uint32_t)(v >> 32), CTRL, ROWS, 0xF, false);
  return ((uint64_t)hi << 32) | lo;
}

// Inclusive uint64 prefix sum across the wave: row_shr 1, 2, 4, 8 inside each
// 16-lane row, then row totals carried by row_bcast:15 and row_bcast:31.
// Integer sums: exact whatever the association.
__device__ __forceinline__ uint64_t wave_inclusive_scan_u64(uint64_t v) {
  v += dpp64<0x111>(v, 0);
  v += dpp64<0x112>(v, 0);
  v += dpp64<0x114>(v, 0);
  v += dpp64<0x118>(v, 0);
  v += dpp64<0x142, 0xA>(v, 0);
  v += dpp64<0x143, 0xC>(v, 0);
  return v;
}

// Block-wide exclusive scan of one uint64 per thread (1024 threads = 16
// waves): wave scans on DPP, the wave totals through LDS (one barrier before
// they are read, one after so the array can be reused).
__device__ __forceinline__ uint64_t block_exclusive_scan(uint64_t v, uint64_t* wave_sums,
                                                         uint64_t& total) {
  const int lane = threadIdx.x & 63;
  const int wave = wave_index();
  const uint64_t incl = wave_inclusive_scan_u64(v);
  if (lane == 63) wave_sums[wave] = incl;
  __syncthreads();
  uint64_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kSchedThreads / 64; ++w) {
    const uint64_t t = wave_sums[w];
    before += w < wave ? t : 0;
    all += t;
  }
  total = all;
  __syncthreads();
  return before + incl - v;
}

// Wave reductions on the DPP path: quad xor 1 and 2, row half mirror and row
// mirror give every lane its row's result, row_bcast:15 / :31 fold the rows
// into lane 63, which is read back for the whole wave.  Lanes without a
// source take the identity.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ int dppi(int v, int fill) {
  return __builtin_amdgcn_update_dpp(fill, v, CTRL, ROWS, 0xF, false);
}
__device__ __forceinline__ int wave_min_i32(int x) {
  x = min(x, dppi<0xB1>(x, 0x7FFFFFFF));
  x = min(x, dppi<0x4E>(x, 0x7FFFFFFF));
  x = min(x, dppi<0x141>(x, 0x7FFFFFFF));
  x = min(x, dppi<0x140>(x, 0x7FFFFFFF));
  x = min(x, dppi<0x142, 0xA>(x, 0x7FFFFFFF));
  x = min(x, dppi<0x143, 0xC>(x, 0x7FFFFFFF));
  return __builtin_amdgcn_readlane(x, 63);
}
// (Theta, n): the larger Theta, on equal Theta the smaller n
__device__ __forceinline__ void best_merge(double& b, int& n, double b2, int n2) {
  if (b2 > b || (b2 == b && n2 < n)) {
    b = b2;
    n = n2;
  }
}
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ void best_step(double& b, int& n) {
  const double b2 = __longlong_as_double(
      (long long)dpp64<CTRL, ROWS>((uint64_t)__double_as_longlong(b), (uint64_t)__double_as_longlong(-INFINITY)));
  const int n2 = dppi<CTRL, ROWS>(n, 0x7FFFFFFF);
  best_merge(b, n, b2, n2);
}
__device__ __forceinline__ void wave_best(double& b, int& n) {
  best_step<0xB1>(b, n);
  best_step<0x4E>(b, n);
  best_step<0x141>(b, n);
  best_step<0x140>(b, n);
  best_step<0x142, 0xA>(b, n);
  best_step<0x143, 0xC>(b, n);
  const uint64_t bits = (uint64_t)__double_as_longlong(b);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)bits, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(bits >> 32), 63);
  b = __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
  n = __builtin_amdgcn_readlane(n, 63);
}

constexpr int kRankKeysPerWG = 2 * (kSchedThreads / 64);  // two keys per wave
constexpr int32_t kNoRank = 0x7FFFFFFF;  // a candidate with a = 0 is never admitted

// Workspace: the sorted keys, every candidate's rank, then (n_c, domain flag).
struct ScheduleWork {
  uint64_t* sorted;
  int32_t* rank;
  int32_t* meta;
};
__host__ __device__ inline size_t sched_align(size_t b) { return (b + 255) & ~(size_t)255; }
inline ScheduleWork schedule_work(void* ws, int n) {
  char* p = reinterpret_cast<char*>(ws);
  return ScheduleWork{reinterpret_cast<uint64_t*>(p), reinterpret_cast<int32_t*>(p + sched_align((size_t)n * 8)),
                      reinterpret_cast<int32_t*>(p + sched_align((size_t)n * 8) + sched_align((size_t)n * 4))};
}

__global__ __launch_bounds__(kSchedThreads) void schedule_rank_kernel(ScheduleArgs a, ScheduleWork w) {
  __shared__ uint64_t keys[kSchedMaxKeys];
  __shared__ int red_i[kSchedThreads / 64];
  __shared__ int bad;
  const int tid = threadIdx.x;
  const int R = a.R, K = a.K;
  const int n = R * K;
  const bool first = blockIdx.x == 0;  // workgroup 0 also writes a_out, n_c and the domain flag
  if (first && tid == 0) bad = 0;
  __syncthreads();
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
        keys[r * K + j] = (acc > 0.0f) ? make_key(acc, j, r) : ~0ull;
        if (first) a.a_out[(size_t)r * K + j] = acc;
        cnt += acc > 0.0f;
      }
    }
    if (first && !ok) bad = 1;
  }
  __syncthreads();
  if (first) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) cnt += __shfl_xor(cnt, off, 64);
    if ((tid & 63) == 0) red_i[wave_index()] = cnt;
  }
  // wave w ranks keys kk0 = 32 g + 2 w and kk0 + 1: lane l counts the keys
  // y = l, l + 64, ... below each (coalesced, conflict-free LDS reads), the
  // two counts are packed in one uint64 and summed across the wave
  const int lane = tid & 63;
  const int kk0 = blockIdx.x * kRankKeysPerWG + 2 * wave_index();
  const uint64_t x0 = kk0 < n ? keys[kk0] : ~0ull;
  const uint64_t x1 = kk0 + 1 < n ? keys[kk0 + 1] : ~0ull;
  uint32_t c0 = 0, c1 = 0;
  for (int y = lane; y < n; y += 64) {
    const uint64_t k = keys[y];
    c0 += k < x0 ? 1u : 0u;
    c1 += k < x1 ? 1u : 0u;
  }
  const uint64_t both = wave_inclusive_scan_u64((uint64_t)c0 | ((uint64_t)c1 << 32));  // lane 63: the totals
  if (lane == 63) {
    const uint32_t r0 = (uint32_t)both, r1 = (uint32_t)(both >> 32);
    if (kk0 < n) {
      if (x0 != ~0ull) w.sorted[r0] = x0;  // rank < number of candidates with a > 0
      w.rank[kk0] = x0 != ~0ull ? (int32_t)r0 : kNoRank;
    }
    if (kk0 + 1 < n) {
      if (x1 != ~0ull) w.sorted[r1] = x1;
      w.rank[kk0 + 1] = x1 != ~0ull ? (int32_t)r1 : kNoRank;
    }
  }
  __syncthreads();  // workgroup 0: every wave's count is in red_i
  if (first && tid == 0) {
    int n_c = 0;
    for (int i = 0; i < kSchedThreads / 64; ++i) n_c += red_i[i];
    w.meta[0] = n_c;
    w.meta[1] = bad;
  }
}

template <int E>
__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(ScheduleArgs a, ScheduleWork w) {
  __shared__ uint64_t wave_sums[kSchedThreads / 64];
  __shared__ int red_i[kSchedThreads / 64];
  __shared__ double red_d[kSchedThreads / 64];
  constexpr int P = kSchedThreads * E;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = wave_index();
  const int R = a.R, K = a.K;
  const int n = R * K;
  const int i0 = tid * E;
  const int i1 = i0 + E;
  const int rper = (R + kSchedThreads - 1) / kSchedThreads;
  const int r0 = min(R, tid * rper);
  const int r1 = min(R, r0 + rper);

  // every input in one round trip: n_c and the domain flag, this thread's
  // sorted keys (those past n_c are masked below), their SPS entries
  // (sps_len > R + n), the TOPK capacity, and with one request per thread
  // its candidates' ranks
  const int n_c = w.meta[0];
  const int bad = w.meta[1];
  uint64_t v[E];
#pragma unroll
  for (int e = 0; e < E; ++e) v[e] = (i0 + e < n) ? w.sorted[i0 + e] : ~0ull;
  double spsv[E + 1];
#pragma unroll
  for (int e = 0; e <= E; ++e) spsv[e] = (i0 + e <= n) ? a.sps[R + i0 + e] : 0.0;
  const int cap = (a.mode == 2 && a.capacity_dev) ? *a.capacity_dev : a.capacity;
  const double sps_R = a.sps[R];
  int32_t rk[kSchedMaxK];
  if (rper == 1) {
#pragma unroll
    for (int j = 0; j < kSchedMaxK; ++j) rk[j] = (j < K && r0 < r1) ? w.rank[(size_t)r0 * K + j] : kNoRank;
  }

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
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (i0 + e >= n_c) v[e] = ~0ull;

  // 1. fixed-point tau over this thread's chunk, Theta per admission count
  uint64_t local = 0;
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (i0 + e < n_c) local += key_increment(v[e]);
  uint64_t total;
  const uint64_t prefix = block_exclusive_scan(local, wave_sums, total);
  const uint64_t tau0 = (uint64_t)R << 32;
  const double theta0 = (double)tau0 * 0x1p-32 * sps_R;

  // candidate answer of this thread: EARLY_STOP -> first n with a drop;
  // GLOBAL -> best (Theta, smallest n)
  int first_drop = 0x7FFFFFFF;
  double best = (tid == 0) ? theta0 : -INFINITY;
  int best_n = (tid == 0) ? 0 : 0x7FFFFFFF;
  if (a.mode != 2 && i0 < n_c) {
    uint64_t tau = tau0 + prefix;
    double prev_theta = (i0 == 0) ? theta0 : (double)tau * 0x1p-32 * spsv[0];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (i0 + e < n_c) {
        tau += key_increment(v[e]);
        const int nn = i0 + e + 1;
        const double theta = (double)tau * 0x1p-32 * spsv[e + 1];
        if (theta <= prev_theta && nn < first_drop) first_drop = nn;
        if (theta > best) {
          best = theta;
          best_n = nn;
        }
        prev_theta = theta;
      }
    }
  }
  // block reductions: min first_drop; max (best, -best_n)
  first_drop = wave_min_i32(first_drop);
  wave_best(best, best_n);
  __shared__ int red_drop[kSchedThreads / 64];
  if (lane == 0) {
    red_drop[wave] = first_drop;
    red_i[wave] = best_n;
    red_d[wave] = best;
  }
  __syncthreads();
  // every thread combines the sixteen wave results (no second barrier)
  int n_star;
  {
    int fd = 0x7FFFFFFF, bn = 0x7FFFFFFF;
    double bv = -INFINITY;
#pragma unroll
    for (int i = 0; i < kSchedThreads / 64; ++i) {
      fd = min(fd, red_drop[i]);
      best_merge(bv, bn, red_d[i], red_i[i]);
    }
    if (a.mode == 0) n_star = (fd == 0x7FFFFFFF) ? n_c : fd - 1;
    else if (a.mode == 1) n_star = bn;
    else n_star = min(max(cap, 0), n_c);
  }
  // Theta of the chosen admission count, from the thread owning index n* - 1
  if (n_star == 0) {
    if (tid == 0) *a.theta_out = theta0;
  } else if (n_star - 1 >= i0 && n_star - 1 < i1) {
    uint64_t tau = tau0 + prefix;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (i0 + e < n_star) tau += key_increment(v[e]);
    *a.theta_out = (double)tau * 0x1p-32 * spsv[n_star - i0];
  }
  if (tid == 0) *a.n_out = n_star;

  // 2. lengths (candidates ranked below n*) and the flattened layout
  uint64_t mine = 0;
  if (rper == 1) {
    if (r0 < r1) {
      int ell = 0;
#pragma unroll
      for (int j = 0; j < kSchedMaxK; ++j) ell += rk[j] < n_star ? 1 : 0;
      a.ell_out[r0] = ell;
      mine = 1 + ell;
      rk[0] = ell;
    }
  } else {
    for (int r = r0; r < r1; ++r) {
      int ell = 0;
      for (int j = 0; j < K; ++j) ell += w.rank[(size_t)r * K + j] < n_star ? 1 : 0;
      a.ell_out[r] = ell;
      mine += 1 + ell;
    }
  }
  uint64_t all;
  uint64_t run = block_exclusive_scan(mine, wave_sums, all);
  if (tid == 0) a.cu_out[0] = 0;
  if (rper == 1) {
    if (r0 < r1) a.cu_out[r0 + 1] = (int32_t)(run + 1 + rk[0]);
  } else {
    for (int r = r0; r < r1; ++r) {
      run += 1 + a.ell_out[r];
      a.cu_out[r + 1] = (int32_t)run;
    }
  }
}

size_t schedule_workspace_bytes(int R, int K) {
  const size_t n = (size_t)R * K;
  return sched_align(n * 8) + sched_align(n * 4) + 256;
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
  const int n = R * K;
  const ScheduleWork w = schedule_work(workspace, n);
  int rc = launch_kernel("schedule_rank", schedule_rank_kernel, dim3((n + kRankKeysPerWG - 1) / kRankKeysPerWG),
                         dim3(kSchedThreads), stream, a, w);
  if (rc) return rc;
  if (n <= kSchedThreads) return launch_kernel("schedule", schedule_kernel<1>, dim3(1), dim3(kSchedThreads), stream, a, w);
  if (n <= 2 * kSchedThreads) return launch_kernel("schedule", schedule_kernel<2>, dim3(1), dim3(kSchedThreads), stream, a, w);
  if (n <= 4 * kSchedThreads) return launch_kernel("schedule", schedule_kernel<4>, dim3(1), dim3(kSchedThreads), stream, a, w);
  if (n <= 8 * kSchedThreads) return launch_kernel("schedule", schedule_kernel<8>, dim3(1), dim3(kSchedThreads), stream, a, w);
  return launch_kernel("schedule", schedule_kernel<16>, dim3(1), dim3(kSchedThreads), stream, a, w);
}

// ---- the schedule without a caller workspace --------------------------------
// The schedule's workspace (sorted candidate keys, candidate ranks, two
// counters) lives in this library-owned device array instead: every GPU the
// library runs on holds its own copy (about 193 KB) until the process ends,
// and every call on that GPU shares it.  In host code the name is a host-side
// stand-in, not a device address: kernels get the address hipGetSymbolAddress
// returns for the current device.
constexpr int kScratchKeys = kSchedMaxKeys;
constexpr size_t kScratchWords = (kScratchKeys * 8 + kScratchKeys * 4 + 256) / 8;  // schedule_workspace_bytes at the cap
static __device__ __align__(256) uint64_t scratch[kScratchWords];

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

// dspark_schedule's launches with their workspace in the scratch array (no
// allocation, no workspace argument).  Returns -1 when R * K exceeds the
// array or its address cannot be had.  Nothing in the array needs to start at
// zero: the rank kernel writes every key, rank and counter the admission
// kernel reads.
int run_schedule_noalloc(int R, int K, const float* c, const double* sps, int mode, int capacity, float* a_out,
                         int32_t* ell_out, int32_t* cu_out, int32_t* n_out, double* theta_out, hipStream_t stream) {
  if ((int64_t)R * K > kScratchKeys || schedule_workspace_bytes(R, K) > sizeof(scratch)) return -1;
  if (R == 0) return run_schedule(R, K, c, sps, mode, capacity, nullptr, a_out, ell_out, cu_out, n_out, theta_out,
                                  nullptr, stream);
  void* ptr = scratch_address();
  if (!ptr) return -1;
  return run_schedule(R, K, c, sps, mode, capacity, nullptr, a_out, ell_out, cu_out, n_out, theta_out, ptr, stream);
}

}  // namespace dspark
