// C ABI of libdspark: argument validation, workspace sizing, dispatch to the
// kernel launchers, and the event-based kernel timer.  Declarations and the
// documented contract live in include/dspark.h.
#include "../../include/dspark.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <deque>
#include <mutex>
#include <string>
#include <vector>

#include "rnn.hpp"

namespace dspark {
size_t draft_workspace_bytes(int B, int K, int V);
size_t w2_swizzle_bytes(int V, int r);
int run_draft(int B, int K, int V, int r, float temperature, const void* U, bool u_bf16, const void* W1,
              const void* W2, const void* W2f, const int32_t* x0, uint64_t seed, uint64_t step, int32_t* x_out,
              float* q_out, float* lse_out, void* workspace, const RnnParams* rnn, hipStream_t stream);
int run_w2_swizzle(const uint16_t* W2, void* out, int V, int r, int kc, bool f16, hipStream_t stream);
size_t schedule_workspace_bytes(int R, int K);
int run_schedule(int R, int K, const float* c, const double* sps, int mode, int capacity,
                 const int32_t* capacity_dev, float* a_out, int32_t* ell_out, int32_t* cu_out, int32_t* n_out,
                 double* theta_out, void* workspace, hipStream_t stream);
int run_schedule_noalloc(int R, int K, const float* c, const double* sps, int mode, int capacity, float* a_out,
                         int32_t* ell_out, int32_t* cu_out, int32_t* n_out, double* theta_out, hipStream_t stream);
int schedule_scratch_keys();
size_t verify_workspace_bytes(int R, int K, int V, int r, int N);
size_t verify_workspace_need(int R, int K, int V, int r, int N, bool lse_given, bool w2f_given, bool margins,
                             float temperature);
size_t label_workspace_bytes(int B, int K, int V, int r);
int run_confidence_head(int B, int K, int d, int r, int V, const void* H, bool h_bf16, const float* w_h,
                        const float* w_e, float bias, const void* W1, const int32_t* x0, const int32_t* x,
                        const float* T, float* c_out, float* logit_out, hipStream_t stream);
size_t sts_workspace_bytes(int N, int G);
int run_sts_fit(int N, int K, const float* logits, const uint8_t* survived, int G, const float* grid, int nbins,
                float* T_out, float* ece_out, void* workspace, hipStream_t stream);
int run_label(int B, int K, int V, float temperature, const void* P, bool p_bf16, const void* D, bool d_bf16,
              const void* W1, const void* W2, const void* W2f, int r, const int32_t* x0, const int32_t* x,
              const float* lse_d, float* c_out, void* workspace, const float* O, const uint16_t* W2h,
              hipStream_t stream);
int run_verify(int R, int K, int V, float temperature, const void* P, bool p_bf16, int N, const int32_t* cu,
               const void* D, bool d_bf16, const void* W1, const void* W2, const void* W2f, int r,
               const int32_t* x0, const int32_t* x, const float* q_tok, const float* lse_d, uint64_t seed,
               uint64_t step, int32_t* n_acc_out, int32_t* tok_out, float* min_margin_out, void* workspace,
               const float* O, const uint16_t* W2h, hipStream_t stream);
int run_uniforms(uint64_t seed, uint64_t step, int n, int position, int purpose, float* out, hipStream_t stream);

// ---- kernel timer --------------------------------------------------------
namespace {
struct Pending {
  int kernel;
  hipEvent_t start, stop;
};
struct KernelTotal {
  std::string name;
  int64_t launches = 0;
  double ms = 0.0;
};
// The timer may be driven from several host threads: the kernel's index is
// looked up, and the finished event pairs are queued, under one lock.
std::atomic<bool> g_prof{false};
std::mutex g_lock;
std::deque<KernelTotal> g_totals;  // a deque keeps each name's storage in place as it grows
std::vector<Pending> g_pending;
thread_local int g_open_kernel = -1;

int kernel_index(const char* name) {
  for (size_t i = 0; i < g_totals.size(); ++i)
    if (g_totals[i].name == name) return (int)i;
  g_totals.push_back(KernelTotal{name, 0, 0.0});
  return (int)g_totals.size() - 1;
}

void drain_pending() {
  for (Pending& p : g_pending) {
    float ms = 0.f;
    if (hipEventSynchronize(p.stop) == hipSuccess && hipEventElapsedTime(&ms, p.start, p.stop) == hipSuccess) {
      g_totals[p.kernel].ms += ms;
      g_totals[p.kernel].launches += 1;
    }
    (void)hipEventDestroy(p.start);
    (void)hipEventDestroy(p.stop);
  }
  g_pending.clear();
}
}  // namespace

bool profiler_on() { return g_prof.load(std::memory_order_relaxed); }

bool profiler_begin(const char* name, hipEvent_t* start, hipEvent_t* stop) {
  {
    std::lock_guard<std::mutex> hold(g_lock);
    g_open_kernel = kernel_index(name);
  }
  *start = *stop = nullptr;
  if (hipEventCreate(start) != hipSuccess) {
    *start = nullptr;
    g_open_kernel = -1;
    return false;
  }
  if (hipEventCreate(stop) != hipSuccess) {
    (void)hipEventDestroy(*start);
    *start = *stop = nullptr;
    g_open_kernel = -1;
    return false;
  }
  return true;
}

void profiler_end(hipEvent_t start, hipEvent_t stop) {
  if (g_open_kernel < 0) return;
  {
    std::lock_guard<std::mutex> hold(g_lock);
    g_pending.push_back(Pending{g_open_kernel, start, stop});
  }
  g_open_kernel = -1;
}
}  // namespace dspark

namespace {
bool is_dtype(int d) { return d == DSPARK_F32 || d == DSPARK_BF16; }
uint64_t dtype_bytes(int d) { return d == DSPARK_BF16 ? 2 : 4; }
// Kernels address each logit and factor buffer with 32-bit byte offsets.
constexpr uint64_t kMaxBufferBytes = (uint64_t)1 << 32;
bool rank_ok(int r) { return r >= 0 && r <= DSPARK_MAX_RANK && r % 8 == 0; }
// RNN head: the state is tiled in 32-column chunks and 16-unit MFMA blocks
bool rnn_rank_ok(int r) { return r >= 32 && r <= DSPARK_MAX_RANK && r % 32 == 0; }
bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }
int hip_status(int rc) { return rc == 0 ? DSPARK_OK : DSPARK_E_HIP; }
}  // namespace

extern "C" {

const char* dspark_status_string(int status) {
  switch (status) {
    case DSPARK_OK: return "ok";
    case DSPARK_E_NULL: return "a required pointer is NULL";
    case DSPARK_E_SHAPE: return "a dimension is out of its documented range";
    case DSPARK_E_DTYPE: return "unsupported dtype";
    case DSPARK_E_RANGE: return "a scalar argument is out of range";
    case DSPARK_E_WORKSPACE: return "workspace missing or too small";
    case DSPARK_E_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int dspark_version(void) { return 200; }

#ifndef DSPARK_BUILD_ID
#define DSPARK_BUILD_ID "unknown-sources!"
#endif
// The marker lets a loader read the id from the file without loading it.
static const char kBuildTag[] = "dspark-build-id:" DSPARK_BUILD_ID;
const char* dspark_build_id(void) { return kBuildTag + 16; }

size_t dspark_markov_w2_frag_bytes(int V, int r) {
  if (V <= 0 || !rank_ok(r)) return 0;
  return dspark::w2_swizzle_bytes(V, r);
}

int dspark_markov_prepare_w2(int V, int r, const void* W2, void* W2f, size_t W2f_bytes, void* stream) {
  if (V <= 0 || !rank_ok(r)) return DSPARK_E_SHAPE;
  if ((uint64_t)V * r * 2 >= kMaxBufferBytes) return DSPARK_E_SHAPE;
  if ((uint64_t)dspark::w2_swizzle_bytes(V, r) >= kMaxBufferBytes) return DSPARK_E_SHAPE;
  if (r == 0) return DSPARK_OK;
  if (!W2 || !W2f) return DSPARK_E_NULL;
  if (W2f_bytes < dspark::w2_swizzle_bytes(V, r)) return DSPARK_E_WORKSPACE;
  if (!aligned16(W2) || !aligned16(W2f)) return DSPARK_E_RANGE;
  return hip_status(dspark::run_w2_swizzle(reinterpret_cast<const uint16_t*>(W2), W2f, V, r, (r + 31) / 32, false,
                                           reinterpret_cast<hipStream_t>(stream)));
}

size_t dspark_markov_draft_workspace_bytes(int B, int K, int V, int r) {
  if (B <= 0 || V <= 0 || r < 0) return 0;
  // slice partials, then (Markov head) W2 in MFMA fragment order
  return dspark::draft_workspace_bytes(B, K, V) + dspark::w2_swizzle_bytes(V, r);
}

// Checks of dspark_markov_draft's arguments, before any work: DSPARK_OK, or
// the status to return (B == 0 returns DSPARK_OK through *empty).
static int check_markov_draft(int B, int K, int V, int r, float temperature, const void* U, int u_dtype,
                              const void* W1, const void* W2, const void* W2f, const int32_t* x0, int32_t* x_out,
                              float* q_tok_out, float* lse_out, void* workspace, size_t workspace_bytes,
                              bool* empty) {
  *empty = false;
  if (B < 0 || K <= 0 || K > DSPARK_MAX_K || V <= 0 || !rank_ok(r)) return DSPARK_E_SHAPE;
  if (!is_dtype(u_dtype)) return DSPARK_E_DTYPE;
  if ((uint64_t)B * K * V * dtype_bytes(u_dtype) >= kMaxBufferBytes) return DSPARK_E_SHAPE;
  if ((uint64_t)V * r * 2 >= kMaxBufferBytes) return DSPARK_E_SHAPE;
  if ((uint64_t)dspark::w2_swizzle_bytes(V, r) >= kMaxBufferBytes) return DSPARK_E_SHAPE;
  if (!(temperature >= 0.f) || std::isinf(temperature)) return DSPARK_E_RANGE;
  if (B == 0) {  // empty batch
    *empty = true;
    return DSPARK_OK;
  }
  if (!U || !x0 || !x_out || !q_tok_out || !lse_out) return DSPARK_E_NULL;
  if (r > 0 && (!W1 || !W2)) return DSPARK_E_NULL;
  const size_t need = dspark::draft_workspace_bytes(B, K, V) + (W2f ? 0 : dspark::w2_swizzle_bytes(V, r));
  if (!workspace || workspace_bytes < need) return DSPARK_E_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return DSPARK_E_WORKSPACE;
  if (r > 0 && (!aligned16(W1) || !aligned16(W2) || !aligned16(W2f))) return DSPARK_E_RANGE;
  return DSPARK_OK;
}

int dspark_markov_draft(int B, int K, int V, int r, float temperature, const void* U, int u_dtype,
                        const void* W1, const void* W2, const void* W2f, const int32_t* x0, uint64_t seed,
                        uint64_t step, int32_t* x_out, float* q_tok_out, float* lse_out, void* workspace,
                        size_t workspace_bytes, void* stream) {
  bool empty;
  const int st = check_markov_draft(B, K, V, r, temperature, U, u_dtype, W1, W2, W2f, x0, x_out, q_tok_out, lse_out,
                                    workspace, workspace_bytes, &empty);
  if (st != DSPARK_OK || empty) return st;
  return hip_status(dspark::run_draft(B, K, V, r, temperature, U, u_dtype == DSPARK_BF16, W1, W2, r > 0 ? W2f : nullptr,
                                      x0, seed, step, x_out, q_tok_out, lse_out, workspace, nullptr,
                                      reinterpret_cast<hipStream_t>(stream)));
}

int dspark_markov_draft_with_confidence(int B, int K, int V, int r, float temperature, const void* U, int u_dtype,
                                        const void* W1, const void* W2, const void* W2f, const int32_t* x0,
                                        uint64_t seed, uint64_t step, int32_t* x_out, float* q_tok_out,
                                        float* lse_out, int d, const void* H, int h_dtype, const float* w_h,
                                        const float* w_e, float bias, const float* sts_temperature, float* c_out,
                                        float* logit_out, void* workspace, size_t workspace_bytes, void* stream) {
  bool empty;
  const int st = check_markov_draft(B, K, V, r, temperature, U, u_dtype, W1, W2, W2f, x0, x_out, q_tok_out, lse_out,
                                    workspace, workspace_bytes, &empty);
  if (st != DSPARK_OK) return st;
  // the confidence head's checks (those of dspark_confidence_head)
  if (d <= 0) return DSPARK_E_SHAPE;
  if (!is_dtype(h_dtype)) return DSPARK_E_DTYPE;
  if ((uint64_t)B * K * d * dtype_bytes(h_dtype) >= kMaxBufferBytes) return DSPARK_E_SHAPE;
  if (!std::isfinite(bias)) return DSPARK_E_RANGE;
  if (empty) return DSPARK_OK;
  if (!H || !w_h || !c_out) return DSPARK_E_NULL;
  if (r > 0 && !w_e) return DSPARK_E_NULL;
  // the head runs as its own launch right after the draft, on the drafted
  // tokens: evaluated inside the draft's locate pass it cost more (its
  // hidden-state row and w_h more than double that latency-bound pass's
  // memory traffic)
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int rc = dspark::run_draft(B, K, V, r, temperature, U, u_dtype == DSPARK_BF16, W1, W2, r > 0 ? W2f : nullptr,
                                   x0, seed, step, x_out, q_tok_out, lse_out, workspace, nullptr, s);
  if (rc) return hip_status(rc);
  return hip_status(dspark::run_confidence_head(B, K, d, r, V, H, h_dtype == DSPARK_BF16, w_h, r > 0 ? w_e : nullptr,
                                                bias, W1, x0, x_out, sts_temperature, c_out, logit_out, s));
}

size_t dspark_rnn_w2_f16_bytes(int V, int r) {
  if (V <= 0 || !rnn_rank_ok(r)) return 0;
  return dspark::w2_f16_bytes(V, r);
}

int dspark_rnn_prepare_w2(int V, int r, const void* W2, void* W2h, size_t W2h_bytes, void* stream) {
  if (V <= 0 || !rnn_rank_ok(r)) return DSPARK_E_SHAPE;
  if ((uint64_t)V * r * 2 >= kMaxBufferBytes) return DSPARK_E_SHAPE;
  if ((uint64_t)dspark::w2_f16_bytes(V, r) >= kMaxBufferBytes) return DSPARK_E_SHAPE;
  if (!W2 || !W2h) return DSPARK_E_NULL;
  if (W2h_bytes < dspark::w2_f16_bytes(V, r)) return DSPARK_E_WORKSPACE;
  if (!aligned16(W2) || !aligned16(W2h)) return DSPARK_E_RANGE;
  return hip_status(dspark::run_w2_to_f16(reinterpret_cast<const uint16_t*>(W2), reinterpret_cast<uint16_t*>(W2h),
                                          V, r, reinterpret_cast<hipStream_t>(stream)));
}

size_t dspark_rnn_draft_workspace_bytes(int B, int K, int V, int r, int d) {
  if (B <= 0 || K <= 0 || V <= 0 || r <= 0 || d < 64) return 0;
  const size_t base = (dspark::draft_workspace_bytes(B, K, V) + 255) / 256 * 256;
  return base + dspark::rnn_workspace_bytes(B, K, V, r, d);
}

int dspark_rnn_draft(int B, int K, int V, int r, int d, float temperature, const void* U, int u_dtype,
                     const void* H, int h_dtype, const void* W, const void* W1, const void* W2, const void* W2h,
                     const int32_t* x0, uint64_t seed, uint64_t step, int32_t* x_out, float* q_tok_out,
                     float* lse_out, float* o_out, void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 0 || K <= 0 || K > DSPARK_MAX_K || V <= 0 || !rnn_rank_ok(r)) return DSPARK_E_SHAPE;
  if (d < 64 || d % 64 != 0) return DSPARK_E_SHAPE;
  if (!is_dtype(u_dtype) || h_dtype != DSPARK_BF16) return DSPARK_E_DTYPE;
  if ((uint64_t)B * K * V * dtype_bytes(u_dtype) >= kMaxBufferBytes) return DSPARK_E_SHAPE;
  if ((uint64_t)V * r * 2 >= kMaxBufferBytes) return DSPARK_E_SHAPE;
  if ((uint64_t)dspark::w2_f16_bytes(V, r) >= kMaxBufferBytes) return DSPARK_E_SHAPE;
  if ((uint64_t)B * K * d * 2 >= kMaxBufferBytes) return DSPARK_E_SHAPE;
  if ((uint64_t)3 * r * ((uint64_t)2 * r + (uint64_t)d) * 2 >= kMaxBufferBytes) return DSPARK_E_SHAPE;
  if (!(temperature >= 0.f) || std::isinf(temperature)) return DSPARK_E_RANGE;
  if (B == 0) return DSPARK_OK;  // empty batch
  if (!U || !H || !W || !W1 || !W2 || !x0 || !x_out || !q_tok_out || !lse_out || !o_out) return DSPARK_E_NULL;
  const size_t base = (dspark::draft_workspace_bytes(B, K, V) + 255) / 256 * 256;
  const size_t need = base + dspark::rnn_workspace_bytes(B, K, V, r, d, W2h == nullptr);
  if (!workspace || workspace_bytes < need) return DSPARK_E_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return DSPARK_E_WORKSPACE;
  if (!aligned16(W1) || !aligned16(W2) || !aligned16(H) || !aligned16(W) || !aligned16(o_out) || !aligned16(W2h))
    return DSPARK_E_RANGE;
  dspark::RnnParams p{};
  p.B = B;
  p.K = K;
  p.V = V;
  p.r = r;
  p.d = d;
  p.H = reinterpret_cast<const uint16_t*>(H);
  p.W = reinterpret_cast<const uint16_t*>(W);
  p.W1 = reinterpret_cast<const uint16_t*>(W1);
  p.x0 = x0;
  p.x = x_out;
  p.O = o_out;
  p.W2 = reinterpret_cast<const uint16_t*>(W2);
  p.w2h_ready = W2h != nullptr;
  p.W2h = const_cast<uint16_t*>(reinterpret_cast<const uint16_t*>(W2h));
  dspark::rnn_bind_workspace(p, reinterpret_cast<char*>(workspace) + base);
  return hip_status(dspark::run_draft(B, K, V, r, temperature, U, u_dtype == DSPARK_BF16, W1, W2, nullptr, x0, seed,
                                      step, x_out, q_tok_out, lse_out, workspace, &p,
                                      reinterpret_cast<hipStream_t>(stream)));
}

size_t dspark_schedule_workspace_bytes(int R, int K) {
  if (R <= 0 || K <= 0 || K > DSPARK_MAX_K || (int64_t)R * K > DSPARK_MAX_CANDIDATES) return 0;
  return dspark::schedule_workspace_bytes(R, K);
}

int dspark_schedule(int R, int K, const float* c, const double* sps, int sps_len, int mode, int capacity,
                    float* a_out, int32_t* ell_out, int32_t* cu_seqlens_out, int32_t* n_admitted_out,
                    double* theta_out, void* workspace, size_t workspace_bytes, void* stream) {
  if (R < 0 || K <= 0 || K > DSPARK_MAX_K || (int64_t)R * K > DSPARK_MAX_CANDIDATES) return DSPARK_E_SHAPE;
  if (mode < DSPARK_SCHED_EARLY_STOP || mode > DSPARK_SCHED_TOPK) return DSPARK_E_RANGE;
  if (capacity < 0) return DSPARK_E_RANGE;
  if ((int64_t)sps_len <= (int64_t)R * (K + 1)) return DSPARK_E_RANGE;
  if (!sps || !cu_seqlens_out || !n_admitted_out || !theta_out) return DSPARK_E_NULL;
  if (R > 0 && (!c || !a_out || !ell_out)) return DSPARK_E_NULL;
  if (R > 0 && (!workspace || workspace_bytes < dspark::schedule_workspace_bytes(R, K))) return DSPARK_E_WORKSPACE;
  return hip_status(dspark::run_schedule(R, K, c, sps, mode, capacity, nullptr, a_out, ell_out, cu_seqlens_out,
                                         n_admitted_out, theta_out, workspace,
                                         reinterpret_cast<hipStream_t>(stream)));
}

int dspark_schedule_noalloc(int R, int K, const float* c, const double* sps, int sps_len, int mode, int capacity,
                            float* a_out, int32_t* ell_out, int32_t* cu_seqlens_out, int32_t* n_admitted_out,
                            double* theta_out, void* stream) {
  if (R < 0 || K <= 0 || K > DSPARK_MAX_K || (int64_t)R * K > DSPARK_MAX_CANDIDATES) return DSPARK_E_SHAPE;
  if ((int64_t)R * K > DSPARK_NOALLOC_MAX_CANDIDATES || (int64_t)R * K > dspark::schedule_scratch_keys())
    return DSPARK_E_SHAPE;
  if (mode < DSPARK_SCHED_EARLY_STOP || mode > DSPARK_SCHED_TOPK) return DSPARK_E_RANGE;
  if (capacity < 0) return DSPARK_E_RANGE;
  if ((int64_t)sps_len <= (int64_t)R * (K + 1)) return DSPARK_E_RANGE;
  if (!sps || !cu_seqlens_out || !n_admitted_out || !theta_out) return DSPARK_E_NULL;
  if (R > 0 && (!c || !a_out || !ell_out)) return DSPARK_E_NULL;
  return hip_status(dspark::run_schedule_noalloc(R, K, c, sps, mode, capacity, a_out, ell_out, cu_seqlens_out,
                                                 n_admitted_out, theta_out, reinterpret_cast<hipStream_t>(stream)));
}

int dspark_schedule_async(int R, int K, const float* c, const double* sps, int sps_len, const int32_t* capacity,
                          float* a_out, int32_t* ell_out, int32_t* cu_seqlens_out, int32_t* n_admitted_out,
                          double* theta_out, void* workspace, size_t workspace_bytes, void* stream) {
  if (R < 0 || K <= 0 || K > DSPARK_MAX_K || (int64_t)R * K > DSPARK_MAX_CANDIDATES) return DSPARK_E_SHAPE;
  if ((int64_t)sps_len <= (int64_t)R * (K + 1)) return DSPARK_E_RANGE;
  if (!sps || !cu_seqlens_out || !n_admitted_out || !theta_out) return DSPARK_E_NULL;
  if (R > 0 && (!c || !capacity || !a_out || !ell_out)) return DSPARK_E_NULL;
  if (R > 0 && (!workspace || workspace_bytes < dspark::schedule_workspace_bytes(R, K))) return DSPARK_E_WORKSPACE;
  return hip_status(dspark::run_schedule(R, K, c, sps, DSPARK_SCHED_TOPK, 0, capacity, a_out, ell_out,
                                         cu_seqlens_out, n_admitted_out, theta_out, workspace,
                                         reinterpret_cast<hipStream_t>(stream)));
}

size_t dspark_verify_workspace_bytes(int R, int K, int V, int r, int N) {
  if (R <= 0 || K <= 0 || K > DSPARK_MAX_K || V <= 0 || N <= 0 || !rank_ok(r)) return 0;
  return dspark::verify_workspace_bytes(R, K, V, r, N);
}

int dspark_verify(int R, int K, int V, float temperature, const void* P, int p_dtype, int N,
                  const int32_t* cu_seqlens, const void* D, int d_dtype, const void* W1, const void* W2,
                  const void* W2f, int r, const int32_t* x0, const int32_t* x, const float* q_tok,
                  const float* lse_d, uint64_t seed, uint64_t step, int32_t* n_acc_out, int32_t* tok_out,
                  float* min_margin_out, void* workspace, size_t workspace_bytes, void* stream) {
  if (R < 0 || K <= 0 || K > DSPARK_MAX_K || V <= 0 || !rank_ok(r)) return DSPARK_E_SHAPE;
  if (N < R || (int64_t)N > (int64_t)R * (K + 1)) return DSPARK_E_SHAPE;
  if (!is_dtype(p_dtype) || !is_dtype(d_dtype)) return DSPARK_E_DTYPE;
  if ((uint64_t)N * V * dtype_bytes(p_dtype) >= kMaxBufferBytes) return DSPARK_E_SHAPE;
  if ((uint64_t)R * K * V * dtype_bytes(d_dtype) >= kMaxBufferBytes) return DSPARK_E_SHAPE;
  if ((uint64_t)V * r * 2 >= kMaxBufferBytes) return DSPARK_E_SHAPE;
  if ((uint64_t)dspark::w2_swizzle_bytes(V, r) >= kMaxBufferBytes) return DSPARK_E_SHAPE;
  if (!(temperature >= 0.f) || std::isinf(temperature)) return DSPARK_E_RANGE;
  if (R == 0) return DSPARK_OK;  // empty batch
  if (!P || !cu_seqlens || !D || !x0 || !x || !n_acc_out || !tok_out) return DSPARK_E_NULL;
  if (r > 0 && (!W1 || !W2)) return DSPARK_E_NULL;
  const size_t need = dspark::verify_workspace_need(R, K, V, r, N, lse_d != nullptr, W2f != nullptr,
                                                    min_margin_out != nullptr, temperature);
  if (!workspace || workspace_bytes < need) return DSPARK_E_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return DSPARK_E_WORKSPACE;
  if (r > 0 && (!aligned16(W1) || !aligned16(W2) || !aligned16(W2f))) return DSPARK_E_RANGE;
  return hip_status(dspark::run_verify(R, K, V, temperature, P, p_dtype == DSPARK_BF16, N, cu_seqlens, D,
                                       d_dtype == DSPARK_BF16, W1, W2, r > 0 ? W2f : nullptr, r, x0, x, q_tok, lse_d,
                                       seed, step, n_acc_out, tok_out, min_margin_out, workspace, nullptr, nullptr,
                                       reinterpret_cast<hipStream_t>(stream)));
}

size_t dspark_rnn_verify_workspace_bytes(int R, int K, int V, int r, int N) {
  if (R <= 0 || K <= 0 || K > DSPARK_MAX_K || V <= 0 || N <= 0 || !rnn_rank_ok(r)) return 0;
  return (dspark::verify_workspace_need(R, K, V, 0, N, true, true, true, 1.f) + 255) / 256 * 256 +
         dspark::w2_f16_bytes(V, r);
}

int dspark_rnn_verify(int R, int K, int V, float temperature, const void* P, int p_dtype, int N,
                      const int32_t* cu_seqlens, const void* D, int d_dtype, const float* O, const void* W2,
                      const void* W2h, int r, const int32_t* x0, const int32_t* x, const float* q_tok,
                      const float* lse_d, uint64_t seed, uint64_t step, int32_t* n_acc_out, int32_t* tok_out,
                      float* min_margin_out, void* workspace, size_t workspace_bytes, void* stream) {
  if (R < 0 || K <= 0 || K > DSPARK_MAX_K || V <= 0 || !rnn_rank_ok(r)) return DSPARK_E_SHAPE;
  if (N < R || (int64_t)N > (int64_t)R * (K + 1)) return DSPARK_E_SHAPE;
  if (!is_dtype(p_dtype) || !is_dtype(d_dtype)) return DSPARK_E_DTYPE;
  if ((uint64_t)N * V * dtype_bytes(p_dtype) >= kMaxBufferBytes) return DSPARK_E_SHAPE;
  if ((uint64_t)R * K * V * dtype_bytes(d_dtype) >= kMaxBufferBytes) return DSPARK_E_SHAPE;
  if ((uint64_t)V * r * 2 >= kMaxBufferBytes) return DSPARK_E_SHAPE;
  if ((uint64_t)dspark::w2_f16_bytes(V, r) >= kMaxBufferBytes) return DSPARK_E_SHAPE;
  if (!(temperature >= 0.f) || std::isinf(temperature)) return DSPARK_E_RANGE;
  if (R == 0) return DSPARK_OK;  // empty batch
  if (!P || !cu_seqlens || !D || !O || !W2 || !x0 || !x || !n_acc_out || !tok_out) return DSPARK_E_NULL;
  if (temperature > 0.f && (!q_tok || !lse_d)) return DSPARK_E_NULL;
  // the verify passes see r = 0 (the bias comes from O); margins sized always
  const size_t base = (dspark::verify_workspace_need(R, K, V, 0, N, true, true, true, 1.f) + 255) / 256 * 256;
  if (!workspace || workspace_bytes < base + (W2h ? 0 : dspark::w2_f16_bytes(V, r))) return DSPARK_E_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return DSPARK_E_WORKSPACE;
  if (!aligned16(O) || !aligned16(W2) || !aligned16(W2h)) return DSPARK_E_RANGE;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const uint16_t* W2hp = reinterpret_cast<const uint16_t*>(W2h);
  if (!W2hp) {
    uint16_t* own = reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(workspace) + base);
    if (dspark::run_w2_to_f16(reinterpret_cast<const uint16_t*>(W2), own, V, r, s)) return DSPARK_E_HIP;
    W2hp = own;
  }
  return hip_status(dspark::run_verify(R, K, V, temperature, P, p_dtype == DSPARK_BF16, N, cu_seqlens, D,
                                       d_dtype == DSPARK_BF16, nullptr, W2, nullptr, r, x0, x, q_tok, lse_d, seed,
                                       step, n_acc_out, tok_out, min_margin_out, workspace, O, W2hp, s));
}

size_t dspark_acceptance_label_workspace_bytes(int B, int K, int V, int r) {
  if (B <= 0 || K <= 0 || K > DSPARK_MAX_K || V <= 0 || r < 0) return 0;
  return dspark::label_workspace_bytes(B, K, V, r);
}

int dspark_acceptance_label(int B, int K, int V, float temperature, const void* P, int p_dtype, const void* D,
                            int d_dtype, const void* W1, const void* W2, const void* W2f, int r, const int32_t* x0,
                            const int32_t* x, const float* lse_d, float* c_out, void* workspace,
                            size_t workspace_bytes, void* stream) {
  if (B < 0 || K <= 0 || K > DSPARK_MAX_K || V <= 0 || !rank_ok(r)) return DSPARK_E_SHAPE;
  if (!is_dtype(p_dtype) || !is_dtype(d_dtype)) return DSPARK_E_DTYPE;
  if ((uint64_t)B * K * V * dtype_bytes(p_dtype) >= kMaxBufferBytes) return DSPARK_E_SHAPE;
  if ((uint64_t)B * K * V * dtype_bytes(d_dtype) >= kMaxBufferBytes) return DSPARK_E_SHAPE;
  if ((uint64_t)V * r * 2 >= kMaxBufferBytes) return DSPARK_E_SHAPE;
  if ((uint64_t)dspark::w2_swizzle_bytes(V, r) >= kMaxBufferBytes) return DSPARK_E_SHAPE;
  if (!(temperature >= 0.f) || std::isinf(temperature)) return DSPARK_E_RANGE;
  if (B == 0) return DSPARK_OK;  // empty batch
  if (!P || !D || !x0 || !x || !c_out) return DSPARK_E_NULL;
  if (temperature > 0.f && !lse_d) return DSPARK_E_NULL;
  if (r > 0 && (!W1 || !W2)) return DSPARK_E_NULL;
  const size_t need = dspark::label_workspace_bytes(B, K, V, W2f ? 0 : r);
  if (!workspace || workspace_bytes < need) return DSPARK_E_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return DSPARK_E_WORKSPACE;
  if (r > 0 && (!aligned16(W1) || !aligned16(W2) || !aligned16(W2f))) return DSPARK_E_RANGE;
  return hip_status(dspark::run_label(B, K, V, temperature, P, p_dtype == DSPARK_BF16, D, d_dtype == DSPARK_BF16,
                                      W1, W2, r > 0 ? W2f : nullptr, r, x0, x, lse_d, c_out, workspace, nullptr,
                                      nullptr, reinterpret_cast<hipStream_t>(stream)));
}

size_t dspark_rnn_acceptance_label_workspace_bytes(int B, int K, int V, int r) {
  if (B <= 0 || K <= 0 || K > DSPARK_MAX_K || V <= 0 || r <= 0) return 0;
  return (dspark::label_workspace_bytes(B, K, V, 0) + 255) / 256 * 256 + dspark::w2_f16_bytes(V, r);
}

int dspark_rnn_acceptance_label(int B, int K, int V, float temperature, const void* P, int p_dtype, const void* D,
                                int d_dtype, const float* O, const void* W2, const void* W2h, int r,
                                const int32_t* x0, const int32_t* x, const float* lse_d, float* c_out,
                                void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 0 || K <= 0 || K > DSPARK_MAX_K || V <= 0 || !rnn_rank_ok(r)) return DSPARK_E_SHAPE;
  if (!is_dtype(p_dtype) || !is_dtype(d_dtype)) return DSPARK_E_DTYPE;
  if ((uint64_t)B * K * V * dtype_bytes(p_dtype) >= kMaxBufferBytes) return DSPARK_E_SHAPE;
  if ((uint64_t)B * K * V * dtype_bytes(d_dtype) >= kMaxBufferBytes) return DSPARK_E_SHAPE;
  if ((uint64_t)V * r * 2 >= kMaxBufferBytes) return DSPARK_E_SHAPE;
  if ((uint64_t)dspark::w2_f16_bytes(V, r) >= kMaxBufferBytes) return DSPARK_E_SHAPE;
  if (!(temperature >= 0.f) || std::isinf(temperature)) return DSPARK_E_RANGE;
  if (B == 0) return DSPARK_OK;  // empty batch
  if (!P || !D || !O || !W2 || !x0 || !x || !c_out) return DSPARK_E_NULL;
  if (temperature > 0.f && !lse_d) return DSPARK_E_NULL;
  const size_t base = (dspark::label_workspace_bytes(B, K, V, 0) + 255) / 256 * 256;
  if (!workspace || workspace_bytes < base + (W2h ? 0 : dspark::w2_f16_bytes(V, r))) return DSPARK_E_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return DSPARK_E_WORKSPACE;
  if (!aligned16(O) || !aligned16(W2) || !aligned16(W2h)) return DSPARK_E_RANGE;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const uint16_t* W2hp = reinterpret_cast<const uint16_t*>(W2h);
  if (!W2hp) {
    uint16_t* own = reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(workspace) + base);
    if (dspark::run_w2_to_f16(reinterpret_cast<const uint16_t*>(W2), own, V, r, s)) return DSPARK_E_HIP;
    W2hp = own;
  }
  return hip_status(dspark::run_label(B, K, V, temperature, P, p_dtype == DSPARK_BF16, D, d_dtype == DSPARK_BF16,
                                      nullptr, W2, nullptr, r, x0, x, lse_d, c_out, workspace, O, W2hp, s));
}

int dspark_confidence_head(int B, int K, int V, int d, int r, const void* H, int h_dtype, const float* w_h,
                           const float* w_e, float bias, const void* W1, const int32_t* x0, const int32_t* x,
                           const float* sts_temperature, float* c_out, float* logit_out, void* stream) {
  if (B < 0 || K <= 0 || K > DSPARK_MAX_K || V <= 0 || d <= 0 || !rank_ok(r)) return DSPARK_E_SHAPE;
  if (!is_dtype(h_dtype)) return DSPARK_E_DTYPE;
  if ((uint64_t)B * K * d * dtype_bytes(h_dtype) >= kMaxBufferBytes) return DSPARK_E_SHAPE;
  if (!std::isfinite(bias)) return DSPARK_E_RANGE;
  if (B == 0) return DSPARK_OK;  // empty batch
  if (!H || !w_h || !x0 || !x || !c_out) return DSPARK_E_NULL;
  if (r > 0 && (!W1 || !w_e)) return DSPARK_E_NULL;
  return hip_status(dspark::run_confidence_head(B, K, d, r, V, H, h_dtype == DSPARK_BF16, w_h, w_e, bias, W1, x0,
                                                x, sts_temperature, c_out, logit_out,
                                                reinterpret_cast<hipStream_t>(stream)));
}

size_t dspark_sts_fit_workspace_bytes(int N, int K, int n_grid) {
  if (N <= 0 || K <= 0 || n_grid <= 0 || n_grid > DSPARK_STS_MAX_GRID) return 0;
  return dspark::sts_workspace_bytes(N, n_grid);
}

int dspark_sts_fit(int N, int K, const float* logits, const uint8_t* survived, int n_grid, const float* grid,
                   int n_bins, float* T_out, float* ece_out, void* workspace, size_t workspace_bytes,
                   void* stream) {
  if (N <= 0 || K <= 0 || K > DSPARK_MAX_K || n_grid <= 0 || n_grid > DSPARK_STS_MAX_GRID) return DSPARK_E_SHAPE;
  if ((uint64_t)N * K * sizeof(float) >= kMaxBufferBytes) return DSPARK_E_SHAPE;
  if (n_bins < 1 || n_bins > DSPARK_STS_MAX_BINS) return DSPARK_E_RANGE;
  if (!logits || !survived || !grid || !T_out) return DSPARK_E_NULL;
  if (!workspace || workspace_bytes < dspark::sts_workspace_bytes(N, n_grid)) return DSPARK_E_WORKSPACE;
  return hip_status(dspark::run_sts_fit(N, K, logits, survived, n_grid, grid, n_bins, T_out, ece_out, workspace,
                                        reinterpret_cast<hipStream_t>(stream)));
}

int dspark_uniforms(uint64_t seed, uint64_t step, int n, int position, int purpose, float* out, void* stream) {
  if (n < 0) return DSPARK_E_SHAPE;
  if (position < 0 || position >= (1 << 30) || purpose < 0 || purpose > 2) return DSPARK_E_RANGE;
  if (n == 0) return DSPARK_OK;
  if (!out) return DSPARK_E_NULL;
  return hip_status(dspark::run_uniforms(seed, step, n, position, purpose, out, reinterpret_cast<hipStream_t>(stream)));
}

int dspark_profiler_enable(int on) {
  dspark::g_prof.store(on != 0);
  return DSPARK_OK;
}

int dspark_profiler_reset(void) {
  std::lock_guard<std::mutex> hold(dspark::g_lock);
  dspark::drain_pending();
  dspark::g_totals.clear();
  return DSPARK_OK;
}

int dspark_profiler_read(int index, const char** name, int64_t* launches, double* total_ms) {
  std::lock_guard<std::mutex> hold(dspark::g_lock);
  dspark::drain_pending();
  if (!name) return (int)dspark::g_totals.size();
  if (index < 0 || index >= (int)dspark::g_totals.size()) return DSPARK_E_RANGE;
  *name = dspark::g_totals[index].name.c_str();
  if (launches) *launches = dspark::g_totals[index].launches;
  if (total_ms) *total_ms = dspark::g_totals[index].ms;
  return DSPARK_OK;
}

}  // extern "C"
