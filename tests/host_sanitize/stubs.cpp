// Host-only stand-ins for the kernel launchers and the HIP event calls, so
// that the C ABI's host code (argument validation, workspace checks, the
// kernel timer) can be built with g++ under AddressSanitizer and
// UndefinedBehaviorSanitizer and run without a GPU.  Test infrastructure: the
// launchers only count calls and drive the kernel timer the way a launch
// does; the workspace sizes follow the library's layout in shape (size_t
// arithmetic, growing with every argument), not its exact values.
#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cstddef>
#include <cstdint>

#include "../../draft_verify_schedule_amd/csrc/rnn.hpp"

std::atomic<int> g_launches{0};

extern "C" hipError_t hipEventCreate(hipEvent_t* e) {
  static std::atomic<uintptr_t> next{0x1000};
  *e = reinterpret_cast<hipEvent_t>(next.fetch_add(16));
  return hipSuccess;
}
extern "C" hipError_t hipEventDestroy(hipEvent_t) { return hipSuccess; }
extern "C" hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }
extern "C" hipError_t hipEventElapsedTime(float* ms, hipEvent_t, hipEvent_t) {
  *ms = 0.25f;
  return hipSuccess;
}

namespace dspark {
bool profiler_on();
bool profiler_begin(const char* name, hipEvent_t* start, hipEvent_t* stop);
void profiler_end(hipEvent_t start, hipEvent_t stop);

static int launch(const char* name, hipStream_t) {
  hipEvent_t a = nullptr, b = nullptr;
  const bool prof = profiler_on() && profiler_begin(name, &a, &b);
  g_launches.fetch_add(1);
  if (prof) profiler_end(a, b);
  return 0;
}
static size_t al(size_t b) { return (b + 255) & ~(size_t)255; }

size_t draft_workspace_bytes(int B, int K, int V) {
  (void)K;
  return al((size_t)B * (size_t)(((int64_t)V + 63) / 64) * 8);
}
size_t w2_swizzle_bytes(int V, int r) {
  return r <= 0 ? 0 : (size_t)(((int64_t)V + 63) / 64) * 4 * (size_t)((r + 31) / 32) * 1024;
}
size_t w2_f16_bytes(int V, int r) { return (size_t)(((int64_t)V + 63) / 64) * 4 * (size_t)((r + 31) / 32) * 1024; }
size_t schedule_workspace_bytes(int R, int K) { return al((size_t)R * K * 8) + al((size_t)R * K * 4) + 256; }
int schedule_scratch_keys() { return 16384; }
size_t verify_workspace_need(int R, int K, int V, int r, int N, bool lse_given, bool w2f_given, bool margins,
                             float temperature) {
  size_t b = al((size_t)N * (size_t)(((int64_t)V + 255) / 256) * 16) + al((size_t)R * 64);
  if (!lse_given && temperature > 0.f) b += al((size_t)R * K * (size_t)(((int64_t)V + 63) / 64) * 8);
  if (!w2f_given) b += w2_swizzle_bytes(V, r);
  if (margins) b += al((size_t)R * 8);
  return b;
}
size_t verify_workspace_bytes(int R, int K, int V, int r, int N) {
  return verify_workspace_need(R, K, V, r, N, false, false, true, 1.f);
}
size_t label_workspace_bytes(int B, int K, int V, int r) {
  return al((size_t)B * K * (size_t)(((int64_t)V + 255) / 256) * 16) + w2_swizzle_bytes(V, r);
}
size_t sts_workspace_bytes(int N, int G) {
  return al((size_t)N * 16) + 2 * al((size_t)G * (size_t)((N + 4095) / 4096) * 32 * 8);
}
size_t rnn_workspace_bytes(int B, int K, int V, int r, int d, bool with_w2h) {
  return 4 * al((size_t)B * K * 3 * r * 4) + 2 * al((size_t)B * r * 4) + (with_w2h ? w2_f16_bytes(V, r) : 0) +
         (size_t)d * 0;
}
void rnn_bind_workspace(RnnParams& p, void* ws) {
  char* c = reinterpret_cast<char*>(ws);
  p.Hp = reinterpret_cast<float*>(c);
  p.s[0] = reinterpret_cast<float*>(c + al((size_t)p.B * p.K * 3 * p.r * 4));
  p.s[1] = p.s[0] + p.B * p.r;
  if (!p.w2h_ready) p.W2h = reinterpret_cast<uint16_t*>(c + al((size_t)p.B * p.K * 3 * p.r * 4) + 2 * al((size_t)p.B * p.r * 4));
}

int run_draft(int, int, int, int, float, const void*, bool, const void*, const void*, const void*, const int32_t*,
              uint64_t, uint64_t, int32_t*, float*, float*, void*, const RnnParams*, hipStream_t s) {
  return launch("draft_partials", s) | launch("draft_locate", s);
}
int run_w2_swizzle(const uint16_t*, void*, int, int, int, bool, hipStream_t s) { return launch("w2_swizzle", s); }
int run_w2_to_f16(const uint16_t*, uint16_t*, int, int, hipStream_t s) { return launch("w2_to_f16", s); }
int run_schedule(int, int, const float*, const double*, int, int, const int32_t*, float*, int32_t*, int32_t*, int32_t*,
                 double*, void*, hipStream_t s) {
  return launch("schedule_rank", s) | launch("schedule", s);
}
int run_schedule_noalloc(int, int, const float*, const double*, int, int, float*, int32_t*, int32_t*, int32_t*,
                         double*, hipStream_t s) {
  return launch("schedule_rank", s) | launch("schedule", s);
}
int run_verify(int, int, int, float, const void*, bool, int, const int32_t*, const void*, bool, const void*,
               const void*, const void*, int, const int32_t*, const int32_t*, const float*, const float*, uint64_t,
               uint64_t, int32_t*, int32_t*, float*, void*, const float*, const uint16_t*, hipStream_t s) {
  return launch("verify_rowstats", s) | launch("verify_accept", s);
}
int run_label(int, int, int, float, const void*, bool, const void*, bool, const void*, const void*, const void*, int,
              const int32_t*, const int32_t*, const float*, float*, void*, const float*, const uint16_t*,
              hipStream_t s) {
  return launch("label", s);
}
int run_confidence_head(int, int, int, int, int, const void*, bool, const float*, const float*, float, const void*,
                        const int32_t*, const int32_t*, const float*, float*, float*, hipStream_t s) {
  return launch("confidence_head", s);
}
int run_sts_fit(int, int, const float*, const uint8_t*, int, const float*, int, float*, float*, void*, hipStream_t s) {
  return launch("sts_fit", s);
}
int run_uniforms(uint64_t, uint64_t, int, int, int, float*, hipStream_t s) { return launch("uniforms", s); }
int run_rnn_hproj(const RnnParams&, hipStream_t s) { return launch("rnn_hproj", s); }
int run_rnn_step(const RnnParams&, int, hipStream_t s) { return launch("rnn_step", s); }
}  // namespace dspark
