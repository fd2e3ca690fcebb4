// Drives every entry point of the C ABI through its argument validation
// (valid calls, each documented error, extreme sizes) with host buffers and
// the launcher stand-ins of stubs.cpp; built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_host_sanitize.py.  Exits non-zero
// on the first status that differs from the documented one; the sanitizers
// abort on any memory error or undefined behaviour.
#include <atomic>
#include <climits>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <thread>
#include <vector>

#include "../../include/dspark.h"

extern std::atomic<int> g_launches;
static int g_fail = 0;

#define EXPECT(expr, want)                                                                      \
  do {                                                                                          \
    const long long got_ = (long long)(expr);                                                   \
    if (got_ != (long long)(want)) {                                                            \
      std::printf("FAIL line %d: %s = %lld, want %lld\n", __LINE__, #expr, got_, (long long)(want)); \
      ++g_fail;                                                                                 \
    }                                                                                           \
  } while (0)

// 256-byte aligned host buffer with room to spare
struct Buf {
  std::vector<unsigned char> raw;
  unsigned char* p;
  explicit Buf(size_t n) : raw(n + 512, 0) {
    p = raw.data() + (256 - reinterpret_cast<uintptr_t>(raw.data()) % 256) % 256;
  }
  template <typename T>
  T* as() { return reinterpret_cast<T*>(p); }
};

static void draft_cases() {
  const int B = 8, K = 7, V = 1000, r = 64;
  Buf U((size_t)B * K * V * 4), W1((size_t)V * r * 2), W2((size_t)V * r * 2), x0(B * 4), x(B * K * 4), q(B * K * 4),
      l(B * K * 4);
  const size_t wsb = dspark_markov_draft_workspace_bytes(B, K, V, r);
  EXPECT(wsb > 0, 1);
  Buf ws(wsb);
  auto call = [&](int b, int k, int v, int rr, float T, int dt, size_t wb, void* w, const void* w1) {
    return dspark_markov_draft(b, k, v, rr, T, U.p, dt, w1, W2.p, nullptr, x0.as<int32_t>(), 1, 2, x.as<int32_t>(),
                               q.as<float>(), l.as<float>(), w, wb, nullptr);
  };
  const int before = g_launches.load();
  EXPECT(call(B, K, V, r, 1.f, DSPARK_F32, wsb, ws.p, W1.p), DSPARK_OK);
  EXPECT(g_launches.load() > before, 1);
  EXPECT(call(B, K, V, r, 0.f, DSPARK_BF16, wsb, ws.p, W1.p), DSPARK_OK);
  EXPECT(call(0, K, V, r, 1.f, DSPARK_F32, 0, nullptr, W1.p), DSPARK_OK);  // empty batch
  EXPECT(call(-1, K, V, r, 1.f, DSPARK_F32, wsb, ws.p, W1.p), DSPARK_E_SHAPE);
  EXPECT(call(B, 0, V, r, 1.f, DSPARK_F32, wsb, ws.p, W1.p), DSPARK_E_SHAPE);
  EXPECT(call(B, DSPARK_MAX_K + 1, V, r, 1.f, DSPARK_F32, wsb, ws.p, W1.p), DSPARK_E_SHAPE);
  EXPECT(call(B, K, 0, r, 1.f, DSPARK_F32, wsb, ws.p, W1.p), DSPARK_E_SHAPE);
  EXPECT(call(B, K, V, 7, 1.f, DSPARK_F32, wsb, ws.p, W1.p), DSPARK_E_SHAPE);
  EXPECT(call(B, K, V, DSPARK_MAX_RANK + 8, 1.f, DSPARK_F32, wsb, ws.p, W1.p), DSPARK_E_SHAPE);
  EXPECT(call(B, K, V, r, 1.f, 7, wsb, ws.p, W1.p), DSPARK_E_DTYPE);
  EXPECT(call(INT_MAX, DSPARK_MAX_K, INT_MAX, r, 1.f, DSPARK_F32, wsb, ws.p, W1.p), DSPARK_E_SHAPE);
  EXPECT(call(B, K, INT_MAX, DSPARK_MAX_RANK, 1.f, DSPARK_F32, wsb, ws.p, W1.p), DSPARK_E_SHAPE);
  EXPECT(call(B, K, V, r, -1.f, DSPARK_F32, wsb, ws.p, W1.p), DSPARK_E_RANGE);
  EXPECT(call(B, K, V, r, NAN, DSPARK_F32, wsb, ws.p, W1.p), DSPARK_E_RANGE);
  EXPECT(call(B, K, V, r, INFINITY, DSPARK_F32, wsb, ws.p, W1.p), DSPARK_E_RANGE);
  EXPECT(call(B, K, V, r, 1.f, DSPARK_F32, wsb, ws.p, nullptr), DSPARK_E_NULL);
  EXPECT(call(B, K, V, r, 1.f, DSPARK_F32, wsb - 1, ws.p, W1.p), DSPARK_E_WORKSPACE);
  EXPECT(call(B, K, V, r, 1.f, DSPARK_F32, wsb, nullptr, W1.p), DSPARK_E_WORKSPACE);
  EXPECT(call(B, K, V, r, 1.f, DSPARK_F32, wsb - 8, ws.p + 8, W1.p), DSPARK_E_WORKSPACE);  // misaligned
  EXPECT(call(B, K, V, r, 1.f, DSPARK_F32, wsb, ws.p, W1.p + 2), DSPARK_E_RANGE);          // W1 not 16-byte aligned
  EXPECT(dspark_markov_draft_workspace_bytes(0, K, V, r), 0);
  EXPECT(dspark_markov_draft_workspace_bytes(INT_MAX, K, INT_MAX, r) > 0, 1);  // no overflow in the query
  // prepared W2
  const size_t fb = dspark_markov_w2_frag_bytes(V, r);
  Buf W2f(fb);
  EXPECT(dspark_markov_prepare_w2(V, r, W2.p, W2f.p, fb, nullptr), DSPARK_OK);
  EXPECT(dspark_markov_prepare_w2(V, r, W2.p, W2f.p, fb - 1, nullptr), DSPARK_E_WORKSPACE);
  EXPECT(dspark_markov_prepare_w2(V, r, nullptr, W2f.p, fb, nullptr), DSPARK_E_NULL);
  EXPECT(dspark_markov_prepare_w2(V, 12, W2.p, W2f.p, fb, nullptr), DSPARK_E_SHAPE);
  EXPECT(dspark_markov_prepare_w2(V, 0, nullptr, nullptr, 0, nullptr), DSPARK_OK);
  EXPECT(dspark_markov_prepare_w2(INT_MAX, DSPARK_MAX_RANK, W2.p, W2f.p, fb, nullptr), DSPARK_E_SHAPE);
  EXPECT(dspark_markov_prepare_w2(V, r, W2.p + 4, W2f.p, fb, nullptr), DSPARK_E_RANGE);
  // with W2f the workspace need drops to the partials
  const size_t small = dspark_markov_draft_workspace_bytes(B, K, V, 0);
  EXPECT(dspark_markov_draft(B, K, V, r, 1.f, U.p, DSPARK_F32, W1.p, W2.p, W2f.p, x0.as<int32_t>(), 1, 2,
                             x.as<int32_t>(), q.as<float>(), l.as<float>(), ws.p, small, nullptr),
         DSPARK_OK);
  // with the confidence head evaluated inside the draft
  const int d = 96;
  Buf H((size_t)B * K * d * 2), wh(d * 4), we(r * 4), c(B * K * 4), z(B * K * 4), T(K * 4);
  auto head = [&](int b, int dd, int ht, float bias, const void* h, const float* w_e, float* c_out) {
    return dspark_markov_draft_with_confidence(b, K, V, r, 1.f, U.p, DSPARK_F32, W1.p, W2.p, W2f.p, x0.as<int32_t>(),
                                               1, 2, x.as<int32_t>(), q.as<float>(), l.as<float>(), dd, h, ht,
                                               wh.as<float>(), w_e, bias, T.as<float>(), c_out, z.as<float>(), ws.p,
                                               small, nullptr);
  };
  EXPECT(head(B, d, DSPARK_BF16, 0.5f, H.p, we.as<float>(), c.as<float>()), DSPARK_OK);
  EXPECT(head(0, d, DSPARK_BF16, 0.5f, nullptr, nullptr, nullptr), DSPARK_OK);  // empty batch
  EXPECT(head(B, 0, DSPARK_BF16, 0.5f, H.p, we.as<float>(), c.as<float>()), DSPARK_E_SHAPE);
  EXPECT(head(B, INT_MAX, DSPARK_F32, 0.5f, H.p, we.as<float>(), c.as<float>()), DSPARK_E_SHAPE);
  EXPECT(head(B, d, 7, 0.5f, H.p, we.as<float>(), c.as<float>()), DSPARK_E_DTYPE);
  EXPECT(head(B, d, DSPARK_BF16, INFINITY, H.p, we.as<float>(), c.as<float>()), DSPARK_E_RANGE);
  EXPECT(head(B, d, DSPARK_BF16, 0.5f, nullptr, we.as<float>(), c.as<float>()), DSPARK_E_NULL);
  EXPECT(head(B, d, DSPARK_BF16, 0.5f, H.p, nullptr, c.as<float>()), DSPARK_E_NULL);
  EXPECT(head(B, d, DSPARK_BF16, 0.5f, H.p, we.as<float>(), nullptr), DSPARK_E_NULL);
}

static void schedule_cases() {
  const int R = 64, K = 7;
  Buf c(R * K * 4), sps((size_t)(R * (K + 1) + 1) * 8), a(R * K * 4), ell(R * 4), cu((R + 1) * 4), n(4), th(8), cap(4);
  const size_t wsb = dspark_schedule_workspace_bytes(R, K);
  Buf ws(wsb);
  const int sl = R * (K + 1) + 1;
  auto call = [&](int rr, int k, int len, int mode, int capacity, size_t wb, void* w) {
    return dspark_schedule(rr, k, c.as<float>(), sps.as<double>(), len, mode, capacity, a.as<float>(),
                           ell.as<int32_t>(), cu.as<int32_t>(), n.as<int32_t>(), th.as<double>(), w, wb, nullptr);
  };
  for (int mode = 0; mode <= 2; ++mode) EXPECT(call(R, K, sl, mode, 5, wsb, ws.p), DSPARK_OK);
  EXPECT(call(0, K, 1, 0, 0, 0, nullptr), DSPARK_OK);  // empty batch: no workspace needed
  EXPECT(call(-1, K, sl, 0, 0, wsb, ws.p), DSPARK_E_SHAPE);
  EXPECT(call(R, 0, sl, 0, 0, wsb, ws.p), DSPARK_E_SHAPE);
  EXPECT(call(R, DSPARK_MAX_K + 1, sl, 0, 0, wsb, ws.p), DSPARK_E_SHAPE);
  EXPECT(call(DSPARK_MAX_CANDIDATES, 2, sl, 0, 0, wsb, ws.p), DSPARK_E_SHAPE);
  EXPECT(call(INT_MAX, DSPARK_MAX_K, INT_MAX, 0, 0, wsb, ws.p), DSPARK_E_SHAPE);
  EXPECT(call(R, K, sl, 3, 0, wsb, ws.p), DSPARK_E_RANGE);
  EXPECT(call(R, K, sl, -1, 0, wsb, ws.p), DSPARK_E_RANGE);
  EXPECT(call(R, K, sl, 2, -1, wsb, ws.p), DSPARK_E_RANGE);
  EXPECT(call(R, K, R * (K + 1), 0, 0, wsb, ws.p), DSPARK_E_RANGE);  // sps too short
  EXPECT(call(R, K, sl, 0, 0, wsb - 1, ws.p), DSPARK_E_WORKSPACE);
  EXPECT(dspark_schedule(R, K, nullptr, sps.as<double>(), sl, 0, 0, a.as<float>(), ell.as<int32_t>(), cu.as<int32_t>(),
                         n.as<int32_t>(), th.as<double>(), ws.p, wsb, nullptr),
         DSPARK_E_NULL);
  EXPECT(dspark_schedule_workspace_bytes(INT_MAX, DSPARK_MAX_K), 0);
  // without a workspace
  EXPECT(dspark_schedule_noalloc(R, K, c.as<float>(), sps.as<double>(), sl, 0, 0, a.as<float>(), ell.as<int32_t>(),
                                 cu.as<int32_t>(), n.as<int32_t>(), th.as<double>(), nullptr),
         DSPARK_OK);
  EXPECT(dspark_schedule_noalloc(DSPARK_NOALLOC_MAX_CANDIDATES + 1, 1, c.as<float>(), sps.as<double>(), INT_MAX, 0, 0,
                                 a.as<float>(), ell.as<int32_t>(), cu.as<int32_t>(), n.as<int32_t>(), th.as<double>(),
                                 nullptr),
         DSPARK_E_SHAPE);
  // device-side capacity
  EXPECT(dspark_schedule_async(R, K, c.as<float>(), sps.as<double>(), sl, cap.as<int32_t>(), a.as<float>(),
                               ell.as<int32_t>(), cu.as<int32_t>(), n.as<int32_t>(), th.as<double>(), ws.p, wsb, nullptr),
         DSPARK_OK);
  EXPECT(dspark_schedule_async(0, K, nullptr, sps.as<double>(), 1, nullptr, nullptr, nullptr, cu.as<int32_t>(),
                               n.as<int32_t>(), th.as<double>(), nullptr, 0, nullptr),
         DSPARK_OK);
  EXPECT(dspark_schedule_async(R, K, c.as<float>(), sps.as<double>(), sl, nullptr, a.as<float>(), ell.as<int32_t>(),
                               cu.as<int32_t>(), n.as<int32_t>(), th.as<double>(), ws.p, wsb, nullptr),
         DSPARK_E_NULL);
}

static void verify_cases() {
  const int R = 8, K = 7, V = 1000, r = 64, N = R * (K + 1);
  Buf P((size_t)N * V * 4), D((size_t)R * K * V * 4), W1((size_t)V * r * 2), W2((size_t)V * r * 2), cu((R + 1) * 4),
      x0(R * 4), x(R * K * 4), q(R * K * 4), l(R * K * 4), na(R * 4), tok(R * 4), mm(R * 4);
  const size_t wsb = dspark_verify_workspace_bytes(R, K, V, r, N);
  Buf ws(wsb);
  auto call = [&](int rr, int k, int v, int rk, int n, float T, int pd, const float* qq, const float* ll, float* m,
                  size_t wb) {
    return dspark_verify(rr, k, v, T, P.p, pd, n, cu.as<int32_t>(), D.p, DSPARK_F32, W1.p, W2.p, nullptr, rk,
                         x0.as<int32_t>(), x.as<int32_t>(), qq, ll, 3, 4, na.as<int32_t>(), tok.as<int32_t>(), m, ws.p,
                         wb, nullptr);
  };
  EXPECT(call(R, K, V, r, N, 1.f, DSPARK_F32, q.as<float>(), l.as<float>(), mm.as<float>(), wsb), DSPARK_OK);
  EXPECT(call(R, K, V, r, N, 1.f, DSPARK_BF16, nullptr, nullptr, nullptr, wsb), DSPARK_OK);  // from logits
  EXPECT(call(R, K, V, r, N, 0.f, DSPARK_F32, nullptr, nullptr, mm.as<float>(), wsb), DSPARK_OK);
  EXPECT(call(0, K, V, r, 0, 1.f, DSPARK_F32, nullptr, nullptr, nullptr, 0), DSPARK_OK);
  EXPECT(call(R, K, V, r, R - 1, 1.f, DSPARK_F32, nullptr, nullptr, nullptr, wsb), DSPARK_E_SHAPE);
  EXPECT(call(R, K, V, r, N + 1, 1.f, DSPARK_F32, nullptr, nullptr, nullptr, wsb), DSPARK_E_SHAPE);
  EXPECT(call(INT_MAX, DSPARK_MAX_K, INT_MAX, r, INT_MAX, 1.f, DSPARK_F32, nullptr, nullptr, nullptr, wsb),
         DSPARK_E_SHAPE);
  EXPECT(call(R, K, V, r, N, 1.f, 9, nullptr, nullptr, nullptr, wsb), DSPARK_E_DTYPE);
  EXPECT(call(R, K, V, r, N, -0.5f, DSPARK_F32, nullptr, nullptr, nullptr, wsb), DSPARK_E_RANGE);
  EXPECT(call(R, K, V, r, N, 1.f, DSPARK_F32, nullptr, nullptr, mm.as<float>(), wsb - 1), DSPARK_E_WORKSPACE);
  EXPECT(dspark_verify_workspace_bytes(INT_MAX, DSPARK_MAX_K, INT_MAX, DSPARK_MAX_RANK, INT_MAX) > 0, 1);
  // RNN head
  const int rr = 64;
  Buf O((size_t)R * K * rr * 4), W2h(dspark_rnn_w2_f16_bytes(V, rr));
  const size_t rwb = dspark_rnn_verify_workspace_bytes(R, K, V, rr, N);
  Buf rws(rwb);
  EXPECT(dspark_rnn_verify(R, K, V, 1.f, P.p, DSPARK_F32, N, cu.as<int32_t>(), D.p, DSPARK_F32, O.as<float>(), W2.p,
                           nullptr, rr, x0.as<int32_t>(), x.as<int32_t>(), q.as<float>(), l.as<float>(), 3, 4,
                           na.as<int32_t>(), tok.as<int32_t>(), mm.as<float>(), rws.p, rwb, nullptr),
         DSPARK_OK);
  EXPECT(dspark_rnn_verify(R, K, V, 1.f, P.p, DSPARK_F32, N, cu.as<int32_t>(), D.p, DSPARK_F32, O.as<float>(), W2.p,
                           nullptr, rr, x0.as<int32_t>(), x.as<int32_t>(), nullptr, nullptr, 3, 4, na.as<int32_t>(),
                           tok.as<int32_t>(), nullptr, rws.p, rwb, nullptr),
         DSPARK_E_NULL);  // T > 0 needs q_tok and lse_d
  EXPECT(dspark_rnn_verify(R, K, V, 1.f, P.p, DSPARK_F32, N, cu.as<int32_t>(), D.p, DSPARK_F32, O.as<float>(), W2.p,
                           nullptr, 48, x0.as<int32_t>(), x.as<int32_t>(), q.as<float>(), l.as<float>(), 3, 4,
                           na.as<int32_t>(), tok.as<int32_t>(), nullptr, rws.p, rwb, nullptr),
         DSPARK_E_SHAPE);  // RNN rank: multiple of 32
}

static void label_rnn_cases() {
  const int B = 4, K = 7, V = 1000, r = 64, d = 128;
  Buf P((size_t)B * K * V * 4), D((size_t)B * K * V * 4), W1((size_t)V * r * 2), W2((size_t)V * r * 2), x0(B * 4),
      x(B * K * 4), l(B * K * 4), c(B * K * 4), H((size_t)B * K * d * 2), W((size_t)3 * r * (2 * r + d) * 2),
      O((size_t)B * K * r * 4), q(B * K * 4);
  const size_t lwb = dspark_acceptance_label_workspace_bytes(B, K, V, r);
  Buf lws(lwb);
  EXPECT(dspark_acceptance_label(B, K, V, 1.f, P.p, DSPARK_F32, D.p, DSPARK_BF16, W1.p, W2.p, nullptr, r,
                                 x0.as<int32_t>(), x.as<int32_t>(), l.as<float>(), c.as<float>(), lws.p, lwb, nullptr),
         DSPARK_OK);
  EXPECT(dspark_acceptance_label(B, K, V, 1.f, P.p, DSPARK_F32, D.p, DSPARK_BF16, W1.p, W2.p, nullptr, r,
                                 x0.as<int32_t>(), x.as<int32_t>(), nullptr, c.as<float>(), lws.p, lwb, nullptr),
         DSPARK_E_NULL);
  EXPECT(dspark_acceptance_label(B, K, V, 0.f, P.p, DSPARK_F32, D.p, DSPARK_BF16, W1.p, W2.p, nullptr, r,
                                 x0.as<int32_t>(), x.as<int32_t>(), nullptr, c.as<float>(), lws.p, lwb, nullptr),
         DSPARK_OK);
  const size_t rlwb = dspark_rnn_acceptance_label_workspace_bytes(B, K, V, r);
  Buf rlws(rlwb);
  EXPECT(dspark_rnn_acceptance_label(B, K, V, 1.f, P.p, DSPARK_F32, D.p, DSPARK_F32, O.as<float>(), W2.p, nullptr, r,
                                     x0.as<int32_t>(), x.as<int32_t>(), l.as<float>(), c.as<float>(), rlws.p, rlwb,
                                     nullptr),
         DSPARK_OK);
  // RNN draft
  const size_t dwb = dspark_rnn_draft_workspace_bytes(B, K, V, r, d);
  Buf dws(dwb);
  auto rnn = [&](int b, int dd, int rk, size_t wb) {
    return dspark_rnn_draft(b, K, V, rk, dd, 1.f, P.p, DSPARK_F32, H.p, DSPARK_BF16, W.p, W1.p, W2.p, nullptr,
                            x0.as<int32_t>(), 1, 2, x.as<int32_t>(), q.as<float>(), l.as<float>(), O.as<float>(), dws.p,
                            wb, nullptr);
  };
  EXPECT(rnn(B, d, r, dwb), DSPARK_OK);
  EXPECT(rnn(B, 96, r, dwb), DSPARK_E_SHAPE);   // d a multiple of 64
  EXPECT(rnn(B, d, 40, dwb), DSPARK_E_SHAPE);   // rank a multiple of 32
  EXPECT(rnn(B, d, r, dwb - 1), DSPARK_E_WORKSPACE);
  EXPECT(rnn(1, INT_MAX - 63, r, dwb), DSPARK_E_SHAPE);  // the weight size must not overflow
  EXPECT(rnn(0, d, r, 0), DSPARK_OK);
  const size_t hb = dspark_rnn_w2_f16_bytes(V, r);
  Buf W2h(hb);
  EXPECT(dspark_rnn_prepare_w2(V, r, W2.p, W2h.p, hb, nullptr), DSPARK_OK);
  EXPECT(dspark_rnn_prepare_w2(V, 16, W2.p, W2h.p, hb, nullptr), DSPARK_E_SHAPE);
}

static void misc_cases() {
  const int B = 4, K = 7, V = 1000, d = 64, r = 32;
  Buf H((size_t)B * K * d * 4), wh(d * 4), we(r * 4), W1((size_t)V * r * 2), x0(B * 4), x(B * K * 4), c(B * K * 4),
      lg(B * K * 4), T(K * 4), u(1024 * 4);
  EXPECT(dspark_confidence_head(B, K, V, d, r, H.p, DSPARK_F32, wh.as<float>(), we.as<float>(), 0.5f, W1.p,
                                x0.as<int32_t>(), x.as<int32_t>(), T.as<float>(), c.as<float>(), lg.as<float>(), nullptr),
         DSPARK_OK);
  EXPECT(dspark_confidence_head(B, K, V, d, r, H.p, DSPARK_F32, wh.as<float>(), we.as<float>(), NAN, W1.p,
                                x0.as<int32_t>(), x.as<int32_t>(), nullptr, c.as<float>(), nullptr, nullptr),
         DSPARK_E_RANGE);
  EXPECT(dspark_confidence_head(B, K, V, d, r, H.p, DSPARK_F32, wh.as<float>(), nullptr, 0.5f, W1.p, x0.as<int32_t>(),
                                x.as<int32_t>(), nullptr, c.as<float>(), nullptr, nullptr),
         DSPARK_E_NULL);
  const int N = 100, G = 16;
  Buf logits(N * K * 4), surv(N * K), grid(G * 4), To(K * 4), ece(4);
  const size_t sw = dspark_sts_fit_workspace_bytes(N, K, G);
  Buf sws(sw);
  EXPECT(dspark_sts_fit(N, K, logits.as<float>(), surv.as<uint8_t>(), G, grid.as<float>(), 10, To.as<float>(),
                        ece.as<float>(), sws.p, sw, nullptr),
         DSPARK_OK);
  EXPECT(dspark_sts_fit(N, K, logits.as<float>(), surv.as<uint8_t>(), G, grid.as<float>(), DSPARK_STS_MAX_BINS + 1,
                        To.as<float>(), ece.as<float>(), sws.p, sw, nullptr),
         DSPARK_E_RANGE);
  EXPECT(dspark_uniforms(1, 2, 1024, 3, 0, u.as<float>(), nullptr), DSPARK_OK);
  EXPECT(dspark_uniforms(1, 2, -1, 3, 0, u.as<float>(), nullptr), DSPARK_E_SHAPE);
  EXPECT(dspark_uniforms(1, 2, 8, 1 << 30, 0, u.as<float>(), nullptr), DSPARK_E_RANGE);
  EXPECT(dspark_uniforms(1, 2, 8, 3, 3, u.as<float>(), nullptr), DSPARK_E_RANGE);
  for (int s = 1; s >= -7; --s) EXPECT(std::strlen(dspark_status_string(s)) > 0, 1);
  EXPECT(dspark_version() >= 200, 1);
  EXPECT(std::strlen(dspark_build_id()) > 0, 1);
}

int main() {
  // the kernel timer on, driven from several host threads at once
  EXPECT(dspark_profiler_enable(1), DSPARK_OK);
  std::vector<std::thread> th;
  for (int t = 0; t < 8; ++t)
    th.emplace_back([t] {
      for (int i = 0; i < 3; ++i) {
        draft_cases();
        schedule_cases();
        if (t % 2) verify_cases();
        else label_rnn_cases();
        misc_cases();
      }
    });
  for (auto& t : th) t.join();
  const int kinds = dspark_profiler_read(0, nullptr, nullptr, nullptr);
  EXPECT(kinds > 5, 1);
  int64_t total = 0;
  for (int i = 0; i < kinds; ++i) {
    const char* name = nullptr;
    int64_t launches = 0;
    double ms = 0.0;
    EXPECT(dspark_profiler_read(i, &name, &launches, &ms), DSPARK_OK);
    total += launches;
  }
  EXPECT(total, g_launches.load());
  const char* past = nullptr;
  EXPECT(dspark_profiler_read(kinds, &past, nullptr, nullptr), DSPARK_E_RANGE);
  EXPECT(dspark_profiler_reset(), DSPARK_OK);
  EXPECT(dspark_profiler_read(0, nullptr, nullptr, nullptr), 0);
  EXPECT(dspark_profiler_enable(0), DSPARK_OK);
  std::printf("%s: %d launches checked, %d failures\n", g_fail ? "FAILED" : "ok", g_launches.load(), g_fail);
  return g_fail ? 1 : 0;
}
