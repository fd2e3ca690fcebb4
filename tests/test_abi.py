"""The C-ABI library: it loads, exports every entry point include/dspark.h
declares, and rejects bad arguments on the host before touching the GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dspark.h")


@pytest.fixture(scope="module")
def lib():
    import __graft_entry__  # noqa: F401  (build helper)
    from draft_verify_schedule_amd import binding
    __graft_entry__._ensure_built()
    return binding.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dspark_[a-z_]+)\s*\(", text)))


def test_header_declares_the_three_calls():
    names = declared_functions()
    for n in ("dspark_markov_draft", "dspark_schedule", "dspark_verify"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for st in range(-6, 1):
        assert lib.dspark_status_string(st)
    assert lib.dspark_version() >= 200


def test_build_id_matches_the_sources(lib):
    """The library carries the hash of the sources it was built from, the one
    the build helper computes from the tree (a stale library would differ)."""
    from draft_verify_schedule_amd import _build
    bid = lib.dspark_build_id().decode()
    assert len(bid) == 16 and bid == _build.built_id() == _build.source_hash()


def test_workspace_queries(lib):
    assert lib.dspark_markov_draft_workspace_bytes(512, 7, 151936, 256) >= 512 * 2374 * 8
    assert lib.dspark_markov_draft_workspace_bytes(512, 7, 151936, 256) % 256 == 0
    # the Markov head adds W2 in MFMA fragment order: ceil(V / 64) blocks of 4 x ceil(r / 32) KB
    for r in (8, 24, 64, 256):
        extra = lib.dspark_markov_draft_workspace_bytes(512, 7, 151936, r) - \
            lib.dspark_markov_draft_workspace_bytes(512, 7, 151936, 0)
        assert extra == 2374 * 4 * ((r + 31) // 32) * 1024
    assert lib.dspark_verify_workspace_bytes(512, 7, 151936, 256, 4096) > 0
    assert lib.dspark_verify_workspace_bytes(0, 7, 10, 0, 1) == 0
    assert lib.dspark_schedule_workspace_bytes(512, 7) >= 512 * 7 * 8
    assert lib.dspark_schedule_workspace_bytes(512, 7) % 256 == 0
    assert lib.dspark_schedule_workspace_bytes(4096, 7) == 0
    assert lib.dspark_acceptance_label_workspace_bytes(512, 7, 151936, 256) >= 512 * 7 * 2374 * 4
    assert lib.dspark_acceptance_label_workspace_bytes(0, 7, 10, 0) == 0


NULL = ctypes.c_void_p(0)
FAKE = ctypes.c_void_p(0x100000)   # never dereferenced: every case fails validation first
WS = ctypes.c_size_t(1 << 30)


def test_schedule_argument_errors(lib):
    # R < 0, K too large, too many candidates
    assert lib.dspark_schedule(-1, 7, FAKE, FAKE, 100, 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, WS, NULL) == -2
    assert lib.dspark_schedule(4, 17, FAKE, FAKE, 100, 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, WS, NULL) == -2
    assert lib.dspark_schedule(4096, 7, FAKE, FAKE, 10 ** 6, 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, WS, NULL) == -2
    # SPS table too short, bad mode, negative capacity
    assert lib.dspark_schedule(4, 7, FAKE, FAKE, 32, 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, WS, NULL) == -4
    assert lib.dspark_schedule(4, 7, FAKE, FAKE, 33, 3, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, WS, NULL) == -4
    assert lib.dspark_schedule(4, 7, FAKE, FAKE, 33, 2, -1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, WS, NULL) == -4
    # NULL input
    assert lib.dspark_schedule(4, 7, NULL, FAKE, 33, 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, WS, NULL) == -1
    # workspace missing or too small
    assert lib.dspark_schedule(4, 7, FAKE, FAKE, 33, 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, WS, NULL) == -5
    small = ctypes.c_size_t(lib.dspark_schedule_workspace_bytes(4, 7) - 1)
    assert lib.dspark_schedule(4, 7, FAKE, FAKE, 33, 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, small, NULL) == -5


def test_schedule_async_argument_errors(lib):
    def call(R=4, K=7, c=FAKE, sps=FAKE, n=33, cap=FAKE, out=FAKE, ws=FAKE, wsb=WS):
        return lib.dspark_schedule_async(R, K, c, sps, n, cap, out, out, out, out, out, ws, wsb, NULL)
    assert call(R=-1) == -2
    assert call(K=17) == -2
    assert call(n=32) == -4
    assert call(cap=NULL) == -1
    assert call(c=NULL) == -1
    assert call(ws=NULL) == -5
    assert call(wsb=ctypes.c_size_t(lib.dspark_schedule_workspace_bytes(4, 7) - 1)) == -5


def test_acceptance_label_argument_errors(lib):
    f = ctypes.c_float

    def call(B=4, K=7, V=1024, r=16, T=1.0, P=FAKE, pt=0, D=FAKE, dt=0, W=FAKE, x0=FAKE, x=FAKE, lse=FAKE,
             out=FAKE, wsp=FAKE, wsb=WS):
        return lib.dspark_acceptance_label(B, K, V, f(T), P, pt, D, dt, W, W, NULL, r, x0, x, lse, out, wsp, wsb,
                                           NULL)
    assert call(B=-1) == -2
    assert call(K=17) == -2
    assert call(r=12) == -2
    assert call(pt=7) == -3
    assert call(T=-1.0) == -4
    assert call(P=NULL) == -1
    assert call(lse=NULL) == -1
    assert call(T=0.0, lse=NULL, wsp=NULL) == -5     # lse_d not needed when greedy
    assert call(W=NULL) == -1
    assert call(wsb=ctypes.c_size_t(lib.dspark_acceptance_label_workspace_bytes(4, 7, 1024, 16) - 1)) == -5
    # with a prepared W2 copy the label needs no room for its own
    assert lib.dspark_acceptance_label(4, 7, 1024, f(1.0), FAKE, 0, FAKE, 0, FAKE, FAKE, ctypes.c_void_p(0x100008),
                                       16, FAKE, FAKE, FAKE, FAKE, FAKE, WS, NULL) == -4   # W2f not 16-byte aligned


def test_confidence_and_sts_argument_errors(lib):
    f = ctypes.c_float

    def head(B=4, K=7, V=100, d=32, r=8, H=FAKE, ht=0, wh=FAKE, we=FAKE, b=0.0, W1=FAKE, x0=FAKE, x=FAKE, out=FAKE):
        return lib.dspark_confidence_head(B, K, V, d, r, H, ht, wh, we, f(b), W1, x0, x, NULL, out, NULL, NULL)
    assert head(B=-1) == -2
    assert head(d=0) == -2
    assert head(r=12) == -2
    assert head(ht=5) == -3
    assert head(H=NULL) == -1
    assert head(W1=NULL) == -1
    assert head(b=float("inf")) == -4

    def sts(N=100, K=7, lg=FAKE, sv=FAKE, G=9, grid=FAKE, nb=10, T=FAKE, ws=FAKE, wsb=WS):
        return lib.dspark_sts_fit(N, K, lg, sv, G, grid, nb, T, NULL, ws, wsb, NULL)
    assert sts(N=0) == -2
    assert sts(G=0) == -2
    assert sts(G=65536) == -2        # more grid temperatures than one launch dimension holds
    assert lib.dspark_sts_fit_workspace_bytes(100, 7, 65536) == 0
    assert sts(nb=0) == -4
    assert sts(nb=33) == -4
    assert sts(lg=NULL) == -1
    assert sts(ws=NULL) == -5
    # the samples' fp64 cumulative products and per-bin partials of every grid value
    assert lib.dspark_sts_fit_workspace_bytes(100, 7, 9) >= 100 * 16 + 9 * 32 * 12


def test_draft_argument_errors(lib):
    f = ctypes.c_float
    ws = ctypes.c_size_t(1 << 30)
    base = dict(B=4, K=7, V=1024, r=16)

    def call(B=4, K=7, V=1024, r=16, T=1.0, U=FAKE, dt=1, W1=FAKE, W2=FAKE, W2f=NULL, x0=FAKE, out=FAKE, wsp=FAKE,
             wsb=ws):
        return lib.dspark_markov_draft(B, K, V, r, f(T), U, dt, W1, W2, W2f, x0, ctypes.c_uint64(1),
                                       ctypes.c_uint64(0), out, out, out, wsp, wsb, NULL)
    assert call(K=0) == -2
    assert call(K=17) == -2
    assert call(r=12) == -2          # not a multiple of 8
    # W2 itself fits (1.1 GB) but its fragment-ordered copy (4 KB per 64 columns at r = 8) would not
    assert call(B=1, K=1, V=70_000_000, r=8) == -2
    assert call(r=264) == -2         # above DSPARK_MAX_RANK
    assert call(dt=5) == -3
    assert call(T=-1.0) == -4
    assert call(T=float("nan")) == -4
    assert call(U=NULL) == -1
    assert call(W1=NULL) == -1
    assert call(wsb=ctypes.c_size_t(16)) == -5
    assert call(wsp=NULL) == -5
    # the partials alone are enough workspace when the caller brings the W2 copy
    part = lib.dspark_markov_draft_workspace_bytes(4, 7, 1024, 0)
    assert call(wsb=ctypes.c_size_t(part), W2f=ctypes.c_void_p(0x100008)) == -4    # W2f not 16-byte aligned
    assert call(wsb=ctypes.c_size_t(part)) == -5                                    # without it: too small


def test_draft_with_confidence_argument_errors(lib):
    """The draft's checks first, then the head's (those of dspark_confidence_head)."""
    f = ctypes.c_float
    ws = ctypes.c_size_t(1 << 30)

    def call(B=4, K=7, V=1024, r=16, T=1.0, U=FAKE, W1=FAKE, x0=FAKE, d=64, H=FAKE, ht=1, wh=FAKE, we=FAKE, b=0.0,
             c=FAKE, wsp=FAKE, wsb=ws):
        return lib.dspark_markov_draft_with_confidence(B, K, V, r, f(T), U, 1, W1, FAKE, NULL, x0, ctypes.c_uint64(1),
                                                       ctypes.c_uint64(0), FAKE, FAKE, FAKE, d, H, ht, wh, we, f(b),
                                                       NULL, c, NULL, wsp, wsb, NULL)
    assert call(K=17) == -2
    assert call(r=12) == -2
    assert call(T=-1.0) == -4
    assert call(U=NULL) == -1
    assert call(W1=NULL) == -1
    assert call(wsb=ctypes.c_size_t(16)) == -5
    assert call(d=0) == -2
    assert call(ht=5) == -3
    assert call(b=float("nan")) == -4
    assert call(H=NULL) == -1
    assert call(wh=NULL) == -1
    assert call(c=NULL) == -1
    assert call(we=NULL) == -1           # the Markov part needs w_e when r > 0
    # empty batch: a no-op that still checks shapes and scalars
    assert call(B=0, U=NULL, W1=NULL, x0=NULL, H=NULL, wh=NULL, we=NULL, c=NULL, wsp=NULL) == 0
    assert call(B=0, d=0, U=NULL, H=NULL) == -2


def test_prepare_w2_argument_errors(lib):
    V, r = 1000, 64
    need = lib.dspark_markov_w2_frag_bytes(V, r)
    assert need == 16 * 4 * 2 * 1024 == lib.dspark_markov_draft_workspace_bytes(4, 7, V, r) - \
        lib.dspark_markov_draft_workspace_bytes(4, 7, V, 0)
    assert lib.dspark_markov_w2_frag_bytes(V, 12) == 0
    assert lib.dspark_markov_prepare_w2(V, 12, FAKE, FAKE, need, NULL) == -2
    assert lib.dspark_markov_prepare_w2(V, r, NULL, FAKE, need, NULL) == -1
    assert lib.dspark_markov_prepare_w2(V, r, FAKE, NULL, need, NULL) == -1
    assert lib.dspark_markov_prepare_w2(V, r, FAKE, FAKE, need - 1, NULL) == -5
    assert lib.dspark_markov_prepare_w2(V, r, FAKE, ctypes.c_void_p(0x100008), need, NULL) == -4
    assert lib.dspark_markov_prepare_w2(V, 0, NULL, NULL, 0, NULL) == 0       # nothing to prepare
    need_h = lib.dspark_rnn_w2_f16_bytes(V, r)
    assert need_h == 16 * 32 * 1024
    assert lib.dspark_rnn_w2_f16_bytes(V, 48) == 0
    assert lib.dspark_rnn_prepare_w2(V, 48, FAKE, FAKE, need_h, NULL) == -2
    assert lib.dspark_rnn_prepare_w2(V, r, FAKE, NULL, need_h, NULL) == -1
    assert lib.dspark_rnn_prepare_w2(V, r, FAKE, FAKE, need_h - 1, NULL) == -5


def test_verify_argument_errors(lib):
    f = ctypes.c_float
    ws = ctypes.c_size_t(1 << 30)

    def call(R=4, K=7, V=1024, T=1.0, N=32, pdt=0, ddt=0, r=0, P=FAKE, q=FAKE, mm=NULL, wsp=FAKE, wsb=ws):
        return lib.dspark_verify(R, K, V, f(T), P, pdt, N, FAKE, FAKE, ddt, NULL, NULL, NULL, r, FAKE, FAKE, q, q,
                                 ctypes.c_uint64(1), ctypes.c_uint64(0), FAKE, FAKE, mm, wsp, wsb, NULL)
    assert call(N=3) == -2           # fewer rows than requests
    assert call(N=33) == -2          # more than R (K + 1)
    assert call(pdt=7) == -3
    assert call(T=-0.5) == -4
    assert call(P=NULL) == -1
    assert call(r=16) == -1          # Markov bias without factors
    assert call(wsb=ctypes.c_size_t(0)) == -5
    # the query covers recomputed draft normalisers and the margins; one byte less is refused
    full = lib.dspark_verify_workspace_bytes(4, 7, 1024, 0, 32)
    assert call(q=NULL, mm=FAKE, wsb=ctypes.c_size_t(full - 1)) == -5


def test_uniforms_argument_errors(lib):
    assert lib.dspark_uniforms(ctypes.c_uint64(1), ctypes.c_uint64(0), -1, 1, 0, FAKE, NULL) == -2
    assert lib.dspark_uniforms(ctypes.c_uint64(1), ctypes.c_uint64(0), 10, 1, 3, FAKE, NULL) == -4
    assert lib.dspark_uniforms(ctypes.c_uint64(1), ctypes.c_uint64(0), 10, 1, 0, NULL, NULL) == -1


def test_rnn_argument_errors(lib):
    B, K, V, r, d = 4, 7, 1024, 64, 128
    need = lib.dspark_rnn_draft_workspace_bytes(B, K, V, r, d)
    # the RNN head reuses the slice partials of the draft (the Markov head's W2 copy is not needed)
    assert need >= lib.dspark_markov_draft_workspace_bytes(B, K, V, 0) + B * K * 3 * r * 4 + 2 * B * r * 4 + V * r * 2
    assert lib.dspark_rnn_verify_workspace_bytes(4, K, V, r, 8) >= \
        lib.dspark_verify_workspace_bytes(4, K, V, r, 8) + V * r * 2
    # the RNN head's label adds the fp16 W2 copy (and no fragment-ordered copy)
    assert lib.dspark_rnn_acceptance_label_workspace_bytes(4, K, V, r) >= \
        lib.dspark_acceptance_label_workspace_bytes(4, K, V, 0) + V * r * 2
    assert need % 256 == 0

    def draft(B=B, K=K, V=V, r=r, d=d, T=1.0, U=FAKE, ud=1, H=FAKE, hd=1, W=FAKE, W1=FAKE, W2=FAKE, W2h=NULL,
              x0=FAKE, o=FAKE, ws=FAKE, wsb=WS):
        return lib.dspark_rnn_draft(B, K, V, r, d, T, U, ud, H, hd, W, W1, W2, W2h, x0, 1, 2, FAKE, FAKE, FAKE, o,
                                    ws, wsb, NULL)
    assert draft(r=48) == -2          # not a multiple of 32
    assert draft(r=0) == -2
    assert draft(r=288) == -2
    assert draft(d=100) == -2         # not a multiple of 64
    assert draft(d=0) == -2
    assert draft(K=17) == -2
    assert draft(hd=0) == -3          # f32 hidden states are not taken
    assert draft(ud=2) == -3
    assert draft(T=-1.0) == -4
    assert draft(H=NULL) == -1
    assert draft(W=NULL) == -1
    assert draft(o=NULL) == -1
    assert draft(wsb=ctypes.c_size_t(need - 1)) == -5
    assert draft(ws=ctypes.c_void_p(0x100010)) == -5     # not 256-byte aligned
    assert draft(W=ctypes.c_void_p(0x100008)) == -4      # not 16-byte aligned
    assert draft(W2h=ctypes.c_void_p(0x100008)) == -4    # the prepared copy too
    assert draft(W2h=FAKE, wsb=ctypes.c_size_t(need - lib.dspark_rnn_w2_f16_bytes(V, r) - 1)) == -5

    def verify(R=4, K=7, V=V, T=1.0, N=8, O=FAKE, W2=FAKE, r=r, q=FAKE, wsb=WS):
        return lib.dspark_rnn_verify(R, K, V, T, FAKE, 1, N, FAKE, FAKE, 1, O, W2, NULL, r, FAKE, FAKE, q, q, 1, 2,
                                     FAKE, FAKE, NULL, FAKE, wsb, NULL)
    assert verify(r=40) == -2
    assert verify(N=3) == -2
    assert verify(O=NULL) == -1
    assert verify(W2=NULL) == -1
    assert verify(q=NULL) == -1       # the RNN head's verification takes the draft's q_tok and lse_d
    assert verify(O=ctypes.c_void_p(0x100004)) == -4
    assert verify(wsb=ctypes.c_size_t(16)) == -5

    def label(B=4, K=7, V=V, T=1.0, O=FAKE, r=r, wsb=WS):
        return lib.dspark_rnn_acceptance_label(B, K, V, T, FAKE, 1, FAKE, 1, O, FAKE, NULL, r, FAKE, FAKE, FAKE,
                                               FAKE, FAKE, wsb, NULL)
    assert label(r=16) == -2
    assert label(O=NULL) == -1
    assert label(T=float("inf")) == -4
    assert label(wsb=ctypes.c_size_t(16)) == -5


def test_empty_batches_are_noops(lib):
    """No requests: every call returns DSPARK_OK without enqueuing anything
    and without reading its (NULL) array and workspace pointers; the shape and
    scalar checks still apply.  The schedule calls are the exception: with
    R = 0 they write the empty layout, so they still need those outputs."""
    f = ctypes.c_float
    u64 = ctypes.c_uint64
    Z = ctypes.c_size_t(0)
    assert lib.dspark_markov_draft(0, 7, 1024, 16, f(1.0), NULL, 1, NULL, NULL, NULL, NULL, u64(1), u64(0),
                                   NULL, NULL, NULL, NULL, Z, NULL) == 0
    assert lib.dspark_markov_draft(0, 7, 1024, 16, f(-1.0), NULL, 1, NULL, NULL, NULL, NULL, u64(1), u64(0),
                                   NULL, NULL, NULL, NULL, Z, NULL) == -4
    assert lib.dspark_markov_draft(0, 17, 1024, 16, f(1.0), NULL, 1, NULL, NULL, NULL, NULL, u64(1), u64(0),
                                   NULL, NULL, NULL, NULL, Z, NULL) == -2
    assert lib.dspark_rnn_draft(0, 7, 1024, 64, 128, f(1.0), NULL, 1, NULL, 1, NULL, NULL, NULL, NULL, NULL, u64(1),
                                u64(0), NULL, NULL, NULL, NULL, NULL, Z, NULL) == 0
    assert lib.dspark_verify(0, 7, 1024, f(1.0), NULL, 1, 0, NULL, NULL, 1, NULL, NULL, NULL, 16, NULL, NULL, NULL,
                             NULL, u64(1), u64(0), NULL, NULL, NULL, NULL, Z, NULL) == 0
    assert lib.dspark_verify(0, 7, 1024, f(1.0), NULL, 1, 1, NULL, NULL, 1, NULL, NULL, NULL, 16, NULL, NULL, NULL,
                             NULL, u64(1), u64(0), NULL, NULL, NULL, NULL, Z, NULL) == -2     # rows without requests
    assert lib.dspark_rnn_verify(0, 7, 1024, f(1.0), NULL, 1, 0, NULL, NULL, 1, NULL, NULL, NULL, 64, NULL, NULL,
                                 NULL, NULL, u64(1), u64(0), NULL, NULL, NULL, NULL, Z, NULL) == 0
    assert lib.dspark_acceptance_label(0, 7, 1024, f(1.0), NULL, 1, NULL, 1, NULL, NULL, NULL, 16, NULL, NULL, NULL,
                                       NULL, NULL, Z, NULL) == 0
    assert lib.dspark_rnn_acceptance_label(0, 7, 1024, f(1.0), NULL, 1, NULL, 1, NULL, NULL, NULL, 64, NULL, NULL,
                                           NULL, NULL, NULL, Z, NULL) == 0
    assert lib.dspark_confidence_head(0, 7, 100, 32, 8, NULL, 0, NULL, NULL, f(0.0), NULL, NULL, NULL, NULL, NULL,
                                      NULL, NULL) == 0
    assert lib.dspark_uniforms(u64(1), u64(0), 0, 1, 0, NULL, NULL) == 0
    # the schedule writes cu_seqlens[0], n_admitted and theta even for R = 0
    assert lib.dspark_schedule(0, 7, NULL, FAKE, 1, 0, 0, NULL, NULL, NULL, FAKE, FAKE, NULL, Z, NULL) == -1
    assert lib.dspark_schedule(0, 7, NULL, NULL, 1, 0, 0, NULL, NULL, FAKE, FAKE, FAKE, NULL, Z, NULL) == -1
    assert lib.dspark_schedule(0, 7, NULL, FAKE, 0, 0, 0, NULL, NULL, FAKE, FAKE, FAKE, NULL, Z, NULL) == -4
    assert lib.dspark_schedule_async(0, 7, NULL, FAKE, 1, NULL, NULL, NULL, FAKE, NULL, FAKE, NULL, Z, NULL) == -1
    for q in (lib.dspark_markov_draft_workspace_bytes(0, 7, 1024, 16), lib.dspark_schedule_workspace_bytes(0, 7),
              lib.dspark_verify_workspace_bytes(0, 7, 1024, 16, 0),
              lib.dspark_acceptance_label_workspace_bytes(0, 7, 1024, 16),
              lib.dspark_rnn_draft_workspace_bytes(0, 7, 1024, 64, 128)):
        assert q == 0


def test_profiler_without_launches(lib):
    """The kernel timer's host side: nothing recorded reads as no kernels."""
    assert lib.dspark_profiler_enable(1) == 0
    assert lib.dspark_profiler_reset() == 0
    assert lib.dspark_profiler_read(0, None, None, None) == 0
    assert lib.dspark_profiler_read(0, ctypes.byref(ctypes.c_char_p()), None, None) == -4
    assert lib.dspark_profiler_enable(0) == 0


def test_binding_exports_resolve(lib):
    """Every name the package exports resolves to a binding function or constant."""
    import draft_verify_schedule_amd as m
    for name in m.__all__:
        assert getattr(m, name) is not None, name
    for name in declared_functions():
        assert hasattr(m, name), name
