"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Every test feeds both sides the same seeded inputs from
draft_verify_schedule_amd.workloads (or an inline seeded generator for odd
shapes); the oracle never sees an output of the HIP path.  Comparison rules
are in tests/parity.py.
"""
import numpy as np
import pytest
import torch
from scipy import stats

import oracle
from tests.parity import Report, compare_draft, compare_margins, compare_verify

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import __graft_entry__
    __graft_entry__._ensure_built()
    import draft_verify_schedule_amd.binding as b
    b.load_library()


def ds():
    import draft_verify_schedule_amd as m
    return m


def wl():
    from draft_verify_schedule_amd import workloads
    return workloads


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def _say(msg):
    print(msg, flush=True)


# ------------------------------------------------------------------ uniforms
@pytest.mark.parametrize("seed,step,position,purpose", [(0x5EED0001, 0, 1, 0), (7, 3, 5, 1),
                                                        (2 ** 40 + 11, 2 ** 33 + 5, 8, 2)])
def test_uniforms_bit_exact(seed, step, position, purpose):
    n = 1 << 20
    u = ds().dspark_uniforms(seed, step, n, position, purpose)
    ref = oracle.uniform(seed, step, np.arange(n), position, purpose)
    np.testing.assert_array_equal(u.cpu().numpy().astype(np.float64), ref)


# --------------------------------------------------------------------- draft
def _run_draft(U, W1, W2, x0, T, seed, step=0):
    x, q, lse = ds().dspark_markov_draft(U.to(DEV), None if W1 is None else W1.to(DEV),
                                         None if W2 is None else W2.to(DEV), x0.to(DEV), T, seed, step)
    torch.cuda.synchronize()
    return x.cpu().numpy(), q.cpu().numpy(), lse.cpu().numpy()


def _oracle_draft(U, W1, W2, x0, T, seed, step=0, request_ids=None):
    return oracle.draft_ref(f64(U), None if W1 is None else f64(W1), None if W2 is None else f64(W2).T,
                            x0.cpu().numpy(), T, seed, step, request_ids)


def _random_draft_inputs(B, K, V, r, dtype, seed, scale=3.0, wscale=0.3):
    g = torch.Generator().manual_seed(seed)
    U = (torch.randn((B, K, V), generator=g) * scale).to(dtype)
    W1 = W2 = None
    if r:
        W1 = (torch.randn((V, r), generator=g) * wscale).to(torch.bfloat16)
        W2 = (torch.randn((V, r), generator=g) * wscale).to(torch.bfloat16)
    x0 = torch.randint(0, V, (B,), generator=g, dtype=torch.int32)
    return U, W1, W2, x0


@pytest.mark.parametrize("T", [1.0, 0.7, 0.0])
def test_draft_tiny_workload(T):
    w = wl().make("tiny")
    _say("draft tiny T=%g" % T)
    got = _run_draft(w.U, w.W1, w.W2, w.x0, T, w.rng_seed, 2)
    ref = _oracle_draft(w.U, w.W1, w.W2, w.x0, T, w.rng_seed, 2)
    rep = Report("draft tiny T=%g" % T)
    same = compare_draft(rep, *got, ref, bf16_inputs=False, greedy=(T == 0))
    rep.check_near_ties()
    assert same.sum() >= 0.9 * same.size
    _say(str(rep))


@pytest.mark.parametrize("B,K,V,r,dtype,T", [
    (37, 3, 1000, 24, torch.float32, 1.0),     # ragged rows and vocab tail, vector path
    (5, 2, 1003, 8, torch.bfloat16, 1.0),      # V not a multiple of 8: scalar path
    (70, 2, 4096, 256, torch.bfloat16, 1.0),   # full rank, two row stages
    (3, 4, 64, 16, torch.float32, 0.9),        # a single slice
    (1, 1, 7, 0, torch.float32, 1.0),          # V smaller than a wave, no Markov head
    (17, 3, 2000, 64, torch.bfloat16, 0.0),    # greedy with bf16 ties
    (9, 2, 520, 0, torch.bfloat16, 0.0),       # greedy, no bias, ragged tail
    (2, 16, 300, 32, torch.float32, 1.0),      # the largest K
    (384, 2, 4096, 256, torch.bfloat16, 1.0),  # a 256-row stage pair and a leftover full 128-row stage
    (300, 2, 2048, 64, torch.bfloat16, 0.8),   # a 256-row stage pair and a partial stage
    (272, 3, 2048, 128, torch.bfloat16, 0.0),  # greedy over a 256-row stage pair
    (260, 2, 2056, 64, torch.bfloat16, 1.0),   # a 256-row stage pair with a column tail of 8
    (256, 2, 1000, 32, torch.bfloat16, 0.0),   # greedy, a 256-row stage pair with a column tail of 40
])
def test_draft_shapes(B, K, V, r, dtype, T):
    _say("draft shape B=%d K=%d V=%d r=%d %s T=%g" % (B, K, V, r, dtype, T))
    U, W1, W2, x0 = _random_draft_inputs(B, K, V, r, dtype, seed=B * 1000 + V)
    got = _run_draft(U, W1, W2, x0, T, 99, 1)
    ref = _oracle_draft(U, W1, W2, x0, T, 99, 1)
    rep = Report("draft shape")
    compare_draft(rep, *got, ref, bf16_inputs=(dtype == torch.bfloat16), greedy=(T == 0))
    rep.check_near_ties()
    _say(str(rep))


def test_draft_invalid_anchor_flags_request():
    U, W1, W2, x0 = _random_draft_inputs(4, 3, 256, 16, torch.float32, seed=5)
    x0[1] = 256
    x0[3] = -4
    x, q, lse = _run_draft(U, W1, W2, x0, 1.0, 3)
    assert np.all(x[[1, 3]] == -1) and np.all(np.isnan(q[[1, 3]]))
    assert np.all((x[[0, 2]] >= 0) & (x[[0, 2]] < 256))


# ------------------------------------------------------------------ schedule
def _sched_gpu(c, sps, mode, cap=0):
    out = ds().dspark_schedule(c.to(DEV), sps.to(DEV), mode, cap)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def _sched_compare(c, sps, mode, cap=0):
    got = _sched_gpu(c, sps, mode, cap)
    ref = oracle.schedule_ref(c.numpy(), sps.numpy(), mode, cap)
    np.testing.assert_array_equal(got["a"].view(np.uint32), ref["a"].view(np.uint32))
    np.testing.assert_array_equal(got["ell"], ref["ell"])
    np.testing.assert_array_equal(got["cu_seqlens"], ref["cu_seqlens"])
    assert int(got["n_admitted"][0]) == ref["n_admitted"]
    assert got["theta"].view(np.uint64)[0] == np.float64(ref["theta"]).view(np.uint64)
    return got, ref


@pytest.mark.parametrize("name", ["tiny", "ds_stepped", "sched_stress", "full_step"])
@pytest.mark.parametrize("mode", [0, 1, 2])
def test_schedule_workloads_bit_exact(name, mode):
    w = wl().make(name, device="cpu", V=64)      # V does not affect the schedule inputs
    cap = (w.B * w.K) // 3
    _say("schedule %s mode %d" % (name, mode))
    got, ref = _sched_compare(w.c, w.sps, mode, cap)
    _say("  n_admitted=%d theta=%.6f" % (ref["n_admitted"], ref["theta"]))


def test_schedule_random_bit_exact():
    rng = np.random.default_rng(77)
    for i in range(60):
        R = int(rng.integers(1, 600))
        K = int(rng.integers(1, 17))
        if R * K > 16384:
            R = 16384 // K
        c = rng.uniform(0, 1, size=(R, K)).astype(np.float32)
        c[rng.uniform(size=(R, K)) < 0.1] = 1.0
        c[rng.uniform(size=(R, K)) < 0.03] = 0.0
        n = R * (K + 1) + 1 + int(rng.integers(0, 5))
        kind = i % 3
        if kind == 0:
            sps = 1000.0 / (1.0 + np.arange(n) / rng.uniform(4, 400))
        elif kind == 1:
            sps = wl().sps_staircase(n, flat_until=max(64, int(R * rng.uniform(1, 5))))
        else:
            sps = rng.uniform(0.5, 2.0, size=n)
        mode = int(rng.integers(0, 3))
        _sched_compare(torch.from_numpy(c), torch.from_numpy(sps), mode, int(rng.integers(0, R * K + 2)))


def test_schedule_maximum_candidates():
    rng = np.random.default_rng(5)
    c = torch.from_numpy(rng.uniform(0.3, 1, size=(1024, 16)).astype(np.float32))
    sps = torch.from_numpy(wl().sps_staircase(1024 * 17 + 1, flat_until=4096))
    for mode in (0, 1):
        _sched_compare(c, sps, mode)


@pytest.mark.parametrize("name", ["ds_stepped", "sched_stress", "full_step"])
def test_schedule_async_capacity_bit_exact(name):
    """Asynchronous capacity: GLOBAL on the confidences of an earlier block
    gives the capacity on the device; the async call admits the top-capacity
    candidates of the current block without the capacity leaving the GPU."""
    w = wl().make(name, device="cpu", V=64)
    rng = np.random.default_rng(91)
    c_old = w.c.numpy().copy()
    c_old = np.clip(c_old * rng.uniform(0.8, 1.2, size=c_old.shape), 0, 1).astype(np.float32)   # an older block
    sps = w.sps.to(DEV)
    old = ds().dspark_schedule(torch.from_numpy(c_old).to(DEV), sps, 1, 0)
    got = ds().dspark_schedule_async(w.c.to(DEV), sps, old["n_admitted"])
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in got.items()}
    ref = oracle.schedule_async_ref(w.c.numpy(), c_old, w.sps.numpy())
    _say("async %s capacity %d n_admitted %d" % (name, ref["capacity"], ref["n_admitted"]))
    assert int(old["n_admitted"].cpu()[0]) == ref["capacity"]
    np.testing.assert_array_equal(got["ell"], ref["ell"])
    np.testing.assert_array_equal(got["cu_seqlens"], ref["cu_seqlens"])
    assert int(got["n_admitted"][0]) == ref["n_admitted"]
    assert got["theta"].view(np.uint64)[0] == np.float64(ref["theta"]).view(np.uint64)


def test_schedule_async_capacity_edges():
    c = torch.from_numpy(np.random.default_rng(3).uniform(0.2, 1, size=(40, 5)).astype(np.float32))
    sps = torch.ones(40 * 6 + 1, dtype=torch.float64)
    for cap in (-1, 0, 1, 17, 200, 10 ** 6):
        got = ds().dspark_schedule_async(c.to(DEV), sps.to(DEV), torch.tensor([cap], dtype=torch.int32, device=DEV))
        torch.cuda.synchronize()
        ref = oracle.schedule_ref(c.numpy(), sps.numpy(), 2, max(cap, 0))
        assert int(got["n_admitted"].cpu()[0]) == ref["n_admitted"] == min(max(cap, 0), 200)
        np.testing.assert_array_equal(got["cu_seqlens"].cpu().numpy(), ref["cu_seqlens"])


def test_empty_batch_end_to_end():
    """A step with no requests: every call succeeds and returns empty outputs;
    the schedule overwrites its layout outputs with the empty layout the
    oracle gives (cu_seqlens = [0], nothing admitted, Theta = 0)."""
    _say("empty batch")
    K, V, r, d = 5, 300, 32, 64
    g = torch.Generator().manual_seed(11)
    W1 = (0.1 * torch.randn(V, r, generator=g)).to(torch.bfloat16).to(DEV)
    W2 = (0.1 * torch.randn(V, r, generator=g)).to(torch.bfloat16).to(DEV)
    W = (0.1 * torch.randn(3 * r, 2 * r + d, generator=g)).to(torch.bfloat16).to(DEV)
    U = torch.empty((0, K, V), dtype=torch.bfloat16, device=DEV)
    x0 = torch.empty(0, dtype=torch.int32, device=DEV)
    x, q, lse = ds().dspark_markov_draft(U, W1, W2, x0, 1.0, 5, 0)
    assert x.shape == q.shape == lse.shape == (0, K)
    H = torch.empty((0, K, d), dtype=torch.bfloat16, device=DEV)
    xr, qr, lr, O = ds().dspark_rnn_draft(U, H, W, W1, W2, x0, 1.0, 5, 0)
    assert xr.shape == (0, K) and O.shape == (0, K, r)
    c = torch.empty((0, K), dtype=torch.float32, device=DEV)
    sps = torch.tensor([4.0, 3.0], dtype=torch.float64, device=DEV)
    ref = oracle.schedule_ref(np.zeros((0, K), dtype=np.float32), np.array([4.0, 3.0]), 0)
    for call in ("sync", "async"):
        out = {"a": torch.empty((0, K), dtype=torch.float32, device=DEV),
               "ell": torch.empty(0, dtype=torch.int32, device=DEV),
               "cu_seqlens": torch.full((1,), 77, dtype=torch.int32, device=DEV),
               "n_admitted": torch.full((1,), 77, dtype=torch.int32, device=DEV),
               "theta": torch.full((1,), 77.0, dtype=torch.float64, device=DEV)}
        if call == "sync":
            ds().dspark_schedule(c, sps, 0, out=out)
        else:
            ds().dspark_schedule_async(c, sps, torch.tensor([3], dtype=torch.int32, device=DEV), out=out)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(out["cu_seqlens"].cpu().numpy(), ref["cu_seqlens"])
        assert int(out["n_admitted"].cpu()[0]) == ref["n_admitted"] == 0
        assert float(out["theta"].cpu()[0]) == ref["theta"] == 0.0
    P = torch.empty((0, V), dtype=torch.bfloat16, device=DEV)
    cu = torch.zeros(1, dtype=torch.int32, device=DEV)
    n_acc, tok = ds().dspark_verify(P, cu, U, W1, W2, x0, x, q, lse, 1.0, 5, 0)
    assert n_acc.shape == tok.shape == (0,)
    n_acc, tok = ds().dspark_rnn_verify(P, cu, U, O, W2, x0, xr, qr, lr, 1.0, 5, 0)
    assert n_acc.shape == (0,)
    P3 = torch.empty((0, K, V), dtype=torch.bfloat16, device=DEV)
    assert ds().dspark_acceptance_label(P3, U, W1, W2, x0, x, lse, 1.0).shape == (0, K)
    assert ds().dspark_rnn_acceptance_label(P3, U, O, W2, x0, xr, lr, 1.0).shape == (0, K)
    w_h = torch.zeros(d, dtype=torch.float32, device=DEV)
    w_e = torch.zeros(r, dtype=torch.float32, device=DEV)
    assert ds().dspark_confidence_head(H, w_h, w_e, 0.0, W1, x0, x, V).shape == (0, K)
    assert ds().dspark_uniforms(1, 0, 0, 1, 0).shape == (0,)
    torch.cuda.synchronize()


def test_schedule_invalid_confidence():
    c = torch.full((5, 3), 0.5)
    c[2, 1] = float("nan")
    got = _sched_gpu(c, torch.ones(64, dtype=torch.float64), 0)
    assert got["n_admitted"][0] == -1 and np.isnan(got["theta"][0])
    np.testing.assert_array_equal(got["cu_seqlens"], np.arange(6))


# -------------------------------------------------------------------- verify
def _verify_case(w, T, cu, x, q, lse, requests=None, step=0):
    """GPU verify on (w, cu, x, q, lse) against the oracle's verify."""
    P = wl().flat_target_rows(w.t, torch.as_tensor(cu, dtype=torch.int32))
    n_acc, tok = ds().dspark_verify(P.to(DEV), torch.as_tensor(cu, dtype=torch.int32).to(DEV), w.U.to(DEV),
                                    None if w.W1 is None else w.W1.to(DEV), None if w.W2 is None else w.W2.to(DEV),
                                    w.x0.to(DEV), torch.as_tensor(x, dtype=torch.int32).to(DEV),
                                    torch.as_tensor(q, dtype=torch.float32).to(DEV),
                                    torch.as_tensor(lse, dtype=torch.float32).to(DEV), T, w.rng_seed, step)
    torch.cuda.synchronize()
    ref = oracle.verify_ref(f64(P), np.asarray(cu), f64(w.U), None if w.W1 is None else f64(w.W1),
                            None if w.W2 is None else f64(w.W2).T, w.x0.numpy(), np.asarray(x), T, w.rng_seed, step)
    return n_acc.cpu().numpy(), tok.cpu().numpy(), ref


@pytest.mark.parametrize("name,T", [("tiny", 1.0), ("tiny", 0.0), ("qwen_verify", 1.0), ("qwen_verify", 0.0)])
def test_verify_all_positions(name, T):
    w = wl().make(name)
    _say("verify %s T=%g" % (name, T))
    d = oracle.draft_ref(f64(w.U), None if w.W1 is None else f64(w.W1), None if w.W2 is None else f64(w.W2).T,
                         w.x0.numpy(), T, w.rng_seed, 0)
    cu = np.arange(0, w.B * (w.K + 1) + 1, w.K + 1)
    n_acc, tok, ref = _verify_case(w, T, cu, d["x"], d["q_tok"], d["lse"])
    rep = Report("verify %s T=%g" % (name, T))
    compare_verify(rep, n_acc, tok, ref)
    rep.check_near_ties()
    _say(str(rep) + " mean n_acc %.3f" % n_acc.mean())


@pytest.mark.parametrize("name,T", [("ds_stepped", 1.0), ("sched_stress", 1.0),
                                    ("sched_stress", 0.0)])  # fp32 rows, greedy over full 2048-column waves
def test_verify_scheduled_prefixes(name, T):
    w = wl().make(name)
    _say("verify scheduled %s T=%g" % (name, T))
    s = oracle.schedule_ref(w.c.numpy(), w.sps.numpy(), 0)
    d = oracle.draft_ref(f64(w.U), None, None, w.x0.numpy(), T, w.rng_seed, 0)
    n_acc, tok, ref = _verify_case(w, T, s["cu_seqlens"], d["x"], d["q_tok"], d["lse"])
    rep = Report("verify %s T=%g" % (name, T))
    compare_verify(rep, n_acc, tok, ref)
    rep.check_near_ties()
    _say(str(rep) + " N=%d" % s["cu_seqlens"][-1])


def test_verify_many_corrections_two_stages():
    """More than 256 correcting requests with bf16 rows and a Markov head: the
    residual pass's 256-request stages run twice, the second one partial.
    Target rows independent of the draft make most requests reject early."""
    w = wl().make("full_step", B=320, V=4096)
    B, K, V = w.B, w.K, w.V
    d = oracle.draft_ref(f64(w.U), f64(w.W1), f64(w.W2).T, w.x0.numpy(), 1.0, w.rng_seed, 0)
    cu = np.arange(0, B * (K + 1) + 1, K + 1)
    g = torch.Generator().manual_seed(4321)
    P = (torch.randn((B * (K + 1), V), generator=g) * 3).to(torch.bfloat16)
    n_acc, tok = ds().dspark_verify(P.to(DEV), torch.as_tensor(cu, dtype=torch.int32).to(DEV), w.U.to(DEV),
                                    w.W1.to(DEV), w.W2.to(DEV), w.x0.to(DEV),
                                    torch.as_tensor(d["x"], dtype=torch.int32).to(DEV),
                                    torch.as_tensor(d["q_tok"], dtype=torch.float32).to(DEV),
                                    torch.as_tensor(d["lse"], dtype=torch.float32).to(DEV), 1.0, w.rng_seed, 0)
    torch.cuda.synchronize()
    n_acc, tok = n_acc.cpu().numpy(), tok.cpu().numpy()
    ref = oracle.verify_ref(f64(P), cu, f64(w.U), f64(w.W1), f64(w.W2).T, w.x0.numpy(), d["x"], 1.0, w.rng_seed, 0)
    rep = Report("verify, %d corrections" % int((ref["n_acc"] < K).sum()))
    compare_verify(rep, n_acc, tok, ref)
    rep.check_near_ties()
    _say(str(rep))
    assert int((ref["n_acc"] < K).sum()) > 256  # the case this test is for


def test_verify_edge_layouts():
    w = wl().make("tiny")
    d = oracle.draft_ref(f64(w.U), f64(w.W1), f64(w.W2).T, w.x0.numpy(), 1.0, w.rng_seed, 0)
    B, K = w.B, w.K
    for ell in (np.zeros(B, dtype=np.int64), np.full(B, K), np.array([0, K, 1, 3])):
        cu = np.concatenate([[0], np.cumsum(ell + 1)])
        n_acc, tok, ref = _verify_case(w, 1.0, cu, d["x"], d["q_tok"], d["lse"], step=4)
        rep = Report("edge")
        compare_verify(rep, n_acc, tok, ref)
        assert rep.near_ties == 0


def test_verify_bad_tokens_flag_request():
    w = wl().make("tiny")
    d = oracle.draft_ref(f64(w.U), f64(w.W1), f64(w.W2).T, w.x0.numpy(), 1.0, w.rng_seed, 0)
    x = d["x"].copy()
    x[2, 0] = w.V + 5
    cu = np.arange(0, w.B * (w.K + 1) + 1, w.K + 1)
    P = wl().flat_target_rows(w.t, torch.as_tensor(cu, dtype=torch.int32))
    n_acc, tok = ds().dspark_verify(P.to(DEV), torch.as_tensor(cu, dtype=torch.int32).to(DEV), w.U.to(DEV),
                                    w.W1.to(DEV), w.W2.to(DEV), w.x0.to(DEV), torch.as_tensor(x, dtype=torch.int32).to(DEV),
                                    torch.as_tensor(d["q_tok"], dtype=torch.float32).to(DEV),
                                    torch.as_tensor(d["lse"], dtype=torch.float32).to(DEV), 1.0, w.rng_seed, 0)
    torch.cuda.synchronize()
    assert n_acc[2].item() == -1 and tok[2].item() == -1
    assert all(n_acc[i].item() >= 0 for i in (0, 1, 3))


def test_verify_p_equals_q_accepts_all():
    """Target rows equal to the draft rows and no Markov head: every scheduled
    draft is accepted (a counted near-tie aside) and the bonus is emitted."""
    w = wl().make("qwen_verify", B=32)
    t = torch.cat([w.U, w.t[:, w.K:]], dim=1).contiguous()
    w.t = t
    x, q, lse = ds().dspark_markov_draft(w.U.to(DEV), None, None, w.x0.to(DEV), 1.0, w.rng_seed, 0)
    cu = np.arange(0, w.B * (w.K + 1) + 1, w.K + 1)
    P = wl().flat_target_rows(t, torch.as_tensor(cu, dtype=torch.int32))
    n_acc, tok = ds().dspark_verify(P.to(DEV), torch.as_tensor(cu, dtype=torch.int32).to(DEV), w.U.to(DEV), None,
                                    None, w.x0.to(DEV), x, q, lse, 1.0, w.rng_seed, 0)
    torch.cuda.synchronize()
    assert (n_acc.cpu().numpy() == w.K).mean() >= 1 - 1e-3


# ------------------------------------------------------------- whole step
def _gpu_step(w, step=0, mode=0, dev_inputs=None):
    U, W1, W2, x0, c, sps, t = dev_inputs or (w.U.to(DEV), w.W1.to(DEV), w.W2.to(DEV), w.x0.to(DEV), w.c.to(DEV),
                                              w.sps.to(DEV), w.t.to(DEV))
    x, q, lse = ds().dspark_markov_draft(U, W1, W2, x0, w.temperature, w.rng_seed, step)
    s = ds().dspark_schedule(c, sps, mode)
    cu = s["cu_seqlens"]
    P = wl().flat_target_rows(t, cu)
    n_acc, tok = ds().dspark_verify(P, cu, U, W1, W2, x0, x, q, lse, w.temperature, w.rng_seed, step)
    torch.cuda.synchronize()
    return {"x": x.cpu().numpy(), "q": q.cpu().numpy(), "lse": lse.cpu().numpy(),
            "cu": cu.cpu().numpy(), "ell": s["ell"].cpu().numpy(), "n_acc": n_acc.cpu().numpy(),
            "tok": tok.cpu().numpy()}


def test_full_step_tiny():
    w = wl().make("tiny")
    for step in range(3):
        g = _gpu_step(w, step)
        tf = f64(w.t)
        ref = oracle.run_step(f64(w.U), f64(w.W1), f64(w.W2).T, w.x0.numpy(), w.c.numpy(), w.sps.numpy(),
                              lambda r, n: tf[r, :n], 1.0, w.rng_seed, step)
        rep = Report("tiny step %d" % step)
        same = compare_draft(rep, g["x"], g["q"], g["lse"], ref["draft"], bf16_inputs=False, greedy=False)
        np.testing.assert_array_equal(g["cu"], ref["schedule"]["cu_seqlens"])
        whole = [r for r in range(w.B) if same[r].all()]
        compare_verify(rep, g["n_acc"], g["tok"], ref["verify"], whole)
        rep.check_near_ties()


def test_full_step_full_size():
    """The full-step workload at its real shape (B=512, K=7, V=151936,
    r=256, bf16), in the launch configuration the benchmark times: draft,
    schedule and verification of every request against the oracle, over
    three RNG steps."""
    w = wl().make("full_step", device=DEV)
    _say("full step generated")
    s = oracle.schedule_ref(w.c.cpu().numpy(), w.sps.cpu().numpy(), 0)
    W1f, W2f = f64(w.W1), f64(w.W2).T
    Uf = f64(w.U)
    x0 = w.x0.cpu().numpy()
    cu_t = torch.as_tensor(s["cu_seqlens"], dtype=torch.int32)
    P = f64(wl().flat_target_rows(w.t, cu_t.to(DEV)))
    rep = Report("full step, all requests, 3 steps")
    for step in range(3):
        g = _gpu_step(w, step=step, dev_inputs=(w.U, w.W1, w.W2, w.x0, w.c, w.sps, w.t))
        _say("full step %d gpu done: N=%d" % (step, g["cu"][-1]))
        np.testing.assert_array_equal(g["cu"], s["cu_seqlens"])
        np.testing.assert_array_equal(g["ell"], s["ell"])
        ref_d = oracle.draft_ref(Uf, W1f, W2f, x0, 1.0, w.rng_seed, step)
        same = compare_draft(rep, g["x"], g["q"], g["lse"], ref_d, bf16_inputs=True, greedy=False)
        ref_v = oracle.verify_ref(P, s["cu_seqlens"], Uf, W1f, W2f, x0, ref_d["x"], 1.0, w.rng_seed, step)
        whole = [r for r in range(w.B) if same[r].all()]
        compare_verify(rep, g["n_acc"], g["tok"], ref_v, whole)
        _say("  %s" % rep)
    rep.check_near_ties()
    assert rep.decisions >= 10 ** 4


def test_offsets_near_the_4gib_limit():
    """U, D and P just under 4 GiB, the limit of the kernels' 32-bit byte
    offsets: draft, verify (two positions, one draft row judged per request)
    and acceptance label of 7000 requests, the oracle on the first and last
    requests, where the offsets are smallest and largest."""
    B, K, V, r, seed = 7000, 2, 151936, 64, 0xB16
    assert B * K * V * 2 < 2 ** 32 and 2 * B * V * 2 < 2 ** 32
    g = torch.Generator(device=DEV).manual_seed(seed)
    U = torch.empty((B, K, V), dtype=torch.bfloat16, device=DEV)
    P = torch.empty((2 * B, V), dtype=torch.bfloat16, device=DEV)
    for i in range(0, B, 1000):
        U[i:i + 1000] = (2.0 * torch.randn((min(1000, B - i), K, V), generator=g, device=DEV)).to(torch.bfloat16)
        P[2 * i:2 * i + 2000] = (2.0 * torch.randn((min(2000, 2 * B - 2 * i), V), generator=g,
                                                   device=DEV)).to(torch.bfloat16)
    W1 = (0.2 * torch.randn((V, r), generator=g, device=DEV)).to(torch.bfloat16)
    W2 = (0.2 * torch.randn((V, r), generator=g, device=DEV)).to(torch.bfloat16)
    x0 = torch.randint(0, V, (B,), generator=g, device=DEV, dtype=torch.int32)
    _say("near-4GiB inputs generated")
    x, q, lse = ds().dspark_markov_draft(U, W1, W2, x0, 1.0, seed, 0)
    cu = torch.arange(0, 2 * B + 1, 2, dtype=torch.int32, device=DEV)
    n_acc, tok = ds().dspark_verify(P, cu, U, W1, W2, x0, x, q, lse, 1.0, seed, 0)
    torch.cuda.synchronize()
    _say("near-4GiB gpu done")
    sample = np.array([0, 1, 3333, B - 2, B - 1])
    sel = torch.as_tensor(sample, device=DEV)
    W1f, W2f = f64(W1), f64(W2).T
    Us = f64(U[sel])
    ref_d = oracle.draft_ref(Us, W1f, W2f, x0.cpu().numpy()[sample], 1.0, seed, 0, request_ids=sample)
    rep = Report("near 4 GiB")
    same = compare_draft(rep, x.cpu().numpy()[sample], q.cpu().numpy()[sample], lse.cpu().numpy()[sample], ref_d,
                         bf16_inputs=True, greedy=False)
    rows = torch.stack([2 * sel, 2 * sel + 1], 1).reshape(-1)
    Ps = f64(P[rows])
    cu_s = np.arange(0, 2 * len(sample) + 1, 2)
    ref_v = oracle.verify_ref(Ps, cu_s, Us, W1f, W2f, x0.cpu().numpy()[sample], ref_d["x"], 1.0, seed, 0,
                              request_ids=sample)
    whole = [i for i in range(len(sample)) if same[i].all()]
    compare_verify(rep, n_acc.cpu().numpy()[sample], tok.cpu().numpy()[sample], ref_v, whole)
    rep.check_near_ties()
    _say(str(rep))
    # the acceptance label over the same buffers, P read as [B, K, V]
    got, ref = _label_case(P.view(B, K, V), U, W1, W2, x0, 1.0, rows=sample, seed=seed)
    _say("near-4GiB label max |diff| %.2e" % np.abs(got - ref).max())
    np.testing.assert_allclose(got, ref, rtol=2e-3, atol=1e-6)


def test_kernel_timer_from_several_threads():
    """Draft calls from twelve host threads, each on its own stream (more
    streams than hardware queues), with the kernel timer on: every launch is
    counted once and every thread's draft equals the one-thread result."""
    import threading
    w = wl().make("tiny", device=DEV)
    ref = [t.cpu() for t in ds().dspark_markov_draft(w.U, w.W1, w.W2, w.x0, 1.0, w.rng_seed, 0)]
    torch.cuda.synchronize()
    ds().dspark_profiler_reset()
    ds().dspark_profiler_enable(True)
    n_threads = 12
    results, errors = [None] * n_threads, []

    def run(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(3):
                    out = ds().dspark_markov_draft(w.U, w.W1, w.W2, w.x0, 1.0, w.rng_seed, 0)
                s.synchronize()
            results[i] = [t.cpu() for t in out]
        except Exception as e:  # reported after the join
            errors.append(e)

    threads = [threading.Thread(target=run, args=(i,)) for i in range(n_threads)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    ds().dspark_profiler_enable(False)
    torch.cuda.synchronize()
    assert not errors, errors
    totals = ds().dspark_profiler_read()
    ds().dspark_profiler_reset()
    K = w.U.shape[1]
    assert totals["draft_locate"][0] == n_threads * 3 * K
    assert totals["draft_partials"][0] >= n_threads * 3 * K
    for res in results:
        for a, b in zip(res, ref):
            np.testing.assert_array_equal(a.numpy(), b.numpy())


# ------------------------------------------------------- statistics on GPU
def test_gpu_emitted_token_follows_target_and_acceptance_is_one_minus_tv():
    n, V = 1_000_000, 8
    lp = torch.tensor([1.5, -0.2, 0.3, 0.0, -1.1, 0.7, 0.2, -2.5])
    lq = torch.tensor([-0.4, 0.4, 0.9, 0.8, -0.2, 0.3, 1.6, -1.0])
    p = torch.softmax(lp.double(), 0).numpy()
    q = torch.softmax(lq.double(), 0).numpy()
    U = lq.expand(n, 1, V).contiguous().to(DEV)
    x0 = torch.zeros(n, dtype=torch.int32, device=DEV)
    x, qt, lse = ds().dspark_markov_draft(U, None, None, x0, 1.0, 4242, 0)
    P = lp.expand(2 * n, V).contiguous().to(DEV)
    cu = torch.arange(0, 2 * n + 1, 2, dtype=torch.int32, device=DEV)
    n_acc, tok = ds().dspark_verify(P, cu, U, None, None, x0, x, qt, lse, 1.0, 4242, 0)
    torch.cuda.synchronize()
    n_acc, tok, x = n_acc.cpu().numpy(), tok.cpu().numpy(), x.cpu().numpy()[:, 0]
    assert stats.chisquare(np.bincount(x, minlength=V), q * n).pvalue > 1e-6
    alpha = np.minimum(p, q).sum()
    assert abs((n_acc == 1).mean() - alpha) < 5 * np.sqrt(alpha * (1 - alpha) / n)
    first = np.where(n_acc >= 1, x, tok)
    assert stats.chisquare(np.bincount(first, minlength=V), p * n).pvalue > 1e-6

# ------------------------------------------------------- acceptance label
def _label_case(P, U, W1, W2, x0, T, rows=None, seed=7):
    """GPU label on the oracle's own draft (x, lse) of the checked requests
    (the other requests get token 0 and are not checked), against the
    oracle's label of those requests."""
    f64 = lambda t: None if t is None else t.detach().to("cpu", torch.float64).numpy()
    B, K, V = U.shape
    rows = np.arange(B) if rows is None else np.asarray(rows)
    sel = torch.as_tensor(rows)
    W1n, W2n = f64(W1), (None if W2 is None else f64(W2).T.copy())
    Us = f64(U[sel.to(U.device)])
    x0n = x0.cpu().numpy()
    d = oracle.draft_ref(Us, W1n, W2n, x0n[rows], T, seed, 0, request_ids=rows)
    x = torch.zeros((B, K), dtype=torch.int32)
    lse = torch.zeros((B, K), dtype=torch.float32)
    x[sel] = torch.as_tensor(d["x"], dtype=torch.int32)
    lse[sel] = torch.as_tensor(d["lse"], dtype=torch.float32)
    got = ds().dspark_acceptance_label(P.to(DEV), U.to(DEV), None if W1 is None else W1.to(DEV),
                                       None if W2 is None else W2.to(DEV), x0.to(DEV), x.to(DEV), lse.to(DEV), T)
    torch.cuda.synchronize()
    got = got.cpu().numpy()[rows]
    ref = oracle.acceptance_label_ref(f64(P[sel.to(P.device)]), Us, W1n, W2n, x0n[rows], d["x"], T)
    return got, ref


@pytest.mark.parametrize("T", [1.0, 0.7, 0.0])
def test_label_tiny(T):
    w = wl().make("tiny", device="cpu")
    P = w.t[:, :w.K].contiguous()
    got, ref = _label_case(P, w.U, w.W1, w.W2, w.x0, T)
    _say("label tiny T=%g max |diff| %.2e" % (T, np.abs(got - ref).max()))
    if T == 0:
        np.testing.assert_array_equal(got, ref)
    else:
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-5)


@pytest.mark.parametrize("T", [1.0, 0.0])
def test_label_qwen_vocab(T):
    w = wl().make("qwen_verify", device="cpu")
    P = w.t[:, :w.K].contiguous()
    got, ref = _label_case(P, w.U, None, None, w.x0, T, rows=np.arange(0, w.B, 4))
    _say("label qwen T=%g max |diff| %.2e" % (T, np.abs(got - ref).max()))
    if T == 0:
        np.testing.assert_array_equal(got, ref)
    else:
        np.testing.assert_allclose(got, ref, rtol=2e-3, atol=1e-6)


def test_label_ragged_unaligned():
    """V not a multiple of the vector width: the generic residual path."""
    g = torch.Generator().manual_seed(404)
    B, K, V, r = 3, 4, 999, 8
    P = torch.randn((B, K, V), generator=g) * 2
    U = P + torch.randn((B, K, V), generator=g)
    W1 = (torch.randn((V, r), generator=g) * 0.1).to(torch.bfloat16)
    W2 = (torch.randn((V, r), generator=g) * 0.1).to(torch.bfloat16)
    x0 = torch.randint(0, V, (B,), generator=g, dtype=torch.int32)
    got, ref = _label_case(P, U, W1, W2, x0, 1.0)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-5)


def test_label_bf16_odd_groups():
    """bf16 rows, 37 requests x 7 positions = 259 items: stages of 128, 128
    and 3 items, so the last stage has one 16-row group (an odd count: the
    next block's rows are not requested early there, its W2 still is) and
    every wave sweeps several 64-column blocks of the full vocabulary; the
    oracle checks requests 0, 18 and 36 (36 holds the last stage's items)."""
    g = torch.Generator().manual_seed(4242)
    B, K, V, r = 37, 7, 151936, 256
    P = (torch.randn((B, K, V), generator=g) * 2).to(torch.bfloat16)
    U = (P.float() + torch.randn((B, K, V), generator=g)).to(torch.bfloat16)
    W1 = (torch.randn((V, r), generator=g) * 0.05).to(torch.bfloat16)
    W2 = (torch.randn((V, r), generator=g) * 0.05).to(torch.bfloat16)
    x0 = torch.randint(0, V, (B,), generator=g, dtype=torch.int32)
    got, ref = _label_case(P, U, W1, W2, x0, 1.0, rows=np.array([0, 18, 36]))
    _say("label bf16 odd groups max |diff| %.2e" % np.abs(got - ref).max())
    np.testing.assert_allclose(got, ref, rtol=2e-3, atol=1e-6)


def test_label_full_step():
    """Full-size workload (B=512, K=7, V=151936, r=256, bf16), the launch the
    bench times: all 3584 positions against the oracle."""
    w = wl().make("full_step", device=DEV)
    P = w.t[:, :w.K].contiguous()
    got, ref = _label_case(P, w.U, w.W1, w.W2, w.x0, w.temperature)
    _say("label full_step (all %d positions) max |diff| %.2e" % (got.size, np.abs(got - ref).max()))
    np.testing.assert_allclose(got, ref, rtol=2e-3, atol=1e-6)


# ------------------------------------------- confidence head and STS
@pytest.mark.parametrize("h_dtype,d", [(torch.float32, 160), (torch.bfloat16, 160), (torch.bfloat16, 4096),
                                       (torch.bfloat16, 157)])
def test_confidence_head(h_dtype, d):
    """Against the oracle on a drafted block: the head reads the hidden state
    and the previous drafted token's Markov embedding (the anchor at k = 1)."""
    w = wl().make("tiny", device="cpu")
    g = torch.Generator().manual_seed(321)
    B, K, V, r = w.B, w.K, w.V, w.r
    H = (torch.randn((B, K, d), generator=g)).to(h_dtype)
    w_h = torch.randn(d, generator=g) * 0.1
    w_e = torch.randn(r, generator=g) * 2.0
    x = torch.randint(0, V, (B, K), generator=g, dtype=torch.int32)
    T = torch.tensor([0.5, 0.8, 1.0, 1.3, 2.0, 3.0, 0.7])[:K]
    c, z = ds().dspark_confidence_head(H.to(DEV), w_h.to(DEV), w_e.to(DEV), 0.25, w.W1.to(DEV), w.x0.to(DEV),
                                       x.to(DEV), V, sts_temperature=T.to(DEV), logits_out=True)
    torch.cuda.synchronize()
    f64 = lambda t: t.to(torch.float64).numpy()
    zr = oracle.confidence_logits_ref(f64(H), f64(w_h), f64(w_e), 0.25, f64(w.W1), w.x0.numpy(), x.numpy())
    cr = oracle.confidence_head_ref(f64(H), f64(w_h), f64(w_e), 0.25, f64(w.W1), w.x0.numpy(), x.numpy(),
                                    T.numpy())
    np.testing.assert_allclose(z.cpu().numpy(), zr, rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(c.cpu().numpy(), cr, rtol=0, atol=2e-6)


def test_confidence_head_bad_previous_token():
    B, K, V, d = 2, 3, 10, 8
    x = torch.tensor([[1, 2, 3], [4, 99, 5]], dtype=torch.int32)
    c = ds().dspark_confidence_head(torch.ones((B, K, d), device=DEV), torch.ones(d, device=DEV),
                                    torch.ones(8, device=DEV), 0.0,
                                    torch.zeros((V, 8), dtype=torch.bfloat16, device=DEV),
                                    torch.tensor([0, 1], dtype=torch.int32, device=DEV), x.to(DEV), V)
    c = c.cpu().numpy()
    assert np.isnan(c[1, 2]) and np.all(np.isfinite(np.delete(c.ravel(), 5)))


@pytest.mark.parametrize("name,T,h_dtype,d", [
    ("tiny", 1.0, torch.bfloat16, 160), ("tiny", 0.0, torch.bfloat16, 160), ("tiny", 1.0, torch.float32, 160),
    ("tiny", 1.0, torch.bfloat16, 157), ("tiny", 1.0, torch.bfloat16, 4104), ("tiny", 0.0, torch.float32, 157),
    ("full_step", 1.0, torch.bfloat16, 4096), ("full_step", 0.0, torch.bfloat16, 4096)])
def test_draft_with_confidence(name, T, h_dtype, d):
    """The draft with the confidence head evaluated inside it: x, q_tok and
    lse bit-equal to dspark_markov_draft's; c and the head's logits bit-equal
    to dspark_confidence_head's on the drafted tokens, and within the head's
    tolerance of the oracle.  Two requests have an invalid anchor (their
    confidences are NaN).  Hidden widths: vector steps (160, 4096), wider
    than the locate pass's prefetch (4104), and the element-wise path (157)."""
    _say("draft with confidence %s T=%g %s d=%d" % (name, T, h_dtype, d))
    w = wl().make(name, device=DEV)
    B, K, V, r = w.B, w.K, w.V, w.r
    g = torch.Generator().manual_seed(777 + d)
    H = torch.randn((B, K, d), generator=g).to(h_dtype).to(DEV)
    w_h = (torch.randn(d, generator=g) * 0.05).to(DEV)
    w_e = (torch.randn(r, generator=g) * 2.0).to(DEV)
    T_sts = torch.linspace(0.6, 1.8, K).to(DEV)
    x0 = w.x0.clone()
    x0[1] = -3
    x0[B - 1] = V
    x, q, lse, c, z = ds().dspark_markov_draft_with_confidence(
        w.U, w.W1, w.W2, x0, T, 11, 2, H, w_h, w_e, 0.25, sts_temperature=T_sts, logits_out=True)
    xs, qs, ls = ds().dspark_markov_draft(w.U, w.W1, w.W2, x0, T, 11, 2)
    cs, zs = ds().dspark_confidence_head(H, w_h, w_e, 0.25, w.W1, x0, xs, V, sts_temperature=T_sts,
                                         logits_out=True)
    torch.cuda.synchronize()
    bits = lambda t: t.cpu().view(torch.int32).numpy()
    np.testing.assert_array_equal(x.cpu().numpy(), xs.cpu().numpy())
    np.testing.assert_array_equal(bits(q), bits(qs))
    np.testing.assert_array_equal(bits(lse), bits(ls))
    np.testing.assert_array_equal(bits(c), bits(cs))
    np.testing.assert_array_equal(bits(z), bits(zs))
    c, z, xs = c.cpu().numpy(), z.cpu().numpy(), xs.cpu().numpy()
    assert np.all(np.isnan(c[[1, B - 1]])) and np.all(np.isnan(z[[1, B - 1]]))
    ok = np.setdiff1d(np.arange(B), [1, B - 1])
    zr = oracle.confidence_logits_ref(f64(H)[ok], f64(w_h), f64(w_e), 0.25, f64(w.W1), x0.cpu().numpy()[ok], xs[ok])
    cr = oracle.confidence_head_ref(f64(H)[ok], f64(w_h), f64(w_e), 0.25, f64(w.W1), x0.cpu().numpy()[ok], xs[ok],
                                    f64(T_sts))
    _say("  max |dz| %.2e, max |dc| %.2e" % (np.abs(z[ok] - zr).max(), np.abs(c[ok] - cr).max()))
    np.testing.assert_allclose(z[ok], zr, rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(c[ok], cr, rtol=0, atol=2e-6)


def test_draft_with_confidence_without_markov_head():
    """r = 0 (no W1, W2 or w_e): the head is w_h . h + bias alone; outputs
    bit-equal to the two separate calls, and the oracle's."""
    g = torch.Generator().manual_seed(909)
    B, K, V, d = 6, 4, 700, 96
    U = (torch.randn((B, K, V), generator=g) * 2).to(DEV)
    x0 = torch.randint(0, V, (B,), generator=g, dtype=torch.int32).to(DEV)
    H = torch.randn((B, K, d), generator=g).to(torch.bfloat16).to(DEV)
    w_h = (torch.randn(d, generator=g) * 0.1).to(DEV)
    x, q, lse, c = ds().dspark_markov_draft_with_confidence(U, None, None, x0, 1.0, 3, 0, H, w_h, None, -0.2)
    xs, qs, ls = ds().dspark_markov_draft(U, None, None, x0, 1.0, 3, 0)
    cs = ds().dspark_confidence_head(H, w_h, None, -0.2, None, x0, xs, V)
    torch.cuda.synchronize()
    for a, b in ((x, xs), (q, qs), (lse, ls), (c, cs)):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    cr = oracle.confidence_head_ref(f64(H), f64(w_h), None, -0.2, None, x0.cpu().numpy(), xs.cpu().numpy())
    np.testing.assert_allclose(c.cpu().numpy(), cr, rtol=0, atol=2e-6)


def _sts_data(seed, N, K, T_true):
    rng = np.random.default_rng(seed)
    logits = rng.normal(1.5, 2.0, size=(N, K)).astype(np.float32)
    p = 1.0 / (1.0 + np.exp(-logits.astype(np.float64) / T_true))
    alive = np.ones(N, dtype=bool)
    surv = np.zeros((N, K), dtype=np.uint8)
    for k in range(K):
        alive &= rng.uniform(size=N) < p[:, k]
        surv[:, k] = alive
    return logits, surv


@pytest.mark.parametrize("n_bins", [10, 15, 32])
def test_sts_fit_matches_oracle(n_bins):
    N, K = 20000, 5
    logits, surv = _sts_data(17 + n_bins, N, K, np.array([2.0, 1.5, 0.8, 1.2, 1.0]))
    grid = np.exp(np.linspace(np.log(0.25), np.log(4.0), 97)).astype(np.float32)
    T, ece = ds().dspark_sts_fit(torch.from_numpy(logits).to(DEV), torch.from_numpy(surv).to(DEV),
                                 torch.from_numpy(grid).to(DEV), n_bins)
    torch.cuda.synchronize()
    Tr, er = oracle.sts_fit_ref(logits, surv, grid.astype(np.float64), n_bins)
    _say("sts n_bins=%d T=%s ece=%s" % (n_bins, np.round(T.cpu().numpy(), 3), np.round(er, 4)))
    np.testing.assert_array_equal(T.cpu().numpy(), Tr.astype(np.float32))
    np.testing.assert_allclose(ece.cpu().numpy(), er, rtol=1e-5, atol=1e-7)


@pytest.mark.parametrize("N,K,G,n_bins,nan", [(300, 4, 33, 7, False), (1, 2, 5, 3, False),
                                               (9000, 7, 121, 15, False), (5000, 5, 61, 10, True)])
def test_sts_fit_small_ragged_and_repeatable(N, K, G, n_bins, nan):
    """Fewer samples than one chunk, a single sample, chunks with a ragged
    last one, and held-out logits with NaN (invalid tokens: no prediction from
    that position on): temperatures equal the oracle's, and a second call
    gives the same bits (every sum runs in a fixed order)."""
    logits, surv = _sts_data(5 + N, N, K, np.linspace(0.7, 2.0, K))
    if nan:
        rng = np.random.default_rng(N)
        logits[rng.integers(0, N, 200), rng.integers(0, K, 200)] = np.nan
    grid = np.exp(np.linspace(np.log(0.3), np.log(3.0), G)).astype(np.float32)
    args = (torch.from_numpy(logits).to(DEV), torch.from_numpy(surv).to(DEV), torch.from_numpy(grid).to(DEV), n_bins)
    T1, e1 = ds().dspark_sts_fit(*args)
    T2, e2 = ds().dspark_sts_fit(*args)
    torch.cuda.synchronize()
    Tr, er = oracle.sts_fit_ref(logits, surv, grid.astype(np.float64), n_bins)
    np.testing.assert_array_equal(T1.cpu().numpy(), Tr.astype(np.float32))
    np.testing.assert_allclose(e1.cpu().numpy(), er, rtol=1e-5, atol=1e-7)
    assert torch.equal(T1, T2) and torch.equal(e1.view(torch.int32), e2.view(torch.int32))



# ------------------------------------------------------------- RNN head
def _rnn_inputs(B, K, V, r, d, dtype, seed, scale=3.0, wscale=0.3):
    U, W1, W2, x0 = _random_draft_inputs(B, K, V, r, dtype, seed, scale, wscale)
    H, W = wl().rnn_head(B, K, r, d, seed + 1)
    return U, H, W, W1, W2, x0


def _oracle_rnn(U, H, W, W1, W2, x0, T, seed, step=0, request_ids=None):
    return oracle.rnn_draft_ref(f64(U), f64(H), f64(W), f64(W1), f64(W2).T, x0.cpu().numpy(), T, seed, step,
                                request_ids)


def _compare_rnn(rep, got, ref, bf16_inputs, greedy):
    x, q, lse, O = got
    same = compare_draft(rep, x, q, lse, ref, bf16_inputs=bf16_inputs, greedy=greedy)
    # o_k depends on the tokens before k: compare it where those agree
    ok = np.ones_like(same)
    ok[:, 1:] = same[:, :-1]
    rep.err("O", O[ok], ref["O"][ok])
    np.testing.assert_allclose(O[ok], ref["O"][ok], rtol=1e-4, atol=2e-5)
    return same


@pytest.mark.parametrize("B,K,V,r,d,dtype,T", [
    (4, 7, 1024, 32, 64, torch.float32, 1.0),      # the tiny workload's shape
    (37, 3, 1000, 64, 128, torch.float32, 0.8),    # ragged rows and vocabulary tail
    (5, 2, 1003, 32, 64, torch.bfloat16, 1.0),     # V not a multiple of 8: scalar path
    (130, 3, 4096, 256, 256, torch.bfloat16, 1.0), # full rank, a full and a partial row stage
    (17, 3, 2000, 96, 192, torch.bfloat16, 0.0),   # greedy, r below the padded eight chunks
    (1, 1, 7, 32, 64, torch.float32, 1.0),         # one request, one position, V below one slice
    (3, 16, 300, 64, 64, torch.float32, 0.5),      # the largest K: sixteen state updates
])
def test_rnn_draft_shapes(B, K, V, r, d, dtype, T):
    _say("rnn draft B=%d K=%d V=%d r=%d d=%d %s T=%g" % (B, K, V, r, d, dtype, T))
    U, H, W, W1, W2, x0 = _rnn_inputs(B, K, V, r, d, dtype, seed=B * 100 + r)
    out = ds().dspark_rnn_draft(U.to(DEV), H.to(DEV), W.to(DEV), W1.to(DEV), W2.to(DEV), x0.to(DEV), T, 77, 3)
    torch.cuda.synchronize()
    got = [t.cpu().numpy() for t in out]
    ref = _oracle_rnn(U, H, W, W1, W2, x0, T, 77, 3)
    rep = Report("rnn draft")
    same = _compare_rnn(rep, got, ref, bf16_inputs=(dtype == torch.bfloat16), greedy=(T == 0))
    rep.check_near_ties()
    assert same.sum() >= 0.9 * same.size
    _say(str(rep))


def test_rnn_draft_markov_special_case():
    """W_o = [0 | I | 0]: the RNN head's draft is the Markov head's, against
    the Markov oracle."""
    B, K, V, r, d = 9, 5, 2048, 64, 64
    U, H, W, W1, W2, x0 = _rnn_inputs(B, K, V, r, d, torch.bfloat16, seed=808)
    W = W.clone()
    W[2 * r:] = 0
    W[2 * r:, r:2 * r] = torch.eye(r, dtype=torch.bfloat16)
    x, q, lse, O = ds().dspark_rnn_draft(U.to(DEV), H.to(DEV), W.to(DEV), W1.to(DEV), W2.to(DEV), x0.to(DEV), 1.0,
                                         5, 1)
    torch.cuda.synchronize()
    ref = _oracle_draft(U, W1, W2, x0, 1.0, 5, 1)
    rep = Report("rnn as markov")
    same = compare_draft(rep, x.cpu().numpy(), q.cpu().numpy(), lse.cpu().numpy(), ref, bf16_inputs=True,
                         greedy=False)
    rep.check_near_ties()
    prev = np.concatenate([x0.numpy()[:, None], ref["x"][:, :-1]], axis=1)
    ok = np.ones_like(same)
    ok[:, 1:] = same[:, :-1]
    np.testing.assert_array_equal(O.cpu().numpy()[ok], f64(W1)[prev][ok])


def test_rnn_draft_invalid_anchor_flags_request():
    U, H, W, W1, W2, x0 = _rnn_inputs(4, 3, 256, 32, 64, torch.float32, seed=6)
    x0[2] = 256
    x, q, lse, O = ds().dspark_rnn_draft(U.to(DEV), H.to(DEV), W.to(DEV), W1.to(DEV), W2.to(DEV), x0.to(DEV), 1.0,
                                         3, 0)
    torch.cuda.synchronize()
    x, q = x.cpu().numpy(), q.cpu().numpy()
    assert np.all(x[2] == -1) and np.all(np.isnan(q[2]))
    ref = _oracle_rnn(U, H, W, W1, W2, x0, 1.0, 3, 0)
    np.testing.assert_array_equal(x, ref["x"])


def _rnn_verify_case(B, K, V, r, d, dtype, T, seed, all_rows=True):
    """The oracle's RNN draft (tokens, probabilities, output parts) verified on
    the GPU and by the oracle, the same fp32 output parts on both sides."""
    g = torch.Generator().manual_seed(seed)
    U, H, W, W1, W2, x0 = _rnn_inputs(B, K, V, r, d, dtype, seed)
    t = (0.8 * U.float() + 0.6 * torch.randn((B, K + 1, V), generator=g)[:, :K] * 3).to(dtype)
    t = torch.cat([t, (torch.randn((B, 1, V), generator=g) * 3).to(dtype)], dim=1).contiguous()
    d_ref = _oracle_rnn(U, H, W, W1, W2, x0, T, seed, 0)
    O32 = torch.as_tensor(d_ref["O"], dtype=torch.float32)
    if all_rows:
        cu = np.arange(0, B * (K + 1) + 1, K + 1)
    else:
        ell = np.random.default_rng(seed).integers(0, K + 1, size=B)
        cu = np.concatenate([[0], np.cumsum(ell + 1)])
    cu_t = torch.as_tensor(cu, dtype=torch.int32)
    P = wl().flat_target_rows(t, cu_t)
    n_acc, tok = ds().dspark_rnn_verify(P.to(DEV), cu_t.to(DEV), U.to(DEV), O32.to(DEV), W2.to(DEV), x0.to(DEV),
                                        torch.as_tensor(d_ref["x"], dtype=torch.int32).to(DEV),
                                        torch.as_tensor(d_ref["q_tok"], dtype=torch.float32).to(DEV),
                                        torch.as_tensor(d_ref["lse"], dtype=torch.float32).to(DEV), T, seed, 0)
    torch.cuda.synchronize()
    ref = oracle.verify_ref(f64(P), cu, f64(U), None, f64(W2).T, x0.numpy(), d_ref["x"], T, seed, 0,
                            O=O32.double().numpy())
    return n_acc.cpu().numpy(), tok.cpu().numpy(), ref


@pytest.mark.parametrize("B,K,V,r,d,dtype,T,all_rows", [
    (4, 7, 1024, 32, 64, torch.float32, 1.0, True),
    (4, 7, 1024, 32, 64, torch.float32, 0.0, True),
    (16, 7, 151936, 256, 256, torch.bfloat16, 1.0, True),   # aligned rows: the streaming residual pass
    (9, 4, 999, 64, 64, torch.float32, 1.0, False),         # unaligned rows: the generic residual pass
    (150, 3, 2048, 128, 128, torch.bfloat16, 0.7, False),   # two row stages of corrections
])
def test_rnn_verify(B, K, V, r, d, dtype, T, all_rows):
    _say("rnn verify B=%d K=%d V=%d r=%d %s T=%g" % (B, K, V, r, dtype, T))
    n_acc, tok, ref = _rnn_verify_case(B, K, V, r, d, dtype, T, seed=B + V, all_rows=all_rows)
    rep = Report("rnn verify")
    compare_verify(rep, n_acc, tok, ref)
    rep.check_near_ties()
    _say(str(rep) + " mean n_acc %.3f" % n_acc.mean())


@pytest.mark.parametrize("B,K,V,r,d,dtype,T", [
    (4, 7, 1024, 32, 64, torch.float32, 1.0),
    (4, 7, 1024, 32, 64, torch.float32, 0.0),
    (3, 4, 999, 64, 64, torch.float32, 0.8),                # generic residual pass
    (24, 7, 151936, 256, 256, torch.bfloat16, 1.0),         # streaming residual pass
])
def test_rnn_label(B, K, V, r, d, dtype, T):
    _say("rnn label B=%d V=%d T=%g" % (B, V, T))
    seed = 31 + V
    g = torch.Generator().manual_seed(seed)
    U, H, W, W1, W2, x0 = _rnn_inputs(B, K, V, r, d, dtype, seed)
    P = (0.8 * U.float() + 0.6 * torch.randn((B, K, V), generator=g) * 3).to(dtype).contiguous()
    d_ref = _oracle_rnn(U, H, W, W1, W2, x0, T, seed, 0)
    O32 = torch.as_tensor(d_ref["O"], dtype=torch.float32)
    got = ds().dspark_rnn_acceptance_label(P.to(DEV), U.to(DEV), O32.to(DEV), W2.to(DEV), x0.to(DEV),
                                           torch.as_tensor(d_ref["x"], dtype=torch.int32).to(DEV),
                                           torch.as_tensor(d_ref["lse"], dtype=torch.float32).to(DEV), T)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    ref = oracle.acceptance_label_ref(f64(P), f64(U), None, f64(W2).T, x0.numpy(), d_ref["x"], T,
                                      O=O32.double().numpy())
    _say("rnn label max |diff| %.2e" % np.abs(got - ref).max())
    if T == 0:
        np.testing.assert_array_equal(got, ref)
    elif dtype == torch.bfloat16:
        np.testing.assert_allclose(got, ref, rtol=2e-3, atol=1e-6)
    else:
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-5)


def test_rnn_draft_full_size():
    """The full-step workload with the RNN head (r = 256, d = 4096), the
    launch configuration the benchmark times: every request against the
    oracle."""
    w = wl().make("full_step", device=DEV)
    H, W = wl().rnn_head(w.B, w.K, w.r, 4096, 1005, device=DEV)
    _say("rnn full size generated")
    x, q, lse, O = ds().dspark_rnn_draft(w.U, H, W, w.W1, w.W2, w.x0, 1.0, w.rng_seed, 0)
    torch.cuda.synchronize()
    _say("rnn full size gpu done")
    ref = oracle.rnn_draft_ref(f64(w.U), f64(H), f64(W), f64(w.W1), f64(w.W2).T, w.x0.cpu().numpy(), 1.0,
                               w.rng_seed, 0)
    rep = Report("rnn full size")
    got = [t.cpu().numpy() for t in (x, q, lse, O)]
    _compare_rnn(rep, got, ref, bf16_inputs=True, greedy=False)
    rep.check_near_ties()
    _say(str(rep))


def test_verify_largest_k():
    """K = 16 (the ABI's limit): every position verified, and a ragged
    schedule; the decide kernel's fixed flag window covers all 17 rows."""
    g = torch.Generator().manual_seed(1616)
    B, K, V, r = 6, 16, 500, 16
    U = torch.randn((B, K, V), generator=g) * 2
    t = (0.9 * torch.cat([U, torch.randn((B, 1, V), generator=g) * 2], dim=1)
         + 0.4 * torch.randn((B, K + 1, V), generator=g)).contiguous()
    W1 = (torch.randn((V, r), generator=g) * 0.1).to(torch.bfloat16)
    W2 = (torch.randn((V, r), generator=g) * 0.1).to(torch.bfloat16)
    x0 = torch.randint(0, V, (B,), generator=g, dtype=torch.int32)
    d = oracle.draft_ref(f64(U), f64(W1), f64(W2).T, x0.numpy(), 1.0, 77, 0)
    for ell in (np.full(B, K), np.array([16, 0, 7, 15, 1, 16])):
        cu = np.concatenate([[0], np.cumsum(ell + 1)])
        cu_t = torch.as_tensor(cu, dtype=torch.int32)
        P = wl().flat_target_rows(t, cu_t)
        n_acc, tok = ds().dspark_verify(P.to(DEV), cu_t.to(DEV), U.to(DEV), W1.to(DEV), W2.to(DEV), x0.to(DEV),
                                        torch.as_tensor(d["x"], dtype=torch.int32).to(DEV),
                                        torch.as_tensor(d["q_tok"], dtype=torch.float32).to(DEV),
                                        torch.as_tensor(d["lse"], dtype=torch.float32).to(DEV), 1.0, 77, 0)
        torch.cuda.synchronize()
        ref = oracle.verify_ref(f64(P), cu, f64(U), f64(W1), f64(W2).T, x0.numpy(), d["x"], 1.0, 77, 0)
        rep = Report("verify K=16")
        compare_verify(rep, n_acc.cpu().numpy(), tok.cpu().numpy(), ref)
        rep.check_near_ties()
        _say(str(rep) + " n_acc %s" % n_acc.cpu().numpy().tolist())
