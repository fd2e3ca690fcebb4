"""GPU parity of the verify call's full contract, through the C ABI, against
the CPU oracle:

* verification from the logits alone (the draft's q_tok and lse_d not
  given: the draft rows' normalisers are recomputed in an extra pass, with
  the Markov bias when the draft had one), including the Qwen3-vocabulary
  verify-only workload (B=64, K=7, V=151936, bf16) on every request at
  T = 1 and T = 0;
* each request's smallest decision margin (min_margin_out) against the
  margins the oracle reports;
* the prepared fragment-ordered W2 copies (Markov head and RNN head): every
  call that takes one returns exactly what it returns without it.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.parity import Report, compare_margins, compare_verify

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


def _dev(t):
    return None if t is None else t.to(DEV)


def _verify_from_logits(w, T, cu, x, step=0, q=None, lse=None, w2f=None):
    """GPU verify with the margins output; q / lse None: recomputed."""
    cu_t = torch.as_tensor(cu, dtype=torch.int32)
    P = wl().flat_target_rows(w.t, cu_t)
    n_acc, tok, mm = ds().dspark_verify(P.to(DEV), cu_t.to(DEV), w.U.to(DEV), _dev(w.W1), _dev(w.W2),
                                        w.x0.to(DEV), torch.as_tensor(x, dtype=torch.int32).to(DEV),
                                        None if q is None else torch.as_tensor(q, dtype=torch.float32).to(DEV),
                                        None if lse is None else torch.as_tensor(lse, dtype=torch.float32).to(DEV),
                                        T, w.rng_seed, step, w2f=w2f, min_margin=True)
    torch.cuda.synchronize()
    ref = oracle.verify_ref(f64(P), np.asarray(cu), f64(w.U), None if w.W1 is None else f64(w.W1),
                            None if w.W2 is None else f64(w.W2).T, w.x0.numpy(), np.asarray(x), T, w.rng_seed, step)
    return n_acc.cpu().numpy(), tok.cpu().numpy(), mm.cpu().numpy(), ref


@pytest.mark.parametrize("T", [1.0, 0.0])
def test_qwen_verify_only_from_logits(T):
    """The verify-only Qwen3-vocabulary workload as specified: lse_d and
    q_tok not given, all K positions of all 64 requests verified."""
    w = wl().make("qwen_verify")
    _say("qwen verify-only from logits T=%g" % T)
    d = oracle.draft_ref(f64(w.U), None, None, w.x0.numpy(), T, w.rng_seed, 0)
    cu = np.arange(0, w.B * (w.K + 1) + 1, w.K + 1)
    n_acc, tok, mm, ref = _verify_from_logits(w, T, cu, d["x"])
    rep = Report("qwen verify-only T=%g" % T)
    compare_verify(rep, n_acc, tok, ref)
    rep.check_near_ties()
    if T == 0:
        n = compare_margins(mm, n_acc, ref, atol=1e-6, rtol=1e-6)
    else:
        n = compare_margins(mm, n_acc, ref, atol=2e-5, rtol=2e-3)
    _say(str(rep) + " margins compared on %d requests, mean n_acc %.3f" % (n, n_acc.mean()))


@pytest.mark.parametrize("name,T", [("tiny", 1.0), ("tiny", 0.7), ("tiny", 0.0), ("ds_stepped", 1.0)])
def test_verify_margins_and_recomputed_normalisers(name, T):
    """Scheduled prefixes (ragged rows): verify with the oracle's own q_tok and
    lse against verify from the logits alone; both against the oracle, with
    the margins (the ragged layout exercises the filtered pass over the
    judged draft rows only)."""
    w = wl().make(name)
    d = oracle.draft_ref(f64(w.U), None if w.W1 is None else f64(w.W1), None if w.W2 is None else f64(w.W2).T,
                         w.x0.numpy(), T, w.rng_seed, 0)
    s = oracle.schedule_ref(w.c.numpy(), w.sps.numpy(), 0)
    fp32 = w.U.dtype == torch.float32
    tol = dict(atol=1e-5, rtol=1e-4) if fp32 else dict(atol=2e-5, rtol=2e-3)
    if T == 0:
        tol = dict(atol=1e-6, rtol=1e-6)
    for given in (True, False):
        n_acc, tok, mm, ref = _verify_from_logits(w, T, s["cu_seqlens"], d["x"], step=3,
                                                  q=d["q_tok"] if given else None, lse=d["lse"] if given else None)
        rep = Report("verify %s T=%g normalisers %s" % (name, T, "given" if given else "recomputed"))
        compare_verify(rep, n_acc, tok, ref)
        rep.check_near_ties()
        n = compare_margins(mm, n_acc, ref, **tol)
        _say(str(rep) + " margins on %d requests" % n)


@pytest.mark.parametrize("B,K,V,r,dtype,T", [
    (4, 7, 1024, 16, torch.float32, 1.0),      # one partial stage of the fused bias pass
    (130, 3, 4096, 256, torch.bfloat16, 1.0),  # a full and a partial stage
    (37, 4, 1000, 24, torch.float32, 0.8),     # ragged vocabulary tail
])
def test_verify_markov_from_logits(B, K, V, r, dtype, T):
    """With a Markov head and no lse_d / q_tok, the draft rows' normalisers
    come from the draft's fused bias pass at every position; all requests
    verified at every position, against the oracle (which always rebuilds q
    from the factored inputs)."""
    g = torch.Generator().manual_seed(B * 7 + V)
    U = (torch.randn((B, K, V), generator=g) * 2.5).to(dtype)
    t = (0.8 * torch.cat([U.float(), torch.randn((B, 1, V), generator=g) * 2.5], dim=1)
         + 0.6 * torch.randn((B, K + 1, V), generator=g) * 2.5).to(dtype).contiguous()
    W1 = (torch.randn((V, r), generator=g) * 0.2).to(torch.bfloat16)
    W2 = (torch.randn((V, r), generator=g) * 0.2).to(torch.bfloat16)
    x0 = torch.randint(0, V, (B,), generator=g, dtype=torch.int32)
    d = oracle.draft_ref(f64(U), f64(W1), f64(W2).T, x0.numpy(), T, 55, 0)
    cu = np.arange(0, B * (K + 1) + 1, K + 1)
    cu_t = torch.as_tensor(cu, dtype=torch.int32)
    P = wl().flat_target_rows(t, cu_t)
    ref = oracle.verify_ref(f64(P), cu, f64(U), f64(W1), f64(W2).T, x0.numpy(), d["x"], T, 55, 0)
    x_t = torch.as_tensor(d["x"], dtype=torch.int32).to(DEV)
    w2f = ds().dspark_markov_prepare_w2(W2.to(DEV))
    for use_w2f in (False, True):
        n_acc, tok, mm = ds().dspark_verify(P.to(DEV), cu_t.to(DEV), U.to(DEV), W1.to(DEV), W2.to(DEV), x0.to(DEV),
                                            x_t, None, None, T, 55, 0, w2f=w2f if use_w2f else None,
                                            min_margin=True)
        torch.cuda.synchronize()
        n_acc, tok, mm = n_acc.cpu().numpy(), tok.cpu().numpy(), mm.cpu().numpy()
        rep = Report("markov verify from logits B=%d V=%d r=%d w2f=%s" % (B, V, r, use_w2f))
        compare_verify(rep, n_acc, tok, ref)
        rep.check_near_ties()
        fp32 = dtype == torch.float32
        compare_margins(mm, n_acc, ref, atol=(1e-5 if fp32 else 2e-5), rtol=(1e-4 if fp32 else 2e-3))
        _say(str(rep) + " mean n_acc %.3f" % n_acc.mean())


def test_verify_bad_tokens_margin_is_nan():
    w = wl().make("tiny")
    d = oracle.draft_ref(f64(w.U), f64(w.W1), f64(w.W2).T, w.x0.numpy(), 1.0, w.rng_seed, 0)
    x = d["x"].copy()
    x[1, 2] = -3
    cu = np.arange(0, w.B * (w.K + 1) + 1, w.K + 1)
    n_acc, tok, mm, _ = _verify_from_logits(w, 1.0, cu, x)
    assert n_acc[1] == -1 and tok[1] == -1 and np.isnan(mm[1])
    assert np.all(np.isfinite(mm[[0, 2, 3]])) and np.all(mm[[0, 2, 3]] >= 0)


def test_prepared_w2_full_step_identical():
    """The full-step workload (B=512, K=7, V=151936, r=256): draft, verify
    (with and without the draft's normalisers) and acceptance label with the
    prepared W2 copy return bit for bit what they return with the copy made
    inside each call."""
    w = wl().make("full_step", device=DEV)
    w2f = ds().dspark_markov_prepare_w2(w.W2)
    a = ds().dspark_markov_draft(w.U, w.W1, w.W2, w.x0, 1.0, w.rng_seed, 4)
    b = ds().dspark_markov_draft(w.U, w.W1, w.W2, w.x0, 1.0, w.rng_seed, 4, w2f=w2f)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)
    x, q, lse = a
    s = ds().dspark_schedule(w.c, w.sps, 0)
    cu = s["cu_seqlens"]
    P = wl().flat_target_rows(w.t, cu)
    ref = ds().dspark_verify(P, cu, w.U, w.W1, w.W2, w.x0, x, q, lse, 1.0, w.rng_seed, 4)
    for kw in (dict(w2f=w2f), dict(w2f=w2f, min_margin=True)):
        got = ds().dspark_verify(P, cu, w.U, w.W1, w.W2, w.x0, x, q, lse, 1.0, w.rng_seed, 4, **kw)
        assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1])
    Pk = w.t[:, :w.K].contiguous()
    la = ds().dspark_acceptance_label(Pk, w.U, w.W1, w.W2, w.x0, x, lse, 1.0)
    lb = ds().dspark_acceptance_label(Pk, w.U, w.W1, w.W2, w.x0, x, lse, 1.0, w2f=w2f)
    torch.cuda.synchronize()
    assert torch.equal(la, lb)
    # verification from the logits alone, with and without the copy: same decisions
    n1, t1 = ds().dspark_verify(P, cu, w.U, w.W1, w.W2, w.x0, x, None, None, 1.0, w.rng_seed, 4)
    n2, t2 = ds().dspark_verify(P, cu, w.U, w.W1, w.W2, w.x0, x, None, None, 1.0, w.rng_seed, 4, w2f=w2f)
    torch.cuda.synchronize()
    assert torch.equal(n1, n2) and torch.equal(t1, t2)
    agree = (n1 == ref[0]).float().mean().item()
    _say("full step: recomputed normalisers agree with the draft's on %.4f of requests" % agree)
    assert agree >= 0.99


def test_prepared_w2_rnn_identical():
    """The RNN head's draft, verification and label with its prepared fp16
    copy of W2 equal the calls that make the copy themselves."""
    B, K, V, r, d = 130, 3, 4096, 256, 256
    g = torch.Generator().manual_seed(909)
    U = (torch.randn((B, K, V), generator=g) * 3).to(torch.bfloat16).to(DEV)
    W1 = (torch.randn((V, r), generator=g) * 0.2).to(torch.bfloat16).to(DEV)
    W2 = (torch.randn((V, r), generator=g) * 0.2).to(torch.bfloat16).to(DEV)
    x0 = torch.randint(0, V, (B,), generator=g, dtype=torch.int32).to(DEV)
    H, W = wl().rnn_head(B, K, r, d, 910, device=DEV)
    w2h = ds().dspark_rnn_prepare_w2(W2)
    a = ds().dspark_rnn_draft(U, H, W, W1, W2, x0, 1.0, 3, 0)
    b = ds().dspark_rnn_draft(U, H, W, W1, W2, x0, 1.0, 3, 0, w2h=w2h)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)
    x, q, lse, O = a
    cu = torch.arange(0, B * (K + 1) + 1, K + 1, dtype=torch.int32, device=DEV)
    t = (torch.randn((B * (K + 1), V), generator=g) * 3).to(torch.bfloat16).to(DEV)
    va = ds().dspark_rnn_verify(t, cu, U, O, W2, x0, x, q, lse, 1.0, 3, 0)
    vb = ds().dspark_rnn_verify(t, cu, U, O, W2, x0, x, q, lse, 1.0, 3, 0, w2h=w2h)
    Pk = t.view(B, K + 1, V)[:, :K].contiguous()
    la = ds().dspark_rnn_acceptance_label(Pk, U, O, W2, x0, x, lse, 1.0)
    lb = ds().dspark_rnn_acceptance_label(Pk, U, O, W2, x0, x, lse, 1.0, w2h=w2h)
    torch.cuda.synchronize()
    assert torch.equal(va[0], vb[0]) and torch.equal(va[1], vb[1]) and torch.equal(la, lb)
