"""Robustness of the HIP path, beside parity: no kernel writes outside its
outputs, results repeat bit for bit, and a request's draft does not depend
on which row stage of the sweep it falls in.

* Canaries: every output and workspace lives in the middle of a buffer whose
  4 KB margins hold 0xA5; after the call the margins must be untouched
  (draft, draft with the confidence head, schedule with and without a
  workspace, verify from logits with margins, acceptance label, RNN draft
  and verify, prepared weights, uniforms).
* Determinism: the draft -> schedule -> verify -> label chain run twice on
  the same inputs gives the same bits.
* Batch split: the draft of B = 384 bf16 requests sweeps requests 0..255 as
  one 256-row stage and 256..383 as a 128-row stage; requests 0..127 run
  alone (one 128-row stage) and 128..383 run alone (one 256-row stage) must
  give the same greedy tokens, probabilities and normalisers, and the same
  first-position normalisers when sampling (later positions draw with the
  request index, which a split renumbers).
"""
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
CANARY = 0xA5
PAD = 4096


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


class Guarded:
    """A tensor (or raw workspace) between two canary margins."""

    def __init__(self, shape, dtype, label):
        nbytes = int(torch.Size(shape).numel()) * torch.empty((), dtype=dtype).element_size()
        self.label, self.n = label, nbytes
        room = (nbytes + 255) // 256 * 256
        self.raw = torch.full((PAD + room + PAD,), CANARY, dtype=torch.uint8, device=DEV)
        self.t = self.raw[PAD:PAD + nbytes].view(dtype).view(shape)

    def check(self):
        head = self.raw[:PAD]
        tail = self.raw[PAD + self.n:]
        bad_head = int((head != CANARY).sum())
        bad_tail = int((tail != CANARY).sum())
        assert bad_head == 0 and bad_tail == 0, "%s: %d bytes before and %d after the buffer were written" % (
            self.label, bad_head, bad_tail)


def ws(nbytes, label):
    return Guarded((max(int(nbytes), 256),), torch.uint8, label)


def bits(t):
    t = t.detach()
    if t.dtype in (torch.float32, torch.int32):
        return t.view(torch.int32).cpu()
    if t.dtype == torch.float64:
        return t.view(torch.int64).cpu()
    return t.cpu()


def _chain(w, step, lib, guarded=None):
    """draft -> schedule -> verify (margins, from logits too) -> label on workload w."""
    G = guarded if guarded is not None else []

    def g(shape, dtype, label):
        x = Guarded(shape, dtype, label)
        G.append(x)
        return x.t

    def gw(nbytes, label):
        x = ws(nbytes, label)
        G.append(x)
        return x.t

    B, K, V, r = w.B, w.K, w.V, w.r
    w2f = g((lib.dspark_markov_w2_frag_bytes(V, r),), torch.uint8, "W2f")
    ds().dspark_markov_prepare_w2(w.W2, out=w2f)
    x, q, lse = ds().dspark_markov_draft(
        w.U, w.W1, w.W2, w.x0, w.temperature, w.rng_seed, step,
        out=(g((B, K), torch.int32, "x"), g((B, K), torch.float32, "q"), g((B, K), torch.float32, "lse")),
        workspace=gw(lib.dspark_markov_draft_workspace_bytes(B, K, V, 0), "draft workspace"), w2f=w2f)
    # the same draft with the confidence head inside it (hidden width 264:
    # vector steps, the last one partial for some lanes)
    gen = torch.Generator().manual_seed(606)
    d = 264
    H = (torch.randn((B, K, d), generator=gen)).to(torch.bfloat16).to(DEV)
    w_h = (torch.randn(d, generator=gen) * 0.05).to(DEV)
    w_e = (torch.randn(r, generator=gen) * 0.5).to(DEV)
    xh, qh, lh, c, z = ds().dspark_markov_draft_with_confidence(
        w.U, w.W1, w.W2, w.x0, w.temperature, w.rng_seed, step, H, w_h, w_e, 0.1,
        out=(g((B, K), torch.int32, "x (with head)"), g((B, K), torch.float32, "q (with head)"),
             g((B, K), torch.float32, "lse (with head)"), g((B, K), torch.float32, "c")),
        workspace=gw(lib.dspark_markov_draft_workspace_bytes(B, K, V, 0), "draft workspace (with head)"), w2f=w2f,
        logits_out=g((B, K), torch.float32, "head logits"))
    sched_out = {"a": g((B, K), torch.float32, "a"), "ell": g((B,), torch.int32, "ell"),
                 "cu_seqlens": g((B + 1,), torch.int32, "cu"), "n_admitted": g((1,), torch.int32, "n"),
                 "theta": g((1,), torch.float64, "theta")}
    s = ds().dspark_schedule(w.c, w.sps, 0, out=sched_out,
                             workspace=gw(lib.dspark_schedule_workspace_bytes(B, K), "schedule workspace"))
    s2 = ds().dspark_schedule_noalloc(w.c, w.sps, 1, out={k: g(tuple(v.shape), v.dtype, "noalloc " + k)
                                                         for k, v in sched_out.items()})
    cu = s["cu_seqlens"]
    P = wl().flat_target_rows(w.t, cu)
    N = P.shape[0]
    vneed = lib.dspark_verify_workspace_bytes(B, K, V, r, N)
    n_acc, tok, mm = ds().dspark_verify(
        P, cu, w.U, w.W1, w.W2, w.x0, x, q, lse, w.temperature, w.rng_seed, step,
        out=(g((B,), torch.int32, "n_acc"), g((B,), torch.int32, "tok")), workspace=gw(vneed, "verify workspace"),
        w2f=w2f, min_margin=g((B,), torch.float32, "min_margin"))
    n_acc2, tok2, mm2 = ds().dspark_verify(
        P, cu, w.U, w.W1, w.W2, w.x0, x, None, None, w.temperature, w.rng_seed, step,
        out=(g((B,), torch.int32, "n_acc (from logits)"), g((B,), torch.int32, "tok (from logits)")),
        workspace=gw(vneed, "verify workspace (from logits)"), w2f=None,
        min_margin=g((B,), torch.float32, "min_margin (from logits)"))
    c_lab = ds().dspark_acceptance_label(
        w.t[:, :w.K].contiguous(), w.U, w.W1, w.W2, w.x0, x, lse, w.temperature,
        out=g((B, K), torch.float32, "label"),
        workspace=gw(lib.dspark_acceptance_label_workspace_bytes(B, K, V, 0), "label workspace"), w2f=w2f)
    u = ds().dspark_uniforms(w.rng_seed, step, 4099, 1, 0, out=g((4099,), torch.float32, "uniforms"))
    torch.cuda.synchronize()
    return {"x": x, "q": q, "lse": lse, "a": s["a"], "ell": s["ell"], "cu": cu, "n": s["n_admitted"],
            "theta": s["theta"], "ell_global": s2["ell"], "n_acc": n_acc, "tok": tok, "mm": mm, "n_acc2": n_acc2,
            "tok2": tok2, "mm2": mm2, "label": c_lab, "u": u, "x_head": xh, "q_head": qh, "lse_head": lh, "c": c,
            "z": z}


def test_canaries_markov_chain():
    import draft_verify_schedule_amd.binding as b
    lib = b.load_library()
    w = wl().make("full_step", device=DEV, B=300, V=4100)  # a stage pair, a partial stage, a ragged vocabulary
    guarded = []
    _chain(w, 0, lib, guarded)
    assert len(guarded) >= 20
    for x in guarded:
        x.check()


def test_canaries_rnn():
    B, K, V, r, d = 37, 3, 1000, 64, 128
    g = torch.Generator().manual_seed(4242)
    U = (torch.randn((B, K, V), generator=g) * 3).to(torch.bfloat16).to(DEV)
    H = (torch.randn((B, K, d), generator=g) * 0.5).to(torch.bfloat16).to(DEV)
    W = (torch.randn((3 * r, 2 * r + d), generator=g) * 0.1).to(torch.bfloat16).to(DEV)
    W1 = (torch.randn((V, r), generator=g) * 0.3).to(torch.bfloat16).to(DEV)
    W2 = (torch.randn((V, r), generator=g) * 0.3).to(torch.bfloat16).to(DEV)
    x0 = torch.randint(0, V, (B,), generator=g, dtype=torch.int32).to(DEV)
    import draft_verify_schedule_amd.binding as b
    lib = b.load_library()
    guarded = []

    def gg(shape, dtype, label):
        x = Guarded(shape, dtype, label)
        guarded.append(x)
        return x.t

    w2h = gg((lib.dspark_rnn_w2_f16_bytes(V, r),), torch.uint8, "W2h")
    ds().dspark_rnn_prepare_w2(W2, out=w2h)
    x, q, lse, O = ds().dspark_rnn_draft(
        U, H, W, W1, W2, x0, 1.0, 9, 0,
        out=(gg((B, K), torch.int32, "x"), gg((B, K), torch.float32, "q"), gg((B, K), torch.float32, "lse"),
             gg((B, K, r), torch.float32, "O")),
        workspace=gg((lib.dspark_rnn_draft_workspace_bytes(B, K, V, r, d),), torch.uint8, "rnn draft workspace"))
    cu = torch.arange(0, B * (K + 1) + 1, K + 1, dtype=torch.int32, device=DEV)
    P = (torch.randn((B * (K + 1), V), generator=g) * 3).to(torch.bfloat16).to(DEV)
    ds().dspark_rnn_verify(
        P, cu, U, O, W2, x0, x, q, lse, 1.0, 9, 0,
        out=(gg((B,), torch.int32, "n_acc"), gg((B,), torch.int32, "tok")),
        workspace=gg((lib.dspark_rnn_verify_workspace_bytes(B, K, V, r, B * (K + 1)),), torch.uint8,
                     "rnn verify workspace"), w2h=w2h, min_margin=gg((B,), torch.float32, "min_margin"))
    torch.cuda.synchronize()
    for x in guarded:
        x.check()


def test_repeat_bitwise():
    import draft_verify_schedule_amd.binding as b
    lib = b.load_library()
    w = wl().make("full_step", device=DEV, B=300, V=4100)
    first = _chain(w, 2, lib)
    again = _chain(w, 2, lib)
    for k in first:
        assert torch.equal(bits(first[k]), bits(again[k])), k


@pytest.mark.parametrize("T", [0.0, 1.0])
def test_draft_batch_split_bitwise(T):
    B, K, V, r = 384, 3, 4096, 256
    g = torch.Generator().manual_seed(31337)
    U = (torch.randn((B, K, V), generator=g) * 3).to(torch.bfloat16).to(DEV)
    W1 = (torch.randn((V, r), generator=g) * 0.3).to(torch.bfloat16).to(DEV)
    W2 = (torch.randn((V, r), generator=g) * 0.3).to(torch.bfloat16).to(DEV)
    x0 = torch.randint(0, V, (B,), generator=g, dtype=torch.int32).to(DEV)
    w2f = ds().dspark_markov_prepare_w2(W2)
    whole = ds().dspark_markov_draft(U, W1, W2, x0, T, 5, 0, w2f=w2f)
    head = ds().dspark_markov_draft(U[:128].contiguous(), W1, W2, x0[:128].contiguous(), T, 5, 0, w2f=w2f)
    tail = ds().dspark_markov_draft(U[128:].contiguous(), W1, W2, x0[128:].contiguous(), T, 5, 0, w2f=w2f)
    torch.cuda.synchronize()
    parts = [torch.cat([h, t]) for h, t in zip(head, tail)]
    if T == 0:
        for name, a, b_ in zip(("x", "q", "lse"), whole, parts):
            assert torch.equal(bits(a), bits(b_)), name
    else:
        assert torch.equal(bits(whole[2][:, 0].contiguous()), bits(parts[2][:, 0].contiguous()))
        # the first position's draw of the first 128 requests keeps its request index
        assert torch.equal(bits(whole[0][:128, 0].contiguous()), bits(parts[0][:128, 0].contiguous()))
