"""Comparison rules between the HIP path and the CPU oracle.

* Integer results (tokens, accepted counts, lengths, layouts) must be equal.
  The one exception is a decision whose oracle margin is below MARGIN (the
  distance of the uniform from the CDF boundary or from the accept ratio, or
  the top-2 logit gap in greedy mode): such a mismatch is counted, the rest
  of that request's chain is excluded (its inputs differ from there on), and
  the counted fraction must stay below MAX_NEAR_TIE_FRACTION.
* Probabilities agree within 1e-5 absolute for float32 inputs and 2e-3
  relative for bfloat16 inputs.

The near-tie rate is asserted on a pooled count, not waived per test: every
parity test adds its decisions and counted near-ties to POOL, and the last
GPU test (tests/test_zy_pooled_near_ties.py) asserts the pooled fraction is
below MAX_NEAR_TIE_FRACTION.  A test with at least 1 / MAX_NEAR_TIE_FRACTION
decisions of its own must also meet the rate alone (no floor of one tie);
smaller tests are held to the rule through the pool only.
"""
import numpy as np

MARGIN = 1e-5
MAX_NEAR_TIE_FRACTION = 1e-4

# session totals over every parity test that called check_near_ties
POOL = {"tests": 0, "decisions": 0, "near_ties": 0, "excluded": 0, "with_ties": []}


class Report:
    def __init__(self, name):
        self.name = name
        self.decisions = 0
        self.near_ties = 0
        self.excluded = 0
        self.max_abs = {}
        self.max_rel = {}

    def err(self, key, gpu, ref):
        gpu = np.asarray(gpu, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        if gpu.size == 0:
            return
        d = np.abs(gpu - ref)
        self.max_abs[key] = max(self.max_abs.get(key, 0.0), float(d.max()))
        rel = d / np.maximum(np.abs(ref), 1e-30)
        self.max_rel[key] = max(self.max_rel.get(key, 0.0), float(rel.max()))

    def check_near_ties(self):
        POOL["tests"] += 1
        POOL["decisions"] += self.decisions
        POOL["near_ties"] += self.near_ties
        POOL["excluded"] += self.excluded
        if self.near_ties:
            POOL["with_ties"].append(str(self))
        if self.decisions * MAX_NEAR_TIE_FRACTION >= 1:
            assert self.near_ties < MAX_NEAR_TIE_FRACTION * self.decisions, str(self)

    def __str__(self):
        return ("%s: decisions=%d near_ties=%d excluded=%d max_abs=%s max_rel=%s"
                % (self.name, self.decisions, self.near_ties, self.excluded, self.max_abs, self.max_rel))


def compare_draft(rep, x_gpu, q_gpu, lse_gpu, ref, bf16_inputs, greedy):
    """Position-by-position draft comparison; returns a [B, K] mask of the
    positions whose inputs were identical on both sides."""
    x_gpu = np.asarray(x_gpu)
    B, K = x_gpu.shape
    same = np.zeros((B, K), dtype=bool)
    for b in range(B):
        for k in range(K):
            rep.decisions += 1
            if x_gpu[b, k] != ref["x"][b, k]:
                margin = ref["margin"][b, k]
                assert margin < MARGIN, ("draft token mismatch at request %d position %d: gpu %d oracle %d, "
                                         "oracle margin %.3g" % (b, k + 1, x_gpu[b, k], ref["x"][b, k], margin))
                rep.near_ties += 1
                rep.excluded += K - k - 1
                break
            same[b, k] = True
    q_gpu = np.asarray(q_gpu, dtype=np.float64)
    lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
    rep.err("q_tok", q_gpu[same], ref["q_tok"][same])
    rep.err("lse", lse_gpu[same], ref["lse"][same])
    if greedy:
        assert np.all(q_gpu[same] == 1.0)
    elif bf16_inputs:
        np.testing.assert_allclose(q_gpu[same], ref["q_tok"][same], rtol=2e-3, atol=0)
        np.testing.assert_allclose(lse_gpu[same], ref["lse"][same], rtol=2e-3, atol=0)
    else:
        np.testing.assert_allclose(q_gpu[same], ref["q_tok"][same], rtol=0, atol=1e-5)
        np.testing.assert_allclose(lse_gpu[same], ref["lse"][same], rtol=1e-5, atol=1e-5)
    return same


def compare_verify(rep, n_acc_gpu, tok_gpu, ref, requests=None):
    n_acc_gpu = np.asarray(n_acc_gpu)
    tok_gpu = np.asarray(tok_gpu)
    R = len(n_acc_gpu)
    rs = range(R) if requests is None else requests
    for r in rs:
        n_o = int(ref["n_acc"][r])
        rep.decisions += n_o + 1
        if n_acc_gpu[r] != n_o:
            j = min(int(n_acc_gpu[r]), n_o)          # first position whose decision differs (0-based)
            margin = ref["accept_margin"][r, j]
            assert margin < MARGIN, ("accept mismatch at request %d position %d: gpu n_acc %d oracle %d, "
                                     "oracle margin %.3g" % (r, j + 1, n_acc_gpu[r], n_o, margin))
            rep.near_ties += 1
            rep.excluded += 1
            continue
        if tok_gpu[r] != ref["tok"][r]:
            margin = ref["sample_margin"][r]
            assert margin < MARGIN, ("emitted token mismatch at request %d: gpu %d oracle %d (mode %d), "
                                     "oracle margin %.3g" % (r, tok_gpu[r], ref["tok"][r], ref["mode"][r], margin))
            rep.near_ties += 1


def oracle_min_margin(ref, r):
    """A request's smallest decision margin from the oracle's verification:
    the accept tests it made (NaN where a position was not examined) and the
    final draw's margin."""
    am = np.asarray(ref["accept_margin"][r], dtype=np.float64)
    vals = [float(ref["sample_margin"][r])] + [float(v) for v in am if not np.isnan(v)]
    return min(vals)


def compare_margins(gpu_margin, n_acc_gpu, ref, atol, rtol, requests=None):
    """min_margin_out against the oracle's margins, on the requests whose
    accepted count matches (the others already counted as near-ties)."""
    gpu_margin = np.asarray(gpu_margin, dtype=np.float64)
    rs = range(len(gpu_margin)) if requests is None else requests
    got, exp = [], []
    for r in rs:
        if int(n_acc_gpu[r]) != int(ref["n_acc"][r]):
            continue
        got.append(gpu_margin[r])
        exp.append(oracle_min_margin(ref, r))
    np.testing.assert_allclose(np.array(got), np.array(exp), rtol=rtol, atol=atol)
    return len(got)
