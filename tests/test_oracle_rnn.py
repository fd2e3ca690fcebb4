"""Pins for the RNN-head drafter and the output-part bias in verification.

The recurrence is pinned by closed forms: with a zero gate matrix every gate
is one half, so the state is a geometric blend of the candidates; with
candidates that read only the hidden state (or only the previous token's
embedding) and an output part that reads only the state, the output of every
position is a known sum.  The gate's orientation is pinned by saturating it
both ways; the Markov head is the special case W_o = [0 | I | 0]; the
output-part bias in verification and in the acceptance label reduces to the
Markov bias when the rows are the Markov embeddings.
"""
import numpy as np

from oracle.draft import draft_ref
from oracle.label import acceptance_label_ref
from oracle.rnn import rnn_cell_ref, rnn_draft_ref
from oracle.verify import verify_ref


def _weights(rng, r, d, blocks):
    """W = [W_g; W_c; W_o], each r x (2r + d) and built from its three column
    blocks (state, embedding, hidden); blocks maps 'g', 'c', 'o' to a tuple of
    three matrices or None for zeros."""
    rows = []
    for name in ("g", "c", "o"):
        parts = blocks.get(name) or (None, None, None)
        cols = []
        for j, width in enumerate((r, r, d)):
            cols.append(np.zeros((r, width)) if parts[j] is None else parts[j])
        rows.append(np.concatenate(cols, axis=1))
    return np.concatenate(rows, axis=0)


def _problem(rng, B=5, K=6, V=40, r=4, d=7):
    U = rng.normal(size=(B, K, V))
    H = rng.normal(size=(B, K, d))
    W1 = rng.normal(size=(V, r))
    W2 = rng.normal(size=(r, V)) * 0.5
    x0 = rng.integers(0, V, size=B)
    return U, H, W1, W2, x0


def test_markov_head_is_the_special_case():
    """W_o = [0 | I | 0]: o_k = W1[x_{k-1}] and the draft is the Markov
    head's, token for token, whatever the gate and candidate parts are."""
    rng = np.random.default_rng(11)
    U, H, W1, W2, x0 = _problem(rng)
    r, d = W1.shape[1], H.shape[2]
    W = _weights(rng, r, d, {"g": (rng.normal(size=(r, r)), rng.normal(size=(r, r)), rng.normal(size=(r, d))),
                             "c": (rng.normal(size=(r, r)), None, rng.normal(size=(r, d))),
                             "o": (None, np.eye(r), None)})
    for T in (1.0, 0.6, 0.0):
        a = rnn_draft_ref(U, H, W, W1, W2, x0, T, seed=3, step=9)
        m = draft_ref(U, W1, W2, x0, T, seed=3, step=9)
        np.testing.assert_array_equal(a["x"], m["x"])
        np.testing.assert_allclose(a["q_tok"], m["q_tok"], rtol=1e-13, atol=0)
        np.testing.assert_allclose(a["lse"], m["lse"], rtol=1e-13, atol=1e-13)
        prev = np.concatenate([x0[:, None], m["x"][:, :-1]], axis=1)
        np.testing.assert_array_equal(a["O"], W1[prev])


def test_half_gates_blend_hidden_state_candidates():
    """W_g = 0 gives g = 1/2; candidates tanh(A h_k); W_o = [I | 0 | 0] gives
    o_k = s_{k-1}.  Then s_k = sum_{i<=k} 2^-(k-i+1) tanh(A h_i), s_0 = 0."""
    rng = np.random.default_rng(12)
    U, H, W1, W2, x0 = _problem(rng)
    B, K, _ = U.shape
    r, d = W1.shape[1], H.shape[2]
    A = rng.normal(size=(r, d))
    W = _weights(rng, r, d, {"c": (None, None, A), "o": (np.eye(r), None, None)})
    out = rnn_draft_ref(U, H, W, W1, W2, x0, 1.0, seed=1, step=2)
    cand = np.tanh(H @ A.T)                          # [B, K, r]
    s = np.zeros((B, r))
    for k in range(1, K + 1):
        np.testing.assert_allclose(out["O"][:, k - 1], s, rtol=0, atol=1e-14)
        expect = sum(2.0 ** -(k - i + 1) * cand[:, i - 1] for i in range(1, k + 1))
        np.testing.assert_allclose(out["S"][:, k - 1], expect, rtol=0, atol=1e-14)
        s = expect


def test_state_carries_tokens_two_back():
    """Candidates tanh(C W1[x_{k-1}]) with half gates and o_k = s_{k-1}: the
    bias of position 3 depends on the anchor and on x_1, which the Markov head
    cannot see.  Tokens are forced by base logits that dwarf the bias (greedy
    draw)."""
    rng = np.random.default_rng(13)
    B, K, V, r, d = 4, 5, 30, 3, 2
    forced = rng.integers(0, V, size=(B, K))
    U = np.zeros((B, K, V))
    np.put_along_axis(U, forced[:, :, None], 1e3, axis=2)
    H = rng.normal(size=(B, K, d))
    W1 = rng.normal(size=(V, r))
    W2 = rng.normal(size=(r, V))
    x0 = rng.integers(0, V, size=B)
    C = rng.normal(size=(r, r))
    W = _weights(rng, r, d, {"c": (None, C, None), "o": (np.eye(r), None, None)})
    out = rnn_draft_ref(U, H, W, W1, W2, x0, 0.0, seed=0, step=0)
    np.testing.assert_array_equal(out["x"], forced)
    prev = np.concatenate([x0[:, None], forced[:, :-1]], axis=1)
    cand = np.tanh(W1[prev] @ C.T)                   # c~_i from x_{i-1}
    for k in range(1, K + 1):
        s_prev = sum((2.0 ** -(k - 1 - i + 1) * cand[:, i - 1] for i in range(1, k)), np.zeros((B, r)))
        np.testing.assert_allclose(out["O"][:, k - 1], s_prev, rtol=0, atol=1e-14)
    # changing x_1 alone changes o_3 (through s_2) but not o_1 or o_2
    U2 = U.copy()
    alt = (forced[:, 0] + 1) % V
    U2[:, 0, :] = 0.0
    U2[np.arange(B), 0, alt] = 1e3
    out2 = rnn_draft_ref(U2, H, W, W1, W2, x0, 0.0, seed=0, step=0)
    np.testing.assert_array_equal(out2["O"][:, :2], out["O"][:, :2])
    assert np.all(np.abs(out2["O"][:, 2] - out["O"][:, 2]).max(axis=1) > 0)


def test_gate_orientation():
    """A gate saturated at 1 replaces the state by the candidate; at 0 it
    keeps the state (zero from s_0)."""
    rng = np.random.default_rng(14)
    n, r, d = 6, 3, 1
    s_prev = rng.normal(size=(n, r))
    e = rng.normal(size=(n, r))
    h = np.full((n, d), 1.0)
    Cs, Ce = rng.normal(size=(r, r)), rng.normal(size=(r, r))
    for big, expect_keep in ((80.0, False), (-80.0, True)):
        W = _weights(rng, r, d, {"g": (None, None, np.full((r, d), big)), "c": (Cs, Ce, None)})
        s, o = rnn_cell_ref(s_prev, e, h, W)
        cand = np.tanh(s_prev @ Cs.T + e @ Ce.T)
        np.testing.assert_allclose(s, s_prev if expect_keep else cand, rtol=0, atol=1e-30 + 1e-15)
        np.testing.assert_array_equal(o, np.zeros((n, r)))


def test_cell_against_scalar_loops():
    """The batched cell against a written-out per-element loop on a tiny case
    (sigmoid through exp, tanh through its exponential form)."""
    rng = np.random.default_rng(15)
    n, r, d = 2, 2, 3
    s_prev, e, h = rng.normal(size=(n, r)), rng.normal(size=(n, r)), rng.normal(size=(n, d))
    W = rng.normal(size=(3 * r, 2 * r + d))
    s, o = rnn_cell_ref(s_prev, e, h, W)
    for b in range(n):
        z = list(s_prev[b]) + list(e[b]) + list(h[b])
        for j in range(r):
            pg = sum(W[j, i] * z[i] for i in range(len(z)))
            pc = sum(W[r + j, i] * z[i] for i in range(len(z)))
            po = sum(W[2 * r + j, i] * z[i] for i in range(len(z)))
            g = 1.0 / (1.0 + np.exp(-pg))
            c = (np.exp(2 * pc) - 1.0) / (np.exp(2 * pc) + 1.0)
            assert abs(s[b, j] - ((1 - g) * s_prev[b, j] + g * c)) < 1e-14
            assert abs(o[b, j] - po) < 1e-13


def test_invalid_anchor_ends_the_chain():
    rng = np.random.default_rng(16)
    U, H, W1, W2, x0 = _problem(rng, B=3)
    r, d = W1.shape[1], H.shape[2]
    W = rng.normal(size=(3 * r, 2 * r + d)) * 0.3
    x0 = x0.copy()
    x0[1] = U.shape[2]
    out = rnn_draft_ref(U, H, W, W1, W2, x0, 1.0, seed=4, step=4)
    assert np.all(out["x"][1] == -1) and np.all(np.isnan(out["q_tok"][1]))
    assert np.all(out["x"][[0, 2]] >= 0)


def test_verify_and_label_with_output_rows_reduce_to_markov():
    """Passing O = W1[x_{j-1}] rows gives the Markov verification and label."""
    rng = np.random.default_rng(17)
    R, K, V, r = 6, 4, 50, 5
    D = rng.normal(size=(R, K, V))
    W1 = rng.normal(size=(V, r))
    W2 = rng.normal(size=(r, V)) * 0.5
    x0 = rng.integers(0, V, size=R)
    d = draft_ref(D, W1, W2, x0, 1.0, seed=8, step=1)
    x = d["x"]
    prev = np.concatenate([x0[:, None], x[:, :-1]], axis=1)
    O = W1[prev]
    ell = rng.integers(0, K + 1, size=R)
    cu = np.concatenate([[0], np.cumsum(ell + 1)])
    P = rng.normal(size=(cu[-1], V))
    for T in (1.0, 0.0):
        a = verify_ref(P, cu, D, W1, W2, x0, x, T, seed=8, step=1)
        b = verify_ref(P, cu, D, None, W2, x0, x, T, seed=8, step=1, O=O)
        np.testing.assert_array_equal(a["n_acc"], b["n_acc"])
        np.testing.assert_array_equal(a["tok"], b["tok"])
    Pl = rng.normal(size=(R, K, V))
    for T in (1.0, 0.5, 0.0):
        np.testing.assert_allclose(acceptance_label_ref(Pl, D, None, W2, x0, x, T, O=O),
                                   acceptance_label_ref(Pl, D, W1, W2, x0, x, T), rtol=0, atol=1e-14)
    # and a different O changes the label: the rows are used, not W1
    assert np.abs(acceptance_label_ref(Pl, D, None, W2, x0, x, 1.0, O=O + 1.0)
                  - acceptance_label_ref(Pl, D, W1, W2, x0, x, 1.0)).max() > 1e-3
