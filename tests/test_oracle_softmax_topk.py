"""Pins for the oracle's log-softmax and top-K (CPU only)."""
import os

import numpy as np
import pytest
import torch

from block_diffusion_draft_ddtree_amd import synth
from oracle import softmax_topk as st
from oracle import tree as ot

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_log_softmax_normalises_and_is_nonpositive():
    g = synth.rng("test", 0, 0)
    x = (3.0 * g.standard_normal((5, 777))).astype(np.float32)
    lp = st.log_softmax(x)
    assert np.all(lp <= 0.0)
    np.testing.assert_allclose(np.exp(lp).sum(axis=1), 1.0, atol=1e-12)


def test_log_softmax_closed_forms():
    # Uniform row: every entry is -log V.
    V = 1000
    lp = st.log_softmax(np.full((1, V), 1.25, dtype=np.float32))
    np.testing.assert_allclose(lp, -np.log(V), atol=1e-13)
    # Two entries: log-sigmoid of the difference.
    a, b = np.float32(0.75), np.float32(-2.5)
    lp = st.log_softmax(np.array([[a, b]], dtype=np.float32))
    d = float(b) - float(a)
    np.testing.assert_allclose(lp[0, 0], -np.log1p(np.exp(d)), atol=1e-15)
    np.testing.assert_allclose(lp[0, 1], d - np.log1p(np.exp(d)), atol=1e-15)
    # Shift invariance.
    g = synth.rng("test", 1, 0)
    x = g.standard_normal((3, 50)).astype(np.float32)
    np.testing.assert_allclose(st.log_softmax(x), st.log_softmax(x + np.float32(4.0)), atol=1e-12)


def test_log_softmax_matches_torch_fp64():
    g = synth.rng("test", 2, 0)
    x = (2.0 * g.standard_normal((4, 5000))).astype(np.float32)
    ref = torch.log_softmax(torch.from_numpy(x).double(), dim=1).numpy()
    np.testing.assert_allclose(st.log_softmax(x), ref, atol=1e-12)


def _topk_by_repeated_max(row, K):
    """Independent selection: K times, take the remaining entry that is
    largest, the smaller id winning exact ties."""
    left = list(range(len(row)))
    out = []
    for _ in range(K):
        best = left[0]
        for t in left[1:]:
            if row[t] > row[best] or (row[t] == row[best] and t < best):
                best = t
        out.append(best)
        left.remove(best)
    return out


@pytest.mark.parametrize("ties", [False, True])
def test_topk_matches_repeated_max(ties):
    g = synth.rng("test", 3, int(ties))
    if ties:
        x = synth.tie_logits(3, 60, g, levels=3)
    else:
        x = g.standard_normal((3, 60)).astype(np.float32)
    lp, tok = st.topk(x, 17)
    for i in range(3):
        assert list(tok[i]) == _topk_by_repeated_max(list(x[i]), 17)
    full = st.log_softmax(x)
    np.testing.assert_array_equal(lp, np.take_along_axis(full, tok.astype(np.int64), axis=1))


def test_topk_signed_zero_ties_by_id():
    x = np.array([[0.0, -0.0, 0.0, -1.0, -0.0]], dtype=np.float32)
    _, tok = st.topk(x, 5)
    assert list(tok[0]) == [0, 1, 2, 4, 3]


def test_topk_invariants_on_peaked_generator():
    w = synth.TINY
    lg = synth.drafter_logits(w)
    lp, tok = st.topk(lg.x, w.K)
    for i in range(w.L):
        assert len(set(tok[i].tolist())) == w.K
        assert np.all(np.diff(lp[i]) <= 0)
        chosen = set(tok[i].tolist())
        worst = min(float(lg.x[i, t]) for t in chosen)
        rest = np.delete(lg.x[i], tok[i])
        assert np.all(rest <= worst)
        assert lg.peak[i] in chosen  # the +6 boost lands in the top K at this seed


def _read_marginal_example():
    probs, discarded = {}, None
    with open(os.path.join(GOLDEN, "marginal_example.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split()
            if k == "discarded_by_greedy":
                discarded = float(v)
            else:
                probs[k] = float(v)
    return probs, discarded


def test_pages_marginal_example():
    """Deep-dive section 1 example: top-3 keeps 'the', 'a', 'an'; greedy keeps
    only 'the' and drops the 0.55 that the alternatives carry."""
    probs, discarded = _read_marginal_example()
    names = list(probs)
    # A toy vocabulary: the three named tokens plus 5 others sharing 0.05.
    p = np.array([probs[n] for n in names] + [0.01] * 5)
    x = np.log(p).astype(np.float32)[None, :]
    lp, tok = st.topk(x, 3)
    assert [names[t] for t in tok[0]] == ["the", "a", "an"]
    np.testing.assert_allclose(np.exp(lp[0]), [0.40, 0.35, 0.20], atol=1e-7)
    # Expected accepted length with one drafted position is the summed
    # probability of the tree's nodes; greedy (B=1) vs the 3-node tree:
    t1 = ot.build_tree(lp.astype(np.float32), tok, 1, root_token=-1)
    t3 = ot.build_tree(lp.astype(np.float32), tok, 3, root_token=-1)
    e1 = float(np.exp(t1.score[1:].astype(np.float64)).sum())
    e3 = float(np.exp(t3.score[1:].astype(np.float64)).sum())
    np.testing.assert_allclose(e3 - e1, discarded, atol=1e-6)
