"""Pins for the oracle's cost-aware budget choice (CPU only).

Expected acceptance: "DDTree Deep Dive" page, section 2, Proposition 1,
checked here by walking every drafted sequence through the budget-B tree.
The budget optimum and its cost trade-off: the autobench Qwen3-Coder-30B
page's results table and notes."""
import itertools

import numpy as np
import pytest

from block_diffusion_draft_ddtree_amd import synth
from oracle import budget as ob
from oracle import commit as oc
from oracle import softmax_topk as st
from oracle import tree as ot


def test_hand_case():
    """q of the pops 0.6, 0.3, 0.1, 0.05; t0 = 1, t1 = 0.25:
    B = 0..4 gives 1/1.25, 1.6/1.5, 1.9/1.75, 2.0/2.0, 2.05/2.25, so B* = 2."""
    score = np.log(np.array([1.0, 0.6, 0.3, 0.1, 0.05]))
    ea = ob.expected_accept(score)
    np.testing.assert_allclose(ea, [0.0, 0.6, 0.9, 1.0, 1.05], rtol=1e-7)
    obj = ob.budget_objective(score, 1.0, 0.25)
    np.testing.assert_allclose(obj, [0.8, 1.6 / 1.5, 1.9 / 1.75, 1.0, 2.05 / 2.25], rtol=1e-7)
    assert ob.select_budget(score, 1.0, 0.25) == 2
    assert ob.select_budget(score, 1.0, 0.25, B_min=3) == 3
    assert ob.select_budget(score, 1.0, 0.25, B_max=1) == 1


def test_limits_of_the_cost_model():
    score = np.log(np.array([1.0, 0.5, 0.2, 0.2, 0.01, 1e-6]))
    # Free verification: every extra node adds expected tokens.
    assert ob.select_budget(score, 1.0, 0.0) == 5
    # Verification dominated by per-node cost: 1 / (B + 1) shape, smallest B.
    assert ob.select_budget(score, 0.0, 1.0, B_min=1) == 1
    # Equal objectives pick the smaller budget: two certain pops (q = 1)
    # with t0 = 0 give 2 / 2 == 3 / 3 exactly.
    tie = np.zeros(3, dtype=np.float32)
    obj = ob.budget_objective(tie, 0.0, 1.0)
    assert obj[1] == obj[2] == 1.0
    assert ob.select_budget(tie, 0.0, 1.0, B_min=1) == 1


@pytest.mark.parametrize("seed", range(3))
def test_expected_accept_is_proposition1_on_every_prefix(seed):
    """E[alpha](B) from the first B pops of one B_max build equals the
    expected accepted length of the budget-B tree under Q, by enumerating
    every drafted sequence; and the budget-B build is that prefix."""
    g = synth.rng("test", 30 + seed, 0)
    L, V = 3, 4 + seed
    q = g.dirichlet(np.ones(V) * 0.7, size=L)
    x = np.log(q).astype(np.float32)
    lp, tok = st.topk(x, V)
    lp32 = lp.astype(np.float32)
    B_max = 12
    big = ot.build_tree(lp32, tok, B_max, root_token=0)
    ea = ob.expected_accept(big.score)
    for B in (1, 4, 7, 12):
        t = ot.build_tree(lp32, tok, B, root_token=0)
        assert t.parent.tolist() == big.parent[: B + 1].tolist()
        assert t.token.tolist() == big.token[: B + 1].tolist()
        lhs = 0.0
        for Y in itertools.product(range(V), repeat=L):
            tgt = np.array([Y[d] if d < L else 0 for d in t.depth], dtype=np.int32)
            _, a, _ = oc.accept_walk(t.parent, t.token, tgt, L)
            lhs += float(np.prod([q[i, Y[i]] for i in range(L)])) * a
        assert abs(lhs - ea[B]) < 1e-6  # scores are fp32 sums of fp32 log-probs


def test_objective_against_brute_force_on_tables():
    g = synth.rng("test", 33, 0)
    for _ in range(20):
        B1 = int(g.integers(2, 60))
        score = np.concatenate([[0.0], -np.sort(g.exponential(2.0, size=B1))]).astype(np.float32)
        t0, t1 = float(g.uniform(0.1, 2)), float(g.uniform(0.0, 0.2))
        vals = []
        for B in range(0, B1 + 1):
            acc = 1.0 + sum(np.exp(np.float64(score[n])) for n in range(1, B + 1))
            vals.append(acc / (t0 + t1 * (B + 1)))
        want = int(np.argmax(vals[1:])) + 1
        assert ob.select_budget(score, t0, t1, B_min=1) == want


def test_rejects_bad_inputs():
    with pytest.raises(ValueError):
        ob.expected_accept(np.array([0.0, 0.5], dtype=np.float32))  # a probability above 1
    with pytest.raises(ValueError):
        ob.expected_accept(np.array([0.0, np.nan], dtype=np.float32))
    with pytest.raises(ValueError):
        ob.budget_objective(np.array([0.0, -1.0]), 0.0, 0.0)
    with pytest.raises(ValueError):
        ob.select_budget(np.array([0.0, -1.0]), 1.0, 0.1, B_min=2)
