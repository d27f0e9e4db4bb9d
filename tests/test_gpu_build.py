"""GPU parity: ddtree_build against the oracle tree, bit for bit.

Both sides take the identical fp32 [L, K] table (either a synthetic sorted
table or the GPU top-K output downloaded), so parent, depth, token, score
(compared as bits) and the packed ancestor mask must be equal exactly."""
import numpy as np
import pytest
import torch

from block_diffusion_draft_ddtree_amd import binding as bd
from block_diffusion_draft_ddtree_amd import synth
from oracle import softmax_topk as st
from oracle import tree as ot

from gpu_helpers import down, say, up

pytestmark = pytest.mark.gpu

ROOT_TOKEN = 4242


def _gpu_tree(lp32, tok, B, W=None):
    L, K = lp32.shape
    say(f"build L={L} K={K} B={B} W={W}")
    root = up(np.array([ROOT_TOKEN], dtype=np.int32))
    out = bd.ddtree_build(up(lp32), up(tok.astype(np.int32)), B, root, mask_words=W)
    return [down(t) for t in out]


def _compare(lp32, tok, B, W=None, twice=False):
    lp32 = np.ascontiguousarray(lp32, dtype=np.float32)
    parent, depth, ntok, score, anc = _gpu_tree(lp32, tok, B, W)
    ref = ot.build_tree(lp32, tok, B, ROOT_TOKEN, mask_words=W)
    np.testing.assert_array_equal(parent, ref.parent)
    np.testing.assert_array_equal(depth, ref.depth)
    np.testing.assert_array_equal(ntok, ref.token)
    np.testing.assert_array_equal(score.view(np.uint32), ref.score.view(np.uint32))
    np.testing.assert_array_equal(anc.view(np.uint32), ref.anc)
    if twice:
        again = _gpu_tree(lp32, tok, B, W)
        for a, b in zip(again, (parent, depth, ntok, score, anc)):
            np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))
    return ref


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("ties", [False, True])
def test_random_tables(seed, ties):
    g = synth.rng("test", 600 + seed, int(ties))
    L = int(g.integers(1, 7))
    K = int(g.integers(1, 9))
    lp, tok = synth.sorted_logp_table(L, K, 1000, g, scale=float(g.uniform(0.1, 2.0)), ties=ties)
    total = ot.num_prefixes(L, K)
    for B in sorted({1, min(total, 7), min(total, 64), min(total, 300)}):
        _compare(lp, tok, B, twice=(B == 64))


def test_tiny_workload_from_gpu_topk():
    w = synth.TINY
    x = synth.drafter_logits(w).x
    say("tiny topk for build")
    lp, tok = bd.ddtree_topk(up(x), w.K)
    lp32, tok = down(lp), down(tok)
    _compare(lp32, tok, w.B, twice=True)


@pytest.mark.parametrize("name", ["qwen3_8b", "coder30b_b64", "coder30b_b256", "sweep_b512"])
def test_full_workloads_from_gpu_topk(name):
    w = synth.WORKLOADS[name]
    x = synth.drafter_logits(w).x
    say(f"{name} topk for build")
    lp, tok = bd.ddtree_topk(up(x), w.K)
    ref = _compare(down(lp), down(tok), w.B)
    assert ref.N == w.N


@pytest.mark.parametrize("B", [40, 200, 1024])
def test_deep_trees(B):
    g = synth.rng("test", 610, B)
    x = synth.deep_logits(16, 500, g)
    lp, tok = st.topk(x, 8)
    ref = _compare(lp.astype(np.float32), tok, B, twice=True)
    assert ref.depth.max() >= 5


@pytest.mark.parametrize("ties", [False, True])
@pytest.mark.parametrize("B", [63, 64, 130, 200, 290])
def test_wide_root_runs(ties, B):
    """A flat first position: the root's children pop in runs longer than a
    wave (63 ranks per step) until a first child or an exact tie interrupts
    them; the order must match the serial best-first pops bit for bit."""
    g = synth.rng("test", 640 + B, int(ties))
    L, K = 4, 300
    first = np.linspace(0.0, -3.0, K, dtype=np.float32)
    if ties:
        first = np.round(first * 8.0) / 8.0  # runs of equal log-probs
    lp = np.empty((L, K), dtype=np.float32)
    lp[0] = first
    for d in range(1, L):  # every step below the root costs at least 1.5
        lp[d] = np.float32(-1.5) - np.sort(np.abs(g.standard_normal(K)).astype(np.float32))
    lp[1, 0] = np.float32(-1.5)  # a first child ties a root child in the ties case
    tok = np.stack([g.choice(100000, size=K, replace=False) for _ in range(L)]).astype(np.int32)
    ref = _compare(lp, tok, B, twice=True)
    assert (ref.depth == 1).sum() >= min(B, 100)


def test_root_run_one_position():
    """L = 1: the whole tree is the root's first B children."""
    g = synth.rng("test", 650, 0)
    lp, tok = synth.sorted_logp_table(1, 200, 1000, g)
    ref = _compare(lp, tok, 150)
    assert ref.parent.tolist() == [-1] + [0] * 150


def test_special_cases():
    g = synth.rng("test", 620, 0)
    lp, tok = synth.sorted_logp_table(16, 1, 1000, g)
    ref = _compare(lp, tok, 16)               # K = 1: a chain of depth L
    assert ref.parent.tolist() == [-1] + list(range(16))
    lp, tok = synth.sorted_logp_table(3, 4, 1000, g)
    _compare(lp, tok, ot.num_prefixes(3, 4))  # complete tree
    _compare(lp, tok, 1)                      # one node
    _compare(lp, tok, 20, W=4)                # extra mask words stay zero


def test_certain_positions_child_ties_parent():
    """log-prob 0 at a position makes a child tie its parent exactly."""
    lp = np.array([[-0.5, -1.0, -1.0], [0.0, -2.0, -3.0], [0.0, 0.0, -1.0]], dtype=np.float32)
    tok = np.arange(9, dtype=np.int32).reshape(3, 3)
    _compare(lp, tok, 25, twice=True)


def test_max_table():
    g = synth.rng("test", 630, 0)
    lp, tok = synth.sorted_logp_table(32, 16, 100000, g, scale=0.3)
    _compare(lp, tok, 1024)
    lp, tok = synth.sorted_logp_table(16, 1024, 200000, g, scale=3.0)
    _compare(lp, tok, 64)


def test_table_at_the_lds_limit():
    """L * K = 32768 (L = 32, K = 1024), the largest table the build keeps in
    LDS (DDTREE_MAX_LK), with a narrow and a wide spread of log-probs (trees
    of depth 8 and 9 at budget 192; a larger budget makes the sort-based
    oracle take minutes)."""
    g = synth.rng("test", 631, 0)
    lp, tok = synth.sorted_logp_table(32, 1024, 200000, g, scale=0.05)
    ref = _compare(lp, tok, 192)
    assert ref.depth.max() >= 8
    lp, tok = synth.sorted_logp_table(32, 1024, 200000, g, scale=3.0)
    _compare(lp, tok, 192)


def _sweep_case(i: int):
    """Seeded table shape for case i: L in 1..32, K log-uniform in 1..128 with
    L K <= 32768, B log-uniform in 1..min(1024, prefixes); half the cases
    with heavy ties, the others normal at scale 0.05..3."""
    g = synth.rng("test", 610, i)
    L = int(g.integers(1, 33))
    K = max(1, min(128, 32768 // L, int(np.exp(g.uniform(0, np.log(129))))))
    total = ot.num_prefixes(L, K)
    B = max(1, min(1024, total, int(np.exp(g.uniform(0, np.log(1025))))))
    lp, tok = synth.sorted_logp_table(L, K, 151936, g, scale=float(g.uniform(0.05, 3.0)),
                                      ties=bool(i % 2))
    return lp, tok, B


@pytest.mark.parametrize("i", range(16))
def test_seeded_shape_sweep(i):
    """Against Proposition 3's best-first search (pinned against brute force
    in the oracle's tests), whose pop order is the sorted order of the set."""
    lp, tok, B = _sweep_case(i)
    parent, depth, ntok, score, anc = _gpu_tree(lp, tok, B)
    ref = ot.tree_from_prefixes(ot.top_b_best_first(lp, B), lp, tok, ROOT_TOKEN)
    np.testing.assert_array_equal(parent, ref.parent)
    np.testing.assert_array_equal(depth, ref.depth)
    np.testing.assert_array_equal(ntok, ref.token)
    np.testing.assert_array_equal(score.view(np.uint32), ref.score.view(np.uint32))
    np.testing.assert_array_equal(anc.view(np.uint32), ref.anc)
