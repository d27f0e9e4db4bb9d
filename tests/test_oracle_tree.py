"""Pins for the oracle's tree construction and mask (CPU only).

Propositions 1-3 and Lemma 1 are those of the "DDTree Deep Dive" page,
section 2; the mask rule is its section 4 and the alanhou.org summary's
Key Concepts; the figure fixture is that summary's Core Mechanism figure."""
import itertools
import os

import numpy as np
import pytest

from block_diffusion_draft_ddtree_amd import synth
from oracle import commit as oc
from oracle import softmax_topk as st
from oracle import tree as ot

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _check_tree_shape(t: ot.Tree, L, K, B):
    assert t.N == B + 1
    assert t.parent[0] == -1 and t.depth[0] == 0
    for n in range(1, t.N):
        p = t.parent[n]
        assert 0 <= p < n
        assert t.depth[n] == t.depth[p] + 1 <= L
        assert t.ranks[n][:-1] == t.ranks[p]  # prefix-closed (Prop. 2)
    keys = [ot.order_key(t.score[n], t.ranks[n]) for n in range(1, t.N)]
    assert keys == sorted(keys)  # listed in order
    assert len(set(t.ranks)) == t.N


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("ties", [False, True])
def test_three_selections_agree(seed, ties):
    """Brute force == sort-and-expand == best-first heap (Props. 2 and 3)."""
    g = synth.rng("test", 100 + seed, int(ties))
    L = int(g.integers(1, 5))
    K = int(g.integers(1, 5))
    lp, _ = synth.sorted_logp_table(L, K, 50, g, scale=float(g.uniform(0.2, 3)), ties=ties)
    total = ot.num_prefixes(L, K)
    for B in sorted({1, 2, max(1, total // 3), total}):
        bf = ot.top_b_brute_force(lp, B)
        assert ot.top_b_sort_expand(lp, B) == bf
        assert ot.top_b_best_first(lp, B) == bf


def test_tiny_workload_tree_is_valid_and_methods_agree():
    w = synth.TINY
    lg = synth.drafter_logits(w)
    lp, tok = st.topk(lg.x, w.K)
    lp32 = lp.astype(np.float32)
    t = ot.build_tree(lp32, tok, w.B, root_token=7)
    _check_tree_shape(t, w.L, w.K, w.B)
    assert ot.top_b_sort_expand(lp32, w.B) == t.ranks[1:]
    assert ot.top_b_best_first(lp32, w.B) == t.ranks[1:]
    for n in range(1, t.N):
        assert t.token[n] == tok[t.depth[n] - 1][t.ranks[n][-1]]
        assert t.score[n] == ot.prefix_score(lp32, t.ranks[n])


def test_deep_tree_methods_agree():
    g = synth.rng("test", 7, 0)
    x = synth.deep_logits(6, 40, g)
    lp, tok = st.topk(x, 5)
    lp32 = lp.astype(np.float32)
    for B in (10, 37, 120):
        bf = ot.top_b_brute_force(lp32, B)
        assert ot.top_b_sort_expand(lp32, B) == bf
        assert ot.top_b_best_first(lp32, B) == bf
        assert max(len(r) for r in bf) >= 3


def test_hand_derived_tie_orders():
    # All log-probs equal: ties at each depth go lexicographically.
    lp = np.full((2, 2), -1.0, dtype=np.float32)
    assert ot.top_b(lp, 6) == [(0,), (1,), (0, 0), (0, 1), (1, 0), (1, 1)]
    # A certain second position (log-prob 0): each child ties its parent and
    # follows it directly, being the parent's extension.
    lp = np.array([[-0.5, -1.0], [0.0, -2.0]], dtype=np.float32)
    assert ot.top_b(lp, 6) == [(0,), (0, 0), (1,), (1, 0), (0, 1), (1, 1)]
    t = ot.build_tree(lp, np.array([[10, 11], [20, 21]]), 4, root_token=5)
    assert t.parent.tolist() == [-1, 0, 1, 0, 3]
    assert t.token.tolist() == [5, 10, 20, 11, 20]


def test_special_cases():
    g = synth.rng("test", 8, 0)
    # K = 1: the single greedy trajectory (DFlash's argmax line).
    L = 5
    lp, tok = synth.sorted_logp_table(L, 1, 100, g)
    t = ot.build_tree(lp, tok, L, root_token=0)
    assert t.parent.tolist() == [-1] + list(range(L))
    assert t.token[1:].tolist() == tok[:, 0].tolist()
    # B = 1: one node, the argmax of the first position.
    lp, tok = synth.sorted_logp_table(4, 6, 100, g)
    t = ot.build_tree(lp, tok, 1, root_token=0)
    assert t.ranks[1:] == [(0,)] and t.token[1] == tok[0, 0]
    # B = every prefix: the complete K-ary tree of depth L.
    lp, tok = synth.sorted_logp_table(3, 2, 100, g)
    t = ot.build_tree(lp, tok, ot.num_prefixes(3, 2), root_token=0)
    assert sorted(t.ranks[1:]) == sorted(
        r for d in range(1, 4) for r in itertools.product(range(2), repeat=d))


def test_lemma1_topk_suffices():
    """Selecting over the whole vocabulary gives the same tree as selecting
    over the top K = min(B, |V|) tokens per position."""
    g = synth.rng("test", 9, 0)
    L, V, B = 3, 20, 8
    x = (1.5 * g.standard_normal((L, V))).astype(np.float32)
    lp_full, tok_full = st.topk(x, V)
    full = ot.build_tree(lp_full.astype(np.float32), tok_full, B, root_token=0)
    K = min(B, V)
    lp_k, tok_k = st.topk(x, K)
    small = ot.build_tree(lp_k.astype(np.float32), tok_k, B, root_token=0)
    assert full.parent.tolist() == small.parent.tolist()
    assert full.token.tolist() == small.token.tolist()
    np.testing.assert_array_equal(full.score, small.score)


def _marginals(g, L, V):
    return g.dirichlet(np.ones(V) * 0.7, size=L)


def _tree_value(q, ranks_tokens):
    """Sum over nodes of q(u) = prod_i q_i(u_i) (fp64)."""
    tot = 0.0
    for u in ranks_tokens:
        p = 1.0
        for i, t in enumerate(u):
            p *= q[i, t]
        tot += p
    return tot


def _node_token_paths(t: ot.Tree):
    paths = []
    for n in range(1, t.N):
        seq = []
        j = n
        while j != 0:
            seq.append(int(t.token[j]))
            j = int(t.parent[j])
        paths.append(tuple(reversed(seq)))
    return paths


@pytest.mark.parametrize("seed", range(3))
def test_proposition1_additivity_exhaustive(seed):
    """E_{Y~Q}[accepted length] == sum over tree nodes of q(u), by walking
    every Y in V^L through the tree with the oracle's accept walk."""
    g = synth.rng("test", 10 + seed, 0)
    L, V = 3 + seed % 2, 4 + seed
    q = _marginals(g, L, V)
    x = np.log(q).astype(np.float32)
    lp, tok = st.topk(x, V)
    for B in (1, 5, 11):
        t = ot.build_tree(lp.astype(np.float32), tok, B, root_token=0)
        lhs = 0.0
        for Y in itertools.product(range(V), repeat=L):
            tgt = np.array([Y[d] if d < L else 0 for d in t.depth], dtype=np.int32)
            _, a, _ = oc.accept_walk(t.parent, t.token, tgt, L)
            pY = float(np.prod([q[i, Y[i]] for i in range(L)]))
            lhs += pY * a
        rhs = _tree_value(q, _node_token_paths(t))
        assert abs(lhs - rhs) < 1e-12


def test_proposition2_optimal_among_prefix_closed_trees():
    """The selected B nodes maximise the summed q(u) over all prefix-closed
    node sets of size B (exhaustive over a 12-prefix trie)."""
    g = synth.rng("test", 20, 0)
    L, V = 2, 3
    q = _marginals(g, L, V)
    x = np.log(q).astype(np.float32)
    lp, tok = st.topk(x, V)
    prefixes = [p for d in (1, 2) for p in itertools.product(range(V), repeat=d)]
    for B in range(1, 7):
        best = 0.0
        for sub in itertools.combinations(prefixes, B):
            s = set(sub)
            if all(len(u) == 1 or u[:-1] in s for u in sub):
                best = max(best, _tree_value(q, sub))
        t = ot.build_tree(lp.astype(np.float32), tok, B, root_token=0)
        got = _tree_value(q, _node_token_paths(t))
        assert got == pytest.approx(best, rel=1e-6)


def test_mask_invariants():
    g = synth.rng("test", 21, 0)
    x = synth.deep_logits(5, 30, g)
    lp, tok = st.topk(x, 4)
    t = ot.build_tree(lp.astype(np.float32), tok, 70, root_token=0)
    W = t.anc.shape[1]
    assert W == (t.N + 31) // 32
    for n in range(t.N):
        bits = [j for j in range(32 * W) if (int(t.anc[n, j >> 5]) >> (j & 31)) & 1]
        assert len(bits) == t.depth[n] + 1
        assert max(bits) == n
        if n:
            p = t.parent[n]
            want = t.anc[p].copy()
            want[n >> 5] |= np.uint32(1 << (n & 31))
            np.testing.assert_array_equal(t.anc[n], want)
    wide = ot.ancestor_mask(t.parent, W + 2)
    np.testing.assert_array_equal(wide[:, :W], t.anc)
    assert not wide[:, W:].any()


def test_mask_matches_pages_figure():
    names, parent_of, visible, hidden = [], {}, {}, {}
    with open(os.path.join(GOLDEN, "ancestor_mask_figure.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("visible") or line.startswith("hidden"):
                kind, node, _, *rest = line.split()
                (visible if kind == "visible" else hidden)[node] = rest
                continue
            n, p = line.split()
            names.append(n)
            parent_of[n] = p
    idx = {n: i for i, n in enumerate(names)}
    parent = [-1 if parent_of[n] == "-" else idx[parent_of[n]] for n in names]
    anc = ot.ancestor_mask(parent)
    for node, vis in visible.items():
        row = anc[idx[node]]
        seen = {names[j] for j in range(len(names)) if (int(row[j >> 5]) >> (j & 31)) & 1}
        assert seen == set(vis)
        assert not seen & set(hidden[node])
