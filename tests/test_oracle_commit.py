"""Pins for the oracle's target argmax, accept walk and KV compaction (CPU
only).

Argmax and walk: "DDTree Deep Dive" page, section 6 (the target's greedy
choice after each node; descend into the child matching it; the first
unmatched token becomes the bonus). Compaction: section 5 (keep only the
accepted path, gathered in place)."""
import numpy as np
import pytest

from block_diffusion_draft_ddtree_amd import synth
from oracle import commit as oc
from oracle import softmax_topk as st
from oracle import tree as ot


def _descend(parent, token, tgt, L):
    """Independent state machine: start at the root, repeatedly look for a
    child whose token equals the target's choice, stop when there is none."""
    children = {}
    for n in range(1, len(parent)):
        children.setdefault(int(parent[n]), []).append(n)
    cur, path = 0, [0]
    while True:
        nxt = [c for c in children.get(cur, []) if int(token[c]) == int(tgt[cur])]
        if not nxt:
            break
        cur = nxt[0]
        path.append(cur)
    return path, int(tgt[cur])


def _deep_tree(seed, B=60, L=6):
    g = synth.rng("test", 400 + seed, 0)
    x = synth.deep_logits(L, 50, g)
    lp, tok = st.topk(x, 4)
    return ot.build_tree(lp.astype(np.float32), tok, B, root_token=1), g


@pytest.mark.parametrize("seed", range(5))
def test_walk_matches_descent_and_planted_paths(seed):
    t, g = _deep_tree(seed)
    L = 6
    for leaf in range(t.N):
        path = []
        j = leaf
        while j != -1:
            path.append(j)
            j = int(t.parent[j])
        path.reverse()
        tgt = synth.target_argmax_planted(t.parent, t.token, path, 50, g)
        acc, a, bonus = oc.accept_walk(t.parent, t.token, tgt, L)
        assert a == len(path) - 1 == t.depth[leaf]
        assert acc[: a + 1].tolist() == path and np.all(acc[a + 1:] == -1)
        assert bonus == tgt[leaf]
        dp, db = _descend(t.parent, t.token, tgt, L)
        assert dp == path and db == bonus
    # random targets
    for _ in range(20):
        tgt = synth.target_argmax_tiny(t.parent, t.token, 50, g)
        acc, a, bonus = oc.accept_walk(t.parent, t.token, tgt, L)
        dp, db = _descend(t.parent, t.token, tgt, L)
        assert acc[: a + 1].tolist() == dp and bonus == db


def test_walk_all_off_tree_and_full_depth():
    t, g = _deep_tree(9)
    tgt = synth.target_argmax_planted(t.parent, t.token, [0], 50, g)
    acc, a, bonus = oc.accept_walk(t.parent, t.token, tgt, 6)
    assert a == 0 and acc[0] == 0 and bonus == tgt[0]
    # Chain of depth L: accepting every node reaches a = L.
    L = 5
    parent = np.array([-1, 0, 1, 2, 3, 4])
    token = np.array([9, 1, 2, 3, 4, 5])
    tgt = np.array([1, 2, 3, 4, 5, 77])
    acc, a, bonus = oc.accept_walk(parent, token, tgt, L)
    assert a == L and acc.tolist() == [0, 1, 2, 3, 4, 5] and bonus == 77


def test_compaction_patterns():
    g = synth.rng("test", 420, 0)
    layers, Hkv, D, S, N, L = 2, 3, 8, 10, 12, 6
    kv = g.integers(0, 65535, size=(layers, 2, Hkv, S + N, D)).astype(np.uint16)
    for acc in ([0, 2, 3], [0, 1, 2, 3], [0, 5, 9, 11], [0, 11], [0], [0, 1, 4, 5, 6, 10]):
        a = len(acc) - 1
        out = oc.kv_compact(kv, S, acc, a)
        # Rows up to S and from S + 1 + a on are untouched.
        np.testing.assert_array_equal(out[..., : S + 1, :], kv[..., : S + 1, :])
        np.testing.assert_array_equal(out[..., S + 1 + a:, :], kv[..., S + 1 + a:, :])
        # In-place sequential gather (increasing k) gives the same bytes:
        # acc is increasing with acc[k] >= k, so no source is overwritten
        # before it is read.
        inplace = kv.copy()
        for k in range(1, a + 1):
            inplace[..., S + k, :] = inplace[..., S + acc[k], :]
        np.testing.assert_array_equal(out, inplace)
        for k in range(1, a + 1):
            np.testing.assert_array_equal(out[..., S + k, :], kv[..., S + acc[k], :])


# ---------------------------------------------------------------------------
# target argmax
# ---------------------------------------------------------------------------

def test_argmax_hand_cases():
    ninf = -np.inf
    rows = [
        ([1.0, 3.0, 3.0, 2.0], 1),          # equal maxima: the smaller id
        ([ninf, ninf, ninf], 0),            # a fully masked row
        ([-0.0, 0.0, -1.0], 0),             # -0 and +0 are equal maxima
        ([0.0, -0.0, 1e-45], 2),            # a denormal beats both zeros
        ([-5.0, ninf, -4.0, -4.0], 2),
        ([7.0], 0),
    ]
    for vals, want in rows:
        got = oc.target_argmax(np.array([vals], dtype=np.float32))
        assert got.tolist() == [want], (vals, got)


def test_argmax_matches_sort_order():
    """Independent route: rank every token by (value desc, id asc) with a
    lexicographic sort and take the first; rows carry many exact ties."""
    g = synth.rng("test", 660, 0)
    x = np.round(g.standard_normal((40, 3001)).astype(np.float32) * 2.0) / 2.0
    x[5] = -np.inf
    x[6, 17] = np.inf
    got = oc.target_argmax(x)
    for n in range(x.shape[0]):
        order = np.lexsort((np.arange(x.shape[1]), -x[n].astype(np.float64)))
        assert got[n] == order[0]
        assert np.all(x[n, : got[n]] < x[n, got[n]])   # nothing earlier ties it
        assert np.all(x[n] <= x[n, got[n]])


def test_argmax_bf16_rows_widen_exactly():
    g = synth.rng("test", 661, 0)
    bits, vals = synth.normal_bf16(g, (8, 999))
    widened = (bits.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(widened, vals)
    assert np.array_equal(oc.target_argmax(vals), oc.target_argmax(widened))


def test_argmax_rejects_nan():
    with pytest.raises(ValueError):
        oc.target_argmax(np.array([[1.0, np.nan]], dtype=np.float32))
