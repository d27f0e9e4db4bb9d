"""GPU parity: ddtree_accept_walk and ddtree_kv_compact, bit for bit."""
import numpy as np
import pytest
import torch

from block_diffusion_draft_ddtree_amd import binding as bd
from block_diffusion_draft_ddtree_amd import synth
from oracle import commit as oc
from oracle import softmax_topk as st
from oracle import tree as ot

from gpu_helpers import down, down_bf16_bits, say, up, up_bf16

pytestmark = pytest.mark.gpu


def _walk(tree, tgt, L):
    say(f"walk N={tree.N} L={L}")
    acc, n_acc, bonus = bd.ddtree_accept_walk(up(tree.parent), up(tree.token), L,
                                              up(tgt.astype(np.int32)))
    ref_acc, ref_a, ref_bonus = oc.accept_walk(tree.parent, tree.token, tgt, L)
    np.testing.assert_array_equal(down(acc), ref_acc)
    assert int(down(n_acc)[0]) == ref_a
    assert int(down(bonus)[0]) == ref_bonus
    return ref_a


def _deep_tree(seed, B, L=8, K=4):
    g = synth.rng("test", 800 + seed, 0)
    x = synth.deep_logits(L, 300, g)
    lp, tok = st.topk(x, K)
    return ot.build_tree(lp.astype(np.float32), tok, B, root_token=5), g


@pytest.mark.parametrize("seed", range(3))
def test_walk_planted_paths(seed):
    tree, g = _deep_tree(seed, 120)
    L = 8
    leaves = [n for n in range(tree.N) if n not in set(tree.parent.tolist())]
    for leaf in leaves[:12] + [0]:
        path = []
        j = leaf
        while j != -1:
            path.append(j)
            j = int(tree.parent[j])
        path.reverse()
        tgt = synth.target_argmax_planted(tree.parent, tree.token, path, 300, g)
        assert _walk(tree, tgt, L) == len(path) - 1


def test_walk_random_targets_and_full_depth():
    tree, g = _deep_tree(7, 1000, L=16, K=3)
    for _ in range(10):
        _walk(tree, synth.target_argmax_tiny(tree.parent, tree.token, 300, g), 16)
    # a chain accepted to depth L = 32
    L = 32
    parent = np.array([-1] + list(range(L)), dtype=np.int32)
    token = np.arange(100, 101 + L, dtype=np.int32)
    chain = ot.Tree(parent, np.arange(L + 1, dtype=np.int32), token,
                    np.zeros(L + 1, np.float32), ot.ancestor_mask(parent), [])
    tgt = np.concatenate([token[1:], [7]]).astype(np.int32)
    assert _walk(chain, tgt, L) == L


@pytest.mark.parametrize("name", ["coder30b_b64", "coder30b_b64_deep"])
def test_walk_coder30b_follow_peak(name):
    w = synth.WORKLOADS[name]
    lg = synth.drafter_logits(w)
    lp, tok = st.topk(lg.x, w.K)
    tree = ot.build_tree(lp.astype(np.float32), tok, w.B, 0)
    for r in range(5):
        g = synth.rng(w.family, r, synth.STREAM_TARGET)
        _walk(tree, synth.target_argmax_follow_peak(tree.depth, lg.peak, w.L, w.V, g), w.L)


def _compact(layers, Hkv, S, N, D, L, acc, seed):
    g = synth.rng("test", 850 + seed, 0)
    S_cap = S + N + 3
    kv = g.integers(0, 1 << 16, size=(layers, 2, Hkv, S_cap, D), dtype=np.uint16)
    a = len(acc) - 1
    acc_full = np.full(L + 1, -1, dtype=np.int32)
    acc_full[: a + 1] = acc
    say(f"compact layers={layers} Hkv={Hkv} S={S} N={N} D={D} a={a}")
    dev = up_bf16(kv)
    bd.ddtree_kv_compact(dev, S, N, L, up(acc_full), up(np.array([a], dtype=np.int32)))
    got = down_bf16_bits(dev)
    np.testing.assert_array_equal(got, oc.kv_compact(kv, S, acc_full, a))


@pytest.mark.parametrize("acc", [[0], [0, 1], [0, 2, 3], [0, 1, 2, 3, 4], [0, 5, 9, 11, 30],
                                 [0, 3, 4, 5, 6, 7, 8, 9, 10, 20, 21, 22, 23, 24, 25, 26, 27]])
def test_compact_patterns(acc):
    _compact(3, 2, 50, 33, 128, 16, acc, len(acc))


def test_compact_d64_and_max_depth():
    acc = [0] + list(range(2, 66, 2))  # a = 32 rows with gaps
    _compact(2, 3, 10, 70, 64, 32, acc, 99)


def test_compact_coder30b_cache():
    """The full 48-layer, 4-kv-head cache at S = 4096 (409 MB), whole buffer."""
    w = synth.CODER30B_B64
    g = synth.rng(w.family, 0, synth.STREAM_ACCEPT)
    acc = synth.accepted_path(w.B, w.L, g)
    _compact(w.layers, w.Hkv, w.S, w.N, w.D, w.L, acc, 100)
