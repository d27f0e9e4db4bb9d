"""Pins for the oracle's tree attention (CPU only).

The mask rule is that of the "DDTree Deep Dive" page, section 4: prefix,
root, ancestors and self. Reductions checked here: a chain-shaped tree is
plain causal attention; every root-to-leaf path is causal attention on that
path alone; a one-node tree is decode attention. The textbook side is
torch's scaled_dot_product_attention in fp64 on the CPU."""
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from block_diffusion_draft_ddtree_amd import synth
from oracle import attention as oa
from oracle import softmax_topk as st
from oracle import tree as ot

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _sdpa(q, k, v, allowed, scale):
    """q [N,Hq,D]; k, v [Hkv, R, D]; allowed bool [N, R]; GQA by repetition."""
    Hq, Hkv = q.shape[1], k.shape[0]
    G = Hq // Hkv
    qq = torch.from_numpy(np.ascontiguousarray(q, dtype=np.float64)).permute(1, 0, 2)
    kk = torch.from_numpy(np.ascontiguousarray(k, dtype=np.float64)).repeat_interleave(G, dim=0)
    vv = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float64)).repeat_interleave(G, dim=0)
    m = torch.from_numpy(allowed)[None, None]
    out = F.scaled_dot_product_attention(qq[None], kk[None], vv[None], attn_mask=m, scale=scale)
    return out[0].permute(1, 0, 2).numpy()


def _inputs(N, Hq, Hkv, D, S, seed):
    g = synth.rng("test", 300 + seed, 1)
    _, q = synth.normal_bf16(g, (N, Hq, D))
    _, kv = synth.normal_bf16(g, (2, Hkv, S + N, D))
    return q, kv[0], kv[1]


@pytest.mark.parametrize("Hq,Hkv,D", [(4, 2, 64), (8, 2, 128), (4, 4, 32)])
def test_chain_tree_is_causal_attention(Hq, Hkv, D):
    N, S = 9, 40
    q, k, v = _inputs(N, Hq, Hkv, D, S, Hq + D)
    parent = [-1] + list(range(N - 1))
    anc = ot.ancestor_mask(parent)
    scale = 1.0 / np.sqrt(D)
    got = oa.tree_attention(q, k, v, S, anc, scale)
    allowed = np.zeros((N, S + N), dtype=bool)
    allowed[:, :S] = True
    for n in range(N):
        allowed[n, S:S + n + 1] = True
    np.testing.assert_allclose(got, _sdpa(q, k, v, allowed, scale), atol=1e-12)


def test_every_root_to_leaf_path_is_causal_attention_alone():
    g = synth.rng("test", 310, 0)
    x = synth.deep_logits(4, 25, g)
    lp, tok = st.topk(x, 3)
    t = ot.build_tree(lp.astype(np.float32), tok, 20, root_token=0)
    N, Hq, Hkv, D, S = t.N, 4, 2, 64, 33
    q, k, v = _inputs(N, Hq, Hkv, D, S, 11)
    scale = 0.125
    got = oa.tree_attention(q, k, v, S, t.anc, scale)
    leaves = [n for n in range(N) if n not in set(t.parent.tolist())]
    assert len(leaves) >= 3
    for leaf in leaves:
        path = []
        j = leaf
        while j != -1:
            path.append(j)
            j = int(t.parent[j])
        path.reverse()
        rows = np.concatenate([np.arange(S), S + np.array(path)])
        P = len(path)
        allowed = np.ones((P, S + P), dtype=bool)
        allowed[:, S:] = np.tril(np.ones((P, P), dtype=bool))
        ref = _sdpa(q[path], k[:, rows], v[:, rows], allowed, scale)
        np.testing.assert_allclose(got[path], ref, atol=1e-12)


def test_single_node_is_decode_attention():
    Hq, Hkv, D, S = 8, 4, 64, 100
    q, k, v = _inputs(1, Hq, Hkv, D, S, 12)
    anc = ot.ancestor_mask([-1])
    got = oa.tree_attention(q, k, v, S, anc, None)
    ref = _sdpa(q, k, v, np.ones((1, S + 1), dtype=bool), 1.0 / np.sqrt(D))
    np.testing.assert_allclose(got, ref, atol=1e-12)


def test_star_tree_sees_prefix_root_and_self():
    N, Hq, Hkv, D, S = 12, 4, 1, 32, 17
    q, k, v = _inputs(N, Hq, Hkv, D, S, 13)
    anc = ot.ancestor_mask([-1] + [0] * (N - 1))
    got = oa.tree_attention(q, k, v, S, anc, 0.3)
    allowed = np.zeros((N, S + N), dtype=bool)
    allowed[:, :S + 1] = True
    allowed[np.arange(N), S + np.arange(N)] = True
    np.testing.assert_allclose(got, _sdpa(q, k, v, allowed, 0.3), atol=1e-12)


def test_planted_key_gives_order_one_output():
    """A query parallel to one visible key (large scale) returns that key's
    value row almost exactly; an invisible planted key has no effect."""
    N, Hq, Hkv, D, S = 3, 2, 1, 16, 20
    q, k, v = _inputs(N, Hq, Hkv, D, S, 14)
    parent = [-1, 0, 0]
    anc = ot.ancestor_mask(parent)
    k = k.copy()
    k[0, 5] = 4.0 * q[2, 0]  # prefix row: visible to everybody
    k[0, S + 1] = 4.0 * q[2, 1]  # node 1: not visible to node 2
    got = oa.tree_attention(q, k, v, S, anc, 4.0)
    np.testing.assert_allclose(got[2, 0], v[0, 5], atol=1e-6)
    assert np.abs(got[2, 1] - v[0, S + 1]).max() > 0.1


def test_pages_figure_node_d():
    """Figure tree root, A, B, C, D(A), E(A), F(C): node D's output uses the
    prefix and rows root, A, D only."""
    parent = [-1, 0, 0, 0, 1, 1, 3]
    N, Hq, Hkv, D, S = 7, 2, 1, 16, 9
    q, k, v = _inputs(N, Hq, Hkv, D, S, 15)
    got = oa.tree_attention(q, k, v, S, ot.ancestor_mask(parent), 0.25)
    rows = np.concatenate([np.arange(S), S + np.array([0, 1, 4])])
    allowed = np.ones((1, len(rows)), dtype=bool)
    ref = _sdpa(q[[4]], k[:, rows], v[:, rows], allowed, 0.25)
    np.testing.assert_allclose(got[[4]], ref, atol=1e-12)
