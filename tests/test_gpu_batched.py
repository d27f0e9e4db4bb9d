"""GPU parity of the batched entry points: R requests per call, each with its
own tree and its own prefix length (ragged S).

Every request's slice of a batched call must equal the oracle on that
request alone (integer and index outputs bit for bit, attention to
2e-2 + 1e-2 |ref|), and the integer outputs must also equal the
single-request entry points' on the same slice. Cited operations: top-K and
the tree ("DDTree Deep Dive", sections 1-4), tree attention (section 4),
the accept walk and the compaction (sections 5-6)."""
import numpy as np
import pytest
import torch

from block_diffusion_draft_ddtree_amd import binding as bd
from block_diffusion_draft_ddtree_amd import synth
from oracle import attention as oa
from oracle import commit as oc
from oracle import softmax_topk as st
from oracle import tree as ot

from gpu_helpers import assert_attn_close, down, down_bf16_f32, say, up, up_bf16

pytestmark = pytest.mark.gpu


def _tables(R, L, V, K, seed):
    g = synth.rng("test", 720 + seed, 0)
    V = max(V, K)
    tabs = [st.topk(synth.deep_logits(L, V, g), K) for _ in range(R)]
    lp = np.stack([t[0] for t in tabs]).astype(np.float32)
    tok = np.stack([t[1] for t in tabs]).astype(np.int32)
    return lp, tok, g


@pytest.mark.parametrize("R,L,K,B", [(1, 6, 4, 40), (5, 6, 4, 40), (3, 16, 64, 64), (8, 4, 8, 300)])
def test_build_batched(R, L, K, B):
    lp, tok, g = _tables(R, L, 60, K, R * 100 + B)
    roots = g.integers(0, 1000, size=R).astype(np.int32)
    say(f"build_batched R={R} L={L} K={K} B={B}")
    parent, depth, node_token, score, anc = bd.ddtree_build_batched(
        up(lp), up(tok), B, up(roots))
    parent, depth, node_token, score, anc = (down(t) for t in (parent, depth, node_token, score, anc))
    for r in range(R):
        tree = ot.build_tree(lp[r], tok[r], B, int(roots[r]), anc.shape[2])
        np.testing.assert_array_equal(parent[r], tree.parent)
        np.testing.assert_array_equal(depth[r], tree.depth)
        np.testing.assert_array_equal(node_token[r], tree.token)
        np.testing.assert_array_equal(score[r], tree.score)
        np.testing.assert_array_equal(anc[r].view(np.uint32), tree.anc)
        one = bd.ddtree_build(up(lp[r]), up(tok[r]), B, up(roots[r:r + 1]), anc.shape[2])
        np.testing.assert_array_equal(down(one[0]), parent[r])
        np.testing.assert_array_equal(down(one[4]), anc[r])


def test_topk_stacked_rows_equal_per_request_calls():
    """R requests' rows stacked in one ddtree_topk call equal R separate calls."""
    w = synth.WORKLOADS["coder30b_b64"]
    R = 4
    g = synth.rng("test", 730, 0)
    x = np.concatenate([synth.drafter_logits(w, r).x for r in range(R)], axis=0)
    say(f"topk stacked rows R={R} L={w.L} V={w.V}")
    lp_all, tok_all = bd.ddtree_topk(up(x), w.K)
    lp_all, tok_all = down(lp_all), down(tok_all)
    for r in range(R):
        lp1, tok1 = bd.ddtree_topk(up(x[r * w.L:(r + 1) * w.L]), w.K)
        np.testing.assert_array_equal(down(tok1), tok_all[r * w.L:(r + 1) * w.L])
        np.testing.assert_array_equal(down(lp1), lp_all[r * w.L:(r + 1) * w.L])
    for i in g.choice(R * w.L, size=3, replace=False):
        lp_ref, tok_ref = st.topk(x[i:i + 1], w.K)
        np.testing.assert_array_equal(tok_all[i], tok_ref[0])
        np.testing.assert_allclose(lp_all[i], lp_ref[0], atol=1e-5, rtol=0)


def test_walk_batched():
    R, L, K, B = 6, 6, 4, 40
    lp, tok, g = _tables(R, L, 50, K, 7)
    trees = [ot.build_tree(lp[r], tok[r], B, 1) for r in range(R)]
    parent = np.stack([t.parent for t in trees]).astype(np.int32)
    token = np.stack([t.token for t in trees]).astype(np.int32)
    tgt = np.empty_like(parent)
    for r, t in enumerate(trees):
        # Follow a planted path for a few requests, random choices for others.
        tgt[r] = g.integers(0, 50, size=t.N)
        if r % 2 == 0:
            leaf = int(np.argmax(t.depth))
            j = leaf
            while t.parent[j] != -1:
                tgt[r][t.parent[j]] = t.token[j]
                j = int(t.parent[j])
    say(f"walk_batched R={R}")
    acc, n_acc, bonus = bd.ddtree_accept_walk_batched(up(parent), up(token), L, up(tgt))
    acc, n_acc, bonus = down(acc), down(n_acc), down(bonus)
    for r, t in enumerate(trees):
        a_ref, n_ref, b_ref = oc.accept_walk(t.parent, t.token, tgt[r], L)
        np.testing.assert_array_equal(acc[r], a_ref)
        assert n_acc[r] == n_ref and bonus[r] == b_ref
    assert n_acc.max() >= 3


def test_kv_compact_batched():
    R, layers, Hkv, D, N, L = 5, 3, 2, 64, 33, 6
    S = [0, 17, 64, 100, 5]
    S_cap = max(S) + N + 3
    g = synth.rng("test", 731, 0)
    bits, _ = synth.normal_bf16(g, (R, layers, 2, Hkv, S_cap, D))
    acc = np.full((R, L + 1), -1, dtype=np.int32)
    n_acc = np.zeros(R, dtype=np.int32)
    for r in range(R):
        a = int(g.integers(0, L + 1))
        path = np.sort(g.choice(np.arange(1, N), size=a, replace=False)) if a else []
        acc[r, 0] = 0
        acc[r, 1:a + 1] = path
        n_acc[r] = a
    say(f"kv_compact_batched R={R} S={S}")
    kv = up_bf16(bits)
    bd.ddtree_kv_compact_batched(kv, S, N, L, up(acc), up(n_acc))
    got = down(kv.view(torch.int16)).view(np.uint16)
    for r in range(R):
        want = oc.kv_compact(bits[r], S[r], acc[r], int(n_acc[r]))
        np.testing.assert_array_equal(got[r], want)


def _attn_batch(R, N, Hq, Hkv, D, S, seed, layers=2, layer=1):
    g = synth.rng("test", 740 + seed, 1)
    S_cap = max(S) + N + 5
    q_bits, q = synth.normal_bf16(g, (R, N, Hq, D))
    kv_bits, kv = synth.normal_bf16(g, (R, layers, 2, Hkv, S_cap, D))
    ancs = []
    for r in range(R):
        parent = [-1] + [int(g.integers(0, n)) for n in range(1, N)]
        ancs.append(ot.ancestor_mask(parent))
    anc = np.stack(ancs)
    say(f"attn_batched R={R} N={N} Hq={Hq} Hkv={Hkv} D={D} S={S}")
    out = bd.ddtree_tree_attn_batched(up_bf16(q_bits), up_bf16(kv_bits), layer, S,
                                      up(anc.view(np.int32)))
    return q_bits, q, kv_bits, kv, anc, down_bf16_f32(out), g


@pytest.mark.parametrize("R,N,Hq,Hkv,D,S", [
    (1, 17, 8, 2, 128, [300]),
    (3, 17, 8, 2, 128, [0, 1000, 37]),
    (5, 33, 4, 1, 64, [64, 0, 513, 5, 200]),
    (2, 65, 16, 4, 128, [700, 129]),
    (3, 129, 32, 4, 128, [0, 700, 2000]),  # 1032 rows per kv-head: 128-row tiles
    (2, 257, 8, 2, 64, [300, 5]),          # 1028 rows, D = 64
])
def test_attn_batched_small(R, N, Hq, Hkv, D, S):
    q_bits, q, kv_bits, kv, anc, got, _ = _attn_batch(R, N, Hq, Hkv, D, S, R + N)
    for r in range(R):
        ref = oa.tree_attention(q[r], kv[r, 1, 0], kv[r, 1, 1], S[r], anc[r])
        assert_attn_close(got[r], ref, f"request {r} S={S[r]}")
        # The single-request call on the same slices agrees to the same bound.
        one = bd.ddtree_tree_attn(up_bf16(q_bits[r]), up_bf16(kv_bits[r, 1, 0]),
                                  up_bf16(kv_bits[r, 1, 1]), S[r], up(anc[r].view(np.int32)))
        assert_attn_close(got[r], down_bf16_f32(one), f"request {r} vs single call")


def test_attn_batched_workload_shape_sampled():
    """Four requests of the 30B verifier shape (N = 65, Hq = 32, Hkv = 4,
    D = 128) with ragged prefixes; sampled (node, head) rows per request."""
    S = [4096, 1000, 2500, 64]
    q_bits, q, kv_bits, kv, anc, got, g = _attn_batch(4, 65, 32, 4, 128, S, 99, layers=1, layer=0)
    for r in range(4):
        nodes = sorted(g.choice(65, size=5, replace=False).tolist())
        heads = sorted(g.choice(32, size=4, replace=False).tolist())
        ref = oa.tree_attention(q[r], kv[r, 0, 0], kv[r, 0, 1], S[r], anc[r], nodes=nodes,
                                heads=heads)
        assert_attn_close(got[r][np.ix_(nodes, heads)], ref[np.ix_(nodes, heads)],
                          f"request {r} S={S[r]}")


def test_batched_round_matches_single_request_rounds():
    """topk (stacked rows) -> build_batched -> attn_batched (every layer) ->
    walk_batched -> kv_compact_batched against the same requests run one by
    one through the single-request entry points."""
    R, L, V, K, B = 3, 6, 300, 8, 32
    N = B + 1
    Hq, Hkv, D, layers = 8, 2, 64, 2
    S = [50, 0, 130]
    S_cap = max(S) + N
    g = synth.rng("test", 750, 0)
    x = np.concatenate([synth.deep_logits(L, V, g) for _ in range(R)], axis=0).astype(np.float32)
    roots = g.integers(0, V, size=R).astype(np.int32)
    q_bits, _ = synth.normal_bf16(g, (layers, R, N, Hq, D))
    kv_bits, _ = synth.normal_bf16(g, (R, layers, 2, Hkv, S_cap, D))
    say("batched round vs single rounds")
    lp, tok = bd.ddtree_topk(up(x), K)
    parent, depth, ntok, score, anc = bd.ddtree_build_batched(
        lp.view(R, L, K), tok.view(R, L, K), B, up(roots))
    kvd = up_bf16(kv_bits)
    outs = [bd.ddtree_tree_attn_batched(up_bf16(q_bits[l]), kvd, l, S, anc) for l in range(layers)]
    # Targets: follow each request's first child chain for two steps.
    tgt = down(ntok).copy()
    par = down(parent)
    for r in range(R):
        tgt[r] = g.integers(0, V, size=N)
        kids = np.flatnonzero(par[r] == 0)
        if kids.size:
            tgt[r][0] = down(ntok)[r][kids[0]]
    acc, n_acc, bonus = bd.ddtree_accept_walk_batched(parent, ntok, L, up(tgt))
    bd.ddtree_kv_compact_batched(kvd, S, N, L, acc, n_acc)
    kv_after = down(kvd.view(torch.int16)).view(np.uint16)
    for r in range(R):
        lp1, tok1 = bd.ddtree_topk(up(x[r * L:(r + 1) * L]), K)
        p1, d1, t1, s1, a1 = bd.ddtree_build(lp1, tok1, B, up(roots[r:r + 1]), anc.shape[2])
        np.testing.assert_array_equal(down(t1), down(ntok)[r])
        np.testing.assert_array_equal(down(a1), down(anc)[r])
        kv1 = up_bf16(kv_bits[r])
        for l in range(layers):
            o1 = bd.ddtree_tree_attn(up_bf16(q_bits[l, r]), kv1[l, 0], kv1[l, 1], S[r], a1)
            assert_attn_close(down_bf16_f32(outs[l])[r], down_bf16_f32(o1), f"r={r} layer={l}")
        acc1, n1, b1 = bd.ddtree_accept_walk(p1, t1, L, up(tgt[r]))
        np.testing.assert_array_equal(down(acc1), down(acc)[r])
        assert int(down(n1)[0]) == int(down(n_acc)[r]) and int(down(b1)[0]) == int(down(bonus)[r])
        bd.ddtree_kv_compact(kv1, S[r], N, L, acc1, n1)
        np.testing.assert_array_equal(down(kv1.view(torch.int16)).view(np.uint16), kv_after[r])
