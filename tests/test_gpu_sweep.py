"""GPU parity over a seeded sweep of shapes: tree attention (single and
batched calls), top-K and the tree build, each against the oracle.

Every case draws its shape from a fixed seed: node counts across the tile
and mask-word boundaries, both head sizes, group sizes 1-8, prefixes from
empty to several splits, slack in the cache capacity, extra mask words,
random tree shapes; top-K rows of odd lengths and K up to the row; trees
from tie-rich and deep tables. Bounds as in the per-kernel tests:
attention |gpu - oracle| <= 2e-2 + 1e-2 |oracle|, integer outputs exact,
log-probs within 1e-5."""
import numpy as np
import pytest

from block_diffusion_draft_ddtree_amd import binding as bd
from block_diffusion_draft_ddtree_amd import synth
from oracle import attention as oa
from oracle import softmax_topk as st
from oracle import tree as ot

from gpu_helpers import assert_attn_close, down, down_bf16_bits, down_bf16_f32, say, up, up_bf16

pytestmark = pytest.mark.gpu


def _random_parent(g, N):
    kind = g.integers(0, 3)
    if kind == 0:
        return [-1] + list(range(N - 1))                       # chain
    if kind == 1:
        return [-1] + [0] * (N - 1)                            # star
    return [-1] + [int(g.integers(0, n)) for n in range(1, N)]  # random recursive


@pytest.mark.parametrize("case", range(64))
def test_attention_shapes(case):
    g = synth.rng("test", 800, case)
    D = int(g.choice([64, 128]))
    Hkv = int(g.choice([1, 2, 4]))
    G = int(g.choice([1, 2, 4, 8]))
    Hq = Hkv * G
    N = int(g.choice([1, 2, 31, 32, 33, 63, 64, 65, 97, 129, 200]))
    S = int(g.choice([0, 1, 37, 128, 255, 600, 1500]))
    S_cap = S + N + int(g.integers(0, 40))
    W = (N + 31) // 32 + int(g.integers(0, 2))
    scale = float(g.uniform(0.05, 0.2))
    say(f"sweep attn case={case} N={N} Hq={Hq} Hkv={Hkv} D={D} S={S} S_cap={S_cap} W={W}")
    q_bits, q = synth.normal_bf16(g, (N, Hq, D))
    kv_bits, kv = synth.normal_bf16(g, (2, Hkv, S_cap, D))
    anc = ot.ancestor_mask(_random_parent(g, N), W)
    out = bd.ddtree_tree_attn(up_bf16(q_bits), up_bf16(kv_bits[0]), up_bf16(kv_bits[1]), S,
                              up(anc.view(np.int32)), scale)
    ref = oa.tree_attention(q, kv[0], kv[1], S, anc, scale)
    assert_attn_close(down_bf16_f32(out), ref, f"case {case}")


@pytest.mark.parametrize("case", range(16))
def test_tall_attention_shapes(case):
    """Shapes with at least 1024 query rows per kv-head (128-row tiles):
    node counts from 128 to 1025, group sizes 1-8, both head sizes, prefixes
    from empty to several splits, random tree shapes; sampled (node, head)
    rows, the first and last node included."""
    g = synth.rng("test", 803, case)
    D = int(g.choice([64, 128]))
    Hkv = int(g.choice([1, 2, 4]))
    G = int(g.choice([1, 2, 4, 8]))
    Hq = Hkv * G
    N = int(g.integers(-(-1024 // G), 1026))
    S = int(g.choice([0, 1, 100, 777, 3000]))
    S_cap = S + N + int(g.integers(0, 40))
    W = (N + 31) // 32 + int(g.integers(0, 2))
    scale = float(g.uniform(0.05, 0.2))
    say(f"sweep tall attn case={case} N={N} Hq={Hq} Hkv={Hkv} D={D} S={S} S_cap={S_cap} W={W}")
    q_bits, q = synth.normal_bf16(g, (N, Hq, D))
    kv_bits, kv = synth.normal_bf16(g, (2, Hkv, S_cap, D))
    anc = ot.ancestor_mask(_random_parent(g, N), W)
    out = bd.ddtree_tree_attn(up_bf16(q_bits), up_bf16(kv_bits[0]), up_bf16(kv_bits[1]), S,
                              up(anc.view(np.int32)), scale)
    nodes = sorted({0, N - 1} | set(g.choice(N, size=min(N, 24), replace=False).tolist()))
    heads = sorted({0, Hq - 1} | set(g.choice(Hq, size=min(Hq, 3), replace=False).tolist()))
    ref = oa.tree_attention(q, kv[0], kv[1], S, anc, scale, nodes=nodes, heads=heads)
    got = down_bf16_f32(out)
    assert_attn_close(got[np.ix_(nodes, heads)], ref[np.ix_(nodes, heads)], f"tall case {case}")


@pytest.mark.parametrize("case", range(16))
def test_batched_attention_shapes(case):
    g = synth.rng("test", 801, case)
    R = int(g.integers(2, 7))
    D = int(g.choice([64, 128]))
    Hkv = int(g.choice([1, 2, 4]))
    Hq = Hkv * int(g.choice([1, 4, 8]))
    N = int(g.choice([1, 17, 33, 65]))
    S = [int(x) for x in g.choice([0, 5, 100, 513, 1024, 2000], size=R)]
    layers = 2
    S_cap = max(S) + N + int(g.integers(0, 9))
    say(f"sweep batched case={case} R={R} N={N} Hq={Hq} Hkv={Hkv} D={D} S={S}")
    q_bits, q = synth.normal_bf16(g, (R, N, Hq, D))
    kv_bits, kv = synth.normal_bf16(g, (R, layers, 2, Hkv, S_cap, D))
    anc = np.stack([ot.ancestor_mask(_random_parent(g, N)) for _ in range(R)])
    out = down_bf16_f32(bd.ddtree_tree_attn_batched(up_bf16(q_bits), up_bf16(kv_bits), 1, S,
                                                    up(anc.view(np.int32))))
    for r in range(R):
        ref = oa.tree_attention(q[r], kv[r, 1, 0], kv[r, 1, 1], S[r], anc[r])
        assert_attn_close(out[r], ref, f"case {case} request {r}")


@pytest.mark.parametrize("case", range(32))
def test_topk_and_build_shapes(case):
    g = synth.rng("test", 802, case)
    L = int(g.integers(1, 9))
    V = int(g.choice([5, 64, 257, 1000, 4097, 9000]))
    K = int(min(V, g.choice([1, 2, 8, 33, 64, 100])))
    if g.uniform() < 0.4:
        x = synth.deep_logits(L, V, g).astype(np.float32)
    else:
        x = np.round(g.standard_normal((L, V)) * 3).astype(np.float32)  # tie-rich
    say(f"sweep topk/build case={case} L={L} V={V} K={K}")
    lp, tok = bd.ddtree_topk(up(x), K)
    lp, tok = down(lp), down(tok)
    lp_ref, tok_ref = st.topk(x, K)
    np.testing.assert_array_equal(tok, tok_ref)
    np.testing.assert_allclose(lp, lp_ref, atol=1e-5, rtol=0)
    total = sum(K ** d for d in range(1, L + 1))
    B = int(min(total, g.choice([1, 5, 16, 64, 100, 300])))
    root = int(g.integers(0, V))
    parent, depth, ntok, score, anc = bd.ddtree_build(up(lp), up(tok), B, up(np.array([root], np.int32)))
    tree = ot.build_tree(lp, tok, B, root)
    np.testing.assert_array_equal(down(parent), tree.parent)
    np.testing.assert_array_equal(down(depth), tree.depth)
    np.testing.assert_array_equal(down(ntok), tree.token)
    np.testing.assert_array_equal(down(anc).view(np.uint32), tree.anc)


def test_budget_sweep_rounds_chained():
    """Four chained decode rounds of the budget-sweep recipe (B = 32, flat
    logits, 32q/8kv heads, D = 128, two layers, prefix from 8192): each
    round writes fresh K/V rows for its tree at rows S..S+N-1, runs top-K,
    build, both layers' attention at the current S, the walk, and the
    compaction of a drawn accepted path (a ~ U[1, L]); S then grows by
    1 + a. One attention workspace serves every round (sized once at the
    last round's S). Tree, attention (every element), walk and the whole
    cache after each compaction are compared with the oracle."""
    from dataclasses import replace

    import torch

    from oracle import commit as oc
    from block_diffusion_draft_ddtree_amd.round import DraftTreeRound, RoundShape

    rounds = 4
    w = replace(synth.sweep(32), layers=2)
    acc_np, a_np = synth.sweep_accepts(w.B, w.L, rounds)
    S_r = synth.sweep_prefix_lengths(w.S, a_np)
    S_cap = int(S_r[-1]) + w.N
    g = synth.rng("test", 803, 0)
    kv_bits, _ = synth.normal_bf16(g, (w.layers, 2, w.Hkv, S_cap, w.D))
    kv_dev = up_bf16(kv_bits)
    shape = RoundShape(w.L, w.V, w.K, w.B, w.Hq, w.Hkv, w.D, w.layers, S_cap)
    rnd = DraftTreeRound(shape, int(S_r[-1]), "cuda:0")
    ws0 = rnd.ws_attn.numel()
    for r in range(rounds):
        S = int(S_r[r])
        say(f"sweep decode round={r} S={S} B={w.B}")
        fresh_bits, _ = synth.normal_bf16(g, (w.layers, 2, w.Hkv, w.N, w.D))
        kv_bits[:, :, :, S:S + w.N] = fresh_bits
        kv_dev[:, :, :, S:S + w.N] = up_bf16(fresh_bits)
        q_bits, q = synth.normal_bf16(g, (w.layers, w.N, w.Hq, w.D))
        q_dev = up_bf16(q_bits)
        lg = synth.drafter_logits(w, r)
        root = int(g.integers(0, w.V))
        rnd.root_token.fill_(root)
        rnd.topk(up(lg.x))
        rnd.build()
        lp, tok = down(rnd.logp), down(rnd.token)
        lp_ref, tok_ref = st.topk(lg.x, w.K)
        np.testing.assert_array_equal(tok, tok_ref)
        tree = ot.build_tree(lp, tok, w.B, root)
        np.testing.assert_array_equal(down(rnd.parent), tree.parent)
        np.testing.assert_array_equal(down(rnd.anc).view(np.uint32), tree.anc)
        for layer in range(w.layers):
            rnd.attn(layer, q_dev, kv_dev, S)
        kv_f = synth.bf16_bits_to_f32(kv_bits)
        for layer in range(w.layers):
            ref = oa.tree_attention(q[layer], kv_f[layer, 0], kv_f[layer, 1], S, tree.anc)
            assert_attn_close(down_bf16_f32(rnd.attn_out[layer]), ref, f"round {r} layer {layer}")
        tgt = g.integers(0, w.V, size=w.N).astype(np.int32)
        rnd.walk(up(tgt))
        acc_w, a_w, bonus = oc.accept_walk(tree.parent, tree.token, tgt, w.L)
        assert int(down(rnd.n_acc)[0]) == a_w and int(down(rnd.next_bonus)[0]) == bonus
        acc_d = up(acc_np[r])
        n_d = up(a_np[r:r + 1])
        bd.ddtree_kv_compact(kv_dev, S, w.N, w.L, acc_d, n_d)
        for layer in range(w.layers):
            kv_bits[layer] = oc.kv_compact(kv_bits[layer], S, acc_np[r][:1 + a_np[r]],
                                           int(a_np[r]))
        np.testing.assert_array_equal(down_bf16_bits(kv_dev), kv_bits)
        torch.cuda.synchronize()
    assert rnd.ws_attn.numel() == ws0
