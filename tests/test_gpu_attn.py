"""GPU parity: ddtree_tree_attn against the naive fp64 oracle.

Element-wise bound |gpu - oracle| <= 2e-2 + 1e-2 * |oracle| (bf16 inputs,
fp32 accumulation, bf16 softmax weights in the P.V product, bf16 output).
Small shapes compare every output; the full workload shapes compare a
sample of (node, head) rows the oracle computes one by one."""
import numpy as np
import pytest
import torch

from block_diffusion_draft_ddtree_amd import binding as bd
from block_diffusion_draft_ddtree_amd import synth
from oracle import attention as oa
from oracle import softmax_topk as st
from oracle import tree as ot

from gpu_helpers import assert_attn_close, down_bf16_bits, down_bf16_f32, say, up, up_bf16

pytestmark = pytest.mark.gpu


def _tree_anc(kind, N, g, W=None):
    if kind == "chain":
        parent = [-1] + list(range(N - 1))
    elif kind == "star":
        parent = [-1] + [0] * (N - 1)
    else:  # random recursive tree
        parent = [-1] + [int(g.integers(0, n)) for n in range(1, N)]
    return ot.ancestor_mask(parent, W)


def _run(q_bits, q, kv_bits, kv, S, anc, scale=None, nodes=None, heads=None, twice=False):
    N, Hq, D = q.shape
    Hkv, S_cap = kv.shape[1], kv.shape[2]
    say(f"attn N={N} Hq={Hq} Hkv={Hkv} D={D} S={S} S_cap={S_cap}")
    qd = up_bf16(q_bits)
    kvd = up_bf16(kv_bits)
    ancd = up(anc.view(np.int32))
    out = bd.ddtree_tree_attn(qd, kvd[0], kvd[1], S, ancd, scale)
    got = down_bf16_f32(out)
    ref = oa.tree_attention(q, kv[0], kv[1], S, anc, scale, nodes=nodes, heads=heads)
    if nodes is not None or heads is not None:
        nn = list(range(N)) if nodes is None else list(nodes)
        hh = list(range(Hq)) if heads is None else list(heads)
        got, ref = got[np.ix_(nn, hh)], ref[np.ix_(nn, hh)]
    stats = assert_attn_close(got, ref, f"N={N} Hq={Hq} Hkv={Hkv} D={D} S={S}")
    if twice:
        again = bd.ddtree_tree_attn(qd, kvd[0], kvd[1], S, ancd, scale)
        np.testing.assert_array_equal(down_bf16_bits(again), down_bf16_bits(out))
    return stats


def _inputs(N, Hq, Hkv, D, S, seed, S_cap=None):
    g = synth.rng("test", 700 + seed, 1)
    S_cap = S + N if S_cap is None else S_cap
    q_bits, q = synth.normal_bf16(g, (N, Hq, D))
    kv_bits, kv = synth.normal_bf16(g, (2, Hkv, S_cap, D))
    return q_bits, q, kv_bits, kv, g


def test_tiny_workload():
    w = synth.TINY
    lg = synth.drafter_logits(w)
    lp, tok = st.topk(lg.x, w.K)
    tree = ot.build_tree(lp.astype(np.float32), tok, w.B, 0)
    qkv = synth.attention_inputs(w)
    _run(qkv.q_bits, qkv.q, qkv.kv_bits[0], qkv.kv[0], w.S, tree.anc, twice=True)


@pytest.mark.parametrize("N,Hq,Hkv,D,S,kind", [
    (1, 4, 2, 64, 128, "chain"),      # decode: one node
    (17, 4, 2, 64, 0, "random"),      # no prefix at all
    (129, 4, 4, 128, 0, "random"),    # no prefix, G = 1: blocks where only some columns see keys
    (65, 32, 4, 128, 0, "random"),    # no prefix at the 30B head layout
    (257, 32, 8, 128, 0, "random"),
    (33, 8, 2, 128, 100, "random"),   # ragged prefix (not a multiple of 64)
    (65, 8, 1, 128, 64, "chain"),
    (65, 16, 4, 64, 37, "star"),
    (130, 4, 4, 128, 300, "random"),  # G = 1
    (257, 32, 8, 128, 513, "random"),
    (513, 4, 1, 64, 700, "random"),
])
def test_shapes_and_masks(N, Hq, Hkv, D, S, kind):
    q_bits, q, kv_bits, kv, g = _inputs(N, Hq, Hkv, D, S, N + S + D)
    anc = _tree_anc(kind, N, g)
    _run(q_bits, q, kv_bits, kv, S, anc, twice=True)


def test_slack_capacity_and_extra_mask_words():
    N, Hq, Hkv, D, S = 40, 8, 2, 128, 190
    q_bits, q, kv_bits, kv, g = _inputs(N, Hq, Hkv, D, S, 1, S_cap=S + N + 77)
    anc = _tree_anc("random", N, g, W=5)
    _run(q_bits, q, kv_bits, kv, S, anc, scale=0.05)


def test_planted_keys_order_one_outputs():
    """Queries parallel to one visible key with a large scale: the output is
    that key's value row, an O(1) signal the tolerance can see."""
    N, Hq, Hkv, D, S = 9, 4, 2, 64, 70
    q_bits, q, kv_bits, kv, g = _inputs(N, Hq, Hkv, D, S, 2)
    parent = [-1, 0, 1, 2, 0, 4, 5, 1, 7]
    anc = ot.ancestor_mask(parent)
    kv = kv.copy()
    G = Hq // Hkv
    for n in range(N):
        for h in range(Hq):
            target = S + parent[n] if n else 3  # parent's tree row, or a prefix row
            kv[0, h // G, target] = q[n, h]
    kv_bits = synth.f32_to_bf16_bits(kv)
    kv = synth.bf16_bits_to_f32(kv_bits)
    _run(q_bits, q, kv_bits, kv, S, anc, scale=2.0)


@pytest.mark.parametrize("name", ["coder30b_b64", "qwen3_8b"])
def test_full_workload_every_element(name):
    """The metric shapes in full: every output element of one layer (65
    nodes x 32 heads x 128 dims) against the oracle, through the launch
    plan bench.py times (7 splits of 5 superblocks at the 30B shape)."""
    w = synth.WORKLOADS[name]
    lg = synth.drafter_logits(w)
    lp, tok = st.topk(lg.x, w.K)
    tree = ot.build_tree(lp.astype(np.float32), tok, w.B, 0)
    qkv = synth.attention_inputs(w, layers=1)
    _run(qkv.q_bits, qkv.q, qkv.kv_bits[0], qkv.kv[0], w.S, tree.anc)


def test_planted_keys_through_splits_at_metric_shape():
    """O(1) outputs through the split path at the 30B shape (32q/4kv heads,
    D = 128, S = 4096, N = 65; the key range runs as 7 splits whose fp16
    outputs are merged). Query (n, h) finds a copy of itself among the
    prefix keys at a row past the first split (rows 640 ... 3760, a
    different one for every query of a kv-head), or, for one query head per
    kv-head and node, at the node's own tree row; with the default scale it
    takes about 90 % of the weight and the rest blends in, so every output
    is an O(1) mixture that the tolerance resolves. Random tree with depth,
    every element compared."""
    N, Hq, Hkv, D, S = 65, 32, 4, 128, 4096
    q_bits, q, kv_bits, kv, g = _inputs(N, Hq, Hkv, D, S, 11)
    parent = [-1] + [int(g.integers(max(0, n - 4), n)) for n in range(1, N)]
    anc = ot.ancestor_mask(parent)
    kv = kv.copy()
    G = Hq // Hkv
    tree_rows = 0
    for gk in range(Hkv):
        i = 0
        for n in range(N):
            for hh in range(G):
                h = gk * G + hh
                if n > 0 and hh == n % G:
                    kv[0, gk, S + n] = q[n, h]   # the node's own row: always visible
                    tree_rows += 1
                else:
                    kv[0, gk, 640 + 6 * i] = q[n, h]
                    i += 1
    assert tree_rows == Hkv * (N - 1)
    kv_bits = synth.f32_to_bf16_bits(kv)
    kv = synth.bf16_bits_to_f32(kv_bits)
    ws = bd.ddtree_tree_attn_workspace_bytes(N, Hq, Hkv, D, S)
    assert ws > 0  # the key range is split
    stats = _run(q_bits, q, kv_bits, kv, S, anc)
    assert stats["max_abs"] < 0.1


@pytest.mark.parametrize("name", ["coder30b_b256", "coder30b_b64_deep", "sweep_b512"])
def test_full_workload_sampled(name):
    w = synth.WORKLOADS[name]
    lg = synth.drafter_logits(w)
    lp, tok = st.topk(lg.x, w.K)
    tree = ot.build_tree(lp.astype(np.float32), tok, w.B, 0)
    qkv = synth.attention_inputs(w, layers=1)
    g = synth.rng("test", 790, 0)
    nodes = sorted(set([0, w.N - 1] + g.choice(w.N, 6, replace=False).tolist()))
    heads = sorted(set([0, w.Hq - 1] + g.choice(w.Hq, 3, replace=False).tolist()))
    _run(qkv.q_bits, qkv.q, qkv.kv_bits[0], qkv.kv[0], w.S, tree.anc, nodes=nodes, heads=heads)


def test_long_context_sampled():
    w = synth.LONGCTX
    lg = synth.drafter_logits(w)
    lp, tok = st.topk(lg.x, w.K)
    tree = ot.build_tree(lp.astype(np.float32), tok, w.B, 0)
    qkv = synth.attention_inputs(w, layers=1)
    nodes = [0, 1, 100, 256]
    heads = [0, 13, 31]
    _run(qkv.q_bits, qkv.q, qkv.kv_bits[0], qkv.kv[0], w.S, tree.anc, nodes=nodes, heads=heads)


def test_max_nodes_random_tree_sampled():
    """The largest tree (N = DDTREE_MAX_B + 1 = 1025 nodes, 33 mask words) of
    random depth at the budget-sweep shape (Hq = 32, Hkv = 8, D = 128,
    S = 8192); sampled (node, head) rows, the deepest node included."""
    N, Hq, Hkv, D, S = 1025, 32, 8, 128, 8192
    q_bits, q, kv_bits, kv, g = _inputs(N, Hq, Hkv, D, S, 5)
    anc = _tree_anc("random", N, g)
    popc = np.array([sum(bin(int(w)).count("1") for w in row) for row in anc.view(np.uint32)])
    deepest = int(np.argmax(popc))
    nodes = sorted({0, 1, 511, 1024, deepest})
    _run(q_bits, q, kv_bits, kv, S, anc, nodes=nodes, heads=[0, 5, 31])


def test_max_nodes_d64_full():
    """1025 nodes at D = 64, G = 4: every output element."""
    q_bits, q, kv_bits, kv, g = _inputs(1025, 4, 1, 64, 300, 6)
    anc = _tree_anc("random", 1025, g)
    _run(q_bits, q, kv_bits, kv, 300, anc)


def test_large_values_through_split_partials():
    """The split path stores each split's normalised output as fp16, whose
    range ends at 65504 (the documented limit on |V|): V at magnitudes up to
    2^15 (bf16-exact) at the 30B shape, where the key range runs as 7
    splits. Every element compared after dividing both sides by V's scale
    (the tolerance is stated for unit-scale values), so an overflow or a
    lost split shows."""
    N, Hq, Hkv, D, S = 65, 32, 4, 128, 4096
    q_bits, q, kv_bits, kv, g = _inputs(N, Hq, Hkv, D, S, 12)
    big = np.float32(2.0 ** 14)
    kv = kv.copy()
    kv[1] = np.clip(kv[1] * big, -2.0 * big, 2.0 * big)
    kv_bits = synth.f32_to_bf16_bits(kv)
    kv = synth.bf16_bits_to_f32(kv_bits)
    parent = [-1] + [int(g.integers(max(0, n - 4), n)) for n in range(1, N)]
    anc = ot.ancestor_mask(parent)
    assert bd.ddtree_tree_attn_workspace_bytes(N, Hq, Hkv, D, S) > 0  # the split path
    say(f"attn large V N={N} S={S}")
    kvd = up_bf16(kv_bits)
    out = bd.ddtree_tree_attn(up_bf16(q_bits), kvd[0], kvd[1], S, up(anc.view(np.int32)), 0.25)
    got = down_bf16_f32(out)
    assert np.isfinite(got).all()
    ref = oa.tree_attention(q, kv[0], kv[1], S, anc, 0.25)
    assert np.abs(ref).max() > 1000.0  # the outputs do reach the large scale
    assert_attn_close(got / big, ref / big, "large V through the split path")


@pytest.mark.parametrize("N,Hq,Hkv,D,S,kind", [
    (127, 32, 4, 128, 1000, "random"),  # 1016 rows per kv-head: 64-row tiles
    (128, 32, 4, 128, 1000, "random"),  # 1024 rows: 128-row tiles from here on
    (129, 32, 4, 128, 1000, "random"),  # 1032 rows: a last tile of 8 rows
    (129, 8, 1, 64, 0, "random"),       # D = 64, no prefix
    (300, 16, 4, 128, 2500, "chain"),   # several splits
    (1025, 4, 4, 128, 300, "random"),   # G = 1: 128 nodes per tile
    (1025, 8, 4, 64, 77, "star"),
])
def test_tall_tiles_every_element(N, Hq, Hkv, D, S, kind):
    """Both tile shapes around the switch at 1024 query rows per kv-head
    (N * G): every output element against the oracle, and a second call
    bit-identical to the first."""
    q_bits, q, kv_bits, kv, g = _inputs(N, Hq, Hkv, D, S, 40 + N + S + D)
    anc = _tree_anc(kind, N, g)
    _run(q_bits, q, kv_bits, kv, S, anc, twice=True)


@pytest.mark.parametrize("S", [200, 3000])
def test_pruned_rows_in_tall_tiles(S):
    """A star of 1025 nodes at G = 1 (128 nodes per tile) with rows of
    dropped leaves emptied as ddtree_tree_prune leaves them: a whole tile
    dropped (nodes 256-383), a tile whose first 64 nodes are dropped and
    last 64 kept (640-703), one whose last 64 are dropped (960-1023), and
    scattered single nodes. A tile with any kept node must run: the kept
    rows are compared with the oracle (the dropped rows are unspecified)."""
    N, Hq, Hkv, D = 1025, 2, 2, 128
    q_bits, q, kv_bits, kv, g = _inputs(N, Hq, Hkv, D, S, 60 + S)
    anc = _tree_anc("star", N, g)
    dropped = set(range(256, 384)) | set(range(640, 704)) | set(range(960, 1024)) | {5, 130, 517}
    anc = anc.copy()
    for n in dropped:
        anc[n] = 0
    kept = [n for n in range(N) if n not in dropped]
    say(f"attn pruned tall tiles S={S} kept={len(kept)}")
    qd = up_bf16(q_bits)
    kvd = up_bf16(kv_bits)
    out = bd.ddtree_tree_attn(qd, kvd[0], kvd[1], S, up(anc.view(np.int32)))
    got = down_bf16_f32(out)[kept]
    ref = oa.tree_attention(q, kv[0], kv[1], S, anc, nodes=kept)[kept]
    assert_attn_close(got, ref, f"pruned star N={N} S={S}")
