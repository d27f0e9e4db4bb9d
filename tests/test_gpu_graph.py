"""GPU: a whole round captured in a HIP graph and replayed equals the same
round run eagerly, replay after replay.

The round (top-K, build, every layer's tree attention, accept walk, KV
compaction; "DDTree Deep Dive", section 3) is captured once and replayed
four times, with eager work between the replays: the inputs are reset by
ordinary copies (the compaction rewrites the cache in place) and a
throwaway eager call of every kernel runs on other buffers. Every output of
every replay must equal the eager round bit for bit (the kernels are
deterministic for a fixed launch plan). The round enqueues only libddtree
kernels, none of which records a memset. Also: two rounds chained on the
device (the walk's next bonus becomes the next root) against the oracle."""
import numpy as np
import pytest
import torch

from block_diffusion_draft_ddtree_amd import synth
from block_diffusion_draft_ddtree_amd.round import DraftTreeRound, RoundShape
from oracle import commit as oc
from oracle import softmax_topk as st
from oracle import tree as ot

from gpu_helpers import say

pytestmark = pytest.mark.gpu


def _setup(layers=3):
    w = synth.TINY
    dev = torch.device("cuda:0")
    g = synth.rng("test", 760, 0)
    S_cap = w.S + w.N
    shape = RoundShape(w.L, w.V, w.K, w.B, w.Hq, w.Hkv, w.D, layers, S_cap)
    logits = torch.from_numpy(synth.deep_logits(w.L, w.V, g).astype(np.float32)).to(dev)
    qb, _ = synth.normal_bf16(g, (layers, w.N, w.Hq, w.D))
    kvb, _ = synth.normal_bf16(g, (layers, 2, w.Hkv, S_cap, w.D))
    q = torch.from_numpy(qb.view(np.int16)).to(dev).view(torch.bfloat16)
    kv0 = torch.from_numpy(kvb.view(np.int16)).to(dev).view(torch.bfloat16)
    tgt = torch.from_numpy(g.integers(0, w.V, size=w.N).astype(np.int32)).to(dev)
    return w, dev, shape, logits, q, kv0, tgt


def _outputs(rnd, kv):
    return [t.clone() for t in (rnd.logp, rnd.token, rnd.parent, rnd.depth, rnd.node_token,
                                rnd.score, rnd.anc, rnd.attn_out, rnd.acc, rnd.n_acc,
                                rnd.next_bonus, kv)]


def test_graph_replays_equal_eager_round():
    w, dev, shape, logits, q, kv0, tgt = _setup()
    rnd = DraftTreeRound(shape, w.S, dev)
    rnd.root_token.fill_(7)
    kv = kv0.clone()
    say("graph: eager round")
    rnd.run(logits, q, kv, w.S, tgt)
    torch.cuda.synchronize()
    want = _outputs(rnd, kv)
    other = DraftTreeRound(shape, w.S, dev)
    kv_other = kv0.clone()
    kv.copy_(kv0)
    torch.cuda.synchronize()
    say("graph: capture")
    graph = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        rnd.run(logits, q, kv, w.S, tgt)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    kv.copy_(kv0)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        rnd.run(logits, q, kv, w.S, tgt)
    torch.cuda.synchronize()
    for rep in range(4):
        say(f"graph: replay {rep}")
        for t in (rnd.logp, rnd.parent, rnd.attn_out, rnd.acc, rnd.next_bonus):
            t.zero_()
        kv.copy_(kv0)
        other.run(logits, q, kv_other, w.S, tgt)  # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        got = _outputs(rnd, kv)
        for i, (a, b) in enumerate(zip(got, want)):
            assert torch.equal(a, b), f"replay {rep}: output {i} differs from the eager round"


def test_two_rounds_chain_on_device():
    """The second decoding round's root is the first one's next bonus, copied on the device; its
    prefix grows by the accepted path plus the bonus row. Both rounds are
    checked against the oracle (top-K, tree, walk, compaction)."""
    w, dev, shape, logits, q, kv0, tgt = _setup(layers=1)
    S_cap = w.S + 2 * (w.L + 1) + w.N
    shape = RoundShape(w.L, w.V, w.K, w.B, w.Hq, w.Hkv, w.D, 1, S_cap)
    g = synth.rng("test", 761, 0)
    kvb, _ = synth.normal_bf16(g, (1, 2, w.Hkv, S_cap, w.D))
    kv = torch.from_numpy(kvb.view(np.int16)).to(dev).view(torch.bfloat16)
    kv_ref = kvb.copy()
    root = 7
    S = w.S
    rnd_tok = torch.tensor([root], dtype=torch.int32, device=dev)
    for r in range(2):
        say(f"chained round {r} S={S}")
        rnd = DraftTreeRound(shape, S, dev)
        rnd.root_token.copy_(rnd_tok)
        x = synth.deep_logits(w.L, w.V, g).astype(np.float32)
        # Targets that follow the tree for a step or two.
        lp_ref, tok_ref = st.topk(x, w.K)
        tree = ot.build_tree(lp_ref.astype(np.float32), tok_ref, w.B, root)
        t_np = g.integers(0, w.V, size=tree.N).astype(np.int32)
        kids = np.flatnonzero(tree.parent == 0)
        t_np[0] = tree.token[kids[0]]
        rnd.topk(torch.from_numpy(x).to(dev))
        rnd.build()
        rnd.walk(torch.from_numpy(t_np).to(dev))
        rnd.compact(kv, S)
        rnd_tok = rnd.next_bonus.clone()  # device to device: the next root
        torch.cuda.synchronize()
        np.testing.assert_array_equal(rnd.node_token.cpu().numpy(), tree.token)
        acc, a, bonus = oc.accept_walk(tree.parent, tree.token, t_np, w.L)
        np.testing.assert_array_equal(rnd.acc.cpu().numpy(), acc)
        assert int(rnd.next_bonus.cpu()[0]) == bonus
        kv_ref = oc.kv_compact(kv_ref, S, acc, a)
        np.testing.assert_array_equal(kv.view(torch.int16).cpu().numpy().view(np.uint16), kv_ref)
        root = bonus
        S = S + a + 1  # the root row and the accepted rows stay in the cache
