"""GPU parity: ddtree_budget_select against the oracle's cost-aware budget.

Expected acceptance per budget is Proposition 1 of the "DDTree Deep Dive"
page (section 2) over the first B pops; the budget maximises expected tokens
per unit of round time (the autobench Qwen3-Coder-30B page's budget
optimum). Both sides sum in fp64, in different orders, so the budget is
compared exactly unless the oracle's best objective and the objective of the
device's pick differ by less than 1e-12 relative, where either is right."""
import numpy as np
import pytest
import torch

from block_diffusion_draft_ddtree_amd import binding as bd
from block_diffusion_draft_ddtree_amd import synth
from oracle import budget as ob

from gpu_helpers import say

pytestmark = pytest.mark.gpu

# Round-time model fitted to the autobench page's two DDTree rows (budget 64:
# 3.22 tokens per step at 20.75 tok/s; budget 256: 3.69 at 17.32 tok/s), in
# seconds: t(B) = t0 + t1 (B + 1).
_T1 = (3.69 / 17.32 - 3.22 / 20.75) / (257 - 65)
_T0 = 3.22 / 20.75 - _T1 * 65


def _table(g, B_max):
    return np.concatenate([[0.0], -np.sort(g.exponential(1.5, size=B_max))]).astype(np.float32)


def _check(score, B_max, B_min, t0, t1):
    say(f"budget B_max={B_max} B_min={B_min} t0={t0:.4g} t1={t1:.4g}")
    b, e = bd.ddtree_budget_select(torch.from_numpy(score).cuda(), B_max, t0, t1, B_min)
    got_b, got_e = int(b.cpu()[0]), e.cpu().numpy()
    want_e = ob.expected_accept(score[: B_max + 1])
    np.testing.assert_allclose(got_e, want_e, rtol=2e-7, atol=1e-30)
    obj = ob.budget_objective(score[: B_max + 1], t0, t1)
    want_b = ob.select_budget(score[: B_max + 1], t0, t1, B_min, B_max)
    if got_b != want_b:
        assert B_min <= got_b <= B_max
        assert obj[got_b] >= obj[want_b] * (1 - 1e-12), (got_b, want_b)
    return got_b


@pytest.mark.parametrize("B_max", [1, 2, 63, 64, 65, 257, 1000, 1024])
def test_random_tables(B_max):
    g = synth.rng("test", 690, B_max)
    for _ in range(6):
        score = _table(g, B_max)
        t0 = float(g.uniform(0.0, 2.0))
        t1 = float(10 ** g.uniform(-4, -0.5))
        B_min = int(g.integers(0, B_max + 1)) if g.uniform() < 0.3 else 1
        _check(score, B_max, B_min, t0, t1)


def test_cost_model_from_the_pages_numbers():
    g = synth.rng("test", 691, 0)
    score = _table(g, 1024)
    b = _check(score, 1024, 1, _T0, _T1)
    assert 1 <= b <= 1024


def test_exact_tie_picks_the_smaller_budget():
    score = np.zeros(9, dtype=np.float32)  # eight certain pops
    assert _check(score, 8, 1, 0.0, 1.0) == 1
    assert _check(score, 8, 3, 0.0, 1.0) == 3


def test_extremes_and_no_expected_output():
    g = synth.rng("test", 692, 0)
    score = _table(g, 300)
    assert _check(score, 300, 1, 1.0, 0.0) == 300  # free verification
    say("budget without expected output")
    b = torch.empty(1, dtype=torch.int32, device="cuda")
    lib = bd.lib()
    st = lib.ddtree_budget_select(torch.from_numpy(score).cuda().data_ptr(), 300, 1, 1.0, 0.05,
                                  None, b.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == 0
    assert int(b.cpu()[0]) == ob.select_budget(score, 1.0, 0.05, 1, 300)


def test_on_device_build_scores():
    """ddtree_topk -> ddtree_build (budget 256) -> ddtree_budget_select on
    the device, against the oracle on the downloaded scores."""
    w = synth.WORKLOADS["coder30b_b64_deep"]
    lg = synth.drafter_logits(w, 0)
    L, K, B_max = w.L, 64, 256
    say("budget on device build scores")
    logits = torch.from_numpy(lg.x).cuda()
    logp = torch.empty((L, K), dtype=torch.float32, device="cuda")
    token = torch.empty((L, K), dtype=torch.int32, device="cuda")
    ws = bd.workspace(bd.ddtree_topk_workspace_bytes(L, w.V, K), "cuda")
    bd.ddtree_topk(logits, K, logp, token, ws)
    N = B_max + 1
    W = (N + 31) // 32
    i32 = dict(dtype=torch.int32, device="cuda")
    root = torch.zeros(1, **i32)
    parent, depth, tok = torch.empty(N, **i32), torch.empty(N, **i32), torch.empty(N, **i32)
    score = torch.empty(N, dtype=torch.float32, device="cuda")
    anc = torch.empty((N, W), **i32)
    bd.ddtree_build(logp, token, B_max, root, W, parent, depth, tok, score, anc)
    b, e = bd.ddtree_budget_select(score, B_max, _T0, _T1, 1)
    s_np = score.cpu().numpy()
    np.testing.assert_allclose(e.cpu().numpy(), ob.expected_accept(s_np), rtol=2e-7, atol=1e-30)
    assert int(b.cpu()[0]) == ob.select_budget(s_np, _T0, _T1, 1, B_max)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_pruned_round_equals_the_budget_tree(seed):
    """The round consumes the cost-aware budget on the device: build with
    budget 64, ddtree_budget_select, ddtree_tree_prune, then the attention
    and the walk on the pruned tree. The kept nodes' parents and mask rows,
    their attention rows and the walk (with a target planted along the
    deepest path of the full tree, so that it runs past the budget) equal
    the oracle's on a build with the selected budget."""
    from oracle import attention as oa
    from oracle import commit as oc
    from oracle import softmax_topk as st
    from oracle import tree as ot

    from gpu_helpers import assert_attn_close, down, down_bf16_f32, up, up_bf16

    g = synth.rng("test", 693, seed)
    L, V, K, B_max = 8, 512, 8, 64
    N = B_max + 1
    W = (N + 31) // 32
    x = synth.deep_logits(L, V, g).astype(np.float32)
    root = int(g.integers(0, V))
    say(f"pruned round seed={seed}")
    i32 = dict(dtype=torch.int32, device="cuda")
    logp = torch.empty((L, K), dtype=torch.float32, device="cuda")
    token = torch.empty((L, K), **i32)
    bd.ddtree_topk(up(x), K, logp, token)
    lp_ref, tok_ref = st.topk(x, K)
    np.testing.assert_array_equal(down(token), tok_ref)
    # The oracle builds from the device's [L, K] table (the tree parity rule).
    full = ot.build_tree(down(logp), down(token), B_max, root)
    # A time model whose optimum lies well inside (0, B_max).
    for t1 in (0.02, 0.05, 0.1, 0.2, 0.5, 1.0):
        want_b = ob.select_budget(full.score, 1.0, t1, 1, B_max)
        if 2 <= want_b <= B_max - 8:
            break
    assert 2 <= want_b <= B_max - 8
    parent, depth, ntok = torch.empty(N, **i32), torch.empty(N, **i32), torch.empty(N, **i32)
    score = torch.empty(N, dtype=torch.float32, device="cuda")
    anc = torch.empty((N, W), **i32)
    bd.ddtree_build(logp, token, B_max, up(np.array([root], np.int32)), W, parent, depth, ntok,
                    score, anc)
    b, _ = bd.ddtree_budget_select(score, B_max, 1.0, t1, 1)
    bd.ddtree_tree_prune(b, parent, anc)
    Bp = int(down(b)[0])
    assert Bp == want_b
    Np = Bp + 1
    kept = ot.build_tree(down(logp), down(token), Bp, root, mask_words=W)
    got_parent = down(parent)
    np.testing.assert_array_equal(got_parent[:Np], kept.parent)
    assert (got_parent[Np:] == -1).all()
    got_anc = down(anc).view(np.uint32)
    np.testing.assert_array_equal(got_anc[:Np], kept.anc)
    assert (got_anc[Np:] == 0).all()
    # Attention of the pruned tree: the kept rows against the oracle on the
    # budget-B' tree (its tree rows are the first Np of the cache's).
    Hq, Hkv, D, S = 8, 2, 128, 200
    q_bits, q = synth.normal_bf16(g, (N, Hq, D))
    kv_bits, kv = synth.normal_bf16(g, (2, Hkv, S + N, D))
    kvd = up_bf16(kv_bits)
    out = bd.ddtree_tree_attn(up_bf16(q_bits), kvd[0], kvd[1], S, anc)
    ref = oa.tree_attention(q[:Np], kv[0], kv[1], S, kept.anc)
    assert_attn_close(down_bf16_f32(out)[:Np], ref, f"pruned tree, {Np} nodes")
    # The walk: a target planted along the full tree's path to its last pop,
    # which the budget drops.
    path = [N - 1]
    while path[-1] != 0:
        path.append(int(full.parent[path[-1]]))
    tgt = synth.target_argmax_planted(full.parent, full.token, path[::-1], V, g)
    acc, n_acc, bonus = bd.ddtree_accept_walk(parent, ntok, L, up(tgt))
    want_acc, want_a, want_bonus = oc.accept_walk(kept.parent, kept.token, tgt[:Np], L)
    assert int(down(n_acc)[0]) == want_a
    np.testing.assert_array_equal(down(acc)[: want_a + 1], want_acc[: want_a + 1])
    assert int(down(bonus)[0]) == want_bonus
    assert want_a < int(full.depth[N - 1])  # the budget cut the planted path
