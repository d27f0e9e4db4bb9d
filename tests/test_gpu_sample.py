"""GPU parity: ddtree_target_sample against the oracle's Gumbel-max draw.

Temperature > 0 verification ("DDTree Deep Dive", section 6): the target
samples its token at every tree node and the walk follows the samples. The
device forms the Gumbel key in fp32 with its own logarithms and the oracle in
fp64 from the same Philox4x32-10 words, so the picks are compared exactly
wherever the oracle's best key leads the runner-up by more than the device's
rounding bound, and elsewhere the device's pick must be one of the tokens
within that bound of the best (in practice every row here is exact; the test
counts them). Rows are placed at every alignment so that each residue of a
row's first vector start modulo 4 (the Philox block offset) is exercised."""
import numpy as np
import pytest
import torch
from scipy import stats

from block_diffusion_draft_ddtree_amd import binding as bd
from block_diffusion_draft_ddtree_amd import synth
from oracle import commit as oc
from oracle import sampling as osm
from oracle import softmax_topk as st
from oracle import tree as ot

from gpu_helpers import say

pytestmark = pytest.mark.gpu

_WS = {}


def _ws():
    if "ws" not in _WS:
        _WS["ws"] = torch.full((1 << 20,), 255, dtype=torch.uint8, device="cuda")
    return _WS["ws"]


def _tol(x, T):
    """Bound on |device key - exact key| in natural-log units: fp32 rounding
    of log2(e)/T, of x * c and of the sum, plus the two hardware log2 calls
    (about one ulp each), with a tenfold margin."""
    xm = float(np.max(np.abs(x[np.isfinite(x)]))) if np.isfinite(x).any() else 0.0
    return 1e-4 + 1e-6 * xm / T


def _check_rows(got, x32, T, seed, offset):
    keys = osm.sample_keys(x32, T, seed, offset)
    tol = _tol(x32, T)
    exact = 0
    for n in range(x32.shape[0]):
        cand = osm.near_tie_candidates(keys[n], tol)
        assert int(got[n]) in cand.tolist(), (n, int(got[n]), cand[:8], keys[n].max())
        exact += int(cand.size == 1)
    return exact


def _run(x32, dtype, T, seed, offset, stride=None):
    N, V = x32.shape
    stride = V if stride is None else stride
    say(f"target_sample N={N} V={V} stride={stride} dtype={dtype} T={T} seed={seed} off={offset}")
    buf = torch.zeros((N, stride), dtype=torch.float32)
    buf[:, :V] = torch.from_numpy(x32)
    dev = buf.to(dtype).cuda()
    return bd.ddtree_target_sample(dev[:, :V], T, seed, offset, ws=_ws()).cpu().numpy()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("T", [1.0, 0.7])
def test_workload_shapes(dtype, T):
    g = synth.rng("test", 680, int(dtype == torch.bfloat16) * 2 + int(T == 1.0))
    seed, offset = 0x9E37_79B9_7F4A_7C15, (5 << 32) + 17  # both words of each in use
    for N in (1, 17, 65):
        _, x = synth.target_logits(g, N, 151936, peaks=g.integers(0, 151936, size=N))
        got = _run(x, dtype, T, seed, offset + N)
        assert _check_rows(got, x, T, seed, offset + N) >= N - 1


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("V", [1, 3, 5, 7, 9, 17, 1000, 4099])
def test_alignments_and_ragged_rows(dtype, V):
    g = synth.rng("test", 681, V)
    N = 9
    x = (g.standard_normal((N, V)) * 1.5).astype(np.float32)
    x = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x))  # exact in both dtypes
    for stride in range(V, V + 8):  # every row start residue
        got = _run(x, dtype, 1.0, 11, stride)
        _check_rows(got, x, 1.0, 11, stride)


def test_low_temperature_matches_argmax_kernel():
    g = synth.rng("test", 682, 0)
    _, x = synth.target_logits(g, 65, 151936, peaks=g.integers(0, 151936, size=65), boost=30.0)
    say("target_sample T=1e-3 vs target_argmax")
    dev = torch.from_numpy(x).to(torch.bfloat16).cuda()
    s = bd.ddtree_target_sample(dev, 1e-3, 1, 2, ws=_ws()).cpu().numpy()
    a = bd.ddtree_target_argmax(dev, ws=_ws()).cpu().numpy()
    np.testing.assert_array_equal(s, a)
    np.testing.assert_array_equal(a, oc.target_argmax(x))


def test_masked_tokens_never_drawn():
    V = 5000
    x = np.full((64, V), -np.inf, dtype=np.float32)
    allowed = np.array([3, 700, 701, 4999])
    x[:, allowed] = np.array([0.0, 1.0, -1.0, 0.5], dtype=np.float32)
    got = _run(x, torch.bfloat16, 1.0, 5, 6)
    assert set(got.tolist()) <= set(allowed.tolist())
    _check_rows(got, x, 1.0, 5, 6)


def test_draws_follow_softmax():
    """20 calls x 1025 nodes of one 5-token row: chi-square against
    softmax(x / T) on the device's draws alone."""
    x = np.array([1.0, 0.0, -0.5, 2.0, 0.25], dtype=np.float32)
    T = 1.3
    dev = torch.from_numpy(np.repeat(x[None], 1025, axis=0)).cuda()
    say("target_sample draw distribution")
    counts = np.zeros(5)
    for r in range(20):
        counts += np.bincount(bd.ddtree_target_sample(dev, T, 8, r, ws=_ws()).cpu().numpy(),
                              minlength=5)
    p = np.exp(x.astype(np.float64) / T)
    p /= p.sum()
    assert stats.chisquare(counts, p * counts.sum()).pvalue > 1e-4


def test_sampled_walk_on_device():
    """Device sample feeding the device walk equals the oracle's sample
    feeding the oracle's walk, on deep trees."""
    for seed in range(3):
        g = synth.rng("test", 683, seed)
        L, Vd, K, B = 6, 50, 4, 40
        lp, tok = st.topk(synth.deep_logits(L, Vd, g), K)
        tree = ot.build_tree(lp.astype(np.float32), tok, B, root_token=1)
        parent, token = tree.parent, tree.token
        N = len(parent)
        # Target rows that favour each node's likeliest child, so walks go deep.
        x = (g.standard_normal((N, Vd)) * 0.5).astype(np.float32)
        for n in range(1, N):
            x[parent[n], token[n]] += 5.0
        say(f"sampled walk seed={seed} N={N}")
        s_dev = bd.ddtree_target_sample(torch.from_numpy(x).cuda(), 1.0, 40 + seed, 0, ws=_ws())
        acc, n_acc, bonus = bd.ddtree_accept_walk(
            torch.from_numpy(parent.astype(np.int32)).cuda(),
            torch.from_numpy(token.astype(np.int32)).cuda(), L, s_dev)
        s_ref = osm.target_sample(x, 1.0, 40 + seed, 0)
        keys = osm.sample_keys(x, 1.0, 40 + seed, 0)
        srt = np.sort(keys, axis=1)
        assert np.all(srt[:, -1] - srt[:, -2] > _tol(x, 1.0)), "a near tie; pick another seed"
        np.testing.assert_array_equal(s_dev.cpu().numpy(), s_ref)
        acc_r, a_r, bonus_r = oc.accept_walk(parent, token, s_ref, L)
        np.testing.assert_array_equal(acc.cpu().numpy(), acc_r)
        assert int(n_acc.cpu()[0]) == a_r and int(bonus.cpu()[0]) == bonus_r


def test_max_rows_sampled():
    g = synth.rng("test", 684, 0)
    N, V = 1025, 151936
    bits, _ = synth.target_logits(g, N, V, peaks=g.integers(0, V, size=N), boost=2.0)
    say(f"target_sample N={N} V={V} bf16 sampled rows")
    dev = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    got = bd.ddtree_target_sample(dev, 1.0, 123456789, 1 << 40, ws=_ws()).cpu().numpy()
    rows = np.sort(g.choice(N, size=24, replace=False))
    x = synth.bf16_bits_to_f32(bits[rows])
    # The node index in the counter is the row's index in the full call.
    for i, n in enumerate(rows):
        u = osm.uniforms([n], V, 123456789, 1 << 40)[0]
        key = x[i].astype(np.float64) - np.log(-np.log(u))
        assert int(got[n]) in osm.near_tie_candidates(key, _tol(x, 1.0)).tolist()
