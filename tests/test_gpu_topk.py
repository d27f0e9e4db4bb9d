"""GPU parity: ddtree_topk against the oracle's log-softmax and top-K.

Token ids must match exactly, in rank order (ties by smaller id); log-probs
within 1e-5 absolute of the fp64 oracle."""
import numpy as np
import pytest
import torch

from block_diffusion_draft_ddtree_amd import binding as bd
from block_diffusion_draft_ddtree_amd import synth
from oracle import softmax_topk as st

from gpu_helpers import LOGP_ATOL, down, say, up

pytestmark = pytest.mark.gpu


def _check(x: np.ndarray, K: int, stride: int | None = None, twice: bool = True,
           lp_atol: float = LOGP_ATOL):
    L, V = x.shape
    if stride is not None and stride > V:
        buf = np.full((L, stride), 1e30, dtype=np.float32)  # poison beyond V
        buf[:, :V] = x
        dev = up(buf)[:, :V]
    else:
        dev = up(x)
    say(f"topk L={L} V={V} K={K} stride={stride}")
    lp, tok = bd.ddtree_topk(dev, K)
    lp_g, tok_g = down(lp), down(tok)
    ref_lp, ref_tok = st.topk(x, K)
    np.testing.assert_array_equal(tok_g, ref_tok)
    assert np.abs(lp_g.astype(np.float64) - ref_lp).max() <= lp_atol
    if twice:
        lp2, tok2 = bd.ddtree_topk(dev, K)
        np.testing.assert_array_equal(down(tok2), tok_g)
        np.testing.assert_array_equal(down(lp2).view(np.uint32), lp_g.view(np.uint32))
    return lp_g, tok_g


def test_tiny_workload():
    w = synth.TINY
    _check(synth.drafter_logits(w).x, w.K)


@pytest.mark.parametrize("name,K", [("qwen3_8b", 64), ("coder30b_b256", 256), ("sweep_b16", 16),
                                    ("sweep_b512", 512)])
def test_full_vocab_workloads(name, K):
    w = synth.WORKLOADS[name]
    _check(synth.drafter_logits(w).x, K)


def test_ties_smaller_id_first():
    g = synth.rng("test", 500, 0)
    x = synth.tie_logits(3, 20000, g, levels=4)
    _check(x, 100)
    _check(x, 1024)


def test_ties_beyond_lds():
    """Rows where more than 16 K candidates share the K-th largest's first
    digit bucket (a constant row; a row whose top level holds 30000 equal
    values): the merge then selects over the candidates in global memory."""
    g = synth.rng("test", 504, 0)
    x = np.zeros((2, 151936), dtype=np.float32)
    x[1, :] = -1.0
    x[1, g.choice(151936, 30000, replace=False)] = 2.5
    _check(x, 1024)


def test_many_survivors_small_k():
    """K <= 64 (the merge counts the digit histogram only on demand) with
    more survivors than it ranks all against all: a tie-heavy row (the
    survivors fit LDS), and 64 chunks of 4096 that each hold 300 values tied
    at the row maximum (19200 survivors, more than LDS holds: a counting
    pass over the candidates); also K = 128 on the latter."""
    g = synth.rng("test", 505, 0)
    _check(synth.tie_logits(2, 20000, g, levels=3), 64)
    V = 64 * 4096
    x = (-1.0 - g.random((2, V))).astype(np.float32)
    for c in range(64):
        x[:, c * 4096 + g.choice(4096, 300, replace=False)] = 3.0
    _check(x, 64)
    _check(x, 128)


def test_signed_zero_and_few_values():
    x = np.zeros((2, 5000), dtype=np.float32)
    x[0, ::3] = -0.0
    x[1, 7] = 1.0
    _check(x, 37)


@pytest.mark.parametrize("V,K", [(1, 1), (7, 7), (300, 300), (4097, 1), (4096, 4096 // 4),
                                 (8193, 1024), (151936, 1)])
def test_edge_shapes(V, K):
    g = synth.rng("test", 501, V)
    x = (2.0 * g.standard_normal((3, V))).astype(np.float32)
    _check(x, min(K, V))


def test_row_stride_and_max_rows():
    g = synth.rng("test", 502, 0)
    x = (1.5 * g.standard_normal((32, 9000))).astype(np.float32)
    _check(x, 200, stride=9216)


def test_wide_spread_logits():
    """Values spread over many octaves exercise the far bins of the first digit.
    Log-probs reach about -3000 here, where one fp32 ulp is 2.4e-4, so the
    log-prob bound is 4 ulp of the largest magnitude instead of 1e-5."""
    g = synth.rng("test", 503, 0)
    x = (g.standard_normal((4, 50000)) * np.exp(g.uniform(-3, 6, (4, 50000)))).astype(np.float32)
    ref, _ = st.topk(x, 700)
    tol = 4 * float(np.spacing(np.float32(np.abs(ref).max())))
    _check(x, 700, lp_atol=tol)


@pytest.mark.parametrize("K", [1, 2, 3, 16, 63, 64, 65, 128, 129, 256, 257, 512, 1000, 1024])
def test_bounds_every_k(K):
    """Each K takes its own per-thread order statistic q (1, 2, 4, 8, 16) and
    wave ranks r for the chunk bound and for the merge's row threshold; four
    rows of the peaked and of the confident drafter families."""
    xs = [synth.drafter_logits(synth.WORKLOADS[name]).x[:2] for name in ("coder30b_b64", "sweep_b16")]
    _check(np.concatenate(xs), K, twice=False)


@pytest.mark.parametrize("K", [16, 64, 200, 1024])
def test_bounds_top_values_bunched(K):
    """The largest values of every 4096-logit chunk sit in the 16-value slices
    of the fewest threads that can hold them (row 0), in the lanes of one wave
    (row 1), or as exact ties in a few threads (row 2): the per-thread and
    per-wave order statistics behind the bounds see them bunched together."""
    g = synth.rng("test", 505, K)
    L, V = 3, 40000
    x = g.standard_normal((L, V)).astype(np.float32)
    nthreads = -(-K // 16)
    for base in range(0, V, 4096):
        n = min(4096, V - base)
        for t in range(nthreads):
            pos = base + t + 256 * np.arange(16)
            pos = pos[pos < base + n]
            x[0, pos] = 10.0 + g.standard_normal(pos.size).astype(np.float32)
            x[2, pos] = 10.0
        steps = -(-K // 64)
        pos = base + 128 + np.arange(64)[None, :] + 256 * np.arange(steps)[:, None]
        pos = pos[pos < base + n]
        x[1, pos] = 10.0 + g.standard_normal(pos.size).astype(np.float32)
    _check(x, K)


def _sweep_case(i: int):
    """Seeded shape and value mix for case i: L in 1..20, V log-uniform in
    1..160000, K log-uniform in 1..min(V, 1024), a padded row stride in a
    third of the cases; values normal at scale 0.5..4, with boosted peaks,
    rounded to integers (heavy ties) or uniform."""
    g = synth.rng("test", 600, i)
    L = int(g.integers(1, 21))
    V = int(np.exp(g.uniform(0, np.log(160000))))
    K = max(1, min(V, 1024, int(np.exp(g.uniform(0, np.log(1025))))))
    kind = i % 4
    x = g.standard_normal((L, V)) * g.uniform(0.5, 4.0)
    if kind == 1:
        for r in range(L):
            x[r, g.integers(0, V, size=min(V, 3))] += g.uniform(5, 12)
    elif kind == 2:
        x = np.round(x)
    elif kind == 3:
        x = g.uniform(-3, 3, (L, V))
    stride = V + int(g.integers(1, 300)) if i % 3 == 0 else None
    return x.astype(np.float32), K, stride


@pytest.mark.parametrize("i", range(24))
def test_seeded_shape_sweep(i):
    x, K, stride = _sweep_case(i)
    _check(x, K, stride=stride, twice=False)
