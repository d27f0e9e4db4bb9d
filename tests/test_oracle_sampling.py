"""Pins for the oracle's temperature > 0 verification (CPU only).

The walk at temperature > 0: "DDTree Deep Dive" page, section 6 (the target
samples at each node, the walk descends into the matching child, the first
unmatched token is the bonus; the target's distribution is kept exactly).
The generator is pinned to the published known-answer vectors of
Philox4x32-10; the sampler to the distribution it must draw from (chi-square
against softmax(x / T)); the walk to the target's own sequence probabilities
on a small tree, enumerated independently."""
import numpy as np
import pytest
from scipy import stats

from block_diffusion_draft_ddtree_amd import synth
from oracle import commit as oc
from oracle import sampling as osm

# Known-answer vectors of Philox4x32-10 distributed with the Random123
# library of Salmon et al. (counter, key) -> output.
PHILOX_KAT = [
    ((0x00000000, 0x00000000, 0x00000000, 0x00000000), (0x00000000, 0x00000000),
     (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF), (0xFFFFFFFF, 0xFFFFFFFF),
     (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


@pytest.mark.parametrize("ctr,key,want", PHILOX_KAT)
def test_philox_known_answers(ctr, key, want):
    got = osm.philox4x32_10(np.array(ctr, dtype=np.uint32), np.array(key, dtype=np.uint32))
    assert tuple(int(w) for w in got) == want


def test_philox_vectorised_equals_single_calls():
    g = np.random.default_rng(5)
    ctr = g.integers(0, 1 << 32, size=(50, 4), dtype=np.uint64).astype(np.uint32)
    key = g.integers(0, 1 << 32, size=2, dtype=np.uint64).astype(np.uint32)
    batch = osm.philox4x32_10(ctr, key)
    for i in range(50):
        np.testing.assert_array_equal(batch[i], osm.philox4x32_10(ctr[i], key))


def test_uniform_range_and_fp32_exactness():
    w = np.array([0, 511, 512, 0x7FFFFFFF, 0xFFFFFFFF], dtype=np.uint32)
    u = osm.uniform_from_word(w)
    assert u[0] == 2.0 ** -24 and u[1] == 2.0 ** -24  # the low 9 bits are dropped
    assert u[2] == 3 * 2.0 ** -24
    assert u[3] == 0.5 - 2.0 ** -24
    assert u[-1] == 1.0 - 2.0 ** -24
    every = osm.uniform_from_word(np.arange(0, 1 << 32, 1 << 9, dtype=np.uint64).astype(np.uint32))
    np.testing.assert_array_equal(every.astype(np.float32).astype(np.float64), every)
    assert np.all(np.diff(every) > 0)


def test_uniforms_layout():
    """Token v of node n reads word v & 3 of the block at counter
    (v >> 2, n, offset lo, offset hi)."""
    seed, offset = 0x1234_5678_9ABC_DEF0, (7 << 32) + 3
    u = osm.uniforms([2, 9], 10, seed, offset)
    for row, n in enumerate((2, 9)):
        for v in range(10):
            blk = osm.philox4x32_10(
                np.array([v >> 2, n, offset & 0xFFFFFFFF, offset >> 32], dtype=np.uint32),
                np.array([seed & 0xFFFFFFFF, seed >> 32], dtype=np.uint32))
            assert u[row, v] == osm.uniform_from_word(blk[v & 3])


def test_uniform_moments():
    u = osm.uniforms(np.arange(64), 4096, 99, 0).reshape(-1)
    assert abs(u.mean() - 0.5) < 2e-3
    assert abs(u.var() - 1.0 / 12.0) < 1e-3
    counts = np.bincount(np.minimum((u * 32).astype(int), 31), minlength=32)
    assert stats.chisquare(counts).pvalue > 1e-4


@pytest.mark.parametrize("T", [0.5, 1.0, 2.0])
def test_gumbel_max_draws_softmax(T):
    """Many independent draws of one small row (one node per draw) follow
    softmax(x / T)."""
    x = np.array([1.0, 0.0, -0.5, 2.0, 0.25], dtype=np.float32)
    draws = 40000
    rows = np.repeat(x[None, :], draws, axis=0)
    got = osm.target_sample(rows, T, seed=2024, offset=11)
    p = np.exp(x.astype(np.float64) / T)
    p /= p.sum()
    counts = np.bincount(got, minlength=5)
    assert stats.chisquare(counts, p * draws).pvalue > 1e-4
    # A transposed or unscaled reading would be far off: T = 2 halves the
    # spread, so the top token's share moves by several sigma.
    assert abs(counts[3] / draws - p[3]) < 5 * np.sqrt(p[3] * (1 - p[3]) / draws)


def test_masked_tokens_never_drawn():
    x = np.array([[0.0, -np.inf, 1.0, -np.inf]] * 2000, dtype=np.float32)
    got = osm.target_sample(x, 1.0, 3, 0)
    assert set(np.unique(got).tolist()) <= {0, 2}


def test_low_temperature_is_the_argmax():
    """With a top-2 gap of at least 0.05 and T = 1e-3 the scaled gap (>= 50)
    exceeds the whole range of the Gumbel noise of the 23-bit uniforms
    (-ln(-ln u) lies in [-2.82, 16.7]), so the sample is the argmax."""
    g = synth.rng("test", 700, 0)
    x = np.round(g.standard_normal((40, 3000)) * 8) / 8  # steps of 0.125
    x = x.astype(np.float32)
    top2 = np.sort(x, axis=1)[:, -2:]
    keep = top2[:, 1] - top2[:, 0] >= 0.05
    assert keep.sum() >= 10
    got = osm.target_sample(x[keep], 1e-3, 77, 5)
    np.testing.assert_array_equal(got, oc.target_argmax(x[keep]))


def test_counters_separate_nodes_seeds_and_offsets():
    base = osm.uniforms([0, 1], 64, 1, 0)
    assert not np.array_equal(base[0], base[1])
    assert not np.array_equal(base, osm.uniforms([0, 1], 64, 2, 0))
    assert not np.array_equal(base, osm.uniforms([0, 1], 64, 1, 1))
    assert not np.array_equal(base, osm.uniforms([0, 1], 64, 1, 1 << 32))


def test_rejects_bad_inputs():
    ok = np.zeros((2, 3), dtype=np.float32)
    for bad in (np.array([[0.0, np.nan]], np.float32), np.array([[0.0, np.inf]], np.float32),
                np.array([[-np.inf, -np.inf]], np.float32)):
        with pytest.raises(ValueError):
            osm.target_sample(bad, 1.0, 0, 0)
    for T in (0.0, -1.0, np.inf, np.nan):
        with pytest.raises(ValueError):
            osm.target_sample(ok, T, 0, 0)


# --- the walk at temperature > 0 keeps the target's distribution -----------

def _tree():
    """Root (bonus 9) with children carrying tokens 0 and 1; node 1 (token 0)
    has children with tokens 2 and 3; node 3 (token 2) has a child with
    token 1. V = 4, L = 3."""
    parent = np.array([-1, 0, 0, 1, 1, 3], dtype=np.int32)
    token = np.array([9, 0, 1, 2, 3, 1], dtype=np.int32)
    return parent, token


def _exact_sequences(parent, token, probs):
    """Enumerate what the target itself would emit until it leaves the tree:
    at node u draw t with probability probs[u][t]; if a child of u carries t
    continue there, else stop with t as the last token."""
    kids = {}
    for n in range(1, len(parent)):
        kids.setdefault(int(parent[n]), {})[int(token[n])] = n
    out = {}

    def rec(u, prefix, pr):
        for t in range(probs.shape[1]):
            q = pr * probs[u, t]
            c = kids.get(u, {}).get(t)
            if c is None:
                out[prefix + (t,)] = out.get(prefix + (t,), 0.0) + q
            else:
                rec(c, prefix + (t,), q)

    rec(0, (), 1.0)
    return out


@pytest.mark.parametrize("T", [0.7, 1.0])
def test_sampled_walk_emits_target_sequences(T):
    parent, token = _tree()
    g = np.random.default_rng(31)
    x = (g.standard_normal((6, 4)) * 1.2).astype(np.float32)
    p = np.exp(x.astype(np.float64) / T)
    p /= p.sum(axis=1, keepdims=True)
    exact = _exact_sequences(parent, token, p)
    assert abs(sum(exact.values()) - 1.0) < 1e-12
    draws = 6000
    seen = {}
    for r in range(draws):
        tgt = osm.target_sample(x, T, seed=555, offset=r)
        acc, a, bonus = oc.accept_walk(parent, token, tgt, 3)
        seq = tuple(int(token[acc[k]]) for k in range(1, a + 1)) + (int(bonus),)
        seen[seq] = seen.get(seq, 0) + 1
    assert set(seen) <= set(exact)
    keys = sorted(exact)
    obs = np.array([seen.get(k, 0) for k in keys], dtype=np.float64)
    exp = np.array([exact[k] for k in keys]) * draws
    # Pool the rare sequences so that every expected count is >= 5.
    rare = exp < 5
    if rare.any():
        obs = np.append(obs[~rare], obs[rare].sum())
        exp = np.append(exp[~rare], exp[rare].sum())
    assert stats.chisquare(obs, exp).pvalue > 1e-4
