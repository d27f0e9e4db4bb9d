"""Oracle: verification at temperature > 0 -- the target's sampled token per
tree node, and the counter-based random numbers the sampling draws.

Test infrastructure only (see the package docstring).

Sources
-------
* "DDTree Deep Dive" (zhichai.net), section 6: at each node of the walk the
  target samples (or, greedy, takes the argmax of) its next token, the walk
  descends into the child holding that token, and the first token with no
  matching child becomes the bonus; at temperature > 0 the usual
  speculative-sampling rules keep the output distributed exactly as the
  target's.
* Same page, section 9: the tree helps more at temperature 1.0 than greedy.
* Philox4x32-10: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw,
  "Parallel random numbers: as easy as 1, 2, 3", SC 2011 (the Philox
  round, its two multipliers and the Weyl key schedule).
* Gumbel-max: the index of the largest of (log-weight + independent standard
  Gumbel noise) is distributed as the normalised weights (E. J. Gumbel,
  1954; the "Gumbel-max trick").

Readings where the pages are silent
-----------------------------------
* The tree is a fixed function of the drafter's output, so each child is a
  point-mass draft. The standard rule (accept a draft token c with
  probability min(1, p(c) / 1) = p(c), otherwise draw from the residual p
  with c removed and renormalised, child after child) emits every token t
  with probability exactly p(t), and descends into a child precisely when
  the emitted token is that child's. So the walk is the greedy walk fed with
  one target sample per node instead of the argmax: ``accept_walk`` of
  ``oracle.commit`` with ``target_sample`` below.
* p at node n is softmax(logits[n] / T), T > 0 (T = 1: the plain target
  distribution).
* Random numbers: one uniform per (node n, token v) from Philox4x32-10 with
  key (seed mod 2^32, seed >> 32) and counter (v >> 2, n, offset mod 2^32,
  offset >> 32); word v & 3 of the output gives
  u = ((word >> 9) + 0.5) * 2^-23, exact in fp32 (an odd multiple of
  2^-24), in [2^-24, 1 - 2^-24].
  ``offset`` advances per round so that rounds draw fresh numbers.
* Decision precision: the key x / T - ln(-ln u) is formed here in fp64 from
  the exact u and the fp32 (or bf16-widened) logits. A device forms it in
  fp32 with its own logarithms, so the two can differ only where two tokens'
  keys lie within that rounding of each other; the parity tests compare the
  pick exactly wherever the oracle's margin exceeds the device's error
  bound, and elsewhere check that the device's pick is one of the tied
  candidates (``near_tie_candidates``).
"""
from __future__ import annotations

import numpy as np

PHILOX_M0 = np.uint64(0xD2511F53)
PHILOX_M1 = np.uint64(0xCD9E8D57)
PHILOX_W0 = np.uint64(0x9E3779B9)
PHILOX_W1 = np.uint64(0xBB67AE85)
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(ctr, key) -> np.ndarray:
    """Philox4x32 with 10 rounds. ctr: uint32 [..., 4]; key: uint32 [..., 2]
    (broadcast against ctr). Returns uint32 [..., 4].

    One round: the products M0 * c0 and M1 * c2 split into high and low
    words; the new counter is (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2),
    hi(M0 c0) ^ c3 ^ k1, lo(M0 c0)). The key gains (W0, W1), mod 2^32,
    between rounds."""
    c = np.array(ctr, dtype=np.uint32)
    k = np.array(key, dtype=np.uint32)
    c0, c1, c2, c3 = (c[..., i].astype(np.uint64) for i in range(4))
    k0 = np.broadcast_to(k[..., 0], c[..., 0].shape).astype(np.uint64)
    k1 = np.broadcast_to(k[..., 1], c[..., 0].shape).astype(np.uint64)
    for r in range(10):
        if r > 0:
            k0 = (k0 + PHILOX_W0) & _MASK32
            k1 = (k1 + PHILOX_W1) & _MASK32
        p0 = PHILOX_M0 * c0  # < 2^64: exact in uint64
        p1 = PHILOX_M1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        c0 = hi1 ^ c1 ^ k0
        c1 = lo1
        c2 = hi0 ^ c3 ^ k1
        c3 = lo0
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def uniform_from_word(word) -> np.ndarray:
    """The top 23 bits of a 32-bit word, centred in their cell: fp64 values
    ((word >> 9) + 0.5) / 2^23 = (2 (word >> 9) + 1) / 2^24, each exactly
    representable in fp32 (24 significant bits)."""
    w = np.asarray(word, dtype=np.uint32)
    return ((w >> np.uint32(9)).astype(np.float64) + 0.5) * 2.0 ** -23


def uniforms(nodes, V: int, seed: int, offset: int) -> np.ndarray:
    """fp64 [len(nodes), V]: u for tokens 0..V-1 of each listed node (layout
    in the module doc)."""
    nodes = np.atleast_1d(np.asarray(nodes, dtype=np.uint32))
    G = (V + 3) // 4
    ctr = np.zeros((nodes.size, G, 4), dtype=np.uint32)
    ctr[:, :, 0] = np.arange(G, dtype=np.uint32)[None, :]
    ctr[:, :, 1] = nodes[:, None]
    ctr[:, :, 2] = np.uint32(offset & 0xFFFFFFFF)
    ctr[:, :, 3] = np.uint32((offset >> 32) & 0xFFFFFFFF)
    key = np.array([seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF], dtype=np.uint32)
    words = philox4x32_10(ctr, key).reshape(nodes.size, 4 * G)[:, :V]
    return uniform_from_word(words)


def _check(logits, temperature):
    x = np.asarray(logits, dtype=np.float32)
    if x.ndim != 2 or x.shape[1] < 1:
        raise ValueError("logits must be [N, V] with V >= 1")
    if np.isnan(x).any() or (x == np.inf).any():
        raise ValueError("logits must be finite or -inf")
    if not np.isfinite(x.max(axis=1)).all():
        raise ValueError("every row needs a finite logit")
    if not (np.isfinite(temperature) and temperature > 0):
        raise ValueError("temperature must be finite and > 0")
    return x


def sample_keys(logits, temperature: float, seed: int, offset: int) -> np.ndarray:
    """fp64 [N, V]: x / T + G with G = -ln(-ln u), the Gumbel-perturbed
    scaled logits whose row argmax is the sample (-inf logits stay -inf)."""
    x = _check(logits, temperature)
    N, V = x.shape
    keys = np.empty((N, V), dtype=np.float64)
    step = max(1, (1 << 22) // V)  # rows per block, bounding the temporaries
    for n0 in range(0, N, step):
        rows = np.arange(n0, min(N, n0 + step))
        u = uniforms(rows, V, seed, offset)
        keys[rows] = x[rows].astype(np.float64) / float(temperature) - np.log(-np.log(u))
    return keys


def target_sample(logits, temperature: float, seed: int, offset: int) -> np.ndarray:
    """int32 [N]: the target's sampled token per node, argmax of
    ``sample_keys`` (smallest id on an exact tie)."""
    keys = sample_keys(logits, temperature, seed, offset)
    return np.argmax(keys, axis=1).astype(np.int32)


def near_tie_candidates(keys_row: np.ndarray, tol: float) -> np.ndarray:
    """Token ids whose fp64 key is within tol of the row's maximum."""
    return np.flatnonzero(keys_row >= keys_row.max() - tol)
