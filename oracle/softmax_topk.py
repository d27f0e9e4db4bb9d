"""Oracle: per-position log-softmax and top-K of the drafter's marginals.

Test infrastructure only (see the package docstring).

Sources
-------
* "DDTree Deep Dive" (zhichai.net), section 1: one drafter pass yields a
  marginal distribution q_i over the vocabulary for every block position i.
* Same page, section 2, Lemma 1: only the K = min(B, |V|) most probable
  tokens of each position can appear in an optimal tree.
* "DDTree: Turning Block Diffusion Drafters into Tree-Based Speculative
  Decoders" (alanhou.org), Key Concepts, best-first heap: nodes are scored
  by summed log-probabilities, so the per-position quantity is log q_i.

Readings where the pages are silent
-----------------------------------
* Ranking uses the raw fp32 logits (larger first) and breaks exact ties by
  the smaller token id; +0 and -0 compare equal. Log-softmax is monotone, so
  this is the same order as by probability.
* log q_i is computed in fp64: lse = m + log(sum exp(x - m)).
"""
from __future__ import annotations

import numpy as np


def log_softmax(x: np.ndarray) -> np.ndarray:
    """Row-wise log-softmax in fp64 (the definition, with max subtraction)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    for i in range(x.shape[0]):
        m = np.max(x[i])
        s = np.sum(np.exp(x[i] - m))
        out[i] = x[i] - (m + np.log(s))
    return out


def rank_order(row: np.ndarray) -> np.ndarray:
    """Token ids of one row sorted by (logit descending, id ascending).

    The fp32 logits are widened exactly to fp64 before sorting, so the
    comparison is the exact fp32 comparison (with -0 == +0)."""
    row = np.asarray(row, dtype=np.float32).astype(np.float64)
    ids = np.arange(row.shape[0])
    return np.lexsort((ids, -row))


def topk(x: np.ndarray, K: int):
    """Top-K per block position.

    Returns ``(logp, token)``: fp64 log-probabilities [L, K] and int32 token
    ids [L, K], both in rank order (rank 0 = most probable)."""
    x = np.asarray(x, dtype=np.float32)
    L, V = x.shape
    if not 1 <= K <= V:
        raise ValueError("K must be in [1, V]")
    lp_full = log_softmax(x)
    tok = np.empty((L, K), dtype=np.int32)
    lp = np.empty((L, K), dtype=np.float64)
    for i in range(L):
        order = rank_order(x[i])[:K]
        tok[i] = order
        lp[i] = lp_full[i, order]
    return lp, tok
