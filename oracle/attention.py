"""Oracle: ancestor-only tree attention of the target's verify pass (naive).

Test infrastructure only (see the package docstring).

Sources
-------
* "DDTree Deep Dive" (zhichai.net), section 4: every tree node attends to
  the past context held in the KV cache, the root (bonus token), its
  ancestors and itself, never to siblings or other branches.
* "DDTree: Turning Block Diffusion Drafters into Tree-Based Speculative
  Decoders" (alanhou.org), Core Mechanism and Key Concepts: all nodes are
  verified in one target forward pass under that mask.
* Same deep-dive page, section 10: the verifier attention is grouped-query
  attention as in Qwen3.

Readings where the pages are silent
-----------------------------------
* Every node sees all S prefix rows. Logits are scaled by ``scale``
  (1/sqrt(D) by default); no window, no soft-cap. Query head h reads
  kv-head floor(h / G) with G = Hq / Hkv.
* Tree node m's key and value live at cache row S + m.
* Arithmetic in fp64 on the bf16 inputs widened exactly.
"""
from __future__ import annotations

import numpy as np


def visible_rows(S: int, anc_row: np.ndarray, N: int) -> np.ndarray:
    """Cache rows node n may attend to: the prefix and its ancestors-or-self."""
    tree = [S + m for m in range(N) if (int(anc_row[m >> 5]) >> (m & 31)) & 1]
    return np.concatenate([np.arange(S, dtype=np.int64), np.asarray(tree, dtype=np.int64)])


def tree_attention(q, k, v, S: int, anc, scale: float | None = None,
                   nodes=None, heads=None) -> np.ndarray:
    """O[n, h] = sum_j softmax_j(scale * q[n,h] . k[g, j]) v[g, j] over the
    visible rows j of node n, g = h // G.

    q: [N, Hq, D]; k, v: [Hkv, rows, D]; anc: uint32 [N, W].
    ``nodes``/``heads`` restrict the computation to a sample (other entries
    of the result stay zero). Returns fp64 [N, Hq, D]."""
    q = np.asarray(q, dtype=np.float64)
    N, Hq, D = q.shape
    Hkv = k.shape[0]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    nodes = range(N) if nodes is None else nodes
    heads = range(Hq) if heads is None else heads
    out = np.zeros((N, Hq, D), dtype=np.float64)
    for n in nodes:
        rows = visible_rows(S, anc[n], N)
        cache = {}
        for h in heads:
            g = h // G
            if g not in cache:
                cache[g] = (np.asarray(k[g, rows], dtype=np.float64),
                            np.asarray(v[g, rows], dtype=np.float64))
            kk, vv = cache[g]
            z = scale * (kk @ q[n, h])
            z = z - np.max(z)
            p = np.exp(z)
            p = p / np.sum(p)
            out[n, h] = p @ vv
    return out
