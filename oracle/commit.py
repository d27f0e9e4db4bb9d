"""Oracle: the target's greedy choice per node, the greedy accept walk and
the KV-cache compaction of a round.

Test infrastructure only (see the package docstring).

Sources
-------
* "DDTree Deep Dive" (zhichai.net), section 6: verification walks the tree;
  the target's choice at the current node selects the matching child if one
  exists, and the first target token with no matching child becomes the
  next round's bonus token.
* Same page, section 5: after verification only the accepted path stays in
  the cache; tree tokens are interleaved in the tail, so the accepted rows
  are gathered in place (without compaction the cache would grow by the
  budget every round).
* "DDTree: Turning Block Diffusion Drafters into Tree-Based Speculative
  Decoders" (alanhou.org), Core Mechanism: the longest matching prefix is
  accepted.

Readings where the pages are silent
-----------------------------------
* Greedy only: ``target_argmax[n]`` is the target's argmax after node n,
  taken over the V logits the verifier's head gives node n: the largest
  value compared as fp32 (bf16 logits widen exactly; -0 equals +0, -inf is
  allowed, NaN is not), the smallest token id among equal maxima (the same
  tie rule as the top-K rank order).
* The walk is computed here by path consistency rather than by descending:
  node n is consistent iff every edge p -> c on the root-to-n path has
  token[c] == target_argmax[p]. Siblings carry distinct tokens, so the
  consistent nodes form a chain from the root; the deepest one, f, ends the
  walk: accepted nodes are that chain, a = depth(f), bonus = argmax[f].
* ``acc`` has L + 1 entries: acc[0] = 0 (root), acc[1..a] the accepted
  nodes, the rest -1.
* Compaction: cache row S + k takes row S + acc[k] for k = 1..a in every
  layer, K/V half and kv-head; rows below S + 1 and rows from S + 1 + a on
  are left as they were.
"""
from __future__ import annotations

import numpy as np


def target_argmax(logits) -> np.ndarray:
    """int32 [N]: for each row, the first index holding the row's maximum."""
    x = np.asarray(logits, dtype=np.float32)
    if x.ndim != 2 or x.shape[1] < 1:
        raise ValueError("logits must be [N, V] with V >= 1")
    if np.isnan(x).any():
        raise ValueError("NaN logits")
    out = np.empty(x.shape[0], dtype=np.int32)
    for n in range(x.shape[0]):
        out[n] = int(np.flatnonzero(x[n] == x[n].max())[0])
    return out


def accept_walk(parent, node_token, target_argmax, L: int):
    """Returns ``(acc, a, bonus)`` with acc int32 [L + 1]."""
    parent = np.asarray(parent)
    node_token = np.asarray(node_token)
    tgt = np.asarray(target_argmax)
    N = len(parent)
    depth = np.zeros(N, dtype=np.int64)
    consistent = np.zeros(N, dtype=bool)
    consistent[0] = True
    for n in range(1, N):
        p = int(parent[n])
        if not 0 <= p < n:
            raise ValueError("parents must precede their children")
        depth[n] = depth[p] + 1
        consistent[n] = consistent[p] and int(node_token[n]) == int(tgt[p])
    cons = np.flatnonzero(consistent)
    f = int(cons[np.argmax(depth[cons])])
    if np.count_nonzero(depth[cons] == depth[f]) != 1:
        raise ValueError("two siblings share a token")
    path = []
    j = f
    while j != -1:
        path.append(j)
        j = int(parent[j])
    path.reverse()
    a = len(path) - 1
    if a > L:
        raise ValueError("tree deeper than L")
    acc = np.full(L + 1, -1, dtype=np.int32)
    acc[: a + 1] = path
    return acc, a, int(tgt[f])


def kv_compact(kv: np.ndarray, S: int, acc, a: int) -> np.ndarray:
    """Out-of-place compaction of a cache laid out [..., rows, D]."""
    out = np.array(kv, copy=True)
    for k in range(1, a + 1):
        out[..., S + k, :] = kv[..., S + int(acc[k]), :]
    return out
