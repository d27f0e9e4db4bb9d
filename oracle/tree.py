"""Oracle: the budget-B draft tree and its ancestor-only visibility mask.

Test infrastructure only (see the package docstring).

Sources
-------
* "DDTree Deep Dive" (zhichai.net), section 1: the drafter's factorised
  distribution Q(y) = prod_i q_i(y_i) is the surrogate objective.
* Same page, section 2: Proposition 2 (the B most probable prefixes form a
  prefix-closed tree and are optimal, so selection is a sort), Lemma 1
  (top-K per position suffices), Proposition 3 (a max-heap over rank tuples
  that pushes the next sibling and the first child of each popped prefix
  pops exactly the top-B prefixes).
* Same page, section 3: the tree is encoded as (position in tree, parent
  position) pairs.
* Same page, section 4, and "DDTree: Turning Block Diffusion Drafters into
  Tree-Based Speculative Decoders" (alanhou.org), Key Concepts: a node sees
  the root, its ancestors and itself, never a sibling or another branch.

Readings where the pages are silent
-----------------------------------
* A prefix is a rank tuple r = (r_1..r_d), 1 <= d <= L, 0 <= r_j < K; its
  token is the rank-r_d token of block position d.
* Its score is the fp32 left-to-right sum s_1 = logp[0][r_1],
  s_j = fl32(s_{j-1} + logp[j-1][r_j]). The device takes the same integer
  decision (which prefixes, in which order) from these fp32 sums, so the
  oracle mirrors that precision here.
* Order: r precedes r' iff score(r) > score(r'), or the scores are equal
  and r is lexicographically smaller (a proper prefix is smaller). With
  logp <= 0 and ranks sorted by probability this keeps the top-B set
  prefix-closed even when rounding makes a child tie its parent.
* Node 0 is the root (the bonus token, depth 0, score 0); nodes 1..B are
  the selected prefixes in that order, so parent(n) < n.
* Mask: bit j of row n is set iff node j is n or an ancestor of n; bit j
  lives in 32-bit word j >> 5 at bit j & 31; unused bits are zero.
"""
from __future__ import annotations

import heapq
import itertools
from dataclasses import dataclass

import numpy as np


def prefix_score(logp32: np.ndarray, ranks) -> np.float32:
    """fp32 left-to-right sum of the log-probs along a rank tuple."""
    s = np.float32(logp32[0, ranks[0]])
    for d in range(1, len(ranks)):
        s = np.float32(s + np.float32(logp32[d, ranks[d]]))
    return s


def order_key(score, ranks):
    """Sort key realising the order on prefixes (smaller key = earlier)."""
    return (-float(score), tuple(ranks))


def num_prefixes(L: int, K: int) -> int:
    return sum(K ** d for d in range(1, L + 1))


def top_b_brute_force(logp32: np.ndarray, B: int):
    """Enumerate every prefix of the K-restricted trie and sort them all."""
    logp32 = np.asarray(logp32, dtype=np.float32)
    L, K = logp32.shape
    keys = []
    for d in range(1, L + 1):
        for r in itertools.product(range(K), repeat=d):
            keys.append(order_key(prefix_score(logp32, r), r))
    keys.sort()
    return [r for _, r in keys[:B]]


def top_b_sort_expand(logp32: np.ndarray, B: int):
    """Top-B set by repeated sorting when the trie is too big to enumerate.

    Start from the K depth-1 prefixes; repeatedly take the first B of the
    sorted candidate set and add the children of those that are shallower
    than L; stop when nothing new is added. At that point every child of a
    selected prefix is a candidate, so the shallowest true top-B prefix
    missing from the selection would itself be a candidate preceded by fewer
    than B others, which is impossible: the selection is exact."""
    logp32 = np.asarray(logp32, dtype=np.float32)
    L, K = logp32.shape
    P = {(r,): np.float32(logp32[0, r]) for r in range(K)}
    while True:
        T = sorted(P, key=lambda r: order_key(P[r], r))[:B]
        grown = False
        for r in T:
            if len(r) < L:
                for c in range(K):
                    ch = r + (c,)
                    if ch not in P:
                        P[ch] = np.float32(P[r] + np.float32(logp32[len(r), c]))
                        grown = True
        if not grown:
            return T


def top_b_best_first(logp32: np.ndarray, B: int):
    """Proposition 3 as a textbook binary heap: pop the best prefix, push its
    next sibling (same depth, next rank) and its first child (one position
    deeper, rank 0)."""
    logp32 = np.asarray(logp32, dtype=np.float32)
    L, K = logp32.shape
    s0 = np.float32(logp32[0, 0])
    # entries: (order key, ranks, score, score of the parent prefix or None)
    heap = [(order_key(s0, (0,)), (0,), s0, None)]
    out = []
    while heap and len(out) < B:
        _, r, s, ps = heapq.heappop(heap)
        out.append(r)
        d = len(r)
        if r[-1] + 1 < K:
            sib = r[:-1] + (r[-1] + 1,)
            if ps is None:
                ss = np.float32(logp32[0, sib[-1]])
            else:
                ss = np.float32(ps + np.float32(logp32[d - 1, sib[-1]]))
            heapq.heappush(heap, (order_key(ss, sib), sib, ss, ps))
        if d < L:
            ch = r + (0,)
            cs = np.float32(s + np.float32(logp32[d, 0]))
            heapq.heappush(heap, (order_key(cs, ch), ch, cs, s))
    return out


def top_b(logp32: np.ndarray, B: int, brute_limit: int = 50_000):
    """The top-B prefixes: brute force where the trie is small enough,
    otherwise the sort-and-expand fixed point."""
    L, K = np.asarray(logp32).shape
    if not 1 <= B <= num_prefixes(L, K):
        raise ValueError("B must be in [1, number of prefixes]")
    if num_prefixes(L, K) <= brute_limit:
        return top_b_brute_force(logp32, B)
    return top_b_sort_expand(logp32, B)


@dataclass
class Tree:
    parent: np.ndarray   # int32 [N]; -1 for the root
    depth: np.ndarray    # int32 [N]
    token: np.ndarray    # int32 [N]
    score: np.ndarray    # fp32  [N]
    anc: np.ndarray      # uint32 [N, mask_words]
    ranks: list          # rank tuple per node; () for the root

    @property
    def N(self) -> int:
        return len(self.parent)


def ancestor_mask(parent, mask_words: int | None = None) -> np.ndarray:
    """Ancestor-or-self bit rows, by walking each node's parent chain."""
    parent = np.asarray(parent)
    N = len(parent)
    W = (N + 31) // 32 if mask_words is None else mask_words
    if W * 32 < N:
        raise ValueError("mask_words too small")
    anc = np.zeros((N, W), dtype=np.uint32)
    for n in range(N):
        j = n
        while j != -1:
            anc[n, j >> 5] |= np.uint32(1 << (j & 31))
            j = int(parent[j])
    return anc


def tree_from_prefixes(T, logp32, tok, root_token: int, mask_words: int | None = None) -> Tree:
    """Lay the ordered prefixes out as node arrays (node 0 = root)."""
    logp32 = np.asarray(logp32, dtype=np.float32)
    index = {(): 0}
    for n, r in enumerate(T, start=1):
        index[tuple(r)] = n
    N = len(T) + 1
    parent = np.full(N, -1, dtype=np.int32)
    depth = np.zeros(N, dtype=np.int32)
    token = np.zeros(N, dtype=np.int32)
    score = np.zeros(N, dtype=np.float32)
    token[0] = root_token
    for n, r in enumerate(T, start=1):
        r = tuple(r)
        parent[n] = index[r[:-1]]  # KeyError here = the set is not prefix-closed
        depth[n] = len(r)
        token[n] = tok[len(r) - 1][r[-1]]
        score[n] = prefix_score(logp32, r)
    return Tree(parent, depth, token, score, ancestor_mask(parent, mask_words),
                [()] + [tuple(r) for r in T])


def build_tree(logp32, tok, B: int, root_token: int, mask_words: int | None = None) -> Tree:
    """Full tree construction: top-B prefixes, node arrays and mask."""
    return tree_from_prefixes(top_b(logp32, B), logp32, tok, root_token, mask_words)
