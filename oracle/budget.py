"""Oracle: cost-aware choice of the node budget B for a round.

Test infrastructure only (see the package docstring).

Sources
-------
* "Qwen3-Coder-30B-A3B - DDTree vs DFlash vs autoregressive" (autobench
  config page), results table and notes: a larger budget raises the
  acceptance length but also the number of nodes the target verifies per
  step; past the optimum the verify cost outgrows the gain (budget 64 beat
  256), and a cost-aware variant is named as the way to pick the budget.
* "DDTree Deep Dive" (zhichai.net), section 2, Proposition 1: under the
  drafter's factorised distribution Q the expected accepted length of a tree
  T is the sum over its nodes u of q(u), the product of the marginals along
  u's path; Propositions 2-3: the best-first pops are the top-B prefixes.
* Same page, section 10: an adaptive node budget is listed as future work.

Readings where the pages are silent
-----------------------------------
* The top-B set of every B is the first B pops of one best-first build
  (Propositions 2-3 pop in score order), so one build with the largest
  budget B_max serves every B <= B_max: the budget-B tree is its first
  B + 1 nodes (root included), and its mask rows are unchanged.
* Expected tokens per round at budget B: 1 + E[alpha](B), where
  E[alpha](B) = sum over the first B popped nodes of exp(score) (score =
  the node's cumulative log-prob, Proposition 1) and the 1 is the bonus
  token every round emits.
* Round time at budget B: t0 + t1 * (B + 1), affine in the N = B + 1 nodes
  the target verifies; t0 and t1 are the caller's calibration.
* B* is the smallest B in [B_min, B_max] that maximises
  (1 + E[alpha](B)) / (t0 + t1 * (B + 1)).
* Everything here is fp64 (exp of the fp32 scores, running sums, ratios).
"""
from __future__ import annotations

import numpy as np


def _scores(score):
    s = np.asarray(score, dtype=np.float32)
    if s.ndim != 1 or s.size < 1:
        raise ValueError("score must be [B_max + 1] (root first)")
    if not np.isfinite(s).all() or (s[1:] > 0).any():
        raise ValueError("scores are finite log-probabilities (<= 0)")
    return s.astype(np.float64)


def expected_accept(score) -> np.ndarray:
    """fp64 [B_max + 1]: entry B = E[alpha] of the tree of the first B pops
    (entry 0 = 0: the root alone accepts nothing)."""
    s = _scores(score)
    out = np.zeros(s.size, dtype=np.float64)
    for B in range(1, s.size):
        out[B] = out[B - 1] + np.exp(s[B])
    return out


def budget_objective(score, t0: float, t1: float) -> np.ndarray:
    """fp64 [B_max + 1]: expected tokens per unit of round time, per B."""
    if not (np.isfinite(t0) and np.isfinite(t1) and t0 >= 0 and t1 >= 0 and t0 + t1 > 0):
        raise ValueError("cost model needs finite t0, t1 >= 0, not both 0")
    ea = expected_accept(score)
    B = np.arange(ea.size, dtype=np.float64)
    return (1.0 + ea) / (t0 + t1 * (B + 1.0))


def select_budget(score, t0: float, t1: float, B_min: int = 1, B_max: int | None = None) -> int:
    """The smallest B in [B_min, B_max] with the largest objective."""
    obj = budget_objective(score, t0, t1)
    B_max = obj.size - 1 if B_max is None else B_max
    if not 0 <= B_min <= B_max <= obj.size - 1:
        raise ValueError("need 0 <= B_min <= B_max <= len(score) - 1")
    best = B_min
    for B in range(B_min + 1, B_max + 1):
        if obj[B] > obj[best]:
            best = B
    return best
