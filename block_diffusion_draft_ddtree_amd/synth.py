"""Seeded synthetic inputs for the DDTree draft-tree hot path.

This module only draws random numbers shaped like the workloads. It holds
none of the method's arithmetic: no softmax, no prefix scores, no tree
selection, no attention and no acceptance rule. The HIP path's tests and
benchmark and the CPU oracle's tests both take their inputs from here, and
nothing else is shared between the two.

Every draw comes from numpy's PCG64 keyed by a SeedSequence of
``[workload_id, round, stream]`` so that any (workload, round) pair can be
regenerated bit for bit.

bf16 tensors are produced as fp32 values rounded to nearest-even bf16; both
the raw uint16 bit patterns (for device upload) and the exactly-equal fp32
values (for host checks) are returned.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

# Stream identifiers inside one (workload, round) seed.
STREAM_LOGITS = 0
STREAM_QKV = 1
STREAM_TARGET = 2
STREAM_ACCEPT = 3
STREAM_EXTRA = 4
STREAM_TARGET_LOGITS = 5

WORKLOAD_IDS = {
    "tiny": 1,
    "qwen3_8b": 2,
    "coder30b": 3,
    "longctx": 4,
    "sweep": 5,
    "test": 6,
}


@dataclass(frozen=True)
class Workload:
    """Sizes of one synthetic workload.

    L: drafted block positions; V: vocabulary; K: top-K kept per position;
    B: node budget (the tree has N = B + 1 nodes including the root);
    Hq / Hkv: query / key-value heads; D: head dim; S: cached prefix length;
    layers: attention layers per verify pass; logits: generator family.
    """

    name: str
    family: str
    L: int
    V: int
    K: int
    B: int
    Hq: int
    Hkv: int
    D: int
    S: int
    layers: int
    logits: str

    @property
    def N(self) -> int:
        return self.B + 1

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def mask_words(self) -> int:
        return (self.N + 31) // 32

    @property
    def S_cap(self) -> int:
        return self.S + self.N


def _w(name, family, **kw) -> Workload:
    return Workload(name=name, family=family, **kw)


TINY = _w("tiny", "tiny", L=4, V=1000, K=8, B=16, Hq=4, Hkv=2, D=64, S=128,
          layers=1, logits="tiny")
QWEN3_8B = _w("qwen3_8b", "qwen3_8b", L=16, V=151936, K=64, B=64, Hq=32,
              Hkv=8, D=128, S=2048, layers=36, logits="peaked")
CODER30B_B64 = _w("coder30b_b64", "coder30b", L=16, V=151936, K=64, B=64,
                  Hq=32, Hkv=4, D=128, S=4096, layers=48, logits="peaked")
CODER30B_B256 = replace(CODER30B_B64, name="coder30b_b256", K=256, B=256)
# The same verifier shape with a confident drafter (deep trees, accepted
# length ~4): exercises deep ancestor masks, the walk and the compaction.
CODER30B_B64_DEEP = replace(CODER30B_B64, name="coder30b_b64_deep", logits="confident")
LONGCTX = _w("longctx", "longctx", L=16, V=151936, K=256, B=256, Hq=32,
             Hkv=4, D=128, S=32768, layers=1, logits="peaked")
SWEEP_BUDGETS = (16, 32, 64, 128, 256, 512)


def sweep(B: int) -> Workload:
    return _w(f"sweep_b{B}", "sweep", L=16, V=151936, K=B, B=B, Hq=32,
              Hkv=8, D=128, S=8192, layers=36, logits="flat")


WORKLOADS = {w.name: w for w in
             (TINY, QWEN3_8B, CODER30B_B64, CODER30B_B256, CODER30B_B64_DEEP, LONGCTX)}
for _b in SWEEP_BUDGETS:
    WORKLOADS[f"sweep_b{_b}"] = sweep(_b)

# Layers reported for the long-context shape (one layer is timed).
LONGCTX_REPORTED_LAYERS = 48
SWEEP_ROUNDS = 1000


def rng(family: str | int, round_idx: int = 0, stream: int = 0) -> np.random.Generator:
    wid = WORKLOAD_IDS[family] if isinstance(family, str) else int(family)
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence([wid, int(round_idx), int(stream)])))


# ----------------------------------------------------------------------------
# bf16 helpers (storage format only)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(g: np.random.Generator, shape) -> tuple[np.ndarray, np.ndarray]:
    """N(0,1) values rounded to bf16: (uint16 bits, equal fp32 values)."""
    bits = f32_to_bf16_bits(g.standard_normal(shape, dtype=np.float32))
    return bits, bf16_bits_to_f32(bits)


# ----------------------------------------------------------------------------
# Drafter logits
# ----------------------------------------------------------------------------

@dataclass
class Logits:
    x: np.ndarray          # fp32 [L, V]
    peak: np.ndarray       # int64 [L]: boosted token per position
    runner: np.ndarray | None  # int64 [L] or None


def drafter_logits(w: Workload, round_idx: int = 0) -> Logits:
    """Per-position drafter logits of the workload's family.

    tiny:   2*N(0,1) plus +6 on one uniform peak token per position.
    peaked: 2*N(0,1) plus (9 - 0.4 i) on a peak and (7 - 0.4 i) on a
            distinct runner-up token at 0-based block position i. Over
            V = 151936 the bulk carries most of the mass (the peak gets
            q ~ 0.01), so best-first trees of B = 64 stay at depth 1.
    confident: a confident drafter: N(0,1) bulk, and at position i a peak
            token with probability p_peak(i) = max(0.85 - 0.03 i, 0.2) and a
            distinct runner-up with p_run(i) = 0.08 + 0.005 i (their logits
            are set from the bulk's own partition sum, so the softmax gives
            these probabilities). Confidence decays along the block, and
            best-first trees grow deep along the peak path with branches
            near the root.
    flat:   1.5*N(0,1) plus +3 on one peak token.
    """
    g = rng(w.family, round_idx, STREAM_LOGITS)
    L, V = w.L, w.V
    if w.logits == "tiny":
        x = np.float32(2.0) * g.standard_normal((L, V), dtype=np.float32)
        peak = g.integers(0, V, size=L)
        x[np.arange(L), peak] += np.float32(6.0)
        return Logits(x, peak, None)
    if w.logits == "peaked":
        x = np.float32(2.0) * g.standard_normal((L, V), dtype=np.float32)
        peak = g.integers(0, V, size=L)
        off = g.integers(1, V, size=L)
        runner = (peak + off) % V
        i = np.arange(L, dtype=np.float32)
        x[np.arange(L), peak] += (np.float32(9.0) - np.float32(0.4) * i).astype(np.float32)
        x[np.arange(L), runner] += (np.float32(7.0) - np.float32(0.4) * i).astype(np.float32)
        return Logits(x, peak, runner)
    if w.logits == "confident":
        x = g.standard_normal((L, V), dtype=np.float32)
        peak = g.integers(0, V, size=L)
        off = g.integers(1, V, size=L)
        runner = (peak + off) % V
        rows = np.arange(L)
        p_peak, p_run = confident_probs(L)
        e = np.exp(x.astype(np.float64))
        z = e.sum(axis=1) - e[rows, peak] - e[rows, runner]  # bulk partition sum
        rest = 1.0 - p_peak - p_run
        x[rows, peak] = np.log(p_peak * z / rest).astype(np.float32)
        x[rows, runner] = np.log(p_run * z / rest).astype(np.float32)
        return Logits(x, peak, runner)
    if w.logits == "flat":
        x = np.float32(1.5) * g.standard_normal((L, V), dtype=np.float32)
        peak = g.integers(0, V, size=L)
        x[np.arange(L), peak] += np.float32(3.0)
        return Logits(x, peak, None)
    raise ValueError(w.logits)


def confident_probs(L: int):
    """Target probabilities of the peak and runner-up tokens per block
    position of the 'confident' drafter."""
    i = np.arange(L, dtype=np.float64)
    return np.maximum(0.85 - 0.03 * i, 0.2), 0.08 + 0.005 * i


def tie_logits(L: int, V: int, g: np.random.Generator, levels: int = 4) -> np.ndarray:
    """Logits drawn from a small integer set so that exact ties are common."""
    return g.integers(0, levels, size=(L, V)).astype(np.float32)


def deep_logits(L: int, V: int, g: np.random.Generator, n_hot: int = 3) -> np.ndarray:
    """Logits whose top few tokens per position carry most of the mass, so
    best-first trees grow deep instead of staying at depth 1."""
    x = np.float32(0.5) * g.standard_normal((L, V), dtype=np.float32)
    for i in range(L):
        hot = g.choice(V, size=n_hot, replace=False)
        x[i, hot] += (np.float32(8.0) + g.standard_normal(n_hot, dtype=np.float32))
    return x


# ----------------------------------------------------------------------------
# Ready-made [L, K] top-K tables for tree-build tests (sorted, non-positive)
# ----------------------------------------------------------------------------

def sorted_logp_table(L: int, K: int, V: int, g: np.random.Generator,
                      scale: float = 1.0, ties: bool = False):
    """A per-position table of K non-increasing, non-positive fp32 values and
    K distinct token ids per row, shaped like a top-K output."""
    if ties:
        vals = -np.float32(0.5) * g.integers(0, 4, size=(L, K)).astype(np.float32)
    else:
        vals = -np.abs(np.float32(scale) * g.standard_normal((L, K), dtype=np.float32))
    vals = -np.sort(-vals, axis=1)  # non-increasing per row
    tok = np.stack([g.choice(V, size=K, replace=False) for _ in range(L)]).astype(np.int32)
    return np.ascontiguousarray(vals, dtype=np.float32), tok


def target_logits(g: np.random.Generator, N: int, V: int, peaks=None,
                  boost: float = 8.0) -> tuple[np.ndarray, np.ndarray]:
    """The verifier head's logits for N tree nodes, bf16 [N, V]: 2 N(0,1)
    rounded to bf16, plus `boost` at peaks[n] when given (the token the
    target prefers after node n). Returns (uint16 bits, equal fp32 values)."""
    x = 2.0 * g.standard_normal((N, V), dtype=np.float32)
    if peaks is not None:
        x[np.arange(N), np.asarray(peaks)] += np.float32(boost)
    bits = f32_to_bf16_bits(x)
    return bits, bf16_bits_to_f32(bits)


# ----------------------------------------------------------------------------
# Attention tensors
# ----------------------------------------------------------------------------

@dataclass
class QKV:
    q_bits: np.ndarray     # uint16 [N, Hq, D]
    q: np.ndarray          # fp32   [N, Hq, D]
    kv_bits: np.ndarray    # uint16 [layers, 2, Hkv, S_cap, D]
    kv: np.ndarray         # fp32   same shape


def attention_inputs(w: Workload, layers: int | None = None, round_idx: int = 0,
                     S_cap: int | None = None, N: int | None = None) -> QKV:
    """bf16 N(0,1) queries for the N tree nodes and a KV cache laid out
    [layers][K|V][Hkv][S_cap][D]; rows [0, S) are the prefix, rows
    [S, S+N) the tree nodes' keys and values."""
    g = rng(w.family, round_idx, STREAM_QKV)
    layers = w.layers if layers is None else layers
    N = w.N if N is None else N
    S_cap = (w.S + N) if S_cap is None else S_cap
    q_bits, q = normal_bf16(g, (N, w.Hq, w.D))
    kv_bits, kv = normal_bf16(g, (layers, 2, w.Hkv, S_cap, w.D))
    return QKV(q_bits, q, kv_bits, kv)


# ----------------------------------------------------------------------------
# Target argmax per tree node (drives the accept walk)
# ----------------------------------------------------------------------------

def _children(parent: np.ndarray) -> list[list[int]]:
    ch: list[list[int]] = [[] for _ in range(len(parent))]
    for n in range(1, len(parent)):
        ch[int(parent[n])].append(n)
    return ch


def _uniform_excluding(g: np.random.Generator, V: int, excl: set[int]) -> int:
    while True:
        t = int(g.integers(0, V))
        if t not in excl:
            return t


def target_argmax_tiny(parent, node_token, V, g, p_off=0.3) -> np.ndarray:
    """Per node: with probability 1 - p_off a uniformly chosen child's token,
    otherwise a token that is not among the node's children (leaves are
    always off-tree)."""
    ch = _children(np.asarray(parent))
    tgt = np.empty(len(parent), dtype=np.int32)
    for n in range(len(parent)):
        toks = [int(node_token[c]) for c in ch[n]]
        if toks and g.random() >= p_off:
            tgt[n] = toks[int(g.integers(0, len(toks)))]
        else:
            tgt[n] = _uniform_excluding(g, V, set(toks))
    return tgt


def target_argmax_follow_peak(depth, peak, L, V, g, p_follow=0.8) -> np.ndarray:
    """Per node at depth d < L: the drafter's peak token of block position d
    with probability p_follow, else a uniform token other than that peak.
    Nodes at depth L get a uniform token."""
    tgt = np.empty(len(depth), dtype=np.int32)
    for n, d in enumerate(np.asarray(depth)):
        d = int(d)
        if d >= L:
            tgt[n] = int(g.integers(0, V))
        elif g.random() < p_follow:
            tgt[n] = int(peak[d])
        else:
            tgt[n] = _uniform_excluding(g, V, {int(peak[d])})
    return tgt


def target_argmax_planted(parent, node_token, path, V, g) -> np.ndarray:
    """Target argmax that matches the tokens along ``path`` (a root-to-node
    list of node ids starting at 0) and is off-tree everywhere else."""
    ch = _children(np.asarray(parent))
    tgt = np.empty(len(parent), dtype=np.int32)
    for n in range(len(parent)):
        tgt[n] = _uniform_excluding(g, V, {int(node_token[c]) for c in ch[n]})
    for a, b in zip(path[:-1], path[1:]):
        tgt[a] = int(node_token[b])
    return tgt


# ----------------------------------------------------------------------------
# Accepted paths for compaction-only tests and the budget sweep
# ----------------------------------------------------------------------------

def accepted_path(B: int, L: int, g: np.random.Generator) -> np.ndarray:
    """acc[0] = 0 followed by a = min(U[1, L], B) strictly increasing node ids
    in [1, B] (the budget-sweep recipe for compaction)."""
    a = min(int(g.integers(1, L + 1)), B)
    picks = np.sort(g.choice(np.arange(1, B + 1), size=a, replace=False))
    return np.concatenate([[0], picks]).astype(np.int32)


def sweep_accepts(B: int, L: int, rounds: int) -> tuple[np.ndarray, np.ndarray]:
    """Accepted paths of `rounds` budget-sweep rounds: a_r ~ U[1, L] from a
    stream that does not depend on B (so the prefix lengths advance the same
    way at every budget), capped at B, and a_r strictly increasing node ids
    in [1, B] from a per-budget stream. Returns acc int32 [rounds, L + 1]
    (acc[r, 0] = 0, unused tail 0) and a int32 [rounds]."""
    ga = rng("sweep", 0, STREAM_ACCEPT)
    gp = rng("sweep", B, STREAM_EXTRA)
    acc = np.zeros((rounds, L + 1), dtype=np.int32)
    a = np.empty(rounds, dtype=np.int32)
    for r in range(rounds):
        a[r] = min(int(ga.integers(1, L + 1)), B)
        picks = np.sort(gp.choice(np.arange(1, B + 1), size=int(a[r]), replace=False))
        acc[r, 1:1 + a[r]] = picks
    return acc, a


def sweep_prefix_lengths(S0: int, a: np.ndarray) -> np.ndarray:
    """Prefix length at the start of each round: S advances by the root plus
    the accepted tokens of the previous round."""
    return (S0 + np.concatenate([[0], np.cumsum(1 + a.astype(np.int64))[:-1]])).astype(np.int64)
