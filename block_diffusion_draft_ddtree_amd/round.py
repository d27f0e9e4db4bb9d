"""One DDTree decode round on the device: topk -> build -> tree attention per
layer -> (target argmax, or target sample at temperature > 0) -> accept walk
-> KV compaction ("DDTree Deep
Dive", section 3: the draft, tree_build, tree_compile, verify, commit
stages; the drafter forward and the target's non-attention layers, LM head
included, are outside this library).

All buffers are allocated once (torch device memory) so a round enqueues
only libddtree kernels, which also makes the round capturable in a HIP
graph. The next round's root token is the walk's ``next_bonus`` buffer.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import binding as bd


@dataclass
class RoundShape:
    L: int
    V: int
    K: int
    B: int
    Hq: int
    Hkv: int
    D: int
    layers: int
    S_cap: int

    @property
    def N(self) -> int:
        return self.B + 1

    @property
    def W(self) -> int:
        return (self.N + 31) // 32


class DraftTreeRound:
    def __init__(self, shape: RoundShape, S_max: int, device="cuda"):
        s = shape
        self.shape = s
        dev = torch.device(device)
        i32 = dict(dtype=torch.int32, device=dev)
        self.logp = torch.empty((s.L, s.K), dtype=torch.float32, device=dev)
        self.token = torch.empty((s.L, s.K), **i32)
        self.ws_topk = bd.workspace(bd.ddtree_topk_workspace_bytes(s.L, s.V, s.K), dev)
        self.root_token = torch.zeros(1, **i32)
        self.parent = torch.empty(s.N, **i32)
        self.depth = torch.empty(s.N, **i32)
        self.node_token = torch.empty(s.N, **i32)
        self.score = torch.empty(s.N, dtype=torch.float32, device=dev)
        self.anc = torch.empty((s.N, s.W), **i32)
        self.attn_out = torch.empty((s.layers, s.N, s.Hq, s.D), dtype=torch.bfloat16, device=dev)
        self.ws_attn = bd.workspace(bd.ddtree_tree_attn_workspace_bytes(s.N, s.Hq, s.Hkv, s.D, S_max), dev)
        self.target_choice = torch.empty(s.N, **i32)
        self.ws_argmax = bd.workspace(
            bd.ddtree_target_argmax_workspace_bytes(bd.DDTREE_DTYPE_BF16, s.N, s.V), dev)
        self.budget = torch.empty(1, **i32)
        self.expected_accept = torch.empty(s.N, dtype=torch.float32, device=dev)
        self.acc = torch.empty(s.L + 1, **i32)
        self.n_acc = torch.empty(1, **i32)
        self.next_bonus = torch.empty(1, **i32)

    def topk(self, logits):
        bd.ddtree_topk(logits, self.shape.K, self.logp, self.token, self.ws_topk)

    def build(self):
        bd.ddtree_build(self.logp, self.token, self.shape.B, self.root_token, self.shape.W,
                        self.parent, self.depth, self.node_token, self.score, self.anc)

    def attn(self, layer: int, q, kv, S: int):
        bd.ddtree_tree_attn(q[layer], kv[layer, 0], kv[layer, 1], S, self.anc,
                            out=self.attn_out[layer], ws=self.ws_attn)

    def select_budget(self, t0: float, t1: float, B_min: int = 1):
        """Cost-aware budget over this round's tree: the first budget[0] + 1
        nodes form the tree to verify (round time model t0 + t1 * nodes)."""
        return bd.ddtree_budget_select(self.score, self.shape.B, t0, t1, B_min,
                                       expected=self.expected_accept, budget=self.budget)

    def prune(self):
        """Keep the budget[0]-tree (set by select_budget) inside this round's
        tree: the walk and the attention then skip the dropped nodes."""
        bd.ddtree_tree_prune(self.budget, self.parent, self.anc)

    def target_argmax(self, target_logits):
        """bf16 [N, V] target head logits -> the target's greedy token per node."""
        return bd.ddtree_target_argmax(target_logits, out=self.target_choice, ws=self.ws_argmax)

    def target_sample(self, target_logits, temperature: float, seed: int, offset: int):
        """Temperature > 0: the target's sampled token per node (the walk then
        runs on these); pass a fresh offset every round."""
        return bd.ddtree_target_sample(target_logits, temperature, seed, offset,
                                       out=self.target_choice, ws=self.ws_argmax)

    def walk(self, target_argmax):
        bd.ddtree_accept_walk(self.parent, self.node_token, self.shape.L, target_argmax,
                              self.acc, self.n_acc, self.next_bonus)

    def compact(self, kv, S: int):
        bd.ddtree_kv_compact(kv, S, self.shape.N, self.shape.L, self.acc, self.n_acc)

    def run(self, logits, q, kv, S: int, target_argmax):
        """Enqueue one full round on the current stream (no host sync)."""
        self.topk(logits)
        self.build()
        for layer in range(self.shape.layers):
            self.attn(layer, q, kv, S)
        self.walk(target_argmax)
        self.compact(kv, S)


class BatchedDraftTreeRound:
    """One round for R requests at once: each has its own drafter rows, tree,
    prefix length S[r] and KV cache (kv: [R, layers, 2, Hkv, S_cap, D]); all
    share L, V, K, B and the attention shape. Every buffer is allocated here,
    so a round enqueues only libddtree kernels."""

    def __init__(self, shape: RoundShape, S, device="cuda"):
        s = shape
        self.shape = s
        self.R = len(S)
        self.S = [int(x) for x in S]
        dev = torch.device(device)
        i32 = dict(dtype=torch.int32, device=dev)
        R, N = self.R, s.N
        self.logp = torch.empty((R * s.L, s.K), dtype=torch.float32, device=dev)
        self.token = torch.empty((R * s.L, s.K), **i32)
        self.ws_topk = bd.workspace(bd.ddtree_topk_workspace_bytes(R * s.L, s.V, s.K), dev)
        self.root_token = torch.zeros(R, **i32)
        self.attn_out = torch.empty((s.layers, R, N, s.Hq, s.D), dtype=torch.bfloat16, device=dev)
        self.ws_attn = bd.workspace(
            bd.ddtree_tree_attn_batched_workspace_bytes(self.S, N, s.Hq, s.Hkv, s.D), dev)
        # parent, depth, node_token, score [R, N]; anc [R, N, W]
        self.tree = (torch.empty((R, N), **i32), torch.empty((R, N), **i32),
                     torch.empty((R, N), **i32),
                     torch.empty((R, N), dtype=torch.float32, device=dev),
                     torch.empty((R, N, s.W), **i32))
        # acc [R, L + 1], n_acc [R], next_bonus [R]
        self.walk_out = (torch.empty((R, s.L + 1), **i32), torch.empty(R, **i32),
                         torch.empty(R, **i32))

    def topk(self, logits):
        """logits fp32 [R * L, V]: request r's block positions at rows r * L ..."""
        bd.ddtree_topk(logits, self.shape.K, self.logp, self.token, self.ws_topk)

    def build(self):
        s = self.shape
        bd.ddtree_build_batched(self.logp.view(self.R, s.L, s.K),
                                self.token.view(self.R, s.L, s.K), s.B, self.root_token, s.W,
                                out=self.tree)

    def attn(self, layer: int, q, kv):
        """q bf16 [R, N, Hq, D] for this layer; kv [R, layers, 2, Hkv, S_cap, D]."""
        bd.ddtree_tree_attn_batched(q, kv, layer, self.S, self.tree[4], out=self.attn_out[layer],
                                    ws=self.ws_attn)

    def walk(self, target):
        """target int32 [R, N]: the target's token per node of every request."""
        parent, _, node_token, _, _ = self.tree
        return bd.ddtree_accept_walk_batched(parent, node_token, self.shape.L, target,
                                             out=self.walk_out)

    def compact(self, kv):
        acc, n_acc, _ = self.walk_out
        bd.ddtree_kv_compact_batched(kv, self.S, self.shape.N, self.shape.L, acc, n_acc)
