"""ctypes binding of libddtree (same names as the C ABI in include/ddtree.h).

Argument marshalling only: torch device tensors become raw device pointers
and the current torch stream becomes the HIP stream; every step of the path
runs in the library's HIP kernels. Outputs and workspaces that are not
passed in are allocated with torch (device memory plumbing). A missing
library is an error: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libddtree.so")

DDTREE_OK = 0
DDTREE_ERR_INVALID_ARGUMENT = 1
DDTREE_ERR_UNSUPPORTED = 2
DDTREE_ERR_WORKSPACE_TOO_SMALL = 3
DDTREE_ERR_HIP = 4

MAX_L, MAX_K, MAX_B, MAX_LK = 32, 1024, 1024, 32768
DDTREE_DTYPE_F32, DDTREE_DTYPE_BF16 = 0, 1

_lib = None
_vp, _i32, _i64, _f32, _sz = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                              ctypes.c_float, ctypes.c_size_t)
_u64 = ctypes.c_uint64

_SIGNATURES = {
    "ddtree_status_string": (ctypes.c_char_p, [_i32]),
    "ddtree_version": (_i32, []),
    "ddtree_topk_workspace_bytes": (_i32, [_i32, _i32, _i32, ctypes.POINTER(_sz)]),
    "ddtree_topk": (_i32, [_vp, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _sz, _vp]),
    "ddtree_build": (_i32, [_vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp]),
    "ddtree_tree_attn_workspace_bytes": (_i32, [_i32, _i32, _i32, _i32, _i32, ctypes.POINTER(_sz)]),
    "ddtree_tree_attn": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _vp,
                                _i32, _vp, _vp, _sz, _vp]),
    "ddtree_tree_attn_noalloc": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
                                        _vp, _i32, _vp, _vp]),
    "ddtree_target_argmax_workspace_bytes": (_i32, [_i32, _i32, _i32, ctypes.POINTER(_sz)]),
    "ddtree_target_argmax": (_i32, [_vp, _i32, _i64, _i32, _i32, _vp, _vp, _sz, _vp]),
    "ddtree_budget_select": (_i32, [_vp, _i32, _i32, ctypes.c_double, ctypes.c_double, _vp, _vp,
                                    _vp]),
    "ddtree_target_sample": (_i32, [_vp, _i32, _i64, _i32, _i32, _f32, _u64, _u64, _vp, _vp, _sz,
                                    _vp]),
    "ddtree_tree_prune": (_i32, [_vp, _i32, _vp, _vp, _i32, _vp]),
    "ddtree_accept_walk": (_i32, [_vp, _vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp]),
    "ddtree_kv_compact": (_i32, [_vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp]),
    "ddtree_build_batched": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                                    _i32, _vp]),
    "ddtree_tree_attn_batched_workspace_bytes": (_i32, [_i32, _vp, _i32, _i32, _i32, _i32,
                                                        ctypes.POINTER(_sz)]),
    "ddtree_tree_attn_batched": (_i32, [_vp, _vp, _vp, _i64, _i32, _vp, _i32, _i32, _i32, _i32,
                                        _i32, _f32, _vp, _i32, _vp, _vp, _sz, _vp]),
    "ddtree_accept_walk_batched": (_i32, [_vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp]),
    "ddtree_kv_compact_batched": (_i32, [_vp, _i32, _i32, _i32, _i32, _i32, _vp, _i32, _i32, _vp,
                                         _vp, _vp]),
}
EXPORTS = tuple(_SIGNATURES)


class DDTreeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {ddtree_status_string(status)}")


def lib() -> ctypes.CDLL:
    """The loaded libddtree.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing; build it with "
                "`python -m block_diffusion_draft_ddtree_amd.build_lib`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(status: int, where: str) -> None:
    if status != DDTREE_OK:
        raise DDTreeError(status, where)


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return int(getattr(stream, "cuda_stream", stream))


def _dev(t: torch.Tensor, dtype, name: str) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def ddtree_status_string(status: int) -> str:
    return lib().ddtree_status_string(int(status)).decode()


def ddtree_version() -> int:
    return lib().ddtree_version()


def ddtree_topk_workspace_bytes(L: int, V: int, K: int) -> int:
    out = _sz(0)
    _check(lib().ddtree_topk_workspace_bytes(L, V, K, ctypes.byref(out)), "ddtree_topk_workspace_bytes")
    return out.value


def ddtree_tree_attn_workspace_bytes(N: int, Hq: int, Hkv: int, D: int, S: int) -> int:
    out = _sz(0)
    _check(lib().ddtree_tree_attn_workspace_bytes(N, Hq, Hkv, D, S, ctypes.byref(out)),
           "ddtree_tree_attn_workspace_bytes")
    return out.value


def ddtree_target_argmax_workspace_bytes(dtype: int, N: int, V: int) -> int:
    out = _sz(0)
    _check(lib().ddtree_target_argmax_workspace_bytes(dtype, N, V, ctypes.byref(out)),
           "ddtree_target_argmax_workspace_bytes")
    return out.value


def workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def ddtree_topk(logits: torch.Tensor, K: int, logp=None, token=None, ws=None, stream=None):
    """fp32 logits [L, V] (row stride may exceed V) -> (logp fp32 [L, K], token int32 [L, K])."""
    if logits.dim() != 2 or logits.stride(1) != 1:
        raise ValueError("logits must be [L, V] with unit column stride")
    L, V = logits.shape
    if logits.dtype != torch.float32 or not logits.is_cuda:
        raise ValueError("logits must be a float32 device tensor")
    dev = logits.device
    logp = torch.empty((L, K), dtype=torch.float32, device=dev) if logp is None else logp
    token = torch.empty((L, K), dtype=torch.int32, device=dev) if token is None else token
    need = ddtree_topk_workspace_bytes(L, V, K)
    ws = workspace(need, dev) if ws is None else ws
    _check(lib().ddtree_topk(logits.data_ptr(), logits.stride(0), L, V, K,
                             _dev(logp, torch.float32, "logp"), _dev(token, torch.int32, "token"),
                             _dev(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)), "ddtree_topk")
    return logp, token


def ddtree_build(logp: torch.Tensor, token: torch.Tensor, B: int, root_token: torch.Tensor,
                 mask_words: int | None = None, parent=None, depth=None, node_token=None,
                 score=None, anc=None, want_score: bool = True, stream=None):
    """[L, K] tables -> (parent, depth, node_token, score, anc) for N = B + 1 nodes."""
    L, K = logp.shape
    N = B + 1
    W = (N + 31) // 32 if mask_words is None else mask_words
    dev = logp.device
    i32 = dict(dtype=torch.int32, device=dev)
    parent = torch.empty(N, **i32) if parent is None else parent
    depth = torch.empty(N, **i32) if depth is None else depth
    node_token = torch.empty(N, **i32) if node_token is None else node_token
    if score is None and want_score:
        score = torch.empty(N, dtype=torch.float32, device=dev)
    anc = torch.empty((N, W), **i32) if anc is None else anc
    _check(lib().ddtree_build(
        _dev(logp, torch.float32, "logp"), _dev(token, torch.int32, "token"), L, K, B,
        _dev(root_token, torch.int32, "root_token"), _dev(parent, torch.int32, "parent"),
        _dev(depth, torch.int32, "depth"), _dev(node_token, torch.int32, "node_token"),
        None if score is None else _dev(score, torch.float32, "score"),
        _dev(anc, anc.dtype, "anc"), W, _stream(stream)), "ddtree_build")
    return parent, depth, node_token, score, anc


def ddtree_tree_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, S: int,
                     anc: torch.Tensor, scale: float | None = None, out=None, ws=None,
                     stream=None) -> torch.Tensor:
    """q bf16 [N, Hq, D]; k, v bf16 [Hkv, S_cap, D]; anc [N, W] -> out bf16 [N, Hq, D]."""
    N, Hq, D = q.shape
    Hkv, S_cap, Dk = k.shape
    if Dk != D or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must be [Hkv, S_cap, D] with q's D")
    if anc.dim() != 2 or anc.shape[0] < N:
        raise ValueError("anc must be [N, mask_words]")
    scale = float(D) ** -0.5 if scale is None else float(scale)
    out = torch.empty_like(q) if out is None else out
    need = ddtree_tree_attn_workspace_bytes(N, Hq, Hkv, D, S)
    if ws is None:
        ws = workspace(need, q.device)
    _check(lib().ddtree_tree_attn(
        _dev(q, torch.bfloat16, "q"), _dev(k, torch.bfloat16, "k"), _dev(v, torch.bfloat16, "v"),
        S, S_cap, N, Hq, Hkv, D, scale, _dev(anc, anc.dtype, "anc"), anc.shape[1],
        _dev(out, torch.bfloat16, "out"), _dev(ws, torch.uint8, "ws"), ws.numel(),
        _stream(stream)), "ddtree_tree_attn")
    return out


def ddtree_tree_attn_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, S: int,
                             anc: torch.Tensor, scale: float | None = None, out=None,
                             stream=None) -> torch.Tensor:
    """ddtree_tree_attn with the library's static scratch instead of a
    workspace (nothing is allocated when `out` is given)."""
    N, Hq, D = q.shape
    Hkv, S_cap, Dk = k.shape
    if Dk != D or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must be [Hkv, S_cap, D] with q's D")
    if anc.dim() != 2 or anc.shape[0] < N:
        raise ValueError("anc must be [N, mask_words]")
    scale = float(D) ** -0.5 if scale is None else float(scale)
    out = torch.empty_like(q) if out is None else out
    _check(lib().ddtree_tree_attn_noalloc(
        _dev(q, torch.bfloat16, "q"), _dev(k, torch.bfloat16, "k"), _dev(v, torch.bfloat16, "v"),
        S, S_cap, N, Hq, Hkv, D, scale, _dev(anc, anc.dtype, "anc"), anc.shape[1],
        _dev(out, torch.bfloat16, "out"), _stream(stream)), "ddtree_tree_attn_noalloc")
    return out


def ddtree_target_argmax(logits: torch.Tensor, out=None, ws=None, stream=None) -> torch.Tensor:
    """fp32 or bf16 logits [N, V] (row stride may exceed V) -> int32 [N] on the device.

    ws: a uint8 device tensor of at least ddtree_target_argmax_workspace_bytes()
    bytes (allocated when None)."""
    if logits.dim() != 2 or logits.stride(1) != 1:
        raise ValueError("logits must be [N, V] with unit column stride")
    if not logits.is_cuda or logits.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("logits must be a float32 or bfloat16 device tensor")
    N, V = logits.shape
    dtype = DDTREE_DTYPE_BF16 if logits.dtype == torch.bfloat16 else DDTREE_DTYPE_F32
    if ws is None:
        ws = workspace(ddtree_target_argmax_workspace_bytes(dtype, N, V), logits.device)
    out = torch.empty(N, dtype=torch.int32, device=logits.device) if out is None else out
    _check(lib().ddtree_target_argmax(logits.data_ptr(), dtype, logits.stride(0), N, V,
                                      _dev(out, torch.int32, "out"), ws.data_ptr(), ws.numel(),
                                      _stream(stream)),
           "ddtree_target_argmax")
    return out


def ddtree_target_sample(logits: torch.Tensor, temperature: float, seed: int, offset: int,
                         out=None, ws=None, stream=None) -> torch.Tensor:
    """fp32 or bf16 logits [N, V] (row stride may exceed V) -> int32 [N]: one
    token per node drawn from softmax(logits / temperature) (Gumbel-max over
    Philox4x32-10 uniforms keyed by seed, counter offset)."""
    if logits.dim() != 2 or logits.stride(1) != 1:
        raise ValueError("logits must be [N, V] with unit column stride")
    if not logits.is_cuda or logits.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("logits must be a float32 or bfloat16 device tensor")
    N, V = logits.shape
    dtype = DDTREE_DTYPE_BF16 if logits.dtype == torch.bfloat16 else DDTREE_DTYPE_F32
    if ws is None:
        ws = workspace(ddtree_target_argmax_workspace_bytes(dtype, N, V), logits.device)
    out = torch.empty(N, dtype=torch.int32, device=logits.device) if out is None else out
    _check(lib().ddtree_target_sample(logits.data_ptr(), dtype, logits.stride(0), N, V,
                                      float(temperature), int(seed) & (2**64 - 1),
                                      int(offset) & (2**64 - 1), _dev(out, torch.int32, "out"),
                                      ws.data_ptr(), ws.numel(), _stream(stream)),
           "ddtree_target_sample")
    return out


def ddtree_budget_select(score: torch.Tensor, B_max: int, t0: float, t1: float, B_min: int = 1,
                         expected=None, budget=None, stream=None):
    """fp32 scores [>= B_max + 1] from ddtree_build -> (budget int32 [1],
    expected fp32 [B_max + 1]) on the device."""
    dev = score.device
    expected = torch.empty(B_max + 1, dtype=torch.float32, device=dev) if expected is None else expected
    budget = torch.empty(1, dtype=torch.int32, device=dev) if budget is None else budget
    if score.numel() < B_max + 1 or expected.numel() < B_max + 1:
        raise ValueError("score and expected need B_max + 1 entries")
    _check(lib().ddtree_budget_select(_dev(score, torch.float32, "score"), B_max, B_min, float(t0),
                                      float(t1), _dev(expected, torch.float32, "expected"),
                                      _dev(budget, torch.int32, "budget"), _stream(stream)),
           "ddtree_budget_select")
    return budget, expected


def ddtree_tree_prune(budget: torch.Tensor, parent: torch.Tensor, anc: torch.Tensor,
                      stream=None) -> None:
    """In place: nodes past budget[0] get parent -1 and an empty mask row."""
    N = parent.shape[0]
    if anc.dim() != 2 or anc.shape[0] != N:
        raise ValueError("anc must be [N, mask_words]")
    _check(lib().ddtree_tree_prune(_dev(budget, torch.int32, "budget"), N,
                                   _dev(parent, torch.int32, "parent"),
                                   _dev(anc, anc.dtype, "anc"), anc.shape[1], _stream(stream)),
           "ddtree_tree_prune")


def ddtree_accept_walk(parent: torch.Tensor, node_token: torch.Tensor, L: int,
                       target_argmax: torch.Tensor, acc=None, n_acc=None, next_bonus=None,
                       stream=None):
    """-> (acc int32 [L + 1], n_acc int32 [1], next_bonus int32 [1]) on the device."""
    N = parent.shape[0]
    dev = parent.device
    i32 = dict(dtype=torch.int32, device=dev)
    acc = torch.empty(L + 1, **i32) if acc is None else acc
    n_acc = torch.empty(1, **i32) if n_acc is None else n_acc
    next_bonus = torch.empty(1, **i32) if next_bonus is None else next_bonus
    _check(lib().ddtree_accept_walk(
        _dev(parent, torch.int32, "parent"), _dev(node_token, torch.int32, "node_token"), N, L,
        _dev(target_argmax, torch.int32, "target_argmax"), _dev(acc, torch.int32, "acc"),
        _dev(n_acc, torch.int32, "n_acc"), _dev(next_bonus, torch.int32, "next_bonus"),
        _stream(stream)), "ddtree_accept_walk")
    return acc, n_acc, next_bonus


def ddtree_kv_compact(kv: torch.Tensor, S: int, N: int, L: int, acc: torch.Tensor,
                      n_acc: torch.Tensor, stream=None) -> None:
    """In place on kv bf16 [layers, 2, Hkv, S_cap, D]."""
    layers, two, Hkv, S_cap, D = kv.shape
    if two != 2:
        raise ValueError("kv must be [layers, 2, Hkv, S_cap, D]")
    _check(lib().ddtree_kv_compact(
        _dev(kv, torch.bfloat16, "kv"), layers, Hkv, S_cap, D, S, N, L,
        _dev(acc, torch.int32, "acc"), _dev(n_acc, torch.int32, "n_acc"), _stream(stream)),
        "ddtree_kv_compact")


# ---- several requests per call ---------------------------------------------

def _host_ints(values) -> ctypes.Array:
    vals = [int(x) for x in values]
    return (ctypes.c_int32 * len(vals))(*vals)


def ddtree_build_batched(logp: torch.Tensor, token: torch.Tensor, B: int,
                         root_token: torch.Tensor, mask_words: int | None = None, out=None,
                         stream=None):
    """[R, L, K] tables, root_token int32 [R] -> (parent, depth, node_token,
    score) int32/fp32 [R, B + 1] and anc [R, B + 1, W]; `out` may supply
    those five tensors (then nothing is allocated)."""
    R, L, K = logp.shape
    N = B + 1
    W = (N + 31) // 32 if mask_words is None else mask_words
    dev = logp.device
    i32 = dict(dtype=torch.int32, device=dev)
    if out is None:
        parent, depth, node_token = (torch.empty((R, N), **i32) for _ in range(3))
        score = torch.empty((R, N), dtype=torch.float32, device=dev)
        anc = torch.empty((R, N, W), **i32)
    else:
        parent, depth, node_token, score, anc = out
    _check(lib().ddtree_build_batched(
        _dev(logp, torch.float32, "logp"), _dev(token, torch.int32, "token"), L, K, B, R,
        _dev(root_token, torch.int32, "root_token"), _dev(parent, torch.int32, "parent"),
        _dev(depth, torch.int32, "depth"), _dev(node_token, torch.int32, "node_token"),
        _dev(score, torch.float32, "score"), _dev(anc, torch.int32, "anc"), W, _stream(stream)),
        "ddtree_build_batched")
    return parent, depth, node_token, score, anc


def ddtree_tree_attn_batched_workspace_bytes(S, N: int, Hq: int, Hkv: int, D: int) -> int:
    out = _sz(0)
    _check(lib().ddtree_tree_attn_batched_workspace_bytes(len(S), _host_ints(S), N, Hq, Hkv, D,
                                                          ctypes.byref(out)),
           "ddtree_tree_attn_batched_workspace_bytes")
    return out.value


def ddtree_tree_attn_batched(q: torch.Tensor, kv: torch.Tensor, layer: int, S, anc: torch.Tensor,
                             scale: float | None = None, out=None, ws=None, stream=None):
    """q bf16 [R, N, Hq, D]; kv bf16 [R, layers, 2, Hkv, S_cap, D] (layer's
    K and V of every request); S host ints [R]; anc [R, N, W] -> out bf16
    [R, N, Hq, D]."""
    R, N, Hq, D = q.shape
    R2, layers, two, Hkv, S_cap, Dk = kv.shape
    if R2 != R or two != 2 or Dk != D or len(S) != R:
        raise ValueError("kv must be [R, layers, 2, Hkv, S_cap, D] matching q, S one per request")
    if not kv.is_contiguous() or kv.dtype != torch.bfloat16 or not kv.is_cuda:
        raise ValueError("kv must be a contiguous bf16 device tensor")
    if anc.dim() != 3 or anc.shape[0] != R or anc.shape[1] < N:
        raise ValueError("anc must be [R, N, mask_words]")
    scale = float(D) ** -0.5 if scale is None else float(scale)
    out = torch.empty_like(q) if out is None else out
    if ws is None:
        ws = workspace(ddtree_tree_attn_batched_workspace_bytes(S, N, Hq, Hkv, D), q.device)
    stride = layers * 2 * Hkv * S_cap * D
    _check(lib().ddtree_tree_attn_batched(
        _dev(q, torch.bfloat16, "q"), kv[0, layer, 0].data_ptr(), kv[0, layer, 1].data_ptr(),
        stride, R, _host_ints(S), S_cap, N, Hq, Hkv, D, scale, _dev(anc, anc.dtype, "anc"),
        anc.shape[2], _dev(out, torch.bfloat16, "out"), _dev(ws, torch.uint8, "ws"), ws.numel(),
        _stream(stream)), "ddtree_tree_attn_batched")
    return out


def ddtree_accept_walk_batched(parent: torch.Tensor, node_token: torch.Tensor, L: int,
                               target: torch.Tensor, out=None, stream=None):
    """[R, N] trees and target tokens -> (acc int32 [R, L + 1], n_acc int32
    [R], next_bonus int32 [R]); `out` may supply those three tensors."""
    R, N = parent.shape
    i32 = dict(dtype=torch.int32, device=parent.device)
    if out is None:
        acc = torch.empty((R, L + 1), **i32)
        n_acc = torch.empty(R, **i32)
        next_bonus = torch.empty(R, **i32)
    else:
        acc, n_acc, next_bonus = out
    _check(lib().ddtree_accept_walk_batched(
        _dev(parent, torch.int32, "parent"), _dev(node_token, torch.int32, "node_token"), N, L, R,
        _dev(target, torch.int32, "target"), _dev(acc, torch.int32, "acc"),
        _dev(n_acc, torch.int32, "n_acc"), _dev(next_bonus, torch.int32, "next_bonus"),
        _stream(stream)), "ddtree_accept_walk_batched")
    return acc, n_acc, next_bonus


def ddtree_kv_compact_batched(kv: torch.Tensor, S, N: int, L: int, acc: torch.Tensor,
                              n_acc: torch.Tensor, stream=None) -> None:
    """In place on kv bf16 [R, layers, 2, Hkv, S_cap, D]; S host ints [R]."""
    R, layers, two, Hkv, S_cap, D = kv.shape
    if two != 2 or len(S) != R:
        raise ValueError("kv must be [R, layers, 2, Hkv, S_cap, D], S one per request")
    _check(lib().ddtree_kv_compact_batched(
        _dev(kv, torch.bfloat16, "kv"), layers, Hkv, S_cap, D, R, _host_ints(S), N, L,
        _dev(acc, torch.int32, "acc"), _dev(n_acc, torch.int32, "n_acc"), _stream(stream)),
        "ddtree_kv_compact_batched")
