"""The C ABI without a GPU: the library loads, exports every function that
include/ddtree.h declares, and rejects invalid arguments on the host with
the documented status codes before any HIP call (null pointers are passed
where a device buffer would go; validation never dereferences them)."""
import ctypes
import os
import re

import pytest

from block_diffusion_draft_ddtree_amd import binding as bd

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "ddtree.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bd.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return bd.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ddtree_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) == 20
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(bd.EXPORTS)


def test_status_strings_and_version(lib):
    assert bd.ddtree_status_string(0) == "DDTREE_OK"
    assert bd.ddtree_status_string(3) == "DDTREE_ERR_WORKSPACE_TOO_SMALL"
    assert bd.ddtree_status_string(99) == "DDTREE_ERR_UNKNOWN"
    assert bd.ddtree_version() >= 100


def test_workspace_queries(lib):
    ws = bd.ddtree_topk_workspace_bytes(16, 151936, 64)
    assert ws >= 16 * 38 * (64 + 256) * 8
    assert bd.ddtree_tree_attn_workspace_bytes(65, 32, 4, 128, 4096) > 0
    # a single split needs no workspace
    assert bd.ddtree_tree_attn_workspace_bytes(1, 1, 1, 64, 0) == 0
    for args in [(0, 10, 1), (1, 10, 11), (32 * 64 + 1, 10, 1), (1, 5000, 1025)]:
        with pytest.raises(bd.DDTreeError):
            bd.ddtree_topk_workspace_bytes(*args)
    with pytest.raises(bd.DDTreeError):
        bd.ddtree_tree_attn_workspace_bytes(65, 30, 4, 128, 4096)  # Hq % Hkv
    with pytest.raises(bd.DDTreeError):
        bd.ddtree_tree_attn_workspace_bytes(65, 32, 4, 96, 4096)   # D


# Head layouts of the workloads (N, Hq, Hkv, D): tiny; the 8B shape and the
# budget sweep at B = 64 and 512; the 30B shape at B = 64 and 256 (also the
# long-context shape); then two layouts at and past the switch to 128-row
# tiles (1024 query rows per kv-head; 1025 nodes at G = 1).
WORKLOAD_LAYOUTS = [(17, 4, 2, 64), (65, 32, 8, 128), (513, 32, 8, 128), (65, 32, 4, 128),
                    (257, 32, 4, 128), (128, 32, 4, 128), (1025, 8, 8, 64)]


@pytest.mark.parametrize("layout", WORKLOAD_LAYOUTS)
def test_attn_workspace_monotone_in_prefix(lib, layout):
    """A workspace sized for prefix length S serves every shorter prefix: the
    query never asks for more at a smaller S (a decode loop sizes it once at
    its largest S while S grows by each round's accepted tokens)."""
    N, Hq, Hkv, D = layout
    prev = 0
    for S in range(0, 65537):
        b = bd.ddtree_tree_attn_workspace_bytes(N, Hq, Hkv, D, S)
        assert b >= prev, (layout, S, b, prev)
        prev = b


@pytest.mark.parametrize("layout", WORKLOAD_LAYOUTS[1:3])
def test_batched_attn_workspace_monotone(lib, layout):
    """The batched query is non-decreasing in each request's prefix length."""
    import numpy as np
    N, Hq, Hkv, D = layout
    g = np.random.default_rng(7)
    for _ in range(200):
        R = int(g.integers(1, 9))
        S = g.integers(0, 20000, size=R)
        full = bd.ddtree_tree_attn_batched_workspace_bytes(S.tolist(), N, Hq, Hkv, D)
        r = int(g.integers(0, R))
        S2 = S.copy()
        S2[r] = int(g.integers(0, S[r] + 1))
        assert bd.ddtree_tree_attn_batched_workspace_bytes(S2.tolist(), N, Hq, Hkv, D) <= full


def P(v):
    return ctypes.c_void_p(v)


FAKE = 0x1000  # a 16-byte aligned non-null value; never dereferenced on error paths


def test_topk_validation(lib):
    f = lib.ddtree_topk
    assert f(P(FAKE), 1000, 4, 1000, 8, P(FAKE), P(FAKE), P(FAKE), 0, None) == bd.DDTREE_ERR_WORKSPACE_TOO_SMALL
    assert f(None, 1000, 4, 1000, 8, P(FAKE), P(FAKE), P(FAKE), 1 << 30, None) == bd.DDTREE_ERR_INVALID_ARGUMENT
    assert f(P(FAKE), 999, 4, 1000, 8, P(FAKE), P(FAKE), P(FAKE), 1 << 30, None) == bd.DDTREE_ERR_INVALID_ARGUMENT
    assert f(P(FAKE), 1000, 4, 1000, 1001, P(FAKE), P(FAKE), P(FAKE), 1 << 30, None) == bd.DDTREE_ERR_INVALID_ARGUMENT
    # Rows: up to DDTREE_MAX_L block positions of up to DDTREE_MAX_REQ requests.
    assert f(P(FAKE), 1000, 32 * 64 + 1, 1000, 8, P(FAKE), P(FAKE), P(FAKE), 1 << 30, None) == bd.DDTREE_ERR_UNSUPPORTED


def test_build_validation(lib):
    f = lib.ddtree_build
    ok = [P(FAKE)] * 2
    outs = [P(FAKE)] * 5
    # B larger than the number of prefixes (K=2, L=2 -> 6)
    assert f(*ok, 2, 2, 7, P(FAKE), *outs, 1, None) == bd.DDTREE_ERR_INVALID_ARGUMENT
    # mask words too few for N = 65
    assert f(*ok, 16, 64, 64, P(FAKE), *outs, 2, None) == bd.DDTREE_ERR_INVALID_ARGUMENT
    assert f(*ok, 16, 64, 1025, P(FAKE), *outs, 33, None) == bd.DDTREE_ERR_UNSUPPORTED
    assert f(*ok, 16, 64, 64, None, *outs, 3, None) == bd.DDTREE_ERR_INVALID_ARGUMENT


def test_attn_validation(lib):
    f = lib.ddtree_tree_attn
    args = lambda **kw: [kw.get("q", P(FAKE)), P(FAKE), P(FAKE), kw.get("S", 4096),
                         kw.get("S_cap", 4161), kw.get("N", 65), 32, 4, kw.get("D", 128),
                         ctypes.c_float(kw.get("scale", 0.088)), P(FAKE), kw.get("W", 3),
                         P(FAKE), P(FAKE), kw.get("ws", 0), None]
    assert f(*args()) == bd.DDTREE_ERR_WORKSPACE_TOO_SMALL
    assert f(*args(S_cap=4160, ws=1 << 40)) == bd.DDTREE_ERR_INVALID_ARGUMENT
    assert f(*args(W=2, ws=1 << 40)) == bd.DDTREE_ERR_INVALID_ARGUMENT
    assert f(*args(q=P(FAKE + 2), ws=1 << 40)) == bd.DDTREE_ERR_INVALID_ARGUMENT
    assert f(*args(D=96, ws=1 << 40)) == bd.DDTREE_ERR_UNSUPPORTED
    assert f(*args(scale=-1.0, ws=1 << 40)) == bd.DDTREE_ERR_INVALID_ARGUMENT
    assert f(*args(N=1026, S_cap=1 << 20, W=40, ws=1 << 40)) == bd.DDTREE_ERR_UNSUPPORTED


def test_attn_noalloc_validation(lib):
    """The allocation-free attention checks its arguments like ddtree_tree_attn
    and refuses, before any HIP call, a plan whose split partials exceed its
    static scratch (DDTREE_NOALLOC_SCRATCH_BYTES = 32 MiB)."""
    f = lib.ddtree_tree_attn_noalloc
    args = lambda S, S_cap, N, Hq, Hkv, D, scale=0.1, W=1: (
        P(FAKE), P(FAKE), P(FAKE), S, S_cap, N, Hq, Hkv, D, ctypes.c_float(scale), P(FAKE), W,
        P(FAKE), None)
    assert f(*args(100, 150, 65, 32, 4, 96, W=3)) == bd.DDTREE_ERR_UNSUPPORTED        # D
    assert f(*args(100, 150, 65, 30, 4, 128, W=3)) == bd.DDTREE_ERR_INVALID_ARGUMENT  # Hq % Hkv
    assert f(*args(100, 150, 65, 32, 4, 128, W=2)) == bd.DDTREE_ERR_INVALID_ARGUMENT  # mask words
    assert f(*args(100, 160, 65, 32, 4, 128, W=3)) == bd.DDTREE_ERR_INVALID_ARGUMENT  # S + N > S_cap
    assert f(*args(100, 200, 65, 32, 4, 128, 0.0, W=3)) == bd.DDTREE_ERR_INVALID_ARGUMENT  # scale
    # The largest tree at a long prefix needs more split partials than the
    # static scratch holds (its workspace query says so too).
    assert bd.ddtree_tree_attn_workspace_bytes(1025, 32, 8, 128, 60000) > 32 << 20
    assert f(*args(60000, 61025, 1025, 32, 8, 128, W=33)) == bd.DDTREE_ERR_WORKSPACE_TOO_SMALL


def test_prune_validation(lib):
    f = lib.ddtree_tree_prune
    assert f(P(FAKE), 65, P(FAKE), P(FAKE), 2, None) == bd.DDTREE_ERR_INVALID_ARGUMENT  # words
    assert f(None, 65, P(FAKE), P(FAKE), 3, None) == bd.DDTREE_ERR_INVALID_ARGUMENT
    assert f(P(FAKE), 0, P(FAKE), P(FAKE), 1, None) == bd.DDTREE_ERR_INVALID_ARGUMENT
    assert f(P(FAKE), 1026, P(FAKE), P(FAKE), 33, None) == bd.DDTREE_ERR_UNSUPPORTED


def test_walk_and_compact_validation(lib):
    w = lib.ddtree_accept_walk
    assert w(P(FAKE), P(FAKE), 65, 33, P(FAKE), P(FAKE), P(FAKE), P(FAKE), None) == bd.DDTREE_ERR_UNSUPPORTED
    assert w(P(FAKE), P(FAKE), 0, 16, P(FAKE), P(FAKE), P(FAKE), P(FAKE), None) == bd.DDTREE_ERR_INVALID_ARGUMENT
    assert w(P(FAKE), None, 65, 16, P(FAKE), P(FAKE), P(FAKE), P(FAKE), None) == bd.DDTREE_ERR_INVALID_ARGUMENT
    c = lib.ddtree_kv_compact
    assert c(P(FAKE), 48, 4, 4160, 128, 4096, 65, 16, P(FAKE), P(FAKE), None) == bd.DDTREE_ERR_INVALID_ARGUMENT
    assert c(P(FAKE), 48, 4, 4161, 96, 4096, 65, 16, P(FAKE), P(FAKE), None) == bd.DDTREE_ERR_UNSUPPORTED
    assert c(P(FAKE + 8), 48, 4, 4161, 128, 4096, 65, 16, P(FAKE), P(FAKE), None) == bd.DDTREE_ERR_INVALID_ARGUMENT


def test_target_argmax_validation(lib):
    a = lib.ddtree_target_argmax
    F32, BF16 = bd.DDTREE_DTYPE_F32, bd.DDTREE_DTYPE_BF16
    WS = 65 * 32 * 8  # 32 chunks of the 152k-entry bf16 row
    assert a(P(FAKE), F32, 151936, 0, 151936, P(FAKE), P(FAKE), WS, None) == bd.DDTREE_ERR_INVALID_ARGUMENT
    assert a(P(FAKE), F32, 151936, 65, 0, P(FAKE), P(FAKE), WS, None) == bd.DDTREE_ERR_INVALID_ARGUMENT
    assert a(P(FAKE), 7, 151936, 65, 151936, P(FAKE), P(FAKE), WS, None) == bd.DDTREE_ERR_INVALID_ARGUMENT
    assert a(P(FAKE), F32, 100, 65, 151936, P(FAKE), P(FAKE), WS, None) == bd.DDTREE_ERR_INVALID_ARGUMENT  # stride < V
    assert a(P(FAKE + 2), F32, 151936, 65, 151936, P(FAKE), P(FAKE), WS, None) == bd.DDTREE_ERR_INVALID_ARGUMENT  # fp32 misaligned
    assert a(None, BF16, 151936, 65, 151936, P(FAKE), P(FAKE), WS, None) == bd.DDTREE_ERR_INVALID_ARGUMENT
    assert a(P(FAKE), BF16, 151936, 65, 151936, None, P(FAKE), WS, None) == bd.DDTREE_ERR_INVALID_ARGUMENT
    assert a(P(FAKE), BF16, 151936, 65, 151936, P(FAKE), None, WS, None) == bd.DDTREE_ERR_INVALID_ARGUMENT
    assert a(P(FAKE), BF16, 151936, 65, 151936, P(FAKE), P(FAKE + 4), WS, None) == bd.DDTREE_ERR_INVALID_ARGUMENT  # ws misaligned
    assert a(P(FAKE), BF16, 151936, 65, 151936, P(FAKE), P(FAKE), WS - 1, None) == bd.DDTREE_ERR_WORKSPACE_TOO_SMALL
    assert a(P(FAKE), BF16, 151936, 1026, 151936, P(FAKE), P(FAKE), 1 << 20, None) == bd.DDTREE_ERR_UNSUPPORTED
    assert a(P(FAKE), BF16, 1 << 23, 65, (1 << 22) + 1, P(FAKE), P(FAKE), WS, None) == bd.DDTREE_ERR_UNSUPPORTED
    nb = ctypes.c_size_t(0)
    assert lib.ddtree_target_argmax_workspace_bytes(BF16, 65, 151936, ctypes.byref(nb)) == 0
    assert nb.value == WS
    assert lib.ddtree_target_argmax_workspace_bytes(BF16, 0, 151936, ctypes.byref(nb)) == bd.DDTREE_ERR_INVALID_ARGUMENT
    assert lib.ddtree_target_argmax_workspace_bytes(BF16, 65, 151936, None) == bd.DDTREE_ERR_INVALID_ARGUMENT


def test_target_sample_validation(lib):
    f = lib.ddtree_target_sample
    BF16 = bd.DDTREE_DTYPE_BF16
    WS = 65 * 32 * 8

    def call(logits=P(FAKE), dtype=BF16, stride=151936, N=65, V=151936, T=1.0, out=P(FAKE),
             w=P(FAKE), ws=WS):
        return f(logits, dtype, stride, N, V, T, 1, 2, out, w, ws, None)

    for T in (0.0, -1.0, float("nan"), float("inf"), 1e-39):
        assert call(T=T) == bd.DDTREE_ERR_INVALID_ARGUMENT, T
    assert call(T=3e38) == bd.DDTREE_ERR_INVALID_ARGUMENT  # log2(e) / T below fp32 normals
    assert call(N=0) == bd.DDTREE_ERR_INVALID_ARGUMENT
    assert call(dtype=5) == bd.DDTREE_ERR_INVALID_ARGUMENT
    assert call(stride=10) == bd.DDTREE_ERR_INVALID_ARGUMENT
    assert call(logits=None) == bd.DDTREE_ERR_INVALID_ARGUMENT
    assert call(out=None) == bd.DDTREE_ERR_INVALID_ARGUMENT
    assert call(w=None) == bd.DDTREE_ERR_INVALID_ARGUMENT
    assert call(w=P(FAKE + 4)) == bd.DDTREE_ERR_INVALID_ARGUMENT
    assert call(ws=WS - 1) == bd.DDTREE_ERR_WORKSPACE_TOO_SMALL
    assert call(N=1026, ws=1 << 20) == bd.DDTREE_ERR_UNSUPPORTED


def test_budget_select_validation(lib):
    f = lib.ddtree_budget_select
    E = bd.DDTREE_ERR_INVALID_ARGUMENT
    assert f(P(FAKE), 0, 0, 1.0, 0.1, None, P(FAKE), None) == E
    assert f(P(FAKE), 64, 65, 1.0, 0.1, None, P(FAKE), None) == E
    assert f(P(FAKE), 64, -1, 1.0, 0.1, None, P(FAKE), None) == E
    assert f(P(FAKE), 1025, 1, 1.0, 0.1, None, P(FAKE), None) == bd.DDTREE_ERR_UNSUPPORTED
    assert f(None, 64, 1, 1.0, 0.1, None, P(FAKE), None) == E
    assert f(P(FAKE), 64, 1, 1.0, 0.1, None, None, None) == E
    for t0, t1 in ((0.0, 0.0), (-1.0, 0.1), (1.0, -0.1), (float("nan"), 0.1), (float("inf"), 0.1),
                   (1.0, float("inf"))):
        assert f(P(FAKE), 64, 1, t0, t1, None, P(FAKE), None) == E, (t0, t1)


def test_batched_validation(lib):
    E, U = bd.DDTREE_ERR_INVALID_ARGUMENT, bd.DDTREE_ERR_UNSUPPORTED
    b = lib.ddtree_build_batched
    args = [P(FAKE), P(FAKE), 16, 64, 64, 4, P(FAKE), P(FAKE), P(FAKE), P(FAKE), None, P(FAKE), 3, None]
    a = list(args); a[5] = 0
    assert b(*a) == E
    a = list(args); a[5] = 65
    assert b(*a) == U
    a = list(args); a[6] = None
    assert b(*a) == E
    w = lib.ddtree_accept_walk_batched
    assert w(P(FAKE), P(FAKE), 65, 16, 0, P(FAKE), P(FAKE), P(FAKE), P(FAKE), None) == E
    assert w(P(FAKE), P(FAKE), 65, 16, 65, P(FAKE), P(FAKE), P(FAKE), P(FAKE), None) == U
    S = bd._host_ints([4096, 100, 0])
    nb = ctypes.c_size_t(0)
    q = lib.ddtree_tree_attn_batched_workspace_bytes
    assert q(3, S, 65, 32, 4, 128, ctypes.byref(nb)) == 0 and nb.value > 0
    assert q(0, S, 65, 32, 4, 128, ctypes.byref(nb)) == E
    assert q(65, S, 65, 32, 4, 128, ctypes.byref(nb)) == U
    assert q(3, None, 65, 32, 4, 128, ctypes.byref(nb)) == E
    assert q(3, bd._host_ints([1, -1, 2]), 65, 32, 4, 128, ctypes.byref(nb)) == E
    t = lib.ddtree_tree_attn_batched
    stride = 48 * 2 * 4 * 4200 * 128
    ok = [P(FAKE), P(FAKE), P(FAKE), stride, 3, S, 4200, 65, 32, 4, 128, 0.088, P(FAKE), 3,
          P(FAKE), P(FAKE), 1 << 30, None]
    x = list(ok); x[6] = 4160  # 4096 + 65 > S_cap
    assert t(*x) == E
    x = list(ok); x[3] = 4 * 4200 * 128 - 8  # stride below one request's block
    assert t(*x) == E
    x = list(ok); x[3] = stride + 4  # stride breaks 16-byte alignment
    assert t(*x) == E
    x = list(ok); x[16] = 0
    assert t(*x) == bd.DDTREE_ERR_WORKSPACE_TOO_SMALL
    c = lib.ddtree_kv_compact_batched
    assert c(P(FAKE), 48, 4, 4160, 128, 3, S, 65, 16, P(FAKE), P(FAKE), None) == E
    assert c(P(FAKE), 48, 4, 4200, 128, 3, None, 65, 16, P(FAKE), P(FAKE), None) == E
    assert c(P(FAKE), 48, 4, 4200, 128, 65, S, 65, 16, P(FAKE), P(FAKE), None) == U
