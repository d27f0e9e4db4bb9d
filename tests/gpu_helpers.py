"""Device helpers for the GPU parity tests (uploads, downloads, tolerances)."""
import sys

import numpy as np
import torch

DEV = "cuda:0"


def say(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a crash names it."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def up(a: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


def up_bf16(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> a bfloat16 device tensor with those bits."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV)
    return t.view(torch.bfloat16)


def down(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def down_bf16_f32(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.detach().float().cpu().numpy()


def down_bf16_bits(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


# Attention tolerance: |gpu - oracle| <= ATOL + RTOL * |oracle| element-wise
# (bf16 inputs, fp32 accumulation, bf16 softmax weights in P.V, bf16 output).
ATTN_ATOL = 2e-2
ATTN_RTOL = 1e-2
LOGP_ATOL = 1e-5

# Relative RMS error of the whole compared output against the fp64 oracle.
# The kernel rounds three times: the softmax weights to bf16 before P.V
# (unit roundoff u = 2^-9; the denominator sums the same rounded weights,
# so the output moves by sum_j w_j d_j (v_j - o), RMS about u / sqrt(3)
# relative to o for independent uniform d_j), each split's normalised
# output to fp16 (2^-11 relative, about 2^-11 / sqrt(3) after the convex
# merge) and the result to bf16 (u / sqrt(3)). In quadrature that is
# 1.6e-3; the bound allows 2.5 times that. Unlike the element-wise bar it
# scales with the output, so it sees errors in outputs of magnitude
# 1 / sqrt(S) (N(0, 1) inputs) that 2e-2 absolute cannot.
ATTN_REL_RMS = 4e-3


def assert_attn_close(got: np.ndarray, ref: np.ndarray, what: str = "") -> dict:
    assert np.isfinite(ref).all(), f"{what}: the oracle produced non-finite values"
    err = np.abs(got.astype(np.float64) - ref)
    bound = ATTN_ATOL + ATTN_RTOL * np.abs(ref)
    bad = ~(err <= bound)  # NaN outputs count as outside
    stats = {
        "max_abs": float(err.max()),
        "max_rel_to_max": float(err.max() / max(np.abs(ref).max(), 1e-30)),
        "rel_rms": float(np.sqrt((err ** 2).mean() / max((ref ** 2).mean(), 1e-30))),
    }
    assert not bad.any(), f"{what}: {int(bad.sum())} elements outside tolerance; {stats}"
    assert stats["rel_rms"] <= ATTN_REL_RMS, f"{what}: relative RMS error too large; {stats}"
    return stats
