"""GPU parity: ddtree_target_argmax against the oracle, index for index.

The target's greedy choice after each tree node ("DDTree Deep Dive", section
6): the first index of the row maximum compared as fp32. Integer output, so
the comparison is exact. Rows are placed at every alignment (row strides that
are not multiples of the 16-byte vector width) so that the scalar head, the
vector body and the scalar tail of a row all hold maxima and ties."""
import numpy as np
import pytest
import torch

from block_diffusion_draft_ddtree_amd import binding as bd
from block_diffusion_draft_ddtree_amd import synth
from oracle import commit as oc

from gpu_helpers import say

pytestmark = pytest.mark.gpu


_WS = {}


def _ws():
    """One workspace shared by every call of this module, as a caller would
    keep it (large enough for every shape here; filled with 0xFF so that a
    slot read before it is written would win every max)."""
    if "ws" not in _WS:
        _WS["ws"] = torch.full((1 << 20,), 255, dtype=torch.uint8, device="cuda")
    return _WS["ws"]


def _run(x32: np.ndarray, dtype, stride=None):
    """x32: fp32 values [N, V] (exactly representable in dtype)."""
    N, V = x32.shape
    stride = V if stride is None else stride
    say(f"target_argmax N={N} V={V} stride={stride} dtype={dtype}")
    buf = torch.zeros((N, stride), dtype=torch.float32)
    buf[:, :V] = torch.from_numpy(x32)
    dev = buf.to(dtype).cuda()
    return bd.ddtree_target_argmax(dev[:, :V], ws=_ws()).cpu().numpy()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_workload_shapes(dtype):
    g = synth.rng("test", 670, int(dtype == torch.bfloat16))
    for N in (1, 17, 65, 257):
        peaks = g.integers(0, 151936, size=N)
        _, x = synth.target_logits(g, N, 151936, peaks=peaks if N % 2 else None)
        got = _run(x, dtype)
        np.testing.assert_array_equal(got, oc.target_argmax(x))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("V", [1, 3, 7, 8, 9, 15, 16, 17, 1000, 4099, 33333])
def test_ties_alignments_and_ragged_rows(dtype, V):
    g = synth.rng("test", 671, V)
    N = 23
    x = np.round(g.standard_normal((N, V)).astype(np.float32) * 2.0) / 2.0  # many exact ties
    x[0] = -np.inf                                  # a fully masked row
    x[1] = 0.0
    x[1, ::2] = -0.0                                # -0 and +0 tie
    for n in range(2, N):                           # the maximum at several places
        m = float(x[n].max()) + 1.0
        for pos in g.choice(V, size=min(V, 3), replace=False):
            x[n, pos] = m
    for stride in (V, V + 1, V + 3, V + 5):         # rows at every alignment
        got = _run(x, dtype, stride)
        np.testing.assert_array_equal(got, oc.target_argmax(x), err_msg=f"stride {stride}")


def test_max_rows_sampled():
    """N = DDTREE_MAX_B + 1 rows of the full vocabulary: sampled rows."""
    g = synth.rng("test", 672, 0)
    N, V = 1025, 151936
    bits, _ = synth.target_logits(g, N, V, peaks=g.integers(0, V, size=N))
    say(f"target_argmax N={N} V={V} bf16 sampled")
    dev = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    got = bd.ddtree_target_argmax(dev, ws=_ws()).cpu().numpy()
    rows = g.choice(N, size=40, replace=False)
    x = synth.bf16_bits_to_f32(bits[rows])
    np.testing.assert_array_equal(got[rows], oc.target_argmax(x))
    assert got.min() >= 0 and got.max() < V


def test_repeated_calls_one_stream():
    """Back-to-back calls on one stream reuse one workspace before the host
    looks at anything: each result still matches."""
    g = synth.rng("test", 673, 0)
    shapes = [(65, 151936), (3, 50000), (65, 151936), (257, 4099), (1, 151936)]
    xs, outs = [], []
    for N, V in shapes:
        _, x = synth.target_logits(g, N, V, peaks=g.integers(0, V, size=N))
        xs.append(x)
    say("target_argmax repeated calls " + str(shapes))
    devs = [torch.from_numpy(x).to(torch.bfloat16).cuda() for x in xs]
    for d in devs:
        outs.append(bd.ddtree_target_argmax(d, ws=_ws()))
    for x, o in zip(xs, outs):
        np.testing.assert_array_equal(o.cpu().numpy(), oc.target_argmax(x))
