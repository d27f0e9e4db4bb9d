"""GPU: ddtree_tree_attn_noalloc (static scratch, no workspace argument)
against ddtree_tree_attn on the same inputs, through the C ABI: two calls in
a row, the second on a smaller input, each bit-identical to the workspace
entry and within the attention bar of the oracle."""
import numpy as np
import pytest

from block_diffusion_draft_ddtree_amd import binding as bd
from block_diffusion_draft_ddtree_amd import synth
from oracle import attention as oa
from oracle import tree as ot

from gpu_helpers import assert_attn_close, down_bf16_bits, down_bf16_f32, say, up, up_bf16

pytestmark = pytest.mark.gpu


def _case(N, Hq, Hkv, D, S, seed):
    g = synth.rng("test", 900 + seed, 0)
    q_bits, q = synth.normal_bf16(g, (N, Hq, D))
    kv_bits, kv = synth.normal_bf16(g, (2, Hkv, S + N, D))
    parent = [-1] + [int(g.integers(0, n)) for n in range(1, N)]
    anc = ot.ancestor_mask(parent)
    return q_bits, q, kv_bits, kv, anc


def _check(N, Hq, Hkv, D, S, seed):
    q_bits, q, kv_bits, kv, anc = _case(N, Hq, Hkv, D, S, seed)
    say(f"attn noalloc N={N} Hq={Hq} Hkv={Hkv} D={D} S={S}")
    qd, kvd, ancd = up_bf16(q_bits), up_bf16(kv_bits), up(anc.view(np.int32))
    got = bd.ddtree_tree_attn_noalloc(qd, kvd[0], kvd[1], S, ancd)
    ref_ws = bd.ddtree_tree_attn(qd, kvd[0], kvd[1], S, ancd)
    np.testing.assert_array_equal(down_bf16_bits(got), down_bf16_bits(ref_ws))
    ref = oa.tree_attention(q, kv[0], kv[1], S, anc)
    assert_attn_close(down_bf16_f32(got), ref, f"noalloc N={N} S={S}")
    return bd.ddtree_tree_attn_workspace_bytes(N, Hq, Hkv, D, S)


def test_noalloc_matches_workspace_entry_two_calls():
    # The 30B verifier shape (7 splits), then a smaller split input, then one
    # that needs no scratch at all.
    assert _check(65, 32, 4, 128, 4096, 1) > 0
    assert _check(33, 8, 2, 64, 700, 2) > 0
    assert _check(9, 4, 2, 64, 20, 3) == 0


def test_noalloc_tall_tiles():
    # 1032 query rows per kv-head (128-row tiles), then the 30B shape again
    # (64-row tiles) in the same scratch array.
    assert _check(129, 32, 4, 128, 2000, 4) > 0
    assert _check(65, 32, 4, 128, 4096, 5) > 0
