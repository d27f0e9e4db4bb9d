"""The seeded input generators: reproducible and shaped as the workloads say."""
import numpy as np
import torch

from block_diffusion_draft_ddtree_amd import synth


def test_same_seed_same_bytes():
    a = synth.drafter_logits(synth.TINY, 3)
    b = synth.drafter_logits(synth.TINY, 3)
    assert a.x.tobytes() == b.x.tobytes()
    c = synth.drafter_logits(synth.TINY, 4)
    assert a.x.tobytes() != c.x.tobytes()
    q1 = synth.attention_inputs(synth.TINY)
    q2 = synth.attention_inputs(synth.TINY)
    assert q1.kv_bits.tobytes() == q2.kv_bits.tobytes()


def test_bf16_rounding_matches_torch():
    g = synth.rng("test", 50, 0)
    x = (g.standard_normal(100000) * 10).astype(np.float32)
    bits = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, ref)
    np.testing.assert_array_equal(synth.bf16_bits_to_f32(bits),
                                  torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_peaked_generator_shape():
    w = synth.QWEN3_8B
    lg = synth.drafter_logits(w)
    assert lg.x.shape == (16, 151936) and lg.x.dtype == np.float32
    assert np.all(lg.peak != lg.runner)
    # Regenerating the unboosted bulk from the same stream isolates the boosts.
    g = synth.rng(w.family, 0, synth.STREAM_LOGITS)
    bulk = np.float32(2.0) * g.standard_normal((16, 151936), dtype=np.float32)
    i = np.arange(16)
    np.testing.assert_allclose(lg.x[i, lg.peak] - bulk[i, lg.peak], 9.0 - 0.4 * i, atol=1e-5)
    np.testing.assert_allclose(lg.x[i, lg.runner] - bulk[i, lg.runner], 7.0 - 0.4 * i, atol=1e-5)


def test_confident_generator():
    w = synth.CODER30B_B64_DEEP
    lg = synth.drafter_logits(w)
    assert lg.x.shape == (16, 151936) and lg.x.dtype == np.float32
    assert np.all(lg.peak != lg.runner)
    # The softmax (fp64) of each row gives the designed peak and runner-up
    # probabilities, and every other token keeps its N(0,1) bulk logit.
    x = lg.x.astype(np.float64)
    q = np.exp(x - x.max(axis=1, keepdims=True))
    q /= q.sum(axis=1, keepdims=True)
    i = np.arange(16)
    p_peak, p_run = synth.confident_probs(16)
    np.testing.assert_allclose(q[i, lg.peak], p_peak, rtol=1e-5)
    np.testing.assert_allclose(q[i, lg.runner], p_run, rtol=1e-5)
    assert np.all(p_peak[:-1] > p_peak[1:])  # confidence decays along the block
    g = synth.rng(w.family, 0, synth.STREAM_LOGITS)
    bulk = g.standard_normal((16, 151936), dtype=np.float32)
    keep = np.ones_like(bulk, dtype=bool)
    keep[i, lg.peak] = keep[i, lg.runner] = False
    np.testing.assert_array_equal(lg.x[keep], bulk[keep])


def test_workload_table():
    w = synth.CODER30B_B64
    assert (w.N, w.G, w.mask_words, w.S_cap) == (65, 8, 3, 4096 + 65)
    assert synth.sweep(512).mask_words == 17
