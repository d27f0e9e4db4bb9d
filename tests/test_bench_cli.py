"""bench.py's command line without a GPU: more than one GPU is refused with
a message, and the help text lists the documented flags."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    res = _run("--gpus", "2")
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def test_help_lists_flags():
    res = _run("--help")
    assert res.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup", "--workload", "--graph", "--no-cpu-baseline",
                 "--batch-requests", "--copy-probe"):
        assert flag in res.stdout, flag


def test_stage_roofline_and_build_forms():
    """The bench helpers that need no GPU: the streaming stages' HBM fractions
    follow from their algorithmic bytes and times, and both oracle top-B
    constructions time the same tree."""
    sys.path.insert(0, ROOT)
    import bench
    from block_diffusion_draft_ddtree_amd import synth
    from oracle import softmax_topk as st
    from oracle import tree as ot

    w = synth.WORKLOADS["coder30b_b64"]
    r = bench.stage_roofline(w, {"topk": 12.0, "target_argmax": 8.0, "kv_compact": 2.0}, 3)
    assert r["topk"]["algorithmic_bytes"] == 4 * w.L * w.V + 8 * w.L * w.K
    assert r["kv_compact"]["algorithmic_bytes"] == 8 * 3 * w.layers * w.Hkv * w.D
    for v in r.values():
        assert abs(v["frac"] - v["algorithmic_bytes"] / (v["us"] * 1e-6) / 8e12) < 1e-4
        assert abs(v["floor_us"] - v["algorithmic_bytes"] / 8e6) < 1e-3
    tiny = synth.TINY
    lg = synth.drafter_logits(tiny)
    forms = bench.oracle_build_forms(tiny, lg)
    assert set(forms) == {"sort_fixed_point", "best_first_heap"}
    lp, _ = st.topk(lg.x, tiny.K)
    lp32 = lp.astype("float32")
    assert ot.top_b_sort_expand(lp32, tiny.B) == ot.top_b_best_first(lp32, tiny.B)
