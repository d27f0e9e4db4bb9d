"""Benchmark of one DDTree verify round on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input
already resident in HBM: ddtree_topk -> ddtree_build -> ddtree_tree_attn for
every layer -> ddtree_accept_walk -> ddtree_kv_compact. Default workload:
the Qwen3-Coder-30B-A3B verifier shape (32 q-heads / 4 kv-heads, head dim
128, 48 layers, prefix 4096) with drafter logits [16, 151936] and budget
B = 64. Prints one JSON line.

The round is timed as three HIP graph replays per step (top-K and build;
the attention of every layer; walk and compaction), with events between
them timing the attention; --eager launches every kernel instead. The
same steps are also timed with eager launches (eager_us_per_step).

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--eager]
    python bench.py --copy-probe     # plain device copy of known size (for
                                     # scaling the HBM byte counters)

roofline.traffic is the measured HBM bytes of one ddtree_tree_attn call
(both of its kernels), read from the counter summary under profiles/ when
that summary was taken on the current attention source (its sha256 is
recorded there); otherwise null.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
ROOT = os.path.dirname(os.path.abspath(__file__))
ATTN_SOURCE = os.path.join(ROOT, "block_diffusion_draft_ddtree_amd", "csrc", "attn.hip")
COPY_PROBE_BYTES = 256 << 20  # bytes read and bytes written by the copy probe
SPIN_CYCLES = 10_000_000      # ~5 ms of device spin ahead of each stage's timed reps
# Round time t0 + t1 * nodes fitted to the autobench Qwen3-Coder-30B page's
# budget-64 and budget-256 rows (tokens per step / tokens per second).
BUDGET_T1 = (3.69 / 17.32 - 3.22 / 20.75) / (257 - 65)
BUDGET_T0 = 3.22 / 20.75 - BUDGET_T1 * 65


def traffic_summary_path(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"tree_attn_{workload}_traffic.txt")


def measured_traffic(workload: str):
    """HBM bytes per ddtree_tree_attn call from the committed counter
    summary, or None when there is none or it predates the current kernel
    source."""
    path = traffic_summary_path(workload)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line:
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    with open(ATTN_SOURCE, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    if fields.get("attn_source_sha256") != sha or "traffic_bytes_per_call" not in fields:
        return None
    return int(fields["traffic_bytes_per_call"])


def copy_probe():
    """A plain device-to-device copy of COPY_PROBE_BYTES, five times: what
    FETCH_SIZE and WRITE_SIZE read for it gives their scale to bytes."""
    import torch
    dev = torch.device("cuda:0")
    n = COPY_PROBE_BYTES // 4
    src = torch.arange(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    assert bool(torch.equal(dst[-8:], src[-8:]))
    print(json.dumps({"copy_probe_bytes": COPY_PROBE_BYTES, "launches": 5}), flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="coder30b_b64")
    ap.add_argument("--graph", action="store_true",
                    help="replay the round as HIP graphs (the default)")
    ap.add_argument("--eager", action="store_true",
                    help="launch every kernel of the timed round instead of replaying graphs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--stage-reps", type=int, default=30)
    ap.add_argument("--copy-probe", action="store_true",
                    help="run only the plain copy used to scale the byte counters")
    ap.add_argument("--batch-requests", type=int, default=8,
                    help="requests in the batched-round leg (0 skips it)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workload shapes (8B, 30B at B = 256, long context)")
    ap.add_argument("--no-budget-round", action="store_true",
                    help="skip the round that selects and prunes the budget on the device")
    ap.add_argument("--sweep-rounds", type=int, default=1000,
                    help="decode rounds per budget in the budget-sweep leg (0 skips it)")
    return ap.parse_args()


def attn_work(w, depth: np.ndarray):
    """Algorithmic bytes and flops of one ddtree_tree_attn launch."""
    W = (w.N + 31) // 32
    nbytes = (4 * w.Hkv * w.S * w.D          # prefix K and V, bf16
              + 4 * w.Hkv * w.N * w.D        # tree-node K and V
              + 4 * w.N * w.Hq * w.D         # Q in, O out
              + 4 * w.N * W)                 # ancestor mask
    flops = 4 * w.N * w.Hq * w.D * w.S + 4 * w.Hq * w.D * int((depth + 1).sum())
    return nbytes, flops


def attn_fracs(nbytes: int, flops: int, us: float) -> dict:
    """Achieved rates of one attention launch and its fractions of the HBM
    and MFMA rooflines; `binding_frac` is the larger floor over the time."""
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9) * 1e6
    t_mfma = flops / (MFMA_BF16_PEAK_TFS * 1e12) * 1e6
    return {"tree_attn_us": round(us, 3),
            "TBps": round(nbytes / (us * 1e-6) / 1e12, 3),
            "TFLOPs": round(flops / (us * 1e-6) / 1e12, 1),
            "hbm_frac": round(t_hbm / us, 4), "mfma_frac": round(t_mfma / us, 4),
            "bound": "mfma" if t_mfma > t_hbm else "hbm",
            "binding_frac": round(max(t_hbm, t_mfma) / us, 4)}


def topk_bytes(w):
    return 4 * w.L * w.V + 8 * w.L * w.K


def argmax_bytes(w):
    """ddtree_target_argmax: the bf16 [N, V] logits once, the int32 [N] ids."""
    return 2 * w.N * w.V + 4 * w.N


def compact_bytes(w, a: int):
    return 8 * a * w.layers * w.Hkv * w.D


def stage_roofline(w, stage: dict, a: int) -> dict:
    """HBM-roofline fractions of the streaming stages from their stage
    times (algorithmic bytes / time against the 8 TB/s peak), and the floor
    each would have at that peak; build, walk and budget selection are
    serial latency (no roofline)."""
    out = {}
    for name, nbytes in (("topk", topk_bytes(w)), ("target_argmax", argmax_bytes(w)),
                         ("kv_compact", compact_bytes(w, a))):
        us = stage[name]
        gbs = nbytes / (us * 1e-6) / 1e9
        out[name] = {"bound": "hbm", "us": round(us, 3), "algorithmic_bytes": int(nbytes),
                     "achieved_GBps": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "floor_us": round(nbytes / (HBM_PEAK_GBS * 1e3), 3)}
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the hot path runs on a single MI355X; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe()
        return

    import torch

    from block_diffusion_draft_ddtree_amd import binding as bd
    from block_diffusion_draft_ddtree_amd import synth
    from block_diffusion_draft_ddtree_amd.round import DraftTreeRound, RoundShape

    bd.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = synth.WORKLOADS[args.workload]
    S_cap = w.S + w.N

    # ---- inputs, resident in HBM -------------------------------------------
    lg = synth.drafter_logits(w, 0)
    logits = torch.from_numpy(lg.x).to(dev)
    g = synth.rng(w.family, 0, synth.STREAM_QKV)
    q = torch.empty((w.layers, w.N, w.Hq, w.D), dtype=torch.bfloat16, device=dev)
    kv = torch.empty((w.layers, 2, w.Hkv, S_cap, w.D), dtype=torch.bfloat16, device=dev)
    for layer in range(w.layers):
        qb, _ = synth.normal_bf16(g, (w.N, w.Hq, w.D))
        q[layer].copy_(torch.from_numpy(qb.view(np.int16)).view(torch.bfloat16))
        kb, _ = synth.normal_bf16(g, (2, w.Hkv, S_cap, w.D))
        kv[layer].copy_(torch.from_numpy(kb.view(np.int16)).view(torch.bfloat16))
    shape = RoundShape(w.L, w.V, w.K, w.B, w.Hq, w.Hkv, w.D, w.layers, S_cap)
    rnd = DraftTreeRound(shape, w.S, dev)

    # The target argmax per node follows the drafter's peak with p = 0.8 per
    # depth; it depends on the tree's depths, so build the tree once first.
    rnd.topk(logits)
    rnd.build()
    torch.cuda.synchronize()
    depth = rnd.depth.cpu().numpy()
    tgt_np = synth.target_argmax_follow_peak(depth, lg.peak, w.L, w.V,
                                             synth.rng(w.family, 0, synth.STREAM_TARGET))
    tgt = torch.from_numpy(tgt_np).to(dev)
    # Target head logits per node whose argmax is that same token (a boost
    # well above the largest of 152k normal draws), for the argmax stage.
    tl_bits, _ = synth.target_logits(synth.rng(w.family, 0, synth.STREAM_TARGET_LOGITS), w.N, w.V,
                                     peaks=tgt_np, boost=40.0)
    tlog = torch.from_numpy(tl_bits.view(np.int16)).to(dev).view(torch.bfloat16)

    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def step(attn_ev=None):
        rnd.topk(logits)
        rnd.build()
        if attn_ev is not None:
            attn_ev[0].record(stream)
        for layer in range(w.layers):
            rnd.attn(layer, q, kv, w.S)
        if attn_ev is not None:
            attn_ev[1].record(stream)
        rnd.walk(tgt)
        rnd.compact(kv, w.S)

    # The same round as three graphs, so that events recorded between the
    # replays time the attention of the timed steps.
    parts = (lambda: (rnd.topk(logits), rnd.build()),
             lambda: [rnd.attn(layer, q, kv, w.S) for layer in range(w.layers)],
             lambda: (rnd.walk(tgt), rnd.compact(kv, w.S)))
    graphs = None
    if not args.eager:
        for _ in range(2):
            step()
        torch.cuda.synchronize()
        graphs = []
        for part in parts:
            gph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gph):
                part()
            graphs.append(gph)
        torch.cuda.synchronize()

    def graph_step(attn_ev=None):
        graphs[0].replay()
        if attn_ev is not None:
            attn_ev[0].record(stream)
        graphs[1].replay()
        if attn_ev is not None:
            attn_ev[1].record(stream)
        graphs[2].replay()

    def timed_steps(run):
        """Device and wall time per step over args.steps steps, and the
        attention's mean time per layer from the events around it."""
        pairs = [(ev(), ev()) for _ in range(args.steps)]
        e0, e1 = ev(), ev()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        for i in range(args.steps):
            run(pairs[i])
        e1.record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        attn = float(np.mean([a.elapsed_time(b) * 1e3 / w.layers for a, b in pairs]))
        return e0.elapsed_time(e1) * 1e3 / args.steps, (t1 - t0) * 1e6 / args.steps, attn

    run_step = graph_step if graphs is not None else step
    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()

    # ---- timed region -------------------------------------------------------
    # The round as it runs (no events between its parts): `value`. Then the
    # same steps with events around the attention calls of every step, which
    # time the attention live; those events cost the round a few
    # microseconds of pipeline gaps, so that pass's total is reported apart.
    def plain_steps(run):
        e0, e1 = ev(), ev()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(args.steps):
            run()
        e1.record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        return e0.elapsed_time(e1) * 1e3 / args.steps, (t1 - t0) * 1e6 / args.steps

    gpu_us, wall_us = plain_steps(run_step)
    instr_us, _, attn_us = timed_steps(run_step)
    eager_us = gpu_us if graphs is None else plain_steps(step)[0]
    # The same round followed by the 4-byte accepted-count readback a host
    # decode loop would make after it (a device-to-host copy and its wait):
    # host wall time per round.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run_step()
        int(rnd.n_acc.cpu()[0])
    readback_us = (time.perf_counter() - t0) * 1e6 / args.steps

    # ---- per-stage device time (HIP events on the launch stream) ----------
    R = args.stage_reps

    def timed(fn, reps):
        # A spin kernel ahead of the reps keeps the device busy while the
        # host enqueues them, so the events see device time, not Python's.
        a, b = ev(), ev()
        fn()
        torch.cuda.synchronize()
        torch.cuda._sleep(SPIN_CYCLES)
        a.record(stream)
        for i in range(reps):
            fn(i)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / reps

    stage = {}
    stage["topk"] = timed(lambda i=0: rnd.topk(logits), R)
    stage["build"] = timed(lambda i=0: rnd.build(), R)
    stage["tree_attn"] = timed(lambda i=0: rnd.attn(i % w.layers, q, kv, w.S), max(R, 2 * w.layers))
    stage["walk"] = timed(lambda i=0: rnd.walk(tgt), R)
    stage["kv_compact"] = timed(lambda i=0: rnd.compact(kv, w.S), R)
    stage["target_argmax"] = timed(lambda i=0: rnd.target_argmax(tlog), R)
    argmax_ok = bool(torch.equal(rnd.target_choice, tgt))
    stage["target_sample"] = timed(lambda i=0: rnd.target_sample(tlog, 1.0, 2024, i), R)
    stage["budget_select"] = timed(lambda i=0: rnd.select_budget(BUDGET_T0, BUDGET_T1), R)
    budget_choice = int(rnd.budget.cpu()[0])
    torch.cuda.synchronize()
    a_acc = int(rnd.n_acc.cpu()[0])
    depth = rnd.depth.cpu().numpy()

    # The round consuming the cost-aware budget on the device: after the
    # build, ddtree_budget_select picks the budget from the build's scores
    # (time model fitted to the autobench page) and ddtree_tree_prune keeps
    # that tree; attention, walk and compaction then work on the kept nodes.
    # Three graph replays per step, as the main round.
    budget_round = None
    if graphs is not None and not args.no_budget_round:
        bparts = (lambda: (rnd.topk(logits), rnd.build(), rnd.select_budget(BUDGET_T0, BUDGET_T1),
                           rnd.prune()),
                  lambda: [rnd.attn(layer, q, kv, w.S) for layer in range(w.layers)],
                  lambda: (rnd.walk(tgt), rnd.compact(kv, w.S)))
        for part in bparts:
            part()
        torch.cuda.synchronize()
        bgraphs = []
        for part in bparts:
            gph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gph):
                part()
            bgraphs.append(gph)
        for _ in range(args.warmup):
            for gph in bgraphs:
                gph.replay()
        pairs = [(ev(), ev()) for _ in range(args.steps)]
        e0, e1 = ev(), ev()
        torch.cuda.synchronize()
        e0.record(stream)
        for a, b in pairs:
            bgraphs[0].replay()
            a.record(stream)
            bgraphs[1].replay()
            b.record(stream)
            bgraphs[2].replay()
        e1.record(stream)
        torch.cuda.synchronize()
        kept = int(rnd.budget.cpu()[0]) + 1
        budget_round = {"budget": kept - 1, "kept_nodes": kept,
                        "round_us": round(e0.elapsed_time(e1) * 1e3 / args.steps, 2),
                        "tree_attn_us": round(float(np.mean(
                            [a.elapsed_time(b) * 1e3 / w.layers for a, b in pairs])), 3),
                        "accepted": int(rnd.n_acc.cpu()[0])}
        del bgraphs
        # Rebuild the full tree for what follows.
        rnd.topk(logits)
        rnd.build()
        torch.cuda.synchronize()

    nbytes, flops = attn_work(w, depth)
    hbm_gbs = nbytes / (attn_us * 1e-6) / 1e9
    tflops = flops / (attn_us * 1e-6) / 1e12
    bound = "mfma" if flops / nbytes > MFMA_BF16_PEAK_TFS * 1e12 / (HBM_PEAK_GBS * 1e9) else "hbm"
    if bound == "mfma":
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFS,
                "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFS, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(hbm_gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(hbm_gbs / HBM_PEAK_GBS, 4)}
    roof["traffic"] = measured_traffic(w.name)
    roof["kernel"] = "ddtree_tree_attn"
    roof["algorithmic_bytes"] = nbytes
    roof["algorithmic_flops"] = flops

    value = gpu_us
    result = {
        "metric": "tree-verify attn µs & HBM TB/s at B=64, ctx 4k; full round µs/step",
        "value": round(value, 2),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(value / 1e3, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded numpy generators; no weights or datasets)",
        "config": {"workload": w.name, "L": w.L, "V": w.V, "K": w.K, "B": w.B, "Hq": w.Hq,
                   "Hkv": w.Hkv, "D": w.D, "S": w.S, "layers": w.layers,
                   "mode": "hip-graph" if graphs is not None else "eager"},
        "eager_us_per_step": round(eager_us, 2),
        "tree_attn_us": round(attn_us, 3),
        "tree_attn_TBps": round(hbm_gbs / 1e3, 3),
        "tree_attn_hbm_frac": round(hbm_gbs / HBM_PEAK_GBS, 4),
        "tree_attn_mfma_frac": round(tflops / MFMA_BF16_PEAK_TFS, 4),
        "round_wall_us": round(wall_us, 2),
        "round_with_attn_events_us": round(instr_us, 2),
        "round_with_readback_us": round(readback_us, 2),
        "stage_us": {k: round(v, 3) for k, v in stage.items()},
        "topk_TBps": round(topk_bytes(w) / (stage["topk"] * 1e-6) / 1e12, 3),
        "target_argmax_TBps": round(argmax_bytes(w) / (stage["target_argmax"] * 1e-6) / 1e12, 3),
        "target_argmax_matches": argmax_ok,
        "target_sample_Gtok_s": round(w.N * w.V / (stage["target_sample"] * 1e-6) / 1e9, 1),
        "budget_choice": budget_choice,
        "accepted": a_acc,
        "depth_hist": np.bincount(depth).tolist(),
        "roofline": roof,
        "stage_roofline": stage_roofline(w, stage, a_acc),
    }
    if budget_round is not None:
        result["budget_round"] = budget_round

    if args.batch_requests > 0:
        result["batched"] = batched_leg(w, args.batch_requests, args.steps, args.warmup,
                                        use_graphs=not args.eager)
    # Free the headline round's buffers before the other shapes allocate theirs.
    del rnd, q, kv, logits, graphs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if not args.no_configs:
        result["configs"] = config_legs(args.steps, args.warmup)
    if args.sweep_rounds > 0:
        result["budget_sweep"] = sweep_leg(args.sweep_rounds)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, lg, depth, tgt_np)
    print(json.dumps(result), flush=True)


def round_leg(w, steps: int, warmup: int, seed: int):
    """One workload's full round (top-K, build, every layer's attention, walk,
    compaction) replayed as three HIP graphs per step, with events around the
    attention: round time, attention time per layer and its roofline
    fractions. Q/K/V are drawn on the device (seeded torch generator); the
    walk follows the drafter's peak with p = 0.8 per depth."""
    import torch

    from block_diffusion_draft_ddtree_amd import synth
    from block_diffusion_draft_ddtree_amd.round import DraftTreeRound, RoundShape

    dev = torch.device("cuda:0")
    S_cap = w.S + w.N
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    lg = synth.drafter_logits(w, 0)
    logits = torch.from_numpy(lg.x).to(dev)
    q = torch.randn((w.layers, w.N, w.Hq, w.D), generator=gen, device=dev).to(torch.bfloat16)
    kv = torch.empty((w.layers, 2, w.Hkv, S_cap, w.D), dtype=torch.bfloat16, device=dev)
    for layer in range(w.layers):
        kv[layer].copy_(torch.randn(kv[layer].shape, generator=gen, device=dev))
    shape = RoundShape(w.L, w.V, w.K, w.B, w.Hq, w.Hkv, w.D, w.layers, S_cap)
    rnd = DraftTreeRound(shape, w.S, dev)
    rnd.topk(logits)
    rnd.build()
    torch.cuda.synchronize()
    depth = rnd.depth.cpu().numpy()
    tgt = torch.from_numpy(synth.target_argmax_follow_peak(
        depth, lg.peak, w.L, w.V, synth.rng(w.family, 0, synth.STREAM_TARGET))).to(dev)
    parts = (lambda: (rnd.topk(logits), rnd.build()),
             lambda: [rnd.attn(layer, q, kv, w.S) for layer in range(w.layers)],
             lambda: (rnd.walk(tgt), rnd.compact(kv, w.S)))
    for _ in range(2):
        for part in parts:
            part()
    torch.cuda.synchronize()
    graphs = []
    for part in parts:
        gph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gph):
            part()
        graphs.append(gph)
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    for _ in range(warmup):
        for gph in graphs:
            gph.replay()
    pairs = [(ev(), ev()) for _ in range(steps)]
    e0, e1 = ev(), ev()
    torch.cuda.synchronize()
    e0.record(stream)
    for a, b in pairs:
        graphs[0].replay()
        a.record(stream)
        graphs[1].replay()
        b.record(stream)
        graphs[2].replay()
    e1.record(stream)
    torch.cuda.synchronize()
    round_us = e0.elapsed_time(e1) * 1e3 / steps
    attn_us = float(np.mean([a.elapsed_time(b) * 1e3 / w.layers for a, b in pairs]))
    nbytes, flops = attn_work(w, depth)
    out = {"S": w.S, "N": w.N, "Hq": w.Hq, "Hkv": w.Hkv, "layers": w.layers,
           "round_us": round(round_us, 2)}
    out.update(attn_fracs(nbytes, flops, attn_us))
    out["algorithmic_bytes"], out["algorithmic_flops"] = nbytes, flops
    del rnd, q, kv, graphs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def config_legs(steps: int, warmup: int) -> dict:
    """The other workload shapes, each as a full round: the Qwen3-8B verifier
    at its prefix 2048 and at 4096 (the HBM-bound case of B = 64 at a 4k
    context), the 30B verifier at B = 256, and the long-context shape (one
    layer timed; its attention reported times 48 layers)."""
    from dataclasses import replace

    from block_diffusion_draft_ddtree_amd import synth

    legs = {}
    legs["qwen3_8b_s2048"] = round_leg(synth.QWEN3_8B, steps, warmup, 31)
    legs["qwen3_8b_s4096"] = round_leg(replace(synth.QWEN3_8B, name="qwen3_8b_s4096", S=4096),
                                       steps, warmup, 32)
    legs["coder30b_b256"] = round_leg(synth.CODER30B_B256, steps, warmup, 33)
    lc = round_leg(synth.LONGCTX, steps, warmup, 34)
    lc["reported_layers"] = synth.LONGCTX_REPORTED_LAYERS
    lc["attn_us_x_layers"] = round(lc["tree_attn_us"] * synth.LONGCTX_REPORTED_LAYERS, 1)
    legs["longctx"] = lc
    return legs


def sweep_leg(rounds: int) -> dict:
    """The budget sweep: for B in 16 ... 512 (K = B, flat logits with weak
    peaks, 32q/8kv heads, 36 layers, prefix from 8192), `rounds` decode
    rounds each: top-K, build, attention of all 36 layers at the current
    prefix length, walk, and compaction of a drawn accepted path (a ~ U[1, L]
    per round); the prefix then grows by 1 + a. One attention workspace per
    budget, sized once at the last round's prefix length. Launched eagerly
    (S changes every round) in chunks held behind a spin kernel, so events
    see device time, not Python's launch rate."""
    import torch

    from block_diffusion_draft_ddtree_amd import binding as bd
    from block_diffusion_draft_ddtree_amd import synth
    from block_diffusion_draft_ddtree_amd.round import DraftTreeRound, RoundShape

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    chunk = 25
    out = {"rounds": rounds, "layers": 36, "Hq": 32, "Hkv": 8, "S0": 8192, "per_budget": {}}
    for B in synth.SWEEP_BUDGETS:
        w = synth.sweep(B)
        acc_np, a_np = synth.sweep_accepts(B, w.L, rounds)
        S_r = synth.sweep_prefix_lengths(w.S, a_np)
        S_cap = int(S_r[-1]) + w.N
        gen = torch.Generator(device=dev)
        gen.manual_seed(5000 + B)
        logits = [torch.from_numpy(synth.drafter_logits(w, i).x).to(dev) for i in range(2)]
        q = torch.randn((w.layers, w.N, w.Hq, w.D), generator=gen, device=dev).to(torch.bfloat16)
        kv = torch.empty((w.layers, 2, w.Hkv, S_cap, w.D), dtype=torch.bfloat16, device=dev)
        for layer in range(w.layers):
            kv[layer].copy_(torch.randn(kv[layer].shape, generator=gen, device=dev))
        acc = torch.from_numpy(acc_np).to(dev)
        n_acc = torch.from_numpy(a_np).to(dev)
        tgt = torch.randint(0, w.V, (w.N,), generator=gen, device=dev, dtype=torch.int32)
        shape = RoundShape(w.L, w.V, w.K, w.B, w.Hq, w.Hkv, w.D, w.layers, S_cap)
        rnd = DraftTreeRound(shape, int(S_r[-1]), dev)
        ws_bytes = int(rnd.ws_attn.numel())

        def one_round(r, attn_ev=None):
            S = int(S_r[r])
            rnd.topk(logits[r % 2])
            rnd.build()
            if attn_ev is not None:
                attn_ev[0].record(stream)
            for layer in range(w.layers):
                rnd.attn(layer, q, kv, S)
            if attn_ev is not None:
                attn_ev[1].record(stream)
            rnd.walk(tgt)
            bd.ddtree_kv_compact(kv, S, w.N, w.L, acc[r], n_acc[r:r + 1])

        one_round(0)
        torch.cuda.synchronize()
        round_ms, attn_ms = 0.0, []
        for c0 in range(0, rounds, chunk):
            c1 = min(rounds, c0 + chunk)
            pairs = [(ev(), ev()) for _ in range(c1 - c0)]
            e0, e1 = ev(), ev()
            torch.cuda._sleep(SPIN_CYCLES * 4)
            e0.record(stream)
            for r in range(c0, c1):
                one_round(r, pairs[r - c0])
            e1.record(stream)
            torch.cuda.synchronize()
            round_ms += e0.elapsed_time(e1)
            attn_ms += [a.elapsed_time(b) / w.layers for a, b in pairs]
        depth = rnd.depth.cpu().numpy()
        S_mean = int(np.mean(S_r))
        from dataclasses import replace
        nbytes, flops = attn_work(replace(w, S=S_mean), depth)
        rec = {"S_first": int(S_r[0]), "S_last": int(S_r[-1]), "accepted_mean": float(a_np.mean()),
               "round_us": round(round_ms * 1e3 / rounds, 2), "attn_workspace_bytes": ws_bytes,
               "depth_hist": np.bincount(depth).tolist()}
        rec.update(attn_fracs(nbytes, flops, float(np.mean(attn_ms)) * 1e3))
        rec["fracs_at_S"] = S_mean
        out["per_budget"][f"B{B}"] = rec
        del rnd, q, kv, logits, acc, n_acc
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out


# Prefix lengths of the batched leg: R requests of the same model shape with
# contexts from 512 to 4096 tokens, taken in this order.
BATCH_S = [4096, 1024, 3072, 2048, 4096, 512, 3584, 2560]


def batched_leg(w, R: int, steps: int, warmup: int, use_graphs: bool = True):
    """R requests of workload w in one batched round (own drafter rows,
    tree, prefix length and KV cache each): topk over the stacked rows,
    build, every layer's attention, walk, compaction. Inputs are drawn on
    the device from a seeded generator. Timed like the main round: three
    graph replays per step with events around the attention, or eager
    launches."""
    import torch

    from block_diffusion_draft_ddtree_amd.round import BatchedDraftTreeRound, RoundShape

    dev = torch.device("cuda:0")
    S = [BATCH_S[r % len(BATCH_S)] for r in range(R)]
    S_cap = max(S) + w.N
    gen = torch.Generator(device=dev)
    gen.manual_seed(20240 + R)
    logits = 2.0 * torch.randn((R * w.L, w.V), generator=gen, device=dev)
    q = torch.randn((w.layers, R, w.N, w.Hq, w.D), generator=gen, device=dev).to(torch.bfloat16)
    kv = torch.empty((R, w.layers, 2, w.Hkv, S_cap, w.D), dtype=torch.bfloat16, device=dev)
    for r in range(R):
        kv[r].copy_(torch.randn(kv[r].shape, generator=gen, device=dev))
    target = torch.randint(0, w.V, (R, w.N), generator=gen, device=dev, dtype=torch.int32)
    shape = RoundShape(w.L, w.V, w.K, w.B, w.Hq, w.Hkv, w.D, w.layers, S_cap)
    rnd = BatchedDraftTreeRound(shape, S, dev)
    stream = torch.cuda.current_stream()

    def step(attn_ev=None):
        rnd.topk(logits)
        rnd.build()
        if attn_ev is not None:
            attn_ev[0].record(stream)
        for layer in range(w.layers):
            rnd.attn(layer, q[layer], kv)
        if attn_ev is not None:
            attn_ev[1].record(stream)
        rnd.walk(target)
        rnd.compact(kv)

    run_step = step
    if use_graphs:
        for _ in range(2):
            step()
        torch.cuda.synchronize()
        graphs = []
        for part in (lambda: (rnd.topk(logits), rnd.build()),
                     lambda: [rnd.attn(layer, q[layer], kv) for layer in range(w.layers)],
                     lambda: (rnd.walk(target), rnd.compact(kv))):
            gph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gph):
                part()
            graphs.append(gph)
        torch.cuda.synchronize()

        def run_step(attn_ev=None):
            graphs[0].replay()
            if attn_ev is not None:
                attn_ev[0].record(stream)
            graphs[1].replay()
            if attn_ev is not None:
                attn_ev[1].record(stream)
            graphs[2].replay()

    for _ in range(warmup):
        run_step()
    torch.cuda.synchronize()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    pairs = [(ev(), ev()) for _ in range(steps)]
    e0, e1 = ev(), ev()
    e0.record(stream)
    for i in range(steps):
        run_step(pairs[i])
    e1.record(stream)
    torch.cuda.synchronize()
    round_us = e0.elapsed_time(e1) * 1e3 / steps
    attn_us = float(np.mean([a.elapsed_time(b) * 1e3 / w.layers for a, b in pairs]))
    # Algorithmic bytes of one batched attention launch: every request's
    # prefix and tree K/V, Q in, O out, the mask rows.
    W = (w.N + 31) // 32
    nbytes = sum(4 * w.Hkv * (s + w.N) * w.D + 4 * w.N * w.Hq * w.D + 4 * w.N * W for s in S)
    depth = rnd.tree[1].cpu().numpy()
    flops = sum(4 * w.N * w.Hq * w.D * s for s in S) + 4 * w.Hq * w.D * int((depth + 1).sum())
    return {"R": R, "S": S, "mode": "hip-graph" if use_graphs else "eager",
            "round_us": round(round_us, 2),
            "us_per_request": round(round_us / R, 2),
            "tree_attn_us": round(attn_us, 3),
            "tree_attn_TBps": round(nbytes / (attn_us * 1e-6) / 1e12, 3),
            "tree_attn_TFLOPs": round(flops / (attn_us * 1e-6) / 1e12, 1),
            "data": "synthetic (seeded torch device generator)"}


def host_info() -> dict:
    """The host the oracle runs on: CPUs visible to the process, its model,
    and the numpy/BLAS build and threads."""
    import platform

    from threadpoolctl import threadpool_info

    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
    return {"cpu_model": model or platform.processor(),
            "os_cpu_count": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0)),
            "numpy": np.__version__,
            "blas": ", ".join(f"{p.get('internal_api')} {p.get('version')}" for p in blas),
            "blas_threads": max([p.get("num_threads", 1) for p in blas] + [1]),
            "python": platform.python_version()}


def oracle_round(w, lg, tgt_np, layers: int) -> dict:
    """Seconds the CPU oracle spends on each stage of one round of workload
    w, with `layers` of its attention layers (each with its own seeded
    inputs, drawn outside the timed calls)."""
    from block_diffusion_draft_ddtree_amd import synth
    from oracle import attention as oa
    from oracle import commit as oc
    from oracle import softmax_topk as st
    from oracle import tree as ot

    t = {"topk": 0.0, "build": 0.0, "attn": 0.0, "walk": 0.0, "compact": 0.0}
    t0 = time.perf_counter()
    lp, tok = st.topk(lg.x, w.K)
    t["topk"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    tree = ot.build_tree(lp.astype(np.float32), tok, w.B, 0)
    t["build"] = time.perf_counter() - t0
    kv_layers = []
    for layer in range(layers):
        qkv = synth.attention_inputs(w, layers=1, round_idx=layer)
        t0 = time.perf_counter()
        oa.tree_attention(qkv.q, qkv.kv[0, 0], qkv.kv[0, 1], w.S, tree.anc)
        t["attn"] += time.perf_counter() - t0
        kv_layers.append(qkv.kv_bits[0])
        del qkv
    t0 = time.perf_counter()
    acc, a, _ = oc.accept_walk(tree.parent, tree.token, tgt_np, w.L)
    t["walk"] = time.perf_counter() - t0
    for kvb in kv_layers:
        t0 = time.perf_counter()
        oc.kv_compact(kvb, w.S, acc, a)
        t["compact"] += time.perf_counter() - t0
    return t


def oracle_build_forms(w, lg) -> dict:
    """Seconds the oracle's two exact top-B constructions take on the round's
    log-prob table: the sort-and-expand fixed point (the build the round
    uses) and Proposition 3 as a textbook binary-heap best-first search."""
    from oracle import softmax_topk as st
    from oracle import tree as ot

    lp, _ = st.topk(lg.x, w.K)
    lp32 = lp.astype(np.float32)
    out = {}
    for name, fn in (("sort_fixed_point", ot.top_b_sort_expand),
                     ("best_first_heap", ot.top_b_best_first)):
        t0 = time.perf_counter()
        fn(lp32, w.B)
        out[name] = round(time.perf_counter() - t0, 5)
    return out


def cpu_baseline(w, lg, depth, tgt_np):
    """The CPU oracle on one whole round of the headline workload (all 48
    layers, not scaled) with numpy's BLAS at its default thread count
    (`cores` = the BLAS threads it used); and the same oracle pinned to one
    thread on a bounded sample (top-K, build, walk, 4 attention layers and
    their compaction), its attention and compaction scaled to all layers."""
    from threadpoolctl import threadpool_limits

    info = host_info()
    t = oracle_round(w, lg, tgt_np, w.layers)
    us = 1e6 * sum(t.values())
    sample_layers = 4
    with threadpool_limits(limits=1):
        t1 = oracle_round(w, lg, tgt_np, sample_layers)
    scale = w.layers / sample_layers
    us1 = 1e6 * (t1["topk"] + t1["build"] + t1["walk"] + scale * (t1["attn"] + t1["compact"]))
    builds = oracle_build_forms(w, lg)
    return {"value": round(us, 1), "unit": "us/step", "cores": info["blas_threads"],
            "kind": "oracle",
            "sample": (f"one whole round of {w.name}: top-K over all {w.L} rows, tree build, "
                       f"attention of all {w.layers} layers, walk, compaction of all "
                       f"{w.layers} layers; not scaled; numpy with {info['blas_threads']} "
                       f"BLAS threads"),
            "stage_s": {k: round(v, 4) for k, v in t.items()},
            "single_thread": {"value": round(us1, 1), "unit": "us/step", "cores": 1,
                              "sample": (f"top-K, build and walk of one round plus "
                                         f"{sample_layers} of its {w.layers} attention layers "
                                         f"and their compaction, those two scaled by "
                                         f"{scale:g}"),
                              "stage_s": {k: round(v, 4) for k, v in t1.items()}},
            "build_forms_s": builds,
            "host": info}


if __name__ == "__main__":
    main()
