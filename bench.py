#!/usr/bin/env python3
"""Benchmark of the decode-step weight stream on one MI355X.

Default workload: one decode step of the 28-layer, hidden-1536 Llama-class
decoder (BF16 weights, 3.09 GB) with final RMSNorm, 151936 x 1536 LM head and
argmax, batch 1 -- one persistent kernel launch per step.  Inputs are seeded
synthetic tensors already resident in HBM when timing starts.

Prints ONE JSON line (rank 0) with the measured throughput (algorithmic bytes /
step time), the roofline of the dominant kernel and the CPU oracle timed on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

METRIC = ("decode-step weight-stream µs and achieved HBM GB/s (% of peak), "
          "1.5B shapes, batch 1")
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode_step_1536x28",
                    choices=["decode_step_1536x28", "decoder_block_1536", "ln_gelu_chain_768x72",
                             "rmsnorm_gemv_256", "rmsnorm_rows_960x1536_f16", "lmhead_151936",
                             "decode_attention_12q2kv128", "decode_step_attn_1536x28",
                             "gemv_int4_lmhead_151936", "ln_gelu_train_768x72"])
    ap.add_argument("--batch", type=int, default=None)
    ap.add_argument("--layers", type=int, default=None,
                    help="decode-step workload: number of decoder blocks (default 28)")
    ap.add_argument("--vocab", type=int, default=None,
                    help="decode-step workload: LM-head rows (default 151936)")
    ap.add_argument("--mode", type=int, default=0, help="0 persistent kernel, 1 one launch per phase")
    ap.add_argument("--path", type=int, default=0,
                    help="0 auto (vector path for batch <= 4, matrix cores above), 1 vector, 2 matrix cores, "
                         "3 stage-by-stage tiled products (the only path above batch 16)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after warm-up, run one plain device copy of this many MiB (the known-size "
                         "reference for HBM byte counters)")
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "OUT_TXT"),
                    help="turn two rocprofv3 --pmc counter files (FETCH_SIZE, WRITE_SIZE) of a run with "
                         "--calib-copy-mib into the traffic summary that later runs report; no GPU used")
    ap.add_argument("--prefetch", default="none", choices=["none", "tune"],
                    help="with --mode 1: tune an Infinity-Cache prefetch plan (touch passes on a second "
                         "stream, wgn_plan_tune) before timing, and time the plan it keeps")
    ap.add_argument("--tune-reps", type=int, default=15, help="rounds of the prefetch tuner")
    ap.add_argument("--attn", default="auto", choices=["auto", "fused", "launches"],
                    help="decode_step_attn: attention as phases of the one chain launch, launches of its own, "
                         "or the faster of the two by batch and cache size")
    ap.add_argument("--ring", type=int, default=0, help="decode_step_attn: streaming ring (0 auto, 1..3)")
    ap.add_argument("--slots", type=int, default=None,
                    help="decode-attention workload: cache slots (all valid: the new token takes the last; default 32768); "
                         "decode step with attention: cache slots (default 1024, the new token at slot 960)")
    ap.add_argument("--cold", action="store_true",
                    help="read a 512 MB scrub buffer between timed steps (evicts the Infinity Cache)")
    ap.add_argument("--bwd-prefetch", default="off", choices=["on", "off"],
                    help="training-step workload: the prefetch setting of the timed steps (both are "
                         "compared in an interleaved A/B pass after the timing)")
    ap.add_argument("--ab-rounds", type=int, default=20,
                    help="training-step workload: rounds of the prefetch on/off comparison")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the measured streaming-read ceiling (a 2 GiB plain read, a few configurations)")
    return ap.parse_args()


def main():
    args = parse()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc, workload=args.workload, batch=args.batch or 1,
                      copy_mib=args.calib_copy_mib, path=args.path)
        return
    if args.gpus != 1:
        print("bench.py: this build measures one GPU only (the weight stream runs on a single "
              "device); --gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    import weight_gemv_norm_amd as W
    from weight_gemv_norm_amd import steps
    from synth import gen

    dev = "cuda"
    torch.cuda.set_device(0)
    wl = args.workload
    B = args.batch if args.batch is not None else (4 if wl in ("ln_gelu_chain_768x72", "ln_gelu_train_768x72") else 1)
    print("[bench] workload %s batch %d mode %d" % (wl, B, args.mode), file=sys.stderr, flush=True)

    # ----------------------------------------------------------- build work
    chain = None
    launch = None
    nbytes = 0
    cfg = {"workload": wl, "batch": B}
    kernel_name = "chain_kernel"
    if wl in ("decode_step_1536x28", "decoder_block_1536") and (B > 16 or args.path == 3):
        # batch 17-128 (or --path 3): stage by stage on the matrix cores
        # (tiled products, norm passes), one HIP graph per step
        inp = gen.make_stage_tensors(wl, device=dev, batch=B, n_layers=args.layers, vocab=args.vocab)
        stages, bufs = steps.decoder_stages(inp, dev)
        bstep = steps.BatchedStep(stages, B, dev)
        nb = steps.decode_step_bytes(inp)
        nbytes = nb["total"]
        flops = 2 * nb["weights"] // 2 * B
        cfg.update({"hidden": gen.H, "intermediate": gen.I, "layers": len(inp["layers"]),
                    "vocab": gen.V if "W_lm" in inp else None, "weight_bytes": nb["weights"],
                    "algorithmic_bytes": nbytes, "flops": flops, "launches_per_step": bstep.n_launches,
                    "launch": "stage by stage (one HIP graph)", "path": "matrix (tiled products)"})
        kernel_name = "gemm_kernel"  # with its norm passes and counter clear: one step's launches
        bgraph = bstep.capture()
        launch = bgraph.replay
        cfg["graph"] = True
    elif wl in ("decode_step_1536x28", "decoder_block_1536"):
        inp = gen.make_stage_tensors(wl, device=dev, batch=B, n_layers=args.layers, vocab=args.vocab)
        stages, bufs = steps.decoder_stages(inp, dev)
        chain = W.Chain(stages, B, mode=args.mode, path=args.path)
        nb = steps.decode_step_bytes(inp)
        nbytes = nb["total"]
        cfg.update({"hidden": gen.H, "intermediate": gen.I, "layers": len(inp["layers"]),
                    "vocab": gen.V if "W_lm" in inp else None, "weight_bytes": nb["weights"],
                    "algorithmic_bytes": nbytes, "phases": chain.num_phases,
                    "launch": "persistent" if args.mode == 0 else "per-phase",
                    "path": "matrix" if (args.path == 2 or (args.path == 0 and B > 4)) else "vector"})
        launch = chain.run
    elif wl == "decode_step_attn_1536x28":
        # the decode step with computed attention: 1,024-slot caches, the new
        # token at slot 960 (after a 960-token prompt) unless --slots says otherwise
        S = args.slots or 1024
        pos = min(960, S - 1)
        inp = gen.make_stage_tensors("decode_step_1536x28", device=dev, batch=B, n_layers=args.layers,
                                     vocab=args.vocab)
        n_layers = len(inp["layers"])
        caches = gen.make_kv_caches(B, S, [pos] * B, n_layers=n_layers, nan_tail=False, device=dev)
        dstep = steps.DecodeStepWithAttention(inp, caches, dev, mode=args.mode,
                                              fused={"auto": None, "fused": True, "launches": False}[args.attn],
                                              ring=args.ring)
        nb = steps.decode_step_bytes(inp)
        kv = n_layers * (2 * B * gen.NKV * (pos + 1) * gen.HEAD_DIM * 2 + 2 * 2 * B * gen.NKV * gen.HEAD_DIM * 2)
        nbytes = nb["total"] + kv
        cfg.update({"hidden": gen.H, "intermediate": gen.I, "layers": n_layers, "vocab": gen.V if "W_lm" in inp
                    else None, "weight_bytes": nb["weights"], "kv_bytes": kv, "slots": S, "position": pos,
                    "algorithmic_bytes": nbytes, "launches_per_step": dstep.n_launches,
                    "launch": ("one persistent launch, attention as phases" if dstep.fused
                               else "persistent chains between attention launches")})
        kernel_name = "chain_kernel" if dstep.fused else "chain_kernel+decode_attention_kernel"
        # one HIP graph per step: 57 launches from Python would leave the GPU idle
        dgraph = dstep.capture()
        launch = dgraph.replay
        cfg["graph"] = True
    elif wl == "gemv_int4_lmhead_151936":
        # the LM head in 4-bit weights (groups of 128): the largest matrix of the step
        t4 = gen.make_int4_weights(gen.V, gen.H, seed=1, device=dev)
        x4 = gen.normal((B, gen.H), 1.0, 5, device=dev)
        y4 = torch.empty((B, gen.V), dtype=torch.bfloat16, device=dev)
        nbytes = gen.V * gen.H // 2 + 2 * gen.V * (gen.H // 128) * 2 + B * gen.H * 2 + B * gen.V * 2
        cfg.update({"N": gen.V, "K": gen.H, "group": 128, "algorithmic_bytes": nbytes})
        kernel_name = "gemv_int4_kernel"
        launch = lambda: W.gemv_int4(x4, t4["W4"], t4["scales"], t4["zeros"], y4)  # noqa: E731
    elif wl == "ln_gelu_chain_768x72":
        inp = gen.make_stage_tensors(wl, device=dev, batch=B)
        stages, bufs = steps.ln_gelu_chain_stages(inp, dev)
        chain = W.Chain(stages, B, mode=args.mode, path=args.path)
        nbytes = sum(L["W"].numel() * 2 + (L["bias"].numel() + L["gamma"].numel() + L["beta"].numel()) * 2
                     for L in inp["layers"]) + (len(inp["layers"]) + 1) * B * 768 * 2
        cfg.update({"width": 768, "blocks": 72, "algorithmic_bytes": nbytes, "phases": chain.num_phases,
                    "launch": "persistent" if args.mode == 0 else "per-phase"})
        launch = chain.run
    elif wl == "ln_gelu_train_768x72":
        # one small-batch training step of the LayerNorm chain: forward (keeping
        # pre-activations), gradient of the mean-square loss, backward pass
        inp = gen.make_stage_tensors("ln_gelu_chain_768x72", device=dev, batch=B, n_layers=args.layers,
                                     seeded_ln_params=True)
        tstep = steps.TrainStep(inp, dev, prefetch=args.bwd_prefetch == "on", keep=False)  # noqa: E501
        tb = steps.train_step_bytes(inp)
        nbytes = tb["total"]
        bwd_bytes = tb["weights_bwd"] + tb["weight_grads"] + tb["small"] // 2 + tb["activations"] // 2
        n_blocks = len(inp["layers"])
        cfg.update({"width": 768, "blocks": n_blocks, "algorithmic_bytes": nbytes, "bytes": tb,
                    "backward_bytes": bwd_bytes, "loss": "mean of the squared chain output",
                    "launch": "forward chain + backward prep + backward, one HIP graph",
                    "launches_per_step": 3, "prefetch": args.bwd_prefetch,
                    "backward_grid": tstep.bwd.grid, "forward_phases": tstep.fwd.num_phases})
        kernel_name = "bwd_kernel"
        tstep.prefetch = True
        g_on = tstep.capture()
        tstep.prefetch = False
        g_off = tstep.capture()
        tstep.prefetch = args.bwd_prefetch == "on"
        launch = g_on.replay if tstep.prefetch else g_off.replay
        cfg["graph"] = True
    elif wl == "rmsnorm_gemv_256":
        t = gen.make_stage_tensors(wl, device=dev, batch=B)
        y = torch.empty((B, 256), dtype=torch.bfloat16, device=dev)
        st = W.make_stage(t["W"], t["x"], y, norm=1, eps=t["eps"], gamma=t["g"])
        nbytes = 256 * 256 * 2 + 256 * 2 + 2 * B * 256 * 2
        cfg.update({"N": 256, "K": 256, "algorithmic_bytes": nbytes})
        launch = lambda: W.gemv_norm(st, B)  # noqa: E731
    elif wl == "lmhead_151936":
        h = gen.normal((B, gen.H), 1.0, 1, device=dev)
        g = gen.normal((gen.H,), 0.1, 2, mean=1.0, device=dev)
        Wl = gen.normal((gen.V, gen.H), 0.02, 3, device=dev)
        idx = torch.empty((B,), dtype=torch.int32, device=dev)
        ws = W.workspace(W.lmhead_argmax_workspace_bytes(B))
        nbytes = gen.V * gen.H * 2 + gen.H * 2 + B * gen.H * 2 + B * 4
        cfg.update({"V": gen.V, "K": gen.H, "algorithmic_bytes": nbytes})
        launch = lambda: W.lmhead_argmax(h, g, 1e-6, Wl, idx, ws=ws)  # noqa: E731
    elif wl == "rmsnorm_rows_960x1536_f16":
        t = gen.make_stage_tensors(wl, device=dev)
        y = torch.empty_like(t["x"])
        nbytes = 2 * 960 * 1536 * 2 + 1536 * 2
        cfg.update({"rows": 960, "K": 1536, "dtype": "f16", "algorithmic_bytes": nbytes})
        launch = lambda: W.rmsnorm_rows(t["x"], t["g"], t["eps"], y)  # noqa: E731
        kernel_name = "rmsnorm_rows_kernel"

    elif wl == "decode_attention_12q2kv128":
        # one decode step's attention: every layer has its own cache (28 x 33.5 MB
        # at 32,768 slots and batch 1, well beyond the 256 MB Infinity Cache)
        n_layers = args.layers or gen.N_LAYERS
        S = args.slots or 32768
        att = [gen.make_attention_tensors(B, S, [S - 1] * B, layer=l, nan_tail=False, device=dev)
               for l in range(n_layers)]
        att_out = [torch.empty_like(t["q"]) for t in att]
        ws = W.workspace(W.decode_attention_workspace_bytes(B, gen.NQ, gen.NKV, S))
        per_layer = (2 * B * gen.NKV * S * gen.HEAD_DIM * 2          # keys and values of the valid slots
                     + 2 * B * gen.NQ * gen.HEAD_DIM * 2             # q in, output out
                     + 2 * 2 * B * gen.NKV * gen.HEAD_DIM * 2)       # new key/value in, appended out
        nbytes = per_layer * n_layers
        cfg.update({"q_heads": gen.NQ, "kv_heads": gen.NKV, "head_dim": gen.HEAD_DIM, "slots": S,
                    "valid_slots": S, "layers": n_layers, "launches_per_step": n_layers,
                    "algorithmic_bytes": nbytes, "bytes_per_launch": per_layer})
        kernel_name = "decode_attention_kernel"

        def launch():
            for t, o in zip(att, att_out):
                W.decode_attention(t["q"], t["k_new"], t["v_new"], t["k_cache"], t["v_cache"], t["pos"], o, ws=ws)

    if chain is not None:
        cfg["ring"] = chain.ring
    # cold runs: a 512 MB plain read between timed steps (read-only, so it
    # leaves no dirty lines whose write-back would slow the step) evicts the
    # 256 MB Infinity Cache and the L2s
    scrub = torch.ones(256 << 20, dtype=torch.int16, device=dev) if args.cold else None
    scrub_sink = torch.zeros(1, dtype=torch.int32, device=dev) if args.cold else None

    if args.prefetch == "tune":
        if chain is None or args.mode != 1:
            print("bench.py: --prefetch tune needs a chain workload and --mode 1", file=sys.stderr)
            sys.exit(2)
        side = torch.cuda.Stream()
        plan = chain.tune_plan(side, reps=args.tune_reps)
        cfg["prefetch_plan"] = {"kept": bool(plan.prefetch), "distance": plan.distance, "blocks": plan.blocks,
                                "frac_pct": plan.frac_pct, "plain_us": round(plan.plain_us, 3),
                                "best_candidate_us": round(plan.best_us, 3),
                                "speedup_ci95_lo": round(plan.speedup_lo, 4), "candidates": plan.candidates,
                                "tune_reps": args.tune_reps}
        print("[bench] prefetch plan: %s" % cfg["prefetch_plan"], file=sys.stderr, flush=True)
        launch = (lambda: chain.run(plan=plan, side=side)) if plan.prefetch else chain.run  # noqa: E731

    # -------------------------------------------------------------- warm up
    for _ in range(args.warmup):
        launch()
    torch.cuda.synchronize()
    if chain is not None:
        chain.check()
    print("[bench] warmup done", file=sys.stderr, flush=True)
    if args.calib_copy_mib:
        ca = torch.ones(args.calib_copy_mib << 20, dtype=torch.uint8, device=dev)
        cb = torch.empty_like(ca)
        torch.cuda.synchronize()
        cb.copy_(ca)
        torch.cuda.synchronize()
        del ca, cb

    # --------------------------------------------------------------- timing
    stream = torch.cuda.current_stream()
    K = args.steps
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    t_all0 = torch.cuda.Event(enable_timing=True)
    t_all1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_all0.record(stream)
    for i in range(K):
        if scrub is not None:
            W.stream_read(scrub, 2048, 256, 1, scrub_sink)
        starts[i].record(stream)
        launch()
        ends[i].record(stream)
    t_all1.record(stream)
    torch.cuda.synchronize()
    wall1 = time.perf_counter()
    if chain is not None:
        chain.check()
    if wl == "ln_gelu_train_768x72":
        tstep.check()
    per = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)]) * 1e3  # us
    total_ms = t_all0.elapsed_time(t_all1)
    # one timing basis for value, ms_per_step and the roofline: the events
    # around each step on the launch stream (the whole-region time, which also
    # holds the gaps between launches and, with --cold, the scrubs, is reported
    # beside them as a cross-check)
    us_step = float(np.mean(per))
    us_med = float(np.median(per))
    ci = ci95_mean(per)
    ms_per_step = us_step / 1e3
    gbs = nbytes / (us_step * 1e-6) / 1e9
    print("[bench] timed %d steps: mean %.2f us (95%% CI %.2f-%.2f), median %.2f us, min %.2f us, wall %.3f s"
          % (K, us_step, ci[0], ci[1], us_med, float(per.min()), wall1 - wall0), file=sys.stderr, flush=True)
    ceiling = None
    if not args.no_ceiling:
        ceiling = read_ceiling(W, torch, dev)
        print("[bench] measured streaming-read ceiling %.1f GB/s (%s)" % (ceiling["gbs"], ceiling["config"]),
              file=sys.stderr, flush=True)

    # several launches per step run back to back on one stream: the average
    # launch is the step time over the launches (the batched path's roofline
    # unit is the whole step: its traffic is recorded per step)
    launches = 1 if kernel_name == "gemm_kernel" else cfg.get("launches_per_step", 1)
    l_mean, l_med = us_step / launches, us_med / launches
    l_bytes = nbytes // launches
    if wl == "ln_gelu_train_768x72":
        # the dominant kernel is the backward launch: timed on its own stream
        # (prep + backward, eager) with events around each call
        train_ab = train_prefetch_ab(tstep, g_on, g_off, torch, args.ab_rounds, scrub, scrub_sink, W)
        cfg["prefetch_ab"] = train_ab
        l_mean, l_med = train_ab["backward_us_mean"], train_ab["backward_us_median"]
        l_bytes = bwd_bytes
    l_gbs = l_bytes / (l_mean * 1e-6) / 1e9
    roofline = {"bound": "hbm", "kernel": kernel_name, "achieved": round(l_gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(l_gbs / HBM_PEAK_GBS, 4),
                "traffic": recorded_traffic(wl, B, kernel_name), "launch_us_mean": round(l_mean, 3),
                "launch_us_median": round(l_med, 3), "bytes_per_launch": l_bytes}
    if wl == "ln_gelu_train_768x72":
        roofline["timed"] = "bwd_prep_kernel + bwd_kernel, back to back on one stream"
        roofline["bytes_per_launch_basis"] = ("backward: every weight read once, every weight gradient written "
                                              "once, block inputs and pre-activations read, small parameters")
    if ceiling is not None:
        roofline["measured_read_ceiling"] = round(ceiling["gbs"], 1)
        roofline["frac_of_measured_ceiling"] = round(l_gbs / ceiling["gbs"], 4)

    # ----------------------------------------------------------- CPU oracle
    cpu = None
    if not args.no_cpu_baseline and wl == "decode_step_1536x28":
        cpu = cpu_baseline_decode(inp, bufs, nbytes)
    elif not args.no_cpu_baseline and wl == "decode_attention_12q2kv128":
        cpu = cpu_baseline_attention(att, cfg["bytes_per_launch"])
    elif not args.no_cpu_baseline and wl == "ln_gelu_train_768x72":
        cpu = cpu_baseline_train(inp, tstep, nbytes)

    out = {
        "metric": METRIC if wl == "decode_step_1536x28" and B == 1 else METRIC.replace("batch 1", "batch %d" % B)
        if wl == "decode_step_1536x28" else ("decode attention GB/s (keys and values read once per step)"
                                             if wl == "decode_attention_12q2kv128" else
                                             ("training step (forward + backward) GB/s of algorithmic bytes, "
                                              "batch %d" % B if wl == "ln_gelu_train_768x72" else
                                              "%s weight-stream GB/s" % wl)),
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "us_per_step": round(us_step, 3),
        "us_per_step_median": round(us_med, 3),
        "us_per_step_ci95": [round(ci[0], 3), round(ci[1], 3)],
        "region_ms_per_step": round(total_ms / K, 6),
        "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "pct_of_measured_read_ceiling": round(100.0 * gbs / ceiling["gbs"], 2) if ceiling else None,
        "measured_read_ceiling": ceiling,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded normals, shapes of the pages' workload; no trained weights)",
        "config": cfg,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "cold": bool(args.cold),
    }
    print(json.dumps(out), flush=True)

def ci95_mean(x):
    """95 % confidence interval of the mean of the per-step times (Student t)."""
    from scipy import stats
    x = np.asarray(x, dtype=np.float64)
    n = len(x)
    if n < 2:
        return (float(x.mean()), float(x.mean()))
    h = stats.t.ppf(0.975, n - 1) * x.std(ddof=1) / np.sqrt(n)
    return (float(x.mean() - h), float(x.mean() + h))


# Launch shapes of the plain streaming read tried for the ceiling (grid,
# threads per workgroup, 16-byte loads in flight per lane): the best of each
# family measured on this GPU.
CEILING_CONFIGS = ((256, 256, 8), (256, 512, 4), (512, 256, 4), (2048, 256, 1), (1024, 256, 2))


def read_ceiling(W, torch, dev, gib=2, reps=5):
    """The measured streaming-read ceiling of this GPU: the best over a few
    launch shapes of wgn_stream_read over a 2 GiB buffer (each shape's median
    over reps reads), in GB/s."""
    buf = torch.empty(gib << 29, dtype=torch.int16, device=dev)  # gib GiB
    buf.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    nbytes = buf.numel() * 2
    best, best_cfg, rows = 0.0, None, []
    for grid, threads, depth in CEILING_CONFIGS:
        W.stream_read(buf, grid, threads, depth, sink)
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            W.stream_read(buf, grid, threads, depth, sink)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        gbs = nbytes / float(np.median(ts)) / 1e9
        rows.append([grid, threads, depth, round(gbs, 1)])
        if gbs > best:
            best, best_cfg = gbs, (grid, threads, depth)
    del buf
    torch.cuda.synchronize()
    return {"gbs": round(best, 1), "bytes": nbytes,
            "config": "grid %d, %d threads, %d loads in flight per lane" % best_cfg,
            "tried": rows, "pct_of_peak": round(100.0 * best / HBM_PEAK_GBS, 2)}


def host_cpu():
    """The host's CPU model and core counts (for the oracle's timing)."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"model": model, "nproc": os.cpu_count(), "usable_cpus": usable}


# ------------------------------------------------------------ HBM counters
ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "weight_gemv_norm_amd", "csrc")


# The sources each kernel's recorded traffic depends on (its code and its host planner).
KERNEL_SOURCES = {
    "chain_kernel": ("wgn_api.cpp", "wgn_kernels.hip", "wgn_loader.h", "wgn_prog.h", "wgn_numerics.h"),
    "gemm_kernel": ("wgn_api.cpp", "wgn_gemm.hip", "wgn_gemm.h", "wgn_numerics.h", "wgn_prog.h"),
    "decode_attention_kernel": ("wgn_attn.h", "wgn_attn.hip"),
    "gemv_int4_kernel": ("wgn_int4.hip",),
    "bwd_kernel": ("wgn_api.cpp", "wgn_bwd.hip", "wgn_bwd.h", "wgn_numerics.h"),
}


def kernel_of(workload: str, batch: int = 1, path: int = 0) -> str:
    if workload in ("decode_step_1536x28", "decoder_block_1536") and (batch > 16 or path == 3):
        return "gemm_kernel"
    return {"decode_attention_12q2kv128": "decode_attention_kernel",
            "gemv_int4_lmhead_151936": "gemv_int4_kernel",
            "ln_gelu_train_768x72": "bwd_kernel"}.get(workload, "chain_kernel")


def kernel_sources_digest(kernel: str = "chain_kernel") -> str:
    """SHA-256 over a kernel's sources: recorded counter figures are reported
    only while the kernel is unchanged since they were taken."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        h.update(name.encode())
        h.update(open(os.path.join(CSRC, name), "rb").read())
    return h.hexdigest()


def traffic_file(workload, batch, kernel):
    return os.path.join(ROOT, "profiles", "%s_%s_b%d_hbm_traffic.txt" % (kernel, workload, batch))


def recorded_traffic(workload, batch, kernel):
    path = traffic_file(workload, batch, kernel)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_sources_sha256") != kernel_sources_digest(kernel):
        return None
    return int(kv["traffic_bytes_per_launch"])


def _pmc_rows(path, counter):
    import csv
    rows = []
    for r in csv.DictReader(open(path)):
        if r.get("Counter_Name") == counter:
            rows.append((r["Kernel_Name"], int(r["Dispatch_Id"]), float(r["Counter_Value"])))
    return rows


def summarize_pmc(fetch_csv, write_csv, out_txt, workload, batch, copy_mib, path=0):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the workload's kernel, scaled
    by what the same counters read for a plain copy of copy_mib MiB.  The
    batched path runs several launches per step (one counter clear, norm
    passes, products): its figure is per step, the sum over the run's launches
    divided by its counter clears."""
    assert copy_mib > 0, "--calib-copy-mib of the profiled run is needed"
    kernel = kernel_of(workload, batch, path)
    out = {}
    for counter, csv_path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _pmc_rows(csv_path, counter)
        # per dispatch, the counter summed over its instances
        per = {}
        for name, d, v in rows:
            per.setdefault((name, d), 0.0)
            per[(name, d)] += v
        # the calibration copy: the runtime's plain buffer copy (not a dtype
        # conversion such as a BF16 copy kernel of the input set-up)
        copies = [v for (n, d), v in per.items() if "copyBuffer" in n]
        if kernel == "gemm_kernel":
            steps = sum(1 for (n, d) in per if "zero_words_kernel" in n)
            tot = sum(v for (n, d), v in per.items()
                      if "gemm_kernel" in n or "norm_rows64" in n or "zero_words_kernel" in n)
            kern = [tot / max(steps, 1)] if steps else []
            nk = steps
        else:
            kern = [v for (n, d), v in per.items() if kernel in n]
            nk = len(kern)
        assert kern and copies, (counter, len(kern), len(copies))
        copy_kib = max(copies)  # the calibration copy is the largest copy of the run
        scale = (copy_mib * 1024.0) / copy_kib
        out[counter] = (float(np.median(kern)), copy_kib, scale, nk)
    fetch = out["FETCH_SIZE"][0] * out["FETCH_SIZE"][2] * 1024
    write = out["WRITE_SIZE"][0] * out["WRITE_SIZE"][2] * 1024
    unit = "step (all launches)" if kernel == "gemm_kernel" else "dispatch"
    with open(out_txt, "w") as f:
        f.write("# HBM traffic of %s, %s, batch %d (rocprofv3 --pmc, one counter per run), per %s\n"
                % (kernel, workload, batch, unit))
        f.write("# commands (from the repository root):\n")
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            f.write("#   rocprofv3 --pmc %s --output-format csv -d gpurun_out/pmc_%s -o run -- python bench.py "
                    "--workload %s --batch %d%s --steps 10 --warmup 3 --no-cpu-baseline --no-ceiling "
                    "--calib-copy-mib %d\n"
                    % (c, c.lower(), workload, batch,
                       " --path 3" if path == 3 else (" --ab-rounds 2" if workload == "ln_gelu_train_768x72" else ""),
                       copy_mib))
        f.write("# calibration: a plain device copy of %d MiB reads and writes %d KiB\n"
                % (copy_mib, copy_mib * 1024))
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            k, cp, sc, n = out[c]
            f.write("%s_kib_per_dispatch_median: %.1f\n" % (c.lower(), k))
            f.write("%s_dispatches: %d\n" % (c.lower(), n))
            f.write("%s_copy_kib: %.1f\n" % (c.lower(), cp))
            f.write("%s_scale: %.5f\n" % (c.lower(), sc))
        f.write("fetch_bytes_per_launch: %d\n" % int(fetch))
        f.write("write_bytes_per_launch: %d\n" % int(write))
        f.write("traffic_bytes_per_launch: %d\n" % int(fetch + write))
        f.write("kernel_sources_sha256: %s\n" % kernel_sources_digest(kernel))
    print(open(out_txt).read())


def cpu_baseline_decode(inp, bufs, nbytes, budget_s=12.0, max_steps=45):
    """Time the CPU oracle (as it stands) on whole decode steps of the same
    workload (all 28 blocks and the LM head, free-running on its own outputs),
    repeated until about budget_s seconds of CPU work have been spent."""
    from oracle import oracle as O
    from synth.gen import bf16_bits_to_numpy as bb
    print("[bench] cpu baseline: copying weights to host", file=sys.stderr, flush=True)
    layers = [{k: bb(v) for k, v in L.items()} for L in inp["layers"]]
    g_f, W_lm, h0 = bb(inp["g_f"]), bb(inp["W_lm"]), bb(inp["h"])
    threads = max(1, min(host_cpu()["usable_cpus"] or 1, 16))
    O.set_threads(threads)
    eps = float(np.float32(inp["eps"]))

    def one_step():
        h = h0
        for L in layers:
            for name in ("wq", "wk", "wv"):
                O.stage(h, L[name], norm=O.NORM_RMS, eps=eps, gamma=L["g1"])
            h1 = O.stage(L["a"], L["wo"], residual=h)
            s = O.stage(h1, L["wg"], norm=O.NORM_RMS, eps=eps, gamma=L["g2"], epi=O.EPI_SWIGLU, W_up=L["wu"])
            h = O.stage(s, L["wd"], residual=h1)
        return O.lmhead_argmax(h, g_f, W_lm, eps=eps)[0]

    t0 = time.perf_counter()
    n = 0
    while n < max_steps:
        one_step()
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = (time.perf_counter() - t0) / n
    print("[bench] cpu baseline: %d steps, %.3f s per step on %d threads" % (n, dt, threads),
          file=sys.stderr, flush=True)
    # the same oracle on one thread: one whole step (its result is bit-identical)
    O.set_threads(1)
    t1 = time.perf_counter()
    one_step()
    dt1 = time.perf_counter() - t1
    O.set_threads(threads)
    print("[bench] cpu baseline: one step on 1 thread %.3f s" % dt1, file=sys.stderr, flush=True)
    return {"value": round(nbytes / dt / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "seconds_per_step": round(dt, 4), "us_per_step": round(dt * 1e6, 1),
            "single_thread_seconds_per_step": round(dt1, 3),
            "single_thread_value": round(nbytes / dt1 / 1e9, 4), "host": host_cpu(),
            "sample": "%d full decode steps (28 blocks + LM head + argmax, batch 1), free-running in the "
                      "binary64 C oracle with OpenMP over rows on %d threads (cores = threads used), then one "
                      "step on 1 thread; value = algorithmic bytes / mean step time" % (n, threads)}


def train_prefetch_ab(ts, g_on, g_off, torch, rounds, scrub=None, scrub_sink=None, W=None, reps=10):
    """Interleaved A/B of the training step with the backward prefetch on and
    off (one HIP graph each), `rounds` rounds of `reps` replays per setting in
    alternating order; then the backward alone (prep + backward launches,
    eager) with events around each call, prefetch on.  Saving = 1 - on / off,
    paired by round, with a 95 % confidence interval."""
    on, off = [], []
    for r in range(rounds):
        order = ((g_on, on), (g_off, off)) if r % 2 == 0 else ((g_off, off), (g_on, on))
        for g, acc in order:
            ev = []
            for _ in range(reps):
                if scrub is not None:
                    W.stream_read(scrub, 2048, 256, 1, scrub_sink)
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                g.replay()
                b.record()
                ev.append((a, b))
            torch.cuda.synchronize()
            acc.append(float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3)
    ts.check()
    on, off = np.array(on), np.array(off)
    sav = 1.0 - on / off
    ci = ci95_mean(sav)
    # the backward launches alone, on the stream they are launched on
    st = torch.cuda.current_stream()
    saved = ts.prefetch
    res = {}
    for pf in (True, False):
        ts.prefetch = pf
        per = []
        for _ in range(rounds * 2):
            ts.forward()
            if scrub is not None:
                W.stream_read(scrub, 2048, 256, 1, scrub_sink)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(st)
            ts.backward()
            b.record(st)
            torch.cuda.synchronize()
            per.append(a.elapsed_time(b) * 1e3)
        res[pf] = np.array(per)
    ts.prefetch = saved
    ts.check()
    out = {"rounds": rounds, "replays_per_round": reps,
           "step_us_prefetch_on": round(float(on.mean()), 3), "step_us_prefetch_off": round(float(off.mean()), 3),
           "saving_pct": round(100.0 * float(sav.mean()), 3),
           "saving_pct_ci95": [round(100.0 * ci[0], 3), round(100.0 * ci[1], 3)],
           # the prefetch rule of the forward plans: kept only if the 95 % CI of
           # the saving clears +1 %
           "prefetch_kept": bool(100.0 * ci[0] > 1.0),
           "backward_us_mean": round(float(res[True].mean()), 3),
           "backward_us_median": round(float(np.median(res[True])), 3),
           "backward_us_mean_prefetch_off": round(float(res[False].mean()), 3)}
    print("[bench] prefetch A/B: %s" % out, file=sys.stderr, flush=True)
    return out


def cpu_baseline_train(inp, ts, nbytes, budget_s=12.0):
    """The CPU oracle (as it stands) on a bounded sample of the training step:
    the forward stage and the block backward of a few blocks (from the last
    one down, on the GPU step's own activations), scaled to all blocks."""
    from oracle import oracle as O
    from synth.gen import bf16_bits_to_numpy as bb
    threads = max(1, min(host_cpu()["usable_cpus"] or 1, 16))
    O.set_threads(threads)
    eps = float(np.float32(inp["eps"]))
    layers = inp["layers"]
    xs = [bb(x) for x in ts.bufs["x"]]
    n = len(layers)
    gy = O.mean_square_grad(xs[n])
    t0 = time.perf_counter()
    done = 0
    for i in range(n - 1, -1, -1):
        L = {k: bb(v) for k, v in layers[i].items()}
        O.stage(xs[i], L["W"], norm=O.NORM_LAYER, eps=eps, gamma=L["gamma"], beta=L["beta"], bias=L["bias"],
                epi=O.EPI_GELU_TANH)
        r = O.block_backward(xs[i], L["W"], gy, gamma=L["gamma"], beta=L["beta"], eps=eps, bias=L["bias"])
        gy = O.to_bf16_bits(r["gx"])
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = (time.perf_counter() - t0) / done * n
    print("[bench] cpu baseline: %d of %d blocks, %.3f s per step on %d threads" % (done, n, dt, threads),
          file=sys.stderr, flush=True)
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "seconds_per_step": round(dt, 4), "host": host_cpu(),
            "sample": "forward stage + block backward of %d of the %d blocks (last first), binary64 C oracle "
                      "with OpenMP over rows on %d threads, scaled to the whole step" % (done, n, threads)}


def cpu_baseline_attention(att, bytes_per_layer, budget_s=10.0, max_reps=200):
    """Time the CPU oracle (as it stands) on the attention of one layer of the
    same workload (the same cache length, every slot valid), repeated until
    about budget_s seconds of CPU work have been spent."""
    from oracle import oracle as O
    from synth.gen import bf16_bits_to_numpy as bb
    t = att[0]
    a = [bb(t[k]) for k in ("q", "k_new", "v_new", "k_cache", "v_cache")]
    pos = t["pos"].cpu().numpy()
    threads = max(1, min(host_cpu()["usable_cpus"] or 1, 16))
    O.set_threads(threads)
    t0 = time.perf_counter()
    n = 0
    while n < max_reps:
        O.decode_attention(*a, pos)
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = (time.perf_counter() - t0) / n
    print("[bench] cpu baseline: %d layer calls, %.4f s each on %d threads" % (n, dt, threads),
          file=sys.stderr, flush=True)
    return {"value": round(bytes_per_layer / dt / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "seconds_per_layer": round(dt, 5), "host": host_cpu(),
            "sample": "%d calls of one layer's attention (same cache length and batch) in the binary64 C "
                      "oracle with OpenMP over query heads; value = algorithmic bytes per layer / mean call "
                      "time" % n}


if __name__ == "__main__":
    main()
