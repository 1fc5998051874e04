"""PACK3D forward benchmark on one MI355X.

A step is one pack3d_forward over one batch of seeded synthetic input that is
already resident in HBM: index build, rotate-then-pool summaries, the
query-to-summary branch on bf16 matrix cores, and the local branch fused
with the gated mix. The default workload is the 65,536-token volume (grid
32 x 32 x 64, batch 1, 8 heads, head dim 48, 2x2x2 blocks -> 8,192
summaries, bf16, block-contiguous packing).

Prints one JSON line: throughput in tokens/s, the roofline of the dominant
kernel (the global branch: algorithmic flops per launch over its average
launch time, timed with HIP events recorded by pack3d_forward on the launch
stream), per-stage times and HBM-roofline fractions, and the CPU oracle
timed on a bounded sample of the same workload on this host's cores.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 3] [--block bz,by,bx]
  python bench.py --copy-calibration    # plain device copy, for counter scaling
"""
import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 matrix peak, TFLOP/s
METRIC = "PACK3D fwd tokens/sec at 65,536 tokens, 1 MI355X; % of HBM/MFMA roofline"
STAGES = ("index", "summarize", "global", "local_mix")
DOMINANT_SRC = os.path.join(ROOT, "geometry_aware_sparse_amd", "csrc", "global_mfma.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_global_mfma.json")


def algorithmic(w, es=2):
    """Algorithmic work per launch of each stage: what the method must read,
    write or compute once (bytes / flops), not what a kernel happens to move."""
    B, N, H, D, M = w.B, w.N, w.H, w.D, w.M
    row = H * D * es              # a token's query (or output) row
    kvrow = w.kv_heads * D * es   # a token's key (or value) row
    return {
        # coords (12 B/token) read, slot map (4 B/site) written, RoPE table
        "index": {"bytes": N * 12 + N * 4},
        # K and V read once, slot map read, summaries (per KV head) written
        "summarize": {"bytes": B * N * 2 * kvrow + N * 4 + B * M * 2 * kvrow},
        # Q read, O_glob written, coords read, summaries read once; 4*D flops
        # per (token, query head, summary) pair (QK^T and PV)
        "global": {"bytes": B * N * 2 * row + N * 12 + B * M * 2 * kvrow,
                   "flops": 4.0 * B * H * N * M * D},
        # Q, K, V read, O_glob and gate read (fused mix), O written, slot map
        "local_mix": {"bytes": B * N * (3 * row + 2 * kvrow + H * es) + N * 4},
    }


def _sha(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def measured_traffic(config):
    """HBM bytes per launch of the dominant kernel from the committed
    rocprofv3 counter summary, or None when the kernel source has changed
    since the counters were taken or the counters were taken on another
    configuration (workload, block shape, KV heads, summary RoPE)."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("source_sha") != _sha(DOMINANT_SRC) or t.get("config") != config:
        return None
    return t.get("hbm_bytes_per_launch")


def traffic_config(line_config):
    """The part of a bench line's config that the counters depend on."""
    return {k: line_config[k] for k in ("workload", "block", "kv_heads", "summary_rope")}


def cpu_baseline(w, coords, q, k, v, g, target_s=15.0):
    """The oracle as it stands, on a bounded sample: rotations and summaries
    over every token, local/global/mix at a seeded sample of query tokens."""
    import numpy as np

    import oracle
    od = oracle.make_desc(w.B, w.N, w.H, w.D, w.grid, w.block, rope_base=w.rope_base,
                          kv_heads=w.kv_heads)
    rng = np.random.default_rng(0)
    # two short probes separate the fixed cost (rotations, summaries) from the
    # per-token cost, to size the sample for ~target_s of work
    t = []
    for n_probe in (64, 512):
        probe = rng.choice(w.N, n_probe, replace=False).astype(np.int32)
        t0 = time.perf_counter()
        oracle.forward(od, coords, q, k, v, g, rows=probe)
        t.append(time.perf_counter() - t0)
    per_row = max((t[1] - t[0]) / 448.0, 1e-7)
    fixed = max(t[0] - 64 * per_row, 0.0)
    n = int(min(w.N, max(512, (target_s - fixed) / per_row)))
    rows = rng.choice(w.N, n, replace=False).astype(np.int32)
    t0 = time.perf_counter()
    oracle.forward(od, coords, q, k, v, g, rows=rows)
    dt = time.perf_counter() - t0
    return {"value": w.B * n / dt, "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": (f"fp64 C oracle, full forward of {w.name} with rotations and summaries over "
                       f"all {w.N} tokens and local/global/mix at {n} seeded query tokens "
                       f"(x batch {w.B}); {dt:.1f} s wall")}


def algorithmic_backward(w, es=2):
    """Algorithmic work of the backward's stages (bytes / flops per launch
    sequence): what the gradients must read, write or compute once."""
    B, N, H, D, M = w.B, w.N, w.H, w.D, w.M
    row, kvrow = H * D * es, w.kv_heads * D * es
    return {
        # coords read, slot map written; K, V read and summaries written
        "geom_summaries": {"bytes": N * 16 + B * N * 2 * kvrow + B * M * 2 * kvrow},
        # 3 contractions per (token, query head, summary) on the query side
        # (scores, dO v_sum^T, dT k_sum) and 4 on the summary side (scores,
        # dO v_sum^T, dT^T q~, P^T dO): 14*D flops per pair
        "global": {"flops": 14.0 * B * H * N * M * D,
                   "bytes": B * N * (3 * row + H * 4) + B * M * 2 * kvrow},
        # Q, dO, O_glob, gate read and dQ, dgate written (query side), K, V
        # read and dK, dV written (key side), fp32 dq~_glob and the summary
        # gradients read once
        "local": {"bytes": B * N * (3 * row + 2 * H * es + 4 * kvrow + H * D * 4)
                  + B * M * 2 * w.kv_heads * D * 4},
    }


def backward_bench(args, w, dt, es):
    """fwd+bwd of the operator: pack3d_forward_train then pack3d_backward."""
    import numpy as np
    import torch

    import geometry_aware_sparse_amd as gas
    import pack3d_inputs as pi

    t_in = time.perf_counter()
    coords = pi.packing_coords(w.grid, w.packing, block=w.block, seed=w.seed("perm"))
    q, k, v, g = pi.pack_fields(pi.make_fields(w), coords, w.grid)
    dout = pi.pack_fields((pi.make_dout(w),), coords, w.grid)[0]
    print(f"{w.name}: host inputs ready in {time.perf_counter() - t_in:.1f} s", file=sys.stderr,
          flush=True)
    dev = torch.device("cuda:0")
    dc = torch.from_numpy(coords).to(dev)
    dq, dk, dv, dg, ddo = (torch.from_numpy(a).to(dev).to(dt).contiguous()
                           for a in (q, k, v, g, dout))
    d = gas.make_desc(w.B, w.N, w.H, w.D, w.grid, w.block, dtype=dt, rope_base=w.rope_base,
                      summary_centre=args.summary_centre, kv_heads=w.kv_heads)
    ws = torch.empty(gas.pack3d_workspace_bytes(d), dtype=torch.uint8, device=dev)
    bws = torch.empty(gas.pack3d_backward_workspace_bytes(d), dtype=torch.uint8, device=dev)
    out = torch.empty_like(dq)
    saved = torch.empty(gas.pack3d_saved_bytes(d), dtype=torch.uint8, device=dev)
    grads = (torch.empty_like(dq), torch.empty_like(dk), torch.empty_like(dv), torch.empty_like(dg))
    nf, nb = 2 * gas.PACK3D_NUM_STAGES, 2 * gas.PACK3D_NUM_BWD_STAGES
    BSTAGES = ("geom_summaries", "global", "local")
    gi = BSTAGES.index("global")

    def make_events(n, count, only=None):
        # materialised HIP events; with `only`, the other marks are None
        evs = [[torch.cuda.Event(enable_timing=True) if only is None or j // 2 == only else None
                for j in range(n)] for _ in range(count)]
        for row in evs:
            for e in row:
                if e is not None:
                    e.record()
        return evs

    # the timed steps time the global backward (its roofline) on every
    # SAMPLE-th step only; the per-stage breakdown comes from extra steps after
    stage_passes = min(args.steps, 10)
    sample = max(1, args.steps // 10)
    tev = make_events(nb, args.steps, only=gi)
    fev = make_events(nf, stage_passes)
    bev = make_events(nb, stage_passes)

    def step(f_events=None, b_events=None):
        gas.pack3d_forward_train(d, dc, dq, dk, dv, dg, out=out, saved=saved, workspace=ws,
                                 stage_events=f_events)
        gas.pack3d_backward(d, dc, dq, dk, dv, dg, saved, ddo, workspace=bws, grads=grads,
                            stage_events=b_events)

    torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for s_ in range(args.steps):
        step(None, tev[s_] if s_ % sample == 0 else None)
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(stop) / args.steps
    global_ms = float(np.mean([tev[s_][2 * gi].elapsed_time(tev[s_][2 * gi + 1])
                               for s_ in range(0, args.steps, sample)]))
    for s_ in range(stage_passes):
        step(fev[s_], bev[s_])
    torch.cuda.synchronize()
    fstage = {n: float(np.mean([e[2 * i].elapsed_time(e[2 * i + 1]) for e in fev]))
              for i, n in enumerate(STAGES)}
    bstage = {n: float(np.mean([e[2 * i].elapsed_time(e[2 * i + 1]) for e in bev]))
              for i, n in enumerate(BSTAGES)}
    bwork = algorithmic_backward(w, es)
    gl_s = global_ms * 1e-3
    achieved = bwork["global"]["flops"] / gl_s / 1e12
    roofline = {"bound": "mfma", "kernel": "global backward (k_bwd_gq_mfma + k_bwd_gk_mfma)",
                "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_BF16_PEAK_TFS, 4), "traffic": None}
    stages = {"fwd_" + n: {"ms": round(v_, 4)} for n, v_ in fstage.items()}
    for n, v_ in bstage.items():
        gbs = bwork[n]["bytes"] / (v_ * 1e-3) / 1e9
        stages["bwd_" + n] = {"ms": round(v_, 4), "algorithmic_bytes": bwork[n]["bytes"],
                              "GB/s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    line = {
        "metric": "PACK3D fwd+bwd tokens/sec (training forward + backward of the operator), 1 MI355X",
        "value": round(w.tokens / (ms_step * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": w.name, "grid_zyx": list(w.grid), "batch": w.B, "heads": w.H,
                   "kv_heads": w.kv_heads, "head_dim": w.D, "block": list(w.block),
                   "summaries": w.M, "tokens": w.tokens, "packing": w.packing,
                   "summary_rope": "centre" if args.summary_centre else "token"},
        "roofline": roofline, "stages": stages,
        "stages_note": (f"global backward timed on every {sample}th timed step; per-stage "
                        f"events from {stage_passes} extra steps after the timed ones"),
        "wall_s_timed_region": round(wall, 4),
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def copy_calibration(nbytes=1 << 30, reps=5):
    """A plain device-to-device copy of known size, for scaling the HBM
    counters (FETCH_SIZE / WRITE_SIZE) of rocprofv3."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps}), flush=True)


def attainable_peaks(reps=20):
    """Attainable, not spec, peaks of this GPU: the HBM rate of a plain
    1 GiB device-to-device copy (read + write bytes over time) and the dense
    bf16 rate of a large library GEMM (the vendor BLAS on the matrix cores).
    Context for the roofline fractions, which stay against the spec peaks."""
    import torch
    out = {}
    a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    n = 8192
    x = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    y = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    for name, fn, work in (("hbm_copy", lambda: b.copy_(a), 2.0 * a.numel()),
                           ("bf16_gemm", lambda: torch.mm(x, y), 2.0 * n * n * n)):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        sec = e0.elapsed_time(e1) * 1e-3 / reps
        out[name] = round(work / sec * 1e-9 if name == "hbm_copy" else work / sec * 1e-12, 1)
    out["units"] = {"hbm_copy": "GB/s (read + write)", "bf16_gemm": "TFLOP/s (8192^3 torch.mm)"}
    print(json.dumps({"attainable_peaks": out}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--peaks", action="store_true",
                    help="measure attainable HBM copy and bf16 GEMM rates on this GPU")
    ap.add_argument("--summary-centre", action="store_true",
                    help="summary-centre variant: pool unrotated keys, rotate at the block centre")
    ap.add_argument("--backward", action="store_true",
                    help="time the training step (forward that keeps the backward's inputs, "
                         "then the backward) instead of the inference forward")
    ap.add_argument("--kv-heads", type=int, default=0,
                    help="grouped key/value heads (GQA/MQA) for the workload; 0 keeps H")
    ap.add_argument("--block", type=str, default="",
                    help="summary block shape 'bz,by,bx' in place of the workload's own")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the PACK3D "
              "forward is a single-GPU operator and the library has no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        copy_calibration()
        return
    if args.peaks:
        attainable_peaks()
        return

    import geometry_aware_sparse_amd as gas
    import pack3d_inputs as pi

    w = pi.workload(args.workload)
    if args.kv_heads:
        w = dataclasses.replace(w, Hkv=args.kv_heads)
    if args.block:
        blk = tuple(int(x) for x in args.block.split(","))
        if len(blk) != 3 or any(b < 1 or n % b for b, n in zip(blk, w.grid)):
            sys.exit(f"--block {args.block}: need three extents that divide the grid {w.grid}")
        w = dataclasses.replace(w, block=blk)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    es = 2 if w.dtype == "bf16" else 4
    if args.backward:
        backward_bench(args, w, dt, es)
        return
    t_in = time.perf_counter()
    coords = pi.packing_coords(w.grid, w.packing, block=w.block, seed=w.seed("perm"))
    q, k, v, g = pi.pack_fields(pi.make_fields(w), coords, w.grid)
    print(f"{w.name}: host inputs ready in {time.perf_counter() - t_in:.1f} s", file=sys.stderr,
          flush=True)
    dev = torch.device("cuda:0")
    dc = torch.from_numpy(coords).to(dev)
    dq, dk, dv, dg = (torch.from_numpy(a).to(dev).to(dt).contiguous() for a in (q, k, v, g))
    d = gas.make_desc(w.B, w.N, w.H, w.D, w.grid, w.block, dtype=dt, rope_base=w.rope_base,
                      summary_centre=args.summary_centre, kv_heads=w.kv_heads)
    ws = torch.empty(gas.pack3d_workspace_bytes(d), dtype=torch.uint8, device=dev)
    out = torch.empty_like(dq)
    nev = 2 * gas.PACK3D_NUM_STAGES
    gi = STAGES.index("global")

    def make_events(n, only=None):
        # HIP events, materialised (recorded once) before they are handed
        # over; with `only`, the other marks are skipped (None)
        evs = [[torch.cuda.Event(enable_timing=True) if only is None or j // 2 == only else None
                for j in range(nev)] for _ in range(n)]
        for row in evs:
            for e in row:
                if e is not None:
                    e.record()
        return evs

    # Each recorded event drains the stream and costs microseconds, so the
    # timed steps time the global kernel (for its roofline) on every
    # SAMPLE-th step only, with its two marks; the per-stage breakdown comes
    # from a separate pass after the timed steps.
    sample = max(1, args.steps // 10)
    timed_events = make_events(args.steps, only=gi)
    stage_passes = min(args.steps, 20)
    stage_events = make_events(stage_passes)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        gas.pack3d_forward(d, dc, dq, dk, dv, dg, out=out, workspace=ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for s in range(args.steps):
        gas.pack3d_forward(d, dc, dq, dk, dv, dg, out=out, workspace=ws,
                           stage_events=timed_events[s] if s % sample == 0 else None)
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(stop)
    ms_step = total_ms / args.steps
    global_ms = float(np.mean([timed_events[s][2 * gi].elapsed_time(timed_events[s][2 * gi + 1])
                               for s in range(0, args.steps, sample)]))
    for s in range(stage_passes):
        gas.pack3d_forward(d, dc, dq, dk, dv, dg, out=out, workspace=ws,
                           stage_events=stage_events[s])
    torch.cuda.synchronize()
    stage_ms = {}
    for si, name in enumerate(STAGES):
        stage_ms[name] = float(np.mean([evs[2 * si].elapsed_time(evs[2 * si + 1])
                                        for evs in stage_events]))
    work = algorithmic(w, es)
    gflops = work["global"]["flops"]
    g_s = global_ms * 1e-3
    achieved = gflops / g_s / 1e12
    kname = (f"k_global_mfma<{w.D}>" if w.dtype == "bf16" and w.D in (48, 96)
             else "k_global_valu")
    roofline = {"bound": "mfma", "kernel": kname, "achieved": round(achieved, 1),
                "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_BF16_PEAK_TFS, 4), "traffic": None,
                "traffic_unit": "bytes/launch"}
    stage_roof = {}
    for name in STAGES:
        gbs = work[name]["bytes"] / (stage_ms[name] * 1e-3) / 1e9
        stage_roof[name] = {"ms": round(stage_ms[name], 4), "algorithmic_bytes": work[name]["bytes"],
                            "GB/s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    line = {
        "metric": METRIC, "value": round(w.tokens / (ms_step * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "grid_zyx": list(w.grid), "batch": w.B, "heads": w.H,
                   "kv_heads": w.kv_heads,
                   "head_dim": w.D, "block": list(w.block), "summaries": w.M,
                   "tokens": w.tokens, "packing": w.packing, "values": w.values,
                   "summary_rope": "centre" if args.summary_centre else "token"},
        "roofline": roofline,
        "stages": stage_roof,
        "stages_note": (f"global kernel timed on every {sample}th timed step; per-stage events "
                        f"from {stage_passes} extra steps after the timed ones"),
        "wall_s_timed_region": round(wall, 4),
    }
    roofline["traffic"] = measured_traffic(traffic_config(line["config"]))
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, coords, q, k, v, g)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
