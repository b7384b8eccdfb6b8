#!/usr/bin/env python3
"""Benchmark of the MXFP4 routed-expert MoE layer on one MI355X (gfx950).

    python bench.py [--steps K] [--warmup W] [--workload decode|tiny|ep_share|prefill|a4|a8|verify_bB]

A step is one whole forward of the layer (route, permutation, gate_up + clamped
SwiGLU, down + weighted combine, output cast) over one batch of seeded synthetic
inputs that are resident in HBM before timing starts.  The default workload is
the decode step (T=16, H=2048, I=1536, 64 experts, top-8).  Expert weights are
rotated over several copies so that the 256 MB MALL cannot serve a step from the
previous one.  Prints one JSON line.

Roofline: per-phase durations come from HIP events that the library records
around its phases on the stream it launches on (mxfp4_moe_forward_timed), in a
second timed loop.  The dominant phase's achieved rate is its algorithmic
bytes (or flops) per launch divided by its mean duration.  Algorithmic bytes
count only the experts the routing touches: each touched expert's packed codes
plus scale bytes of the matrix the kernel streams, plus the activations it must
read and write once.

cpu_baseline: the CPU oracle (test infrastructure, plain C + OpenMP) timed on a
bounded sample of the same workload on this host's cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "fp4": 10100.0}
METRIC = "MXFP4 MoE tokens/s; decode HBM TB/s and prefill MFMA util vs peak"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode")
    ap.add_argument("--copies", type=int, default=0, help="weight copies to rotate (0: auto)")
    ap.add_argument("--deterministic", action="store_true", help="ordered combine")
    ap.add_argument("--shared", action="store_true",
                    help="with the shared expert (one more expert every token reads)")
    ap.add_argument("--bf16-experts", type=int, default=0,
                    help="keep this many experts (evenly spaced) in bf16 inside fused buffers; "
                         "times the whole step only (no phase split, roofline null)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--copy-calibration", type=int, default=0,
                    help="only run a plain device copy of this many bytes (counter calibration)")
    return ap.parse_args()


def source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mxfp4_block_scaled_router_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def copy_calibration(nbytes: int):
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "launches": 10}), flush=True)


def build_inputs(wl, copies, shared=False):
    import numpy as np
    import torch
    import mxfp4_block_scaled_router_amd as mx
    from mxfp4_block_scaled_router_amd import workloads as W
    inp = W.make_inputs(wl)
    dims = mx.Dims.make(wl.T, wl.H, wl.I, wl.E_global, wl.E_local, wl.first_local, a4=wl.a4,
                        shared=shared, a8=wl.a8)
    nw = wl.E_local + (1 if shared else 0)  # experts in the weight buffers
    x = torch.from_numpy(inp["x"].view(np.int16)).view(torch.bfloat16).cuda()
    logits = torch.from_numpy(inp["logits"]).cuda()
    if wl.weight_kind == "uniform":
        if shared:
            inp.update(zip(("w13", "w13s", "w2", "w2s"),
                           W.make_uniform_weights(wl.replace(E_local=nw))))
        canon = [torch.from_numpy(inp[k]).cuda() for k in ("w13", "w13s", "w2", "w2s")]
    else:
        # Student-t weights drawn on the GPU and quantised by the library's OCP
        # quantiser (the load-time step), expert by expert
        E, H, I = nw, wl.H, wl.I
        canon = [torch.empty((E, 2 * I, H // 2), dtype=torch.uint8, device="cuda"),
                 torch.empty((E, 2 * I, H // 32), dtype=torch.uint8, device="cuda"),
                 torch.empty((E, H, I // 2), dtype=torch.uint8, device="cuda"),
                 torch.empty((E, H, I // 32), dtype=torch.uint8, device="cuda")]
        for e in range(E):
            c, s = mx.mxfp4_moe_quantize(W.student_t_expert(wl, e, "w13", device="cuda"))
            canon[0][e].copy_(c)
            canon[1][e].copy_(s)
            c, s = mx.mxfp4_moe_quantize(W.student_t_expert(wl, e, "w2", device="cuda"))
            canon[2][e].copy_(c)
            canon[3][e].copy_(s)
    pw = mx.mxfp4_moe_preshuffle(dims, *canon)
    del canon
    bank = sum(t.numel() for t in pw)
    if copies <= 0:
        copies = max(1, min(8, math.ceil(1.5e9 / bank)))
    banks = [pw] + [tuple(t.clone() for t in pw) for _ in range(copies - 1)]
    torch.cuda.synchronize()
    return inp, dims, x, logits, banks, bank


def cpu_baseline(wl, inp, target_s, shared=False):
    """Oracle on a bounded sample: whole steps when one step is small enough,
    else a subset of tokens (token_mask); returns tokens/s on this host."""
    import numpy as np
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or len(os.sched_getaffinity(0))

    def run(mask):
        t0 = time.perf_counter()
        oracle.moe_forward(inp["x"], inp["logits"], inp["w13"], inp["w13s"], inp["w2"], inp["w2s"],
                           top_k=wl.top_k, clamp_limit=wl.clamp_limit, E_global=wl.E_global,
                           first_local=wl.first_local, a4=wl.a4, a8=wl.a8, shared=shared,
                           token_mask=mask,
                           want_act=False, nthreads=threads)
        return time.perf_counter() - t0

    # probe with a few tokens to size the sample
    n_probe = min(wl.T, 4)
    mask = np.zeros(wl.T, bool)
    mask[:n_probe] = True
    t_probe = run(mask)
    per_tok = t_probe / n_probe
    if per_tok * wl.T <= target_s:
        # one full step sizes the rest (a full step touches more experts than
        # the probe, so the probe's per-token time overestimates it)
        t = run(None)
        reps = min(50, max(1, int(target_s / max(t, 1e-6))))
        t += sum(run(None) for _ in range(reps - 1))
        return {"value": wl.T * reps / t, "unit": "tokens/s", "cores": threads, "kind": "oracle",
                "sample": "%d full steps of the %s workload (%d tokens each), %.1f s" %
                (reps, wl.name, wl.T, t)}
    n = max(1, min(wl.T, int(target_s / max(per_tok, 1e-6))))
    rng = np.random.default_rng(0)
    mask = np.zeros(wl.T, bool)
    mask[rng.choice(wl.T, size=n, replace=False)] = True
    t = run(mask)
    return {"value": n / t, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%d of %d tokens of one %s step (routing of all tokens, expert work and "
                      "combine of the sampled ones), %.1f s" % (n, wl.T, wl.name, t)}


def bench_bf16_experts(args, wl):
    """Whole-step timing of the layer with experts kept in bf16 inside fused
    buffers (mxfp4_moe_forward_mixed), against the all-MXFP4 layer on the same
    packed weights."""
    import numpy as np
    import torch
    import mxfp4_block_scaled_router_amd as mx
    from mxfp4_block_scaled_router_amd import workloads as W
    inp, dims, x, logits, banks, bank_bytes = build_inputs(wl, args.copies, args.shared)
    if wl.weight_kind != "uniform" or args.shared:
        sys.exit("--bf16-experts: uniform-code workloads without --shared only")
    Ew = wl.E_local
    n = min(args.bf16_experts, Ew)
    excluded = np.zeros(Ew, bool)
    excluded[(np.arange(n) * Ew) // n] = True
    idx = np.nonzero(excluded)[0]
    b13 = np.stack([W.bf16_expert(wl, e, "w13") for e in idx])
    b2 = np.stack([W.bf16_expert(wl, e, "w2") for e in idx])
    f13, f13s = W.fuse(inp["w13"], inp["w13s"], b13, excluded)
    f2, f2s = W.fuse(inp["w2"], inp["w2s"], b2, excluded)
    dev = [torch.from_numpy(a).cuda() for a in (f13, f13s, f2, f2s)]
    mixed = [mx.mxfp4_moe_preshuffle_fused(dims, list(excluded), *dev) for _ in range(len(banks))]
    del dev
    k = wl.top_k
    ws = torch.empty(mx.mxfp4_moe_workspace_bytes(dims, k), dtype=torch.uint8, device="cuda")
    out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")

    def time_steps(step):
        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for i in range(args.steps):
            step(i)
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / args.steps

    ms_mixed = time_steps(lambda i: mx.mxfp4_moe_forward_mixed(
        dims, mixed[i % len(mixed)][1], x, logits, *mixed[i % len(mixed)][0], k, wl.clamp_limit,
        out=out, workspace=ws))
    ms_packed = time_steps(lambda i: mx.mxfp4_moe_forward(
        dims, x, logits, *banks[i % len(banks)], k, wl.clamp_limit, out=out, workspace=ws))
    rt = mx.mxfp4_moe_route(dims, logits, k, workspace=ws)
    counts = rt["counts"].cpu().numpy()
    rec = {
        "metric": METRIC, "value": wl.T / (ms_mixed * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_mixed,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded: x~N(0,1) bf16, logits~N(0,1), uniform E2M1 codes; bf16 "
                "experts N(0, 0.16^2))",
        "config": {"workload": "%s with %d of %d experts kept in bf16" % (wl.name, n, Ew),
                   "bf16_experts": [int(e) for e in idx],
                   "rows_on_bf16_experts": int(counts[idx].sum()),
                   "rows_total": int(counts.sum()), "parallelism": "single GPU"},
        "all_mxfp4_ms_per_step": ms_packed,
        "roofline": None,
        "cpu_baseline": None,
    }
    print(json.dumps(rec), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(requested --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    import numpy as np
    import torch
    import mxfp4_block_scaled_router_amd as mx
    from mxfp4_block_scaled_router_amd import workloads as W

    wl = W.WORKLOADS[args.workload]
    mx.load_library()
    if args.bf16_experts:
        return bench_bf16_experts(args, wl)
    inp, dims, x, logits, banks, bank_bytes = build_inputs(wl, args.copies, args.shared)
    if args.deterministic:
        dims.flags |= mx.MXFP4_MOE_DETERMINISTIC
    k = wl.top_k
    ws = torch.empty(mx.mxfp4_moe_workspace_bytes(dims, k), dtype=torch.uint8, device="cuda")
    plan = mx.mxfp4_moe_plan(dims, k)
    out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda")

    # routing statistics (same logits every step)
    rt = mx.mxfp4_moe_route(dims, logits, k, workspace=ws)
    counts = rt["counts"].cpu().numpy()
    touched = int((counts > 0).sum())
    n_assign = int(counts.sum())

    def step(i):
        mx.mxfp4_moe_forward(dims, x, logits, *banks[i % len(banks)], k, wl.clamp_limit, out=out,
                             workspace=ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(args.steps):
        step(i)
    t1.record()
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps

    # per-phase timing loop
    nph = len(mx.PHASES)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nph + 1)] for _ in range(args.steps)]
    for row in evs:
        for e in row:
            e.record()
    torch.cuda.synchronize()
    for i in range(args.steps):
        mx.mxfp4_moe_forward_timed(dims, x, logits, *banks[i % len(banks)], k, wl.clamp_limit,
                                   evs[i], out=out, workspace=ws)
    torch.cuda.synchronize()
    phase_ms = {p: float(np.mean([row[j].elapsed_time(row[j + 1]) for row in evs]))
                for j, p in enumerate(mx.PHASES)}

    # algorithmic work
    H, I, T = wl.H, wl.I, wl.T
    w13_b = 2 * I * H // 2 + 2 * I * H // 32
    w2_b = H * I // 2 + H * I // 32
    bytes_ = {
        "route": T * wl.E_global * 4 + T * k * 8,
        "gate_up": touched * w13_b + T * H * 2 + n_assign * I * 2,
        "down": touched * w2_b + n_assign * I * 2 + T * H * 2,
        # ordered gather reads every local slot's y row; atomic path casts out32
        "combine": (n_assign * H * 4 if plan["ordered_combine"] else T * H * 4) + T * H * 2,
    }
    flops = {"route": 0, "gate_up": 2 * n_assign * 2 * I * H, "down": 2 * n_assign * H * I,
             "combine": 0}
    step_bytes = touched * (w13_b + w2_b) + T * H * 2 + T * wl.E_global * 4 + T * H * 2
    dominant = max(("gate_up", "down"), key=lambda p: phase_ms[p])
    # an FP8 x FP4 product issues at the FP8 rate
    mfma_dtype = "fp4" if wl.a4 else ("fp8" if wl.a8 else "bf16")
    if wl.name in ("prefill", "a4", "a8"):
        achieved = flops[dominant] / (phase_ms[dominant] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": MFMA_PEAK_TFLOPS[mfma_dtype],
                "unit": "TFLOP/s"}
    else:
        achieved = bytes_[dominant] / (phase_ms[dominant] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["kernel"] = dominant
    roof["algorithmic_per_launch"] = bytes_[dominant] if roof["bound"] == "hbm" else flops[dominant]
    roof["mean_launch_ms"] = phase_ms[dominant]
    roof["traffic"] = None
    tfile = os.path.join(ROOT, "profiles", "traffic_%s.json" % wl.name)
    if os.path.exists(tfile):
        with open(tfile) as f:
            tr = json.load(f)
        if tr.get("source_digest") == source_digest() and tr.get("kernel_phase") == dominant:
            roof["traffic"] = tr.get("traffic_bytes_per_launch")

    rec = {
        "metric": METRIC,
        "value": wl.T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": mfma_dtype,
        "data": "synthetic (seeded: %s)" % ("x~N(0,1) bf16, logits~N(0,1), uniform E2M1 codes"
                                            if wl.weight_kind == "uniform" else
                                            "Student-t(3) weights quantised on the GPU"),
        "config": {"workload": "%s T=%d H=%d I=%d E=%d/%d top-%d clamp=%g%s" % (
            wl.name, T, H, I, wl.E_local, wl.E_global, k, wl.clamp_limit,
            (" A4" if wl.a4 else "") + (" A8" if wl.a8 else "") +
            (" +shared expert" if args.shared else "")),
            "T": T, "H": H, "I": I, "E_local": wl.E_local, "shared_expert": bool(args.shared),
            "E_global": wl.E_global, "top_k": k, "touched_experts": touched,
            "local_assignments": n_assign, "weight_copies_rotated": len(banks),
            "bank_bytes": bank_bytes, "combine": "ordered" if plan["ordered_combine"] else "atomic",
            "tile_rows": plan["tile_rows"],
            "parallelism": "single GPU"},
        "roofline": roof,
        "step": {"hbm_bytes": step_bytes, "hbm_GBps": step_bytes / (ms_per_step * 1e-3) / 1e9,
                 "hbm_frac": step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
                 "flops": flops["gate_up"] + flops["down"],
                 "mfma_frac": (flops["gate_up"] + flops["down"]) / (ms_per_step * 1e-3) / 1e12 /
                 MFMA_PEAK_TFLOPS[mfma_dtype]},
        "phase_ms": phase_ms,
        "source_digest": source_digest(),
    }
    if not args.no_cpu_baseline:
        if "w13" not in inp:
            rec["cpu_baseline"] = None   # Student-t weights live on the GPU only
        else:
            rec["cpu_baseline"] = cpu_baseline(wl, inp, args.cpu_seconds, args.shared)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
