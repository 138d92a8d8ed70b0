#!/usr/bin/env python3
"""µs per decode MoE block and achieved HBM GB/s on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload tp16_b1]

A step is one pass of the whole decode MoE block (router scoring, top-k and
plan, routed and shared expert gate/up + SwiGLU + down, weighted combine)
over one batch of synthetic bf16 input, through the C ABI (moe_block).
Default workload: one TP16 weight shard at batch 1 (d=7168, E=384, top-8,
I=Is=128).  Other workloads: tp16_b8, tp8_b64, tiny, dense (the attention
input projection, --batch B), oproj (the attention output projection with
the residual added, --batch B).

Weights are random (seeded torch generator on the GPU) in R rotating full
sets so that the bytes touched between two uses of a set exceed twice the
256 MB Infinity Cache plus L2: each timed step reads HBM, not cache.
Inputs are resident in HBM before the timed region.  W warm-up steps, then
exactly K timed steps between two synchronised HIP events.

Prints ONE JSON line.  Besides the headline, it carries
  roofline:     the dominant kernel (the fused block kernel where the block
                runs as one launch, else the launch with the largest time)
                timed with HIP events
                that its own dispatch records (hipExtLaunchKernel, on the
                launch stream), algorithmic bytes / duration against the
                8 TB/s HBM peak; traffic = counter-measured HBM bytes per
                launch from profiles/traffic.json while the kernels are
                unchanged since it was taken;
  cpu_baseline: the CPU oracle timed on this host on a bounded sample of the
                same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "µs per decode MoE block and achieved HBM GB/s (% of peak), batch 1–64"
MALL_L2_BYTES = 256e6 + 32e6


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="tp16_b1",
                    choices=["tiny", "tp16_b1", "tp16_b8", "tp8_b64", "dense", "oproj", "copy"])
    ap.add_argument("--batch", type=int, default=1, help="dense / oproj workload batch")
    ap.add_argument("--rotate", type=int, default=0, help="weight sets (0: enough to defeat caches)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--kernel-steps", type=int, default=100)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--schedule", default="auto", choices=["auto", "launches", "fused"],
                    help="moe_block schedule: one fused launch where it applies, or three launches")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of HIP graphs (one captured block per weight set) instead of plain "
                         "launches; every replay is first checked against the plain launch's bits")
    return ap.parse_args()


def rotations(bytes_per_step: float, cap_sets: int) -> int:
    r = int(2 * MALL_L2_BYTES // max(bytes_per_step, 1.0)) + 1
    return max(2, min(r, cap_sets))


# ---------------------------------------------------------------- MoE block

def moe_sets(cfg, R, seed, torch):
    """R full weight sets + per-set activations, bf16 (fp32 for tiny)."""
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    sets = []
    for r in range(R):
        g = torch.Generator(device="cuda").manual_seed(seed * 1000003 + r)
        rn = lambda shape, std: (torch.randn(shape, generator=g, device="cuda", dtype=dt) * std).to(dt)
        s = dict(
            X=rn((cfg.B, cfg.d), 1.0),
            Wr=rn((cfg.E, cfg.d), cfg.d ** -0.5),
            W13=rn((cfg.E, 2 * cfg.I, cfg.d), cfg.d ** -0.5),
            W2=rn((cfg.E, cfg.d, cfg.I), cfg.I ** -0.5),
            Ws13=rn((2 * cfg.Is, cfg.d), cfg.d ** -0.5) if cfg.Is else None,
            Ws2=rn((cfg.d, cfg.Is), cfg.Is ** -0.5) if cfg.Is else None,
            bias=None, bias_ld=0,
            ids=torch.empty((cfg.B, cfg.k), dtype=torch.int32, device="cuda"),
            out=torch.empty((cfg.B, cfg.d), dtype=dt, device="cuda"),
        )
        if cfg.routing == "gumbel":
            u = torch.rand((cfg.B, cfg.E), generator=g, device="cuda").clamp_(min=1e-30)
            s["bias"], s["bias_ld"] = (-torch.log(-torch.log(u))).float().contiguous(), cfg.E
        elif cfg.routing == "zipf":
            rank = torch.randperm(cfg.E, generator=g, device="cuda").float() + 1
            s["bias"], s["bias_ld"] = (-cfg.zipf_s * torch.log(rank)).contiguous(), 0
        sets.append(s)
    return sets


def run_moe(args, torch, mb, synth):
    cfg = synth.CONFIGS[args.workload]
    esz = 2 if cfg.dtype == "bf16" else 4
    expert_bytes = 3 * cfg.I * cfg.d * esz
    shared_bytes = 3 * cfg.Is * cfg.d * esz
    est = cfg.E * cfg.d * esz + min(cfg.B * cfg.k, cfg.E) * 0.9 * expert_bytes + shared_bytes
    full_set = (cfg.E * cfg.d + 3 * cfg.E * cfg.I * cfg.d + 3 * cfg.Is * cfg.d) * esz
    R = args.rotate or rotations(est, cap_sets=max(2, int(60e9 // full_set)))
    sets = moe_sets(cfg, R, args.seed, torch)
    dt = mb.DT_BF16 if cfg.dtype == "bf16" else mb.DT_F32
    ws = mb.workspace(mb.workspace_bytes(mb.OP_BLOCK, dt, B=cfg.B, d=cfg.d, E=cfg.E, k=cfg.k,
                                         I=cfg.I, Is=cfg.Is))

    def step(i):
        s = sets[i % R]
        mb.moe_block(s["X"], s["Wr"], cfg.k, s["W13"], s["W2"], s["out"], ws, s["Ws13"], s["Ws2"],
                     s["bias"], s["bias_ld"], topk_ids=s["ids"])

    mb.set_block_schedule(args.schedule)
    if args.graph:
        ms = graph_loop(step, R, args, torch, [s["out"] for s in sets])
    else:
        ms = timed_loop(step, args, torch)
    fused = "fused" in mb.last_variant()
    route_in_up = "top-k/plan" in mb.last_variant()
    # algorithmic bytes per set: every selected expert's weights once, the
    # router and shared expert, x (and bias) read once, out written once
    per_set = []
    for s in sets:
        n = int(torch.unique(s["ids"]).numel())
        bias_b = 0 if s["bias"] is None else s["bias"].numel() * 4
        b = cfg.E * cfg.d * esz + n * expert_bytes + shared_bytes + 2 * cfg.B * cfg.d * esz + bias_b
        per_set.append((n, b, launch_bytes(cfg, n, esz, bias_b, route_in_up)))
    avg_bytes = sum(per_set[i % R][1] for i in range(args.steps)) / args.steps
    avg_n = sum(per_set[i % R][0] for i in range(args.steps)) / args.steps
    kern, kbytes = {}, {}
    launches = ((("block", mb.KERNEL_BLOCK),) if fused else
                (("route", mb.KERNEL_ROUTE), ("expert_up", mb.KERNEL_EXPERT_UP),
                 ("expert_down_combine", mb.KERNEL_EXPERT_DOWN)))
    for name, kid in launches:
        kern[name] = kernel_times(step, kid, args, torch, mb)
        # the profiled launches run sets warmup + steps + i (see kernel_times)
        sel = (lambda i: per_set[i][1]) if fused else (lambda i: per_set[i][2][name])
        kbytes[name] = [sel((args.warmup + args.steps + i) % R) for i in range(len(kern[name]))]
    # the dominant kernel: the largest share of the block's time
    dom = max(kern, key=lambda k: sum(kern[k]))
    durs = kern[dom]
    achieved = sum(kbytes[dom]) / (sum(durs) * 1e-3) / 1e9         # GB/s
    roof = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(achieved / HBM_PEAK_GBS, 4),
                traffic=stored_traffic(cfg.name, dom),
                kernel=KERNEL_SYMBOL[dom], bytes_per_launch=round(sum(kbytes[dom]) / len(durs)),
                avg_us=round(sum(durs) / len(durs) * 1e3, 3))
    per_kernel = {k: dict(us=round(sum(v) / len(v) * 1e3, 3),
                          gbs=round(sum(kbytes[k]) / (sum(v) * 1e-3) / 1e9, 1)) for k, v in kern.items()}
    us = ms * 1e3
    gbs = avg_bytes / (us * 1e-6) / 1e9
    config = dict(workload="%s: decode MoE block, one TP weight shard, B=%d, d=%d, E=%d, top-%d, "
                           "I=%d, Is=%d, %s routing" % (cfg.name, cfg.B, cfg.d, cfg.E, cfg.k, cfg.I,
                                                         cfg.Is, cfg.routing),
                  B=cfg.B, d=cfg.d, E=cfg.E, k=cfg.k, I=cfg.I, Is=cfg.Is, rotate=R,
                  distinct_experts=round(avg_n, 2), algorithmic_bytes=round(avg_bytes),
                  gbs=round(gbs, 1), hbm_frac=round(gbs / HBM_PEAK_GBS, 4),
                  kernels=per_kernel,
                  launch="graph replay" if args.graph else "plain launches",
                  variant=mb.last_variant())
    cpu = None if args.no_cpu_baseline else cpu_baseline_moe(cfg, args)
    return us, ms, cfg.dtype, config, roof, cpu


# symbol (as a kernel trace names it) of each launch of the block
KERNEL_SYMBOL = {"route": "skinny_valu_kernel / skinny_mfma_kernel (router mode)", "expert_up": "expert_up_kernel",
                 "expert_down_combine": "expert_down_combine_kernel", "block": "moe_block_kernel"}


def launch_bytes(cfg, n, esz, bias_b, route_in_up):
    """Algorithmic HBM bytes of each launch of the block, for n distinct
    routed experts: the weights it streams (once), the activations it must
    read and the results it must write.  Workspace traffic between launches
    (h and, when the gate/up launch selects, the logits; fp32) is counted as
    the producer's output and the consumer's input; the completion counter
    and the plan are not.  The shared expert's gate/up runs in the gate/up
    launch when that launch also selects (small batch), else in the router
    launch."""
    B, d, E, k, I, Is = cfg.B, cfg.d, cfg.E, cfg.k, cfg.I, cfg.Is
    x = B * d * esz
    shared_up = 2 * Is * d * esz + B * Is * 4 if Is else 0
    route = E * d * esz + x + bias_b
    up = n * 2 * I * d * esz + x + B * k * I * 4
    if route_in_up:
        route += B * E * 4                      # logits out
        up += B * E * 4 + B * k * 8 + shared_up  # logits in, ids + weights out
    else:
        route += B * k * 8 + shared_up
    down = n * d * I * esz + B * k * I * 4 + B * k * 4 + B * d * esz
    if Is:
        down += d * Is * esz + B * Is * 4
    return {"route": route, "expert_up": up, "expert_down_combine": down}


# ---------------------------------------------------------------- dense

def run_dense(args, torch, mb, synth):
    B, N, K = args.batch, synth.DENSE_N, synth.DENSE_K
    wbytes = N * K * 2
    R = args.rotate or rotations(wbytes, cap_sets=64)
    sets = []
    for r in range(R):
        g = torch.Generator(device="cuda").manual_seed(args.seed * 1000003 + r)
        sets.append(dict(X=torch.randn((B, K), generator=g, device="cuda", dtype=torch.bfloat16),
                         W=(torch.randn((N, K), generator=g, device="cuda", dtype=torch.bfloat16) * K ** -0.5).to(torch.bfloat16),
                         Y=torch.empty((B, N), device="cuda", dtype=torch.bfloat16)))
    ws = mb.workspace(mb.workspace_bytes(mb.OP_SKINNY_GEMM, mb.DT_BF16, B=B, N=N, K=K))

    def step(i):
        s = sets[i % R]
        mb.skinny_gemm(s["X"], s["W"], s["Y"], ws)

    ms = timed_loop(step, args, torch)
    nbytes = wbytes + B * K * 2 + B * N * 2
    durs = kernel_times(step, mb.KERNEL_SKINNY, args, torch, mb)
    achieved = nbytes / (sum(durs) / len(durs) * 1e-3) / 1e9
    roof = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(achieved / HBM_PEAK_GBS, 4),
                traffic=stored_traffic("dense_b%d" % B, "skinny_gemm"),
                kernel="skinny_valu_kernel / skinny_mfma_kernel",
                bytes_per_launch=nbytes, avg_us=round(sum(durs) / len(durs) * 1e3, 3))
    us = ms * 1e3
    config = dict(workload="dense skinny GEMM (attention input projection): Y[%d x %d] = "
                           "X[%d x %d] . W[%d x %d]^T, bf16" % (B, N, B, K, N, K),
                  B=B, N=N, K=K, rotate=R, algorithmic_bytes=nbytes,
                  gbs=round(nbytes / (us * 1e-6) / 1e9, 1),
                  hbm_frac=round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                  variant=mb.last_variant())
    cpu = None if args.no_cpu_baseline else cpu_baseline_dense(B, N, K, args)
    return us, ms, "bf16", config, roof, cpu


# ---------------------------------------------------------------- oproj

def run_oproj(args, torch, mb, synth):
    """Attention output projection with the residual added:
    Y = X . W^T + R, X [B][3072], W [7168][3072], R and Y [B][7168], bf16."""
    B, N, K = args.batch, synth.OPROJ_N, synth.OPROJ_K
    wbytes = N * K * 2
    R_sets = args.rotate or rotations(wbytes, cap_sets=64)
    sets = []
    for r in range(R_sets):
        g = torch.Generator(device="cuda").manual_seed(args.seed * 1000003 + r)
        sets.append(dict(X=torch.randn((B, K), generator=g, device="cuda", dtype=torch.bfloat16),
                         W=(torch.randn((N, K), generator=g, device="cuda", dtype=torch.bfloat16) * K ** -0.5).to(torch.bfloat16),
                         R=torch.randn((B, N), generator=g, device="cuda", dtype=torch.bfloat16),
                         Y=torch.empty((B, N), device="cuda", dtype=torch.bfloat16)))
    ws = mb.workspace(mb.workspace_bytes(mb.OP_SKINNY_GEMM, mb.DT_BF16, B=B, N=N, K=K))

    def step(i):
        s = sets[i % R_sets]
        mb.skinny_gemm_residual(s["X"], s["W"], s["R"], s["Y"], ws)

    ms = timed_loop(step, args, torch)
    nbytes = wbytes + B * K * 2 + 2 * B * N * 2
    durs = kernel_times(step, mb.KERNEL_SKINNY, args, torch, mb)
    achieved = nbytes / (sum(durs) / len(durs) * 1e-3) / 1e9
    roof = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(achieved / HBM_PEAK_GBS, 4),
                traffic=stored_traffic("oproj_b%d" % B, "skinny_gemm"),
                kernel="skinny_valu_kernel / skinny_mfma_kernel",
                bytes_per_launch=nbytes, avg_us=round(sum(durs) / len(durs) * 1e3, 3))
    us = ms * 1e3
    config = dict(workload="attention output projection + residual: Y[%d x %d] = X[%d x %d] . W[%d x %d]^T "
                           "+ R, bf16" % (B, N, B, K, N, K),
                  B=B, N=N, K=K, rotate=R_sets, algorithmic_bytes=nbytes,
                  gbs=round(nbytes / (us * 1e-6) / 1e9, 1),
                  hbm_frac=round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                  variant=mb.last_variant())
    cpu = None if args.no_cpu_baseline else cpu_baseline_oproj(B, args)
    return us, ms, "bf16", config, roof, cpu


# ---------------------------------------------------------------- copy

def run_copy(args, torch):
    """A plain device copy of known size (256 MiB), as the yardstick for the
    HBM byte counters (FETCH_SIZE / WRITE_SIZE) and for achievable
    bandwidth on this GPU: 2 x 256 MiB of compulsory traffic per copy."""
    n = 256 << 20
    R = 4
    src = [torch.empty(n, dtype=torch.uint8, device="cuda").fill_(r) for r in range(R)]
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")

    def step(i):
        dst.copy_(src[i % R])

    ms = timed_loop(step, args, torch)
    us = ms * 1e3
    gbs = 2 * n / (us * 1e-6) / 1e9
    config = dict(workload="device copy of 256 MiB (read + write)", bytes=2 * n, rotate=R,
                  gbs=round(gbs, 1), hbm_frac=round(gbs / HBM_PEAK_GBS, 4))
    roof = dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(gbs / HBM_PEAK_GBS, 4), traffic=None, kernel="copy")
    return us, ms, "u8", config, roof, None


# ---------------------------------------------------------------- traffic

def stored_traffic(workload, launch):
    """HBM bytes per launch of `launch` (route, expert_up, ...) measured by rocprofv3 counters
    (FETCH_SIZE + WRITE_SIZE, each scaled by what it reads for a 256 MiB copy)
    and stored in profiles/traffic.json, or None when the library sources have
    changed since the counters were taken."""
    from moe_block_skinny_amd import build as hip_build
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_digest") != hip_build.source_digest():
        return None
    k = t.get("workloads", {}).get(workload, {}).get(launch)
    return None if k is None else k.get("bytes_per_launch")


# ---------------------------------------------------------------- timing

def timed_loop(step, args, torch):
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        step(args.warmup + i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / args.steps


def graph_loop(step, R, args, torch, outs):
    """Per-step time of graph replays: one graph per weight set, each holding
    one step captured on a side stream.  Before timing, every graph is
    replayed three times with plain launches of the other sets in between,
    and each replay must reproduce the plain launch's output bits."""
    for i in range(max(args.warmup, R)):
        step(i)
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    graphs = []
    side = torch.cuda.Stream()
    for r in range(R):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            step(r)
        graphs.append(g)
    torch.cuda.synchronize()
    for rep in range(3):
        for r in range(R):
            outs[r].fill_(0)
            graphs[r].replay()
            step(r + 1)               # plain launches between the replays
            torch.cuda.synchronize()
            if not torch.equal(outs[r].view(torch.int16), ref[r].view(torch.int16)):
                raise RuntimeError("graph replay %d of set %d differs from the plain launch" % (rep, r))
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        graphs[i % R].replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / args.steps


def kernel_times(step, kernel_id, args, torch, mb):
    """Duration (ms) of each launch of one kernel over kernel-steps steps,
    from HIP events the library records around that launch on its stream."""
    n = max(1, args.kernel_steps)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in evs:
        a.record()
        b.record()
    torch.cuda.synchronize()
    try:
        for i in range(n):
            mb.profile_events(kernel_id, evs[i][0], evs[i][1])
            step(args.warmup + args.steps + i)
    finally:
        mb.profile_events(kernel_id)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


# ---------------------------------------------------------------- CPU oracle

def cpu_baseline_moe(cfg, args):
    import numpy as np
    from moe_block_skinny_amd import synth
    from oracle import oracle as orc

    X, Wr = synth.x(cfg, args.seed), synth.router_w(cfg, args.seed)
    bias, ld = synth.bias(cfg, args.seed)
    _, ids, _, _ = orc.route(X, Wr, cfg.k, bias, ld)
    touched = set(ids.reshape(-1).tolist())
    W13 = [synth.expert_w13(cfg, args.seed, e) if e in touched else None for e in range(cfg.E)]
    W2 = [synth.expert_w2(cfg, args.seed, e) if e in touched else None for e in range(cfg.E)]
    Ws13, Ws2 = synth.shared_w13(cfg, args.seed), synth.shared_w2(cfg, args.seed)
    n, t0 = 0, time.perf_counter()
    while True:
        orc.moe_block(X, Wr, cfg.k, W13, W2, Ws13, Ws2, bias, ld)
        n += 1
        el = time.perf_counter() - t0
        if el >= args.cpu_seconds:
            break
    return dict(value=round(el / n * 1e6, 1), unit="µs", cores=1, kind="oracle",
                sample="%d blocks of the %s workload (seed %d, %d distinct experts), fp64 C oracle, "
                       "one thread, %.1f s" % (n, cfg.name, args.seed, len(touched), el),
                cpu=platform.processor() or platform.machine(), host_cpus=os.cpu_count())


def cpu_baseline_dense(B, N, K, args):
    from moe_block_skinny_amd import synth
    from oracle import oracle as orc

    X, W = synth.dense_x(B), synth.dense_w()
    n, t0 = 0, time.perf_counter()
    while True:
        orc.skinny_gemm(X, W)
        n += 1
        el = time.perf_counter() - t0
        if el >= args.cpu_seconds:
            break
    return dict(value=round(el / n * 1e6, 1), unit="µs", cores=1, kind="oracle",
                sample="%d skinny GEMMs at B=%d, fp64 C oracle, one thread, %.1f s" % (n, B, el),
                host_cpus=os.cpu_count())


def cpu_baseline_oproj(B, args):
    from moe_block_skinny_amd import synth
    from oracle import oracle as orc

    X, W, R = synth.oproj_x(B), synth.oproj_w(), synth.oproj_r(B)
    n, t0 = 0, time.perf_counter()
    while True:
        orc.skinny_gemm_residual(X, W, R)
        n += 1
        el = time.perf_counter() - t0
        if el >= args.cpu_seconds:
            break
    return dict(value=round(el / n * 1e6, 1), unit="µs", cores=1, kind="oracle",
                sample="%d output projections with residual at B=%d, fp64 C oracle, one thread, %.1f s"
                       % (n, B, el), host_cpus=os.cpu_count())


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: the decode MoE block here is one GPU's "
              "tensor-parallel weight shard and this build has no multi-GPU path "
              "(--gpus %d, WORLD_SIZE %d requested)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)
    import torch

    from moe_block_skinny_amd import binding as mb
    from moe_block_skinny_amd import synth

    torch.cuda.set_device(0)
    if args.workload == "copy":
        us, ms, dtype, config, roof, cpu = run_copy(args, torch)
    elif args.workload == "dense":
        us, ms, dtype, config, roof, cpu = run_dense(args, torch, mb, synth)
    elif args.workload == "oproj":
        us, ms, dtype, config, roof, cpu = run_oproj(args, torch, mb, synth)
    else:
        us, ms, dtype, config, roof, cpu = run_moe(args, torch, mb, synth)
    line = dict(metric=METRIC, value=round(us, 3), unit="µs", n_gpus=1, steps=args.steps,
                warmup=args.warmup, ms_per_step=round(ms, 6), higher_is_better=False,
                scaling="weak", vs_baseline=None, dtype=dtype, data="synthetic", config=config,
                roofline=roof, cpu_baseline=cpu)
    print(json.dumps(line, ensure_ascii=False), flush=True)


if __name__ == "__main__":
    main()
