#!/usr/bin/env python3
"""µs per decode MoE block and achieved HBM GB/s on one MI355X, batch 1-64.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--trials T]
                    [--workload sweep|tp8_b64|tp16_b1|tp16_b8|tiny|dense|oproj|stream|copy]

A step is one pass of the whole decode MoE block (router scoring, top-k and
plan, routed and shared expert gate/up + SwiGLU + down, weighted combine)
over one batch of synthetic bf16 input, through the C ABI (moe_block).

Default (--workload sweep): the metric's batch range in one run.  The
headline `value` is the largest single-GPU workload, one TP8 weight shard at
batch 64 (d=7168, E=384, top-8, I=Is=256, Zipf(1.1) routing); config.sweep
holds the TP16 shard at batch 1 and at batch 8 (Gumbel routing), the dense
attention input projection at B = 1, 8, 64, and config.stream the read-only
128-bit streaming yardstick these are compared with.

Timing of every entry, on one stream:
  * every rotation set is run once, untimed, whatever --warmup is (weights
    and page tables of every set touched before timing);
  * W warm-up steps;
  * T trials (default 7), each exactly K steps between two HIP events with
    the device synchronised before and after; sets 0, 1, ... in turn, so
    every trial runs the same sets.  value = median µs per step over the
    trials; p10 / p90 alongside.
Weights are random (seeded torch generator on the GPU) in R rotating full
sets so that the bytes touched between two uses of a set exceed twice the
256 MB Infinity Cache plus L2: each timed step reads HBM, not cache.

Also on the line:
  roofline:     the headline's dominant kernel (the launch with the largest
                share of the block's time) timed with HIP events its own
                dispatch records, on the launch stream; algorithmic bytes /
                duration against the 8 TB/s HBM peak; traffic = counter-
                measured HBM bytes per launch (profiles/traffic.json) while
                the kernels are unchanged since the counters were taken;
  cpu_baseline: the CPU oracle timed on this host on a bounded sample of the
                headline workload, single-threaded and on all cores
                (OpenMP over tokens), with the CPU model and affinity mask.

--timeline (with tp16_b1, tp16_b8 or tp8_b64): instead of timing, run the
instrumented library (libmoe_skinny_stamps.so, built by build()) and print
one JSON line with the per-workgroup clock stamps of --trials single blocks
(each launched alone after every weight set was run once): per launch and
stamp point the min / p10 / median / p90 / max in µs from the block's first
workgroup start, and for the gate/up launch the end times by CU slot (the
grid's first, second, ... 256 workgroups), by XCD and per CU (its last
workgroup), and whether workgroups g and g + 256 ran on the same CU.
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
HEADLINE = "tp8_b64"
SWEEP_MOE = ("tp16_b1", "tp16_b8")
SWEEP_DENSE = (1, 8, 64)
# rotating weight sets per workload: bytes touched between two uses of a set
# above 2 x (Infinity Cache + L2)
ROTATE = {"tiny": 128, "tp16_b1": 16, "tp16_b8": 4, "tp8_b64": 4, "dense": 16, "oproj": 16}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="timed steps per trial")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--trials", type=int, default=7)
    ap.add_argument("--workload", default="sweep",
                    choices=["sweep", "tiny", "tp16_b1", "tp16_b8", "tp8_b64", "dense", "oproj", "latent", "stream",
                             "copy"])
    ap.add_argument("--batch", type=int, default=1, help="dense / oproj workload batch")
    ap.add_argument("--rotate", type=int, default=0, help="weight sets (0: the workload's default)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--kernel-steps", type=int, default=40)
    ap.add_argument("--cpu-seconds", type=float, default=8.0, help="per CPU timing (single thread, all cores)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--schedule", default="auto", choices=["auto", "launches", "fused", "router_in_up"],
                    help="moe_block schedule: one fused launch where it applies, three launches, or "
                         "(B <= 2) two with the router rows in the gate/up launch")
    ap.add_argument("--timeline", action="store_true",
                    help="per-workgroup clock stamps of single blocks (instrumented library)")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of HIP graphs (one captured block per weight set) instead of plain "
                         "launches; every replay is first checked against the plain launch's bits")
    return ap.parse_args()


def rotations(name: str, bytes_per_step: float, args) -> int:
    if args.rotate:
        return args.rotate
    need = int(2 * MALL_L2_BYTES // max(bytes_per_step, 1.0)) + 1
    return max(2, ROTATE.get(name, 2), need)


def pct(v, q):
    import numpy as np
    return float(np.percentile(np.asarray(v, dtype=np.float64), q))


def trial_stats(ms_list):
    us = [m * 1e3 for m in ms_list]
    return dict(n=len(us), median_us=round(pct(us, 50), 3), p10_us=round(pct(us, 10), 3),
                p90_us=round(pct(us, 90), 3), min_us=round(min(us), 3), max_us=round(max(us), 3))


# ---------------------------------------------------------------- timing

_CYCLES_PER_US = None


def hold_stream(torch, us):
    """Keep the current stream busy for about `us` microseconds with a spin
    kernel (torch.cuda._sleep), so that the host can queue a whole trial
    behind it: the timed steps then run back to back on the GPU instead of
    at the rate the Python caller issues them.  The spin rate is measured
    once with events."""
    global _CYCLES_PER_US
    if _CYCLES_PER_US is None:
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        torch.cuda._sleep(2_000_000)
        e1.record()
        torch.cuda.synchronize()
        _CYCLES_PER_US = 2_000_000 / max(e0.elapsed_time(e1) * 1e3, 1.0)
    torch.cuda._sleep(int(us * _CYCLES_PER_US))


def timed_trials(step, R, args, torch, info=None):
    """Every set once (untimed), W warm-up steps, then T trials of exactly K
    steps (sets 0 .. K-1 mod R) between two events.  Each trial is queued
    behind a spin kernel long enough for the host to issue all K steps
    first (twice the host's measured issue time, at least 300 us), so the
    trial measures the GPU running the steps back to back; `info` receives
    the host's issue time per step and whether every trial was fully queued
    before its first step ran.  Returns ms per step of each trial."""
    t0 = time.perf_counter()
    for r in range(R):
        step(r)
    host_us = (time.perf_counter() - t0) * 1e6 / R
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    out, queued = [], True
    hold_us = max(300.0, 2.0 * host_us * args.steps)
    for _ in range(args.trials):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        hold_stream(torch, hold_us)
        t0 = time.perf_counter()
        e0.record()
        for i in range(args.steps):
            step(i)
        e1.record()
        issued = (time.perf_counter() - t0) * 1e6
        queued = queued and issued < hold_us
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / args.steps)
    if info is not None:
        info.update(host_issue_us_per_step=round(host_us, 2), hold_us=round(hold_us, 1), queued_ahead=queued)
    return out
def graph_trials(step, R, args, torch, outs):
    """Trials of graph replays: one graph per weight set, each holding one
    step captured on a side stream.  Before timing, every graph is replayed
    three times with plain launches of the other sets in between, and each
    replay must reproduce the plain launch's output bits."""
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
    res = []
    for _ in range(args.trials):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        hold_stream(torch, max(300.0, 40.0 * args.steps))
        e0.record()
        for i in range(args.steps):
            graphs[i % R].replay()
        e1.record()
        torch.cuda.synchronize()
        res.append(e0.elapsed_time(e1) / args.steps)
    return res


def kernel_times(step, kernel_id, n, torch, mb):
    """Duration (ms) of each launch of one kernel over n steps (sets 0 ..
    n-1 mod R), from HIP events the library's dispatch of that kernel
    records on its stream."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in evs:
        a.record()
        b.record()
    torch.cuda.synchronize()
    try:
        for i in range(n):
            mb.profile_events(kernel_id, evs[i][0], evs[i][1])
            step(i)
    finally:
        mb.profile_events(kernel_id)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def stored_traffic(workload, launch):
    """HBM bytes per launch of `launch` measured by rocprofv3 counters
    (FETCH_SIZE and WRITE_SIZE, each scaled by what it reads for a 256 MiB
    copy) and stored in profiles/traffic.json, or None when the library
    sources have changed since the counters were taken."""
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


# symbol (as a kernel trace names it) of each launch of the block
KERNEL_SYMBOL = {"route": "skinny_valu_kernel / skinny_mfma_kernel + route_finish_kernel (router mode)",
                 "expert_up": "expert_up_kernel", "expert_down_combine": "expert_down_combine_kernel",
                 "block": "moe_block_kernel"}


def launch_bytes(cfg, n, esz, bias_b, route_in_up, rows_in_up=False):
    """Algorithmic HBM bytes of each launch of the block, for n distinct
    routed experts: the weights it streams (once), the activations it must
    read and the results it must write.  Workspace traffic between launches
    (h and, when the gate/up launch selects, the logits; fp32) is counted as
    the producer's output and the consumer's input; the completion counter
    and the plan are not.  The shared expert's gate/up runs in the gate/up
    launch when that launch also selects (small batch), else in the router
    launch (vector shape) or as an entry of the gate/up launch (matrix).
    With the router rows inside the gate/up launch (rows_in_up: two
    launches) that launch also streams the router weights and its logits
    never leave it."""
    B, d, E, k, I, Is = cfg.B, cfg.d, cfg.E, cfg.k, cfg.I, cfg.Is
    x = B * d * esz
    shared_up = 2 * Is * d * esz + B * Is * 4 if Is else 0
    route = E * d * esz + x + bias_b
    up = n * 2 * I * d * esz + x + B * k * I * 4
    if route_in_up:
        route += B * E * 4                      # logits out
        up += B * E * 4 + B * k * 8 + shared_up  # logits in, ids + weights out
    elif B <= 8:
        route += B * k * 8 + shared_up
    else:
        route += B * k * 8
        up += shared_up
    down = n * d * I * esz + B * k * I * 4 + B * k * 4 + B * d * esz
    if Is:
        down += d * Is * esz + B * Is * 4
    if rows_in_up:
        up += E * d * esz + bias_b - B * E * 4   # router weights in, no logits read back
        return {"expert_up": up, "expert_down_combine": down}
    return {"route": route, "expert_up": up, "expert_down_combine": down}


def run_moe(name, args, torch, mb, synth, with_roofline):
    cfg = synth.CONFIGS[name]
    esz = 2 if cfg.dtype == "bf16" else 4
    expert_bytes = 3 * cfg.I * cfg.d * esz
    shared_bytes = 3 * cfg.Is * cfg.d * esz
    est = cfg.E * cfg.d * esz + min(cfg.B * cfg.k, cfg.E) * 0.9 * expert_bytes + shared_bytes
    R = rotations(name, est, args)
    sets = moe_sets(cfg, R, args.seed, torch)
    dt = mb.DT_BF16 if cfg.dtype == "bf16" else mb.DT_F32
    ws = mb.workspace(mb.workspace_bytes(mb.OP_BLOCK, dt, B=cfg.B, d=cfg.d, E=cfg.E, k=cfg.k,
                                         I=cfg.I, Is=cfg.Is))

    def step(i):
        s = sets[i % R]
        mb.moe_block(s["X"], s["Wr"], cfg.k, s["W13"], s["W2"], s["out"], ws, s["Ws13"], s["Ws2"],
                     s["bias"], s["bias_ld"], topk_ids=s["ids"])

    mb.set_block_schedule(args.schedule)
    info = {}
    if args.graph:
        ms = graph_trials(step, R, args, torch, [s["out"] for s in sets])
    else:
        ms = timed_trials(step, R, args, torch, info)
    variant = mb.last_variant()
    fused = "fused" in variant
    route_in_up = "top-k/plan" in variant
    rows_in_up = "rows in the gate/up launch" in variant
    # algorithmic bytes per set: every selected expert's weights once, the
    # router and shared expert, x (and bias) read once, out written once
    per_set = []
    for s in sets:
        n = int(torch.unique(s["ids"]).numel())
        bias_b = 0 if s["bias"] is None else s["bias"].numel() * 4
        b = cfg.E * cfg.d * esz + n * expert_bytes + shared_bytes + 2 * cfg.B * cfg.d * esz + bias_b
        per_set.append((n, b, launch_bytes(cfg, n, esz, bias_b, route_in_up, rows_in_up)))
    avg_bytes = sum(per_set[i % R][1] for i in range(args.steps)) / args.steps
    avg_n = sum(per_set[i % R][0] for i in range(args.steps)) / args.steps
    kern, kbytes = {}, {}
    launches = ((("block", mb.KERNEL_BLOCK),) if fused else
                ((("expert_up", mb.KERNEL_EXPERT_UP),) if rows_in_up else
                 (("route", mb.KERNEL_ROUTE), ("expert_up", mb.KERNEL_EXPERT_UP))) +
                (("expert_down_combine", mb.KERNEL_EXPERT_DOWN),))
    nk = max(1, args.kernel_steps)
    for lname, kid in launches:
        kern[lname] = kernel_times(step, kid, nk, torch, mb)
        sel = (lambda i: per_set[i][1]) if fused else (lambda i, l=lname: per_set[i][2][l])
        kbytes[lname] = [sel(i % R) for i in range(nk)]
    per_kernel = {k: dict(us=round(sum(v) / len(v) * 1e3, 3),
                          gbs=round(sum(kbytes[k]) / (sum(v) * 1e-3) / 1e9, 1),
                          frac=round(sum(kbytes[k]) / (sum(v) * 1e-3) / 1e9 / HBM_PEAK_GBS, 4))
                  for k, v in kern.items()}
    st = trial_stats(ms)
    us = st["median_us"]
    gbs = avg_bytes / (us * 1e-6) / 1e9
    entry = dict(workload="%s: decode MoE block, one TP weight shard, B=%d, d=%d, E=%d, top-%d, "
                          "I=%d, Is=%d, %s routing" % (cfg.name, cfg.B, cfg.d, cfg.E, cfg.k, cfg.I,
                                                        cfg.Is, cfg.routing),
                 B=cfg.B, d=cfg.d, E=cfg.E, k=cfg.k, I=cfg.I, Is=cfg.Is, rotate=R,
                 us=us, trials=dict(st, **info),
                 distinct_experts=round(avg_n, 2), algorithmic_bytes=round(avg_bytes),
                 gbs=round(gbs, 1), hbm_frac=round(gbs / HBM_PEAK_GBS, 4),
                 kernels=per_kernel,
                 launch="graph replay" if args.graph else "plain launches",
                 variant=variant)
    if cfg.B * cfg.k <= 64 and cfg.Is and cfg.dtype == "bf16" and args.schedule == "auto" and not args.graph:
        entry["shared_placements"] = shared_placements(cfg, sets, R, ws, args, torch, mb)
    roof = None
    if with_roofline:
        dom = max(kern, key=lambda k: sum(kern[k]))
        durs = kern[dom]
        achieved = sum(kbytes[dom]) / (sum(durs) * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4),
                    traffic=stored_traffic(cfg.name, dom),
                    kernel=KERNEL_SYMBOL[dom], launch=dom, bytes_per_launch=round(sum(kbytes[dom]) / len(durs)),
                    avg_us=round(sum(durs) / len(durs) * 1e3, 3), launches_timed=len(durs))
    del sets, ws
    torch.cuda.empty_cache()
    return entry, roof, cfg


def shared_placements(cfg, sets, R, ws, args, torch, mb):
    """Block µs with the shared expert's gate/up in the gate/up launch, in the
    router launch (one pass over x), and the whole shared expert on a second
    stream (moe_block_streams), each timed like the headline."""
    side = torch.cuda.Stream()
    fork, join = torch.cuda.Event(), torch.cuda.Event()

    def block(i):
        s = sets[i % R]
        mb.moe_block(s["X"], s["Wr"], cfg.k, s["W13"], s["W2"], s["out"], ws, s["Ws13"], s["Ws2"],
                     s["bias"], s["bias_ld"], topk_ids=s["ids"])

    def streams(i):
        s = sets[i % R]
        mb.moe_block_streams(s["X"], s["Wr"], cfg.k, s["W13"], s["W2"], s["out"], ws, side, fork, join,
                             s["Ws13"], s["Ws2"], s["bias"], s["bias_ld"], topk_ids=s["ids"])

    # the next block's routing-independent weights (router, shared expert)
    # read into the cache by a small kernel on a second stream while this
    # block runs (moe_prefetch); ordered after the block's start by an event
    sink = torch.empty(32, dtype=torch.int32, device="cuda")
    starts = [torch.cuda.Event() for _ in range(4)]

    def prefetched(i):
        ev = starts[i % 4]
        ev.record()
        side.wait_event(ev)
        n = sets[(i + 1) % R]
        mb.prefetch([n["Wr"], n["Ws13"], n["Ws2"]], sink, stream=side)
        block(i)

    out = {}
    for label, place, step in (("gate_up_launch", "up", block), ("router_launch", "router", block),
                               ("side_stream", "up", streams), ("gate_up_launch_next_prefetched", "up", prefetched)):
        prev = mb.set_shared_schedule(place)
        try:
            info = {}
            st = trial_stats(timed_trials(step, R, args, torch, info))
        finally:
            mb.set_shared_schedule(prev)
        out[label] = dict(us=st["median_us"], p10_us=st["p10_us"], p90_us=st["p90_us"],
                          queued_ahead=info.get("queued_ahead"))
    torch.cuda.synchronize()
    return out


# ---------------------------------------------------------------- dense

def run_gemm(kind, B, args, torch, mb, synth, with_roofline):
    """The attention input projection (kind "dense": Y = X . W^T, X [B][7168],
    W [3072][7168]) or the output projection with the residual added (kind
    "oproj": Y = X . W^T + R, X [B][3072], W [7168][3072], R [B][7168]), bf16."""
    if kind == "dense":
        N, K = synth.DENSE_N, synth.DENSE_K
    else:
        N, K = synth.OPROJ_N, synth.OPROJ_K
    wbytes = N * K * 2
    R = rotations(kind, wbytes, args)
    sets = []
    for r in range(R):
        g = torch.Generator(device="cuda").manual_seed(args.seed * 1000003 + r)
        s = dict(X=torch.randn((B, K), generator=g, device="cuda", dtype=torch.bfloat16),
                 W=(torch.randn((N, K), generator=g, device="cuda", dtype=torch.bfloat16) * K ** -0.5).to(torch.bfloat16),
                 Y=torch.empty((B, N), device="cuda", dtype=torch.bfloat16))
        if kind == "oproj":
            s["R"] = torch.randn((B, N), generator=g, device="cuda", dtype=torch.bfloat16)
        sets.append(s)
    ws = mb.workspace(mb.workspace_bytes(mb.OP_SKINNY_GEMM, mb.DT_BF16, B=B, N=N, K=K))

    def step(i):
        s = sets[i % R]
        if kind == "dense":
            mb.skinny_gemm(s["X"], s["W"], s["Y"], ws)
        else:
            mb.skinny_gemm_residual(s["X"], s["W"], s["R"], s["Y"], ws)

    info = {}
    ms = timed_trials(step, R, args, torch, info)
    variant = mb.last_variant()
    nbytes = wbytes + B * K * 2 + B * N * 2 * (2 if kind == "oproj" else 1)
    durs = kernel_times(step, mb.KERNEL_SKINNY, max(1, args.kernel_steps), torch, mb)
    kus = sum(durs) / len(durs) * 1e3
    st = trial_stats(ms)
    us = st["median_us"]
    what = ("dense skinny GEMM (attention input projection): Y[%d x %d] = X[%d x %d] . W[%d x %d]^T, bf16"
            if kind == "dense" else
            "attention output projection + residual: Y[%d x %d] = X[%d x %d] . W[%d x %d]^T + R, bf16")
    entry = dict(workload=what % (B, N, B, K, N, K), B=B, N=N, K=K, rotate=R, us=us, trials=dict(st, **info),
                 algorithmic_bytes=nbytes, gbs=round(nbytes / (us * 1e-6) / 1e9, 1),
                 hbm_frac=round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                 kernel_us=round(kus, 3), kernel_gbs=round(nbytes / (kus * 1e-6) / 1e9, 1),
                 variant=variant)
    roof = None
    if with_roofline:
        achieved = nbytes / (kus * 1e-6) / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4),
                    traffic=stored_traffic("%s_b%d" % (kind, B), "skinny_gemm"),
                    kernel="skinny_valu_kernel / skinny_rows_kernel / skinny_mfma_kernel", launch="skinny_gemm",
                    bytes_per_launch=nbytes, avg_us=round(kus, 3), launches_timed=len(durs))
    del sets, ws
    torch.cuda.empty_cache()
    return entry, roof


# ---------------------------------------------------------------- latent

def run_route_latent(B, args, torch, mb, synth):
    """The router with the latent input projection in one product over x
    (moe_route_latent, L = 1024 latent rows) against the same work as two
    launches (moe_route, then skinny_gemm for the latent rows): d = 7168,
    E = 384, top-8, bf16, plain routing."""
    cfg = synth.CONFIGS["tp16_b1"]
    d, E, k, L = cfg.d, cfg.E, cfg.k, synth.LATENT_L
    wbytes = (E + L) * d * 2
    R = rotations("dense", wbytes, args)
    sets = []
    for r in range(R):
        g = torch.Generator(device="cuda").manual_seed(args.seed * 1000003 + 500 + r)
        sets.append(dict(X=torch.randn((B, d), generator=g, device="cuda", dtype=torch.bfloat16),
                         Wr=(torch.randn((E, d), generator=g, device="cuda") * d ** -0.5).to(torch.bfloat16),
                         Wl=(torch.randn((L, d), generator=g, device="cuda") * d ** -0.5).to(torch.bfloat16),
                         ids=torch.empty((B, k), dtype=torch.int32, device="cuda"),
                         w=torch.empty((B, k), device="cuda"),
                         plan=torch.empty((mb.plan_words(B, k, E),), dtype=torch.int32, device="cuda"),
                         lat=torch.empty((B, L), dtype=torch.bfloat16, device="cuda")))
    ws = mb.workspace(max(mb.workspace_bytes(mb.OP_ROUTE_LATENT, mb.DT_BF16, B=B, d=d, E=E, k=k, N=L),
                          mb.workspace_bytes(mb.OP_SKINNY_GEMM, mb.DT_BF16, B=B, N=L, K=d)))

    def merged(i):
        s = sets[i % R]
        mb.moe_route_latent(s["X"], s["Wr"], s["Wl"], k, s["ids"], s["w"], s["plan"], s["lat"], ws)

    def separate(i):
        s = sets[i % R]
        mb.moe_route(s["X"], s["Wr"], k, s["ids"], s["w"], s["plan"], ws)
        mb.skinny_gemm(s["X"], s["Wl"], s["lat"], ws)

    out = {}
    for label, step in (("merged", merged), ("separate", separate)):
        info = {}
        st = dict(trial_stats(timed_trials(step, R, args, torch, info)), **info)
        nbytes = wbytes + B * d * 2 + B * L * 2
        out[label] = dict(us=st["median_us"], trials=st, gbs=round(nbytes / (st["median_us"] * 1e-6) / 1e9, 1),
                          variant=mb.last_variant())
    out.update(B=B, d=d, E=E, L=L, rotate=R, algorithmic_bytes=wbytes + B * d * 2 + B * L * 2,
               workload="router + latent input projection (L=%d) over x [%d x %d], bf16" % (L, B, d))
    del sets, ws
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------- yardsticks

def run_stream(args, torch, mb):
    """The read-only streaming yardstick (moe_stream_read: 128-bit
    nontemporal loads, one contiguous 1 KB per wave instruction): 4 rotating
    1 GiB buffers (the rate away from launch overheads), and 16 rotating
    44 MB buffers (the dense product's weight size: the rate one launch of
    that size reaches, its fixed launch latency included).  Best grid of a
    few; the XOR of the sink is checked against the buffer's."""
    out = {}
    for label, nbytes, R in (("1gib", 1 << 30, 4), ("44mb", 3072 * 7168 * 2, 16)):
        bufs = []
        for r in range(R):
            g = torch.Generator(device="cuda").manual_seed(77 + r)
            bufs.append(torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), generator=g, device="cuda",
                                      dtype=torch.int32))
        best = None
        for wg in (512, 1024, 2048):
            sink = torch.empty(wg, dtype=torch.int32, device="cuda")

            def step(i, sink=sink):
                mb.stream_read(bufs[i % R], sink)

            info = {}
            ms = timed_trials(step, R, args, torch, info)
            st = dict(trial_stats(ms), **info)
            gbs = nbytes / (st["median_us"] * 1e-6) / 1e9
            if best is None or gbs > best["gbs"]:
                best = dict(bytes=nbytes, rotate=R, workgroups=wg, us=st["median_us"], trials=st,
                            gbs=round(gbs, 1), hbm_frac=round(gbs / HBM_PEAK_GBS, 4))
        # every word read: XOR of the sink == XOR of the buffer
        sink = torch.empty(best["workgroups"], dtype=torch.int32, device="cuda")
        mb.stream_read(bufs[0], sink)
        best["checked"] = _xor_all(sink, torch) == _xor_all(bufs[0], torch)
        out[label] = best
        del bufs
        torch.cuda.empty_cache()
    return out


def _xor_all(t, torch):
    """XOR of every element of an int32 tensor: pairwise halving, exact."""
    t = t.reshape(-1)
    while t.numel() > 1:
        if t.numel() % 2:
            t = torch.cat([t, torch.zeros(1, dtype=t.dtype, device=t.device)])
        t = torch.bitwise_xor(t[0::2], t[1::2])
    return int(t[0].item())


def run_copy(args, torch):
    """A plain device copy of known size (256 MiB), the yardstick for the HBM
    byte counters (FETCH_SIZE / WRITE_SIZE): 2 x 256 MiB of traffic per copy."""
    n = 256 << 20
    R = 4
    src = [torch.empty(n, dtype=torch.uint8, device="cuda").fill_(r) for r in range(R)]
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")

    def step(i):
        dst.copy_(src[i % R])

    ms = timed_trials(step, R, args, torch)
    st = trial_stats(ms)
    gbs = 2 * n / (st["median_us"] * 1e-6) / 1e9
    return dict(workload="device copy of 256 MiB (read + write)", bytes=2 * n, rotate=R, us=st["median_us"],
                trials=st, gbs=round(gbs, 1), hbm_frac=round(gbs / HBM_PEAK_GBS, 4))


# ---------------------------------------------------------------- CPU oracle

def cpu_info():
    model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        aff = sorted(os.sched_getaffinity(0))
    except AttributeError:
        aff = list(range(os.cpu_count() or 1))
    return model, aff


def _ranges(cpus):
    out, i = [], 0
    while i < len(cpus):
        j = i
        while j + 1 < len(cpus) and cpus[j + 1] == cpus[j] + 1:
            j += 1
        out.append(str(cpus[i]) if i == j else "%d-%d" % (cpus[i], cpus[j]))
        i = j + 1
    return ",".join(out)


def cpu_baseline(cfg, args):
    """The oracle as it stands on the host: whole blocks of the headline
    workload (seed 0, only the selected experts' weights drawn), repeated
    until --cpu-seconds have passed, once with the plain single-thread build
    and once with the OpenMP build (tokens on every core it may use)."""
    from moe_block_skinny_amd import synth
    from oracle import oracle as orc

    X, Wr = synth.x(cfg, args.seed), synth.router_w(cfg, args.seed)
    bias, ld = synth.bias(cfg, args.seed)
    _, ids, _, _ = orc.route(X, Wr, cfg.k, bias, ld)
    touched = set(ids.reshape(-1).tolist())
    W13 = [synth.expert_w13(cfg, args.seed, e) if e in touched else None for e in range(cfg.E)]
    W2 = [synth.expert_w2(cfg, args.seed, e) if e in touched else None for e in range(cfg.E)]
    Ws13, Ws2 = synth.shared_w13(cfg, args.seed), synth.shared_w2(cfg, args.seed)
    res = {}
    for par in (False, True):
        n, t0 = 0, time.perf_counter()
        while True:
            orc.moe_block(X, Wr, cfg.k, W13, W2, Ws13, Ws2, bias, ld, parallel=par)
            n += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds:
                break
        res[par] = (el / n * 1e6, n, el, orc.threads(par))
    model, aff = cpu_info()
    (us1, n1, el1, _), (usp, npar, elp, thr) = res[False], res[True]
    return dict(value=round(usp, 1), unit="µs", cores=thr, kind="oracle",
                sample="%d blocks of the %s workload (seed %d, B=%d, %d distinct experts) on %d threads "
                       "(OpenMP over tokens) in %.1f s; single-thread: %d blocks in %.1f s; fp64 C oracle"
                       % (npar, cfg.name, args.seed, cfg.B, len(touched), thr, elp, n1, el1),
                single_thread_us=round(us1, 1), all_cores_us=round(usp, 1), threads=thr,
                cpu_model=model, affinity=_ranges(aff), affinity_cpus=len(aff), host_cpus=os.cpu_count())


def cpu_baseline_gemm(kind, B, args):
    from moe_block_skinny_amd import synth
    from oracle import oracle as orc

    if kind == "dense":
        X, W = synth.dense_x(B), synth.dense_w()
        f = lambda: orc.skinny_gemm(X, W)
    else:
        X, W, R = synth.oproj_x(B), synth.oproj_w(), synth.oproj_r(B)
        f = lambda: orc.skinny_gemm_residual(X, W, R)
    n, t0 = 0, time.perf_counter()
    while True:
        f()
        n += 1
        el = time.perf_counter() - t0
        if el >= args.cpu_seconds:
            break
    model, aff = cpu_info()
    return dict(value=round(el / n * 1e6, 1), unit="µs", cores=1, kind="oracle",
                sample="%d %s products at B=%d, fp64 C oracle, one thread, %.1f s" % (n, kind, B, el),
                cpu_model=model, affinity=_ranges(aff), host_cpus=os.cpu_count())


# ---------------------------------------------------------------- timeline

# stamp points of each instrumented launch (slot -> name); the gate/up's
# meaning depends on its shape (vector: routing inside; matrix: plan from ids)
TIMELINE_POINTS = {
    "route": {0: "start", 1: "product done"},
    "route_finish": {0: "start", 1: "selected"},
    "expert_up": {0: "start", 1: "router rows scored / shared tiles done (vector); plan built (matrix)",
                  2: "plan ready (vector); tasks listed (matrix)", 3: "first routed task done", 4: "end"},
    "expert_down_combine": {0: "start", 1: "staged", 2: "products done", 3: "end"},
}


def run_timeline(name, args, torch, mb, synth):
    """Per-workgroup clock stamps of `args.trials` single blocks (see the
    module docstring).  The stamps are the 100 MHz constant clock."""
    import ctypes

    import numpy as np

    from moe_block_skinny_amd import build as hip_build

    stamps_lib = mb.load(hip_build.LIB_STAMPS)
    for f in (stamps_lib.moe_stamps_route, stamps_lib.moe_stamps_expert):
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.c_void_p, ctypes.c_int]
    prod, mb.lib = mb.lib, stamps_lib
    try:
        mb.set_block_schedule(args.schedule)
        cfg = synth.CONFIGS[name]
        R = 2
        sets = moe_sets(cfg, R, args.seed, torch)
        ws = mb.workspace(mb.workspace_bytes(mb.OP_BLOCK, mb.DT_BF16, B=cfg.B, d=cfg.d, E=cfg.E, k=cfg.k,
                                             I=cfg.I, Is=cfg.Is))

        def step(i):
            s = sets[i % R]
            mb.moe_block(s["X"], s["Wr"], cfg.k, s["W13"], s["W2"], s["out"], ws, s["Ws13"], s["Ws2"],
                         s["bias"], s["bias_ld"], topk_ids=s["ids"])

        for i in range(max(R, args.warmup)):
            step(i)
        torch.cuda.synchronize()
        shape = (4, 1024, 8)   # [kernel][workgroup][slot]
        reps = []
        for rep in range(args.trials):
            for f in (stamps_lib.moe_stamps_route, stamps_lib.moe_stamps_expert):
                if f(None, 1):
                    raise RuntimeError("clearing the stamps failed")
            torch.cuda.synchronize()
            step(rep)
            torch.cuda.synchronize()
            tabs = []
            for f in (stamps_lib.moe_stamps_route, stamps_lib.moe_stamps_expert):
                t = np.zeros(shape, np.uint64)
                if f(t.ctypes.data, 0):
                    raise RuntimeError("reading the stamps failed")
                tabs.append(t.astype(np.int64))
            # route and finish from the router's file, gate/up and down from the experts'
            reps.append(np.stack([tabs[0][0], tabs[0][1], tabs[1][2], tabs[1][3]]))
        variant = mb.last_variant()
    finally:
        mb.lib = prod

    def q(v):
        v = np.sort(np.asarray(v, float))
        return {"n": int(len(v)), "min": round(v[0], 2), "p10": round(float(np.percentile(v, 10)), 2),
                "med": round(float(np.median(v)), 2), "p90": round(float(np.percentile(v, 90)), 2),
                "max": round(v[-1], 2)} if len(v) else None

    names = ("route", "route_finish", "expert_up", "expert_down_combine")
    pooled = {n: {pt: [] for pt in TIMELINE_POINTS[n]} for n in names}
    slots, pairs, tasks, xcds, cu_ends = {}, [], {}, {}, []
    for st in reps:
        live = [st[kk, :, 0] > 0 for kk in range(4)]
        t0 = min(st[kk, live[kk], 0].min() for kk in range(4) if live[kk].any())
        for kk, n in enumerate(names):
            for pt in TIMELINE_POINTS[n]:
                sel = live[kk] & (st[kk, :, pt] > 0)
                pooled[n][pt] += list((st[kk, sel, pt] - t0) / 100.0)
        up = st[2]
        g = np.nonzero(live[2] & (up[:, 4] > 0))[0]
        for w in g:
            key = "slot %d" % (w // 256)
            slots.setdefault(key, []).append((up[w, 4] - t0) / 100.0)
        # HW_ID: CU id bits 8-11, shader array bit 12, engine bits 13-15; XCC_ID above
        cu = (up[:, 7] >> 32) * 256 + ((up[:, 7] >> 8) & 0xff)
        per_cu = {}
        for w in g:
            xcds.setdefault("xcd %d" % (up[w, 7] >> 32), []).append((up[w, 4] - t0) / 100.0)
            per_cu[int(cu[w])] = max(per_cu.get(int(cu[w]), 0.0), (up[w, 4] - t0) / 100.0)
        cu_ends += list(per_cu.values())
        pairs += [bool(cu[w] == cu[w + 256]) for w in g if w + 256 < 1024 and up[w + 256, 4] > 0]
        # matrix-shape gate/up: its first task's duration by token tiles, cut
        # or whole, and CU slot (stamp 6: tokens | cut << 16 | ...)
        for w in g:
            info = int(up[w, 6])
            if info and up[w, 3] > 0:
                m, cut = info & 0xffff, (info >> 16) & 1
                key = "%d token tile%s, %s, slot %d" % ((m + 15) // 16, "" if m <= 16 else "s", "cut" if cut else "whole",
                                                          w // 256)
                tasks.setdefault(key, []).append((up[w, 3] - up[w, 2]) / 100.0)
    out = {n: {TIMELINE_POINTS[n][pt]: q(v) for pt, v in pooled[n].items() if v} for n in names}
    out = {n: v for n, v in out.items() if v}
    return {"workload": name, "variant": variant, "blocks": len(reps),
            "unit": "µs from the block's first workgroup start (100 MHz clock)",
            "points": out, "expert_up_end_by_cu_slot": {k: q(v) for k, v in sorted(slots.items())},
            "expert_up_g_and_g256_same_cu": round(sum(pairs) / len(pairs), 4) if pairs else None,
            "expert_up_first_task_us": {k: q(v) for k, v in sorted(tasks.items())},
            "expert_up_end_by_xcd": {k: q(v) for k, v in sorted(xcds.items())},
            "expert_up_cu_end": q(cu_ends)}


# ---------------------------------------------------------------- main

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
    if args.timeline:
        if args.workload not in synth.CONFIGS or synth.CONFIGS[args.workload].dtype != "bf16":
            print("--timeline takes a bf16 block workload (tp16_b1, tp16_b8, tp8_b64)", file=sys.stderr)
            sys.exit(2)
        print(json.dumps({"timeline": run_timeline(args.workload, args, torch, mb, synth)}, ensure_ascii=False),
              flush=True)
        return
    t_start = time.perf_counter()
    cpu = None
    dtype = "bf16"
    if args.workload in ("sweep",) + tuple(synth.CONFIGS):
        head = HEADLINE if args.workload == "sweep" else args.workload
        entry, roof, cfg = run_moe(head, args, torch, mb, synth, True)
        dtype = cfg.dtype
        print("[bench] %s: %.3f us (p10 %.3f, p90 %.3f)" % (head, entry["us"], entry["trials"]["p10_us"],
                                                          entry["trials"]["p90_us"]), file=sys.stderr, flush=True)
        config = dict(entry)
        if args.workload == "sweep":
            sweep = {}
            for name in SWEEP_MOE:
                e, _, _ = run_moe(name, args, torch, mb, synth, False)
                sweep[name] = e
                print("[bench] %s: %.3f us" % (name, e["us"]), file=sys.stderr, flush=True)
            for B in SWEEP_DENSE:
                e, _ = run_gemm("dense", B, args, torch, mb, synth, False)
                sweep["dense_b%d" % B] = e
                print("[bench] dense B=%d: %.3f us" % (B, e["us"]), file=sys.stderr, flush=True)
            config["sweep"] = sweep
            config["route_latent"] = {}
            for B in (1, 64):
                e = run_route_latent(B, args, torch, mb, synth)
                config["route_latent"]["b%d" % B] = e
                print("[bench] router + latent B=%d: merged %.3f us, separate %.3f us"
                      % (B, e["merged"]["us"], e["separate"]["us"]), file=sys.stderr, flush=True)
            stream = run_stream(args, torch, mb)
            config["stream"] = stream
            ref = stream["1gib"]["gbs"]
            config["stream_frac"] = round(config["gbs"] / ref, 4)
            for e in sweep.values():
                e["stream_frac"] = round(e["gbs"] / ref, 4)
            print("[bench] stream 1 GiB: %.1f GB/s" % ref, file=sys.stderr, flush=True)
        if not args.no_cpu_baseline:
            cpu = cpu_baseline(cfg, args)
        value = entry["us"]
    elif args.workload in ("dense", "oproj"):
        entry, roof = run_gemm(args.workload, args.batch, args, torch, mb, synth, True)
        config = dict(entry)
        if not args.no_cpu_baseline:
            cpu = cpu_baseline_gemm(args.workload, args.batch, args)
        value = entry["us"]
    elif args.workload == "latent":
        e = run_route_latent(args.batch, args, torch, mb, synth)
        config = dict(e)
        m = e["merged"]
        roof = dict(bound="hbm", achieved=m["gbs"], peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(m["gbs"] / HBM_PEAK_GBS, 4), traffic=None,
                    kernel="skinny_valu_kernel / skinny_mfma_kernel + route_finish_kernel (router + latent rows)",
                    launch="route", bytes_per_launch=e["algorithmic_bytes"], avg_us=m["us"])
        value = m["us"]
    elif args.workload == "stream":
        st = run_stream(args, torch, mb)
        config = dict(workload="read-only 128-bit streaming yardstick (moe_stream_read)", stream=st)
        e = st["1gib"]
        roof = dict(bound="hbm", achieved=e["gbs"], peak=HBM_PEAK_GBS, unit="GB/s", frac=e["hbm_frac"],
                    traffic=None, kernel="stream_read_kernel", launch="stream", bytes_per_launch=e["bytes"],
                    avg_us=e["us"])
        value, dtype = e["us"], "u32"
    else:
        entry = run_copy(args, torch)
        config = dict(entry)
        roof = dict(bound="hbm", achieved=entry["gbs"], peak=HBM_PEAK_GBS, unit="GB/s", frac=entry["hbm_frac"],
                    traffic=None, kernel="copy", launch="copy", bytes_per_launch=entry["bytes"], avg_us=entry["us"])
        value, dtype = entry["us"], "u8"
    config["bench_wall_s"] = round(time.perf_counter() - t_start, 1)
    line = dict(metric=METRIC, value=round(value, 3), unit="µs", n_gpus=1, steps=args.steps,
                warmup=args.warmup, trials=args.trials, ms_per_step=round(value / 1e3, 6),
                higher_is_better=False, scaling="weak", vs_baseline=None, dtype=dtype, data="synthetic",
                config=config, roofline=roof, cpu_baseline=cpu)
    print(json.dumps(line, ensure_ascii=False), flush=True)


if __name__ == "__main__":
    main()
