"""Benchmark of the fused AllGather+GEMM hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-secondary] [--no-cpu] [--only OP]

Headline: fused AG+GEMM TFLOP/s on the column-parallel MLP up-projection share
(W=8 emulated ranks, A shards 1024x4096 bf16 -> gathered M=8192, B 4096x1792 bf16,
C 8192x1792 fp32), with peer tiles landing in a seeded random order (copy role) while
the compute role consumes them.  One step = one mk_ag_gemm call; inputs are resident
in HBM before timing starts.  Four copies of every buffer rotate between steps so
consecutive calls never hit in the 256 MiB Infinity Cache.

Reported beside it (same JSON line): kernel-time percentiles; a traced call's phase spans
(copy-phase GB/s, the shader clock the kernel actually ran at); the same kernel with every
tile pre-resident (slowdown of the fused arrival); two comparators for context only (a vendor
BLAS bf16 GEMM of the same shape, and "copy kernels, then the GEMM kernel" as separate
launches); GEMM+ReduceScatter and GEMM+AllReduce (TFLOP/s and epilogue GB/s, resident and
with landing); MoE dispatch + grouped GEMM (routed rows, phase spans, grouped-GEMM TFLOP/s
over its compute span, dispatch GB/s); the MLP block in one launch (AllGather + up-projection,
gelu, down-projection + ReduceScatter) beside the same three steps as separate calls; and, with
peer units paced to the xGMI link rate (7 x 153 GB/s), AG, RS and AR at the default role split
and at the split the library's tuner picks.  Everything is timed with HIP events on the stream
the kernels are launched on.

cpu_baseline: the fp64 oracle of the same workload, timed on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E, published
N_CU, MFMA_FLOP_PER_CLK_CU = 256, 4096  # bf16 dense: 256 CUs x 4096 flop/clk
N_SETS = 4
SETTLE_MS = 300.0  # sustained launches before a timed region (clock ramp)
LINK_GBPS = 7 * 153.0  # one MI355X's xGMI: 7 links x 153 GB/s into each GPU
TRACE_UNTOUCHED = -1

# HBM traffic of the AG+GEMM kernel comes from two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) kept
# in profiles/, each scaled by what the same counter reads for a plain copy of known size.  The
# figures are valid only for the kernel they were taken on: the file records a hash of the sources
# that make up the kernel and its launch, and the traffic is reported as null once they differ.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "ag_gemm_kernel_mlp_ag_traffic.md")
KERNEL_SOURCES = ["mk_ag_gemm.hip", "mk_ag_roles.hpp", "mk_copy_ring.hpp", "mk_gemm_tile.hpp", "mk_gemm_tile16.hpp", "mk_tiles.h", "mk_device.hpp",
                  "mk_internal.h", "mk_host_logic.h", "mk_api.cpp"]


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "communication_gemm_role_amd", "csrc", f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def ag_algorithmic_bytes(s) -> int:
    """HBM bytes one fused AG+GEMM launch must move with the local shard in place: the W-1 peer
    shards read and written into the gathered A, the gathered A and B read once, C written once."""
    copy = (s.world - 1) * s.m_shard * s.k * 2
    return 2 * copy + s.m * s.k * 2 + s.k * s.n * 2 + s.m * s.n * 4


def measured_traffic():
    """HBM bytes per launch from the committed counter summary, or None if absent or stale."""
    try:
        with open(TRAFFIC_FILE) as fh:
            kv = dict(line.strip()[2:].split(": ", 1) for line in fh if line.startswith("- ") and ": " in line)
        if kv.get("source_hash") != kernel_source_hash():
            return None
        fetch = float(kv["fetch_kib_per_dispatch"]) * float(kv["fetch_scale"])
        write = float(kv["write_kib_per_dispatch"]) * float(kv["write_scale"])
        return (fetch + write) * 1024.0
    except (OSError, KeyError, ValueError):
        return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-ms", type=float, default=SETTLE_MS,
                    help="sustained launches before each timed region, in ms of wall time")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only", default="",
                    help="profiling: run only this op (ag, ag_resident, ag_identity, rs, ar, rs_emulated, ar_emulated, "
                         "moe, mlp, mlp_resident, mlp_unfused, ag_link, rs_link, ar_link, mlp_link, ring, ring_resident, "
                         "ring_link, vendor, rs_unfused, ar_unfused, copy)")
    ap.add_argument("--n-copy", type=int, default=0, help="with --only *_link: copy workgroups (0: default)")
    return ap.parse_args()


def _bf16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _f32(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def _i32(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def _region(fns, steps, first=0):
    """`steps` calls back to back between two HIP events on the current stream (where the calls
    launch), with a synchronisation on both sides: (wall ms, event ms) per call."""
    import torch
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        fns[(first + i) % len(fns)]()
    e1.record()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps, e0.elapsed_time(e1) / steps


def time_stats(fns, steps, warmup, settle_ms: float = SETTLE_MS, spread: bool = False) -> dict:
    """Run fns[i % len(fns)] `warmup` times, then keep launching back to back for at least
    `settle_ms` of wall time, then time the region: `steps` calls between two HIP events with a
    synchronisation on both sides.  The part's clocks ramp up over the first few tens of
    milliseconds of sustained work (the same kernel runs about 20 % slower in its first 50 launches
    than after 200), so the settle phase is what makes the region a steady-state rate; the first
    region after the warm-up alone is reported too, as cold_ms.  Returns wall ms per step and
    kernel_ms (event time of the region per launch).  With spread, a last pass records an event
    pair around every launch for the per-launch distribution (p10, p50, p90)."""
    import torch
    for i in range(warmup):
        fns[i % len(fns)]()
    cold_wall, _ = _region(fns, steps)
    t0 = time.perf_counter()
    n_settle = 0
    while (time.perf_counter() - t0) * 1e3 < settle_ms:
        for _ in range(20):
            fns[n_settle % len(fns)]()
            n_settle += 1
        torch.cuda.synchronize()
    wall, ev = _region(fns, steps)
    out = {"wall_ms": wall, "kernel_ms": ev, "cold_ms": cold_wall, "settle_launches": n_settle}
    if spread:
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for i in range(steps):
            evs[i][0].record()
            fns[i % len(fns)]()
            evs[i][1].record()
        torch.cuda.synchronize()
        k = np.array([a.elapsed_time(b) for a, b in evs])
        out.update({"per_launch_events_mean": float(k.mean()), "p10": float(np.percentile(k, 10)),
                    "p50": float(np.percentile(k, 50)), "p90": float(np.percentile(k, 90))})
    return out


# ------------------------------------------------------------------------------------------------
# trace records (mk_opts.trace): 8 int64 per workgroup; wall-clock ticks are 100 MHz
# ------------------------------------------------------------------------------------------------
def new_trace(ctx):
    import torch
    return torch.full((ctx.grid * 8,), TRACE_UNTOUCHED, dtype=torch.int64, device="cuda")


def trace_records(tr) -> np.ndarray:
    r = tr.cpu().numpy().reshape(-1, 8)
    return r[r[:, 0] != TRACE_UNTOUCHED]


def us(ticks) -> float:
    return float(ticks) / 100.0


def clock_ghz(rec) -> float:
    """Average shader clock over the workgroups' lifetimes: cycles / wall time."""
    cyc = float((rec[:, 3] - rec[:, 1]).sum())
    wall = float((rec[:, 2] - rec[:, 0]).sum())
    return cyc / wall * 0.1 if wall > 0 else float("nan")


def traced_call(ctx, fns, opts, lead: int = 100):
    """`lead` untraced calls back to back (the clocks stay up), then one call with tracing on;
    returns its records.  fns: one callable or a list rotated through."""
    import torch
    fns = fns if isinstance(fns, (list, tuple)) else [fns]
    tr = new_trace(ctx)
    try:
        for i in range(lead):
            fns[i % len(fns)]()
        opts.trace = tr
        fns[lead % len(fns)]()
        torch.cuda.synchronize()
    finally:
        opts.trace = None
    return trace_records(tr)


def setup_ag(ctx, resident: bool, identity: bool = False, gbps: float = 0.0, n_copy: int = 0):
    """Four rotating buffer sets; returns (shape, calls, opts) with one Opts shared by the calls."""
    import torch
    import communication_gemm_role_amd as mk
    import workloads as wl
    s = wl.AG_MLP
    d = wl.gen_ag(s, run=0)
    order = _i32(wl.ag_arrival_order(s, trial=0))
    shards0 = [_bf16(x) for x in d["a_shards"]]
    b0 = _bf16(d["b"])
    if resident:
        opts = mk.Opts(arrival_mode=mk.MK_ARRIVAL_RESIDENT)
    else:
        opts = mk.Opts(arrival_mode=mk.MK_ARRIVAL_EMULATED, arrival_order=None if identity else order,
                       arrival_gbps=gbps, n_copy_wg=n_copy)
    calls = []
    for _ in range(N_SETS):
        shards = [x.clone() for x in shards0]
        b = b0.clone()
        ag = torch.empty((s.m, s.k), dtype=torch.bfloat16, device="cuda")
        c = torch.empty((s.m, s.n), dtype=torch.float32, device="cuda")
        if resident:
            ag.copy_(torch.cat(shards, 0))
        else:
            ag[:s.m_shard].copy_(shards[0])
            shards[0] = ag[:s.m_shard]
        calls.append(lambda sh=shards, b=b, ag=ag, c=c: mk.mk_ag_gemm(ctx, sh, s.world, 0, b, ag, c, opts=opts))
    return s, calls, opts


def setup_ag_two_launch(ctx):
    """Comparator: the peer shards copied into the gathered A by separate copy kernels, then the
    GEMM kernel on resident data (overlap only at kernel boundaries)."""
    import torch
    import communication_gemm_role_amd as mk
    import workloads as wl
    s = wl.AG_MLP
    d = wl.gen_ag(s, run=0)
    shards0 = [_bf16(x) for x in d["a_shards"]]
    b0 = _bf16(d["b"])
    opts = mk.Opts(arrival_mode=mk.MK_ARRIVAL_RESIDENT)
    calls = []
    for _ in range(N_SETS):
        shards = [x.clone() for x in shards0]
        b = b0.clone()
        ag = torch.empty((s.m, s.k), dtype=torch.bfloat16, device="cuda")
        ag[:s.m_shard].copy_(shards[0])
        c = torch.empty((s.m, s.n), dtype=torch.float32, device="cuda")

        def step(sh=shards, b=b, ag=ag, c=c):
            for r in range(1, s.world):
                ag[r * s.m_shard:(r + 1) * s.m_shard].copy_(sh[r])
            mk.mk_ag_gemm(ctx, None, s.world, 0, b, ag, c, opts=opts)
        calls.append(step)
    return s, calls


def setup_vendor_gemm():
    """Comparator: torch.matmul (the vendor BLAS) on the same bf16 shape, bf16 output."""
    import torch
    import workloads as wl
    s = wl.AG_MLP
    d = wl.gen_ag(s, run=0)
    a0 = torch.cat([_bf16(x) for x in d["a_shards"]], 0)
    b0 = _bf16(d["b"])
    calls = []
    for _ in range(N_SETS):
        a, b = a0.clone(), b0.clone()
        out = torch.empty((s.m, s.n), dtype=torch.bfloat16, device="cuda")
        calls.append(lambda a=a, b=b, out=out: torch.matmul(a, b, out=out))
    return s, calls


def setup_reduce(ctx, op: str, emulated: bool = False, n_reduce: int = 0, gbps: float = 0.0, n_copy: int = 0):
    import torch
    import communication_gemm_role_amd as mk
    import workloads as wl
    s = wl.RS_DOWN if op == "rs" else wl.AR_DECODE
    d = wl.gen_reduce(s, op, run=0)
    a0, b0 = _bf16(d["a"]), _bf16(d["b"])
    p0 = [None if p is None else _f32(p) for p in d["peers"]]
    order = _i32(wl.reduce_arrival_order(s, op)) if emulated else None
    opts = mk.Opts(arrival_mode=mk.MK_ARRIVAL_EMULATED if emulated else mk.MK_ARRIVAL_RESIDENT, arrival_order=order,
                   n_reduce_wg=n_reduce, arrival_gbps=gbps if emulated else 0.0, n_copy_wg=n_copy if emulated else 0)
    calls = []
    for _ in range(N_SETS):
        a, b = a0.clone(), b0.clone()
        peers = [None if p is None else p.clone() for p in p0]
        if op == "rs":
            own = torch.empty((s.m_slice, s.n), device="cuda")
            ob = [None] + [torch.empty((s.m_slice, s.n), device="cuda") for _ in range(1, s.world)]
            calls.append(lambda a=a, b=b, pe=peers, own=own, ob=ob: mk.mk_gemm_rs(ctx, a, b, s.world, 0, pe, own, ob,
                                                                                  opts=opts))
        else:
            out = torch.empty((s.m, s.n), device="cuda")
            calls.append(lambda a=a, b=b, pe=peers, out=out: mk.mk_gemm_ar(ctx, a, b, s.world, 0, pe, out, opts=opts))
    return s, calls, opts


def setup_reduce_unfused(op: str):
    """Comparator: the vendor BLAS GEMM (torch.matmul, bf16 out) of this rank's partial, then a
    separate sum of the owned rows with the resident peer partials (torch adds, fp32): the
    reduction after the GEMM at kernel boundaries.  RS's outbox slices are left as views of the
    GEMM output (a collective would send them)."""
    import torch
    import workloads as wl
    s = wl.RS_DOWN if op == "rs" else wl.AR_DECODE
    d = wl.gen_reduce(s, op, run=0)
    a0, b0 = _bf16(d["a"]), _bf16(d["b"])
    p0 = [_f32(p) for p in d["peers"] if p is not None]
    rows = s.m_slice if op == "rs" else s.m
    calls = []
    for _ in range(N_SETS):
        a, b = a0.clone(), b0.clone()
        peers = [p.clone() for p in p0]
        prod = torch.empty((s.m, s.n), dtype=torch.bfloat16, device="cuda")
        out = torch.empty((rows, s.n), dtype=torch.float32, device="cuda")

        def step(a=a, b=b, pe=peers, prod=prod, out=out):
            torch.matmul(a, b, out=prod)
            torch.add(pe[0], pe[1], out=out)
            for p in pe[2:]:
                out.add_(p)
            out.add_(prod[:rows])
        calls.append(step)
    return s, calls


def reduce_bytes(sh, op: str, emulated: bool):
    """Algorithmic HBM bytes of one RS/AR call: (epilogue, total)."""
    rows = sh.m_slice if op == "rs" else sh.m
    peers = (sh.world - 1) * rows * sh.n * 4
    epi = peers + rows * sh.n * 4 + ((sh.world - 1) * sh.m_slice * sh.n * 4 if op == "rs" else 0)
    total = epi + sh.m * sh.k * 2 + sh.k * sh.n * 2 + (2 * peers if emulated else 0)
    return epi, total


def setup_moe(ctx):
    import torch
    import communication_gemm_role_amd as mk
    import workloads as wl
    s = wl.MOE_FULL
    d = wl.gen_moe(s, run=0)
    order = _i32(wl.moe_arrival_order(s, 0))
    t0 = [_bf16(t) for t in d["tokens"]]
    lg0, bs0, w0 = _f32(d["logits"]), _f32(d["bias"]), _bf16(d["w_up"])
    calls, offsets = [], []
    opts = mk.Opts(arrival_order=order)
    for _ in range(2):  # 2 sets: ~1 GiB each
        toks = [t.clone() for t in t0]
        lg, bs, w = lg0.clone(), bs0.clone(), w0.clone()
        topk = torch.empty((s.tokens, s.top_k), dtype=torch.int32, device="cuda")
        offs = torch.empty((s.n_local + 1,), dtype=torch.int32, device="cuda")
        segt = torch.empty((s.capacity,), dtype=torch.int32, device="cuda")
        x = torch.empty((s.capacity, s.hidden), dtype=torch.bfloat16, device="cuda")
        y = torch.empty((s.capacity, s.ffn), device="cuda")
        offsets.append(offs)
        calls.append(lambda toks=toks, lg=lg, bs=bs, w=w, topk=topk, offs=offs, segt=segt, x=x, y=y:
                     mk.mk_moe_dispatch_gemm(ctx, toks, lg, bs, s.top_k, s.expert_begin, w, topk, offs, segt, x, y,
                                             opts=opts))
    return s, offsets, calls, opts


def setup_mlp(ctx, resident: bool = False, gbps: float = 0.0):
    """MLP block in one launch (AllGather + up-projection, gelu, down-projection + ReduceScatter),
    two rotating buffer sets; returns (shape, calls, opts)."""
    import torch
    import communication_gemm_role_amd as mk
    import workloads as wl
    s = wl.MLP_FULL
    d = wl.gen_mlp(s, run=0)
    sh0 = [_bf16(x) for x in d["a_shards"]]
    bu0, bd0 = _bf16(d["b_up"]), _bf16(d["b_down"])
    p0 = [None if p is None else _f32(p) for p in d["peers"]]
    if resident:
        opts = mk.Opts(arrival_mode=mk.MK_ARRIVAL_RESIDENT)
    else:
        opts = mk.Opts(arrival_mode=mk.MK_ARRIVAL_EMULATED, arrival_unit_rows=s.unit_rows,
                       arrival_unit_cols=s.unit_cols, arrival_order=_i32(wl.ag_arrival_order(s.ag, trial=0)),
                       arrival_gbps=gbps)
    calls = []
    for _ in range(2):
        shards = [x.clone() for x in sh0]
        bu, bd = bu0.clone(), bd0.clone()
        peers = [None if p is None else p.clone() for p in p0]
        ag = torch.empty((s.m, s.k), dtype=torch.bfloat16, device="cuda")
        if resident:
            ag.copy_(torch.cat(shards, 0))
        else:
            ag[:s.m_shard].copy_(shards[0])
            shards[0] = ag[:s.m_shard]
        h = torch.empty((s.m, s.n_up), dtype=torch.bfloat16, device="cuda")
        own = torch.empty((s.m_shard, s.n_out), device="cuda")
        ob = [None] + [torch.empty((s.m_shard, s.n_out), device="cuda") for _ in range(1, s.world)]
        calls.append(lambda sh=shards, bu=bu, bd=bd, pe=peers, ag=ag, h=h, own=own, ob=ob:
                     mk.mk_mlp_ag_rs(ctx, sh, s.world, 0, bu, bd, pe, ag, h, own, ob, opts=opts))
    return s, calls, opts


def setup_mlp_unfused(ctx):
    """Comparator: the same block as three steps, mk_ag_gemm (fp32 U), torch's gelu and bf16
    conversion, then mk_gemm_rs on H (peers' partials resident)."""
    import torch
    import communication_gemm_role_amd as mk
    import workloads as wl
    s = wl.MLP_FULL
    d = wl.gen_mlp(s, run=0)
    sh0 = [_bf16(x) for x in d["a_shards"]]
    bu0, bd0 = _bf16(d["b_up"]), _bf16(d["b_down"])
    p0 = [None if p is None else _f32(p) for p in d["peers"]]
    o_ag = mk.Opts(arrival_mode=mk.MK_ARRIVAL_EMULATED, arrival_unit_rows=s.unit_rows, arrival_unit_cols=s.unit_cols,
                   arrival_order=_i32(wl.ag_arrival_order(s.ag, trial=0)))
    o_rs = mk.Opts(arrival_mode=mk.MK_ARRIVAL_RESIDENT)
    calls = []
    for _ in range(2):
        shards = [x.clone() for x in sh0]
        bu, bd = bu0.clone(), bd0.clone()
        peers = [None if p is None else p.clone() for p in p0]
        ag = torch.empty((s.m, s.k), dtype=torch.bfloat16, device="cuda")
        ag[:s.m_shard].copy_(shards[0])
        shards[0] = ag[:s.m_shard]
        u = torch.empty((s.m, s.n_up), device="cuda")
        own = torch.empty((s.m_shard, s.n_out), device="cuda")
        ob = [None] + [torch.empty((s.m_shard, s.n_out), device="cuda") for _ in range(1, s.world)]

        def step(sh=shards, bu=bu, bd=bd, pe=peers, ag=ag, u=u, own=own, ob=ob):
            mk.mk_ag_gemm(ctx, sh, s.world, 0, bu, ag, u, opts=o_ag)
            h = torch.nn.functional.gelu(u).to(torch.bfloat16)
            mk.mk_gemm_rs(ctx, h, bd, s.world, 0, pe, own, ob, opts=o_rs)
        calls.append(step)
    return s, calls


def setup_ring(ctx, resident: bool = False, gbps: float = 0.0, n_copy: int = 0):
    """Ring attention, one rank's share (8 ranks x 4096 tokens, 8 heads of 128), two buffer sets."""
    import torch
    import communication_gemm_role_amd as mk
    import workloads as wl
    s = wl.RING_FULL
    d = wl.gen_ring(s, run=0)
    q0 = _bf16(d["q"])
    k0 = [_bf16(k) for k in d["k_shards"]]
    v0 = [_bf16(v) for v in d["v_shards"]]
    if resident:
        opts = mk.Opts(arrival_mode=mk.MK_ARRIVAL_RESIDENT)
    else:
        opts = mk.Opts(arrival_mode=mk.MK_ARRIVAL_EMULATED, arrival_order=_i32(wl.ring_arrival_order(s)),
                       arrival_gbps=gbps, n_copy_wg=n_copy)
    calls = []
    for _ in range(2):
        q, ks, vs = q0.clone(), [k.clone() for k in k0], [v.clone() for v in v0]
        out = torch.empty((s.heads, s.s_local, s.d), device="cuda")
        lse = torch.empty((s.heads, s.s_local), device="cuda")
        kr = None if resident else torch.empty((s.world, s.heads, s.s_local, s.d), dtype=torch.bfloat16, device="cuda")
        vr = None if resident else torch.empty_like(kr)
        calls.append(lambda q=q, ks=ks, vs=vs, out=out, lse=lse, kr=kr, vr=vr:
                     mk.mk_ring_attention(ctx, q, ks, vs, 0, out, lse, kr, vr, opts=opts))
    return s, calls, opts


def tune_and_time(ctx, kind: str, gbps: float, settle_ms: float) -> dict:
    """Role-split tuning at a link rate: the library's tuner picks n_copy_wg among the candidates,
    then the default and the chosen split are each timed like every other secondary."""
    import torch
    import communication_gemm_role_amd as mk
    import workloads as wl
    if kind == "ag":
        s, calls, opts = setup_ag(ctx, False, gbps=gbps)
        d = wl.gen_ag(s, run=0)
        shards = [_bf16(x) for x in d["a_shards"]]
        b = _bf16(d["b"])
        ag = torch.empty((s.m, s.k), dtype=torch.bfloat16, device="cuda")
        ag[:s.m_shard].copy_(shards[0])
        shards[0] = ag[:s.m_shard]
        c = torch.empty((s.m, s.n), device="cuda")
        cands = [16, 24, 32, 48, 64, 96, 128, 160, 192]
        best, us = mk.mk_ag_gemm_tune(ctx, shards, s.world, 0, b, ag, c, cands, reps=30, opts=opts)
        del shards, b, ag, c
        setup = lambda nc: setup_ag(ctx, False, gbps=gbps, n_copy=nc)[1]
    else:
        sh, calls, opts = setup_reduce(ctx, kind, emulated=True, gbps=gbps)
        d = wl.gen_reduce(sh, kind, run=0)
        a, b = _bf16(d["a"]), _bf16(d["b"])
        peers = [None if p is None else _f32(p) for p in d["peers"]]
        cands = [16, 32, 48, 64, 96, 128, 160, 192, 224]
        if kind == "rs":
            own = torch.empty((sh.m_slice, sh.n), device="cuda")
            ob = [None] + [torch.empty((sh.m_slice, sh.n), device="cuda") for _ in range(1, sh.world)]
            best, us = mk.mk_gemm_rs_tune(ctx, a, b, sh.world, 0, peers, own, ob, cands, reps=30, opts=opts)
        else:
            out = torch.empty((sh.m, sh.n), device="cuda")
            best, us = mk.mk_gemm_ar_tune(ctx, a, b, sh.world, 0, peers, out, cands, reps=30, opts=opts)
        del a, b, peers
        setup = lambda nc: setup_reduce(ctx, kind, emulated=True, gbps=gbps, n_copy=nc)[1]
    t_def = time_stats(calls, 100, 3, settle_ms)["kernel_ms"]
    del calls
    torch.cuda.empty_cache()
    cb = setup(best)
    t_best = time_stats(cb, 100, 3, settle_ms)["kernel_ms"]
    del cb
    torch.cuda.empty_cache()
    return {"default_kernel_ms": round(t_def, 5), "tuned_n_copy": best, "tuned_kernel_ms": round(t_best, 5),
            "tuner_us": dict(zip([str(c) for c in cands], [round(u, 1) for u in us]))}


def mlp_trace_summary(rec) -> dict:
    t0 = rec[:, 0].min()
    up = rec[:, 6]
    return {"kernel_span_us": round(us(rec[:, 2].max() - t0), 2), "shader_clock_GHz": round(clock_ghz(rec), 3),
            "up_projection_done_us": {"min": round(us(up.min() - t0), 2), "median": round(us(np.median(up) - t0), 2),
                                      "max": round(us(up.max() - t0), 2)}}


def cpu_info() -> dict:
    model = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas, threads = "unknown", None
    try:
        from threadpoolctl import threadpool_info
        info = [x for x in threadpool_info() if x.get("user_api") == "blas"]
        if info:
            blas, threads = info[0].get("internal_api", "unknown"), int(info[0]["num_threads"])
    except Exception:
        pass
    return {"cpu": model, "affinity_cores": len(os.sched_getaffinity(0)), "blas": blas, "blas_threads": threads}


def cpu_baseline(budget_s: float = 12.0):
    """The fp64 oracle on the headline workload, repeated for about budget_s seconds."""
    import oracle
    import workloads as wl
    s = wl.AG_MLP
    d = wl.gen_ag(s, run=0)
    ci = cpu_info()
    threads = ci["blas_threads"] or ci["affinity_cores"]
    reps, t_total = 0, 0.0
    while t_total < budget_s and reps < 1000:
        t0 = time.perf_counter()
        oracle.ag_gemm(d["a_shards"], d["b"])
        t_total += time.perf_counter() - t0
        reps += 1
    t = t_total / reps
    return {"value": s.flops / t / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"full AG+GEMM workload (W=8, M=8192, N=1792, K=4096) in fp64 NumPy matmul, {reps} "
                      f"repetitions, {t:.2f} s each; the oracle computes in fp64 while the GPU uses bf16 MFMA, "
                      "so the ratio is context, not a like-for-like speed claim",
            "host": ci}


def ag_trace_summary(rec, s) -> dict:
    t0 = rec[:, 0].min()
    cp, co = rec[rec[:, 4] == 0], rec[rec[:, 4] == 1]
    out = {"kernel_span_us": round(us(rec[:, 2].max() - t0), 2), "shader_clock_GHz": round(clock_ghz(co), 3)}
    if len(cp):
        copy_end = cp[:, 5].max()
        copy_bytes = 2 * (s.world - 1) * s.m_shard * s.k * 2
        out["copy_span_us"] = round(us(copy_end - t0), 2)
        out["copy_GBs"] = round(copy_bytes / (us(copy_end - t0) * 1e-6) / 1e9, 1)
    ready = co[co[:, 5] > 0, 5]
    if len(ready):
        out["first_operands_ready_us"] = {"min": round(us(ready.min() - t0), 2),
                                          "median": round(us(np.median(ready) - t0), 2),
                                          "max": round(us(ready.max() - t0), 2)}
    return out


def moe_trace_summary(rec, s, R) -> dict:
    t0 = rec[:, 0].min()
    cp, co = rec[rec[:, 4] == 0], rec[rec[:, 4] == 1]
    route_end, scan_seen, disp_end = cp[:, 5].max(), cp[:, 6].min(), cp[:, 7].max()
    ready = co[co[:, 5] > 0, 5]
    end = rec[:, 2].max()
    out = {"kernel_span_us": round(us(end - t0), 2), "routing_done_us": round(us(route_end - t0), 2),
           "scan_seen_us": round(us(scan_seen - t0), 2), "dispatch_done_us": round(us(disp_end - t0), 2),
           "dispatch_GBs": round(16384 * R / (us(disp_end - scan_seen) * 1e-6) / 1e9, 1),
           "shader_clock_GHz": round(clock_ghz(rec), 3)}
    if len(ready):
        span = us(end - ready.min())
        out["gemm_span_us"] = round(span, 2)
        out["gemm_tflops_over_span"] = round(s.flops(R) / (span * 1e-6) / 1e12, 1)
    return out


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}), flush=True)
        sys.exit(2)
    import torch
    import communication_gemm_role_amd as mk
    assert torch.cuda.is_available(), "no GPU visible"
    ctx = mk.Context(0)

    if a.only:
        if a.only in ("ag", "ag_resident", "ag_identity"):
            _, calls, _ = setup_ag(ctx, a.only == "ag_resident", identity=a.only == "ag_identity")
        elif a.only == "ag_link":
            _, calls, _ = setup_ag(ctx, False, gbps=LINK_GBPS, n_copy=a.n_copy)
        elif a.only in ("rs_link", "ar_link"):
            _, calls, _ = setup_reduce(ctx, a.only[:2], emulated=True, gbps=LINK_GBPS, n_copy=a.n_copy)
        elif a.only == "mlp_link":
            _, calls, _ = setup_mlp(ctx, gbps=LINK_GBPS)
        elif a.only in ("ring", "ring_resident", "ring_link"):
            _, calls, _ = setup_ring(ctx, resident=a.only == "ring_resident",
                                     gbps=LINK_GBPS if a.only == "ring_link" else 0.0, n_copy=a.n_copy)
        elif a.only in ("rs", "ar"):
            _, calls, _ = setup_reduce(ctx, a.only)
        elif a.only in ("rs_emulated", "ar_emulated"):
            _, calls, _ = setup_reduce(ctx, a.only[:2], emulated=True)
        elif a.only == "moe":
            _, _, calls, _ = setup_moe(ctx)
        elif a.only in ("mlp", "mlp_resident"):
            _, calls, _ = setup_mlp(ctx, resident=a.only == "mlp_resident")
        elif a.only == "mlp_unfused":
            _, calls = setup_mlp_unfused(ctx)
        elif a.only in ("rs_unfused", "ar_unfused"):
            _, calls = setup_reduce_unfused(a.only[:2])
        elif a.only == "vendor":
            _, calls = setup_vendor_gemm()
        elif a.only == "copy":
            # calibration for the HBM byte counters: a plain device copy of 256 MiB per launch
            src = torch.empty(64 << 20, dtype=torch.float32, device="cuda").fill_(1.0)
            dst = torch.empty_like(src)
            calls = [lambda: dst.copy_(src)]
        else:
            raise SystemExit(f"unknown --only {a.only}")
        t = time_stats(calls, a.steps, a.warmup, a.settle_ms)
        st = ctx.status()
        print(json.dumps({"only": a.only, "ms_per_step": t["wall_ms"], "kernel_ms": t["kernel_ms"],
                          "cold_ms": t["cold_ms"], "settle_launches": t["settle_launches"], "status": st}),
              flush=True)
        return

    s, calls, opts = setup_ag(ctx, resident=False)
    t = time_stats(calls, a.steps, a.warmup, a.settle_ms, spread=True)
    status = ctx.status()
    if status != mk.MK_OK:
        raise SystemExit(f"device status {status}: {mk.strerror(status)}")
    rec = traced_call(ctx, calls, opts)
    tr = ag_trace_summary(rec, s)
    value = s.flops / (t["wall_ms"] * 1e-3) / 1e12
    achieved = s.flops / (t["kernel_ms"] * 1e-3) / 1e12
    clk = tr["shader_clock_GHz"]
    peak_clk = N_CU * MFMA_FLOP_PER_CLK_CU * clk * 1e9 / 1e12
    result = {
        "metric": "fused AG+GEMM TFLOP/s on 1 MI355X and % of bf16 MFMA peak; RS/AR epilogue GB/s",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(t["wall_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "AG+GEMM column-parallel MLP up-proj share: W=8 emulated ranks, A shards 1024x4096 "
                               "bf16 (gathered M=8192), B 4096x1792 bf16, C 8192x1792 fp32, 128x128 units landing "
                               "in a seeded random order", "arrival": "emulated", "sets_rotated": N_SETS},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "traffic_unit": "HBM bytes per launch", "algorithmic_bytes": ag_algorithmic_bytes(s),
                     "measured_clock_GHz": clk, "peak_at_measured_clock": round(peak_clk, 1),
                     "frac_at_measured_clock": round(achieved / peak_clk, 4) if peak_clk > 0 else None},
        "kernel_ms": {k: round(v, 5) for k, v in t.items() if k not in ("wall_ms", "cold_ms", "settle_launches")},
        "timing": {"region": "steps launches back to back between two HIP events, synchronised on both sides",
                   "settle_ms": a.settle_ms, "settle_launches": t["settle_launches"],
                   "cold_ms_per_step": round(t["cold_ms"], 5),
                   "note": "cold = the same region right after the warm-up steps, before the clocks have ramped"},
        "trace": tr,
        "env": {"gpu": torch.cuda.get_device_name(0), "hip": torch.version.hip, "torch": torch.__version__},
    }
    traffic = measured_traffic()
    if traffic is not None:
        result["roofline"]["traffic"] = round(traffic)
    del calls
    if not a.no_secondary:
        sec = {}
        _, calls_r, _ = setup_ag(ctx, resident=True)
        tr_ = time_stats(calls_r, 100, 3, a.settle_ms)
        sec["ag_resident"] = {"kernel_ms": round(tr_["kernel_ms"], 5),
                              "tflops": round(s.flops / (tr_["kernel_ms"] * 1e-3) / 1e12, 2),
                              "fused_slowdown": round(t["kernel_ms"] / tr_["kernel_ms"] - 1.0, 4)}
        del calls_r
        _, calls_2 = setup_ag_two_launch(ctx)
        t2 = time_stats(calls_2, 100, 3, a.settle_ms)
        sec["ag_copy_then_gemm"] = {"ms_per_step": round(t2["kernel_ms"], 5),
                                    "tflops": round(s.flops / (t2["kernel_ms"] * 1e-3) / 1e12, 2),
                                    "note": "comparator: 7 copy kernels then the GEMM kernel, separate launches"}
        del calls_2
        _, calls_v = setup_vendor_gemm()
        tv = time_stats(calls_v, 100, 3, a.settle_ms)
        sec["vendor_gemm"] = {"kernel_ms": round(tv["kernel_ms"], 5),
                              "tflops": round(s.flops / (tv["kernel_ms"] * 1e-3) / 1e12, 2),
                              "note": "comparator: torch.matmul bf16 -> bf16 on the gathered shape, operands resident"}
        del calls_v
        torch.cuda.empty_cache()
        for op in ("rs", "ar"):
            for emulated in (False, True):
                sh, cr, _ = setup_reduce(ctx, op, emulated=emulated)
                tt = time_stats(cr, 100, 3, a.settle_ms)
                k_ = tt["kernel_ms"]
                epi, total = reduce_bytes(sh, op, emulated)
                sec[op + ("_landing" if emulated else "")] = {
                    "kernel_ms": round(k_, 5), "tflops": round(sh.flops / (k_ * 1e-3) / 1e12, 2),
                    "epilogue_GBs": round(epi / (k_ * 1e-3) / 1e9, 1),
                    "total_GBs": round(total / (k_ * 1e-3) / 1e9, 1),
                    "hbm_frac": round(total / (k_ * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
                del cr
                torch.cuda.empty_cache()
            _, cu = setup_reduce_unfused(op)
            tu = time_stats(cu, 100, 3, a.settle_ms)
            sec[op]["unfused_ms"] = round(tu["kernel_ms"], 5)
            sec[op]["unfused_note"] = ("comparator: torch.matmul bf16 -> bf16, then torch adds of the peer "
                                       "partials into the owned rows (fp32), separate launches")
            del cu
            torch.cuda.empty_cache()
        sm, offs, cm, mopts = setup_moe(ctx)
        tm = time_stats(cm, 100, 2, a.settle_ms)
        o = offs[0].cpu().numpy()
        R = int(o[-1])
        mrec = traced_call(ctx, cm, mopts)
        sec["moe"] = {"kernel_ms": round(tm["kernel_ms"], 5), "routed_rows": R,
                      "rows_per_expert": np.diff(o).tolist(),
                      "tflops": round(sm.flops(R) / (tm["kernel_ms"] * 1e-3) / 1e12, 2),
                      "trace": moe_trace_summary(mrec, sm, R)}
        del cm
        torch.cuda.empty_cache()
        ms_, cmlp, mlopts = setup_mlp(ctx)
        tml = time_stats(cmlp, 100, 3, a.settle_ms)
        mlrec = traced_call(ctx, cmlp, mlopts)
        del cmlp
        _, cmlr, _ = setup_mlp(ctx, resident=True)
        tmr = time_stats(cmlr, 100, 3, a.settle_ms)
        del cmlr
        _, cmu = setup_mlp_unfused(ctx)
        tmu = time_stats(cmu, 100, 3, a.settle_ms)
        del cmu
        torch.cuda.empty_cache()
        sec["mlp"] = {"kernel_ms": round(tml["kernel_ms"], 5),
                      "tflops": round(ms_.flops / (tml["kernel_ms"] * 1e-3) / 1e12, 2),
                      "resident_kernel_ms": round(tmr["kernel_ms"], 5),
                      "unfused_ms": round(tmu["kernel_ms"], 5),
                      "unfused_tflops": round(ms_.flops / (tmu["kernel_ms"] * 1e-3) / 1e12, 2),
                      "trace": mlp_trace_summary(mlrec),
                      "note": "W=8 emulated ranks, A shards 1024x4096, B_up 4096x1792, B_down 1792x4096, peers' "
                              "partials resident; unfused = mk_ag_gemm, torch gelu + bf16, mk_gemm_rs"}
        rsh, crg, ropts = setup_ring(ctx)
        trg = time_stats(crg, 50, 3, a.settle_ms)
        rrec = traced_call(ctx, crg, ropts, lead=20)
        del crg
        _, crr, _ = setup_ring(ctx, resident=True)
        trr = time_stats(crr, 50, 3, a.settle_ms)
        del crr
        _, crl, _ = setup_ring(ctx, gbps=LINK_GBPS)
        trl = time_stats(crl, 50, 3, a.settle_ms)
        del crl
        torch.cuda.empty_cache()
        cp = rrec[rrec[:, 4] == 0]
        sec["ring_attention"] = {
            "kernel_ms": round(trg["kernel_ms"], 5), "tflops": round(rsh.flops / (trg["kernel_ms"] * 1e-3) / 1e12, 2),
            "resident_kernel_ms": round(trr["kernel_ms"], 5),
            "link_rate_kernel_ms": round(trl["kernel_ms"], 5),
            "trace": {"kernel_span_us": round(us(rrec[:, 2].max() - rrec[:, 0].min()), 2),
                      "ring_landed_us": round(us(cp[:, 5].max() - rrec[:, 0].min()), 2) if len(cp) else None,
                      "shader_clock_GHz": round(clock_ghz(rrec), 3)},
            "note": "8 ranks x 4096 tokens, 8 heads of 128, no mask; peers' K/V blocks land in ring order (192 copy "
                    "workgroups); flops = 4*heads*s_local*(world*s_local)*128 (P enters as two bf16 terms: the "
                    "P.V MFMAs are issued twice)"}
        link = {"gbps": LINK_GBPS, "note": "peer units paced to 7 xGMI links x 153 GB/s (mk_opts.arrival_gbps); "
                                          "tuned = the fastest n_copy_wg found by mk_*_tune, then timed"}
        for kind in ("ag", "rs", "ar"):
            link[kind] = tune_and_time(ctx, kind, LINK_GBPS, a.settle_ms)
        link["ag"]["tuned_tflops"] = round(s.flops / (link["ag"]["tuned_kernel_ms"] * 1e-3) / 1e12, 2)
        link["ag"]["exposed_vs_resident"] = round(link["ag"]["tuned_kernel_ms"] / tr_["kernel_ms"] - 1.0, 4)
        sec["link_rate"] = link
        st = ctx.status()
        if st != mk.MK_OK:
            raise SystemExit(f"device status {st}: {mk.strerror(st)}")
        result["secondary"] = sec
    if not a.no_cpu:
        result["cpu_baseline"] = cpu_baseline()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
