"""Benchmark of the fused AllGather+GEMM hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-secondary] [--no-cpu]

Headline: fused AG+GEMM TFLOP/s on the column-parallel MLP up-projection share
(W=8 emulated ranks, A shards 1024x4096 bf16 -> gathered M=8192, B 4096x1792 bf16,
C 8192x1792 fp32), with peer tiles landing in a seeded random order (copy role) while
the compute role consumes them.  One step = one mk_ag_gemm call; inputs are resident
in HBM before timing starts.  Four copies of every buffer rotate between steps so
consecutive calls never hit in the 256 MiB Infinity Cache.

Secondary (same JSON line): the same kernel with every tile pre-resident (slowdown of
the fused arrival), GEMM+ReduceScatter and GEMM+AllReduce (epilogue GB/s) and MoE
dispatch + grouped GEMM, each timed with HIP events on the launch stream.

cpu_baseline: the fp64 oracle of the same workload, timed on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E, published
N_SETS = 4

# HBM traffic of the AG+GEMM kernel comes from two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) kept
# in profiles/, each scaled by what the same counter reads for a plain copy of known size.  The
# figures are valid only for the kernel they were taken on: the file records a hash of the sources
# that make up the kernel and its launch, and the traffic is reported as null once they differ.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "ag_gemm_kernel_mlp_ag_traffic.md")
KERNEL_SOURCES = ["mk_ag_gemm.hip", "mk_gemm_tile.hpp", "mk_device.hpp", "mk_internal.h", "mk_host_logic.h",
                  "mk_api.cpp"]


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
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only", default="",
                    help="profiling: run only this op (ag, ag_resident, ag_identity, rs, ar, rs_emulated, ar_emulated, moe, "
                         "copy)")
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


def time_calls(fns, steps, warmup):
    """Run fns[i % len(fns)] warmup + steps times; return (wall ms per step, mean kernel ms per launch)."""
    import torch
    for i in range(warmup):
        fns[i % len(fns)]()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record()
        fns[i % len(fns)]()
        ev[i][1].record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    kern = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    return wall, kern


# ------------------------------------------------------------------------------------------------
def setup_ag(ctx, resident: bool, identity: bool = False):
    import torch
    import communication_gemm_role_amd as mk
    import workloads as wl
    s = wl.AG_MLP
    d = wl.gen_ag(s, run=0)
    order = _i32(wl.ag_arrival_order(s, trial=0))
    shards0 = [_bf16(x) for x in d["a_shards"]]
    b0 = _bf16(d["b"])
    calls = []
    for _ in range(N_SETS):
        shards = [x.clone() for x in shards0]
        b = b0.clone()
        ag = torch.empty((s.m, s.k), dtype=torch.bfloat16, device="cuda")
        c = torch.empty((s.m, s.n), dtype=torch.float32, device="cuda")
        if resident:
            ag.copy_(torch.cat(shards, 0))
            opts = mk.Opts(arrival_mode=mk.MK_ARRIVAL_RESIDENT)
        else:
            ag[:s.m_shard].copy_(shards[0])
            shards[0] = ag[:s.m_shard]
            opts = mk.Opts(arrival_mode=mk.MK_ARRIVAL_EMULATED, arrival_order=None if identity else order)
        calls.append(lambda sh=shards, b=b, ag=ag, c=c, o=opts: mk.mk_ag_gemm(ctx, sh, s.world, 0, b, ag, c, opts=o))
    return s, calls


def setup_reduce(ctx, op: str, emulated: bool = False, n_reduce: int = 0):
    import torch
    import communication_gemm_role_amd as mk
    import workloads as wl
    s = wl.RS_DOWN if op == "rs" else wl.AR_DECODE
    d = wl.gen_reduce(s, op, run=0)
    a0, b0 = _bf16(d["a"]), _bf16(d["b"])
    p0 = [None if p is None else _f32(p) for p in d["peers"]]
    order = _i32(wl.reduce_arrival_order(s, op)) if emulated else None
    opts = mk.Opts(arrival_mode=mk.MK_ARRIVAL_EMULATED if emulated else mk.MK_ARRIVAL_RESIDENT, arrival_order=order,
                   n_reduce_wg=n_reduce)
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
    return s, calls


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
    for _ in range(2):  # 2 sets: ~1 GiB each
        toks = [t.clone() for t in t0]
        lg, bs, w = lg0.clone(), bs0.clone(), w0.clone()
        topk = torch.empty((s.tokens, s.top_k), dtype=torch.int32, device="cuda")
        offs = torch.empty((s.n_local + 1,), dtype=torch.int32, device="cuda")
        segt = torch.empty((s.capacity,), dtype=torch.int32, device="cuda")
        x = torch.empty((s.capacity, s.hidden), dtype=torch.bfloat16, device="cuda")
        y = torch.empty((s.capacity, s.ffn), device="cuda")
        o = mk.Opts(arrival_order=order)
        offsets.append(offs)
        calls.append(lambda toks=toks, lg=lg, bs=bs, w=w, topk=topk, offs=offs, segt=segt, x=x, y=y:
                     mk.mk_moe_dispatch_gemm(ctx, toks, lg, bs, s.top_k, s.expert_begin, w, topk, offs, segt, x, y,
                                             opts=o))
    return s, offsets, calls


def cpu_baseline(budget_s: float = 12.0):
    """The fp64 oracle on the headline workload, repeated for about budget_s seconds."""
    import oracle
    import workloads as wl
    s = wl.AG_MLP
    d = wl.gen_ag(s, run=0)
    threads = os.cpu_count()
    try:
        from threadpoolctl import threadpool_info
        info = [x for x in threadpool_info() if x.get("user_api") == "blas"]
        if info:
            threads = int(info[0]["num_threads"])
    except Exception:
        pass
    reps, t_total = 0, 0.0
    while t_total < budget_s and reps < 1000:
        t0 = time.perf_counter()
        oracle.ag_gemm(d["a_shards"], d["b"])
        t_total += time.perf_counter() - t0
        reps += 1
    t = t_total / reps
    return {"value": s.flops / t / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"full AG+GEMM workload (W=8, M=8192, N=1792, K=4096) in fp64, {reps} repetitions, "
                      f"{t:.2f} s each"}


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
            _, calls = setup_ag(ctx, a.only == "ag_resident", identity=a.only == "ag_identity")
        elif a.only in ("rs", "ar"):
            _, calls = setup_reduce(ctx, a.only)
        elif a.only in ("rs_emulated", "ar_emulated"):
            _, calls = setup_reduce(ctx, a.only[:2], emulated=True)
        elif a.only == "moe":
            _, _, calls = setup_moe(ctx)
        elif a.only == "copy":
            # calibration for the HBM byte counters: a plain device copy of 256 MiB per launch
            src = torch.empty(64 << 20, dtype=torch.float32, device="cuda").fill_(1.0)
            dst = torch.empty_like(src)
            calls = [lambda: dst.copy_(src)]
        else:
            raise SystemExit(f"unknown --only {a.only}")
        wall, kern = time_calls(calls, a.steps, a.warmup)
        st = ctx.status()
        print(json.dumps({"only": a.only, "ms_per_step": wall, "kernel_ms": kern, "status": st}), flush=True)
        return

    s, calls = setup_ag(ctx, resident=False)
    wall, kern = time_calls(calls, a.steps, a.warmup)
    status = ctx.status()
    if status != mk.MK_OK:
        raise SystemExit(f"device status {status}: {mk.strerror(status)}")
    value = s.flops / (wall * 1e-3) / 1e12
    achieved = s.flops / (kern * 1e-3) / 1e12
    result = {
        "metric": "fused AG+GEMM TFLOP/s on 1 MI355X and % of bf16 MFMA peak; RS/AR epilogue GB/s",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(wall, 5),
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
                     "traffic_unit": "HBM bytes per launch", "algorithmic_bytes": ag_algorithmic_bytes(s)},
    }
    traffic = measured_traffic()
    if traffic is not None:
        result["roofline"]["traffic"] = round(traffic)
    if not a.no_secondary:
        sec = {}
        _, calls_r = setup_ag(ctx, resident=True)
        w_r, k_r = time_calls(calls_r, 30, 3)
        sec["ag_resident"] = {"kernel_ms": round(k_r, 5), "tflops": round(s.flops / (k_r * 1e-3) / 1e12, 2),
                              "fused_slowdown": round(kern / k_r - 1.0, 4)}
        del calls_r
        for op in ("rs", "ar"):
            sh, cr = setup_reduce(ctx, op)
            w_, k_ = time_calls(cr, 30, 3)
            rows = sh.m_slice if op == "rs" else sh.m
            epi = (sh.world - 1) * rows * sh.n * 4 + rows * sh.n * 4 + (
                (sh.world - 1) * sh.m_slice * sh.n * 4 if op == "rs" else 0)
            total = epi + sh.m * sh.k * 2 + sh.k * sh.n * 2
            sec[op] = {"kernel_ms": round(k_, 5), "tflops": round(sh.flops / (k_ * 1e-3) / 1e12, 2),
                       "epilogue_GBs": round(epi / (k_ * 1e-3) / 1e9, 1),
                       "total_GBs": round(total / (k_ * 1e-3) / 1e9, 1),
                       "hbm_frac": round(total / (k_ * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
            del cr
            torch.cuda.empty_cache()
        sm, offs, cm = setup_moe(ctx)
        w_, k_ = time_calls(cm, 20, 2)
        R = int(offs[0][-1].item())  # routed rows, as the kernel computed them
        sec["moe"] = {"kernel_ms": round(k_, 5), "routed_rows": R, "tflops": round(sm.flops(R) / (k_ * 1e-3) / 1e12, 2)}
        del cm
        st = ctx.status()
        if st != mk.MK_OK:
            raise SystemExit(f"device status {st}: {mk.strerror(st)}")
        result["secondary"] = sec
    if not a.no_cpu:
        result["cpu_baseline"] = cpu_baseline()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
