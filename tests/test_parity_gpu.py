"""HIP path vs the fp64 oracle, through the C ABI.

Every output buffer is compared element by element: the small workloads (several tiles plus a
ragged tail) and the full-size workloads in the launch configuration bench.py times, where the
fp64 oracle computes the whole buffer (ring attention: every query of two heads).  The float
tolerance is max |out - ref| <= 1e-3 * RMS(ref) with the RMS over the whole output buffer.
Integer-valued inputs make every fp32 sum exact, so those cases must be bit-identical to the
oracle whatever the arrival order.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ctx():
    import communication_gemm_role_amd as mk
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    c = mk.Context(0)
    yield c
    torch.cuda.synchronize()
    c.close()


def _mk():
    import communication_gemm_role_amd as mk
    return mk


# ----------------------------------------------------------------------------------------------
# AllGather + GEMM
# ----------------------------------------------------------------------------------------------
def _run_ag(ctx, shape, data, order=None, mode=None, in_place=True, poison=False, n_copy=0, **extra):
    from gpu_util import dev_bf16, dev_i32
    mk = _mk()
    W, r = shape.world, shape.rank
    b = dev_bf16(data["b"])
    ag = torch.empty((shape.m, shape.k), dtype=torch.bfloat16, device="cuda")
    if poison:
        ag.view(torch.int16).fill_(0x7FC0)  # bf16 quiet NaN: anything read before it lands shows up
    c = torch.full((shape.m, shape.n), float("nan"), dtype=torch.float32, device="cuda")
    shards = [dev_bf16(s) for s in data["a_shards"]]
    if mode == mk.MK_ARRIVAL_RESIDENT:
        ag.copy_(torch.cat(shards, 0))
    elif in_place:
        ag[r * shape.m_shard:(r + 1) * shape.m_shard].copy_(shards[r])
        shards[r] = ag[r * shape.m_shard:(r + 1) * shape.m_shard]
    opts = mk.Opts(arrival_mode=mode or 0, arrival_unit_rows=shape.unit_rows, arrival_unit_cols=shape.unit_cols,
                   arrival_order=dev_i32(order) if order is not None else None, n_copy_wg=n_copy, **extra)
    mk.mk_ag_gemm(ctx, shards, W, r, b, ag, c, opts=opts)
    assert ctx.status() == mk.MK_OK
    return ag, c


@pytest.mark.parametrize("kind", ["normal", "int"])
@pytest.mark.parametrize("variant,trial", [("flat", 0), ("flat", 1), ("flat", 2), ("flat", 3), ("flat", 4),
                                           ("identity", 0), ("reversed", 0), ("shard", 0)])
def test_ag_tiny(ctx, kind, variant, trial):
    from gpu_util import assert_close, assert_exact, host, host_bits
    s = wl.AG_TINY
    d = wl.gen_ag(s, run=0, kind=kind)
    order = wl.ag_arrival_order(s, trial=trial, variant=variant)
    ag, c = _run_ag(ctx, s, d, order=order, poison=True)
    a_ref, c_ref = oracle.ag_gemm(d["a_shards"], d["b"])
    assert_exact(host_bits(ag), a_ref, "a_gathered")
    if kind == "int":
        assert_exact(host(c), c_ref.astype(np.float32), "C (integer inputs)")
    else:
        assert_close(host(c), c_ref, "C")


def test_ag_tiny_resident_matches_emulated(ctx):
    from gpu_util import assert_exact, host
    mk = _mk()
    s = wl.AG_TINY
    d = wl.gen_ag(s, run=2, kind="int")
    _, c1 = _run_ag(ctx, s, d, mode=mk.MK_ARRIVAL_RESIDENT)
    _, c2 = _run_ag(ctx, s, d, order=wl.ag_arrival_order(s, trial=7))
    assert_exact(host(c1), host(c2), "resident vs emulated")


@pytest.mark.parametrize("in_place", [True, False])
@pytest.mark.parametrize("rank", [0, 2])
def test_ag_ragged(ctx, in_place, rank):
    """Several 256x256 tiles with ragged M and N tails, 64x64 units, local shard copied or in place."""
    from gpu_util import assert_close, assert_exact, host, host_bits
    s = wl.AGShape(world=3, m_shard=192, k=320, n=448, sigma_a=1.0, sigma_b=0.05, unit_rows=64, unit_cols=64,
                   rank=rank, cfg=wl.CFG_AG_TINY)
    d = wl.gen_ag(s, run=5)
    units = wl.ag_peer_units(s, rank)
    if not in_place:  # the local shard is copied like a peer's: its units join the order
        spr = s.m_shard // s.unit_rows
        local = [ur * s.n_unit_cols + uc for ur in range(rank * spr, (rank + 1) * spr) for uc in range(s.n_unit_cols)]
        units = np.concatenate([units, np.asarray(local, np.int32)])
    order = units[np.random.default_rng(11).permutation(len(units))].astype(np.int32)
    ag, c = _run_ag(ctx, s, d, order=order, in_place=in_place, poison=True)
    a_ref, c_ref = oracle.ag_gemm(d["a_shards"], d["b"])
    assert_exact(host_bits(ag), a_ref, "a_gathered")
    assert_close(host(c), c_ref, "C")


def test_ag_identity_order_default(ctx):
    """arrival_order NULL = identity order."""
    from gpu_util import assert_close, host
    s = wl.AG_TINY
    d = wl.gen_ag(s, run=1)
    _, c = _run_ag(ctx, s, d, order=None)
    assert_close(host(c), oracle.ag_gemm(d["a_shards"], d["b"])[1], "C")


@pytest.mark.parametrize("mode", ["emulated", "resident"])
def test_ag_full(ctx, mode):
    """The full AllGather+GEMM workload (W=8, M=8192, N=1792, K=4096), bench launch configuration;
    every element of C against the fp64 oracle."""
    from gpu_util import assert_close, assert_exact, host, host_bits, log
    mk = _mk()
    s = wl.AG_MLP
    d = wl.gen_ag(s, run=0)
    log(f"ag full {mode}: launching")
    m = mk.MK_ARRIVAL_EMULATED if mode == "emulated" else mk.MK_ARRIVAL_RESIDENT
    ag, c = _run_ag(ctx, s, d, order=wl.ag_arrival_order(s, trial=0) if mode == "emulated" else None, mode=m)
    torch.cuda.synchronize()
    a_ref, c_ref = oracle.ag_gemm(d["a_shards"], d["b"])
    assert_exact(host_bits(ag), a_ref, "a_gathered")
    assert_close(host(c), c_ref, "C")


def test_ag_full_integer_order_invariant(ctx):
    """Integer inputs at full size: emulated (two orders) and resident results are bit-identical."""
    from gpu_util import assert_exact, host
    mk = _mk()
    s = wl.AG_MLP
    d = wl.gen_ag(s, run=1, kind="int")
    _, c0 = _run_ag(ctx, s, d, mode=mk.MK_ARRIVAL_RESIDENT)
    _, c1 = _run_ag(ctx, s, d, order=wl.ag_arrival_order(s, trial=1))
    _, c2 = _run_ag(ctx, s, d, order=wl.ag_arrival_order(s, trial=2, variant="shard"))
    h0 = host(c0)
    assert_exact(host(c1), h0, "emulated order 1 vs resident")
    assert_exact(host(c2), h0, "emulated shard order vs resident")
    _, c_ref = oracle.ag_gemm(d["a_shards"], d["b"])
    assert_exact(h0, c_ref.astype(np.float32), "C (integer)")


# ----------------------------------------------------------------------------------------------
# GEMM + ReduceScatter / AllReduce
# ----------------------------------------------------------------------------------------------
def _run_red(ctx, op, shape, data, mode, order=None, n_reduce=0, n_copy=0, **extra):
    from gpu_util import dev_bf16, dev_f32, dev_i32
    mk = _mk()
    W, r = shape.world, shape.rank
    a, b = dev_bf16(data["a"]), dev_bf16(data["b"])
    peers = [None if p is None else dev_f32(p) for p in data["peers"]]
    opts = mk.Opts(arrival_mode=mode, n_reduce_wg=n_reduce, n_copy_wg=n_copy,
                   arrival_unit_rows=shape.unit_rows, arrival_unit_cols=shape.unit_cols,
                   arrival_order=dev_i32(order) if order is not None else None, **extra)
    if op == "rs":
        own = torch.full((shape.m_slice, shape.n), float("nan"), device="cuda")
        outbox = [None if j == r else torch.full((shape.m_slice, shape.n), float("nan"), device="cuda")
                  for j in range(W)]
        mk.mk_gemm_rs(ctx, a, b, W, r, peers, own, outbox, opts=opts)
        assert ctx.status() == mk.MK_OK
        return own, outbox
    out = torch.full((shape.m, shape.n), float("nan"), device="cuda")
    mk.mk_gemm_ar(ctx, a, b, W, r, peers, out, opts=opts)
    assert ctx.status() == mk.MK_OK
    return out, None


RED_CASES = [("resident", 0), ("resident", 16), ("emulated", 0), ("emulated", 16)]


@pytest.mark.parametrize("mode,n_reduce", RED_CASES)
@pytest.mark.parametrize("rank", [0, 3])
@pytest.mark.parametrize("kind", ["normal", "int"])
def test_rs_small(ctx, mode, n_reduce, rank, kind):
    from gpu_util import assert_close, assert_exact, host
    mk = _mk()
    s = wl.replace(wl.RS_SMALL, rank=rank)
    d = wl.gen_reduce(s, "rs", run=0, kind=kind)
    em = mode == "emulated"
    order = wl.reduce_arrival_order(s, "rs", trial=rank) if em else None
    own, outbox = _run_red(ctx, "rs", s, d, mk.MK_ARRIVAL_EMULATED if em else mk.MK_ARRIVAL_RESIDENT, order, n_reduce)
    own_ref, ob_ref = oracle.gemm_rs(d["a"], d["b"], d["peers"], s.world, rank)
    check = (lambda o, r_, w: assert_exact(o, r_.astype(np.float32), w)) if kind == "int" else assert_close
    check(host(own), own_ref, "owned slice")
    for j in range(s.world):
        if j != rank:
            check(host(outbox[j]), ob_ref[j], f"outbox[{j}]")


@pytest.mark.parametrize("mode,n_reduce", RED_CASES)
@pytest.mark.parametrize("rank", [0, 5])
@pytest.mark.parametrize("kind", ["normal", "int"])
def test_ar_small(ctx, mode, n_reduce, rank, kind):
    from gpu_util import assert_close, assert_exact, host
    mk = _mk()
    s = wl.replace(wl.AR_SMALL, rank=rank)
    d = wl.gen_reduce(s, "ar", run=0, kind=kind)
    em = mode == "emulated"
    order = wl.reduce_arrival_order(s, "ar", trial=rank, variant="reversed" if rank else "flat") if em else None
    out, _ = _run_red(ctx, "ar", s, d, mk.MK_ARRIVAL_EMULATED if em else mk.MK_ARRIVAL_RESIDENT, order, n_reduce)
    ref = oracle.gemm_ar(d["a"], d["b"], d["peers"], s.world, rank)
    if kind == "int":
        assert_exact(host(out), ref.astype(np.float32), "AR out")
    else:
        assert_close(host(out), ref, "AR out")


@pytest.mark.parametrize("world,rank,m,n,k", [(2, 1, 256, 2048, 192), (5, 3, 192, 1600, 576), (3, 2, 384, 960, 320),
                                               (8, 6, 128, 640, 128), (8, 0, 512, 8192, 256)])
def test_ar_resident_world_and_tile_counts(ctx, world, rank, m, n, k):
    """Resident AllReduce on the decode-like tile at other world sizes and tile counts.  The split
    workgroups' peer-streaming waves take 2 (world 2), 8 (world 5) and 4 (world 3) peer halves
    against 3, 9 and 5 k-steps, and 14 halves against 2 k-steps (world 8, k = 128: the loop runs on
    for the peers after the K loop ends); 512 tiles on the 256 workgroups use the role kernel with
    leftover claims.  Integer inputs, so every sum is exact."""
    from gpu_util import assert_exact, host, log
    mk = _mk()
    s = wl.RedShape(m=m, n=n, k=k, world=world, rank=rank, unit_rows=64, unit_cols=64, cfg=wl.CFG_AR)
    d = wl.gen_reduce(s, "ar", run=2, kind="int")
    log(f"ar resident world={world} rank={rank} m={m} n={n} k={k}: launching")
    out, _ = _run_red(ctx, "ar", s, d, mk.MK_ARRIVAL_RESIDENT)
    ref = oracle.gemm_ar(d["a"], d["b"], d["peers"], s.world, rank)
    assert_exact(host(out), ref.astype(np.float32), "AR out")


@pytest.mark.parametrize("mode", ["resident", "emulated"])
def test_rs_full(ctx, mode):
    """The full down-projection GEMM + ReduceScatter (A 8192x1792, B 1792x4096, 7 peer partials),
    bench launch configuration: the owned slice and every outbox against the fp64 oracle."""
    from gpu_util import assert_close, host, log
    mk = _mk()
    s = wl.RS_DOWN
    d = wl.gen_reduce(s, "rs", run=0)
    em = mode == "emulated"
    log(f"rs full {mode}: launching")
    own, outbox = _run_red(ctx, "rs", s, d, mk.MK_ARRIVAL_EMULATED if em else mk.MK_ARRIVAL_RESIDENT,
                           wl.reduce_arrival_order(s, "rs") if em else None)
    own_ref, ob_ref = oracle.gemm_rs(d["a"], d["b"], d["peers"], s.world, 0)
    assert_close(host(own), own_ref, "owned slice")
    for j in range(1, s.world):
        assert_close(host(outbox[j]), ob_ref[j], f"outbox[{j}]")


@pytest.mark.parametrize("mode", ["resident", "emulated"])
def test_ar_full(ctx, mode):
    """The full decode-like GEMM + AllReduce (A 256x1024, B 1024x8192, 7 peer partials), bench
    launch configuration: every output element against the fp64 oracle."""
    from gpu_util import assert_close, host, log
    mk = _mk()
    s = wl.AR_DECODE
    d = wl.gen_reduce(s, "ar", run=0)
    em = mode == "emulated"
    log(f"ar full {mode}: launching")
    out, _ = _run_red(ctx, "ar", s, d, mk.MK_ARRIVAL_EMULATED if em else mk.MK_ARRIVAL_RESIDENT,
                      wl.reduce_arrival_order(s, "ar") if em else None)
    ref = oracle.gemm_ar(d["a"], d["b"], d["peers"], s.world, 0)
    assert_close(host(out), ref, "AR out")


# ----------------------------------------------------------------------------------------------
# MoE dispatch + grouped GEMM
# ----------------------------------------------------------------------------------------------
def _run_moe(ctx, shape, data, order=None, mode=None, cap=None, **extra):
    from gpu_util import dev_bf16, dev_f32, dev_i32
    mk = _mk()
    cap = shape.capacity if cap is None else cap
    toks = [dev_bf16(t) for t in data["tokens"]]
    topk = torch.full((shape.tokens, shape.top_k), -7, dtype=torch.int32, device="cuda")
    offs = torch.full((shape.n_local + 1,), -7, dtype=torch.int32, device="cuda")
    segt = torch.full((cap,), -7, dtype=torch.int32, device="cuda")
    x = torch.zeros((cap, shape.hidden), dtype=torch.bfloat16, device="cuda")
    y = torch.full((cap, shape.ffn), float("nan"), device="cuda")
    opts = mk.Opts(arrival_mode=mode or 0, arrival_order=dev_i32(order) if order is not None else None, **extra)
    mk.mk_moe_dispatch_gemm(ctx, toks, dev_f32(data["logits"]), dev_f32(data["bias"]), shape.top_k,
                            shape.expert_begin, dev_bf16(data["w_up"]), topk, offs, segt, x, y, opts=opts)
    st = ctx.status()
    return st, topk, offs, segt, x, y


@pytest.mark.parametrize("kind", ["normal", "int"])
@pytest.mark.parametrize("variant,trial", [("flat", 0), ("flat", 1), ("flat", 2), ("identity", 0), ("reversed", 0)])
def test_moe_small(ctx, kind, variant, trial):
    from gpu_util import assert_close, assert_exact, host, host_bits
    mk = _mk()
    s = wl.MOE_SMALL
    d = wl.gen_moe(s, run=0, kind=kind)
    st, topk, offs, segt, x, y = _run_moe(ctx, s, d, order=wl.moe_arrival_order(s, trial, variant))
    assert st == mk.MK_OK
    ref = oracle.moe_dispatch_gemm(d["tokens"], d["logits"], d["bias"], s.top_k, s.expert_begin, s.n_local, d["w_up"])
    R = int(ref["seg_offsets"][-1])
    assert_exact(host(topk), ref["topk_idx"], "topk_idx")
    assert_exact(host(offs), ref["seg_offsets"], "seg_offsets")
    assert_exact(host(segt)[:R], ref["seg_token"], "seg_token")
    assert_exact(host_bits(x)[:R], ref["x_seg"], "x_seg")
    if kind == "int":
        assert_exact(host(y)[:R], ref["y"].astype(np.float32), "y (integer)")
    else:
        assert_close(host(y)[:R], ref["y"], "y")


@pytest.mark.parametrize("n_copy", [1, 2, 8, 40, 248])
def test_moe_row_split_role_splits(ctx, n_copy):
    """The dispatch splits the routed rows evenly over the copy workgroups: with 1 or 2 a workgroup's
    rows span all 24 chunks or half of them, in several listing windows of 8 chunks, with 248 a
    workgroup moves a few rows of one or two chunks; bit-exact layout and integer-exact grouped GEMM
    either way."""
    from gpu_util import assert_exact, host, host_bits, log
    mk = _mk()
    s = wl.MOE_SMALL
    d = wl.gen_moe(s, run=3, kind="int")
    log(f"moe row split n_copy={n_copy}: launching")
    st, topk, offs, segt, x, y = _run_moe(ctx, s, d, order=wl.moe_arrival_order(s, 4, "flat"), n_copy_wg=n_copy)
    assert st == mk.MK_OK
    ref = oracle.moe_dispatch_gemm(d["tokens"], d["logits"], d["bias"], s.top_k, s.expert_begin, s.n_local, d["w_up"])
    R = int(ref["seg_offsets"][-1])
    assert_exact(host(offs), ref["seg_offsets"], "seg_offsets")
    assert_exact(host(segt)[:R], ref["seg_token"], "seg_token")
    assert_exact(host_bits(x)[:R], ref["x_seg"], "x_seg")
    assert_exact(host(y)[:R], ref["y"].astype(np.float32), "y (integer)")


@pytest.mark.parametrize("case", ["twelve_local_experts", "1032_chunks"])
def test_moe_scan_wide(ctx, case):
    """The scan's general paths: more local experts than waves (each wave scans several experts),
    and more chunks than one load group or one pass of the arrival-order scan holds (the counts are
    reloaded per pass and the order's rows are taken in several groups); bit-exact layout and
    integer-exact grouped GEMM."""
    from dataclasses import replace
    from gpu_util import assert_exact, host, host_bits, log
    mk = _mk()
    if case == "twelve_local_experts":
        s = replace(wl.MOE_SMALL, n_experts=24, expert_begin=6, n_local=12)
    else:
        s = replace(wl.MOE_SMALL, t_local=8256, hidden=64, ffn=64)
    assert (s.n_local > 8) or (s.n_chunks > 1024)
    d = wl.gen_moe(s, run=5, kind="int")
    log(f"moe scan {case}: n_local={s.n_local} n_chunks={s.n_chunks}: launching")
    st, topk, offs, segt, x, y = _run_moe(ctx, s, d, order=wl.moe_arrival_order(s, 2, "flat"))
    assert st == mk.MK_OK
    ref = oracle.moe_dispatch_gemm(d["tokens"], d["logits"], d["bias"], s.top_k, s.expert_begin, s.n_local, d["w_up"])
    R = int(ref["seg_offsets"][-1])
    assert_exact(host(topk), ref["topk_idx"], "topk_idx")
    assert_exact(host(offs), ref["seg_offsets"], "seg_offsets")
    assert_exact(host(segt)[:R], ref["seg_token"], "seg_token")
    assert_exact(host_bits(x)[:R], ref["x_seg"], "x_seg")
    assert_exact(host(y)[:R], ref["y"].astype(np.float32), "y (integer)")


def test_moe_forced_routing(ctx):
    """Huge bias on experts 0 and 1: every token lands in both segments; the other local experts are empty."""
    from gpu_util import assert_close, assert_exact, host
    mk = _mk()
    s = wl.MOE_SMALL
    bias = np.zeros(s.n_experts, np.float32)
    bias[:2] = 1e4
    d = wl.gen_moe(s, run=1, bias_override=bias)
    st, topk, offs, segt, x, y = _run_moe(ctx, s, d)
    assert st == mk.MK_OK
    T = s.tokens
    assert_exact(host(offs), np.array([0, T, 2 * T] + [2 * T] * (s.n_local - 2), np.int32), "seg_offsets")
    ref = oracle.moe_dispatch_gemm(d["tokens"], d["logits"], d["bias"], s.top_k, s.expert_begin, s.n_local, d["w_up"])
    assert_exact(host(segt), ref["seg_token"], "seg_token")
    assert_close(host(y), ref["y"], "y")


def test_moe_no_local_rows(ctx):
    mk = _mk()
    from gpu_util import assert_exact, host
    s = wl.MOE_SMALL
    bias = np.zeros(s.n_experts, np.float32)
    bias[:s.n_local] = -1e4
    d = wl.gen_moe(s, run=1, bias_override=bias)
    st, topk, offs, segt, x, y = _run_moe(ctx, s, d)
    assert st == mk.MK_OK
    assert_exact(host(offs), np.zeros(s.n_local + 1, np.int32), "seg_offsets")
    assert np.isnan(host(y)).all()  # nothing written


def test_moe_full(ctx):
    """The full MoE workload (8 ranks x 4096 tokens, hidden 4096, 64 experts, top-2, experts 0..7
    local with W_up 4096x1536), bench launch configuration: routing, layout and every routed row of
    x_seg bit-exact, every element of y[:R] against the fp64 oracle."""
    from gpu_util import assert_close, assert_exact, host, host_bits, log
    mk = _mk()
    s = wl.MOE_FULL
    d = wl.gen_moe(s, run=0)
    log("moe full: launching")
    st, topk, offs, segt, x, y = _run_moe(ctx, s, d, order=wl.moe_arrival_order(s, 0))
    assert st == mk.MK_OK
    ref = oracle.moe_dispatch_gemm(d["tokens"], d["logits"], d["bias"], s.top_k, s.expert_begin, s.n_local, d["w_up"])
    R = int(ref["seg_offsets"][-1])
    log(f"moe full: R = {R}, n_e = {np.diff(ref['seg_offsets']).tolist()}")
    assert_exact(host(topk), ref["topk_idx"], "topk_idx")
    assert_exact(host(offs), ref["seg_offsets"], "seg_offsets")
    assert_exact(host(segt)[:R], ref["seg_token"], "seg_token")
    assert_exact(host_bits(x)[:R], ref["x_seg"], "x_seg")
    assert_close(host(y)[:R], ref["y"], "y")


# ----------------------------------------------------------------------------------------------
# faults forced from the host
# ----------------------------------------------------------------------------------------------
def test_dropped_unit_times_out_then_reset(ctx):
    from gpu_util import assert_close, dev_bf16, dev_i32, host
    mk = _mk()
    s = wl.AG_TINY
    d = wl.gen_ag(s, run=0)
    order = wl.ag_arrival_order(s, trial=0)
    b = dev_bf16(d["b"])
    ag = torch.zeros((s.m, s.k), dtype=torch.bfloat16, device="cuda")
    c = torch.zeros((s.m, s.n), device="cuda")
    shards = [dev_bf16(x) for x in d["a_shards"]]
    ag[:s.m_shard].copy_(shards[0])
    shards[0] = ag[:s.m_shard]
    opts = mk.Opts(arrival_order=dev_i32(order), test_drop_unit=5, timeout_us=20000)
    mk.mk_ag_gemm(ctx, shards, s.world, 0, b, ag, c, opts=opts)
    assert ctx.status() == mk.MK_ERR_TIMEOUT
    ctx.reset()
    assert ctx.status() == mk.MK_OK
    mk.mk_ag_gemm(ctx, shards, s.world, 0, b, ag, c, opts=mk.Opts(arrival_order=dev_i32(order)))
    assert ctx.status() == mk.MK_OK
    assert_close(host(c), oracle.ag_gemm(d["a_shards"], d["b"])[1], "C after reset")


def test_rs_dropped_unit_times_out(ctx):
    mk = _mk()
    s = wl.RS_SMALL
    d = wl.gen_reduce(s, "rs", run=0)
    from gpu_util import dev_bf16, dev_f32
    a, b = dev_bf16(d["a"]), dev_bf16(d["b"])
    peers = [None if p is None else dev_f32(p) for p in d["peers"]]
    own = torch.zeros((s.m_slice, s.n), device="cuda")
    ob = [None] + [torch.zeros((s.m_slice, s.n), device="cuda") for _ in range(1, s.world)]
    opts = mk.Opts(test_drop_unit=3, timeout_us=20000, arrival_unit_rows=64, arrival_unit_cols=64)
    mk.mk_gemm_rs(ctx, a, b, s.world, 0, peers, own, ob, opts=opts)
    assert ctx.status() == mk.MK_ERR_TIMEOUT
    ctx.reset()


def test_moe_capacity_overflow(ctx):
    mk = _mk()
    s = wl.MOE_SMALL
    d = wl.gen_moe(s, run=0)
    ref = oracle.moe_dispatch_gemm(d["tokens"], d["logits"], d["bias"], s.top_k, s.expert_begin, s.n_local, d["w_up"])
    R = int(ref["seg_offsets"][-1])
    st, topk, offs, segt, x, y = _run_moe(ctx, s, d, cap=R // 2 // 64 * 64)
    assert st == mk.MK_ERR_CAPACITY
    from gpu_util import assert_exact, host
    assert_exact(host(offs), ref["seg_offsets"], "seg_offsets still exact")
    ctx.reset()


def test_calls_do_not_leak_state(ctx):
    """Back-to-back calls of different ops on one context: epoch-tagged flags need no clearing,
    and the counters each kernel uses (leftover tiles, RS pre-sum bands, MoE, the MLP block's H
    row counts) are left zeroed, so a call never sees a previous call's counts (integer inputs:
    any stale pre-sum would show)."""
    from gpu_util import assert_close, assert_exact, host
    mk = _mk()
    s = wl.AG_TINY
    d = wl.gen_ag(s, run=3)
    sr = wl.RS_SMALL
    for t in range(3):
        _, c = _run_ag(ctx, s, d, order=wl.ag_arrival_order(s, trial=t))
        assert_close(host(c), oracle.ag_gemm(d["a_shards"], d["b"])[1], f"C call {t}")
        dr = wl.gen_reduce(sr, "rs", run=t, kind="int")
        own, _ = _run_red(ctx, "rs", sr, dr, mk.MK_ARRIVAL_RESIDENT)
        own_ref, _ = oracle.gemm_rs(dr["a"], dr["b"], dr["peers"], sr.world, sr.rank)
        assert_exact(host(own), own_ref.astype(np.float32), f"RS owned slice call {t}")
        sm = wl.MOE_SMALL
        dm = wl.gen_moe(sm, run=t)
        st, *_ = _run_moe(ctx, sm, dm)
        assert st == mk.MK_OK
        sl = wl.replace(wl.MLP_SMALL, rank=t)
        dl = wl.gen_mlp(sl, run=t, kind="int")
        _, _, own, _ = _run_mlp(ctx, sl, dl, wl.ag_arrival_order(sl.ag, trial=t))
        ref = oracle.mlp_ag_rs(dl["a_shards"], dl["b_up"], dl["b_down"], dl["peers"], sl.world, t)
        assert_exact(host(own), ref["own"].astype(np.float32), f"MLP owned slice call {t}")
        sa = wl.replace(wl.RING_SMALL, rank=t)
        da = wl.gen_ring(sa, run=t)
        st, out, *_ = _run_ring(ctx, sa, da, wl.ring_arrival_order(sa, trial=t, variant="flat"))
        assert st == mk.MK_OK
        assert_close(host(out), oracle.ring_attention(da["q"], da["k_shards"], da["v_shards"])[0], f"ring call {t}")


def test_full_moe_leaves_no_counter_behind():
    """A fresh context, no reset between calls: the full MoE call writes its per-chunk tables and
    m-tile counters over the range that the RS band counters and the MLP row-block counters also
    use, so it must leave all of them at zero.  Then a smaller MoE call (whose m-tile counters fall
    inside the previous call's per-chunk tables), the MLP block and the RS pre-sum must still be
    bit-exact on integer inputs: any stale count would let a tile run before its data is ready."""
    from gpu_util import assert_exact, host, host_bits, log
    mk = _mk()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    c = mk.Context(0)
    try:
        s = wl.MOE_FULL
        d = wl.gen_moe(s, run=0)
        log("moe full then small, mlp, rs on one context: launching")
        st, *_ = _run_moe(c, s, d, order=wl.moe_arrival_order(s, 0))
        assert st == mk.MK_OK
        sm = wl.MOE_SMALL
        dm = wl.gen_moe(sm, run=2, kind="int")
        st, topk, offs, segt, x, y = _run_moe(c, sm, dm, order=wl.moe_arrival_order(sm, 1, "flat"))
        assert st == mk.MK_OK
        ref = oracle.moe_dispatch_gemm(dm["tokens"], dm["logits"], dm["bias"], sm.top_k, sm.expert_begin, sm.n_local,
                                       dm["w_up"])
        R = int(ref["seg_offsets"][-1])
        assert_exact(host(offs), ref["seg_offsets"], "seg_offsets (second MoE call)")
        assert_exact(host_bits(x)[:R], ref["x_seg"], "x_seg (second MoE call)")
        assert_exact(host(y)[:R], ref["y"].astype(np.float32), "y (second MoE call, integer)")
        sl = wl.replace(wl.MLP_SMALL, rank=1)
        dl = wl.gen_mlp(sl, run=4, kind="int")
        _, h, own, _ = _run_mlp(c, sl, dl, wl.ag_arrival_order(sl.ag, trial=2))
        mref = oracle.mlp_ag_rs(dl["a_shards"], dl["b_up"], dl["b_down"], dl["peers"], sl.world, 1)
        assert_exact(host_bits(h), oracle.bf16_bits(mref["h"]), "MLP H after MoE (integer)")
        assert_exact(host(own), mref["own"].astype(np.float32), "MLP owned slice after MoE (integer)")
        sr = wl.RS_SMALL
        dr = wl.gen_reduce(sr, "rs", run=6, kind="int")
        own, outbox = _run_red(c, "rs", sr, dr, mk.MK_ARRIVAL_RESIDENT)
        own_ref, ob_ref = oracle.gemm_rs(dr["a"], dr["b"], dr["peers"], sr.world, sr.rank)
        assert_exact(host(own), own_ref.astype(np.float32), "RS owned slice after MoE (integer)")
        for j in range(sr.world):
            if j != sr.rank:
                assert_exact(host(outbox[j]), ob_ref[j].astype(np.float32), f"RS outbox[{j}] after MoE (integer)")
    finally:
        torch.cuda.synchronize()
        c.close()


# ----------------------------------------------------------------------------------------------
# MLP block: AllGather + up-projection, gelu, down-projection + ReduceScatter in one launch
# ----------------------------------------------------------------------------------------------
def _run_mlp(ctx, shape, data, order=None, mode=None, **extra):
    from gpu_util import dev_bf16, dev_f32, dev_i32
    mk = _mk()
    W, r, ms = shape.world, shape.rank, shape.m_shard
    shards = [dev_bf16(s) for s in data["a_shards"]]
    ag = torch.empty((shape.m, shape.k), dtype=torch.bfloat16, device="cuda")
    ag.view(torch.int16).fill_(0x7FC0)
    h = torch.empty((shape.m, shape.n_up), dtype=torch.bfloat16, device="cuda")
    h.view(torch.int16).fill_(0x7FC0)
    if mode == mk.MK_ARRIVAL_RESIDENT:
        ag.copy_(torch.cat(shards, 0))
    else:
        ag[r * ms:(r + 1) * ms].copy_(shards[r])
        shards[r] = ag[r * ms:(r + 1) * ms]
    peers = [None if p is None else dev_f32(p) for p in data["peers"]]
    own = torch.full((ms, shape.n_out), float("nan"), device="cuda")
    outbox = [None if j == r else torch.full((ms, shape.n_out), float("nan"), device="cuda") for j in range(W)]
    opts = mk.Opts(arrival_mode=mode or 0, arrival_unit_rows=shape.unit_rows, arrival_unit_cols=shape.unit_cols,
                   arrival_order=dev_i32(order) if order is not None else None, **extra)
    mk.mk_mlp_ag_rs(ctx, shards, W, r, dev_bf16(data["b_up"]), dev_bf16(data["b_down"]), peers, ag, h, own, outbox,
                    opts=opts)
    assert ctx.status() == mk.MK_OK
    return ag, h, own, outbox


GELU_LIP = 1.13  # max |gelu'(x)| = Phi(x) + x phi(x), reached near x = 1.41 (1.1289...)


def _assert_h(h_bits, h_ref, u_ref, what, max_frac=1e-2):
    """H is bf16(gelu_f32(U_gpu)) on the GPU, with U_gpu the fp32 up-projection, and the bf16 rounding
    of fp64 gelu(fp64 U) in the oracle.  U_gpu is an fp32 GEMM output, so it is held to the same rule
    as every fp32 output: |U_gpu - U| <= TOL * RMS(U).  gelu moves that by at most GELU_LIP times as
    much, and the two roundings by at most one bf16 step of the larger value, so
        |H - H_ref| <= step(max(|H|, |H_ref|)) + GELU_LIP * TOL * RMS(U)
    for every element.  In practice U_gpu is far closer than TOL: the two differ by one step only
    where gelu(U) lies within fp32 error of a rounding boundary, so at most max_frac of the elements
    may differ at all.  Returns |H - H_ref| for the down-projection's error budget."""
    from gpu_util import TOL, log
    out = oracle.bf16_to_f64(h_bits)
    ref = np.asarray(h_ref, np.float64)
    assert not np.isnan(out).any(), f"{what}: NaN (an element never written)"
    diff = np.abs(out - ref)
    mag = np.maximum(np.abs(ref), np.abs(out))
    step = np.where(mag > 0, np.exp2(np.floor(np.log2(np.where(mag > 0, mag, 1.0))) - 7), 0.0)
    slack = GELU_LIP * TOL * oracle.rms(u_ref)
    bad = diff > step + slack
    assert not bad.any(), f"{what}: {bad.sum()} elements beyond one bf16 step + {slack:.3e}, first at " \
                          f"{np.argwhere(bad)[0].tolist()}"
    frac = float(np.mean(diff > 0))
    assert frac <= max_frac, f"{what}: {frac:.3%} of elements differ"
    over = diff > step
    log(f"{what}: {frac:.4%} of elements differ from the oracle's; {int(over.sum())} by more than one step "
        f"(largest excess {float(np.max(diff - step)) if over.any() else 0.0:.3e}, allowed {slack:.3e})")
    return diff


def _assert_close_down(out, ref, dh, b_down, what):
    """Down-projection output against the oracle's.  The oracle's value is the expected one; the
    budget is the GEMM tolerance plus the linear effect of the H differences that _assert_h has
    bounded to one bf16 step each: |out - ref| <= TOL * RMS(ref) + |H - H_ref| @ |B_down|."""
    from gpu_util import TOL
    out = np.asarray(out, np.float64)
    assert not np.isnan(out).any(), f"{what}: NaN in output"
    prop = dh @ np.abs(oracle.bf16_to_f64(b_down))
    excess = np.abs(out - ref) - (TOL * oracle.rms(ref) + prop)
    assert (excess <= 0).all(), (f"{what}: {int((excess > 0).sum())} elements beyond the budget, worst by "
                                 f"{excess.max():.3e} at {np.unravel_index(np.argmax(excess), excess.shape)}")


@pytest.mark.parametrize("mode", ["emulated", "resident"])
@pytest.mark.parametrize("rank", [0, 2])
def test_mlp_small(ctx, mode, rank):
    """Several tiles with ragged N tails in both GEMMs (n_up 448, n_out 320), 64x64 units."""
    from gpu_util import assert_exact, host, host_bits
    mk = _mk()
    s = wl.replace(wl.MLP_SMALL, rank=rank)
    d = wl.gen_mlp(s, run=rank)
    em = mode == "emulated"
    order = wl.ag_arrival_order(s.ag, trial=rank) if em else None
    ag, h, own, outbox = _run_mlp(ctx, s, d, order, mk.MK_ARRIVAL_EMULATED if em else mk.MK_ARRIVAL_RESIDENT)
    ref = oracle.mlp_ag_rs(d["a_shards"], d["b_up"], d["b_down"], d["peers"], s.world, rank)
    assert_exact(host_bits(ag), ref["a_gathered"], "a_gathered")
    dh = _assert_h(host_bits(h), ref["h"], ref["u"], "H")
    ms = s.m_shard
    _assert_close_down(host(own), ref["own"], dh[rank * ms:(rank + 1) * ms], d["b_down"], "owned slice")
    for j in range(s.world):
        if j != rank:
            _assert_close_down(host(outbox[j]), ref["outbox"][j], dh[j * ms:(j + 1) * ms], d["b_down"],
                               f"outbox[{j}]")


@pytest.mark.parametrize("mode", ["emulated", "resident"])
def test_mlp_small_integer(ctx, mode):
    """Integer inputs: every up-projection output is 0 or a multiple of 16, where gelu is the
    identity in fp32 as in fp64, so H and every reduced output are exact."""
    from gpu_util import assert_exact, host, host_bits
    mk = _mk()
    s = wl.replace(wl.MLP_SMALL, rank=1)
    d = wl.gen_mlp(s, run=3, kind="int")
    em = mode == "emulated"
    order = wl.ag_arrival_order(s.ag, trial=5, variant="reversed") if em else None
    _, h, own, outbox = _run_mlp(ctx, s, d, order, mk.MK_ARRIVAL_EMULATED if em else mk.MK_ARRIVAL_RESIDENT)
    ref = oracle.mlp_ag_rs(d["a_shards"], d["b_up"], d["b_down"], d["peers"], s.world, 1)
    assert_exact(host_bits(h), oracle.bf16_bits(ref["h"]), "H (integer)")
    assert_exact(host(own), ref["own"].astype(np.float32), "owned slice (integer)")
    for j in (0, 2, 3):
        assert_exact(host(outbox[j]), ref["outbox"][j].astype(np.float32), f"outbox[{j}] (integer)")


@pytest.mark.parametrize("mode", ["emulated", "resident"])
def test_mlp_full(ctx, mode):
    """The full block (W=8, 1024-row shards, K 4096, n_up 1792, n_out 4096), bench launch
    configuration: every element of H, the owned slice and every outbox against the fp64 oracle."""
    from gpu_util import assert_exact, host, host_bits, log
    mk = _mk()
    s = wl.MLP_FULL
    d = wl.gen_mlp(s, run=0)
    em = mode == "emulated"
    log(f"mlp full {mode}: launching")
    ag, h, own, outbox = _run_mlp(ctx, s, d, wl.ag_arrival_order(s.ag, trial=0) if em else None,
                                  mk.MK_ARRIVAL_EMULATED if em else mk.MK_ARRIVAL_RESIDENT)
    torch.cuda.synchronize()
    ref = oracle.mlp_ag_rs(d["a_shards"], d["b_up"], d["b_down"], d["peers"], s.world, 0)
    assert_exact(host_bits(ag), ref["a_gathered"], "a_gathered")
    dh = _assert_h(host_bits(h), ref["h"], ref["u"], "H")
    ms = s.m_shard
    _assert_close_down(host(own), ref["own"], dh[:ms], d["b_down"], "owned slice")
    for j in range(1, s.world):
        _assert_close_down(host(outbox[j]), ref["outbox"][j], dh[j * ms:(j + 1) * ms], d["b_down"], f"outbox[{j}]")


# ----------------------------------------------------------------------------------------------
# Link-rate pacing (mk_opts.arrival_gbps): results unchanged, units land no faster than the rate
# ----------------------------------------------------------------------------------------------
def _trace_buf(ctx):
    return torch.full((ctx.grid * 8,), -1, dtype=torch.int64, device="cuda")


def _landing_us(tr):
    """Wall-clock span from the first workgroup's start to the last copy workgroup's last flag."""
    r = tr.cpu().numpy().reshape(-1, 8)
    r = r[r[:, 0] != -1]
    cp = r[r[:, 4] == 0]
    return (cp[:, 5].max() - r[:, 0].min()) / 100.0


def _min_landing_us(n_order, unit_bytes, gbps):
    # arrival position i is not copied before i * unit_bytes / rate (the last one is n_order - 1)
    return (n_order - 1) * unit_bytes / (gbps * 1e9) * 1e6


def test_ag_paced(ctx):
    from gpu_util import assert_exact, host, host_bits
    s = wl.AG_TINY
    d = wl.gen_ag(s, run=4, kind="int")
    order = wl.ag_arrival_order(s, trial=3)
    tr = _trace_buf(ctx)
    gbps = 2.0
    ag, c = _run_ag(ctx, s, d, order=order, poison=True, arrival_gbps=gbps, trace=tr)
    a_ref, c_ref = oracle.ag_gemm(d["a_shards"], d["b"])
    assert_exact(host_bits(ag), a_ref, "a_gathered (paced)")
    assert_exact(host(c), c_ref.astype(np.float32), "C (paced, integer inputs)")
    need = _min_landing_us(len(order), s.unit_rows * s.unit_cols * 2, gbps)
    got = _landing_us(tr)
    assert got >= 0.95 * need, f"units landed in {got:.1f} us, the rate allows no less than {need:.1f} us"


@pytest.mark.parametrize("op", ["rs", "ar"])
def test_reduce_paced(ctx, op):
    from gpu_util import assert_exact, host
    mk = _mk()
    s = wl.RS_SMALL if op == "rs" else wl.AR_SMALL
    d = wl.gen_reduce(s, op, run=5, kind="int")
    order = wl.reduce_arrival_order(s, op, trial=2)
    tr = _trace_buf(ctx)
    gbps = 20.0
    out, outbox = _run_red(ctx, op, s, d, mk.MK_ARRIVAL_EMULATED, order, arrival_gbps=gbps, trace=tr)
    if op == "rs":
        own_ref, ob_ref = oracle.gemm_rs(d["a"], d["b"], d["peers"], s.world, s.rank)
        assert_exact(host(out), own_ref.astype(np.float32), "RS owned slice (paced)")
        for j in range(1, s.world):
            assert_exact(host(outbox[j]), ob_ref[j].astype(np.float32), f"RS outbox[{j}] (paced)")
    else:
        ref = oracle.gemm_ar(d["a"], d["b"], d["peers"], s.world, s.rank)
        assert_exact(host(out), ref.astype(np.float32), "AR out (paced)")
    need = _min_landing_us(len(order), s.unit_rows * s.unit_cols * 4, gbps)
    got = _landing_us(tr)
    assert got >= 0.95 * need, f"units landed in {got:.1f} us, the rate allows no less than {need:.1f} us"


def test_mlp_paced(ctx):
    from gpu_util import assert_exact, host, host_bits
    s = wl.replace(wl.MLP_SMALL, rank=3)
    d = wl.gen_mlp(s, run=6, kind="int")
    _, h, own, _ = _run_mlp(ctx, s, d, wl.ag_arrival_order(s.ag, trial=4), arrival_gbps=5.0)
    ref = oracle.mlp_ag_rs(d["a_shards"], d["b_up"], d["b_down"], d["peers"], s.world, 3)
    assert_exact(host_bits(h), oracle.bf16_bits(ref["h"]), "H (paced, integer)")
    assert_exact(host(own), ref["own"].astype(np.float32), "owned slice (paced, integer)")


def test_ag_full_at_link_rate(ctx):
    """The full AllGather+GEMM at the MI355X's 7 x 153 GB/s of xGMI: sampled rows, landing span."""
    from gpu_util import assert_close, assert_exact, host, host_bits, log
    mk = _mk()
    s = wl.AG_MLP
    d = wl.gen_ag(s, run=0)
    order = wl.ag_arrival_order(s, trial=0)
    tr = _trace_buf(ctx)
    log("ag full at link rate: launching")
    ag, c = _run_ag(ctx, s, d, order=order, mode=mk.MK_ARRIVAL_EMULATED, arrival_gbps=1071.0, trace=tr)
    torch.cuda.synchronize()
    a_ref, c_ref = oracle.ag_gemm(d["a_shards"], d["b"])
    assert_exact(host_bits(ag), a_ref, "a_gathered")
    assert_close(host(c), c_ref, "C (link rate)")
    need = _min_landing_us(len(order), s.unit_rows * s.unit_cols * 2, 1071.0)
    got = _landing_us(tr)
    assert got >= 0.95 * need, f"units landed in {got:.1f} us, the rate allows no less than {need:.1f} us"


# ----------------------------------------------------------------------------------------------
# Role-split tuning: every candidate is timed, rejected splits report -1, results stay exact
# ----------------------------------------------------------------------------------------------
def test_ag_tune(ctx):
    from gpu_util import assert_exact, dev_bf16, dev_i32, host
    mk = _mk()
    s = wl.AG_TINY
    d = wl.gen_ag(s, run=7, kind="int")
    b = dev_bf16(d["b"])
    shards = [dev_bf16(x) for x in d["a_shards"]]
    ag = torch.empty((s.m, s.k), dtype=torch.bfloat16, device="cuda")
    ag[:s.m_shard].copy_(shards[0])  # the local shard in place (rank 0), as the order assumes
    shards[0] = ag[:s.m_shard]
    c = torch.empty((s.m, s.n), dtype=torch.float32, device="cuda")
    opts = mk.Opts(arrival_mode=mk.MK_ARRIVAL_EMULATED, arrival_order=dev_i32(wl.ag_arrival_order(s, trial=1)),
                   arrival_unit_rows=s.unit_rows, arrival_unit_cols=s.unit_cols, arrival_gbps=50.0)
    cands = [4, 16, 100000, 64, 0]
    best, us = mk.mk_ag_gemm_tune(ctx, shards, s.world, s.rank, b, ag, c, cands, reps=5, opts=opts)
    assert us[2] == -1.0, "a split beyond the grid is rejected"
    assert all(u > 0 for i, u in enumerate(us) if i != 2)
    assert best in (4, 16, 64, 0) and us[cands.index(best)] == min(u for u in us if u > 0)
    assert_exact(host(c), oracle.ag_gemm(d["a_shards"], d["b"])[1].astype(np.float32), "C after tuning")
    with pytest.raises(mk.MkError):
        mk.mk_ag_gemm_tune(ctx, shards, s.world, s.rank, b, ag, c, [100000, 200000], reps=2, opts=opts)


@pytest.mark.parametrize("op", ["rs", "ar"])
def test_reduce_tune(ctx, op):
    from gpu_util import assert_exact, dev_bf16, dev_f32, dev_i32, host
    mk = _mk()
    s = wl.RS_SMALL if op == "rs" else wl.AR_SMALL
    d = wl.gen_reduce(s, op, run=8, kind="int")
    a, b = dev_bf16(d["a"]), dev_bf16(d["b"])
    peers = [None if p is None else dev_f32(p) for p in d["peers"]]
    opts = mk.Opts(arrival_mode=mk.MK_ARRIVAL_EMULATED, arrival_order=dev_i32(wl.reduce_arrival_order(s, op)),
                   arrival_unit_rows=s.unit_rows, arrival_unit_cols=s.unit_cols)
    cands = [8, 64, 0, 192]
    if op == "rs":
        own = torch.empty((s.m_slice, s.n), device="cuda")
        ob = [None] + [torch.empty((s.m_slice, s.n), device="cuda") for _ in range(1, s.world)]
        best, us = mk.mk_gemm_rs_tune(ctx, a, b, s.world, 0, peers, own, ob, cands, reps=5, opts=opts)
        own_ref, _ = oracle.gemm_rs(d["a"], d["b"], d["peers"], s.world, 0)
        assert_exact(host(own), own_ref.astype(np.float32), "RS owned slice after tuning")
    else:
        out = torch.empty((s.m, s.n), device="cuda")
        best, us = mk.mk_gemm_ar_tune(ctx, a, b, s.world, 0, peers, out, cands, reps=5, opts=opts)
        ref = oracle.gemm_ar(d["a"], d["b"], d["peers"], s.world, 0)
        assert_exact(host(out), ref.astype(np.float32), "AR out after tuning")
    assert all(u > 0 for u in us) and best == cands[int(np.argmin(us))]


# ----------------------------------------------------------------------------------------------
# Ring attention: one rank's share, peers' K/V blocks landing in ring order (or any order)
# ----------------------------------------------------------------------------------------------
def _run_ring(ctx, shape, data, order=None, mode=None, lse=True, **extra):
    from gpu_util import dev_bf16, dev_i32
    mk = _mk()
    W, H, S, D = shape.world, shape.heads, shape.s_local, shape.d
    q = dev_bf16(data["q"])
    ks = [dev_bf16(k) for k in data["k_shards"]]
    vs = [dev_bf16(v) for v in data["v_shards"]]
    out = torch.full((H, S, D), float("nan"), device="cuda")
    ls = torch.full((H, S), float("nan"), device="cuda") if lse else None
    kr = torch.empty((W, H, S, D), dtype=torch.bfloat16, device="cuda")
    vr = torch.empty((W, H, S, D), dtype=torch.bfloat16, device="cuda")
    kr.view(torch.int16).fill_(0x7FC0)
    vr.view(torch.int16).fill_(0x7FC0)
    opts = mk.Opts(arrival_mode=mode or 0, arrival_order=dev_i32(order) if order is not None else None, **extra)
    mk.mk_ring_attention(ctx, q, ks, vs, shape.rank, out, ls, kr, vr, opts=opts)
    st = ctx.status()
    return st, out, ls, kr, vr


@pytest.mark.parametrize("mode,variant", [("emulated", "ring"), ("emulated", "flat"), ("emulated", "reversed"),
                                          ("resident", None)])
def test_ring_small(ctx, mode, variant):
    """Several query tiles and key blocks per head (world 4, 2 heads, 256 tokens per rank)."""
    from gpu_util import assert_close, assert_exact, host, host_bits
    mk = _mk()
    s = wl.RING_SMALL
    d = wl.gen_ring(s, run=1)
    em = mode == "emulated"
    order = wl.ring_arrival_order(s, trial=3, variant=variant) if em else None
    st, out, lse, kr, vr = _run_ring(ctx, s, d, order, mk.MK_ARRIVAL_EMULATED if em else mk.MK_ARRIVAL_RESIDENT)
    assert st == mk.MK_OK
    ref, lref = oracle.ring_attention(d["q"], d["k_shards"], d["v_shards"])
    assert_close(host(out), ref, "out")
    assert_close(host(lse), lref, "lse")
    if em:  # every peer shard landed bit for bit; the own slot is never written
        for j in range(s.world):
            if j != s.rank:
                assert_exact(host_bits(kr[j]), d["k_shards"][j], f"k_ring[{j}]")
                assert_exact(host_bits(vr[j]), d["v_shards"][j], f"v_ring[{j}]")
        assert (host_bits(kr[s.rank]) == 0x7FC0).all()


@pytest.mark.parametrize("n_copy", [8, 64, 248])
def test_ring_role_splits(ctx, n_copy):
    """32 items (8 heads x 4 query tiles) dealt to the XCDs in blocks of 4: with 248 copy workgroups
    one item per XCD is static and three are claimed from the XCD's counter, with 64 or 8 every
    item is static and the spare workgroups find nothing to claim; every split gives the oracle's
    result."""
    from gpu_util import assert_close, host, log
    mk = _mk()
    s = wl.RingShape(world=4, heads=8, s_local=512, rank=2)
    d = wl.gen_ring(s, run=4)
    log(f"ring role split n_copy={n_copy}: launching")
    st, out, lse, _, _ = _run_ring(ctx, s, d, wl.ring_arrival_order(s, trial=1, variant="flat"), mk.MK_ARRIVAL_EMULATED,
                                   n_copy_wg=n_copy)
    assert st == mk.MK_OK
    ref, lref = oracle.ring_attention(d["q"], d["k_shards"], d["v_shards"])
    assert_close(host(out), ref, "out")
    assert_close(host(lse), lref, "lse")


def test_ring_scale_and_no_lse(ctx):
    from gpu_util import assert_close, host
    mk = _mk()
    s = wl.replace(wl.RING_SMALL, rank=3)
    d = wl.gen_ring(s, run=2)
    from gpu_util import dev_bf16
    st, out, _, _, _ = _run_ring(ctx, s, d, None, mk.MK_ARRIVAL_EMULATED, lse=False)
    assert st == mk.MK_OK
    assert_close(host(out), oracle.ring_attention(d["q"], d["k_shards"], d["v_shards"])[0], "out (no lse)")
    q, ks, vs = dev_bf16(d["q"]), [dev_bf16(k) for k in d["k_shards"]], [dev_bf16(v) for v in d["v_shards"]]
    out2 = torch.empty_like(out)
    mk.mk_ring_attention(ctx, q, ks, vs, s.rank, out2, None, None, None, softmax_scale=0.3,
                         opts=mk.Opts(arrival_mode=mk.MK_ARRIVAL_RESIDENT))
    assert ctx.status() == mk.MK_OK
    assert_close(host(out2), oracle.ring_attention(d["q"], d["k_shards"], d["v_shards"], scale=0.3)[0], "out (scale)")


@pytest.mark.parametrize("mode", ["emulated", "resident"])
def test_ring_full(ctx, mode):
    """8 ranks x 4096 tokens, 8 heads of 128, bench launch configuration: every query of heads 0
    and 5 (head 5 is served by copy workgroups' leftover items in ring order) against the fp64
    oracle, which treats each query on its own, so it is run on 1024 queries at a time."""
    from gpu_util import assert_close, host, log
    mk = _mk()
    s = wl.RING_FULL
    d = wl.gen_ring(s, run=0)
    em = mode == "emulated"
    log(f"ring full {mode}: launching")
    st, out, lse, _, _ = _run_ring(ctx, s, d, wl.ring_arrival_order(s) if em else None,
                                   mk.MK_ARRIVAL_EMULATED if em else mk.MK_ARRIVAL_RESIDENT)
    assert st == mk.MK_OK
    oh, lh = host(out), host(lse)
    for h in (0, 5):
        ks = [k[h:h + 1] for k in d["k_shards"]]
        vs = [v[h:h + 1] for v in d["v_shards"]]
        parts = [oracle.ring_attention(d["q"][h:h + 1, i:i + 1024], ks, vs) for i in range(0, s.s_local, 1024)]
        ref = np.concatenate([p[0] for p in parts], axis=1)
        lref = np.concatenate([p[1] for p in parts], axis=1)
        assert_close(oh[h:h + 1], ref, f"out head {h}")
        assert_close(lh[h:h + 1], lref, f"lse head {h}")


def test_ring_paced(ctx):
    from gpu_util import assert_close, host
    mk = _mk()
    s = wl.RING_SMALL
    d = wl.gen_ring(s, run=3)
    tr = _trace_buf(ctx)
    gbps = 20.0
    order = wl.ring_arrival_order(s)
    st, out, _, _, _ = _run_ring(ctx, s, d, order, mk.MK_ARRIVAL_EMULATED, arrival_gbps=gbps, trace=tr)
    assert st == mk.MK_OK
    assert_close(host(out), oracle.ring_attention(d["q"], d["k_shards"], d["v_shards"])[0], "out (paced)")
    need = _min_landing_us(len(order), 64 * 128 * 2, gbps)
    got = _landing_us(tr)
    assert got >= 0.95 * need, f"blocks landed in {got:.1f} us, the rate allows no less than {need:.1f} us"


def test_ring_dropped_block_times_out(ctx):
    """A block that never lands: the items waiting for it time out, the status says so, and the
    context works again after a reset."""
    from gpu_util import assert_close, host
    mk = _mk()
    s = wl.RING_SMALL
    d = wl.gen_ring(s, run=4)
    st, *_ = _run_ring(ctx, s, d, wl.ring_arrival_order(s), mk.MK_ARRIVAL_EMULATED, timeout_us=20000, test_drop_unit=5)
    assert st == mk.MK_ERR_TIMEOUT
    ctx.reset()
    st, out, *_ = _run_ring(ctx, s, d, wl.ring_arrival_order(s), mk.MK_ARRIVAL_EMULATED)
    assert st == mk.MK_OK
    assert_close(host(out), oracle.ring_attention(d["q"], d["k_shards"], d["v_shards"])[0], "out after reset")
