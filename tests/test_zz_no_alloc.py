"""mk_ag_gemm_noalloc (AllGather + GEMM with its flags, counters and status word in a static device
array, no context and no allocation) against mk_ag_gemm on the same inputs, through the C ABI:
two calls in a row, the second on a smaller workload, then a forced timeout and recovery.

Integer-valued inputs make every fp32 sum exact, so C must be bit-identical to the context path's
whatever the arrival order; the gathered A is compared bit for bit; Gaussian inputs must agree with
the context path and with the fp64 oracle within 1e-3 * RMS."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

import oracle
import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _mk():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import communication_gemm_role_amd as mk
    return mk


def _setup(shape, data, in_place=True):
    from gpu_util import dev_bf16
    W, r = shape.world, shape.rank
    shards = [dev_bf16(s) for s in data["a_shards"]]
    ag = torch.empty((shape.m, shape.k), dtype=torch.bfloat16, device="cuda")
    ag.view(torch.int16).fill_(0x7FC0)  # bf16 NaN: a unit that never landed shows up
    if in_place:
        ag[r * shape.m_shard:(r + 1) * shape.m_shard].copy_(shards[r])
        shards[r] = ag[r * shape.m_shard:(r + 1) * shape.m_shard]
    c = torch.full((shape.m, shape.n), float("nan"), dtype=torch.float32, device="cuda")
    return shards, dev_bf16(data["b"]), ag, c


def _both(mk, ctx, shape, data, order, **extra):
    """The same call through mk_ag_gemm (context) and mk_ag_gemm_noalloc (static scratch)."""
    from gpu_util import dev_i32, host, host_bits
    opts = mk.Opts(arrival_unit_rows=shape.unit_rows, arrival_unit_cols=shape.unit_cols,
                   arrival_order=dev_i32(order), **extra)
    sh1, b1, ag1, c1 = _setup(shape, data)
    mk.mk_ag_gemm(ctx, sh1, shape.world, shape.rank, b1, ag1, c1, opts=opts)
    assert ctx.status() == mk.MK_OK
    sh2, b2, ag2, c2 = _setup(shape, data)
    st = torch.full((1,), -99, dtype=torch.int32, device="cuda")
    mk.mk_ag_gemm_noalloc(sh2, shape.world, shape.rank, b2, ag2, c2, st, opts=opts)
    torch.cuda.synchronize()
    assert int(st.item()) == mk.MK_OK, f"device status {int(st.item())}"
    return host_bits(ag1), host(c1), host_bits(ag2), host(c2)


def test_noalloc_matches_context_call_twice_then_smaller():
    """First the full AllGather+GEMM (W=8, 1024x4096 shards, B 4096x1792), then a smaller ragged one
    (W=3, 192x320 shards, B 320x448, 64x64 units): integer inputs bit-exact against the context
    path, Gaussian inputs within tolerance of it and of the oracle."""
    from gpu_util import assert_close, assert_exact, log
    mk = _mk()
    ctx = mk.Context(0)
    try:
        small = wl.AGShape(world=3, m_shard=192, k=320, n=448, sigma_a=1.0, sigma_b=0.05, unit_rows=64,
                           unit_cols=64, rank=1, cfg=wl.CFG_AG_TINY)
        for shape, trial in ((wl.AG_MLP, 0), (small, 3)):
            for kind in ("int", "normal"):
                log(f"noalloc: m={shape.m} n={shape.n} k={shape.k} {kind}: launching")
                d = wl.gen_ag(shape, run=1, kind=kind)
                units = wl.ag_peer_units(shape, shape.rank)
                order = units[np.random.default_rng(trial).permutation(len(units))].astype(np.int32)
                ag1, c1, ag2, c2 = _both(mk, ctx, shape, d, order)
                a_ref, c_ref = oracle.ag_gemm(d["a_shards"], d["b"])
                assert_exact(ag2, ag1, "a_gathered (noalloc vs context)")
                assert_exact(ag2, a_ref, "a_gathered (noalloc vs oracle)")
                if kind == "int":
                    assert_exact(c2, c1, "C (noalloc vs context, integer)")
                    assert_exact(c2, c_ref.astype(np.float32), "C (noalloc vs oracle, integer)")
                else:
                    assert_close(c2, c1.astype(np.float64), "C (noalloc vs context)")
                    assert_close(c2, c_ref, "C (noalloc vs oracle)")
    finally:
        torch.cuda.synchronize()
        ctx.close()


def test_noalloc_resident_mode():
    from gpu_util import assert_exact, dev_bf16, host
    mk = _mk()
    s = wl.AG_TINY
    d = wl.gen_ag(s, run=2, kind="int")
    ag = torch.cat([dev_bf16(x) for x in d["a_shards"]], 0)
    c = torch.full((s.m, s.n), float("nan"), device="cuda")
    st = torch.full((1,), -99, dtype=torch.int32, device="cuda")
    mk.mk_ag_gemm_noalloc(None, s.world, s.rank, dev_bf16(d["b"]), ag, c, st,
                          opts=mk.Opts(arrival_mode=mk.MK_ARRIVAL_RESIDENT))
    torch.cuda.synchronize()
    assert int(st.item()) == mk.MK_OK
    assert_exact(host(c), oracle.ag_gemm(d["a_shards"], d["b"])[1].astype(np.float32), "C (resident, integer)")


def test_noalloc_dropped_unit_reports_timeout_then_recovers():
    """A unit the copy role skips (forced from the host): the waiting tiles time out, the status
    output says so, and the next call on the same static array is exact again."""
    from gpu_util import assert_exact, dev_i32, host
    mk = _mk()
    s = wl.AG_TINY
    d = wl.gen_ag(s, run=3, kind="int")
    order = wl.ag_arrival_order(s, trial=2)
    sh, b, ag, c = _setup(s, d)
    st = torch.full((1,), -99, dtype=torch.int32, device="cuda")
    mk.mk_ag_gemm_noalloc(sh, s.world, s.rank, b, ag, c, st,
                          opts=mk.Opts(arrival_order=dev_i32(order), test_drop_unit=4, timeout_us=20000))
    torch.cuda.synchronize()
    assert int(st.item()) == mk.MK_ERR_TIMEOUT
    sh, b, ag, c = _setup(s, d)
    mk.mk_ag_gemm_noalloc(sh, s.world, s.rank, b, ag, c, st, opts=mk.Opts(arrival_order=dev_i32(order)))
    torch.cuda.synchronize()
    assert int(st.item()) == mk.MK_OK
    assert_exact(host(c), oracle.ag_gemm(d["a_shards"], d["b"])[1].astype(np.float32), "C after the timeout")


def test_noalloc_rejects_beyond_its_static_flags():
    """More arrival units than the 16384 static flags: MK_ERR_WORKSPACE, returned before any launch
    (the planner rejects it; no buffer is touched)."""
    mk = _mk()
    L = mk.lib()
    world, m_shard, k, n = 8, 4096, 4096, 256
    shards = (ctypes.c_void_p * world)(*[0x100000 * (j + 1) for j in range(world)])
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    o = mk.Opts(arrival_unit_rows=64, arrival_unit_cols=64).to_c()   # (32768/64) * (4096/64) = 32768 units
    rc = L.mk_ag_gemm_noalloc(None, shards, world, 0, m_shard, k, 0x200000, n, 0x300000, 0x400000, st.data_ptr(),
                              ctypes.byref(o))
    assert rc == mk.MK_ERR_WORKSPACE
    rc = L.mk_ag_gemm_noalloc(None, shards, world, 0, m_shard, k, 0x200000, n, 0x300000, 0x400000, None, None)
    assert rc == mk.MK_ERR_INVALID_ARG  # no status output
