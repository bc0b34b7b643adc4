"""Per-workgroup trace records (mk_opts.trace), through the C ABI.

Tracing must not change results (integer-valued inputs make every sum exact, so the outputs
must be identical with and without it), and every record must be ordered: start <= phase
marks <= end, in wall-clock ticks and in shader cycles.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

UNTOUCHED = -1  # records of workgroups the call does not launch keep the fill value


@pytest.fixture(scope="module")
def ctx():
    import communication_gemm_role_amd as mk
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    c = mk.Context(0)
    yield c
    torch.cuda.synchronize()
    c.close()


def _trace(ctx):
    return torch.full((ctx.grid * 8,), UNTOUCHED, dtype=torch.int64, device="cuda")


def _records(tr):
    r = tr.cpu().numpy().reshape(-1, 8)
    return r[r[:, 0] != UNTOUCHED]


def _check_ordered(rec, marks):
    assert len(rec) > 0, "no workgroup wrote a record"
    assert np.all(rec[:, 0] > 0) and np.all(rec[:, 2] >= rec[:, 0]), "end before start"
    assert np.all(rec[:, 3] >= rec[:, 1]), "shader cycles went backwards"
    assert set(np.unique(rec[:, 4])) <= {0, 1, 2}, "unknown role"
    for role, slots in marks.items():
        sel = rec[rec[:, 4] == role]
        prev = sel[:, 0]
        for s in slots:
            m = sel[:, s]
            hit = m != 0
            assert np.all(m[hit] >= prev[hit]) and np.all(m[hit] <= sel[hit, 2]), f"role {role} mark {s} out of order"
            prev = np.where(hit, m, prev)


def test_trace_ag_tiny(ctx):
    import communication_gemm_role_amd as mk
    from gpu_util import assert_exact, dev_bf16, dev_i32, host
    s = wl.AG_TINY
    d = wl.gen_ag(s, run=0, kind="int")
    order = dev_i32(wl.ag_arrival_order(s, trial=0))
    outs = []
    for traced in (False, True):
        b = dev_bf16(d["b"])
        shards = [dev_bf16(x) for x in d["a_shards"]]
        ag = torch.empty((s.m, s.k), dtype=torch.bfloat16, device="cuda")
        ag[:s.m_shard].copy_(shards[0])
        shards[0] = ag[:s.m_shard]
        c = torch.full((s.m, s.n), float("nan"), device="cuda")
        tr = _trace(ctx) if traced else None
        opts = mk.Opts(arrival_order=order, arrival_unit_rows=s.unit_rows, arrival_unit_cols=s.unit_cols, trace=tr)
        mk.mk_ag_gemm(ctx, shards, s.world, 0, b, ag, c, opts=opts)
        assert ctx.status() == mk.MK_OK
        outs.append(host(c))
        if traced:
            rec = _records(tr)
            _check_ordered(rec, {0: [5], 1: [5]})
            assert (rec[:, 4] == 0).sum() > 0 and (rec[:, 4] == 1).sum() > 0, "both roles ran"
            assert np.all(rec[rec[:, 4] == 0, 5] > 0), "every copy workgroup marks its end of copy"
    _, c_ref = oracle.ag_gemm(d["a_shards"], d["b"])
    assert_exact(outs[1], outs[0], "C with trace vs without")
    assert_exact(outs[1], c_ref.astype(np.float32), "C with trace vs oracle")


def test_trace_rs_small_with_reduce(ctx):
    import communication_gemm_role_amd as mk
    from gpu_util import assert_exact, dev_bf16, dev_f32, dev_i32, host
    s = wl.RS_SMALL
    d = wl.gen_reduce(s, "rs", run=0, kind="int")
    order = dev_i32(wl.reduce_arrival_order(s, "rs"))
    outs = []
    for traced in (False, True):
        a, b = dev_bf16(d["a"]), dev_bf16(d["b"])
        peers = [None if p is None else dev_f32(p) for p in d["peers"]]
        own = torch.full((s.m_slice, s.n), float("nan"), device="cuda")
        outbox = [None if j == s.rank else torch.full((s.m_slice, s.n), float("nan"), device="cuda")
                  for j in range(s.world)]
        tr = _trace(ctx) if traced else None
        opts = mk.Opts(arrival_mode=mk.MK_ARRIVAL_EMULATED, arrival_order=order, n_reduce_wg=16,
                       arrival_unit_rows=s.unit_rows, arrival_unit_cols=s.unit_cols, trace=tr)
        mk.mk_gemm_rs(ctx, a, b, s.world, s.rank, peers, own, outbox, opts=opts)
        assert ctx.status() == mk.MK_OK
        outs.append(host(own))
        if traced:
            rec = _records(tr)
            _check_ordered(rec, {0: [5], 1: [5, 6, 7], 2: [5]})
            assert set(np.unique(rec[:, 4])) == {0, 1, 2}, "copy, compute and reduce roles all ran"
    assert_exact(outs[1], outs[0], "owned slice with trace vs without")


def test_trace_moe_small(ctx):
    import communication_gemm_role_amd as mk
    from gpu_util import assert_exact, dev_bf16, dev_f32, dev_i32, host
    s = wl.MOE_SMALL
    d = wl.gen_moe(s, run=0, kind="int")
    order = dev_i32(wl.moe_arrival_order(s, 0))
    outs = []
    for traced in (False, True):
        toks = [dev_bf16(t) for t in d["tokens"]]
        topk = torch.empty((s.tokens, s.top_k), dtype=torch.int32, device="cuda")
        offs = torch.empty((s.n_local + 1,), dtype=torch.int32, device="cuda")
        segt = torch.empty((s.capacity,), dtype=torch.int32, device="cuda")
        x = torch.zeros((s.capacity, s.hidden), dtype=torch.bfloat16, device="cuda")
        y = torch.full((s.capacity, s.ffn), float("nan"), device="cuda")
        tr = _trace(ctx) if traced else None
        opts = mk.Opts(arrival_order=order, trace=tr)
        mk.mk_moe_dispatch_gemm(ctx, toks, dev_f32(d["logits"]), dev_f32(d["bias"]), s.top_k, s.expert_begin,
                                dev_bf16(d["w_up"]), topk, offs, segt, x, y, opts=opts)
        assert ctx.status() == mk.MK_OK
        R = int(host(offs)[-1])
        outs.append(host(y)[:R])
        if traced:
            rec = _records(tr)
            _check_ordered(rec, {0: [5, 6, 7], 1: [5]})
            cp = rec[rec[:, 4] == 0]
            assert np.all(cp[:, 5] > 0) and np.all(cp[:, 6] > 0) and np.all(cp[:, 7] > 0), "every copy mark set"
    assert_exact(outs[1], outs[0], "y with trace vs without")


def test_trace_too_small_is_rejected(ctx):
    import communication_gemm_role_amd as mk
    tr = torch.zeros((ctx.grid * 8 - 1,), dtype=torch.int64, device="cuda")
    with pytest.raises(ValueError):
        mk._opts_ptr(mk.Opts(trace=tr), ctx)
