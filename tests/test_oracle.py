"""The fp64 oracle against its pins (hand-worked examples, brute force, closed forms,
exact integer arithmetic and invariants).  CPU only."""
import numpy as np
import pytest

import oracle
import oracle_pins as P
import workloads as wl

IMPL = P.namespace_of(oracle)


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(IMPL)


def test_generator_bf16_rounding():
    g = P._golden("bf16_bits.json")
    for src, dst, _ in g["round_f32_bits"]:
        f = np.array([int(src, 16)], dtype=np.uint32).view(np.float32)
        assert int(wl.f32_to_bf16_bits(f)[0]) == int(dst, 16), src


def test_generator_is_seeded_and_shaped():
    a = wl.gen_ag(wl.AG_TINY, run=0)
    b = wl.gen_ag(wl.AG_TINY, run=0)
    c = wl.gen_ag(wl.AG_TINY, run=1)
    assert all(np.array_equal(x, y) for x, y in zip(a["a_shards"], b["a_shards"]))
    assert not np.array_equal(a["a_shards"][0], c["a_shards"][0])
    assert a["a_shards"][0].shape == (64, 256) and a["b"].shape == (256, 256)
    # sigma of B is 1/16 for the tiny workload
    sd = float(np.std(oracle.bf16_to_f64(a["b"])))
    assert 0.055 < sd < 0.07


def test_arrival_orders_are_permutations_of_peer_units():
    s = wl.AG_TINY
    units = set(wl.ag_peer_units(s).tolist())
    assert len(units) == 12  # 3 peers x (64/64 rows) x (256/64 cols)
    for variant in ("flat", "shard", "identity", "reversed"):
        o = wl.ag_arrival_order(s, trial=2, variant=variant)
        assert sorted(o.tolist()) == sorted(units)
    s2 = wl.AG_MLP
    o = wl.ag_arrival_order(s2, trial=0)
    assert len(o) == 1792 and len(set(o.tolist())) == 1792
    assert min(o) >= 8 * 32  # rank 0's own 8 unit rows x 32 unit cols stay in place
    m = wl.moe_arrival_order(wl.MOE_FULL)
    assert sorted(m.tolist()) == list(range(512))
    r = wl.reduce_arrival_order(wl.RS_DOWN, "rs")
    assert sorted(r.tolist()) == list(range(7 * 16 * 32))  # 7 peers x (1024 / 64) unit rows x (4096 / 128) unit cols


def test_tolerance_headroom_on_tiny_ag():
    # fp32 accumulation of the same products stays far inside 1e-3 * RMS
    d = wl.gen_ag(wl.AG_TINY, run=0)
    _, c = oracle.ag_gemm(d["a_shards"], d["b"])
    a32 = np.concatenate([oracle.bf16_to_f64(s) for s in d["a_shards"]]).astype(np.float32)
    b32 = oracle.bf16_to_f64(d["b"]).astype(np.float32)
    assert oracle.max_rel_err(a32 @ b32, c) < 1e-5
