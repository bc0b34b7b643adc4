"""C-ABI boundary checks that run without a GPU.

* libmk.so loads and exports every function include/mk.h declares (no compute calls);
* the entry points reject a NULL context synchronously;
* the host planning logic (argument validation, arrival-unit geometry, role split and
  workspace layout), built into libmk_host.so from the same header the GPU library
  uses, returns the documented codes and plans.
"""
from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mk.h")

MK_OK, INVALID, UNSUP, WS = 0, -1, -2, -3
RESIDENT, EMULATED = 1, 2


@pytest.fixture(scope="module")
def gpulib():
    from communication_gemm_role_amd import build as B
    if not os.path.exists(B.LIB):
        B.build_gpu_lib()
    return ctypes.CDLL(B.LIB)


@pytest.fixture(scope="module")
def hostlib():
    from communication_gemm_role_amd import build as B
    B.build_host_lib(sanitize=False)
    return ctypes.CDLL(B.HOSTLIB)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mk_\w+)\s*\(", text)))


def test_header_declares_the_four_ops():
    names = declared_functions()
    for op in ("mk_ag_gemm", "mk_gemm_rs", "mk_gemm_ar", "mk_moe_dispatch_gemm"):
        assert op in names


def test_library_exports_every_declared_symbol(gpulib):
    missing = [n for n in declared_functions() if not hasattr(gpulib, n)]
    assert not missing, f"not exported: {missing}"


def test_binding_names_match_header():
    import communication_gemm_role_amd as mk
    assert sorted(mk.EXPORTED) == declared_functions()
    for op in ("mk_ag_gemm", "mk_gemm_rs", "mk_gemm_ar", "mk_moe_dispatch_gemm"):
        assert callable(getattr(mk, op))


def declared_param_counts():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    out = {}
    for name, params in re.findall(r"\b(mk_\w+)\s*\(([^)]*)\)\s*;", text):
        params = params.strip()
        out[name] = 0 if params in ("", "void") else params.count(",") + 1
    return out


def test_binding_argument_counts_match_header(gpulib):
    """Every ctypes prototype the binding sets up has the header's number of parameters."""
    import communication_gemm_role_amd as mk
    L = mk.lib()
    counts = declared_param_counts()
    assert set(counts) == set(mk.EXPORTED)
    for name, n in counts.items():
        assert len(getattr(L, name).argtypes) == n, f"{name}: {len(getattr(L, name).argtypes)} argtypes, header has {n}"


def test_null_context_is_rejected_synchronously(gpulib):
    vp = ctypes.c_void_p
    gpulib.mk_strerror.restype = ctypes.c_char_p
    assert gpulib.mk_strerror(-5) == b"device wait timed out"
    assert gpulib.mk_ag_gemm(None, None, None, 8, 0, 64, 64, vp(16), 64, vp(16), vp(16), None) == INVALID
    assert gpulib.mk_gemm_rs(None, None, vp(16), vp(16), 64, 64, 64, 1, 0, None, vp(16), None, None) == INVALID
    assert gpulib.mk_gemm_ar(None, None, vp(16), vp(16), 64, 64, 64, 1, 0, None, vp(16), None) == INVALID
    assert gpulib.mk_ctx_destroy(None) == INVALID
    assert gpulib.mk_ctx_create(0, 0, None) == INVALID


# ---------------------------------------------------------------------------------------------
# host planning (libmk_host.so)
# ---------------------------------------------------------------------------------------------
class Opts(ctypes.Structure):
    _fields_ = [("n_copy_wg", ctypes.c_int), ("n_compute_wg", ctypes.c_int), ("n_reduce_wg", ctypes.c_int),
                ("arrival_mode", ctypes.c_int), ("arrival_order", ctypes.c_void_p), ("arrival_len", ctypes.c_int),
                ("arrival_unit_rows", ctypes.c_int), ("arrival_unit_cols", ctypes.c_int),
                ("arrival_chunk_tokens", ctypes.c_int), ("timeout_us", ctypes.c_int64),
                ("test_drop_unit", ctypes.c_int), ("arrival_gbps", ctypes.c_double)]


NF, NC, INBOX, GRID = 1 << 20, 1 << 20, 256 << 20, 256
P = lambda addr: ctypes.c_void_p(addr)  # fake device addresses: only alignment is inspected


def ag(hostlib, world=8, rank=0, m_shard=1024, k=4096, n=1792, shards="peers", opts=None, b=0x10000,
       ag_ptr=0x100000000, c=0x200000000):
    arr = (ctypes.c_void_p * max(world, 1))()
    for r in range(world):
        arr[r] = 0x300000000 + r * 0x10000000
    if shards == "inplace":
        arr[rank] = ag_ptr + rank * m_shard * k * 2
    elif shards == "none":
        arr = None
    out = (ctypes.c_longlong * 16)()
    code = hostlib.mkh_plan_ag(ctypes.c_size_t(NF), ctypes.c_size_t(NC), ctypes.c_size_t(INBOX), GRID,
                               ctypes.byref(opts) if opts else None, arr, world, rank, m_shard, k, P(b), n, P(ag_ptr),
                               P(c), 256, 256, out)
    keys = ["m", "unit_rows", "unit_cols", "n_urows", "n_ucols", "n_order", "local_in_place", "emulated", "drop_pos",
            "n_copy", "n_compute", "tiles_m", "tiles_n", "pace_q16"]
    return code, dict(zip(keys, list(out)))


def test_plan_ag_full_workload(hostlib):
    code, p = ag(hostlib)
    assert code == MK_OK
    assert (p["m"], p["unit_rows"], p["unit_cols"]) == (8192, 128, 128)
    assert p["n_order"] == 8 * 8 * 32 and p["local_in_place"] == 0  # shard 0 at another address: copied too
    code, p = ag(hostlib, shards="inplace")
    assert code == MK_OK and p["local_in_place"] == 1 and p["n_order"] == 7 * 8 * 32
    # unpaced: the compute role is as large as the local shard's 4 x 7 tiles, rounded up to whole
    # XCD rounds (32 workgroups, which take those tiles); every other workgroup copies first
    assert (p["n_copy"], p["n_compute"], p["tiles_m"], p["tiles_n"]) == (224, 32, 32, 7)
    code, p = ag(hostlib, shards="inplace", rank=5)
    assert code == MK_OK and (p["n_copy"], p["n_compute"]) == (224, 32)
    # no local shard in place: one round of 8 compute workgroups
    code, p = ag(hostlib)
    assert code == MK_OK and (p["n_copy"], p["n_compute"]) == (248, 8)
    # paced at a link rate: 160 copy workgroups
    code, p = ag(hostlib, shards="inplace", opts=Opts(arrival_gbps=1071.0))
    assert code == MK_OK and (p["n_copy"], p["n_compute"]) == (160, 96) and p["pace_q16"] > 0
    # resident: no copy role, and the compute role is cut to the 224 tiles (whole XCD rounds)
    code, p = ag(hostlib, shards="none", opts=Opts(arrival_mode=RESIDENT))
    assert code == MK_OK and (p["n_copy"], p["n_compute"]) == (0, 224)
    code, p = ag(hostlib, m_shard=64, world=3, rank=0, shards="none", opts=Opts(arrival_mode=RESIDENT))
    assert code == MK_OK and p["tiles_m"] == 1 and p["n_compute"] == 8
    code, p = ag(hostlib, shards="none", opts=Opts(arrival_mode=RESIDENT, n_compute_wg=250))
    assert code == MK_OK and p["n_compute"] == 250  # an explicit request is kept


def test_plan_ag_errors(hostlib):
    assert ag(hostlib, world=0)[0] == INVALID
    assert ag(hostlib, world=9)[0] == INVALID
    assert ag(hostlib, rank=8)[0] == INVALID
    assert ag(hostlib, m_shard=100)[0] == UNSUP
    assert ag(hostlib, n=1800)[0] == UNSUP
    assert ag(hostlib, b=0x10008)[0] == UNSUP  # misaligned
    assert ag(hostlib, b=0)[0] == INVALID
    assert ag(hostlib, shards="none")[0] == INVALID  # emulated needs shards
    o = Opts(arrival_mode=RESIDENT)
    assert ag(hostlib, shards="none", opts=o)[0] == MK_OK
    o = Opts(arrival_mode=7)
    assert ag(hostlib, opts=o)[0] == INVALID
    o = Opts(arrival_unit_rows=96)
    assert ag(hostlib, opts=o)[0] == UNSUP
    o = Opts(arrival_order=0x5000, arrival_len=5)
    assert ag(hostlib, opts=o)[0] == INVALID  # wrong order length
    o = Opts(arrival_order=0x5000, arrival_len=7 * 8 * 32)
    assert ag(hostlib, shards="inplace", opts=o)[0] == MK_OK
    assert ag(hostlib, k=64 * 128 + 128)[0] == UNSUP  # more than 64 K-units
    o = Opts(n_copy_wg=250)
    assert ag(hostlib, opts=o)[0] == UNSUP  # fewer than 8 compute workgroups left


def test_plan_ag_small_units(hostlib):
    code, p = ag(hostlib, world=4, m_shard=64, k=256, n=256, shards="inplace")
    assert code == MK_OK and (p["unit_rows"], p["unit_cols"], p["n_order"]) == (64, 64, 12)


def red(hostlib, is_rs=1, m=8192, n=4096, k=1792, world=8, rank=0, opts=None, tile=(256, 256, 8, 4), drop_peer=None,
        a=0x10000, inbox=INBOX):
    peers = (ctypes.c_void_p * world)()
    ob = (ctypes.c_void_p * world)()
    for j in range(world):
        if j != rank and j != drop_peer:
            peers[j] = 0x400000000 + j * 0x10000000
            ob[j] = 0x500000000 + j * 0x10000000
    out = (ctypes.c_longlong * 24)()
    code = hostlib.mkh_plan_reduce(ctypes.c_size_t(NF), ctypes.c_size_t(NC), ctypes.c_size_t(inbox), GRID,
                                   ctypes.byref(opts) if opts else None, is_rs, P(a), P(0x20000), m, n, k, world,
                                   rank, peers, P(0x30000), ob, tile[0], tile[1], tile[2], tile[3], out)
    keys = ["m_slice", "p_rows", "unit_rows", "unit_cols", "n_ucols", "units_per_peer", "n_units", "emulated",
            "n_order", "drop_pos", "n_copy", "n_reduce", "n_compute", "tiles_m", "tiles_n", "own_tile_begin",
            "own_tile_end", "inbox_need", "assist", "pace_q16"]
    return code, dict(zip(keys, list(out)))


def test_plan_rs_and_ar(hostlib):
    code, p = red(hostlib)
    assert code == MK_OK
    # the wide tile's copy ring moves 4 KiB per wave and batch (32 KiB slots): 64x128 fp32 units
    assert (p["unit_rows"], p["unit_cols"]) == (64, 128)
    assert (p["m_slice"], p["units_per_peer"], p["n_units"]) == (1024, 16 * 32, 7 * 512)
    assert (p["own_tile_begin"], p["own_tile_end"], p["inbox_need"]) == (0, 4, 7 * 1024 * 4096 * 4)
    code, p = red(hostlib, rank=3)
    assert (p["own_tile_begin"], p["own_tile_end"]) == (12, 16)
    # the skinny AR tile has 4 waves: 8 KiB per wave caps a unit at 32 KiB, so 64x128 by default
    code, p = red(hostlib, is_rs=0, m=256, n=8192, k=1024, tile=(128, 64, 4, 8))
    assert code == MK_OK and p["p_rows"] == 256 and (p["unit_rows"], p["unit_cols"]) == (64, 128)
    assert p["n_units"] == 7 * 4 * 64
    assert (p["own_tile_begin"], p["own_tile_end"]) == (0, 2)
    assert red(hostlib, is_rs=0, m=256, n=8192, k=1024, tile=(128, 64, 4, 8),
               opts=Opts(arrival_unit_rows=128, arrival_unit_cols=128))[0] == UNSUP
    assert red(hostlib, tile=(256, 256, 0, 4))[0] == INVALID
    assert red(hostlib, world=7)[0] == INVALID  # rows not divisible by world
    assert red(hostlib, m=8 * 96)[0] == UNSUP  # slice 96 rows
    assert red(hostlib, drop_peer=2)[0] == INVALID  # missing peer partial
    assert red(hostlib, a=0x10004)[0] == UNSUP
    assert red(hostlib, inbox=1 << 20)[0] == WS  # emulated landing needs the inbox
    assert red(hostlib, inbox=1 << 20, opts=Opts(arrival_mode=RESIDENT))[0] == MK_OK
    code, p = red(hostlib, opts=Opts(n_reduce_wg=32))
    assert (p["n_copy"], p["n_reduce"], p["n_compute"]) == (192, 32, 32)
    code, p = red(hostlib)
    assert (p["n_copy"], p["n_reduce"], p["n_compute"]) == (224, 0, 32)
    code, p = red(hostlib, opts=Opts(arrival_mode=RESIDENT))
    assert (p["n_copy"], p["n_reduce"], p["n_compute"]) == (0, 0, 256)


def test_plan_rs_presum_assist(hostlib):
    """RS with peers and no reduce workgroups pre-sums owned tiles in the compute role (one band
    counter per owned tile after the fixed counters); a reduce role or AllReduce turns it off."""
    assert red(hostlib)[1]["assist"] == 1
    assert red(hostlib, opts=Opts(arrival_mode=RESIDENT))[1]["assist"] == 1
    assert red(hostlib, opts=Opts(n_reduce_wg=16))[1]["assist"] == 0
    assert red(hostlib, is_rs=0, m=256, n=8192, k=1024, tile=(128, 64, 4, 8))[1]["assist"] == 0
    assert red(hostlib, world=1)[1]["assist"] == 0


def moe(hostlib, world=8, t_local=4096, hidden=4096, E=64, top_k=2, eb=0, nl=8, ffn=1536, cap=65536, opts=None,
        logits=0x10000):
    toks = (ctypes.c_void_p * world)()
    for r in range(world):
        toks[r] = 0x600000000 + r * 0x10000000
    out = (ctypes.c_longlong * 16)()
    code = hostlib.mkh_plan_moe(ctypes.c_size_t(NF), ctypes.c_size_t(NC), ctypes.c_size_t(INBOX), GRID,
                                ctypes.byref(opts) if opts else None, toks, world, t_local, hidden, P(logits),
                                P(0x20000), E, top_k, eb, nl, P(0x30000), ffn, P(0x40000), P(0x50000), P(0x60000),
                                P(0x70000), P(0x80000), cap, 128, 256, out)
    keys = ["n_tokens", "n_chunks", "emulated", "drop_pos", "n_copy", "n_compute", "tiles_n", "max_mtiles", "off_misc",
            "off_chunk_cnt", "off_tile_cnt", "counters_need"]
    return code, dict(zip(keys, list(out)))


def test_plan_moe(hostlib):
    code, p = moe(hostlib)
    assert code == MK_OK
    assert (p["n_tokens"], p["n_chunks"], p["tiles_n"]) == (32768, 512, 6)
    assert (p["n_copy"], p["n_compute"]) == (240, 16)  # 15/16 of the workgroups route and dispatch
    assert p["max_mtiles"] == 65536 // 128 + 8 + 1
    assert p["off_tile_cnt"] == 128 + 512 * 8 and p["counters_need"] <= NC
    assert moe(hostlib, top_k=65)[0] == INVALID
    assert moe(hostlib, top_k=9, E=16)[0] == UNSUP
    assert moe(hostlib, eb=60)[0] == INVALID  # experts past n_experts
    assert moe(hostlib, t_local=100)[0] == UNSUP
    assert moe(hostlib, hidden=4160)[0] == UNSUP  # token rows above 8 KiB
    assert moe(hostlib, hidden=320)[0] == MK_OK
    assert moe(hostlib, E=66)[0] == UNSUP  # rows of logits must be 16-byte multiples
    assert moe(hostlib, logits=0x10004)[0] == UNSUP
    assert moe(hostlib, cap=-1)[0] == INVALID
    assert moe(hostlib, opts=Opts(arrival_chunk_tokens=32))[0] == UNSUP
    assert moe(hostlib, opts=Opts(arrival_order=0x9000, arrival_len=3))[0] == INVALID
    assert moe(hostlib, opts=Opts(arrival_order=0x9000, arrival_len=512))[0] == MK_OK


def mlp(hostlib, world=8, rank=0, m_shard=1024, k=4096, n_up=1792, n_out=4096, opts=None, h=0x600000000,
        drop_peer=None):
    arr = (ctypes.c_void_p * world)()
    peers = (ctypes.c_void_p * world)()
    ob = (ctypes.c_void_p * world)()
    for r in range(world):
        arr[r] = 0x300000000 + r * 0x10000000
        if r != rank and r != drop_peer:
            peers[r] = 0x700000000 + r * 0x10000000
            ob[r] = 0x800000000 + r * 0x10000000
    out = (ctypes.c_longlong * 16)()
    code = hostlib.mkh_plan_mlp(ctypes.c_size_t(NF), ctypes.c_size_t(NC), ctypes.c_size_t(INBOX), GRID,
                                ctypes.byref(opts) if opts else None, arr, world, rank, m_shard, k, P(0x10000), n_up,
                                P(0x20000), n_out, peers, P(0x100000000), P(h), P(0x900000000), ob, out)
    keys = ["ag_copy", "ag_compute", "ag_tiles_m", "ag_tiles_n", "red_compute", "red_tiles_m", "red_tiles_n",
            "own_tile_begin", "own_tile_end", "assist"]
    return code, dict(zip(keys, list(out)))


def test_plan_mlp(hostlib):
    """The MLP block plans its up-projection as mk_ag_gemm (role split, units) and its
    down-projection as a resident mk_gemm_rs on every workgroup, over the same 256-row tiles."""
    code, p = mlp(hostlib)
    assert code == MK_OK
    # 256 x 224 up-projection tiles; no local shard in place (every shard is copied): one XCD round
    # of compute workgroups
    assert (p["ag_copy"], p["ag_compute"], p["ag_tiles_m"], p["ag_tiles_n"]) == (248, 8, 32, 8)
    assert (p["red_compute"], p["red_tiles_m"], p["red_tiles_n"], p["assist"]) == (256, 32, 16, 1)
    assert (p["own_tile_begin"], p["own_tile_end"]) == (0, 4)
    code, p = mlp(hostlib, rank=5)
    assert code == MK_OK and (p["own_tile_begin"], p["own_tile_end"]) == (20, 24)
    assert mlp(hostlib, opts=Opts(arrival_mode=RESIDENT))[1]["ag_copy"] == 0
    assert mlp(hostlib, world=4, m_shard=128)[0] == UNSUP  # 512 rows: the down-projection would use 128-row tiles
    assert mlp(hostlib, n_up=1800)[0] == UNSUP  # not a multiple of 64
    assert mlp(hostlib, h=0)[0] == INVALID
    assert mlp(hostlib, h=0x600000004)[0] == UNSUP  # misaligned H
    assert mlp(hostlib, drop_peer=3)[0] == INVALID  # missing peer partial of the down-projection


def test_plan_link_rate_pacing(hostlib):
    """mk_opts.arrival_gbps: arrival position i is copied no earlier than i * unit_bytes / rate; the
    plan carries wall-clock ticks (100 MHz) per position in Q16."""
    code, p = ag(hostlib, opts=Opts(arrival_gbps=1071.0))  # 7 xGMI links x 153 GB/s
    assert code == MK_OK
    unit = 128 * 128 * 2
    assert p["pace_q16"] == round(unit / 1071e9 * 1e8 * 65536)
    assert ag(hostlib, opts=Opts())[1]["pace_q16"] == 0
    assert ag(hostlib, opts=Opts(arrival_mode=RESIDENT, arrival_gbps=5.0))[1]["pace_q16"] == 0  # nothing arrives
    for bad in (-1.0, float("nan"), float("inf")):
        assert ag(hostlib, opts=Opts(arrival_gbps=bad))[0] == INVALID
        assert ag(hostlib, opts=Opts(arrival_mode=RESIDENT, arrival_gbps=bad))[0] == INVALID
    # 2048 units of 32 KiB take 67 ms at 1 GB/s: beyond half of a 100 ms watchdog, inside 2 s
    assert ag(hostlib, opts=Opts(arrival_gbps=1.0, timeout_us=100000))[0] == INVALID
    assert ag(hostlib, opts=Opts(arrival_gbps=1.0))[0] == MK_OK
    code, p = red(hostlib, opts=Opts(arrival_gbps=1071.0))
    assert code == MK_OK and p["pace_q16"] == round(64 * 128 * 4 / 1071e9 * 1e8 * 65536)
    assert red(hostlib, opts=Opts(arrival_mode=RESIDENT, arrival_gbps=1071.0))[1]["pace_q16"] == 0
    assert red(hostlib, opts=Opts(arrival_gbps=-5.0))[0] == INVALID


def ring(hostlib, world=8, rank=0, heads=8, s_local=4096, d=128, scale=0.0, opts=None, ring_bufs=True, drop=None):
    ks = (ctypes.c_void_p * world)()
    vs = (ctypes.c_void_p * world)()
    for j in range(world):
        if j != drop:
            ks[j] = 0x300000000 + j * 0x10000000
            vs[j] = 0x400000000 + j * 0x10000000
    out = (ctypes.c_longlong * 16)()
    sc = ctypes.c_float(0.0)
    code = hostlib.mkh_plan_ring_attn(ctypes.c_size_t(NF), ctypes.c_size_t(NC), ctypes.c_size_t(INBOX), GRID,
                                      ctypes.byref(opts) if opts else None, P(0x10000), ks, vs, world, rank, heads,
                                      s_local, d, ctypes.c_float(scale), P(0x500000000 if ring_bufs else 0),
                                      P(0x600000000 if ring_bufs else 0), P(0x700000000), P(0x800000000), out,
                                      ctypes.byref(sc))
    keys = ["n_blk", "n_qt", "n_items", "n_units", "emulated", "n_order", "drop_pos", "n_copy", "n_compute", "pace_q16"]
    return code, dict(zip(keys, list(out)), scale=sc.value)


def test_plan_ring_attention(hostlib):
    """Items (head, 128-query tile), 64-key K and V blocks with one flag each, the default role
    split, the default softmax scale and the argument checks."""
    code, p = ring(hostlib)
    assert code == MK_OK
    assert (p["n_blk"], p["n_qt"], p["n_items"]) == (64, 32, 256)
    assert p["n_units"] == 8 * 8 * 64 * 2 and p["n_order"] == 7 * 8 * 64 * 2
    assert (p["n_copy"], p["n_compute"]) == (192, 64) and p["emulated"] == 1
    assert abs(p["scale"] - 128 ** -0.5) < 1e-7
    assert abs(ring(hostlib, scale=0.25)[1]["scale"] - 0.25) < 1e-9
    code, p = ring(hostlib, opts=Opts(arrival_mode=RESIDENT), ring_bufs=False)
    assert code == MK_OK and (p["n_copy"], p["n_order"], p["emulated"]) == (0, 0, 0)
    assert ring(hostlib, world=1, ring_bufs=False)[0] == MK_OK  # nothing arrives
    assert ring(hostlib, ring_bufs=False)[0] == INVALID  # emulated needs the landing buffers
    assert ring(hostlib, d=64)[0] == UNSUP
    assert ring(hostlib, s_local=4160)[0] == UNSUP  # not a multiple of 128
    assert ring(hostlib, scale=-1.0)[0] == INVALID and ring(hostlib, scale=float("nan"))[0] == INVALID
    assert ring(hostlib, drop=3)[0] == INVALID
    assert ring(hostlib, rank=8)[0] == INVALID
    assert ring(hostlib, world=8, heads=64, s_local=32768)[0] == UNSUP  # 8 x 512 MiB shards: 4 GiB
    assert ring(hostlib, opts=Opts(arrival_gbps=1071.0))[1]["pace_q16"] == round(16384 / 1071e9 * 1e8 * 65536)
