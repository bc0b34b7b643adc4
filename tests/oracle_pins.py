"""Pins for the fp64 oracle: checks against things the oracle does not compute itself.

Each ``pin_*`` takes an implementation namespace (the oracle module, or a planted
mutant of it in the mutation tests) and raises AssertionError when the
implementation disagrees with:
  * hand-worked examples (tests/golden/*.json, each derived by hand from the
    definitions in the five-fused-kernels table of the mKernel write-up);
  * brute force built a different way (math.fsum over exact products, element
    by element, straight from the shards/partials rather than from stacked
    arrays; Python ``sorted`` over (score, id) pairs for routing);
  * closed forms (B = I gives C = A; zero peers give the plain GEMM slices;
    forced routing by a huge bias gives known segment sizes);
  * exact integer arithmetic (integer-valued inputs make every sum exact);
  * invariants (segment sizes add up, tokens ascend inside a segment, the
    gathered rows equal the routed tokens).
"""
from __future__ import annotations

import json
import math
import os
from types import SimpleNamespace

import numpy as np

import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bf16(x) -> np.ndarray:
    return wl.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def _exact_value(bits: int) -> float:
    """Value of a bf16 bit pattern from sign/exponent/fraction (IEEE layout), by hand."""
    sign = -1.0 if bits & 0x8000 else 1.0
    e = (bits >> 7) & 0xFF
    f = bits & 0x7F
    if e == 0:
        return sign * (f / 128.0) * 2.0 ** -126
    return sign * (1.0 + f / 128.0) * 2.0 ** (e - 127)


def _fsum_dot(row_bits: np.ndarray, col_bits: np.ndarray) -> float:
    return math.fsum(_exact_value(int(a)) * _exact_value(int(b)) for a, b in zip(row_bits, col_bits))


# --------------------------------------------------------------------------------------
def pin_bf16(impl):
    g = _golden("bf16_bits.json")
    for hexbits, val in g["widen"]:
        got = float(impl.bf16_to_f64(np.array([int(hexbits, 16)], dtype=np.uint16))[0])
        assert got == val and math.copysign(1, got) == math.copysign(1, val), (hexbits, got, val)
    # every bf16 pattern that is finite widens to the value given by its fields
    allbits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    exp = (allbits >> 7) & 0xFF
    fin = allbits[exp != 0xFF]
    got = impl.bf16_to_f64(fin)
    ref = np.array([_exact_value(int(b)) for b in fin[::97]])
    assert np.array_equal(got[::97], ref)


def pin_ag(impl):
    g = _golden("ag_hand.json")
    shards = [_bf16(s) for s in g["a_shards"]]
    a_g, c = impl.ag_gemm(shards, _bf16(g["b"]))
    assert np.array_equal(np.asarray(c, dtype=np.float64), np.array(g["c"], dtype=np.float64)), c
    assert np.array_equal(a_g, np.concatenate(shards, axis=0))

    # brute force on the tiny workload's size: each element from the shards directly
    shape = wl.AG_TINY
    d = wl.gen_ag(shape, run=0)
    a_g, c = impl.ag_gemm(d["a_shards"], d["b"])
    assert a_g.dtype == np.uint16
    ref_rms = None
    rng = np.random.default_rng(5)
    pts = [(int(rng.integers(shape.m)), int(rng.integers(shape.n))) for _ in range(96)]
    pts += [(0, 0), (shape.m - 1, shape.n - 1), (shape.m_shard, 7), (2 * shape.m_shard - 1, shape.n - 3)]
    vals = []
    for (i, j) in pts:
        r, ii = divmod(i, shape.m_shard)
        vals.append(_fsum_dot(d["a_shards"][r][ii], d["b"][:, j]))
        assert int(a_g[i, 5]) == int(d["a_shards"][r][ii, 5])
    ref_rms = math.sqrt(sum(v * v for v in vals) / len(vals))
    for (i, j), v in zip(pts, vals):
        assert abs(float(c[i, j]) - v) <= 1e-12 * ref_rms, (i, j, float(c[i, j]), v)

    # closed form: B = I (k = n) gives C = A exactly
    eye = _bf16(np.eye(shape.k, dtype=np.float32))
    _, c_i = impl.ag_gemm(d["a_shards"], eye)
    assert np.array_equal(np.asarray(c_i, dtype=np.float64),
                          np.concatenate([impl.bf16_to_f64(s) for s in d["a_shards"]], axis=0))

    # exact integers: every partial sum is an integer below 2^24
    di = wl.gen_ag(shape, run=3, kind="int")
    _, ci = impl.ag_gemm(di["a_shards"], di["b"])
    ci = np.asarray(ci, dtype=np.float64)
    assert np.array_equal(ci, np.round(ci))
    i, j = 3 * shape.m_shard + 17, 200
    exact = sum(int(_exact_value(int(a))) * int(_exact_value(int(b)))
                for a, b in zip(di["a_shards"][3][17], di["b"][:, j]))
    assert ci[i, j] == exact

    # arrival order does not matter: add K-unit contributions in a seeded arrival order
    order = wl.ag_arrival_order(shape, trial=1)
    per_unit = np.zeros((shape.m, shape.n), dtype=np.float64)
    a64 = np.concatenate([impl.bf16_to_f64(s) for s in di["a_shards"]], axis=0)
    b64 = impl.bf16_to_f64(di["b"])
    done = np.zeros((shape.n_unit_rows, shape.n_unit_cols), dtype=bool)
    local = shape.rank
    spr = shape.m_shard // shape.unit_rows
    done[local * spr:(local + 1) * spr, :] = True
    for ur in range(local * spr, (local + 1) * spr):
        for uc in range(shape.n_unit_cols):
            rs, cs = ur * shape.unit_rows, uc * shape.unit_cols
            per_unit[rs:rs + shape.unit_rows] += a64[rs:rs + shape.unit_rows, cs:cs + shape.unit_cols] @ b64[cs:cs + shape.unit_cols]
    for u in order:
        ur, uc = divmod(int(u), shape.n_unit_cols)
        assert not done[ur, uc]
        done[ur, uc] = True
        rs, cs = ur * shape.unit_rows, uc * shape.unit_cols
        per_unit[rs:rs + shape.unit_rows] += a64[rs:rs + shape.unit_rows, cs:cs + shape.unit_cols] @ b64[cs:cs + shape.unit_cols]
    assert done.all()
    assert np.array_equal(per_unit, ci)

    # W = 1 reduces to a plain GEMM of the single shard
    s1 = wl.AGShape(world=1, m_shard=64, k=128, n=64, cfg=wl.CFG_AG_TINY)
    d1 = wl.gen_ag(s1, run=4, kind="int")
    _, c1 = impl.ag_gemm(d1["a_shards"], d1["b"])
    for (i, j) in [(0, 0), (63, 63), (10, 40)]:
        assert float(c1[i, j]) == _fsum_dot(d1["a_shards"][0][i], d1["b"][:, j])


def _rs_brute(a, b, peers, world, rank, i, j):
    ms = a.shape[0] // world
    return _fsum_dot(a[rank * ms + i], b[:, j]) + math.fsum(float(peers[q][i, j]) for q in range(world) if q != rank)


def pin_rs(impl):
    g = _golden("rs_hand.json")
    a, b = _bf16(g["a"]), _bf16(g["b"])
    for case in g["cases"]:
        peers = [None] * g["world"]
        for k_, v in case["peers"].items():
            peers[int(k_)] = np.array(v, dtype=np.float32)
        own, outbox = impl.gemm_rs(a, b, peers, g["world"], case["rank"])
        assert np.array_equal(np.asarray(own, np.float64), np.array(case["own"], np.float64)), (case["rank"], own)
        for k_, v in case["outbox"].items():
            assert np.array_equal(np.asarray(outbox[int(k_)], np.float64), np.array(v, np.float64))
        assert outbox[case["rank"]] is None

    shape = wl.RedShape(m=256, n=96, k=160, world=4, unit_rows=64, unit_cols=32, cfg=wl.CFG_RS)
    for rank in (0, 2):
        sh = wl.replace(shape, rank=rank)
        d = wl.gen_reduce(sh, "rs", run=1)
        own, outbox = impl.gemm_rs(d["a"], d["b"], d["peers"], sh.world, rank)
        ms = sh.m_slice
        rng = np.random.default_rng(rank)
        pts = [(int(rng.integers(ms)), int(rng.integers(sh.n))) for _ in range(48)] + [(0, 0), (ms - 1, sh.n - 1)]
        vals = [_rs_brute(d["a"], d["b"], d["peers"], sh.world, rank, i, j) for i, j in pts]
        sc = math.sqrt(sum(v * v for v in vals) / len(vals))
        for (i, j), v in zip(pts, vals):
            assert abs(float(own[i, j]) - v) <= 1e-12 * sc, (rank, i, j)
        for q in range(sh.world):
            if q == rank:
                assert outbox[q] is None
                continue
            for (i, j) in pts[:12]:
                v = _fsum_dot(d["a"][q * ms + i], d["b"][:, j])
                assert abs(float(outbox[q][i, j]) - v) <= 1e-12 * max(sc, 1.0), (rank, q, i, j)

    # zero peers: own and outboxes are exactly the slices of the plain GEMM (integer inputs)
    d = wl.gen_reduce(shape, "rs", run=2, kind="int")
    zero = [None if q == 0 else np.zeros_like(d["peers"][q]) for q in range(shape.world)]
    own, outbox = impl.gemm_rs(d["a"], d["b"], zero, shape.world, 0)
    ms = shape.m_slice
    for q in range(shape.world):
        blk = own if q == 0 else outbox[q]
        for (i, j) in [(0, 0), (ms - 1, shape.n - 1), (5, 17)]:
            assert float(blk[i, j]) == _fsum_dot(d["a"][q * ms + i], d["b"][:, j])

    # cancellation: Q_1 = -P[slice 0] leaves the sum of the other peers
    own0, _ = impl.gemm_rs(d["a"], d["b"], zero, shape.world, 0)
    peers = list(d["peers"])
    peers[1] = (-np.asarray(own0)).astype(np.float32)
    own, _ = impl.gemm_rs(d["a"], d["b"], peers, shape.world, 0)
    rest = sum(np.asarray(peers[q], np.float64) for q in range(2, shape.world))
    assert np.array_equal(np.asarray(own, np.float64), rest)

    # W = 1: own is the whole GEMM, no outbox
    s1 = wl.RedShape(m=64, n=64, k=64, world=1, cfg=wl.CFG_RS)
    d1 = wl.gen_reduce(s1, "rs", run=0, kind="int")
    own, outbox = impl.gemm_rs(d1["a"], d1["b"], d1["peers"], 1, 0)
    assert outbox == [None]
    assert float(own[7, 9]) == _fsum_dot(d1["a"][7], d1["b"][:, 9])


def pin_ar(impl):
    g = _golden("ar_hand.json")
    peers = [None] * g["world"]
    for k_, v in g["peers"].items():
        peers[int(k_)] = np.array(v, dtype=np.float32)
    out = impl.gemm_ar(_bf16(g["a"]), _bf16(g["b"]), peers, g["world"], g["rank"])
    assert np.array_equal(np.asarray(out, np.float64), np.array(g["out"], np.float64)), out

    shape = wl.RedShape(m=128, n=96, k=192, world=4, unit_rows=64, unit_cols=32, cfg=wl.CFG_AR)
    for rank in (0, 3):
        sh = wl.replace(shape, rank=rank)
        d = wl.gen_reduce(sh, "ar", run=1)
        out = impl.gemm_ar(d["a"], d["b"], d["peers"], sh.world, rank)
        rng = np.random.default_rng(10 + rank)
        pts = [(int(rng.integers(sh.m)), int(rng.integers(sh.n))) for _ in range(48)] + [(sh.m - 1, sh.n - 1)]
        vals = [_fsum_dot(d["a"][i], d["b"][:, j]) + math.fsum(float(d["peers"][q][i, j]) for q in range(sh.world) if q != rank)
                for i, j in pts]
        sc = math.sqrt(sum(v * v for v in vals) / len(vals))
        for (i, j), v in zip(pts, vals):
            assert abs(float(out[i, j]) - v) <= 1e-12 * sc, (rank, i, j)

    d = wl.gen_reduce(shape, "ar", run=2, kind="int")
    zero = [None if q == 0 else np.zeros_like(d["peers"][q]) for q in range(shape.world)]
    p = impl.gemm_ar(d["a"], d["b"], zero, shape.world, 0)
    for (i, j) in [(0, 0), (127, 95), (64, 3)]:
        assert float(p[i, j]) == _fsum_dot(d["a"][i], d["b"][:, j])
    peers = list(d["peers"])
    peers[2] = (-np.asarray(p)).astype(np.float32)
    out = impl.gemm_ar(d["a"], d["b"], peers, shape.world, 0)
    assert np.array_equal(np.asarray(out, np.float64), np.asarray(peers[1], np.float64) + np.asarray(peers[3], np.float64))


def _route_brute(logits, bias, top_k):
    """Python-level routing: fp32 score per element, sorted on (-score, id)."""
    out = []
    for t in range(logits.shape[0]):
        s = [(-float(np.float32(logits[t, e]) + np.float32(bias[e])), e) for e in range(logits.shape[1])]
        out.append([e for _, e in sorted(s)[:top_k]])
    return np.array(out, dtype=np.int32)


def pin_moe(impl):
    g = _golden("moe_hand.json")
    tokens = [_bf16(t) for t in g["tokens"]]
    w_up = _bf16(g["w_up"])
    res = impl.moe_dispatch_gemm(tokens, np.array(g["logits"], np.float32), np.array(g["bias"], np.float32),
                                 g["top_k"], g["expert_begin"], g["n_local"], w_up)
    assert np.array_equal(res["topk_idx"], np.array(g["topk_idx"])), res["topk_idx"]
    assert np.array_equal(res["seg_offsets"], np.array(g["seg_offsets"])), res["seg_offsets"]
    assert np.array_equal(res["seg_token"], np.array(g["seg_token"])), res["seg_token"]
    assert np.array_equal(np.asarray(res["y"], np.float64), np.array(g["y"], np.float64)), res["y"]
    tok_all = np.concatenate(tokens)
    assert np.array_equal(res["x_seg"], tok_all[np.array(g["seg_token"])])

    # the score is one fp32 add: 1 + 2^-30 rounds to 1 in fp32, so the tie goes to the lower id
    lg = np.array([[1.0, 1.0, -5.0]], np.float32)
    bs = np.array([0.0, 2.0 ** -30, 0.0], np.float32)
    assert impl.moe_route(lg, bs, 1)[0, 0] == 0
    # ... while a difference fp32 can hold is honoured
    bs2 = np.array([0.0, 2.0 ** -20, 0.0], np.float32)
    assert impl.moe_route(lg, bs2, 1)[0, 0] == 1

    # brute-force routing and segments on the small workload
    shape = wl.MOE_SMALL
    d = wl.gen_moe(shape, run=0)
    topk = impl.moe_route(d["logits"], d["bias"], shape.top_k)
    assert np.array_equal(topk, _route_brute(d["logits"], d["bias"], shape.top_k))
    offs, seg_token = impl.moe_segments(topk, shape.expert_begin, shape.n_local)
    segs = [[t for t in range(shape.tokens) if (shape.expert_begin + e) in topk[t].tolist()] for e in range(shape.n_local)]
    exp_offs = [0]
    for s in segs:
        exp_offs.append(exp_offs[-1] + len(s))
    assert offs.tolist() == exp_offs
    assert seg_token.tolist() == [t for s in segs for t in s]

    # all experts local: sizes add up to top_k * T, every segment strictly ascending
    offs_all, st_all = impl.moe_segments(topk, 0, shape.n_experts)
    assert int(offs_all[-1]) == shape.top_k * shape.tokens
    assert np.all(np.diff(offs_all) >= 0)
    for e in range(shape.n_experts):
        seg = st_all[offs_all[e]:offs_all[e + 1]]
        assert np.all(np.diff(seg) > 0)
        assert np.all(np.any(topk[seg] == e, axis=1))

    # forced routing: a huge bias on experts 0 and 1 sends every token to both
    bias = np.zeros(shape.n_experts, np.float32)
    bias[:2] = 1e4
    t2 = impl.moe_route(d["logits"], bias, 2)
    assert np.array_equal(np.sort(t2, axis=1), np.tile(np.array([0, 1], np.int32), (shape.tokens, 1)))
    s01 = d["logits"][:, :2].astype(np.float32) + np.float32(1e4)
    first = np.where(s01[:, 1] > s01[:, 0], 1, 0)  # descending score, ties to the lower id
    assert np.array_equal(t2[:, 0], first)
    o2, _ = impl.moe_segments(t2, 0, shape.n_local)
    assert o2.tolist() == [0, shape.tokens, 2 * shape.tokens] + [2 * shape.tokens] * (shape.n_local - 2)
    # a huge negative bias on the local experts leaves them empty
    bias = np.zeros(shape.n_experts, np.float32)
    bias[:shape.n_local] = -1e4
    t3 = impl.moe_route(d["logits"], bias, 2)
    o3, s3 = impl.moe_segments(t3, 0, shape.n_local)
    assert o3.tolist() == [0] * (shape.n_local + 1) and len(s3) == 0

    # grouped GEMM rows by brute force; gathered rows equal the routed tokens
    res = impl.moe_dispatch_gemm(d["tokens"], d["logits"], d["bias"], shape.top_k, shape.expert_begin,
                                 shape.n_local, d["w_up"])
    tok_all = np.concatenate(d["tokens"])
    assert np.array_equal(res["x_seg"], tok_all[res["seg_token"]])
    offs = res["seg_offsets"]
    y = np.asarray(res["y"], np.float64)
    rng = np.random.default_rng(3)
    R = int(offs[-1])
    rows = [int(rng.integers(R)) for _ in range(24)] + [0, R - 1]
    for i in rows:
        e = int(np.searchsorted(offs, i, side="right") - 1)
        t = int(res["seg_token"][i])
        for j in (0, shape.ffn - 1, int(rng.integers(shape.ffn))):
            v = _fsum_dot(tok_all[t], d["w_up"][e][:, j])
            assert abs(y[i, j] - v) <= 1e-12 * max(1.0, abs(v)), (i, j)

    # a single local expert that every token hits: the grouped GEMM is the plain GEMM of all tokens
    bias = np.zeros(shape.n_experts, np.float32)
    bias[0] = 1e4
    r1 = impl.moe_dispatch_gemm(d["tokens"], d["logits"], bias, 2, 0, 1, d["w_up"][:1])
    assert r1["seg_offsets"].tolist() == [0, shape.tokens]
    assert np.array_equal(r1["seg_token"], np.arange(shape.tokens))
    for t in (0, shape.tokens - 1, 77):
        assert abs(float(r1["y"][t, 5]) - _fsum_dot(tok_all[t], d["w_up"][0][:, 5])) <= 1e-12 * 10


# --------------------------------------------------------------------------------------
# MLP block (reading R16): gelu, bf16 rounding of H, the composition
# --------------------------------------------------------------------------------------
# standard normal CDF from printed tables: Phi(1), Phi(2) and 1 - Phi(2)
_PHI1, _PHI2, _Q2 = 0.8413447460685429, 0.9772498680518208, 0.022750131948179195
_BF16_POS = None


def _bf16_positive_values():
    """Every positive finite normal bf16 value, ascending, from its bit fields."""
    global _BF16_POS
    if _BF16_POS is None:
        _BF16_POS = np.array([_exact_value(b) for b in range(0x0080, 0x7F80)], dtype=np.float64)
    return _BF16_POS


def _round_bf16_brute(x: float) -> float:
    """Nearest bf16 value by bisection over the value list; ties to the even bit pattern."""
    v = _bf16_positive_values()
    ax = abs(x)
    if ax == 0.0:
        return 0.0
    i = int(np.searchsorted(v, ax))
    if i < len(v) and v[i] == ax:
        r = ax
    else:
        lo, hi = v[i - 1], v[i]
        if ax - lo < hi - ax:
            r = lo
        elif hi - ax < ax - lo:
            r = hi
        else:  # tie: the pattern with an even last bit (index parity = pattern parity here)
            r = lo if (0x0080 + i - 1) % 2 == 0 else hi
    return math.copysign(r, x)


def _gelu_brute(x: float) -> float:
    return x * 0.5 * (1.0 + math.erf(x / math.sqrt(2.0)))


def pin_mlp(impl):
    # gelu against table values, the odd-part identity gelu(x) - gelu(-x) = x, and the tails
    g = impl.gelu(np.array([0.0, 1.0, -1.0, 2.0, -2.0, 10.0, -10.0]))
    assert g[0] == 0.0
    assert abs(g[1] - _PHI1) <= 1e-15 and abs(g[2] - (_PHI1 - 1.0)) <= 1e-15
    assert abs(g[3] - 2 * _PHI2) <= 2e-15 and abs(g[4] + 2 * _Q2) <= 1e-15
    assert g[5] == 10.0 and -1e-20 < g[6] <= 0.0
    x = np.random.default_rng(11).standard_normal(257) * 3
    assert np.max(np.abs(impl.gelu(x) - impl.gelu(-x) - x)) <= 1e-14
    # bf16 rounding: bf16 values are fixed points, ties go to even, everything else to nearest
    vals = _bf16_positive_values()[::37]
    assert np.array_equal(impl.round_bf16(vals), vals) and np.array_equal(impl.round_bf16(-vals), -vals)
    ties = [(1 + 2 ** -8, 1.0), (1 + 3 * 2 ** -8, 1 + 2 ** -6), (-(1 + 2 ** -8), -1.0), (3 * 2 ** -9, 3 * 2 ** -9),
            (1 + 2 ** -8 + 2 ** -30, 1 + 2 ** -7), (255.5, 256.0), (254.5, 254.0), (0.0, 0.0)]
    got = impl.round_bf16(np.array([t for t, _ in ties]))
    assert [float(v) for v in got] == [r for _, r in ties], got
    r = np.random.default_rng(12).standard_normal(400) * np.exp(np.random.default_rng(13).uniform(-20, 20, 400))
    assert [float(v) for v in impl.round_bf16(r)] == [_round_bf16_brute(float(v)) for v in r]
    bits = impl.bf16_bits(impl.round_bf16(r[:50]))
    assert [_exact_value(int(b)) for b in bits] == [_round_bf16_brute(float(v)) for v in r[:50]]

    # the composition, brute force on a tiny case: u by fsum, gelu per element, rounded by bisection
    sh = wl.MLPShape(world=2, m_shard=64, k=64, n_up=64, n_out=64, rank=1)
    d = wl.gen_mlp(sh, run=3)
    res = impl.mlp_ag_rs(d["a_shards"], d["b_up"], d["b_down"], d["peers"], sh.world, sh.rank)
    a = np.concatenate(d["a_shards"])
    assert np.array_equal(np.asarray(res["a_gathered"]), a)
    hb = {}
    for i in range(sh.m):
        for c in range(sh.n_up):
            hb[i, c] = _round_bf16_brute(_gelu_brute(_fsum_dot(a[i], d["b_up"][:, c])))
    h = np.asarray(res["h"], np.float64)
    assert all(h[i, c] == v for (i, c), v in hb.items())
    bd = oracle_bf16(d["b_down"])
    ms = sh.m_shard
    for (i, j) in [(0, 0), (ms - 1, sh.n_out - 1), (17, 40), (33, 5)]:
        row = sh.rank * ms + i
        ref = math.fsum([hb[row, c] * bd[c, j] for c in range(sh.n_up)] + [float(d["peers"][0][i, j])])
        assert abs(float(res["own"][i, j]) - ref) <= 1e-12 * max(1.0, abs(ref)), (i, j)
        ob = math.fsum(hb[i, c] * bd[c, j] for c in range(sh.n_up))  # rank 0's rows, unreduced
        assert abs(float(res["outbox"][0][i, j]) - ob) <= 1e-12 * max(1.0, abs(ob))
    assert res["outbox"][1] is None

    # closed forms: A = 0 gives H = 0, the owned rows are the peers' sum and the outboxes zero
    z = dict(d, a_shards=[np.zeros_like(x) for x in d["a_shards"]])
    res = impl.mlp_ag_rs(z["a_shards"], z["b_up"], z["b_down"], z["peers"], sh.world, sh.rank)
    assert not np.any(np.asarray(res["h"])) and not np.any(np.asarray(res["outbox"][0]))
    assert np.array_equal(np.asarray(res["own"], np.float64), np.asarray(d["peers"][0], np.float64))
    # integer inputs: U is 0 or a multiple of 16, where gelu is the identity in fp64 and H is exact
    si = wl.MLPShape(world=4, m_shard=64, k=128, n_up=192, n_out=64, rank=2)
    di = wl.gen_mlp(si, run=4, kind="int")
    res = impl.mlp_ag_rs(di["a_shards"], di["b_up"], di["b_down"], di["peers"], si.world, si.rank)
    ai = np.concatenate([oracle_bf16(x) for x in di["a_shards"]]).astype(np.int64)
    ui = ai @ oracle_bf16(di["b_up"]).astype(np.int64)
    assert np.all(ui % 16 == 0) and np.array_equal(np.asarray(res["h"], np.float64), ui.astype(np.float64))
    pi = ui @ oracle_bf16(di["b_down"]).astype(np.int64)
    own = pi[si.rank * si.m_shard:(si.rank + 1) * si.m_shard] + sum(
        di["peers"][j].astype(np.int64) for j in range(si.world) if j != si.rank)
    assert np.array_equal(np.asarray(res["own"], np.float64), own.astype(np.float64))


def pin_ring(impl):
    # brute force on a tiny case: scores, exponentials and sums per element with math.fsum, from
    # the shards one by one (not the concatenated keys)
    sh = wl.RingShape(world=3, heads=2, s_local=4, d=8, sigma=1.0, rank=1)
    d = wl.gen_ring(sh, run=2)
    out, lse = impl.ring_attention(d["q"], d["k_shards"], d["v_shards"])
    q = oracle_bf16(d["q"])
    ks = [oracle_bf16(k) for k in d["k_shards"]]
    vs = [oracle_bf16(v) for v in d["v_shards"]]
    sc = 1.0 / math.sqrt(sh.d)
    for h in range(sh.heads):
        for i in range(sh.s_local):
            scores, vals = [], []
            for j in range(sh.world):
                for t in range(sh.s_local):
                    scores.append(sc * math.fsum(q[h, i, c] * ks[j][h, t, c] for c in range(sh.d)))
                    vals.append(vs[j][h, t])
            mx = max(scores)
            w = [math.exp(x - mx) for x in scores]
            den = math.fsum(w)
            for c in range(sh.d):
                ref = math.fsum(wi * v[c] for wi, v in zip(w, vals)) / den
                assert abs(float(out[h, i, c]) - ref) <= 1e-12, (h, i, c)
            assert abs(float(lse[h, i]) - (mx + math.log(den))) <= 1e-12
    # an explicit scale is honoured: scale 2/sqrt(d) equals the default on doubled queries' scores
    o2, l2 = impl.ring_attention(d["q"], d["k_shards"], d["v_shards"], scale=2.0 / math.sqrt(sh.d))
    qq = _bf16(2.0 * q)  # exact: doubling a bf16 value
    o3, l3 = impl.ring_attention(qq, d["k_shards"], d["v_shards"])
    assert np.max(np.abs(np.asarray(o2) - np.asarray(o3))) <= 1e-12 and np.max(np.abs(np.asarray(l2) - np.asarray(l3))) <= 1e-12
    # closed form: zero queries weigh every key equally (out = mean of all values, lse = log N)
    z = np.zeros_like(d["q"])
    oz, lz = impl.ring_attention(z, d["k_shards"], d["v_shards"])
    mean = np.mean(np.concatenate(vs, axis=1), axis=1)
    assert np.max(np.abs(np.asarray(oz) - mean[:, None, :])) <= 1e-12
    assert np.max(np.abs(np.asarray(lz) - math.log(sh.world * sh.s_local))) <= 1e-12
    # one dominant key (score 64, every other key 0) selects that key's value
    k1 = np.zeros((sh.heads, sh.s_local, sh.d), np.float32)
    k1[:, 2, 0] = 1.0
    ksh = [_bf16(k1) if j == 2 else _bf16(np.zeros_like(k1)) for j in range(sh.world)]
    qd = np.zeros((sh.heads, sh.s_local, sh.d), np.float32)
    qd[:, :, 0] = 64.0 * math.sqrt(sh.d)  # score 64 for that key, 0 for the rest
    od, _ = impl.ring_attention(_bf16(qd), ksh, d["v_shards"])
    assert np.max(np.abs(np.asarray(od) - vs[2][:, 2, :][:, None, :])) <= 1e-12
    # the ring's order does not matter: shards visited in any rotation give the same result
    rot = [1, 2, 0]
    orr, lr = impl.ring_attention(d["q"], [d["k_shards"][j] for j in rot], [d["v_shards"][j] for j in rot])
    assert np.max(np.abs(np.asarray(orr) - np.asarray(out))) <= 1e-13 and np.max(np.abs(np.asarray(lr) - np.asarray(lse))) <= 1e-13
    # shifting every key by a constant vector c shifts each query's scores by scale*q.c: same out
    c = np.zeros(sh.d, np.float32)
    c[3] = 2.0
    kshift = [_bf16(k + c) for k in ks]
    if all(np.array_equal(oracle_bf16(a), k + c) for a, k in zip(kshift, ks)):  # shift exact in bf16
        os_, ls_ = impl.ring_attention(d["q"], kshift, d["v_shards"])
        assert np.max(np.abs(np.asarray(os_) - np.asarray(out))) <= 1e-12
        assert np.max(np.abs(np.asarray(ls_) - np.asarray(lse) - sc * 2.0 * q[:, :, 3])) <= 1e-12


def oracle_bf16(bits):
    """bf16 bits -> fp64 through the bit fields (not the oracle's widening)."""
    b = np.asarray(bits, dtype=np.uint16)
    flat = np.array([_exact_value(int(x)) for x in np.unique(b)], dtype=np.float64)
    lut = dict(zip(np.unique(b).tolist(), flat.tolist()))
    return np.vectorize(lambda x: lut[int(x)], otypes=[np.float64])(b)


def pin_acceptance(impl):
    """RMS and the relative error that every float parity verdict uses."""
    g = _golden("acceptance_hand.json")
    for case in g["cases"]:
        ref = np.asarray(case["ref"], np.float64)
        out = np.asarray(case["out"], np.float64)
        want_rms = math.sqrt(case["rms_sq"])
        assert abs(impl.rms(ref) - want_rms) <= 1e-15 * want_rms, (case["ref"], impl.rms(ref), want_rms)
        want_err = case["err_num"] / want_rms
        got = impl.max_rel_err(out, ref)
        assert abs(got - want_err) <= 1e-15 * max(want_err, 1e-300), (case["out"], got, want_err)
    # brute force on a random buffer: a Python loop over the elements, math.fsum for the mean square
    rng = np.random.default_rng(7)
    ref = rng.normal(0.0, 3.0, size=(13, 17))
    out = ref + rng.normal(0.0, 1e-3, size=ref.shape)
    flat_r = [float(x) for x in ref.ravel()]
    flat_o = [float(x) for x in out.ravel()]
    r_bf = math.sqrt(math.fsum(x * x for x in flat_r) / len(flat_r))
    e_bf = max(abs(o - r) for o, r in zip(flat_o, flat_r)) / r_bf
    assert abs(impl.rms(ref) - r_bf) <= 1e-13 * r_bf
    assert abs(impl.max_rel_err(out, ref) - e_bf) <= 1e-12 * e_bf
    # the error is taken against the reference's RMS, not the output's: a large output that hits
    # the reference within 1e-3 of its RMS passes, whatever its own size
    assert impl.max_rel_err(ref * (1 + 1e-6), ref) <= 1e-6 * np.max(np.abs(ref)) / r_bf * (1 + 1e-9)
    # homogeneity: RMS scales with |c|, the relative error does not change
    assert abs(impl.rms(-4.0 * ref) - 4.0 * r_bf) <= 1e-13 * r_bf
    assert abs(impl.max_rel_err(-4.0 * out, -4.0 * ref) - e_bf) <= 1e-12 * e_bf
    # one element off by d in an otherwise exact buffer of n equal values v: error d / |v|
    v = np.full(1000, -0.5)
    o = v.copy()
    o[537] += 0.002
    assert abs(impl.max_rel_err(o, v) - 0.004) <= 1e-15
    assert impl.max_rel_err(v, v) == 0.0


ALL_PINS = [pin_bf16, pin_ag, pin_rs, pin_ar, pin_moe, pin_mlp, pin_ring, pin_acceptance]


def run_all(impl):
    """Names of the pins the implementation fails."""
    failed = []
    for p in ALL_PINS:
        try:
            p(impl)
        except AssertionError:
            failed.append(p.__name__)
        except (ValueError, IndexError, TypeError, KeyError, AttributeError) as e:  # a broken mutant may crash
            failed.append(p.__name__ + ":" + type(e).__name__)
    return failed


def namespace_of(mod, **overrides):
    ns = SimpleNamespace(**{k: getattr(mod, k) for k in mod.__all__})
    for k, v in overrides.items():
        setattr(ns, k, v)
    return ns
