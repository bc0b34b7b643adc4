"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins catch each one.

Every mutant is a copy of one oracle function with one slip: a dropped term, a
wrong sign or index, a transposed operand, a wrong precision or tie-break.  The
test passes when at least one pin fails for every mutant."""
import numpy as np
import pytest

import oracle
import oracle.mk_oracle as M
import oracle_pins as P

_ORIG_SEGMENTS = M.moe_segments


def _bf16_shift15(bits):
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64)


def _bf16_via_f16(bits):
    return np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def _allgather_reversed(shards):
    return np.concatenate([np.asarray(s) for s in shards][::-1], axis=0)


def _ag_gemm_bt(shards, b):
    a = M.allgather(shards)
    return a, M._f64(a) @ M._f64(b).T


def _ag_gemm_drop_last(shards, b):
    a = M.allgather(shards)
    a64 = M._f64(a)
    a64[-np.asarray(shards[-1]).shape[0]:] = 0
    return a, a64 @ M._f64(b)


def _rs_drop_peer(a, b, peers, world, rank):
    ms = a.shape[0] // world
    p = M._f64(a) @ M._f64(b)
    own = p[rank * ms:(rank + 1) * ms].copy()
    for j in range(world - 1):
        if j != rank:
            own += M._f64(peers[j])
    return own, [None if j == rank else p[j * ms:(j + 1) * ms].copy() for j in range(world)]


def _rs_slice0(a, b, peers, world, rank):
    ms = a.shape[0] // world
    p = M._f64(a) @ M._f64(b)
    own = p[0:ms].copy()
    for j in range(world):
        if j != rank:
            own += M._f64(peers[j])
    return own, [None if j == rank else p[j * ms:(j + 1) * ms].copy() for j in range(world)]


def _rs_outbox_own_slice(a, b, peers, world, rank):
    ms = a.shape[0] // world
    p = M._f64(a) @ M._f64(b)
    own = p[rank * ms:(rank + 1) * ms].copy()
    for j in range(world):
        if j != rank:
            own += M._f64(peers[j])
    return own, [None if j == rank else p[rank * ms:(rank + 1) * ms].copy() for j in range(world)]


def _rs_sign(a, b, peers, world, rank):
    ms = a.shape[0] // world
    p = M._f64(a) @ M._f64(b)
    own = p[rank * ms:(rank + 1) * ms].copy()
    for j in range(world):
        if j != rank:
            own -= M._f64(peers[j])
    return own, [None if j == rank else p[j * ms:(j + 1) * ms].copy() for j in range(world)]


def _ar_drop_peer(a, b, peers, world, rank):
    out = M._f64(a) @ M._f64(b)
    for j in range(1, world - 1):
        if j != rank:
            out += M._f64(peers[j])
    return out


def _ar_includes_rank_slot_as_zero_but_skips_first_peer(a, b, peers, world, rank):
    out = M._f64(a) @ M._f64(b)
    for j in range(world):
        if j != rank and j != (rank + 1) % world:
            out += M._f64(peers[j])
    return out


def _scores_f64(logits, bias):
    return np.asarray(logits, np.float64) + np.asarray(bias, np.float64)[None, :]


def _route_ties_high(logits, bias, top_k):
    s = M.moe_scores(logits, bias)
    e = s.shape[1]
    order = np.argsort(-s[:, ::-1], axis=1, kind="stable")
    return (e - 1 - order[:, :top_k]).astype(np.int32)


def _route_ascending(logits, bias, top_k):
    s = M.moe_scores(logits, bias)
    return np.argsort(s, axis=1, kind="stable")[:, :top_k].astype(np.int32)


def _route_no_bias(logits, bias, top_k):
    s = np.asarray(logits, np.float32)
    return np.argsort(-s, axis=1, kind="stable")[:, :top_k].astype(np.int32)


def _segments_first_choice_only(topk_idx, expert_begin, n_local):
    return _ORIG_SEGMENTS(topk_idx[:, :1], expert_begin, n_local)


def _segments_slot_major(topk_idx, expert_begin, n_local):
    rows = []
    for e in range(n_local):
        r = []
        for k in range(topk_idx.shape[1]):
            r.extend(np.nonzero(topk_idx[:, k] == expert_begin + e)[0].tolist())
        rows.append(np.array(r, dtype=np.int32))
    offs = np.zeros(n_local + 1, dtype=np.int32)
    offs[1:] = np.cumsum([len(r) for r in rows])
    return offs, (np.concatenate(rows).astype(np.int32) if rows else np.zeros(0, np.int32))


def _segments_ignore_begin(topk_idx, expert_begin, n_local):
    return _ORIG_SEGMENTS(topk_idx, 0, n_local)


def _segments_offsets_shifted(topk_idx, expert_begin, n_local):
    offs, st = _ORIG_SEGMENTS(topk_idx, expert_begin, n_local)
    o = offs.copy()
    o[1:-1] = offs[:-2] if len(offs) > 2 else offs[1:-1]
    return o, st


def _moe_wrong_expert_weight(tokens, logits, bias, top_k, expert_begin, n_local, w_up):
    res = M.moe_dispatch_gemm(tokens, logits, bias, top_k, expert_begin, n_local, w_up)
    offs, x = res["seg_offsets"], res["x_seg"]
    y = np.zeros_like(res["y"])
    for e in range(n_local):
        lo, hi = int(offs[e]), int(offs[e + 1])
        if hi > lo:
            y[lo:hi] = M._f64(x[lo:hi]) @ M._f64(w_up[(e + 1) % n_local])
    res["y"] = y
    return res


def _moe_wrong_token_numbering(tokens, logits, bias, top_k, expert_begin, n_local, w_up):
    res = M.moe_dispatch_gemm(tokens, logits, bias, top_k, expert_begin, n_local, w_up)
    tok_all = np.concatenate([np.asarray(t) for t in tokens[::-1]], axis=0)
    res["x_seg"] = tok_all[res["seg_token"]]
    return res


def _gelu_tanh(x):
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (x + 0.044715 * x ** 3)))


def _gelu_minus(x):
    from scipy.special import erf
    x = np.asarray(x, dtype=np.float64)
    return x * 0.5 * (1.0 - erf(x / np.sqrt(2.0)))


def _round_bf16_truncate(x):
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    scale = np.ldexp(1.0, e - 8)
    return np.trunc(x / scale) * scale


def _round_bf16_ties_up(x):
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    scale = np.ldexp(1.0, e - 8)
    return np.sign(x) * np.floor(np.abs(x) / scale + 0.5) * scale


def _mlp_no_activation(a_shards, b_up, b_down, peers, world, rank):
    a, u = M.ag_gemm(a_shards, b_up)
    h = M.round_bf16(u)
    own, outbox = M.gemm_rs(h, b_down, peers, world, rank)
    return {"a_gathered": a, "u": u, "h": h, "own": own, "outbox": outbox}


def _mlp_h_unrounded(a_shards, b_up, b_down, peers, world, rank):
    a, u = M.ag_gemm(a_shards, b_up)
    h = M.gelu(u)
    own, outbox = M.gemm_rs(h, b_down, peers, world, rank)
    return {"a_gathered": a, "u": u, "h": h, "own": own, "outbox": outbox}


def _mlp_rounded_before_gelu(a_shards, b_up, b_down, peers, world, rank):
    a, u = M.ag_gemm(a_shards, b_up)
    h = M.round_bf16(M.gelu(M.round_bf16(u)))
    own, outbox = M.gemm_rs(h, b_down, peers, world, rank)
    return {"a_gathered": a, "u": u, "h": h, "own": own, "outbox": outbox}


def _mlp_rs_rank0(a_shards, b_up, b_down, peers, world, rank):
    a, u = M.ag_gemm(a_shards, b_up)
    h = M.round_bf16(M.gelu(u))
    own, outbox = M.gemm_rs(h, b_down, peers, world, 0)
    return {"a_gathered": a, "u": u, "h": h, "own": own, "outbox": outbox}


def _ring_parts(q, k_shards, v_shards, scale):
    qf = M.bf16_to_f64(q)
    kf = np.concatenate([M.bf16_to_f64(k) for k in k_shards], axis=1)
    vf = np.concatenate([M.bf16_to_f64(v) for v in v_shards], axis=1)
    sc = 1.0 / np.sqrt(qf.shape[-1]) if not scale else float(scale)
    return qf, kf, vf, sc


def _ring_no_scale(q, k_shards, v_shards, scale=None):
    return M.ring_attention(q, k_shards, v_shards, scale=1.0)


def _ring_scale_ignored(q, k_shards, v_shards, scale=None):
    return M.ring_attention(q, k_shards, v_shards)


def _ring_local_only(q, k_shards, v_shards, scale=None):
    return M.ring_attention(q, k_shards[:1], v_shards[:1], scale=scale)


def _ring_softmax_over_queries(q, k_shards, v_shards, scale=None):
    qf, kf, vf, sc = _ring_parts(q, k_shards, v_shards, scale)
    s = sc * np.matmul(qf, np.swapaxes(kf, 1, 2))
    e = np.exp(s - s.max(axis=-2, keepdims=True))
    l_ = e.sum(axis=-2, keepdims=True)
    return np.matmul(e / l_, vf), np.log(l_.sum(axis=-1))


def _ring_unnormalized(q, k_shards, v_shards, scale=None):
    qf, kf, vf, sc = _ring_parts(q, k_shards, v_shards, scale)
    s = sc * np.matmul(qf, np.swapaxes(kf, 1, 2))
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    return np.matmul(e, vf), (m + np.log(e.sum(axis=-1, keepdims=True)))[..., 0]


def _ring_lse_without_max(q, k_shards, v_shards, scale=None):
    out, lse = M.ring_attention(q, k_shards, v_shards, scale=scale)
    qf, kf, _, sc = _ring_parts(q, k_shards, v_shards, scale)
    return out, lse - (sc * np.matmul(qf, np.swapaxes(kf, 1, 2))).max(axis=-1)


def _ring_values_are_keys(q, k_shards, v_shards, scale=None):
    return M.ring_attention(q, k_shards, k_shards, scale=scale)


def _rms_no_sqrt(x):
    x = np.asarray(x, dtype=np.float64)
    return float(np.mean(x * x)) if x.size else 0.0


def _rms_mean_abs(x):
    x = np.asarray(x, dtype=np.float64)
    return float(np.mean(np.abs(x))) if x.size else 0.0


def _rms_sum_not_mean(x):
    x = np.asarray(x, dtype=np.float64)
    return float(np.sqrt(np.sum(x * x))) if x.size else 0.0


def _rms_max(x):
    x = np.asarray(x, dtype=np.float64)
    return float(np.max(np.abs(x))) if x.size else 0.0


def _err_max_abs_out(out, ref):
    r = M.rms(ref)
    d = float(np.max(np.abs(np.asarray(out, np.float64))))
    return d / r if r > 0 else d


def _err_rms_of_out(out, ref):
    out = np.asarray(out, np.float64)
    d = float(np.max(np.abs(out - np.asarray(ref, np.float64))))
    r = M.rms(out)
    return d / r if r > 0 else d


def _err_signed(out, ref):
    d = float(np.max(np.asarray(out, np.float64) - np.asarray(ref, np.float64)))
    r = M.rms(ref)
    return d / r if r > 0 else d


def _err_mean_diff(out, ref):
    d = float(np.mean(np.abs(np.asarray(out, np.float64) - np.asarray(ref, np.float64))))
    r = M.rms(ref)
    return d / r if r > 0 else d


def _err_absolute(out, ref):
    return float(np.max(np.abs(np.asarray(out, np.float64) - np.asarray(ref, np.float64))))


MUTANTS = {
    "rms_no_sqrt": ("rms", _rms_no_sqrt),
    "rms_mean_abs": ("rms", _rms_mean_abs),
    "rms_sum_not_mean": ("rms", _rms_sum_not_mean),
    "rms_is_max_abs": ("rms", _rms_max),
    "err_max_abs_out": ("max_rel_err", _err_max_abs_out),
    "err_rms_of_out": ("max_rel_err", _err_rms_of_out),
    "err_signed_difference": ("max_rel_err", _err_signed),
    "err_mean_difference": ("max_rel_err", _err_mean_diff),
    "err_not_relative": ("max_rel_err", _err_absolute),
    "ring_no_scale": ("ring_attention", _ring_no_scale),
    "ring_scale_ignored": ("ring_attention", _ring_scale_ignored),
    "ring_local_only": ("ring_attention", _ring_local_only),
    "ring_softmax_over_queries": ("ring_attention", _ring_softmax_over_queries),
    "ring_unnormalized": ("ring_attention", _ring_unnormalized),
    "ring_lse_without_max": ("ring_attention", _ring_lse_without_max),
    "ring_values_are_keys": ("ring_attention", _ring_values_are_keys),
    "gelu_tanh_approximation": ("gelu", _gelu_tanh),
    "gelu_one_minus_erf": ("gelu", _gelu_minus),
    "round_bf16_truncates": ("round_bf16", _round_bf16_truncate),
    "round_bf16_ties_away": ("round_bf16", _round_bf16_ties_up),
    "mlp_no_activation": ("mlp_ag_rs", _mlp_no_activation),
    "mlp_h_not_rounded": ("mlp_ag_rs", _mlp_h_unrounded),
    "mlp_rounds_before_gelu": ("mlp_ag_rs", _mlp_rounded_before_gelu),
    "mlp_reduces_for_rank0": ("mlp_ag_rs", _mlp_rs_rank0),
    "bf16_shift15": ("bf16_to_f64", _bf16_shift15),
    "bf16_as_fp16": ("bf16_to_f64", _bf16_via_f16),
    "gather_reversed": ("allgather", _allgather_reversed),
    "ag_b_transposed": ("ag_gemm", _ag_gemm_bt),
    "ag_drop_last_shard": ("ag_gemm", _ag_gemm_drop_last),
    "rs_drop_peer": ("gemm_rs", _rs_drop_peer),
    "rs_slice0_always": ("gemm_rs", _rs_slice0),
    "rs_outbox_wrong_slice": ("gemm_rs", _rs_outbox_own_slice),
    "rs_sign": ("gemm_rs", _rs_sign),
    "ar_drop_peer": ("gemm_ar", _ar_drop_peer),
    "ar_skip_next_peer": ("gemm_ar", _ar_includes_rank_slot_as_zero_but_skips_first_peer),
    "scores_f64": ("moe_scores", _scores_f64),
    "route_ties_high": ("moe_route", _route_ties_high),
    "route_ascending": ("moe_route", _route_ascending),
    "route_no_bias": ("moe_route", _route_no_bias),
    "segments_first_choice": ("moe_segments", _segments_first_choice_only),
    "segments_slot_major": ("moe_segments", _segments_slot_major),
    "segments_ignore_begin": ("moe_segments", _segments_ignore_begin),
    "segments_offsets_shifted": ("moe_segments", _segments_offsets_shifted),
    "moe_wrong_expert_weight": ("moe_dispatch_gemm", _moe_wrong_expert_weight),
    "moe_wrong_token_numbering": ("moe_dispatch_gemm", _moe_wrong_token_numbering),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    attr, fn = MUTANTS[name]
    if attr in ("moe_dispatch_gemm", "ring_attention"):
        # wrap the original, so keep a handle before patching
        orig = getattr(M, attr)

        def wrapped(*a, _fn=fn, _orig=orig, **k):
            monkeypatch.setattr(M, attr, _orig)
            try:
                return _fn(*a, **k)
            finally:
                monkeypatch.setattr(M, attr, wrapped)

        monkeypatch.setattr(M, attr, wrapped)
    else:
        monkeypatch.setattr(M, attr, fn)
    impl = P.namespace_of(M)
    failed = P.run_all(impl)
    assert failed, f"no pin caught mutant {name}"


def test_unmutated_oracle_passes_every_pin():
    assert P.run_all(P.namespace_of(oracle)) == []
