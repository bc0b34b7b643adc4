"""Python binding of the fused communication+GEMM C ABI (include/mk.h).

Argument marshalling only: every step of every op runs in the HIP library
``libmk.so`` built in this directory (``python -m communication_gemm_role_amd.build``).
PyTorch provides device memory and streams.  There is no fallback: if the
library is missing, every call raises.

bf16 operands are ``torch.bfloat16`` CUDA tensors (their raw bits are what the
kernels read); fp32 operands ``torch.float32``; index outputs ``torch.int32``.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmk.so")
HOSTLIB_PATH = os.path.join(_PKG, "libmk_host.so")

MK_OK = 0
MK_ERR_INVALID_ARG = -1
MK_ERR_UNSUPPORTED = -2
MK_ERR_WORKSPACE = -3
MK_ERR_HIP = -4
MK_ERR_TIMEOUT = -5
MK_ERR_CAPACITY = -6
MK_ARRIVAL_RESIDENT = 1
MK_ARRIVAL_EMULATED = 2

EXPORTED = ["mk_ctx_create", "mk_ctx_destroy", "mk_ctx_status", "mk_ctx_reset", "mk_ctx_grid", "mk_strerror",
            "mk_selftest_flags", "mk_ag_gemm", "mk_gemm_rs", "mk_gemm_ar", "mk_moe_dispatch_gemm", "mk_mlp_ag_rs",
            "mk_ag_gemm_tune", "mk_gemm_rs_tune", "mk_gemm_ar_tune", "mk_ring_attention", "mk_ag_gemm_noalloc"]


class MkError(RuntimeError):
    def __init__(self, code: int, what: str = ""):
        self.code = code
        super().__init__(f"{what}: {strerror(code)} ({code})" if what else f"{strerror(code)} ({code})")


class mk_opts(ctypes.Structure):
    _fields_ = [
        ("n_copy_wg", ctypes.c_int),
        ("n_compute_wg", ctypes.c_int),
        ("n_reduce_wg", ctypes.c_int),
        ("arrival_mode", ctypes.c_int),
        ("arrival_order", ctypes.c_void_p),
        ("arrival_len", ctypes.c_int),
        ("arrival_unit_rows", ctypes.c_int),
        ("arrival_unit_cols", ctypes.c_int),
        ("arrival_chunk_tokens", ctypes.c_int),
        ("timeout_us", ctypes.c_int64),
        ("test_drop_unit", ctypes.c_int),
        ("trace", ctypes.c_void_p),
        ("arrival_gbps", ctypes.c_double),
    ]


@dataclass
class Opts:
    """Python-side mk_opts; ``arrival_order`` is an int32 CUDA tensor (or None); ``trace`` is an
    int64 CUDA tensor of at least ``ctx.grid * 8`` elements (or None), filled with one 8-slot
    record per workgroup as documented for ``mk_opts.trace`` (see ``trace_records``)."""
    n_copy_wg: int = 0
    n_compute_wg: int = 0
    n_reduce_wg: int = 0
    arrival_mode: int = 0
    arrival_order: object = None
    arrival_unit_rows: int = 0
    arrival_unit_cols: int = 0
    arrival_chunk_tokens: int = 0
    timeout_us: int = 0
    test_drop_unit: int = 0
    trace: object = None
    arrival_gbps: float = 0.0

    def to_c(self) -> mk_opts:
        o = mk_opts()
        o.n_copy_wg = self.n_copy_wg
        o.n_compute_wg = self.n_compute_wg
        o.n_reduce_wg = self.n_reduce_wg
        o.arrival_mode = self.arrival_mode
        if self.arrival_order is not None:
            t = self.arrival_order
            _check(t, "int32", "arrival_order")
            o.arrival_order = t.data_ptr()
            o.arrival_len = t.numel()
        o.arrival_unit_rows = self.arrival_unit_rows
        o.arrival_unit_cols = self.arrival_unit_cols
        o.arrival_chunk_tokens = self.arrival_chunk_tokens
        o.timeout_us = self.timeout_us
        o.test_drop_unit = self.test_drop_unit
        o.arrival_gbps = self.arrival_gbps
        if self.trace is not None:
            _check(self.trace, "int64", "trace")
            o.trace = self.trace.data_ptr()
        return o


_lib_handle = None


def lib() -> ctypes.CDLL:
    """The HIP library; raises if it has not been built."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m communication_gemm_role_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
        L.mk_ctx_create.argtypes = [i, sz, ctypes.POINTER(vp)]
        L.mk_ctx_destroy.argtypes = [vp]
        L.mk_ctx_status.argtypes = [vp, vp]
        L.mk_ctx_reset.argtypes = [vp, vp]
        L.mk_ctx_grid.argtypes = [vp]
        L.mk_strerror.argtypes = [i]
        L.mk_strerror.restype = ctypes.c_char_p
        L.mk_ag_gemm.argtypes = [vp, vp, vp, i, i, i, i, vp, i, vp, vp, vp]
        L.mk_gemm_rs.argtypes = [vp, vp, vp, vp, i, i, i, i, i, vp, vp, vp, vp]
        L.mk_gemm_ar.argtypes = [vp, vp, vp, vp, i, i, i, i, i, vp, vp, vp]
        L.mk_moe_dispatch_gemm.argtypes = [vp, vp, vp, i, i, i, vp, vp, i, i, i, i, vp, i, vp, vp, vp, vp, vp, i, vp]
        L.mk_selftest_flags.argtypes = [i, i, i, i, ctypes.POINTER(i64), ctypes.POINTER(i64)]
        L.mk_mlp_ag_rs.argtypes = [vp, vp, vp, i, i, i, i, vp, i, vp, i, vp, vp, vp, vp, vp, vp]
        L.mk_ag_gemm_noalloc.argtypes = [vp, vp, i, i, i, i, vp, i, vp, vp, vp, vp]
        L.mk_ring_attention.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, ctypes.c_float, vp, vp, vp, vp, vp]
        tune = [vp, i, i, vp, vp]  # candidates, count, reps, us_per_call, best
        L.mk_ag_gemm_tune.argtypes = L.mk_ag_gemm.argtypes + tune
        L.mk_gemm_rs_tune.argtypes = L.mk_gemm_rs.argtypes + tune
        L.mk_gemm_ar_tune.argtypes = L.mk_gemm_ar.argtypes + tune
        for name in ("mk_ctx_create", "mk_ctx_destroy", "mk_ctx_status", "mk_ctx_reset", "mk_ctx_grid",
                     "mk_selftest_flags", "mk_ag_gemm", "mk_gemm_rs", "mk_gemm_ar", "mk_moe_dispatch_gemm",
                     "mk_mlp_ag_rs", "mk_ag_gemm_tune", "mk_gemm_rs_tune", "mk_gemm_ar_tune", "mk_ring_attention",
                     "mk_ag_gemm_noalloc"):
            getattr(L, name).restype = i
        _lib_handle = L
    return _lib_handle


def strerror(code: int) -> str:
    try:
        return lib().mk_strerror(int(code)).decode()
    except RuntimeError:
        return f"error {code}"


def _check(t, dtype: str, name: str):
    import torch
    want = {"bf16": torch.bfloat16, "f32": torch.float32, "int32": torch.int32, "int64": torch.int64}[dtype]
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != want:
        raise TypeError(f"{name} must be {want}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream_ptr(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _ptr_array(ts: Sequence, dtype: str, name: str, allow_none_at: Optional[int] = None):
    arr = (ctypes.c_void_p * len(ts))()
    for j, t in enumerate(ts):
        if t is None:
            arr[j] = None
            continue
        _check(t, dtype, f"{name}[{j}]")
        arr[j] = t.data_ptr()
    return arr


def _opts_ptr(opts: Optional[Opts], ctx: "Context"):
    if opts is None:
        return None, None
    if opts.trace is not None and opts.trace.numel() < ctx.grid * 8:
        raise ValueError(f"trace needs {ctx.grid * 8} int64 elements (8 per workgroup), got {opts.trace.numel()}")
    o = opts.to_c()
    return ctypes.byref(o), o


class Context:
    """mk_ctx: flags, counters, status word and landing inbox on one device."""

    def __init__(self, device: int = 0, workspace_bytes: int = 0):
        h = ctypes.c_void_p()
        rc = lib().mk_ctx_create(int(device), int(workspace_bytes), ctypes.byref(h))
        if rc != MK_OK:
            raise MkError(rc, "mk_ctx_create")
        self.handle = h
        self.device = device

    @property
    def grid(self) -> int:
        return lib().mk_ctx_grid(self.handle)

    def status(self, stream=None) -> int:
        return lib().mk_ctx_status(self.handle, _stream_ptr(stream))

    def reset(self, stream=None) -> None:
        rc = lib().mk_ctx_reset(self.handle, _stream_ptr(stream))
        if rc != MK_OK:
            raise MkError(rc, "mk_ctx_reset")

    def close(self) -> None:
        if self.handle:
            lib().mk_ctx_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def mk_selftest_flags(device: int = 0, mode: int = 0, pairs: int = 64, rounds: int = 4096):
    """Cross-XCD handshake self-test (see mk.h); returns (mismatches, timeouts)."""
    mm, to = ctypes.c_int64(-1), ctypes.c_int64(-1)
    rc = lib().mk_selftest_flags(int(device), int(mode), int(pairs), int(rounds), ctypes.byref(mm), ctypes.byref(to))
    if rc != MK_OK:
        raise MkError(rc, "mk_selftest_flags")
    return int(mm.value), int(to.value)


def _call(rc: int, what: str):
    if rc != MK_OK:
        raise MkError(rc, what)


def mk_ag_gemm(ctx: Context, a_shards: Sequence, world: int, rank: int, b, a_gathered, c,
               opts: Optional[Opts] = None, stream=None) -> None:
    """AllGather+GEMM (see mk.h).  a_shards: list of [m_shard, k] bf16 (entry `rank` may be None
    or a view of a_gathered's own rows); b [k, n] bf16; a_gathered [world*m_shard, k] bf16 (out);
    c [world*m_shard, n] fp32 (out)."""
    _check(b, "bf16", "b")
    _check(a_gathered, "bf16", "a_gathered")
    _check(c, "f32", "c")
    k, n = b.shape
    m = a_gathered.shape[0]
    if a_gathered.shape[1] != k or c.shape != (m, n) or m % world:
        raise ValueError("shape mismatch")
    shards = _ptr_array(a_shards, "bf16", "a_shards") if a_shards is not None else None
    op, _keep = _opts_ptr(opts, ctx)
    _call(lib().mk_ag_gemm(ctx.handle, _stream_ptr(stream), shards, world, rank, m // world, k, b.data_ptr(), n,
                           a_gathered.data_ptr(), c.data_ptr(), op), "mk_ag_gemm")


def mk_ag_gemm_noalloc(a_shards: Sequence, world: int, rank: int, b, a_gathered, c, status,
                       opts: Optional[Opts] = None, stream=None) -> None:
    """AllGather+GEMM without a context or any allocation (see mk.h), on the current device: as
    mk_ag_gemm, with `status` a one-element int32 device tensor that receives MK_OK or the device
    fault code when the kernel ends."""
    import torch
    _check(b, "bf16", "b")
    _check(a_gathered, "bf16", "a_gathered")
    _check(c, "f32", "c")
    _check(status, "int32", "status")
    if status.numel() < 1:
        raise ValueError("status needs one int32 element")
    k, n = b.shape
    m = a_gathered.shape[0]
    if a_gathered.shape[1] != k or c.shape != (m, n) or m % world:
        raise ValueError("shape mismatch")
    shards = _ptr_array(a_shards, "bf16", "a_shards") if a_shards is not None else None
    op, _keep = None, None
    if opts is not None:
        cu = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
        if opts.trace is not None and opts.trace.numel() < cu * 8:
            raise ValueError(f"trace needs {cu * 8} int64 elements (8 per workgroup), got {opts.trace.numel()}")
        _keep = opts.to_c()
        op = ctypes.byref(_keep)
    _call(lib().mk_ag_gemm_noalloc(_stream_ptr(stream), shards, world, rank, m // world, k, b.data_ptr(), n,
                                   a_gathered.data_ptr(), c.data_ptr(), status.data_ptr(), op), "mk_ag_gemm_noalloc")


def mk_gemm_rs(ctx: Context, a, b, world: int, rank: int, peer_partials: Sequence, owned_out, outbox: Sequence,
               opts: Optional[Opts] = None, stream=None) -> None:
    """GEMM+ReduceScatter (see mk.h).  a [m, k], b [k, n] bf16; peer_partials[j] [m/world, n] fp32
    (None at rank); owned_out [m/world, n] fp32 (out); outbox[j] [m/world, n] fp32 (out, None at rank)."""
    _check(a, "bf16", "a")
    _check(b, "bf16", "b")
    _check(owned_out, "f32", "owned_out")
    m, k = a.shape
    n = b.shape[1]
    peers = _ptr_array(peer_partials, "f32", "peer_partials")
    ob = _ptr_array(outbox, "f32", "outbox")
    op, _keep = _opts_ptr(opts, ctx)
    _call(lib().mk_gemm_rs(ctx.handle, _stream_ptr(stream), a.data_ptr(), b.data_ptr(), m, n, k, world, rank, peers,
                           owned_out.data_ptr(), ob, op), "mk_gemm_rs")


def mk_gemm_ar(ctx: Context, a, b, world: int, rank: int, peer_partials: Sequence, out,
               opts: Optional[Opts] = None, stream=None) -> None:
    """GEMM+AllReduce (see mk.h).  a [m, k], b [k, n] bf16; peer_partials[j] [m, n] fp32 (None at
    rank); out [m, n] fp32 (out)."""
    _check(a, "bf16", "a")
    _check(b, "bf16", "b")
    _check(out, "f32", "out")
    m, k = a.shape
    n = b.shape[1]
    peers = _ptr_array(peer_partials, "f32", "peer_partials")
    op, _keep = _opts_ptr(opts, ctx)
    _call(lib().mk_gemm_ar(ctx.handle, _stream_ptr(stream), a.data_ptr(), b.data_ptr(), m, n, k, world, rank, peers,
                           out.data_ptr(), op), "mk_gemm_ar")


def mk_ring_attention(ctx: Context, q, k_shards: Sequence, v_shards: Sequence, rank: int, out, lse=None,
                      k_ring=None, v_ring=None, softmax_scale: float = 0.0, opts: Optional[Opts] = None,
                      stream=None) -> None:
    """Ring attention, one rank's share (see mk.h).  q [heads, s_local, d] bf16; k_shards[j] and
    v_shards[j] [heads, s_local, d] bf16 for every rank j; out [heads, s_local, d] fp32 (out);
    lse [heads, s_local] fp32 (out, optional); k_ring / v_ring [world, heads, s_local, d] bf16
    landing buffers (emulated arrival)."""
    _check(q, "bf16", "q")
    _check(out, "f32", "out")
    heads, s_local, d = q.shape
    world = len(k_shards)
    if len(v_shards) != world or out.shape != q.shape:
        raise ValueError("shape mismatch")
    if lse is not None:
        _check(lse, "f32", "lse")
        if lse.shape != (heads, s_local):
            raise ValueError("shape mismatch")
    for t in list(k_shards) + list(v_shards):
        if tuple(t.shape) != tuple(q.shape):
            raise ValueError("shape mismatch")
    for t, name in ((k_ring, "k_ring"), (v_ring, "v_ring")):
        if t is not None:
            _check(t, "bf16", name)
            if tuple(t.shape) != (world, heads, s_local, d):
                raise ValueError("shape mismatch")
    ks = _ptr_array(k_shards, "bf16", "k_shards")
    vs = _ptr_array(v_shards, "bf16", "v_shards")
    op, _keep = _opts_ptr(opts, ctx)
    _call(lib().mk_ring_attention(ctx.handle, _stream_ptr(stream), q.data_ptr(), ks, vs, world, rank, heads, s_local,
                                  d, float(softmax_scale), k_ring.data_ptr() if k_ring is not None else None,
                                  v_ring.data_ptr() if v_ring is not None else None, out.data_ptr(),
                                  lse.data_ptr() if lse is not None else None, op), "mk_ring_attention")


def _tune(fn, name, args, candidates, reps):
    cand = (ctypes.c_int * len(candidates))(*[int(c) for c in candidates])
    us = (ctypes.c_float * len(candidates))()
    best = ctypes.c_int(0)
    _call(fn(*args, cand, len(candidates), int(reps), us, ctypes.byref(best)), name)
    return best.value, [float(u) for u in us]


def mk_ag_gemm_tune(ctx: Context, a_shards: Sequence, world: int, rank: int, b, a_gathered, c, candidates: Sequence,
                    reps: int = 20, opts: Optional[Opts] = None, stream=None):
    """Role-split tuning of mk_ag_gemm (see mk.h): times each n_copy_wg in `candidates` with the
    other options of `opts`; returns (fastest n_copy_wg, [us per call or -1 per candidate])."""
    _check(b, "bf16", "b")
    _check(a_gathered, "bf16", "a_gathered")
    _check(c, "f32", "c")
    k, n = b.shape
    m = a_gathered.shape[0]
    if a_gathered.shape[1] != k or c.shape != (m, n) or m % world:
        raise ValueError("shape mismatch")
    shards = _ptr_array(a_shards, "bf16", "a_shards") if a_shards is not None else None
    op, _keep = _opts_ptr(opts, ctx)
    return _tune(lib().mk_ag_gemm_tune, "mk_ag_gemm_tune",
                 (ctx.handle, _stream_ptr(stream), shards, world, rank, m // world, k, b.data_ptr(), n,
                  a_gathered.data_ptr(), c.data_ptr(), op), candidates, reps)


def mk_gemm_rs_tune(ctx: Context, a, b, world: int, rank: int, peer_partials: Sequence, owned_out, outbox: Sequence,
                    candidates: Sequence, reps: int = 20, opts: Optional[Opts] = None, stream=None):
    """Role-split tuning of mk_gemm_rs (see mk.h); returns (fastest n_copy_wg, [us per call or -1])."""
    _check(a, "bf16", "a")
    _check(b, "bf16", "b")
    _check(owned_out, "f32", "owned_out")
    m, k = a.shape
    n = b.shape[1]
    peers = _ptr_array(peer_partials, "f32", "peer_partials")
    ob = _ptr_array(outbox, "f32", "outbox")
    op, _keep = _opts_ptr(opts, ctx)
    return _tune(lib().mk_gemm_rs_tune, "mk_gemm_rs_tune",
                 (ctx.handle, _stream_ptr(stream), a.data_ptr(), b.data_ptr(), m, n, k, world, rank, peers,
                  owned_out.data_ptr(), ob, op), candidates, reps)


def mk_gemm_ar_tune(ctx: Context, a, b, world: int, rank: int, peer_partials: Sequence, out, candidates: Sequence,
                    reps: int = 20, opts: Optional[Opts] = None, stream=None):
    """Role-split tuning of mk_gemm_ar (see mk.h); returns (fastest n_copy_wg, [us per call or -1])."""
    _check(a, "bf16", "a")
    _check(b, "bf16", "b")
    _check(out, "f32", "out")
    m, k = a.shape
    n = b.shape[1]
    peers = _ptr_array(peer_partials, "f32", "peer_partials")
    op, _keep = _opts_ptr(opts, ctx)
    return _tune(lib().mk_gemm_ar_tune, "mk_gemm_ar_tune",
                 (ctx.handle, _stream_ptr(stream), a.data_ptr(), b.data_ptr(), m, n, k, world, rank, peers,
                  out.data_ptr(), op), candidates, reps)


def mk_moe_dispatch_gemm(ctx: Context, tokens: Sequence, logits, bias, top_k: int, expert_begin: int, w_up,
                         topk_idx, seg_offsets, seg_token, x_seg, y, opts: Optional[Opts] = None,
                         stream=None) -> None:
    """MoE dispatch + grouped GEMM (see mk.h).  tokens: list of [t_local, hidden] bf16; logits
    [T, E] fp32; bias [E] fp32; w_up [n_local, hidden, ffn] bf16; outputs topk_idx [T, top_k] int32,
    seg_offsets [n_local+1] int32, seg_token [cap] int32, x_seg [cap, hidden] bf16, y [cap, ffn] fp32."""
    world = len(tokens)
    t_local, hidden = tokens[0].shape
    _check(logits, "f32", "logits")
    _check(bias, "f32", "bias")
    _check(w_up, "bf16", "w_up")
    _check(topk_idx, "int32", "topk_idx")
    _check(seg_offsets, "int32", "seg_offsets")
    _check(seg_token, "int32", "seg_token")
    _check(x_seg, "bf16", "x_seg")
    _check(y, "f32", "y")
    n_local, _, ffn = w_up.shape
    n_experts = logits.shape[1]
    cap = x_seg.shape[0]
    toks = _ptr_array(tokens, "bf16", "tokens")
    op, _keep = _opts_ptr(opts, ctx)
    _call(lib().mk_moe_dispatch_gemm(ctx.handle, _stream_ptr(stream), toks, world, t_local, hidden, logits.data_ptr(),
                                     bias.data_ptr(), n_experts, top_k, expert_begin, n_local, w_up.data_ptr(), ffn,
                                     topk_idx.data_ptr(), seg_offsets.data_ptr(), seg_token.data_ptr(),
                                     x_seg.data_ptr() if cap else None, y.data_ptr() if cap else None, cap, op),
          "mk_moe_dispatch_gemm")


def mk_mlp_ag_rs(ctx: Context, a_shards: Sequence, world: int, rank: int, b_up, b_down, peer_partials: Sequence,
                 a_gathered, h, owned_out, outbox: Sequence, opts: Optional[Opts] = None, stream=None) -> None:
    """MLP block in one launch (see mk.h): AllGather + up-projection, gelu, down-projection +
    ReduceScatter.  a_shards as in mk_ag_gemm; b_up [k, n_up], b_down [n_up, n_out] bf16;
    peer_partials[j] [m_shard, n_out] fp32 (None at rank); a_gathered [world*m_shard, k] bf16,
    h [world*m_shard, n_up] bf16, owned_out [m_shard, n_out] fp32 and outbox[j] [m_shard, n_out]
    fp32 (None at rank) are outputs."""
    _check(b_up, "bf16", "b_up")
    _check(b_down, "bf16", "b_down")
    _check(a_gathered, "bf16", "a_gathered")
    _check(h, "bf16", "h")
    _check(owned_out, "f32", "owned_out")
    k, n_up = b_up.shape
    n_out = b_down.shape[1]
    m = a_gathered.shape[0]
    if (a_gathered.shape[1] != k or b_down.shape[0] != n_up or h.shape != (m, n_up) or m % world
            or owned_out.shape != (m // world, n_out)):
        raise ValueError("shape mismatch")
    shards = _ptr_array(a_shards, "bf16", "a_shards") if a_shards is not None else None
    peers = _ptr_array(peer_partials, "f32", "peer_partials")
    ob = _ptr_array(outbox, "f32", "outbox")
    op, _keep = _opts_ptr(opts, ctx)
    _call(lib().mk_mlp_ag_rs(ctx.handle, _stream_ptr(stream), shards, world, rank, m // world, k, b_up.data_ptr(),
                             n_up, b_down.data_ptr(), n_out, peers, a_gathered.data_ptr(), h.data_ptr(),
                             owned_out.data_ptr(), ob, op), "mk_mlp_ag_rs")


__all__ = ["Context", "Opts", "MkError", "mk_selftest_flags", "mk_ag_gemm", "mk_gemm_rs", "mk_gemm_ar", "mk_moe_dispatch_gemm",
           "mk_mlp_ag_rs", "mk_ag_gemm_tune", "mk_gemm_rs_tune", "mk_gemm_ar_tune", "mk_ring_attention", "lib",
           "strerror", "MK_OK", "MK_ERR_INVALID_ARG", "MK_ERR_UNSUPPORTED", "MK_ERR_WORKSPACE", "MK_ERR_HIP",
           "MK_ERR_TIMEOUT", "MK_ERR_CAPACITY", "MK_ARRIVAL_RESIDENT", "MK_ARRIVAL_EMULATED", "EXPORTED"]
