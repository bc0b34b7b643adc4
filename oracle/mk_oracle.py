"""fp64 CPU oracle for the fused communication+GEMM ops.  TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The HIP library never calls it, and it
shares no code, table or helper with the HIP path: the only thing both sides
see is the seeded input data from ``workloads``.

What is computed is the plain definition of each fused op, as the mKernel
write-up states it (page "mKernel：多GPU、多节点融合内核库，实现GPU驱动通信",
news.chathome.org, section "五种融合内核" — the five-fused-kernels table):

* AllGather + GEMM: every rank holds one shard of A; the result is the GEMM of
  the gathered A (shards stacked by rows in rank order) with B.
* GEMM + ReduceScatter: C = A @ B, reduce-scattered: the rank that owns a row
  slice receives the sum of all ranks' partials of that slice.
* GEMM + AllReduce: C = A @ B, and every output is the sum of the partial
  outputs of all ranks.
* MoE dispatch + GEMM: tokens are routed to experts and a per-expert grouped
  GEMM runs on the tokens each expert received.

The fused kernels reach exactly these results (up to fp32 rounding order);
tile arrival order and role split change only the order of fp32 additions.
All arithmetic below is fp64 on bf16 inputs widened exactly, except where the
router score must be formed in fp32 (see ``moe_route``).

Readings where the pages are silent (each is also listed in the design notes):
  R1 the gather dimension is rows, in rank order;
  R2 in RS, rank r owns rows [r*M/W, (r+1)*M/W); peer j's partial handed to
     this rank is j's partial of *this rank's* slice; the outbox for owner j
     holds this rank's unreduced partial of j's slice (one-hop reduce-scatter);
  R3 in AR, peer j's partial covers all of [M, N];
  R4 no alpha/beta, bias or activation in any epilogue; outputs are fp32;
  R5 router score = fp32(logit + bias); top-k by descending score, equal
     scores to the lower expert id; no softmax, no capacity limit, no drop;
  R6 inside an expert's segment tokens appear in ascending global token id;
     a token routed to two local experts appears once in each segment;
  R7 gate weights are not applied to the grouped-GEMM output;
  R16 the MLP block (the page's roadmap section: the transformer-layer megakernel
     as the next step) is the AllGather + GEMM up-projection, the activation
     gelu(x) = x * Phi(x) (Phi the standard normal CDF), H stored as bf16 (the
     down-projection's operand type, rounded to nearest, ties to even), then the
     GEMM + ReduceScatter down-projection of H;
  R18 ring attention (five-fused-kernels table, Ring Attention row) is the attention of this
     rank's queries over the keys and values of every rank's sequence shard, with no mask (the
     pages name no causal variant) and the usual softmax scale 1/sqrt(head_dim) unless given;
     the ring only changes the order in which key blocks are visited, which softmax does not
     see.  ``lse`` is the natural log of the softmax denominator.
"""
from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np


# ----------------------------------------------------------------------------------------
# bf16 widening (exact)
# ----------------------------------------------------------------------------------------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp64.  bf16 is the upper half of an fp32 word, so the
    widening is exact: shift into the high 16 bits, reinterpret as fp32, widen."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _f64(x: np.ndarray) -> np.ndarray:
    if x.dtype == np.uint16:
        return bf16_to_f64(x)
    return np.asarray(x, dtype=np.float64)


# ----------------------------------------------------------------------------------------
# AllGather + GEMM
# ----------------------------------------------------------------------------------------
def allgather(a_shards: Sequence[np.ndarray]) -> np.ndarray:
    """Gathered A: the shards stacked by rows in rank order (reading R1).  Bitwise."""
    return np.concatenate([np.asarray(s) for s in a_shards], axis=0)


def ag_gemm(a_shards: Sequence[np.ndarray], b: np.ndarray):
    """AllGather+GEMM (five-fused-kernels table, AllGather + GEMM row).

    Returns (a_gathered as the input dtype, C = A_gathered @ B in fp64)."""
    a = allgather(a_shards)
    return a, _f64(a) @ _f64(b)


# ----------------------------------------------------------------------------------------
# GEMM + ReduceScatter
# ----------------------------------------------------------------------------------------
def gemm_rs(a: np.ndarray, b: np.ndarray, peer_partials: Sequence[Optional[np.ndarray]], world: int, rank: int):
    """GEMM+ReduceScatter (five-fused-kernels table, GEMM + ReduceScatter row), one rank's share.

    P = A @ B is this rank's partial of the whole output.  Reading R2:
      own        = P[slice rank] + sum over j != rank of peer_partials[j]
      outbox[j]  = P[slice j]                 for j != rank  (None at j == rank)
    Returns (own, outbox list)."""
    m = a.shape[0]
    if m % world:
        raise ValueError("rows must divide by world")
    ms = m // world
    p = _f64(a) @ _f64(b)
    own = p[rank * ms:(rank + 1) * ms].copy()
    for j in range(world):
        if j != rank:
            own += _f64(peer_partials[j])
    outbox = [None if j == rank else p[j * ms:(j + 1) * ms].copy() for j in range(world)]
    return own, outbox


# ----------------------------------------------------------------------------------------
# GEMM + AllReduce
# ----------------------------------------------------------------------------------------
def gemm_ar(a: np.ndarray, b: np.ndarray, peer_partials: Sequence[Optional[np.ndarray]], world: int, rank: int):
    """GEMM+AllReduce (five-fused-kernels table, GEMM + AllReduce row), one rank's share.

    out = A @ B + sum over j != rank of peer_partials[j] (reading R3).  The shape of
    the reduction tree only changes rounding, which fp64 makes immaterial."""
    out = _f64(a) @ _f64(b)
    for j in range(world):
        if j != rank:
            out += _f64(peer_partials[j])
    return out


# ----------------------------------------------------------------------------------------
# MLP block (roadmap section: transformer-layer megakernel), reading R16
# ----------------------------------------------------------------------------------------
def gelu(x: np.ndarray) -> np.ndarray:
    """gelu(x) = x * Phi(x) = x * (1 + erf(x / sqrt 2)) / 2, in fp64 (erf from scipy)."""
    from scipy.special import erf
    x = np.asarray(x, dtype=np.float64)
    return x * 0.5 * (1.0 + erf(x / np.sqrt(2.0)))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Nearest bf16 value of each fp64 value, ties to even (returned in fp64, exact).  bf16 keeps
    8 significant bits: with x = f * 2**e, 0.5 <= |f| < 1, the spacing is 2**(e - 8), and
    np.rint rounds halves to even.  Normal range only (|x| >= 2**-126 or 0)."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    scale = np.ldexp(1.0, e - 8)
    return np.rint(x / scale) * scale


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of values already representable in bf16 (e.g. round_bf16's output)."""
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def mlp_ag_rs(a_shards: Sequence[np.ndarray], b_up: np.ndarray, b_down: np.ndarray,
              peer_partials: Sequence[Optional[np.ndarray]], world: int, rank: int) -> dict:
    """MLP block, one rank's share (reading R16): A gathered as in ag_gemm, U = A @ B_up,
    H = bf16(gelu(U)), then the GEMM + ReduceScatter of H @ B_down as in gemm_rs.
    Returns dict(a_gathered, u (fp64), h (fp64 values of the bf16 H), own, outbox)."""
    a, u = ag_gemm(a_shards, b_up)
    h = round_bf16(gelu(u))
    own, outbox = gemm_rs(h, b_down, peer_partials, world, rank)
    return {"a_gathered": a, "u": u, "h": h, "own": own, "outbox": outbox}


# ----------------------------------------------------------------------------------------
# Ring attention (five-fused-kernels table, Ring Attention row), reading R18
# ----------------------------------------------------------------------------------------
def ring_attention(q: np.ndarray, k_shards: Sequence[np.ndarray], v_shards: Sequence[np.ndarray],
                   scale: Optional[float] = None):
    """One rank's share: q [H, S, D] and every rank's k/v shards [H, S_j, D] as bf16 bits.
    Scores s[h, i, t] = scale * q[h, i] . k[h, t] over the keys t of all shards in rank order,
    out[h, i] = sum_t softmax_t(s[h, i, :]) v[h, t], lse[h, i] = log sum_t exp(s[h, i, t]).
    Returns (out [H, S, D], lse [H, S]) in fp64."""
    qf = bf16_to_f64(q)
    kf = np.concatenate([bf16_to_f64(k) for k in k_shards], axis=1)
    vf = np.concatenate([bf16_to_f64(v) for v in v_shards], axis=1)
    d = qf.shape[-1]
    sc = 1.0 / np.sqrt(d) if not scale else float(scale)
    s = sc * np.matmul(qf, np.swapaxes(kf, 1, 2))
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    l_ = e.sum(axis=-1, keepdims=True)
    out = np.matmul(e, vf) / l_
    lse = (m + np.log(l_))[..., 0]
    return out, lse


# ----------------------------------------------------------------------------------------
# MoE dispatch + grouped GEMM
# ----------------------------------------------------------------------------------------
def moe_scores(logits: np.ndarray, bias: np.ndarray) -> np.ndarray:
    """Router score s[t, e] = fp32(logit[t, e] + bias[e]) — one IEEE fp32 add (reading R5)."""
    lg = np.asarray(logits, dtype=np.float32)
    bs = np.asarray(bias, dtype=np.float32)
    return (lg + bs[None, :]).astype(np.float32)


def moe_route(logits: np.ndarray, bias: np.ndarray, top_k: int) -> np.ndarray:
    """Top-k experts per token: descending fp32 score, equal scores to the lower id.

    A stable sort on -score keeps equal scores in ascending expert id."""
    s = moe_scores(logits, bias)
    order = np.argsort(-s, axis=1, kind="stable")
    return order[:, :top_k].astype(np.int32)


def moe_segments(topk_idx: np.ndarray, expert_begin: int, n_local: int):
    """Per-local-expert segments (readings R6): returns (seg_offsets [n_local+1], seg_token [R]).

    Segment e holds, in ascending global token id, every token whose top-k list
    contains expert expert_begin + e."""
    rows = []
    for e in range(n_local):
        hit = np.any(topk_idx == expert_begin + e, axis=1)
        rows.append(np.nonzero(hit)[0].astype(np.int32))
    counts = np.array([len(r) for r in rows], dtype=np.int64)
    offs = np.zeros(n_local + 1, dtype=np.int32)
    offs[1:] = np.cumsum(counts)
    seg_token = np.concatenate(rows).astype(np.int32) if rows else np.zeros(0, np.int32)
    return offs, seg_token


def moe_dispatch_gemm(tokens: Sequence[np.ndarray], logits: np.ndarray, bias: np.ndarray, top_k: int,
                      expert_begin: int, n_local: int, w_up: np.ndarray):
    """MoE dispatch + grouped GEMM (five-fused-kernels table, MoE Dispatch + GEMM row).

    Returns dict(topk_idx, seg_offsets, seg_token, x_seg (input dtype), y (fp64)).
    x_seg row i is the token seg_token[i] (all ranks' tokens numbered rank-major);
    y[segment e] = x_seg[segment e] @ W_up[e] (reading R7: no gate weights)."""
    tok_all = np.concatenate([np.asarray(t) for t in tokens], axis=0)
    topk = moe_route(logits, bias, top_k)
    offs, seg_token = moe_segments(topk, expert_begin, n_local)
    x = tok_all[seg_token]
    y = np.zeros((len(seg_token), w_up.shape[2]), dtype=np.float64)
    for e in range(n_local):
        lo, hi = int(offs[e]), int(offs[e + 1])
        if hi > lo:
            y[lo:hi] = _f64(x[lo:hi]) @ _f64(w_up[e])
    return {"topk_idx": topk, "seg_offsets": offs, "seg_token": seg_token, "x_seg": x, "y": y}


# ----------------------------------------------------------------------------------------
# acceptance
# ----------------------------------------------------------------------------------------
def rms(x: np.ndarray) -> float:
    x = np.asarray(x, dtype=np.float64)
    return float(np.sqrt(np.mean(x * x))) if x.size else 0.0


def max_rel_err(out: np.ndarray, ref: np.ndarray) -> float:
    """max |out - ref| / RMS(ref) over one output buffer."""
    ref = np.asarray(ref, dtype=np.float64)
    d = np.max(np.abs(np.asarray(out, dtype=np.float64) - ref)) if ref.size else 0.0
    r = rms(ref)
    return float(d / r) if r > 0 else float(d)


__all__ = [
    "bf16_to_f64", "allgather", "ag_gemm", "gemm_rs", "gemm_ar", "moe_scores", "moe_route", "moe_segments",
    "moe_dispatch_gemm", "gelu", "round_bf16", "bf16_bits", "mlp_ag_rs", "ring_attention", "rms", "max_rel_err",
]
