"""Seeded synthetic inputs for the five workloads of the fused comm+GEMM path.

This module only draws random numbers and lays them out; it holds none of the
arithmetic the fused ops compute.  Both the fp64 oracle (via the tests) and the
HIP path (via the Python binding) are fed from here, so a parity test compares
the two on bit-identical inputs.

Every tensor comes from ``numpy.random.default_rng(SeedSequence([cfg, tensor_id, run]))``.
Floating-point inputs are drawn in fp32; bf16 inputs are the fp32 draws rounded
to bf16 (round to nearest, ties to even, on the fp32 bit pattern) and are
handed around as ``uint16`` arrays of raw bf16 bits.  fp32 inputs (peer
partials, router logits and bias) stay fp32.

Workload shapes follow the five synthetic configurations of the fused-kernel
description (mKernel, "Five fused kernels" table on the news.chathome.org page:
AllGather+GEMM, GEMM+ReduceScatter, GEMM+AllReduce, MoE dispatch+GEMM).  The
pages fix no sizes; the sizes here are the ones this project measures.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import List, Optional

import numpy as np

# workload ids used as the first SeedSequence word
CFG_AG_TINY = 1
CFG_AG = 2
CFG_RS = 3
CFG_AR = 4
CFG_MOE = 5
CFG_MLP = 6
CFG_RING = 7
ORDER_STREAM = 99  # second SeedSequence word for arrival orders


def rng(cfg: int, tensor_id: int, run: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(cfg), int(tensor_id), int(run)]))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)  # keep NaN quiet
    return rounded


def normal_bf16(cfg: int, tensor_id: int, run: int, shape, sigma: float) -> np.ndarray:
    x = rng(cfg, tensor_id, run).standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return f32_to_bf16_bits(x)


def normal_f32(cfg: int, tensor_id: int, run: int, shape, sigma: float = 1.0) -> np.ndarray:
    x = rng(cfg, tensor_id, run).standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return x


def int_bf16(cfg: int, tensor_id: int, run: int, shape, lo: int = -4, hi: int = 4) -> np.ndarray:
    """Integer values in [lo, hi] (exact in bf16) as bf16 bits."""
    x = rng(cfg, tensor_id, run).integers(lo, hi + 1, size=shape).astype(np.float32)
    return f32_to_bf16_bits(x)


def int_f32(cfg: int, tensor_id: int, run: int, shape, lo: int = -8, hi: int = 8) -> np.ndarray:
    return rng(cfg, tensor_id, run).integers(lo, hi + 1, size=shape).astype(np.float32)


def permutation(cfg: int, trial: int, n: int) -> np.ndarray:
    """Seeded arrival permutation of n units (int32)."""
    return rng(cfg, ORDER_STREAM, trial).permutation(n).astype(np.int32)


# --------------------------------------------------------------------------------------
# AllGather + GEMM
# --------------------------------------------------------------------------------------
@dataclass(frozen=True)
class AGShape:
    world: int
    m_shard: int
    k: int
    n: int
    sigma_a: float = 1.0
    sigma_b: float = 1.0
    unit_rows: int = 64
    unit_cols: int = 64
    rank: int = 0
    cfg: int = CFG_AG_TINY

    @property
    def m(self) -> int:
        return self.world * self.m_shard

    @property
    def n_unit_rows(self) -> int:
        return self.m // self.unit_rows

    @property
    def n_unit_cols(self) -> int:
        return self.k // self.unit_cols

    @property
    def flops(self) -> float:
        return 2.0 * self.m * self.n * self.k


AG_TINY = AGShape(world=4, m_shard=64, k=256, n=256, sigma_a=1.0, sigma_b=1.0 / 16.0,
                  unit_rows=64, unit_cols=64, cfg=CFG_AG_TINY)
AG_MLP = AGShape(world=8, m_shard=1024, k=4096, n=1792, sigma_a=1.0, sigma_b=0.02,
                 unit_rows=128, unit_cols=128, cfg=CFG_AG)


def gen_ag(shape: AGShape, run: int = 0, kind: str = "normal") -> dict:
    """A shards (tensor ids 0..W-1) and B (tensor id W)."""
    W = shape.world
    if kind == "normal":
        shards = [normal_bf16(shape.cfg, r, run, (shape.m_shard, shape.k), shape.sigma_a) for r in range(W)]
        b = normal_bf16(shape.cfg, W, run, (shape.k, shape.n), shape.sigma_b)
    elif kind == "int":
        shards = [int_bf16(shape.cfg, r, run, (shape.m_shard, shape.k)) for r in range(W)]
        b = int_bf16(shape.cfg, W, run, (shape.k, shape.n))
    else:
        raise ValueError(kind)
    return {"a_shards": shards, "b": b}


def ag_peer_units(shape: AGShape, rank: Optional[int] = None) -> np.ndarray:
    """Ids of the arrival units that come from peers (rank-major, then row-major)."""
    rank = shape.rank if rank is None else rank
    per_shard_rows = shape.m_shard // shape.unit_rows
    ids = []
    for r in range(shape.world):
        if r == rank:
            continue
        for ur in range(r * per_shard_rows, (r + 1) * per_shard_rows):
            for uc in range(shape.n_unit_cols):
                ids.append(ur * shape.n_unit_cols + uc)
    return np.asarray(ids, dtype=np.int32)


def ag_arrival_order(shape: AGShape, trial: int = 0, variant: str = "flat", rank: Optional[int] = None) -> np.ndarray:
    """Arrival order of the peer units.

    flat        one seeded permutation of all peer units
    shard       shards in seeded order, units shuffled within each shard
    identity    rank-major, row-major
    reversed    identity reversed
    """
    units = ag_peer_units(shape, rank)
    if variant == "identity":
        return units.copy()
    if variant == "reversed":
        return units[::-1].copy()
    if variant == "flat":
        return units[permutation(shape.cfg, trial, len(units))]
    if variant == "shard":
        rank = shape.rank if rank is None else rank
        per = (shape.m_shard // shape.unit_rows) * shape.n_unit_cols
        peers = [r for r in range(shape.world) if r != rank]
        g = rng(shape.cfg, ORDER_STREAM, 1000 + trial)
        out = []
        for pi in g.permutation(len(peers)):
            block = units[pi * per:(pi + 1) * per]
            out.append(block[g.permutation(len(block))])
        return np.concatenate(out).astype(np.int32) if out else units.copy()
    raise ValueError(variant)


# --------------------------------------------------------------------------------------
# GEMM + ReduceScatter / GEMM + AllReduce
# --------------------------------------------------------------------------------------
@dataclass(frozen=True)
class RedShape:
    m: int
    n: int
    k: int
    world: int
    sigma_a: float = 1.0
    sigma_b: float = 0.02
    sigma_q: float = 1.0
    unit_rows: int = 128
    unit_cols: int = 128
    rank: int = 0
    cfg: int = CFG_RS

    @property
    def m_slice(self) -> int:
        return self.m // self.world

    @property
    def flops(self) -> float:
        return 2.0 * self.m * self.n * self.k


# 64x128 fp32 landing units (32 KiB): a batch of the copy ring holds whole units, and the ring moves
# 4 KiB per wave on the eight-wave wide tile (32 KiB slots) and 8 KiB per wave on the decode-like
# AR's four-wave tile
RS_DOWN = RedShape(m=8192, n=4096, k=1792, world=8, sigma_a=1.0, sigma_b=0.02, sigma_q=1.0, unit_rows=64,
                   unit_cols=128, cfg=CFG_RS)
AR_DECODE = RedShape(m=256, n=8192, k=1024, world=8, sigma_a=1.0, sigma_b=0.02, sigma_q=1.0, unit_rows=64,
                     unit_cols=128, cfg=CFG_AR)
# small versions (same structure, a few tiles and a ragged count of units) for parity at CPU speed
RS_SMALL = RedShape(m=1024, n=768, k=320, world=8, unit_rows=64, unit_cols=64, cfg=CFG_RS)
AR_SMALL = RedShape(m=192, n=1152, k=448, world=8, unit_rows=64, unit_cols=64, cfg=CFG_AR)


def gen_reduce(shape: RedShape, op: str, run: int = 0, kind: str = "normal") -> dict:
    """A (id 0), B (id 1), peer partials Q_j (id 2 + j) for j != rank.

    op == "rs": Q_j is peer j's partial of this rank's owned row slice, [m/W, n].
    op == "ar": Q_j is peer j's full partial, [m, n].
    """
    rows = shape.m_slice if op == "rs" else shape.m
    if kind == "normal":
        a = normal_bf16(shape.cfg, 0, run, (shape.m, shape.k), shape.sigma_a)
        b = normal_bf16(shape.cfg, 1, run, (shape.k, shape.n), shape.sigma_b)
        peers = [None if j == shape.rank else normal_f32(shape.cfg, 2 + j, run, (rows, shape.n), shape.sigma_q)
                 for j in range(shape.world)]
    elif kind == "int":
        a = int_bf16(shape.cfg, 0, run, (shape.m, shape.k))
        b = int_bf16(shape.cfg, 1, run, (shape.k, shape.n))
        peers = [None if j == shape.rank else int_f32(shape.cfg, 2 + j, run, (rows, shape.n))
                 for j in range(shape.world)]
    else:
        raise ValueError(kind)
    return {"a": a, "b": b, "peers": peers}


def reduce_peer_units(shape: RedShape, op: str) -> np.ndarray:
    """Landing units of the peer partials: id = j_index * units_per_peer + unit, j over peers in rank order."""
    rows = shape.m_slice if op == "rs" else shape.m
    per = (rows // shape.unit_rows) * (shape.n // shape.unit_cols)
    return np.arange((shape.world - 1) * per, dtype=np.int32)


def reduce_arrival_order(shape: RedShape, op: str, trial: int = 0, variant: str = "flat") -> np.ndarray:
    units = reduce_peer_units(shape, op)
    if variant == "identity":
        return units.copy()
    if variant == "reversed":
        return units[::-1].copy()
    if variant == "flat":
        return units[permutation(shape.cfg, trial, len(units))]
    raise ValueError(variant)


# --------------------------------------------------------------------------------------
# MoE dispatch + grouped GEMM
# --------------------------------------------------------------------------------------
@dataclass(frozen=True)
class MoEShape:
    world: int
    t_local: int
    hidden: int
    n_experts: int
    top_k: int
    expert_begin: int
    n_local: int
    ffn: int
    sigma_w: float = 0.02
    chunk_tokens: int = 64
    cfg: int = CFG_MOE

    @property
    def tokens(self) -> int:
        return self.world * self.t_local

    @property
    def n_chunks(self) -> int:
        return self.world * (self.t_local // self.chunk_tokens)

    @property
    def capacity(self) -> int:
        return self.tokens * min(self.top_k, self.n_local)

    def flops(self, routed_rows: int) -> float:
        return 2.0 * routed_rows * self.hidden * self.ffn


MOE_FULL = MoEShape(world=8, t_local=4096, hidden=4096, n_experts=64, top_k=2, expert_begin=0, n_local=8, ffn=1536)
MOE_SMALL = MoEShape(world=8, t_local=192, hidden=512, n_experts=16, top_k=2, expert_begin=0, n_local=4, ffn=320)


def gen_moe(shape: MoEShape, run: int = 0, kind: str = "normal", bias_override: Optional[np.ndarray] = None) -> dict:
    """tokens_r (ids 0..W-1), logits (id W), bias (id W+1), W_up per local expert (ids W+2+e)."""
    W = shape.world
    if kind == "normal":
        tokens = [normal_bf16(shape.cfg, r, run, (shape.t_local, shape.hidden), 1.0) for r in range(W)]
        w_up = np.stack([normal_bf16(shape.cfg, W + 2 + e, run, (shape.hidden, shape.ffn), shape.sigma_w)
                         for e in range(shape.n_local)])
    elif kind == "int":
        tokens = [int_bf16(shape.cfg, r, run, (shape.t_local, shape.hidden)) for r in range(W)]
        w_up = np.stack([int_bf16(shape.cfg, W + 2 + e, run, (shape.hidden, shape.ffn)) for e in range(shape.n_local)])
    else:
        raise ValueError(kind)
    logits = normal_f32(shape.cfg, W, run, (shape.tokens, shape.n_experts))
    bias = normal_f32(shape.cfg, W + 1, run, (shape.n_experts,))
    if bias_override is not None:
        bias = np.asarray(bias_override, dtype=np.float32).copy()
    return {"tokens": tokens, "logits": logits, "bias": bias, "w_up": w_up}


def moe_arrival_order(shape: MoEShape, trial: int = 0, variant: str = "flat") -> np.ndarray:
    """Arrival order of (rank, 64-token block) chunks; chunk id = global first token / chunk_tokens."""
    n = shape.n_chunks
    if variant == "identity":
        return np.arange(n, dtype=np.int32)
    if variant == "reversed":
        return np.arange(n, dtype=np.int32)[::-1].copy()
    if variant == "flat":
        return permutation(shape.cfg, trial, n)
    raise ValueError(variant)


__all__ = [
    "AGShape", "RedShape", "MoEShape", "AG_TINY", "AG_MLP", "RS_DOWN", "AR_DECODE", "RS_SMALL", "AR_SMALL",
    "MOE_FULL", "MOE_SMALL", "gen_ag", "gen_reduce", "gen_moe", "ag_peer_units", "ag_arrival_order",
    "reduce_peer_units", "reduce_arrival_order", "moe_arrival_order", "f32_to_bf16_bits", "normal_bf16",
    "normal_f32", "int_bf16", "int_f32", "permutation", "rng", "replace",
]


# --------------------------------------------------------------------------------------
# MLP block: AllGather + up-projection, gelu, down-projection + ReduceScatter
# --------------------------------------------------------------------------------------
@dataclass(frozen=True)
class MLPShape:
    """The up-projection is the AllGather + GEMM shape (world, m_shard, k, n_up); the
    down-projection is GEMM + ReduceScatter over [world*m_shard, n_out] with K = n_up."""
    world: int
    m_shard: int
    k: int
    n_up: int
    n_out: int
    sigma_a: float = 1.0
    sigma_up: float = 1.0 / 16.0
    sigma_down: float = 1.0 / 16.0
    sigma_q: float = 1.0
    unit_rows: int = 64
    unit_cols: int = 64
    rank: int = 0
    cfg: int = CFG_MLP

    @property
    def m(self) -> int:
        return self.world * self.m_shard

    @property
    def ag(self) -> AGShape:
        """The up-projection's AllGather + GEMM shape (for its arrival units and orders)."""
        return AGShape(world=self.world, m_shard=self.m_shard, k=self.k, n=self.n_up, unit_rows=self.unit_rows,
                       unit_cols=self.unit_cols, rank=self.rank, cfg=self.cfg)

    @property
    def flops(self) -> float:
        return 2.0 * self.m * self.k * self.n_up + 2.0 * self.m * self.n_up * self.n_out


# several tiles and ragged tails in both phases (n_up = 1.75 tiles, n_out = 1.25 tiles)
MLP_SMALL = MLPShape(world=4, m_shard=256, k=256, n_up=448, n_out=320)
# the AllGather + GEMM up-projection of the MLP workload followed by the ReduceScatter
# down-projection of the row-parallel workload (its K is the up-projection's N)
MLP_FULL = MLPShape(world=8, m_shard=1024, k=4096, n_up=1792, n_out=4096, sigma_up=0.02, sigma_down=0.02,
                    unit_rows=128, unit_cols=128)


def gen_mlp(shape: MLPShape, run: int = 0, kind: str = "normal") -> dict:
    """A shards (tensor ids 0..W-1), B_up (W), B_down (W+1), peer partials of this rank's rows of the
    down-projection (W+2+j).  kind "int": A in {0, 16}, B_up in {0, 1}, so every up-projection
    output is 0 or a multiple of 16 (gelu is then the identity to fp64 and bf16 precision for
    k <= 256), B_down and the partials small integers: every result is exact."""
    W, ms = shape.world, shape.m_shard
    if kind == "normal":
        shards = [normal_bf16(shape.cfg, r, run, (ms, shape.k), shape.sigma_a) for r in range(W)]
        b_up = normal_bf16(shape.cfg, W, run, (shape.k, shape.n_up), shape.sigma_up)
        b_down = normal_bf16(shape.cfg, W + 1, run, (shape.n_up, shape.n_out), shape.sigma_down)
        peers = [None if j == shape.rank else normal_f32(shape.cfg, W + 2 + j, run, (ms, shape.n_out), shape.sigma_q)
                 for j in range(W)]
    elif kind == "int":
        if shape.k > 256:
            raise ValueError("integer MLP inputs stay exact only for k <= 256")
        shards = [f32_to_bf16_bits(16.0 * rng(shape.cfg, r, run).integers(0, 2, size=(ms, shape.k)).astype(np.float32))
                  for r in range(W)]
        b_up = int_bf16(shape.cfg, W, run, (shape.k, shape.n_up), 0, 1)
        b_down = int_bf16(shape.cfg, W + 1, run, (shape.n_up, shape.n_out), -2, 2)
        peers = [None if j == shape.rank else int_f32(shape.cfg, W + 2 + j, run, (ms, shape.n_out))
                 for j in range(W)]
    else:
        raise ValueError(kind)
    return {"a_shards": shards, "b_up": b_up, "b_down": b_down, "peers": peers}


# --------------------------------------------------------------------------------------
# Ring attention
# --------------------------------------------------------------------------------------
@dataclass(frozen=True)
class RingShape:
    """Sequence-parallel attention: every rank holds s_local queries, keys and values of each
    head; rank `rank`'s share attends over all world * s_local keys."""
    world: int
    heads: int
    s_local: int
    d: int = 128
    sigma: float = 1.0
    rank: int = 0
    cfg: int = CFG_RING

    @property
    def n_blk(self) -> int:
        return self.s_local // 64

    @property
    def flops(self) -> float:
        """Q K^T and P V: 4 * heads * s_local * (world * s_local) * d."""
        return 4.0 * self.heads * self.s_local * self.world * self.s_local * self.d


# several query tiles and key blocks per head
RING_SMALL = RingShape(world=4, heads=2, s_local=256, rank=1)
# 8 ranks x 4096 tokens (32768 in all), 8 heads of 128: one 128-query item per CU
RING_FULL = RingShape(world=8, heads=8, s_local=4096)


def gen_ring(shape: RingShape, run: int = 0) -> dict:
    """q (tensor id 0), k shards (1 + j), v shards (1 + world + j), N(0, sigma^2) rounded to bf16."""
    sz = (shape.heads, shape.s_local, shape.d)
    q = normal_bf16(shape.cfg, 0, run, sz, shape.sigma)
    ks = [normal_bf16(shape.cfg, 1 + j, run, sz, shape.sigma) for j in range(shape.world)]
    vs = [normal_bf16(shape.cfg, 1 + shape.world + j, run, sz, shape.sigma) for j in range(shape.world)]
    return {"q": q, "k_shards": ks, "v_shards": vs}


def ring_peer_units(shape: RingShape) -> np.ndarray:
    """Unit ids of the peers' 64-key K and V blocks in the ring's order: step t = 1, 2, ... brings
    rank (rank - t) mod world, head by head, block by block, K (even id) before V (odd id)."""
    per = shape.heads * shape.n_blk * 2
    out = []
    for t in range(1, shape.world):
        j = (shape.rank - t) % shape.world
        out.extend(range(j * per, (j + 1) * per))
    return np.asarray(out, dtype=np.int32)


def ring_arrival_order(shape: RingShape, trial: int = 0, variant: str = "ring") -> np.ndarray:
    units = ring_peer_units(shape)
    if variant == "ring":
        return units.copy()
    if variant == "flat":
        return units[permutation(shape.cfg, trial, len(units))]
    if variant == "reversed":
        return units[::-1].copy()
    raise ValueError(variant)
