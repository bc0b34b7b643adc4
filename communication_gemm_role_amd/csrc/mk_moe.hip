// MoE token dispatch + per-expert grouped GEMM, one rank's share, as one persistent launch.
//
// Operation (mKernel write-up, news.chathome.org page, five-fused-kernels table, MoE
// Dispatch + GEMM row): tokens are routed to the ranks of their experts and the
// per-expert grouped GEMM runs in the same kernel on tokens as they arrive, with no
// staging-buffer round trip.  Here this rank owns experts [expert_begin, +n_local); the
// tokens of every rank are device buffers and their arrival is the copy role.
//
// Phases and roles (workgroup ids [0, n_copy) route and copy; the rest compute):
//   route   each route wave takes 64-token chunks: score = fp32(logit + bias) for every
//           expert, top-k by descending score with equal scores to the lower id (insertion
//           in ascending expert order, replacing only on a strictly larger score), writes
//           topk_idx and the chunk's row count per local expert.
//   scan    the last route workgroup to finish (arrival counter) turns the per-chunk counts
//           into segment offsets and per-(chunk, expert) first slots: an exclusive scan in
//           chunk order, i.e. ascending global token id inside each expert's segment.  It
//           also numbers the m-tiles of every segment, then raises the scan flag.
//   copy    after the scan flag, chunks in the caller's arrival order: every routed
//           (token, local expert) row is copied straight into its final slot of x_seg, its
//           token id into seg_token, and the per-m-tile landed-row counter is raised.
//   compute after the scan flag, (m-tile, n-tile) jobs of the ragged grouped GEMM: an m-tile
//           runs once all of its rows have landed; y[slot] = x_seg[slot] @ w_up[expert].
// Route/copy workgroups never wait on compute workgroups, and have the lowest ids.  The
// last workgroup to exit re-zeroes the counters, so every call starts from zero.
#include "mk_internal.h"
#include "mk_gemm_tile.hpp"

namespace mk {

using MoeTile = TileGemmDma<128, 256, 2, 2>;
constexpr int MOE_KMAX = 8;

int moe_tile_m() { return MoeTile::BM; }
int moe_tile_n() { return MoeTile::BN; }

struct MoeShared {
  int list_tok[64 * MOE_KMAX];
  int list_slot[64 * MOE_KMAX];
  int n_list;
  int ok;
  int is_last;
  int seg_off[65];
  int tile_base[65];
  int totals[64];
};

__device__ __forceinline__ uint32_t* moe_misc(const MoeParams& p) { return p.counters + p.off_misc; }
// misc layout: [0] route-done arrivals, [1] exits, [2 .. 2+n_local] m-tile base per expert (prefix)

// ------------------------------------------------------------------------------------------
// route (one wave per 64-token chunk)
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ void moe_route_chunk(const MoeParams& p, int chunk, int lane) {
  const int t = chunk * 64 + lane;
  float tv[MOE_KMAX];
  int ti[MOE_KMAX];
#pragma unroll
  for (int j = 0; j < MOE_KMAX; ++j) {
    tv[j] = 0.f;
    ti[j] = -1;
  }
  const auto lr = make_rsrc(p.logits + (size_t)t * p.n_experts, (uint32_t)p.n_experts * 4u);
  const auto brs = make_rsrc(p.bias, (uint32_t)p.n_experts * 4u);
  for (int e0 = 0; e0 < p.n_experts; e0 += 4) {
    const f32x4 lg = __builtin_bit_cast(f32x4, bload16(lr, (uint32_t)e0 * 4u));
    const f32x4 bs = __builtin_bit_cast(f32x4, bload16(brs, (uint32_t)e0 * 4u));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float v = lg[q] + bs[q];  // one fp32 add, round to nearest even
      int id = e0 + q;
#pragma unroll
      for (int j = 0; j < MOE_KMAX; ++j) {
        if (j < p.top_k) {
          const bool take = (id >= 0) && ((ti[j] < 0) || (v > tv[j]));  // empty slots sit at the end
          if (take) {
            const float fv = tv[j];
            const int fi = ti[j];
            tv[j] = v;
            ti[j] = id;
            v = fv;
            id = fi;
          }
        }
      }
    }
  }
  const auto tr = make_rsrc(p.topk_idx + (size_t)t * p.top_k, (uint32_t)p.top_k * 4u);
#pragma unroll
  for (int j = 0; j < MOE_KMAX; ++j)
    if (j < p.top_k) bstore4_sc1(tr, (uint32_t)j * 4u, (uint32_t)ti[j]);
  // rows of this chunk per local expert
  uint32_t* cnt = p.counters + p.off_chunk_cnt + (size_t)chunk * p.n_local;
  for (int el = 0; el < p.n_local; ++el) {
    const int e = p.expert_begin + el;
    bool hit = false;
#pragma unroll
    for (int j = 0; j < MOE_KMAX; ++j)
      if (j < p.top_k) hit |= (ti[j] == e);
    const uint64_t m = __ballot(hit);
    if (lane == 0) __hip_atomic_store(cnt + el, (uint32_t)__popcll(m), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Exclusive scan of the per-chunk counts (run by one workgroup, the last router).
__device__ __forceinline__ void moe_scan(const MoeParams& p, MoeShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint32_t* cnt = p.counters + p.off_chunk_cnt;
  // pass 1: per-expert totals
  for (int el = wave; el < p.n_local; el += 4) {
    uint32_t s = 0;
    for (int c = lane; c < p.n_chunks; c += 64) s += flag_load(cnt + (size_t)c * p.n_local + el);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
    if (lane == 0) sh.totals[el] = (int)s;
  }
  __syncthreads();
  if (tid == 0) {
    int acc = 0, tacc = 0;
    for (int el = 0; el < p.n_local; ++el) {
      sh.seg_off[el] = acc;
      sh.tile_base[el] = tacc;
      acc += sh.totals[el];
      tacc += (sh.totals[el] + MoeTile::BM - 1) / MoeTile::BM;
    }
    sh.seg_off[p.n_local] = acc;
    sh.tile_base[p.n_local] = tacc;
    if (acc > p.capacity) raise_status(p.status, ST_CAPACITY);
  }
  __syncthreads();
  // pass 2: first slot of every (chunk, expert), in chunk order
  for (int el = wave; el < p.n_local; el += 4) {
    uint32_t run = (uint32_t)sh.seg_off[el];
    for (int c0 = 0; c0 < p.n_chunks; c0 += 64) {
      const int c = c0 + lane;
      const uint32_t v = c < p.n_chunks ? flag_load(cnt + (size_t)c * p.n_local + el) : 0u;
      uint32_t inc = v;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(inc, o);
        if (lane >= o) inc += y;
      }
      if (c < p.n_chunks) __hip_atomic_store(cnt + (size_t)c * p.n_local + el, run + inc - v, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
      run += __shfl(inc, 63);
    }
  }
  for (int i = tid; i <= p.n_local; i += 256) {
    bstore4_sc1(make_rsrc(p.seg_offsets, (uint32_t)(p.n_local + 1) * 4u), (uint32_t)i * 4u, (uint32_t)sh.seg_off[i]);
    __hip_atomic_store(moe_misc(p) + 2 + i, (uint32_t)sh.tile_base[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  wait_mem();
  __syncthreads();
  if (tid == 0) flag_store(&p.flags[0], p.epoch);
}

// ------------------------------------------------------------------------------------------
// route + copy role
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ void moe_copy_role(const MoeParams& p, int cid, MoeShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // route: chunks (cid*4 + wave) + i * (n_copy*4)
  for (int c = cid * 4 + wave; c < p.n_chunks; c += p.n_copy * 4) moe_route_chunk(p, c, lane);
  wait_mem();
  __syncthreads();
  if (tid == 0) sh.is_last = atomic_add_agent(moe_misc(p) + 0, 1u) == (uint32_t)(p.n_copy - 1);
  __syncthreads();
  if (sh.is_last) moe_scan(p, sh);

  // dispatch
  if (tid == 0) sh.ok = spin_until_eq(&p.flags[0], p.epoch, p.timeout_ticks, p.status);
  __syncthreads();
  if (!sh.ok) return;
  const int tile_m = MoeTile::BM;
  const uint32_t row_b = (uint32_t)p.hidden * 2u;
  const int cpr = p.hidden >> 3;  // 16-byte chunks per token row
  for (int pos = cid; pos < p.n_chunks; pos += p.n_copy) {
    if (pos + 1 == p.drop_pos) continue;
    const int c = p.emulated && p.order ? p.order[pos] : pos;
    if (c < 0 || c >= p.n_chunks) continue;
    const int g0 = c * 64;
    const int r = g0 / p.t_local, i0 = g0 - r * p.t_local;
    if (wave == 0) {
      const int t = g0 + lane;
      int ti[MOE_KMAX];
      const auto tr = make_rsrc(p.topk_idx + (size_t)t * p.top_k, (uint32_t)p.top_k * 4u);
#pragma unroll
      for (int j = 0; j < MOE_KMAX; ++j) ti[j] = j < p.top_k ? (int)bload4_sc1(tr, (uint32_t)j * 4u) : -1;
      const uint32_t* base = p.counters + p.off_chunk_cnt + (size_t)c * p.n_local;
      const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
      int n = 0;
      for (int el = 0; el < p.n_local; ++el) {
        const int e = p.expert_begin + el;
        bool hit = false;
#pragma unroll
        for (int j = 0; j < MOE_KMAX; ++j)
          if (j < p.top_k) hit |= (ti[j] == e);
        const uint64_t m = __ballot(hit);
        if (hit) {
          const int rk = __popcll(m & lt);
          sh.list_tok[n + rk] = t;
          sh.list_slot[n + rk] = (int)flag_load(base + el) + rk;
        }
        n += __popcll(m);
      }
      if (lane == 0) sh.n_list = n;
    }
    __syncthreads();
    const int n = sh.n_list;
    // copy rows: wave w takes rows w, w+4, ...; 64 lanes x 16 B per instruction
    for (int i = wave; i < n; i += 4) {
      const int slot = sh.list_slot[i];
      if (slot >= p.capacity) continue;
      const int t = sh.list_tok[i];
      const auto src = make_rsrc(p.tokens[r] + (size_t)(i0 + (t - g0)) * p.hidden, row_b);
      const auto dst = make_rsrc(p.x_seg + (size_t)slot * p.hidden, row_b);
      for (int cc0 = 0; cc0 < cpr; cc0 += 64 * 8) {
        u32x4 v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int cc = cc0 + q * 64 + lane;
          if (cc < cpr) v[q] = bload16_nt(src, (uint32_t)cc * 16u);
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int cc = cc0 + q * 64 + lane;
          if (cc < cpr) bstore16_sc1(dst, (uint32_t)cc * 16u, v[q]);
        }
      }
      if (lane == 0) bstore4_sc1(make_rsrc(p.seg_token + slot, 4u), 0u, (uint32_t)t);
    }
    wait_mem();
    __syncthreads();
    // landed rows per m-tile: each local expert's rows of this chunk are a contiguous slot range
    if (wave == 0) {
      // per local expert: rows of this chunk (ballot over the chunk's tokens), first slot from the scan
      const int t = g0 + lane;
      int ti[MOE_KMAX];
      const auto tr = make_rsrc(p.topk_idx + (size_t)t * p.top_k, (uint32_t)p.top_k * 4u);
#pragma unroll
      for (int j = 0; j < MOE_KMAX; ++j) ti[j] = j < p.top_k ? (int)bload4_sc1(tr, (uint32_t)j * 4u) : -1;
      const uint32_t* base = p.counters + p.off_chunk_cnt + (size_t)c * p.n_local;
      for (int el = 0; el < p.n_local; ++el) {
        const int e = p.expert_begin + el;
        bool hit = false;
#pragma unroll
        for (int j = 0; j < MOE_KMAX; ++j)
          if (j < p.top_k) hit |= (ti[j] == e);
        const int cnt_e = __popcll(__ballot(hit));
        if (cnt_e == 0) continue;
        if (lane == 0) {
          const int first = (int)flag_load(base + el);
          const uint32_t* misc = moe_misc(p);
          // slot -> (expert-relative row) -> m-tile; clip to capacity
          const int off_e = (int)flag_load((const uint32_t*)p.seg_offsets + el);
          const int tb = (int)flag_load(misc + 2 + el);
          int s = first;
          const int s_end = min(first + cnt_e, p.capacity);
          while (s < s_end) {
            const int mt = (s - off_e) / tile_m;
            const int tile_end = off_e + (mt + 1) * tile_m;
            const int hi = min(s_end, tile_end);
            atomic_add_agent(p.counters + p.off_tile_cnt + tb + mt, (uint32_t)(hi - s));
            s = hi;
          }
        }
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------------------------------
// compute role: ragged grouped GEMM
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ void moe_compute_role(const MoeParams& p, int slot, char* st0, char* st1, char* st2, MoeShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (tid == 0) sh.ok = spin_until_eq(&p.flags[0], p.epoch, p.timeout_ticks, p.status);
  __syncthreads();
  if (!sh.ok) return;
  for (int i = tid; i <= p.n_local; i += 256) {
    sh.seg_off[i] = (int)flag_load((const uint32_t*)p.seg_offsets + i);
    sh.tile_base[i] = (int)flag_load(moe_misc(p) + 2 + i);
  }
  __syncthreads();
  MoeTile g;
  const int wm = wave / MoeTile::WN, wn = wave % MoeTile::WN;
  const int n_mt = sh.tile_base[p.n_local];
  const int n_tiles = n_mt * p.tiles_n;
  const int nk = p.hidden >> 6;
  const int C = p.n_compute;
  const int rs = ((C & 7) == 0) ? (slot & 7) * (C >> 3) + (slot >> 3) : slot;
  const uint32_t lda_b = (uint32_t)p.hidden * 2u, ldb_b = (uint32_t)p.ffn * 2u;
  g.init(wm, wn, lane, lda_b, ldb_b);
  for (int t = rs; t < n_tiles; t += C) {
    const int gm = t / p.tiles_n, tn = t - gm * p.tiles_n;
    int el = 0;
    while (el + 1 < p.n_local && sh.tile_base[el + 1] <= gm) ++el;
    const int mt = gm - sh.tile_base[el];
    const int row0 = sh.seg_off[el] + mt * MoeTile::BM;
    int rows_valid = min(MoeTile::BM, sh.seg_off[el + 1] - row0);
    rows_valid = min(rows_valid, p.capacity - row0);
    if (rows_valid <= 0) continue;
    const int n0 = tn * MoeTile::BN;
    const int cols_valid = min(MoeTile::BN, p.ffn - n0);
    // wait until every row of this m-tile has landed
    if (tid == 0)
      sh.ok = spin_until_ge(p.counters + p.off_tile_cnt + gm, (uint32_t)rows_valid, p.timeout_ticks, p.status);
    __syncthreads();
    if (!sh.ok) return;
    const char* a_tile = reinterpret_cast<const char*>(p.x_seg + (size_t)row0 * p.hidden);
    const uint32_t a_tile_bytes = (uint32_t)rows_valid * lda_b;
    const char* b_col = reinterpret_cast<const char*>(p.w_up + (size_t)el * p.hidden * p.ffn + n0);
    const uint32_t b_col_bytes = ((uint32_t)p.hidden * (uint32_t)p.ffn - (uint32_t)n0) * 2u;
    auto load_step = [&](int ks, char* dst) {
      const uint32_t ca = (uint32_t)ks * 128u, rb = (uint32_t)ks * 64u * ldb_b;
      g.dma_a(a_tile + ca, a_tile_bytes - ca, lda_b, dst, wave);
      g.dma_b(b_col + rb, b_col_bytes - rb, ldb_b, dst, wave);
    };
    g.zero();
    k_loop3(g, nk, st0, st1, st2, load_step, [](int) {});
    g.epilogue(st0, st1, wm, wn, lane, wave, [&](int row, int col, f32x4 v) {
      if (row < rows_valid && col < cols_valid)
        *reinterpret_cast<f32x4*>(p.y + (size_t)(row0 + row) * p.ffn + (n0 + col)) = v;
    });
    __syncthreads();  // the next tile's prologue reuses the LDS
  }
}

__global__ __launch_bounds__(256, 1) void moe_kernel(MoeParams p) {
  __shared__ __attribute__((aligned(16))) char st0[MoeTile::STAGE];
  __shared__ __attribute__((aligned(16))) char st1[MoeTile::STAGE];
  __shared__ __attribute__((aligned(16))) char st2[MoeTile::STAGE];
  __shared__ MoeShared sh;
  const int wg = blockIdx.x;
  if (wg < p.n_copy) moe_copy_role(p, wg, sh);
  else if (wg - p.n_copy < p.n_compute) moe_compute_role(p, wg - p.n_copy, st0, st1, st2, sh);
  // exit accounting: the last workgroup out re-zeroes the counters for the next call
  wait_mem();
  __syncthreads();
  if (threadIdx.x == 0) sh.is_last = atomic_add_agent(moe_misc(p) + 1, 1u) == (uint32_t)(gridDim.x - 1);
  __syncthreads();
  if (sh.is_last) {
    const int n_mt_max = p.max_mtiles;
    for (int i = threadIdx.x; i < n_mt_max; i += 256)
      __hip_atomic_store(p.counters + p.off_tile_cnt + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (threadIdx.x == 0) {
      __hip_atomic_store(moe_misc(p) + 0, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(moe_misc(p) + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

hipError_t launch_moe(const MoeParams& p, int grid, hipStream_t s) {
  hipLaunchKernelGGL(moe_kernel, dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

// Small fill kernel (used by context reset): plain vector stores, safe under graph capture.
__global__ void fill_u32_kernel(uint32_t* p, uint32_t v, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = v;
}
hipError_t launch_fill_u32(uint32_t* p, uint32_t v, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int blocks = (int)((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024);
  hipLaunchKernelGGL(fill_u32_kernel, dim3(blocks), dim3(256), 0, s, p, v, n);
  return hipGetLastError();
}

}  // namespace mk
