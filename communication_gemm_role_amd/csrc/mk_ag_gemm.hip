// AllGather + GEMM, one rank's share, as one persistent launch.
//
// Operation (mKernel write-up, news.chathome.org page, five-fused-kernels table,
// AllGather + GEMM row): each rank holds one row shard of A; while the other shards
// arrive, the local GEMM consumes A tiles as soon as they land.  Here the other ranks'
// shards are device buffers and "arrival" is the copy role.
//
// Roles (section "mKernel的功能" of the same page: CTAs self-assign roles, a per-shape
// number of SMs per role):
//   workgroups [0, n_copy)          copy: for queue positions cid, cid + n_copy, ... of the
//                                   arrival order, copy that unit of a peer shard into its
//                                   rows of a_gathered, then raise the unit's ready flag.
//                                   Copy workgroups never wait, so they always finish.
//   workgroups [n_copy, grid)       compute: 256 x 256 output tiles of C.  In emulated mode the
//                                   K loop visits K-units (unit_cols columns of K) ready-first:
//                                   wave 0 polls the flags of the tile's unit rows and picks the
//                                   lowest-numbered K-unit that has fully landed, one unit ahead
//                                   of the prefetch, so landed data is consumed immediately.
// A compute workgroup only ever waits on copy workgroups, which have lower ids and are therefore
// dispatched first; every wait is bounded by the watchdog.
#include "mk_internal.h"
#include "mk_gemm_tile.hpp"

namespace mk {

using AgTile = TileGemmDma<256, 128, 2, 2>;

int ag_tile_m() { return AgTile::BM; }
int ag_tile_n() { return AgTile::BN; }

// ------------------------------------------------------------------------------------------
// copy role
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ int ag_identity_unit(const AgParams& p, int pos) {
  // queue position -> unit id, rank-major then row-major, skipping the local shard when in place
  const int spr = p.m_shard / p.unit_rows;
  int ur = pos / p.n_ucols;
  const int uc = pos - ur * p.n_ucols;
  if (p.local_in_place && ur >= p.rank * spr) ur += spr;
  return ur * p.n_ucols + uc;
}

__device__ void ag_copy_role(const AgParams& p, int cid) {
  const int tid = threadIdx.x;
  const int cpr = p.unit_cols >> 3;              // 16-byte chunks per unit row
  const int per_t = (p.unit_rows * cpr) >> 8;    // chunks per thread: 2 (64x64) or 8 (128x128)
  const uint32_t ldb = (uint32_t)p.k * 2u;
  const int n_units = p.n_urows * p.n_ucols;
  for (int pos = cid; pos < p.n_order; pos += p.n_copy) {
    if (pos + 1 == p.drop_pos) continue;  // testing: this unit never lands
    const int u = p.order ? p.order[pos] : ag_identity_unit(p, pos);
    if (u < 0 || u >= n_units) continue;
    const int ur = u / p.n_ucols, uc = u - ur * p.n_ucols;
    const int grow = ur * p.unit_rows;
    const int r = grow / p.m_shard, srow = grow - r * p.m_shard;
    const uint32_t extent = ((uint32_t)(p.unit_rows - 1) * (uint32_t)p.k + (uint32_t)p.unit_cols) * 2u;
    const auto src = make_rsrc(p.shards[r] + (size_t)srow * p.k + (size_t)uc * p.unit_cols, extent);
    const auto dst = make_rsrc(p.ag + (size_t)grow * p.k + (size_t)uc * p.unit_cols, extent);
    u32x4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i < per_t) {
        const int c = tid + (i << 8);
        const int row = c / cpr, cc = c - row * cpr;
        v[i] = bload16_nt(src, (uint32_t)row * ldb + (uint32_t)cc * 16u);
      }
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i < per_t) {
        const int c = tid + (i << 8);
        const int row = c / cpr, cc = c - row * cpr;
        bstore16_sc1(dst, (uint32_t)row * ldb + (uint32_t)cc * 16u, v[i]);
      }
    wait_mem();
    __syncthreads();
    if (tid == 0) flag_store(&p.flags[u], p.epoch);
  }
}

// ------------------------------------------------------------------------------------------
// compute role
// ------------------------------------------------------------------------------------------
// Wave 0: is unit row `ur` always present (local shard already in place)?
__device__ __forceinline__ bool ag_row_local(const AgParams& p, int ur) {
  const int spr = p.m_shard / p.unit_rows;
  return p.local_in_place && ur >= p.rank * spr && ur < (p.rank + 1) * spr;
}

// Wave 0, all lanes: landed-K-unit mask for the tile's unit rows [ur0, ur0 + n_ur).
__device__ __forceinline__ uint64_t ag_ready_mask(const AgParams& p, int ur0, int n_ur, uint64_t all, int lane) {
  uint64_t ready = all;
  for (int q = 0; q < n_ur; ++q) {
    const int ur = ur0 + q;
    if (ag_row_local(p, ur)) continue;
    const bool up = lane < p.n_ucols && flag_load(&p.flags[ur * p.n_ucols + lane]) == p.epoch;
    ready &= __ballot(up);
  }
  return ready;
}

// Wave 0: pick the next K-unit (lowest landed, not yet scheduled); -1 on timeout or fault.
// Every value that steers control flow here is wave-uniform (ballots, readfirstlane), so all 64
// lanes take the same path and every ballot sees every unit's flag.  The scheduled-set mask lives
// in LDS (volatile: re-read each call) so no register is held across the MFMA loop for it.
__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ int ag_pick(const AgParams& p, int ur0, int n_ur, uint64_t* s_done, int lane) {
  volatile uint64_t* vd = s_done;
  const uint64_t all = (p.n_ucols >= 64) ? ~0ull : ((1ull << p.n_ucols) - 1ull);
  const uint64_t done = uniform64(*vd);
  uint64_t cand = ag_ready_mask(p, ur0, n_ur, all, lane) & ~done;
  if (!cand) {
    const uint64_t t0 = wall_ticks();
    int n = 0;
    while (true) {
      __builtin_amdgcn_s_sleep(2);
      cand = ag_ready_mask(p, ur0, n_ur, all, lane) & ~done;
      if (cand) break;
      if ((++n & 7) == 0) {
        const bool bad = __builtin_amdgcn_readfirstlane(status_bad(p.status) ? 1 : 0) != 0;
        if (bad) return -1;
        if (wall_ticks() - t0 > p.timeout_ticks) {
          if (lane == 0) raise_status(p.status, ST_TIMEOUT);
          return -1;
        }
      }
    }
  }
  const int u = __builtin_ctzll(cand);
  *vd = done | (1ull << u);  // every lane stores the same value
  return u;
}

__device__ void ag_compute_role(const AgParams& p, int slot, char* st0, char* st1, int* s_next, uint64_t* s_done) {
  AgTile g;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  (void)tid;
  const int wm = wave / AgTile::WN, wn = wave % AgTile::WN;
  const int n_tiles = p.tiles_m * p.tiles_n;
  const int nk = p.k >> 6;
  const int spu = p.unit_cols >> 6;  // k-steps per K-unit
  const int n_ku = p.n_ucols;
  const int C = p.n_compute;
  // XCD-aware slot order: workgroup w runs on XCD w % 8; consecutive logical tiles (which share
  // A row blocks) go to one XCD so its L2 keeps reusing them.
  const int rs = ((C & 7) == 0) ? (slot & 7) * (C >> 3) + (slot >> 3) : slot;
  const uint32_t lda_b = (uint32_t)p.k * 2u, ldb_b = (uint32_t)p.n * 2u;
  g.init(wm, wn, lane, lda_b, ldb_b);

  for (int t = rs; t < n_tiles; t += C) {
    const int tm = t / p.tiles_n, tn = t - tm * p.tiles_n;
    const int m0 = tm * AgTile::BM, n0 = tn * AgTile::BN;
    const int rows_valid = min(AgTile::BM, p.m - m0), cols_valid = min(AgTile::BN, p.n - n0);
    const int ur0 = m0 / p.unit_rows, n_ur = rows_valid / p.unit_rows;
    // Operand windows of the k-step: A rows of the tile from the step's first column, B rows of
    // the step from column n0.  Only scalar values change from step to step.
    const char* a_tile = reinterpret_cast<const char*>(p.ag + (size_t)m0 * p.k);
    const uint32_t a_tile_bytes = (uint32_t)rows_valid * lda_b;
    const char* b_col = reinterpret_cast<const char*>(p.b + n0);
    const uint32_t b_col_bytes = ((uint32_t)p.k * (uint32_t)p.n - (uint32_t)n0) * 2u;
    auto load_step = [&](int ks, char* dst) {
      const uint32_t ca = (uint32_t)ks * 128u;           // byte column of the step in A
      const uint32_t rb = (uint32_t)ks * 64u * ldb_b;    // byte row of the step in B
      g.dma_a(a_tile + ca, a_tile_bytes - ca, lda_b, dst, wave);
      g.dma_b(b_col + rb, b_col_bytes - rb, ldb_b, dst, wave);
    };

    g.zero();

    int unit;  // K-unit of the step being prefetched
    if (p.emulated) {
      if (wave == 0) {
        *(volatile uint64_t*)s_done = 0;
        const int u0 = ag_pick(p, ur0, n_ur, s_done, lane);
        const int u1 = (u0 >= 0 && n_ku > 1) ? ag_pick(p, ur0, n_ur, s_done, lane) : (u0 >= 0 ? 0 : -1);
        if (lane == 0) {
          s_next[0] = u0;
          s_next[1] = u1;
        }
      }
      __syncthreads();
      unit = __builtin_amdgcn_readfirstlane(s_next[0]);
      if (unit < 0 || (n_ku > 1 && __builtin_amdgcn_readfirstlane(s_next[1]) < 0)) return;  // before any MFMA
    } else {
      unit = 0;
    }
    // A failed wait (watchdog or another workgroup's fault) inside the K loop does not leave the
    // loop: the remaining steps drain on K-unit 0 (in bounds, result discarded) and the tile's
    // stores are skipped.  Keeping the loop single-exit keeps the accumulators in AGPRs.
    bool aborted = false;
    load_step(unit * spu, st0);
    wait_mem();
    __syncthreads();

    // One pipeline step: prefetch step s+1 into `nxt` while the MFMAs consume `cur`.  The loop is
    // unrolled by two so each half names its stage buffers statically: the compiler can then see
    // that the MFMA operand reads never alias the LDS DMA in flight and issues no wait between them.
    auto step = [&](int s, char* cur, char* nxt) {
      const int pf = s + 1;
      bool decide = false;
      int jn = 0;
      if (pf < nk) {
        const int sub = pf % spu;
        if (sub == 0) {
          const int j = pf / spu;
          unit = p.emulated ? __builtin_amdgcn_readfirstlane(s_next[j & 1]) : j;
          aborted |= unit < 0;
          unit = unit < 0 ? 0 : unit;
          decide = p.emulated && (j + 1 < n_ku);
          jn = j + 1;
        }
        load_step(unit * spu + sub, nxt);
      }
      g.mma(cur);
      if (decide && wave == 0) {
        const int u = ag_pick(p, ur0, n_ur, s_done, lane);
        if (lane == 0) s_next[jn & 1] = u;
      }
      wait_mem();
      __syncthreads();
    };
    for (int s = 0; s < nk; s += 2) {
      step(s, st0, st1);
      if (s + 1 < nk) step(s + 1, st1, st0);
    }

    // epilogue: fp32 C tile, staged through LDS into row-contiguous 16-byte stores
    g.epilogue(st0, st1, wm, wn, lane, wave, [&](int row, int col, f32x4 v) {
      if (!aborted && row < rows_valid && col < cols_valid)
        *reinterpret_cast<f32x4*>(p.c + (size_t)(m0 + row) * p.n + (n0 + col)) = v;
    });
    __syncthreads();  // the next tile's prologue reuses the LDS
    if (aborted) break;
  }
}

__global__ __launch_bounds__(256, 1) void ag_gemm_kernel(AgParams p) {
  __shared__ __attribute__((aligned(16))) char st0[AgTile::STAGE];
  __shared__ __attribute__((aligned(16))) char st1[AgTile::STAGE];
  __shared__ int s_next[2];
  __shared__ uint64_t s_done;
  const int wg = blockIdx.x;
  if (wg < p.n_copy) {
    ag_copy_role(p, wg);
    return;
  }
  const int slot = wg - p.n_copy;
  if (slot < p.n_compute) ag_compute_role(p, slot, st0, st1, s_next, &s_done);
}

hipError_t launch_ag_gemm(const AgParams& p, int grid, hipStream_t s) {
  hipLaunchKernelGGL(ag_gemm_kernel, dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace mk
