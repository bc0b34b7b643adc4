// GEMM + ReduceScatter / GEMM + AllReduce roles (copy, reduce, compute), one rank's share; the
// kernels that run them are gemm_reduce_kernel (mk_gemm_reduce.hip) and the MLP kernel (mk_mlp.hip).
//
// Operations (mKernel write-up, news.chathome.org page, five-fused-kernels table, GEMM +
// AllReduce and GEMM + ReduceScatter rows): rank j holds a partial P_j = A_j @ B_j of the same
// [M, N] output.  AllReduce: every rank ends with sum_j P_j.  ReduceScatter: rank r ends with
// sum_j P_j on its own row slice only.  A tile of P enters the reduction right after its K loop,
// inside the same launch.
//
// This rank's partial is P = A @ B.  Owned rows (RS: the rank's slice; AR: all rows) need
// out = P + sum of the peers' partials; in RS every other tile goes unreduced to the outbox
// of its owner.
//
// Roles, in workgroup-id order (each waits only on lower ids, which dispatch first):
//   [0, n_copy)                 copy (emulated mode): lands peer-partial units in the inbox in
//                               the caller's arrival order and raises each unit's flag, then
//                               joins the compute role on tiles left over past n_compute.
//   [n_copy, n_copy+n_reduce)   reduce: for each owned tile, waits for its peer units, sums the
//                               peer partials with coalesced 16-byte fp32 loads, writes the sum
//                               into the output tile and raises the tile's pre-sum flag.
//   the rest                    compute: MFMA tile of P; epilogue adds P to the pre-sum (or, for
//                               AllReduce with no reduce workgroups, sums the peers itself) and
//                               stores the owned tile, or stores P to the owner's outbox.  Owned
//                               tiles are scheduled last so the pre-sum is ready for them: done by
//                               the reduce role, or (ReduceScatter with no reduce workgroups) by
//                               every workgroup in 64-row bands between its tiles.
#pragma once
#include "mk_internal.h"
#include "mk_gemm_tile.hpp"
#include "mk_gemm_tile16.hpp"
#include "mk_copy_ring.hpp"

namespace mk {

// wide outputs (e.g. 8192 x 4096, also the MLP block's down-projection): eight waves on the
// 16 x 16 x 32 core, A two steps ahead in three 32 KiB slots and B in two; few output rows
// (decode-like): four waves on the 32 x 32 x 16 core
using RedBig = TileGemm16T<mk_tiles::kRedBig.bn>;
static_assert(RedBig::BM == mk_tiles::kRedBig.bm && RedBig::WM == mk_tiles::kRedBig.wm &&
                  RedBig::WN == mk_tiles::kRedBig.wn, "kRedBig is the 16 x 16 x 32 core");
using RedSkinny =
    TileGemmDma<mk_tiles::kRedSkinny.bm, mk_tiles::kRedSkinny.bn, mk_tiles::kRedSkinny.wm, mk_tiles::kRedSkinny.wn>;

// Cores with separate A and B slots (mk_gemm_tile16.hpp) against the two-stage TileGemmDma.
template <class T>
constexpr bool kCore16 = false;
template <int BN>
constexpr bool kCore16<TileGemm16T<BN>> = true;

// KiB per wave and batch of the copy ring, whose two slots are the first two stage buffers:
// 32 KiB A slots (4 KiB per wave) on the 16 x 16 x 32 core, else 8 KiB per wave.
template <class T>
constexpr int red_ring_kib() {
  return kCore16<T> ? mk_tiles::kRedBig.ring_kib : 8;
}

inline bool red_skinny(int m, int n) { (void)n; return mk_tiles::red_skinny(m); }

// Peer partial q (0..world-2) is rank q < rank ? q : q + 1.
__device__ __forceinline__ int peer_rank(int rank, int q) { return q < rank ? q : q + 1; }

// Source of peer q's partial: landed inbox copy (emulated) or the resident buffer.
__device__ __forceinline__ const float* peer_src(const RedParams& p, int q) {
  return p.emulated ? p.inbox + (size_t)q * p.p_rows * p.n : p.peers[peer_rank(p.rank, q)];
}

// ------------------------------------------------------------------------------------------
// copy role (emulated landing of peer partials)
// ------------------------------------------------------------------------------------------
// Peer partials land in the inbox through the two-slot LDS ring of mk_copy_ring.hpp:
// red_ring_kib<T>() KiB per wave and batch; IPU is a unit's DMA instructions per wave (a 64x64
// fp32 unit is 16 KiB).
template <class T, int IPU>
__device__ __forceinline__ void red_copy_dma(const RedParams& p, int cid, char* st0, char* st1) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int cpr = p.unit_cols >> 2;  // 16-byte chunks per unit row (fp32)
  const uint32_t ld = (uint32_t)p.n * 4u;
  const uint32_t extent = ((uint32_t)(p.unit_rows - 1) * (uint32_t)p.n + (uint32_t)p.unit_cols) * 4u;
  const int n_units = (p.world - 1) * p.units_per_peer;
  const int n_mine = p.n_order > cid ? (p.n_order - cid + p.n_copy - 1) / p.n_copy : 0;
  const __attribute__((address_space(4))) int32_t* order = (const __attribute__((address_space(4))) int32_t*)p.order;
  uint32_t off[IPU];  // byte offset inside a unit of this lane's chunk, per instruction of the unit
#pragma unroll
  for (int i = 0; i < IPU; ++i) {
    const int c = (wave * IPU + i) * 64 + lane;
    const int row = c / cpr, cc = c - row * cpr;
    off[i] = (uint32_t)row * ld + (uint32_t)cc * 16u;
  }
  auto unit_at = [&](int i) -> int {  // i-th unit of this workgroup's queue, or -1
    if (i >= n_mine) return -1;
    const int pos = cid + i * p.n_copy;
    if (pos + 1 == p.drop_pos) return -1;  // testing: this unit never lands
    const int u = order ? order[pos] : pos;
    return (u < 0 || u >= n_units) ? -1 : u;
  };
  auto elem_of = [&](int u) -> size_t {  // first element of unit u inside a partial
    const int q = u / p.units_per_peer, w = u - q * p.units_per_peer;
    const int ur = w / p.n_ucols, uc = w - ur * p.n_ucols;
    return (size_t)ur * p.unit_rows * p.n + (size_t)uc * p.unit_cols;
  };
  auto src_of = [&](int u) {
    if (u < 0) return make_rsrc(p.inbox, 0u);
    const int q = u / p.units_per_peer;
    return make_rsrc(p.peers[peer_rank(p.rank, q)] + elem_of(u), extent);
  };
  auto dst_of = [&](int u) {
    if (u < 0) return make_rsrc(p.inbox, 0u);
    const int q = u / p.units_per_peer;
    return make_rsrc(p.inbox + (size_t)q * p.p_rows * p.n + elem_of(u), extent);
  };
  const uint64_t t0 = wall_ticks();
  copy_ring<red_ring_kib<T>(), IPU>(n_mine, st0, st1, off, unit_at, src_of, dst_of,
                    [&](int u) { flag_store(&p.flags[u], p.epoch); },
                    [&](int i) {  // queue entry i is arrival position cid + i * n_copy
                      if (p.pace_q16) wait_wall_until(t0 + (((uint64_t)(cid + i * p.n_copy) * p.pace_q16) >> 16));
                    });
}

template <class T>
__device__ __forceinline__ void red_copy_role(const RedParams& p, int cid, char* st0, char* st1) {
  // DMA instructions per wave per unit (the planner keeps them within red_ring_kib<T>())
  const int ipu = (p.unit_rows * p.unit_cols * 4) / (T::NW * 64 * 16);
  if constexpr (red_ring_kib<T>() >= 8) {
    if (ipu >= 8) {
      red_copy_dma<T, 8>(p, cid, st0, st1);
      return;
    }
  }
  if (ipu >= 4) red_copy_dma<T, 4>(p, cid, st0, st1);
  else if (ipu == 2) red_copy_dma<T, 2>(p, cid, st0, st1);
  else red_copy_dma<T, 1>(p, cid, st0, st1);
}

// Rows of the owned region covered by tile row tm: [lr0, lr1) in partial coordinates
// (RS: relative to the owned slice; AR: global rows).  Empty when the tile owns nothing.
template <class T>
__device__ __forceinline__ void owned_rows(const RedParams& p, int tm, int& lr0, int& lr1) {
  const int m0 = tm * T::BM, m1 = min(m0 + T::BM, p.m);
  if (p.is_rs) {
    const int o0 = p.rank * p.m_slice, o1 = o0 + p.m_slice;
    lr0 = max(m0, o0) - o0;
    lr1 = min(m1, o1) - o0;
  } else {
    lr0 = m0;
    lr1 = m1;
  }
}

// One lane of wave 0 per call: wait until every peer unit covering partial rows [lr0, lr1),
// columns [c0, c1) has landed.  All lanes of the wave call it; returns false on timeout/fault.
__device__ __forceinline__ bool wait_units(const RedParams& p, int lr0, int lr1, int c0, int c1, int lane) {
  const int ur0 = lr0 / p.unit_rows, ur1 = (lr1 + p.unit_rows - 1) / p.unit_rows;
  const int uc0 = c0 / p.unit_cols, uc1 = (c1 + p.unit_cols - 1) / p.unit_cols;
  const int per_peer = (ur1 - ur0) * (uc1 - uc0);
  const int total = per_peer * (p.world - 1);
  bool ok = true;
  for (int base = 0; base < total; base += 64) {
    const int i = base + lane;
    if (i < total) {
      const int q = i / per_peer, w = i - q * per_peer;
      const int a = w / (uc1 - uc0), b = w - a * (uc1 - uc0);
      const int u = q * p.units_per_peer + (ur0 + a) * p.n_ucols + (uc0 + b);
      ok = spin_until_eq(&p.flags[u], p.epoch, p.timeout_ticks, p.status);
    }
    if (__ballot(!ok)) return false;
  }
  return true;
}

// ------------------------------------------------------------------------------------------
// pre-sum of the peers' partials of owned rows
// ------------------------------------------------------------------------------------------
// out[lr0, lr1) x [c0, c1) = sum of the peers' partials there (partial coordinates), with every
// thread's loads of all peers in flight before its adds (up to 4 x 7 per thread).  Write-through
// stores; the caller waits for them before raising the region's flag or counter.
template <class T>
__device__ __forceinline__ void red_sum_peers(const RedParams& p, int lr0, int lr1, int c0, int c1) {
  constexpr int NT = T::NW * 64;
  const int tid = threadIdx.x;
  const int cpr = T::BN >> 2;  // 16-byte chunks per tile row
  const int rows = lr1 - lr0, cols = c1 - c0;
  const int ccols = cols >> 2;  // 16-byte chunks per row in this region
  const uint32_t extent = ((uint32_t)(rows - 1) * (uint32_t)p.n + (uint32_t)cols) * 4u;
  const size_t off = (size_t)lr0 * p.n + c0;
  const auto dst = make_rsrc(p.out + off, extent);
  const int total = rows * cpr;
  for (int base = 0; base < total; base += NT * 4) {
    // byte offsets of this thread's 4 chunks; a chunk outside the region gets an offset past
    // every window, so its loads read 0 and its store is dropped
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = base + tid + i * NT;
      const int row = c / cpr, cc = c - row * cpr;
      o[i] = (c < total && cc < ccols) ? ((uint32_t)row * (uint32_t)p.n + (uint32_t)cc * 4u) * 4u : 0xfffffff0u;
    }
    f32x4 t[4][MK_MAX_WORLD - 1];
#pragma unroll
    for (int q = 0; q < MK_MAX_WORLD - 1; ++q) {
      if (q < p.world - 1) {  // (no `break`: it would keep t in memory)
        const auto src = make_rsrc(peer_src(p, q) + off, extent);
#pragma unroll
        for (int i = 0; i < 4; ++i) t[i][q] = __builtin_bit_cast(f32x4, bload16_nt(src, o[i]));
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < MK_MAX_WORLD - 1; ++q)
        if (q < p.world - 1) s += t[i][q];
      bstore16_sc1(dst, o[i], __builtin_bit_cast(u32x4, s));
    }
  }
}

// Reduce role: pre-sums whole owned tiles, raising each tile's pre-sum flag.
template <class T>
__device__ __forceinline__ void red_reduce_role(const RedParams& p, int rid, int* s_ok) {
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int own_rows = p.own_tile_end - p.own_tile_begin;
  const int n_jobs = own_rows * p.tiles_n;
  for (int job = rid; job < n_jobs; job += p.n_reduce) {
    const int tm = p.own_tile_begin + job / p.tiles_n, tn = job % p.tiles_n;
    int lr0, lr1;
    owned_rows<T>(p, tm, lr0, lr1);
    const int c0 = tn * T::BN, c1 = min(c0 + T::BN, p.n);
    if (p.emulated) {
      if (wave == 0) {
        const bool ok = wait_units(p, lr0, lr1, c0, c1, lane);
        if (lane == 0) *s_ok = ok;
      }
      __syncthreads();
      if (!*s_ok) return;
    }
    red_sum_peers<T>(p, lr0, lr1, c0, c1);
    wait_mem();
    __syncthreads();
    if (tid == 0) flag_store(&p.presum_flags[tm * p.tiles_n + tn], p.epoch);
  }
}

// RS without reduce workgroups: a compute workgroup about to claim a tile first takes pre-sum
// jobs, 64-row bands of owned tiles, until none is left (or max_jobs are done), adding one to the
// tile's band counter per band done.  Owned tiles come last in the tile order, so their bands
// are done by the time their epilogues need them, and the peer reads spread over every
// workgroup instead of piling up in the owned tiles' epilogues.  Returns false on a timeout or
// fault.
template <class T>
__device__ __forceinline__ bool red_presum_jobs(const RedParams& p, int* s_ok, int* s_claim, int max_jobs) {
  constexpr int J = T::BM / 64;  // bands per owned tile
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n_jobs = (p.own_tile_end - p.own_tile_begin) * p.tiles_n * J;
  for (int taken = 0; taken < max_jobs; ++taken) {
    __syncthreads();  // every thread has read the last claim
    if (tid == 0) *s_claim = (int)atomic_add_agent(p.counters + CTR_RED_PRESUM, 1u);
    __syncthreads();
    const int job = *s_claim;
    if (job >= n_jobs) return true;
    const int ot = job / J, band = job - ot * J;
    const int tm = p.own_tile_begin + ot / p.tiles_n, tn = ot % p.tiles_n;
    int lr0, lr1;
    owned_rows<T>(p, tm, lr0, lr1);
    const int b0 = lr0 + band * 64, b1 = min(lr1, b0 + 64);
    if (b0 < b1) {
      const int c0 = tn * T::BN, c1 = min(c0 + T::BN, p.n);
      if (p.emulated) {
        if (wave == 0) {
          const bool ok = wait_units(p, b0, b1, c0, c1, lane);
          if (lane == 0) *s_ok = ok;
        }
        __syncthreads();
        if (!*s_ok) return false;
      }
      red_sum_peers<T>(p, b0, b1, c0, c1);
      wait_mem();
    }
    __syncthreads();
    if (tid == 0) atomic_add_agent(p.counters + CTR_RED_BAND0 + ot, 1u);
  }
  return true;
}

// ------------------------------------------------------------------------------------------
// compute role
// ------------------------------------------------------------------------------------------
template <class T>
// Compute role.  Compute workgroup `slot` first runs its static tile; tiles from n_compute on are
// left over and claimed, in logical order (owned tiles last), from a shared counter by every
// workgroup that has finished its own work: compute workgroups after their static tile, copy
// workgroups (slot -1) after landing their units.
__device__ __forceinline__ void red_compute_role(const RedParams& p, int slot, char* st0, char* st1, char* st2,
                                                 char* st3, char* st4, int* s_ok, int* s_claim) {
  T g;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / T::WN, wn = wave % T::WN;
  const int n_tiles = p.tiles_m * p.tiles_n;
  const int nk = p.k >> 6;
  const int C = p.n_compute;
  const int rs = ((C & 7) == 0) ? (slot & 7) * (C >> 3) + (slot >> 3) : slot;
  const uint32_t lda_b = (uint32_t)p.k * 2u, ldb_b = (uint32_t)p.n * 2u;
  if constexpr (kCore16<T>) g.init(wm, wn, wave, lane, lda_b, ldb_b);
  else g.init(wm, wn, lane, lda_b, ldb_b);

  int t = (slot >= 0 && rs < n_tiles) ? rs : -1;
  bool first = slot >= 0, claimed = false;
  // With resident partials, the workgroups of odd XCDs take one pre-sum band before their first
  // tile: their peer reads (HBM) then overlap the even XCDs' first K loops (mostly L2), and the
  // two halves reach their epilogues' stores at different times instead of all at once.
  if (p.assist && !p.emulated && slot >= 0 && (slot & 1) && !red_presum_jobs<T>(p, s_ok, s_claim, 1)) return;
  while (true) {
    if (t < 0) {
      if (p.assist && !red_presum_jobs<T>(p, s_ok, s_claim, 1 << 30)) return;
      if (tid == 0) *s_claim = C + (int)atomic_add_agent(p.counters + CTR_RED_TILE, 1u);
      if (!claimed) trace_mark(p.trace, 7);  // first leftover tile claimed (after any pre-sum jobs)
      claimed = true;
      __syncthreads();
      t = *s_claim;  // rewritten only after the next tile's barriers
      if (t >= n_tiles) break;
    }
    // logical tile rows start right after the owned rows, so owned tiles come last
    const int tml = t / p.tiles_n, tn = t - tml * p.tiles_n;
    const int tm = (tml + p.own_tile_end) % p.tiles_m;
    const int m0 = tm * T::BM, n0 = tn * T::BN;
    const int rows_valid = min(T::BM, p.m - m0), cols_valid = min(T::BN, p.n - n0);
    const char* a_tile = reinterpret_cast<const char*>(p.a + (size_t)m0 * p.k);
    const uint32_t a_tile_bytes = (uint32_t)rows_valid * lda_b;
    const char* b_col = reinterpret_cast<const char*>(p.b + n0);
    const uint32_t b_col_bytes = ((uint32_t)p.k * (uint32_t)p.n - (uint32_t)n0) * 2u;
    auto dma_a = [&](int ks, char* dst) {
      const uint32_t ca = (uint32_t)ks * 128u;
      g.dma_a(a_tile + ca, a_tile_bytes - ca, lda_b, dst, wave);
    };
    auto dma_b = [&](int ks, char* dst) {
      const uint32_t rb = (uint32_t)ks * 64u * ldb_b;
      if constexpr (kCore16<T>) g.dma_b(b_col + rb, b_col_bytes - rb, dst, wave);
      else g.dma_b(b_col + rb, b_col_bytes - rb, ldb_b, dst, wave);
    };
    int lr0, lr1;
    owned_rows<T>(p, tm, lr0, lr1);
    const bool has_owned = lr1 > lr0;
    // AllReduce with resident partials and no reduce workgroups: a workgroup sums its static
    // tile's peer partials into the output before the K loop (every workgroup reads HBM first, then
    // runs its K loop, mostly L2 hits, undisturbed), and its epilogue then only adds P.  Measured
    // 2 % faster than splitting the XCDs between summing first and summing in the epilogue.
    const bool self_presum = has_owned && !p.is_rs && !p.emulated && p.n_reduce == 0 && first;
    // The four-wave tile gives each wave one 32-row slab in its epilogue, 8 values of 4 per lane:
    // the pre-sum of exactly those values is kept in registers (32 per lane) across the K loop
    // instead of going to the output and back (the lane's slab positions are the epilogue's).
    constexpr bool REG_PRESUM = !kCore16<T> && T::NW == 4 && T::FM == 1;
    f32x4 ps[T::SLAB_Q];
    if (self_presum) {
      if constexpr (REG_PRESUM) {
        constexpr int C4 = T::WTN / 4, H = T::SLAB_Q / 2;
        const size_t base = (size_t)m0 * p.n + n0;
        // two halves of the lane's values, each with all its peers' loads in flight (112 registers)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          f32x4 t[H][MK_MAX_WORLD - 1];
#pragma unroll
          for (int pq = 0; pq < MK_MAX_WORLD - 1; ++pq) {
            if (pq < p.world - 1) {  // (no `break`: it would keep t in memory)
              const float* src = peer_src(p, pq) + base;
#pragma unroll
              for (int i = 0; i < H; ++i) {
                const int idx = (h * H + i) * 64 + lane;
                const int row = wm * T::WTM + idx / C4, col = wn * T::WTN + (idx % C4) * 4;
                t[i][pq] = (row < rows_valid && col < cols_valid)
                               ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src + (size_t)row * p.n + col))
                               : f32x4{0.f, 0.f, 0.f, 0.f};
              }
            }
          }
#pragma unroll
          for (int i = 0; i < H; ++i) {
            f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int pq = 0; pq < MK_MAX_WORLD - 1; ++pq)
              if (pq < p.world - 1) a += t[i][pq];
            ps[h * H + i] = a;
          }
        }
      } else {
        red_sum_peers<T>(p, lr0, lr1, n0, n0 + cols_valid);
        wait_mem();
      }
    }
    if (p.a_ready) {  // A is produced in this launch (the MLP kernel's H): its rows must be complete
      if (tid == 0) *s_ok = spin_until_ge(p.a_ready + tm, p.a_ready_need, p.timeout_ticks, p.status);
      __syncthreads();
      if (!*s_ok) return;
    }
    g.zero();
    if (first) trace_mark(p.trace, 5);  // operands are resident: ready at once
    if constexpr (kCore16<T>) {
      // st0..st2: A slots, st3, st4: B slots
      auto prologue = [&](char* pa0, char* pb0, char* pa1) {
        dma_a(0, pa0);
        dma_b(0, pb0);
        if (nk > 1) dma_a(1, pa1);
      };
      auto none = [](int, auto) {};
      k_loop_a3b2(g, nk, st0, st1, st2, st3, st4, prologue, dma_a, dma_b, none, none, none, [] { return true; });
    } else {
      auto load_step = [&](int ks, char* dst) {
        dma_a(ks, dst);
        dma_b(ks, dst);
      };
      k_loop(g, nk, st0, st1, st2, st3, st4, [](int) {}, load_step, [](int) {});
    }
    if (first) trace_mark(p.trace, 6);  // the first tile's K loop is done; its epilogue follows
    first = false;

    const bool presum = has_owned && (p.n_reduce > 0 || p.assist || self_presum);
    if (has_owned && !self_presum) {
      // the peer data this tile adds must have landed (emulated) or been pre-summed (reduce role,
      // or every band by the compute workgroups' pre-sum jobs)
      if (wave == 0) {
        bool ok = true;
        if (presum) {
          if (lane == 0)
            ok = p.assist ? spin_until_ge(p.counters + CTR_RED_BAND0 + (tm - p.own_tile_begin) * p.tiles_n + tn,
                                          (uint32_t)(T::BM / 64), p.timeout_ticks, p.status)
                          : spin_until_eq(&p.presum_flags[tm * p.tiles_n + tn], p.epoch, p.timeout_ticks, p.status);
          ok = __ballot(!ok) == 0;
        } else if (p.emulated) {
          ok = wait_units(p, lr0, lr1, n0, n0 + cols_valid, lane);
        }
        if (lane == 0) *s_ok = ok;
      }
      __syncthreads();
      if (!*s_ok) return;
    }
    const int own0 = p.is_rs ? p.rank * p.m_slice : 0;
    // A slab (16 or 32 rows) lies inside one owner's slice (slices and valid row counts are
    // multiples of 64 rows) and inside or outside the valid rows as a whole.  Every load a slab's reduction
    // needs is issued before any of its adds, so the loads overlap instead of each waiting for
    // the one before.
    constexpr int Q = T::SLAB_Q;
    auto store_slab = [&](int srow, f32x4(&v)[Q], const int(&r)[Q], const int(&c)[Q]) {
      if (srow >= rows_valid) return;
      if (p.is_rs) {
        const int owner = (m0 + srow) / p.m_slice;
        if (owner != p.rank) {  // unreduced partial of another rank's slice -> its outbox
          float* ob = p.outbox[owner] + (size_t)(m0 - owner * p.m_slice) * p.n + n0;
#pragma unroll
          for (int q = 0; q < Q; ++q)
            if (c[q] < cols_valid)  // written once, read by no one here: streaming stores
              __builtin_nontemporal_store(v[q], reinterpret_cast<f32x4*>(ob + (size_t)r[q] * p.n + c[q]));
          return;
        }
      }
      const size_t base = (size_t)(m0 - own0) * p.n + n0;
      if (presum) {
        f32x4 t[Q];
        bool in_regs = false;
        if constexpr (REG_PRESUM) {
          in_regs = self_presum;
          if (in_regs) {
#pragma unroll
            for (int q = 0; q < Q; ++q) t[q] = ps[q];
          }
        }
        if (!in_regs) {
#pragma unroll
          for (int q = 0; q < Q; ++q)
            t[q] = c[q] < cols_valid ? *reinterpret_cast<const f32x4*>(p.out + base + (size_t)r[q] * p.n + c[q])
                                     : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int q = 0; q < Q; ++q)
          if (c[q] < cols_valid)  // the final value: nothing reads it back here
            __builtin_nontemporal_store(v[q] + t[q], reinterpret_cast<f32x4*>(p.out + base + (size_t)r[q] * p.n + c[q]));
      } else {
        // values per group: G * (world - 1) loads in flight.  The eight-wave tile's accumulators
        // leave room for one value; the four-wave tile (one wave per SIMD) takes the whole slab.
        constexpr int G = T::NW == 8 ? 1 : Q;
        static_assert(Q % G == 0, "slab values split into whole groups");
#pragma unroll
        for (int g0 = 0; g0 < Q; g0 += G) {
          f32x4 t[G][MK_MAX_WORLD - 1];
#pragma unroll
          for (int pq = 0; pq < MK_MAX_WORLD - 1; ++pq) {
            if (pq >= p.world - 1) break;
            const float* src = peer_src(p, pq) + base;
#pragma unroll
            for (int gi = 0; gi < G; ++gi)
              t[gi][pq] = c[g0 + gi] < cols_valid
                              ? *reinterpret_cast<const f32x4*>(src + (size_t)r[g0 + gi] * p.n + c[g0 + gi])
                              : f32x4{0.f, 0.f, 0.f, 0.f};
          }
#pragma unroll
          for (int gi = 0; gi < G; ++gi) {
            f32x4 s = v[g0 + gi];
#pragma unroll
            for (int pq = 0; pq < MK_MAX_WORLD - 1; ++pq)
              if (pq < p.world - 1) s += t[gi][pq];
            if (c[g0 + gi] < cols_valid)
              __builtin_nontemporal_store(s, reinterpret_cast<f32x4*>(p.out + base + (size_t)r[g0 + gi] * p.n + c[g0 + gi]));
          }
        }
      }
    };
    if constexpr (kCore16<T>) g.epilogue_slab(T::epi_buf(wave, st0, st1, st2), wm, wn, lane, store_slab);
    else g.epilogue_slab(st0, st1, wm, wn, lane, wave, store_slab);
    __syncthreads();  // the next tile's prologue reuses the LDS
    t = -1;
  }
}

// Two-stage cores: the first two stage buffers double as the copy ring's slots, 8 KiB per wave.
template <class T>
constexpr int red_stage_bytes() {
  return T::STAGE > T::NW * 8192 ? T::STAGE : T::NW * 8192;
}

}  // namespace mk
