// AllGather + GEMM roles (copy and compute), one rank's share; the kernels that run them are
// ag_gemm_kernel (mk_ag_gemm.hip) and the MLP kernel (mk_mlp.hip).
//
// Operation (mKernel write-up, news.chathome.org page, five-fused-kernels table,
// AllGather + GEMM row): C = [A_0; A_1; ...; A_{W-1}] @ B, rank r holding the row shard A_r
// and B being local.  The product does not wait for the gather: a K-unit of a tile's rows
// enters the tile's K loop as soon as it is present.  Here the other ranks' shards are
// device buffers and their arrival is the copy role.
//
// Roles (section "mKernel的功能" of the same page: CTAs self-assign roles, a per-shape
// number of SMs per role):
//   workgroups [0, n_copy)          copy: for queue positions cid, cid + n_copy, ... of the
//                                   arrival order, copy that unit of a peer shard into its
//                                   rows of a_gathered (staged through LDS), then raise the
//                                   unit's ready flag.
//                                   Copy workgroups wait on nothing while copying but the clock
//                                   (link-rate pacing, bounded by the host), so every unit lands.
//   workgroups [n_copy, grid)       compute: 256 x 224 output tiles of C (one static tile per
//                                   workgroup, XCD-aware), then (like copy workgroups once they
//                                   have copied) tiles left over past the grid.  In emulated mode
//                                   a tile whose units have not all landed runs its K loop over
//                                   K-units (unit_cols columns of K) ready-first: wave 0 polls the
//                                   flags of the tile's unit rows and schedules the lowest-numbered
//                                   K-unit that has fully landed, ahead of the prefetch, so landed
//                                   data is consumed as it arrives; a copy workgroup waits until its
//                                   tile's units have landed and runs the loop in K order.
// A compute workgroup only ever waits on copy workgroups, which have lower ids and are therefore
// dispatched first; every wait is bounded by the watchdog.
#pragma once
#include "mk_internal.h"
#include "mk_gemm_tile.hpp"
#include "mk_gemm_tile16.hpp"
#include "mk_copy_ring.hpp"

namespace mk {

constexpr int AG_THREADS = TileGemm16::NW * 64;

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

// Units move through the two-slot LDS ring of mk_copy_ring.hpp (the stage buffers are idle in a
// copy workgroup): IPB KiB per wave and batch -- 8 (64 KiB slots: 2 units of 128x128, 4 of
// 64x128 / 128x64 or 8 of 64x64) or 4 (32 KiB slots: half as many).  IPU is a unit's DMA
// instructions per wave (1 KiB each).  The arrival order is read through the constant address
// space, so its loads are scalar, off the vector-memory counter the ring waits on.
template <int IPB, int IPU>
__device__ __forceinline__ void ag_copy_dma(const AgParams& p, int cid, char* st0, char* st1) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int cpr = p.unit_cols >> 3;  // 16-byte chunks per unit row
  const uint32_t ldb = (uint32_t)p.k * 2u;
  const uint32_t extent = ((uint32_t)(p.unit_rows - 1) * (uint32_t)p.k + (uint32_t)p.unit_cols) * 2u;
  const int n_units = p.n_urows * p.n_ucols;
  const int n_mine = p.n_order > cid ? (p.n_order - cid + p.n_copy - 1) / p.n_copy : 0;
  const __attribute__((address_space(4))) int32_t* order = (const __attribute__((address_space(4))) int32_t*)p.order;
  uint32_t off[IPU];  // byte offset inside a unit of this lane's chunk, per instruction of the unit
#pragma unroll
  for (int i = 0; i < IPU; ++i) {
    const int c = (wave * IPU + i) * 64 + lane;
    const int row = c / cpr, cc = c - row * cpr;
    off[i] = (uint32_t)row * ldb + (uint32_t)cc * 16u;
  }
  auto unit_at = [&](int i) -> int {  // i-th unit of this workgroup's queue, or -1
    if (i >= n_mine) return -1;
    const int pos = cid + i * p.n_copy;
    if (pos + 1 == p.drop_pos) return -1;  // testing: this unit never lands
    const int u = order ? order[pos] : ag_identity_unit(p, pos);
    return (u < 0 || u >= n_units) ? -1 : u;
  };
  auto src_of = [&](int u) {
    if (u < 0) return make_rsrc(p.ag, 0u);
    const int ur = u / p.n_ucols, uc = u - ur * p.n_ucols;
    const int grow = ur * p.unit_rows;
    const int r = grow / p.m_shard, srow = grow - r * p.m_shard;
    return make_rsrc(p.shards[r] + (size_t)srow * p.k + (size_t)uc * p.unit_cols, extent);
  };
  auto dst_of = [&](int u) {
    if (u < 0) return make_rsrc(p.ag, 0u);
    const int ur = u / p.n_ucols, uc = u - ur * p.n_ucols;
    return make_rsrc(p.ag + (size_t)ur * p.unit_rows * p.k + (size_t)uc * p.unit_cols, extent);
  };
  const uint64_t t0 = wall_ticks();
  copy_ring<IPB, IPU>(n_mine, st0, st1, off, unit_at, src_of, dst_of,
                    [&](int u) { flag_store(&p.flags[u], p.epoch); },
                    [&](int i) {  // queue entry i is arrival position cid + i * n_copy
                      if (p.pace_q16) wait_wall_until(t0 + (((uint64_t)(cid + i * p.n_copy) * p.pace_q16) >> 16));
                    });
}

static_assert(AG_THREADS == 512, "copy slots hold 8 waves' batches");

// SLOT_KIB: bytes of each of the two ring slots, in KiB (64 or 32)
template <int SLOT_KIB>
__device__ __forceinline__ void ag_copy_role(const AgParams& p, int cid, char* st0, char* st1) {
  constexpr int IPB = SLOT_KIB / 8;  // KiB per wave and batch
  static_assert(IPB == 8 || IPB == 4, "64 or 32 KiB slots");
  // DMA instructions per wave per unit: 4 (128x128), 2 (64x128, 128x64), 1 (64x64)
  const int ipu = (p.unit_rows * p.unit_cols * 2) / (AG_THREADS * 16);
  if (ipu == 4) ag_copy_dma<IPB, 4>(p, cid, st0, st1);
  else if (ipu == 2) ag_copy_dma<IPB, 2>(p, cid, st0, st1);
  else ag_copy_dma<IPB, 1>(p, cid, st0, st1);
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
// lanes take the same path and every ballot sees every unit's flag.  The scheduled-set mask `done`
// is wave 0's own (uniform, in scalar registers): kept in LDS as a volatile value it became a
// flat access, whose wait drained the K loop's operand loads in flight at every decision.
__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ int ag_pick(const AgParams& p, int ur0, int n_ur, uint64_t& done, int lane) {
  const uint64_t all = (p.n_ucols >= 64) ? ~0ull : ((1ull << p.n_ucols) - 1ull);
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
  done = uniform64(done | (1ull << u));
  return u;
}

// Wave 0: the flags of the tile's unit rows [ur0, ur0 + n_ur) (at most 4) for K-unit `lane`,
// requested straight into LDS (s_poll[q][lane]), so no register is held while the loads are in
// flight across a step's MFMAs.  Lanes past n_ucols read the next row's flags, which the ready
// mask ignores.
__device__ __forceinline__ void ag_poll_lds(const AgParams& p, int ur0, int n_ur, uint32_t* s_poll) {
  const auto rs = make_rsrc(p.flags + (size_t)ur0 * p.n_ucols, (uint32_t)(n_ur * p.n_ucols) * 4u);
#pragma unroll
  for (int q = 0; q < 4; ++q)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(s_poll + q * 64), 4,
                                             (uint32_t)(threadIdx.x & 63) * 4u, (uint32_t)(q * p.n_ucols) * 4u, 0,
                                             CP_SC1);
}
// Wave 0: landed-K-unit mask of a poll in LDS (uniform); the caller has waited for its DMA.
__device__ __forceinline__ uint64_t ag_ready_lds(const AgParams& p, int ur0, int n_ur, int lane,
                                                 const uint32_t* s_poll) {
  uint64_t ready = (p.n_ucols >= 64) ? ~0ull : ((1ull << p.n_ucols) - 1ull);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const bool skip = q >= n_ur || ag_row_local(p, ur0 + q);
    ready &= __ballot(skip || lane >= p.n_ucols || s_poll[q * 64 + lane] == p.epoch);
  }
  return uniform64(ready);
}

// Wave 0: nothing new has landed in the poll: poll again (sleeping between polls) until a unit
// not in `done` has landed.  Returns the new ready mask, or 0 on timeout or when another workgroup
// has recorded a fault.  Reuses the poll's registers, so the K loop that inlines it keeps its
// register budget.
__device__ __forceinline__ uint64_t ag_repoll_until_new(const AgParams& p, int ur0, int n_ur, int lane,
                                                        uint32_t* s_poll, uint64_t done) {
  const uint64_t t0 = wall_ticks();
  for (int n = 1;; ++n) {
    __builtin_amdgcn_s_sleep(2);
    ag_poll_lds(p, ur0, n_ur, s_poll);
    wait_vm<0>();
    const uint64_t ready = ag_ready_lds(p, ur0, n_ur, lane, s_poll);
    if (ready & ~done) return ready;
    if ((n & 7) == 0) {
      if (__builtin_amdgcn_readfirstlane(status_bad(p.status) ? 1 : 0)) return 0;
      if (wall_ticks() - t0 > p.timeout_ticks) {
        if (lane == 0) raise_status(p.status, ST_TIMEOUT);
        return 0;
      }
    }
  }
}

// The MLP block's activation: gelu(x) = x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2)), in fp32.
__device__ __forceinline__ float gelu_f32(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }

// fp32 -> bf16 bits, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// s_sched: entries 0 .. n_ucols - 1 name the K-unit each unit slot of the tile's K loop takes;
// entry AG_SCHED_ALL_IN says that every entry is written (the loop no longer polls).
constexpr int AG_SCHED_ALL_IN = 64;
constexpr int AG_SCHED_WORDS = AG_SCHED_ALL_IN + 1;

// One tile of the AllGather + GEMM kernel on the 256 x 224 core (mk_gemm_tile16.hpp), A loaded two
// steps ahead.  EMU: some of the tile's units have not landed yet, and the K loop visits K-units
// ready-first: before a step's DMA, wave 0 polls the flags of the tile's unit rows (straight into
// LDS), and after the step's MFMAs it names the lowest landed K-unit not yet scheduled as the one
// that starts four steps later (three steps of lead: the A of a step is requested two steps ahead,
// and every wave reads the schedule one step before that, so the LDS read's latency hides behind a
// step of MFMAs instead of delaying the DMA).  Once every unit of the tile's rows has landed, wave 0
// schedules the rest in ascending order and stops polling.  Without EMU every operand of the tile
// is present and the K loop runs in K order with no hooks.  Returns false if a wait failed (the
// tile's stores were skipped).
// EPI 0: fp32 C tile.  EPI 1 (the MLP block's up-projection): H = bf16(gelu(acc)), write-through
// (the down-projection reads it from other XCDs), then h_ready[tile row] += 1 once every wave's
// stores of the tile have completed.
template <bool EMU, int EPI>
__device__ __forceinline__ bool ag_tile16(const AgParams& p, int t, char* a0, char* a1, char* a2, char* b0, char* b1,
                                          int* s_sched, uint32_t* s_poll) {
  using G = TileGemm16;
  G g;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / G::WN, wn = wave % G::WN;
  const int nk = p.k >> 6;
  const int spu = p.unit_cols >> 6;  // k-steps per K-unit
  const int n_ku = p.n_ucols;
  const uint64_t all = (n_ku >= 64) ? ~0ull : ((1ull << n_ku) - 1ull);
  const uint32_t lda_b = (uint32_t)p.k * 2u, ldb_b = (uint32_t)p.n * 2u;
  g.init(wm, wn, wave, lane, lda_b, ldb_b);
  // a decision at the end of step q names the unit starting at step q + 1 + PD
  constexpr int PD = 3;
  const int n_pre = min(n_ku, (PD + spu) / spu);  // units starting at steps 0 .. PD, decided up front
  {
    const int tm = t / p.tiles_n, tn = t - tm * p.tiles_n;
    const int m0 = tm * G::BM, n0 = tn * G::BN;
    const int rows_valid = min(G::BM, p.m - m0), cols_valid = min(G::BN, p.n - n0);
    const int ur0 = m0 / p.unit_rows, n_ur = rows_valid / p.unit_rows;
    const char* a_tile = reinterpret_cast<const char*>(p.ag + (size_t)m0 * p.k);
    const uint32_t a_tile_bytes = (uint32_t)rows_valid * lda_b;
    const char* b_col = reinterpret_cast<const char*>(p.b + n0);
    const uint32_t b_col_bytes = ((uint32_t)p.k * (uint32_t)p.n - (uint32_t)n0) * 2u;
    g.zero();
    uint64_t done = 0;    // wave 0: K-units scheduled for this tile
    bool all_in = false;  // wave 0: every unit has landed and the whole schedule is written
    if constexpr (EMU) {
      if (wave == 0) {
        if (lane == 0) s_sched[AG_SCHED_ALL_IN] = 0;
        for (int j = 0; j < n_pre; ++j) {
          const int u = ag_pick(p, ur0, n_ur, done, lane);
          if (lane == 0) s_sched[j] = u;
          if (u < 0) break;
        }
      }
      __syncthreads();
      bool bad = false;
      for (int j = 0; j < n_pre; ++j) bad |= __builtin_amdgcn_readfirstlane(s_sched[j]) < 0;
      if (bad) return false;  // before any MFMA of this tile
    }
    // A failed wait (watchdog or another workgroup's fault) inside the K loop does not leave the
    // loop: the remaining steps drain on K-unit 0 (in bounds, result discarded) and the tile's
    // stores are skipped.
    bool aborted = false;
    // EMU: K offsets (in steps of 64) of the next B (step q+1) and A (step q+2) DMA, and the raw
    // schedule entry of step q+3's unit, read one step ahead
    int ks_b = 0, ks_a = 0, raw_n = 0;
    auto decode = [&](int raw, int s) -> int {
      const int u = __builtin_amdgcn_readfirstlane(raw);
      aborted |= u < 0;
      return (u < 0 ? 0 : u) * spu + s % spu;
    };
    auto dma_a = [&](int ks, char* dst) {
      const uint32_t ca = (uint32_t)ks * 128u;
      g.dma_a(a_tile + ca, a_tile_bytes - ca, lda_b, dst, wave);
    };
    auto dma_b = [&](int ks, char* dst) {
      const uint32_t rb = (uint32_t)ks * 64u * ldb_b;
      g.dma_b(b_col + rb, b_col_bytes - rb, dst, wave);
    };
    auto prologue = [&](char* pa0, char* pb0, char* pa1) {
      const int k0 = EMU ? decode(s_sched[0], 0) : 0;
      const int k1 = nk > 1 ? (EMU ? decode(s_sched[1 / spu], 1) : 1) : 0;
      dma_a(k0, pa0);
      dma_b(k0, pb0);
      if (nk > 1) dma_a(k1, pa1);
      ks_b = k1;
      raw_n = (EMU && nk > 2) ? s_sched[2 / spu] : 0;
    };
    auto load_a = [&](int s, char* dst) { dma_a(EMU ? ks_a : s, dst); };
    auto load_b = [&](int s, char* dst) { dma_b(EMU ? ks_b : s, dst); };
    bool polled = false;
    auto decided_at = [&](int q) -> int {  // the unit decided at the end of step q, or -1
      const int s = q + 1 + PD;
      if (s >= nk || s % spu) return -1;
      const int jn = s / spu;
      return (jn >= n_pre && jn < n_ku) ? jn : -1;
    };
    auto before_load = [&](int q, auto ph) {
      if constexpr (EMU) {
        ks_a = decode(raw_n, q + 2);
        if constexpr (decltype(ph)::heavy) {
          polled = wave == 0 && !all_in && decided_at(q) >= 0;
          if (polled) ag_poll_lds(p, ur0, n_ur, s_poll);
        }
      }
    };
    auto after_load = [&](int q, auto) {
      if constexpr (EMU) {
        ks_b = ks_a;
        raw_n = q + 3 < nk ? s_sched[(q + 3) / spu] : 0;
      }
    };
    auto before_wait = [&](int q, auto ph) {
      if constexpr (EMU && decltype(ph)::heavy) {
        if (polled) {
          const int jn = decided_at(q);
          // the poll was requested before this step's B and A DMA: only those may still be in flight
          // (wave 0 issues 4 B and 4 A instructions per step)
          wait_vm<4 + G::A_INSTR>();
          uint64_t ready = ag_ready_lds(p, ur0, n_ur, lane, s_poll);
          if ((ready & ~done) == 0) ready = ag_repoll_until_new(p, ur0, n_ur, lane, s_poll, done);
          if (ready == 0) {  // timeout or fault: the loop drains on K-unit 0 and skips the stores
            if (lane == 0) s_sched[jn] = -1;
          } else if (ready == all) {  // every unit is here: the rest in ascending order
            for (int j = jn; j < n_ku; ++j) {
              const int u = __builtin_ctzll(~done & all);
              done |= 1ull << u;
              if (lane == 0) s_sched[j] = u;
            }
            all_in = true;
            if (lane == 0) s_sched[AG_SCHED_ALL_IN] = 1;
          } else {
            const int u = __builtin_ctzll(ready & ~done);
            done |= 1ull << u;
            if (lane == 0) s_sched[jn] = u;
          }
        }
      }
    };
    // every unit scheduled: the rest of the loop runs without the polling and deciding code
    auto leave = [&]() -> bool {
      if constexpr (EMU) return __builtin_amdgcn_readfirstlane(s_sched[AG_SCHED_ALL_IN]) != 0;
      else return true;
    };
    k_loop_a3b2(g, nk, a0, a1, a2, b0, b1, prologue, load_a, load_b, before_load, after_load, before_wait, leave);

    // epilogue: the tile staged through the A slots into row-contiguous 16-byte stores; C is
    // written once and read by no one here: streaming stores
    float* wl = G::epi_buf(wave, a0, a1, a2);
    if constexpr (EPI == 0) {
      g.epilogue(wl, wm, wn, lane, [&](int row, int col, f32x4 v) {
        if (!aborted && row < rows_valid && col < cols_valid)
          __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p.c + (size_t)(m0 + row) * p.n + (n0 + col)));
      });
      __syncthreads();  // the next tile's prologue reuses the LDS
    } else {
      const auto h_rs = make_rsrc(p.h, (uint32_t)p.m * (uint32_t)p.n * 2u);
      g.epilogue(wl, wm, wn, lane, [&](int row, int col, f32x4 v) {
        if (!aborted && row < rows_valid && col < cols_valid) {
          const uint32_t h0 = bf16_rne(gelu_f32(v[0])), h1 = bf16_rne(gelu_f32(v[1]));
          const uint32_t h2 = bf16_rne(gelu_f32(v[2])), h3 = bf16_rne(gelu_f32(v[3]));
          bstore8_sc1(h_rs, (uint32_t)((m0 + row) * p.n + (n0 + col)) * 2u, u32x2{h0 | (h1 << 16), h2 | (h3 << 16)});
        }
      });
      wait_mem();       // this tile's H stores have completed ...
      __syncthreads();  // ... in every wave (and the next tile's prologue reuses the LDS)
      if (!aborted && threadIdx.x == 0) atomic_add_agent(p.h_ready + m0 / G::BM, 1u);  // (tm: not kept live across the loop)
    }
    return !aborted;
  }
}

// Wave 0: spin (sleeping between polls) until every K-unit of unit rows [ur0, ur0 + n_ur) has
// landed; false on timeout or when another workgroup has recorded a fault.
__device__ __forceinline__ bool ag_wait_rows(const AgParams& p, int ur0, int n_ur, int lane) {
  const uint64_t all = (p.n_ucols >= 64) ? ~0ull : ((1ull << p.n_ucols) - 1ull);
  const uint64_t t0 = wall_ticks();
  for (int n = 0; uniform64(ag_ready_mask(p, ur0, n_ur, all, lane)) != all; ++n) {
    __builtin_amdgcn_s_sleep(2);
    if ((n & 7) == 7) {
      if (__builtin_amdgcn_readfirstlane(status_bad(p.status) ? 1 : 0)) return false;
      if (wall_ticks() - t0 > p.timeout_ticks) {
        if (lane == 0) raise_status(p.status, ST_TIMEOUT);
        return false;
      }
    }
  }
  return true;
}

// Tile rows [lt0, lt1) lie wholly inside the local shard's rows when that shard is already in
// place in a_gathered (emulated arrival): their operands are present at launch.
__device__ __forceinline__ void ag_local_tile_rows(const AgParams& p, int& lt0, int& lt1) {
  lt0 = lt1 = 0;
  if (!p.emulated || !p.local_in_place) return;
  constexpr int BM = TileGemm16::BM;
  const int r0 = p.rank * p.m_shard, r1 = r0 + p.m_shard;
  lt0 = (r0 + BM - 1) / BM;
  lt1 = max(lt0, r1 / BM);
}

// Static tile of workgroup wg (or -1).  When the compute workgroups alone can hold every tile they
// do, in XCD-aware order: the k-th of the n compute workgroups runs on XCD k % 8 (workgroup w runs
// on XCD w % 8 and n_copy is a multiple of 8) and owns logical tile (k % 8) * (n / 8) + k / 8, so an
// XCD's tiles are consecutive (whole tile rows, sharing their A rows in its L2).  Otherwise every
// workgroup of the grid owns one (copy workgroups start theirs after copying; tiles past the grid
// are claimed from a counter), taken in order of readiness: the compute workgroups, which start at
// once, take the tiles whose rows are local first, and the copy workgroups the rest, each set
// XCD-aware in the same way.
__device__ __forceinline__ int ag_static_tile(const AgParams& p, int wg, int grid) {
  const int n_tiles = p.tiles_m * p.tiles_n;
  if (n_tiles <= p.n_compute) {
    const int k = wg - p.n_copy, n = p.n_compute;
    if (k < 0 || k >= n) return -1;  // not one of the n (a second owner of a tile would count it twice)
    const int rs = (n & 7) == 0 ? (k & 7) * (n >> 3) + (k >> 3) : k;
    return rs < n_tiles ? rs : -1;
  }
  if (wg < 0 || wg >= grid) return -1;
  const bool comp = wg >= p.n_copy;
  const int base = comp ? p.n_copy : 0, cnt = comp ? grid - p.n_copy : p.n_copy;
  const int k = wg - base;
  const int pos = ((cnt & 7) == 0 && (base & 7) == 0) ? (k & 7) * (cnt >> 3) + (k >> 3) : k;
  const int s = (comp ? 0 : grid - p.n_copy) + pos;  // place in the readiness order
  if (s >= n_tiles) return -1;
  int lt0, lt1;
  ag_local_tile_rows(p, lt0, lt1);
  const int first = lt0 * p.tiles_n, nl = (lt1 - lt0) * p.tiles_n;
  if (s < nl) return first + s;  // the local tile rows, row-major
  const int r = s - nl;          // then the others, row-major
  return r < first ? r : r + nl;
}

// Compute role of the AllGather + GEMM kernel.  The workgroup first runs tile t_static (-1: none),
// then tiles left over past the grid, claimed from a shared counter.  With emulated arrival, wave 0
// looks at the flags of a tile's unit rows first: when every unit has landed the tile runs the K
// loop without hooks (K order, as with resident operands); otherwise a workgroup that starts its
// tiles only after copying (wait_landed) waits until they have -- its copy ends near the end of
// the landing, and the loop without hooks is faster than the ready-first one by more than the
// wait -- and the others run the ready-first loop, consuming each K-unit as soon as it has landed.
// mark_ready: record the first tile's operands-ready time in trace slot 5 (compute workgroups; a
// copy workgroup's slot 5 holds the end of its copy).  READY_FIRST = false leaves the ready-first
// loop out of the build (the caller sets wait_landed everywhere).
template <int EPI, bool READY_FIRST = true>
__device__ __forceinline__ void ag_compute_role16(const AgParams& p, int t_static, bool mark_ready, bool wait_landed,
                                                  char* a0, char* a1, char* a2, char* b0, char* b1, int* s_sched,
                                                  int* s_claim, uint32_t* s_poll) {
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n_tiles = p.tiles_m * p.tiles_n;
  bool first = mark_ready;
  int t = t_static;
  while (true) {
    if (t < 0) {
      if (tid == 0) *s_claim = (int)gridDim.x + (int)atomic_add_agent(p.counters + CTR_AG_TILE, 1u);
      __syncthreads();
      t = *s_claim;  // rewritten only after the tile's barriers
      __syncthreads();
      if (t >= n_tiles) break;
    }
    bool emu = false;
    if (p.emulated) {
      const int m0 = (t / p.tiles_n) * TileGemm16::BM;
      const int ur0 = m0 / p.unit_rows, n_ur = min(TileGemm16::BM, p.m - m0) / p.unit_rows;
      if (wave == 0) {
        const uint64_t all = (p.n_ucols >= 64) ? ~0ull : ((1ull << p.n_ucols) - 1ull);
        int state = uniform64(ag_ready_mask(p, ur0, n_ur, all, lane)) == all ? 0 : 1;  // 0: landed, 1: not yet
        if (state == 1 && wait_landed) state = ag_wait_rows(p, ur0, n_ur, lane) ? 0 : 2;  // 2: failed
        if (lane == 0) *s_claim = state;
      }
      __syncthreads();
      const int state = *s_claim;
      __syncthreads();
      if (state == 2) break;
      emu = state == 1;
    }
    if (first) trace_mark(p.trace, 5);
    first = false;
    bool ok;
    if constexpr (READY_FIRST)
      ok = emu ? ag_tile16<true, EPI>(p, t, a0, a1, a2, b0, b1, s_sched, s_poll)
               : ag_tile16<false, EPI>(p, t, a0, a1, a2, b0, b1, s_sched, s_poll);
    else  // wait_landed is set: a tile never starts before its units have landed
      ok = ag_tile16<false, EPI>(p, t, a0, a1, a2, b0, b1, s_sched, s_poll);
    if (!ok) break;
    t = -1;
  }
}

}  // namespace mk
