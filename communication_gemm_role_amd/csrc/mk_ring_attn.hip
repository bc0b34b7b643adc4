// Ring attention, one rank's share, as one persistent launch.
//
// Operation (mKernel write-up, news.chathome.org page, five-fused-kernels table, Ring Attention
// row).  Rank r holds the queries of its sequence shard; the answer it needs is
//   out[h, i, :] = sum_j softmax_j(scale * q[h, i] . k[h, j]) v[h, j, :]   over all world * s_local keys
// (no mask: the pages name no causal variant).  The peers' K/V shards travel round the ring, and
// the attention starts on each peer block once that block is present, inside the same launch.
// Here the other ranks' K/V shards are device buffers and the ring transfer is the copy role.
//
// Roles:
//   workgroups [0, n_copy)   copy: for arrival positions cid, cid + n_copy, ... land a 64-key
//                            block of K or V of a peer shard in the ring buffers (16 KiB, through
//                            the LDS ring of mk_copy_ring.hpp), then raise its flag.  The default
//                            order is the ring's: step t brings rank (r - t) mod world, step by
//                            step, each step head by head and block by block, K before V.
//   workgroups [n_copy, ..)  compute: items (head, 128-query tile), one static item per workgroup,
//                            then items left over, claimed from a counter (copy workgroups join
//                            once their blocks have landed).  An item visits its own rank's blocks
//                            first and then the ring steps in order, waiting for each peer block's
//                            K and V flags before requesting it.
//
// Compute item: eight waves, two per SIMD: four query groups of 32 queries, each split over the
// two 32-key halves of every 64-key block (wave w: queries 32*(w%4).., keys 32*(w/4).. of each
// block), so one wave's softmax runs while the other wave of its SIMD issues MFMAs; the two halves'
// softmax states are merged at the end of the item.  Per 32-key half-block (three LDS stages of
// 64-key blocks, DMA-fed):
//   S^T = K Q^T       (v_mfma_f32_32x32x16_bf16: A = K rows from LDS, B = Q^T kept in registers),
//   online softmax    per query column: running max and sum in fp32, exp2 with the scale folded
//                     into log2 units; a query's 64 values sit in two lanes (l and l + 32);
//   O^T += V^T P^T    A = V^T by transposed LDS reads, B = P^T straight from the S^T accumulators.
// Computing the transposes makes P^T's MFMA operand layout that of the S^T accumulator (up to an
// order of the keys inside each 16-key step, which V^T's reads follow), and puts each query's
// softmax state in the lanes that hold its O^T column, so no value crosses lanes but the two
// max/sum exchanges.  P^T enters the MFMA as two bf16 terms, hi = bf16(p) and lo = bf16(p - hi),
// so the weights carry 16 significant bits: with one bf16 term the rounding of p alone puts the
// output's error near 1e-3 of its RMS.
#include "mk_internal.h"
#include "mk_gemm_tile.hpp"
#include "mk_copy_ring.hpp"

namespace mk {

constexpr int RA_NW = 8;             // waves per workgroup: 4 query groups x 2 key halves
constexpr int RA_THREADS = RA_NW * 64;
constexpr int RA_QG = 4;             // query groups of 32
constexpr int RA_BQ = RA_QG * 32;    // queries per item
constexpr int RA_BK = 64;            // keys per block
constexpr int RA_ROW = RA_D * 2;     // bytes per K/V row (head dim 128, bf16)
constexpr int RA_BLK = RA_BK * RA_ROW;  // 16 KiB: one block of K or of V
constexpr int RA_STAGE = 2 * RA_BLK;    // K then V
constexpr int RA_INSTR = RA_BLK / RA_NW / 1024;  // 1 KiB DMA instructions per wave per block
static_assert(RA_INSTR == 2, "a wave moves 8 rows of K and 8 of V per block");
constexpr int RA_CP_IPB = RA_STAGE / RA_NW / 1024;  // copy ring: KiB per wave and batch (a slot = a stage)

// ------------------------------------------------------------------------------------------
// copy role
// ------------------------------------------------------------------------------------------
// Unit u = ((j * heads + h) * n_blk + b) * 2 + kv: block b (64 keys) of head h of rank j's K
// (kv = 0) or V (kv = 1).  A block is 16 KiB contiguous in the shard and in the ring buffer.
__device__ __forceinline__ int ra_ring_unit(const RaParams& p, int pos) {
  const int per_step = p.heads * p.n_blk * 2;
  const int t = pos / per_step + 1, w = pos - (t - 1) * per_step;
  const int j = (p.rank - t + p.world) % p.world;
  return j * per_step + w;
}

__device__ __forceinline__ void ra_copy_role(const RaParams& p, int cid, char* st0, char* st1) {
  constexpr int IPU = RA_INSTR;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_mine = p.n_order > cid ? (p.n_order - cid + p.n_copy - 1) / p.n_copy : 0;
  const __attribute__((address_space(4))) int32_t* order = (const __attribute__((address_space(4))) int32_t*)p.order;
  uint32_t off[IPU];
#pragma unroll
  for (int i = 0; i < IPU; ++i) off[i] = (uint32_t)((wave * IPU + i) * 64 + lane) * 16u;
  auto unit_at = [&](int i) -> int {
    if (i >= n_mine) return -1;
    const int pos = cid + i * p.n_copy;
    if (pos + 1 == p.drop_pos) return -1;  // testing: this unit never lands
    const int u = order ? order[pos] : ra_ring_unit(p, pos);
    return (u < 0 || u >= p.n_units || u / (p.heads * p.n_blk * 2) == p.rank) ? -1 : u;
  };
  auto block_elem = [&](int u) -> size_t {  // first element of unit u's block inside a shard
    const int w = u % (p.heads * p.n_blk * 2) / 2;
    return (size_t)w * RA_BK * RA_D;
  };
  auto src_of = [&](int u) {
    if (u < 0) return make_rsrc(p.k_ring, 0u);
    const int j = u / (p.heads * p.n_blk * 2);
    return make_rsrc(((u & 1) ? p.v_src[j] : p.k_src[j]) + block_elem(u), (uint32_t)RA_BLK);
  };
  auto dst_of = [&](int u) {
    if (u < 0) return make_rsrc(p.k_ring, 0u);
    const int j = u / (p.heads * p.n_blk * 2);
    return make_rsrc(((u & 1) ? p.v_ring : p.k_ring) + (size_t)j * p.heads * p.s_local * RA_D + block_elem(u),
                     (uint32_t)RA_BLK);
  };
  const uint64_t t0 = wall_ticks();
  copy_ring<RA_CP_IPB, IPU>(n_mine, st0, st1, off, unit_at, src_of, dst_of,
                    [&](int u) { flag_store(&p.flags[u], p.epoch); },
                    [&](int i) {  // queue entry i is arrival position cid + i * n_copy
                      if (p.pace_q16) wait_wall_until(t0 + (((uint64_t)(cid + i * p.n_copy) * p.pace_q16) >> 16));
                    });
}

// ------------------------------------------------------------------------------------------
// compute role
// ------------------------------------------------------------------------------------------
struct RaLanes {
  uint32_t k_dma[RA_INSTR];  // K DMA: LDS row chunk lane&15 <- global chunk (lane&15) ^ (row & 15)
  uint32_t v_dma;            // V DMA: LDS row chunk lane&15 <- global chunk (lane&15) ^ 4*(row & 3)
  uint32_t k_rd;             // K operand read (key fragment 0, d-step 0)
  uint32_t v_rd[4];          // V^T operand read per 32-wide d fragment (key step 0, first half)
};

__device__ __forceinline__ void ra_lanes(RaLanes& L, int lane, int wave) {
  // instruction i of wave w moves rows 8w + 4i + (lane>>4) of the block (4 rows of 256 bytes)
  const int rr = lane >> 4, c = lane & 15;
#pragma unroll
  for (int i = 0; i < RA_INSTR; ++i)
    L.k_dma[i] = (uint32_t)rr * RA_ROW + (uint32_t)(c ^ ((8 * (wave & 1) + 4 * i + rr) & 15)) * 16u;
  L.v_dma = (uint32_t)rr * RA_ROW + (uint32_t)(c ^ (4 * (rr & 3))) * 16u;
  // K as the A operand: row = key lane%32, 16-byte chunk 2*kk + lane/32 (swizzled by row & 15)
  L.k_rd = (uint32_t)(lane & 31) * RA_ROW;
  // V^T as the A operand: in each 16-lane group g, lane s reads 8 bytes at row 4*(g>>1) + (s>>2)
  // of the key step and columns 32*i + 16*(g&1) + 4*(s&3) .. +3; two reads 8 rows apart give
  // keys {4h + 0..3, 4h + 8..11} of the step (h = lane/32), the order in which the S^T accumulator
  // holds them.
  const int g = lane >> 4, s = lane & 15, jr = s >> 2, q = s & 3;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int nb = 32 * i + 16 * (g & 1) + 4 * q;
    L.v_rd[i] = (uint32_t)(4 * (g >> 1) + jr) * RA_ROW + (uint32_t)(((nb >> 3) ^ (4 * jr)) << 4) +
                (uint32_t)((nb & 7) << 1);
  }
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// The value lane l ^ 32 holds: one swap of the wave's two halves (v_permlane32_swap, a VALU
// instruction) instead of a permute through the LDS unit, which the block's operand reads keep busy.
__device__ __forceinline__ float ra_xor32(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);  // {this half, the other half}
  return __builtin_bit_cast(float, (threadIdx.x & 32) ? r[0] : r[1]);
}
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two softmax weights as packed bf16 hi and lo terms: hi = bf16(p), lo = bf16(p - hi), both
// rounded to nearest even by the hardware's packed conversion (v_cvt_pk_bf16_f32), one
// instruction per pair and term.
__device__ __forceinline__ void ra_split2(float a, float b, uint32_t& hi, uint32_t& lo) {
  const f32x2 v = {a, b};
  const bf16x2 h = __builtin_convertvector(v, bf16x2);
  const f32x2 r = v - __builtin_convertvector(h, f32x2);  // exact: p - hi fits in fp32
  hi = __builtin_bit_cast(uint32_t, h);
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2));
}

// Items and XCDs.  Items (head-major, so consecutive items share a head's K and V) are dealt to
// the 8 XCDs in contiguous blocks, and a workgroup on XCD x (workgroup w runs on XCD w % 8)
// computes items of x's block, so a head's keys and values are pulled into one L2 (one head per
// XCD at 8 heads).  The compute workgroups on XCD x take the head of its block as static items;
// the rest is claimed from XCD x's counter by the workgroups on x that have finished their own
// work (copy workgroups after landing their blocks), and by other XCDs' once theirs are exhausted.
struct RaXcd {
  int b, n, n_static;  // block [b, b + n) of XCD x; its first n_static items are static
};
__device__ __forceinline__ RaXcd ra_xcd(const RaParams& p, int x) {
  RaXcd r;
  r.b = x * (p.n_items >> 3) + min(x, p.n_items & 7);
  r.n = (p.n_items >> 3) + (x < (p.n_items & 7) ? 1 : 0);
  const int off = (x - p.n_copy) & 7;  // first compute workgroup on XCD x: id n_copy + off
  const int c_x = p.n_compute > off ? (p.n_compute - off + 7) >> 3 : 0;
  r.n_static = min(c_x, r.n);
  return r;
}
// Thread 0: the next leftover item for a workgroup on XCD x (its own block first), or n_items.
__device__ __forceinline__ int ra_claim(const RaParams& p, int x) {
  for (int i = 0; i < 8; ++i) {
    const int xx = (x + i) & 7;
    const RaXcd z = ra_xcd(p, xx);
    const uint32_t left = (uint32_t)(z.n - z.n_static);
    if (left == 0 || flag_load(p.counters + CTR_RA_XITEM0 + xx) >= left) continue;
    const uint32_t idx = atomic_add_agent(p.counters + CTR_RA_XITEM0 + xx, 1u);
    if (idx < left) return z.b + z.n_static + (int)idx;
  }
  return p.n_items;
}

__device__ __forceinline__ void ra_compute_role(const RaParams& p, int slot, char* st0, char* st1, char* st2,
                                                int* s_claim) {
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int qg = wave & 3, kh = wave >> 2;  // query group, key half of every block
  RaLanes L;
  ra_lanes(L, lane, wave);
  const int x = blockIdx.x & 7;
  const int nb = p.world * p.n_blk;  // blocks per item
  const size_t shard_elems = (size_t)p.heads * p.s_local * RA_D;
  int t = -1;
  if (slot >= 0) {  // this compute workgroup's static item: its index among XCD x's compute workgroups
    const RaXcd z = ra_xcd(p, x);
    const int j = (int)(blockIdx.x - (p.n_copy + ((x - p.n_copy) & 7))) >> 3;
    t = j < z.n_static ? z.b + j : -1;
  }
  bool first = slot >= 0;
  bool landed = false;  // every peer block has landed (this wave saw the copy role's counter)
  while (true) {
    if (t < 0) {
      if (tid == 0) *s_claim = ra_claim(p, x);
      __syncthreads();
      t = *s_claim;
      if (t >= p.n_items) break;
    }
    const int h = t / p.n_qt, qt = t - h * p.n_qt;
    const int q0 = qt * RA_BQ + qg * 32;  // this wave's first query
    // Q^T as the B operand, kept in registers: lane holds query q0 + lane%32, d = 16*kk + 8*half .. +7
    bf16x8 qf[8];
    {
      const auto qr = make_rsrc(p.q + ((size_t)h * p.s_local + q0) * RA_D, 32u * RA_ROW);
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        qf[kk] = __builtin_bit_cast(bf16x8, bload16(qr, (uint32_t)(lane & 31) * RA_ROW + (uint32_t)(2 * kk + half) * 16u));
    }
    f32x16 o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[i][r] = 0.f;
    float m_run = -__builtin_inff(), l_run = 0.f;
    bool aborted = false;

    // block q of the item: own rank's blocks first, then ring step 1, 2, ...
    auto rank_of = [&](int q) { return (p.rank - q / p.n_blk + p.world) % p.world; };
    auto unit_of = [&](int q) {  // K unit of block q (V is the next one)
      return ((rank_of(q) * p.heads + h) * p.n_blk + q % p.n_blk) * 2;
    };
    // every wave waits for the block's K and V itself, then requests its share of them; once
    // every copy workgroup has landed all of its blocks (one counter, every lane reading the same
    // address), the wave stops polling flags for good
    auto before_load = [&](int q) {
      if (!p.emulated || rank_of(q) == p.rank || landed) return;
      if (p.drop_pos == 0 && p.n_copy > 0 &&
          __builtin_amdgcn_readfirstlane(flag_load(p.counters + CTR_RA_LANDED) >= (uint32_t)p.n_copy ? 1 : 0)) {
        landed = true;
        return;
      }
      const int u = unit_of(q);
      bool ok = true;
      if (lane == 0)
        ok = spin_until_eq(&p.flags[u], p.epoch, p.timeout_ticks, p.status) &&
             spin_until_eq(&p.flags[u + 1], p.epoch, p.timeout_ticks, p.status);
      aborted |= __builtin_amdgcn_readfirstlane((int)ok) == 0;
    };
    auto load = [&](int q, char* dst) {
      // a failed wait drains the loop on the item's first block (in bounds, result discarded)
      const int j = aborted ? p.rank : rank_of(q), b = aborted ? 0 : q % p.n_blk;
      const size_t e = ((size_t)h * p.s_local + (size_t)b * RA_BK) * RA_D;
      const bool ring = p.emulated && j != p.rank;
      const char* kb = reinterpret_cast<const char*>(ring ? p.k_ring + (size_t)j * shard_elems + e : p.k_src[j] + e);
      const char* vb = reinterpret_cast<const char*>(ring ? p.v_ring + (size_t)j * shard_elems + e : p.v_src[j] + e);
#pragma unroll
      for (int i = 0; i < RA_INSTR; ++i) {
        const int r0 = wave * 8 + 4 * i;  // this instruction's 4 rows of the block
        __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(kb + r0 * RA_ROW, 4u * RA_ROW),
                                                 (__attribute__((address_space(3))) void*)(dst + r0 * RA_ROW), 16,
                                                 L.k_dma[i], 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(vb + r0 * RA_ROW, 4u * RA_ROW),
                                                 (__attribute__((address_space(3))) void*)(dst + RA_BLK + r0 * RA_ROW),
                                                 16, L.v_dma, 0, 0, 0);
      }
    };
    // one 64-key block from stage `lds`.  Operand fragments are read ahead of their MFMAs (K two
    // k-steps ahead, V^T one step ahead and its first step before the softmax, whose VALU work
    // hides that latency); the scheduling fences keep the compiler from collapsing the order into
    // read-wait-MFMA pairs (with two waves per SIMD most LDS latency would still be exposed) or from
    // hoisting every read at once (registers).
    auto kread = [&](const char* lds, int kk, int f) -> bf16x8 {
      const int c = 2 * kk + half, row = 32 * f + (lane & 31);
      return *reinterpret_cast<const bf16x8*>(lds + L.k_rd + 32 * f * RA_ROW + ((c ^ (row & 15)) << 4));
    };
    auto vread = [&](const char* lds, int kk, bf16x8* v) {
      const char* vb = lds + RA_BLK + 16 * kk * RA_ROW;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const i16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(const_cast<char*>(vb) + L.v_rd[i]));
        const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(const_cast<char*>(vb) + L.v_rd[i] + 8 * RA_ROW));
        v[i] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    };
    // this wave's half (keys 32*kh .. 32*kh + 31) of one 64-key block from stage `lds`
    auto step = [&](const char* lds) {
      f32x16 sc;
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[r] = 0.f;
      bf16x8 kb[3];
      kb[0] = kread(lds, 0, kh);
      kb[1] = kread(lds, 1, kh);
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        if (kk + 2 < 8) kb[(kk + 2) % 3] = kread(lds, kk + 2, kh);
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb[kk % 3], qf[kk], sc, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      bf16x8 vf[2][4];
      vread(lds, 2 * kh, vf[0]);
      __builtin_amdgcn_sched_barrier(0);
      // online softmax of this lane's query over the half-block (the other 16 of its keys are in
      // lane ^ 32)
      // The scale (in log2 units; the planner admits only positive scales) is applied inside the
      // exponent: the max is taken on the raw scores (rounding is monotone, so scaling the raw max
      // gives the max of the scaled scores) and each weight is exp2(fma(s, scale, -max)).
      const float c = p.scale_log2;
      float mx = -__builtin_inff();
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[r]);
      mx = fmaxf(mx, ra_xor32(mx)) * c;
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      float sum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sc[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[r], c, -m_new));
        sum += sc[r];
      }
      sum += ra_xor32(sum);
      l_run = l_run * alpha + sum;
      m_run = m_new;
      // rescale only when some query's running max moved (alpha == 1 everywhere else: a no-op); after
      // the first blocks the max of a query's scores rarely moves
      if (__builtin_amdgcn_readfirstlane((int)(__ballot(alpha != 1.f) != 0)))
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
      // O^T += V^T P^T over the half-block's two 16-key steps, P^T as hi + lo bf16 terms
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (j == 0) vread(lds, 2 * kh + 1, vf[1]);
        bf16x8 ph, pl;
        {
          u32x4 hw, lw;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            uint32_t hv, lv;
            ra_split2(sc[8 * j + 2 * e], sc[8 * j + 2 * e + 1], hv, lv);
            hw[e] = hv;
            lw[e] = lv;
          }
          ph = __builtin_bit_cast(bf16x8, hw);
          pl = __builtin_bit_cast(bf16x8, lw);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          o[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[j][i], ph, o[i], 0, 0, 0);
          o[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[j][i], pl, o[i], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    if (first) trace_mark(p.trace, 5);
    first = false;
    // three-stage pipeline over static stage buffers: block q+2 is requested before block q's work
    constexpr int D = 2 * RA_INSTR;
    load(0, st0);
    if (nb > 1) {
      before_load(1);
      load(1, st1);
      wait_vm<D>();
    } else {
      wait_vm<0>();
    }
    __syncthreads();
    auto sub = [&](int q, const char* cur, char* pf) {
      if (q >= nb) return;
      const bool more = q + 2 < nb;
      if (more) {
        before_load(q + 2);
        load(q + 2, pf);
      }
      step(cur);
      if (more) wait_vm<D>();
      else wait_vm<0>();
      __syncthreads();
    };
    for (int q = 0; q < nb; q += 3) {
      sub(q, st0, st2);
      sub(q + 1, st1, st0);
      sub(q + 2, st2, st1);
    }

    // a wave that timed out (or saw another workgroup's fault) voids the item for all eight
    aborted = __syncthreads_or(aborted) != 0;
    if (!aborted) {
      // key half 1 hands its softmax state (running max and sum, O^T) to key half 0 of the same
      // queries through the idle stage buffers (every wave has left the K loop's last barrier)
      float* xo = reinterpret_cast<float*>((qg < 2 ? st0 : st1) + (qg & 1) * 16384);
      float* xm = reinterpret_cast<float*>(st2) + qg * 128;
      if (kh == 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) xo[(i * 16 + r) * 64 + lane] = o[i][r];
        xm[lane] = m_run;
        xm[64 + lane] = l_run;
      }
      __syncthreads();
      if (kh == 0) {
        // merge: m = max(m0, m1); O^T = O0 2^(m0 - m) + O1 2^(m1 - m), the sums likewise
        const float m1 = xm[lane], l1 = xm[64 + lane];
        const float m = fmaxf(m_run, m1);
        const float a0 = __builtin_amdgcn_exp2f(m_run - m), a1 = __builtin_amdgcn_exp2f(m1 - m);
        const float l = l_run * a0 + l1 * a1;
        const float inv = 1.f / l;
        // O = O^T / l; lane holds query q0 + lane%32, d = 32*i + 8*(r/4) + 4*half + r%4
        float* orow = p.out + ((size_t)h * p.s_local + q0 + (lane & 31)) * RA_D;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 4 * g4 + e;
              v[e] = (o[i][r] * a0 + xo[(i * 16 + r) * 64 + lane] * a1) * inv;
            }
            __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(orow + 32 * i + 8 * g4 + 4 * half));
          }
        if (p.lse && half == 0)
          p.lse[(size_t)h * p.s_local + q0 + lane] = (m + __builtin_amdgcn_logf(l)) * 0.69314718055994531f;
      }
    }
    __syncthreads();  // the next item's loads reuse the stage buffers
    if (aborted) break;
    t = -1;
  }
}

__global__ __launch_bounds__(RA_THREADS, 1) void ring_attn_kernel(RaParams p) {
  __shared__ __attribute__((aligned(16))) char st0[RA_STAGE];
  __shared__ __attribute__((aligned(16))) char st1[RA_STAGE];
  __shared__ __attribute__((aligned(16))) char st2[RA_STAGE];
  __shared__ int s_claim;
  __shared__ int s_last;
  static_assert(RA_NW * RA_CP_IPB * 1024 == RA_STAGE && RA_CP_IPB % RA_INSTR == 0,
                "copy slots: RA_CP_IPB KiB per wave fill one stage buffer with whole units");
  const int wg = blockIdx.x;
  if (wg < p.n_copy) {
    trace_begin(p.trace, ROLE_COPY);
    ra_copy_role(p, wg, st0, st1);
    trace_mark(p.trace, 5);
    // every unit of this workgroup has been published (the copy ring raised each flag after its
    // stores completed): count the workgroup as landed
    if (threadIdx.x == 0) atomic_add_agent(p.counters + CTR_RA_LANDED, 1u);
    __syncthreads();  // the ring's LDS slots become stage buffers
    ra_compute_role(p, -1, st0, st1, st2, &s_claim);
  } else {
    trace_begin(p.trace, ROLE_COMPUTE);
    const int slot = wg - p.n_copy;
    if (slot < p.n_compute) ra_compute_role(p, slot, st0, st1, st2, &s_claim);
  }
  trace_end(p.trace);
  __syncthreads();
  if (threadIdx.x == 0) s_last = atomic_add_agent(p.counters + CTR_RA_EXIT, 1u) == gridDim.x - 1;
  __syncthreads();
  if (s_last && threadIdx.x == 0) {
    for (int xx = 0; xx < 8; ++xx)
      __hip_atomic_store(p.counters + CTR_RA_XITEM0 + xx, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(p.counters + CTR_RA_EXIT, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(p.counters + CTR_RA_LANDED, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

hipError_t launch_ring_attn(const RaParams& p, int grid, hipStream_t s) {
  hipLaunchKernelGGL(ring_attn_kernel, dim3(grid), dim3(RA_THREADS), 0, s, p);
  return hipGetLastError();
}

}  // namespace mk
