// MoE token dispatch + per-expert grouped GEMM, one rank's share, as one persistent launch.
//
// Operation (mKernel write-up, news.chathome.org page, five-fused-kernels table, MoE
// Dispatch + GEMM row): for each local expert e, y[seg e] = x_seg[seg e] @ w_up[e], where
// segment e of x_seg stacks the token rows whose top-k routing picked e.  The dispatch writes
// each routed row straight into its place in x_seg and the grouped GEMM reads it from there,
// in the same launch.  Here this rank owns experts [expert_begin, +n_local); the tokens of
// every rank are device buffers and their arrival is the copy role.
//
// Phases and roles (workgroup ids [0, n_copy) route and copy; the rest compute):
//   route   every route wave takes 64-token chunks: score = fp32(logit + bias) for every
//           expert, top-k by descending score with equal scores to the lower id (insertion
//           in ascending expert order, replacing only on a strictly larger score), writes
//           topk_idx and the chunk's row count per local expert.
//   scan    the last route workgroup to finish (arrival counter) turns the per-chunk counts
//           into segment offsets and per-(chunk, expert) first slots: an exclusive scan in
//           chunk order, i.e. ascending global token id inside each expert's segment.  It
//           also numbers the m-tiles of every segment, then raises the scan flag.
//   copy    after the scan flag, the routed rows in the caller's arrival order of chunks, split
//           evenly: copy workgroup cid takes rows [R cid / n_copy, R (cid + 1) / n_copy) of that
//           stream (the scan also lays out each arrival position's first row), a window of up to
//           eight chunks at a time: each wave lists one chunk's routed (token, slot) rows, then
//           all waves move the workgroup's part of them into their final slots of x_seg through
//           LDS, and once the window's rows are stored they are added to their m-tiles'
//           landed-row counters.  Once every copy workgroup has finished its dispatch, the copy
//           workgroups join the compute role on the tiles left over after every compute
//           workgroup's first one.
//   compute after the scan flag, (m-tile, n-tile) jobs of the ragged grouped GEMM: an m-tile
//           runs once all of its rows have landed; y[slot] = x_seg[slot] @ w_up[expert].
// Route/copy workgroups never wait on compute workgroups, and have the lowest ids.  The
// last workgroup to exit re-zeroes the counters, so every call starts from zero.
#include "mk_internal.h"
#include "mk_gemm_tile16.hpp"

namespace mk {

// 256 x 256 output tile on the 16 x 16 x 32 core: eight waves of 64 x 128, A two steps ahead in
// three 32 KiB LDS slots, B in two
using MoeTile = TileGemm16T<mk_tiles::kMoe.bn>;
static_assert(MoeTile::BM == mk_tiles::kMoe.bm && MoeTile::WM == mk_tiles::kMoe.wm && MoeTile::WN == mk_tiles::kMoe.wn,
              "kMoe is the 16 x 16 x 32 core");
constexpr int MOE_WAVES = MoeTile::NW;
constexpr int MOE_THREADS = MOE_WAVES * 64;
constexpr int MOE_KMAX = 8;     // top-k
constexpr int MOE_LMAX = 64;    // local experts
constexpr int MOE_LIST = 2048;  // (token, slot) rows listed per copy window

int moe_tile_m() { return MoeTile::BM; }
int moe_tile_n() { return MoeTile::BN; }

struct MoeShared {
  int n_rows[MOE_WAVES];                 // rows of each window chunk this workgroup moves
  int lo[MOE_WAVES];                     // first of them in the chunk's row list
  int p0, p1;                            // first and last arrival position of this workgroup's rows
  int pre[MOE_WAVES + 1];                // their prefix sums
  int chunk_first[MOE_WAVES][MOE_LMAX];  // first slot of each (window chunk, local expert)
  int chunk_cnt[MOE_WAVES][MOE_LMAX];    // rows of each (window chunk, local expert)
  int ok;
  int is_last;
  int claim;
  int seg_off[MOE_LMAX + 1];
  int tile_base[MOE_LMAX + 1];
  int totals[MOE_LMAX];
};

__device__ __forceinline__ uint32_t* moe_misc(const MoeParams& p) { return p.counters + p.off_misc; }

// Inclusive prefix sum over the 64 lanes of a wave: shifts by 1, 2, 4 and 8 lanes inside each row
// of 16, then row 0's last lane added to row 1 and row 2's to row 3, then lane 31 added to rows 2
// and 3 (DPP row shifts and row broadcasts: VALU instructions, where a lane shuffle would be a
// permute through the LDS unit).  Lanes whose source falls outside add 0.
__device__ __forceinline__ uint32_t wave_scan_incl(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true);   // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true);   // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, true);   // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, true);   // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15, rows 1, 3
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31, rows 2, 3
  return x;
}
// the sum over the wave's lanes, in every lane
__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_scan_incl(x), 63);
}
// misc layout: [0] route-done arrivals, [1] exits, [2 .. 2+n_local] m-tile base per expert (prefix),
// [MISC_TILE] next leftover GEMM tile, [MISC_DISP_DONE] copy workgroups done with their dispatch
constexpr int MISC_TILE = 101;
constexpr int MISC_DISP_DONE = 102;

// ------------------------------------------------------------------------------------------
// route (one wave per 64-token chunk)
// ------------------------------------------------------------------------------------------
template <int K>
__device__ __forceinline__ void moe_route_chunk(const MoeParams& p, int chunk, int lane) {
  float tv[K];
  int ti[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    tv[j] = 0.f;
    ti[j] = -1;
  }
  // One buffer window for the chunk's 64 logit rows (a per-lane window would be divergent and
  // turn every load into a loop over the lanes); lane l reads row l.  The bias is the same for
  // every lane and constant for the launch: scalar loads, a 64-expert block at a time.
  const auto lr = make_rsrc(p.logits + (size_t)chunk * 64 * p.n_experts, 64u * (uint32_t)p.n_experts * 4u);
  const uint32_t row_off = (uint32_t)lane * (uint32_t)p.n_experts * 4u;
  const __attribute__((address_space(4))) f32x4* bias4 = (const __attribute__((address_space(4))) f32x4*)p.bias;
  for (int e0 = 0; e0 < p.n_experts; e0 += 64) {
    const int nq = min(16, (p.n_experts - e0) >> 2);  // n_experts is a multiple of 4
    f32x4 lg[16], bs[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      lg[q] = __builtin_bit_cast(f32x4, bload16(lr, row_off + (uint32_t)(e0 + 4 * q) * 4u));
      bs[q] = q < nq ? bias4[(e0 >> 2) + q] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      if (q >= nq) continue;  // uniform; a break would keep the loop rolled and the arrays in memory
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        int id = e0 + 4 * q + r;
        float v = lg[q][r] + bs[q][r];  // one fp32 add, round to nearest even
        // insertion into the descending list: replace only on a strictly larger score (equal
        // scores keep the lower id, seen first); an empty slot (id -1) takes anything, and once
        // the carried candidate is an empty slot nothing further changes
#pragma unroll
        for (int j = 0; j < K; ++j) {
          const bool take = (id >= 0) && ((ti[j] < 0) || (v > tv[j]));
          const float fv = tv[j];
          const int fi = ti[j];
          tv[j] = take ? v : fv;
          ti[j] = take ? id : fi;
          v = take ? fv : v;
          id = take ? fi : id;
        }
      }
    }
  }
  const auto tr = make_rsrc(p.topk_idx + (size_t)chunk * 64 * K, 64u * K * 4u);
#pragma unroll
  for (int j = 0; j < K; ++j) bstore4_sc1(tr, ((uint32_t)lane * K + (uint32_t)j) * 4u, (uint32_t)ti[j]);
  // rows of this chunk per local expert: lane el stores expert el's count
  uint32_t mine = 0;
  for (int el = 0; el < p.n_local; ++el) {
    const int e = p.expert_begin + el;
    bool hit = false;
#pragma unroll
    for (int j = 0; j < K; ++j) hit |= (ti[j] == e);
    const uint32_t c = (uint32_t)__popcll(__ballot(hit));
    mine = lane == el ? c : mine;
  }
  const auto cr = make_rsrc(p.counters + p.off_chunk_cnt + (size_t)chunk * p.n_local, (uint32_t)p.n_local * 4u);
  bstore4_sc1(cr, (uint32_t)lane * 4u, mine);  // lanes past n_local fall outside the window
  const uint32_t tot = wave_sum(mine);
  const auto rr = make_rsrc(p.counters + p.off_chunk_rows + chunk, 4u);
  if (lane == 0) bstore4_sc1(rr, 0u, tot);
}

template <int K>
__device__ __forceinline__ void moe_route_all(const MoeParams& p, int first, int stride, int lane) {
  for (int c = first; c < p.n_chunks; c += stride) moe_route_chunk<K>(p, c, lane);
}

// Exclusive scan of the per-chunk counts (run by one workgroup, the last router).  Each wave
// owns local experts wave, wave + 8, ...; a group of 16 x 64 chunk counts is loaded at once.  When
// every wave owns at most one expert and the chunks fit one group (the usual case), the counts are
// loaded once and stay in registers from the totals to the per-chunk first slots, and the loads of
// the arrival-order pass (which does not depend on them) are issued first, so the whole scan waits
// on memory about twice instead of once per pass.
__device__ __forceinline__ void moe_scan(const MoeParams& p, MoeShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint32_t* cnt = p.counters + p.off_chunk_cnt;
  const auto cr = make_rsrc(cnt, (uint32_t)p.n_chunks * (uint32_t)p.n_local * 4u);
  auto load_group = [&](int el, int g0, uint32_t(&v)[16]) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t c = (uint32_t)(g0 + i * 64 + lane);
      v[i] = bload4_sc1(cr, (c * (uint32_t)p.n_local + (uint32_t)el) * 4u);  // past n_chunks: 0
    }
  };
  // rows of the chunk at arrival position i (pass 3's input)
  const auto rr = make_rsrc(p.counters + p.off_chunk_rows, (uint32_t)p.n_chunks * 4u);
  const int32_t* order = (p.emulated && p.order) ? p.order : nullptr;
  auto rows_at = [&](int i) -> uint32_t {
    if (i >= p.n_chunks) return 0u;
    const int c = order ? order[i] : i;
    return (c >= 0 && c < p.n_chunks) ? bload4_sc1(rr, (uint32_t)c * 4u) : 0u;
  };
  const bool one_pos = p.n_chunks <= MOE_THREADS;
  const uint32_t rows0 = one_pos ? rows_at(tid) : 0u;
  const bool in_regs = p.n_local <= MOE_WAVES && p.n_chunks <= 1024;
  uint32_t vr[16];
  // pass 1: per-expert totals
  if (in_regs) {
    if (wave < p.n_local) {
      load_group(wave, 0, vr);
      uint32_t s = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) s += vr[i];
      s = wave_sum(s);
      if (lane == 0) sh.totals[wave] = (int)s;
    }
  } else {
    for (int el = wave; el < p.n_local; el += MOE_WAVES) {
      uint32_t s = 0;
      for (int g0 = 0; g0 < p.n_chunks; g0 += 1024) {
        uint32_t v[16];
        load_group(el, g0, v);
#pragma unroll
        for (int i = 0; i < 16; ++i) s += v[i];
      }
      s = wave_sum(s);
      if (lane == 0) sh.totals[el] = (int)s;
    }
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
  auto scan_group = [&](int el, int g0, const uint32_t(&v)[16], uint32_t& run) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t inc = wave_scan_incl(v[i]);
      const uint32_t c = (uint32_t)(g0 + i * 64 + lane);
      bstore4_sc1(cr, (c * (uint32_t)p.n_local + (uint32_t)el) * 4u, run + inc - v[i]);  // past the end: dropped
      run += (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
    }
  };
  if (in_regs) {
    if (wave < p.n_local) {
      uint32_t run = (uint32_t)sh.seg_off[wave];
      scan_group(wave, 0, vr, run);
    }
  } else {
    for (int el = wave; el < p.n_local; el += MOE_WAVES) {
      uint32_t run = (uint32_t)sh.seg_off[el];
      for (int g0 = 0; g0 < p.n_chunks; g0 += 1024) {
        uint32_t v[16];
        load_group(el, g0, v);
        scan_group(el, g0, v, run);
      }
    }
  }
  const auto so = make_rsrc(p.seg_offsets, (uint32_t)(p.n_local + 1) * 4u);
  const auto tb = make_rsrc(moe_misc(p) + 2, (uint32_t)(p.n_local + 1) * 4u);
  for (int i = tid; i <= p.n_local; i += MOE_THREADS) {
    bstore4_sc1(so, (uint32_t)i * 4u, (uint32_t)sh.seg_off[i]);
    bstore4_sc1(tb, (uint32_t)i * 4u, (uint32_t)sh.tile_base[i]);
  }
  // pass 3: first row of every arrival position in the stream of routed rows in arrival order
  // (exclusive scan of the chunks' row totals taken in the caller's order), for the copy split
  {
    const auto pp = make_rsrc(p.counters + p.off_pos_pre, (uint32_t)(p.n_chunks + 1) * 4u);
    uint32_t carry = 0;
    for (int base = 0; base < p.n_chunks; base += MOE_THREADS) {
      const int i = base + tid;
      const uint32_t v = one_pos ? rows0 : rows_at(i);
      const uint32_t inc = wave_scan_incl(v);
      if (lane == 63) sh.pre[wave] = (int)inc;  // wave totals
      __syncthreads();
      uint32_t wpre = 0, btot = 0;
      for (int w = 0; w < MOE_WAVES; ++w) {
        const uint32_t t = (uint32_t)sh.pre[w];
        wpre += w < wave ? t : 0u;
        btot += t;
      }
      if (i < p.n_chunks) bstore4_sc1(pp, (uint32_t)i * 4u, carry + wpre + inc - v);
      carry += btot;
      __syncthreads();  // sh.pre is rewritten by the next group
    }
    if (tid == 0) bstore4_sc1(pp, (uint32_t)p.n_chunks * 4u, carry);
  }
  wait_mem();
  __syncthreads();
  if (tid == 0) flag_store(&p.flags[0], p.epoch);
}

// Segment offsets and m-tile bases of the scan, into LDS (every workgroup, after the scan flag).
__device__ __forceinline__ void moe_load_segments(const MoeParams& p, MoeShared& sh) {
  const auto so = make_rsrc(p.seg_offsets, (uint32_t)(p.n_local + 1) * 4u);
  const auto tb = make_rsrc(moe_misc(p) + 2, (uint32_t)(p.n_local + 1) * 4u);
  for (int i = threadIdx.x; i <= p.n_local; i += MOE_THREADS) {
    sh.seg_off[i] = (int)bload4_sc1(so, (uint32_t)i * 4u);
    sh.tile_base[i] = (int)bload4_sc1(tb, (uint32_t)i * 4u);
  }
}

// ------------------------------------------------------------------------------------------
// copy role
// ------------------------------------------------------------------------------------------
// One wave lists the rows of window chunk w (chunk id c): every (token, local expert) pair, in
// token order per expert, with slot = the expert's first slot for the chunk + rank; it also
// writes seg_token, and the per-expert first slots and counts go to sh.
__device__ __forceinline__ void moe_list_chunk(const MoeParams& p, MoeShared& sh, int2* list, int w, int c, int lane) {
  const int t = c * 64 + lane;
  int ti[MOE_KMAX];
  const auto tr = make_rsrc(p.topk_idx + (size_t)c * 64 * p.top_k, 64u * (uint32_t)p.top_k * 4u);
#pragma unroll
  for (int j = 0; j < MOE_KMAX; ++j)
    ti[j] = j < p.top_k ? (int)bload4_sc1(tr, ((uint32_t)lane * (uint32_t)p.top_k + (uint32_t)j) * 4u) : -1;
  const auto fr = make_rsrc(p.counters + p.off_chunk_cnt + (size_t)c * p.n_local, (uint32_t)p.n_local * 4u);
  const int first = (int)bload4_sc1(fr, (uint32_t)lane * 4u);  // lane el: first slot of expert el
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const auto st = make_rsrc(p.seg_token, (uint32_t)p.capacity * 4u);
  int n = 0;
  for (int el = 0; el < p.n_local; ++el) {
    const int e = p.expert_begin + el;
    bool hit = false;
#pragma unroll
    for (int j = 0; j < MOE_KMAX; ++j)
      if (j < p.top_k) hit |= (ti[j] == e);
    const uint64_t m = __ballot(hit);
    const int fe = __builtin_amdgcn_readlane(first, el);
    if (hit) {
      const int rk = __popcll(m & lt);
      list[n + rk] = make_int2(t, fe + rk);
      bstore4_sc1(st, (uint32_t)(fe + rk) * 4u, (uint32_t)t);  // slots past capacity fall outside
    }
    if (lane == 0) {
      sh.chunk_first[w][el] = fe;
      sh.chunk_cnt[w][el] = __popcll(m);
    }
    n += __popcll(m);
  }
  if (lane == 0) sh.n_rows[w] = n;
}

// Add the stored rows of window chunk j (its list entries [lo, lo + n_rows)) to their m-tiles'
// counters (wave 0; lane el: expert el).  The list holds the chunk's rows expert by expert, so
// expert el's rows are entries [cum, cum + cnt) with cum the rows of the experts before it.
__device__ __forceinline__ void moe_raise_chunk(const MoeParams& p, const MoeShared& sh, int j, int lane) {
  const int cnt = lane < p.n_local ? sh.chunk_cnt[j][lane] : 0;
  const int inc = (int)wave_scan_incl((uint32_t)cnt);
  const int cum = inc - cnt;
  const int a = max(sh.lo[j], cum), b = min(sh.lo[j] + sh.n_rows[j], cum + cnt);
  if (lane >= p.n_local || b <= a) return;
  const int first = sh.chunk_first[j][lane] + (a - cum);
  const int off_e = sh.seg_off[lane], tb = sh.tile_base[lane];
  int s = first;
  const int s_end = min(first + (b - a), p.capacity);
  while (s < s_end) {
    const int mt = (s - off_e) / MoeTile::BM;
    const int hi = min(s_end, off_e + (mt + 1) * MoeTile::BM);
    atomic_add_agent(p.counters + p.off_tile_cnt + tb + mt, (uint32_t)(hi - s));
    s = hi;
  }
}

// Rows move global -> LDS (DMA) -> VGPRs -> global through two 64 KiB ring slots, each made of two
// 32 KiB GEMM slots (waves 0-3 in the first, 4-7 in the second: s0 = lo0/hi0, s1 = lo1/hi1), as
// in the AllGather copy: batch b gives wave w the window rows (8b + w) * RPB + i, i < RPB, each
// IPR 1 KiB DMA instructions (RPB * IPR = 8 per wave and batch; lanes past a row's end fall
// outside its buffer window).  Per batch and wave: 8 DMA loads and 8 stores, completing in issue
// order, so batch b has landed at vmcnt <= 16 (8 for b = 0).  The window's chunks raise their
// m-tile counters after the last store: counter atomics inside the loop would come in a
// data-dependent number, and the compiler would then drain the whole pipeline before every LDS
// read.  An m-tile spans chunks from the whole token range, so under a random arrival order it
// completes near the end of the dispatch either way.
template <int IPR>
__device__ __forceinline__ void moe_copy_window(const MoeParams& p, const MoeShared& sh, const int2* list, int stride,
                                                int n_win, char* lo0, char* hi0, char* lo1, char* hi1) {
  constexpr int RPB = 8 / IPR;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  (void)tid;
  const int R = sh.pre[n_win];
  const int nb = (R + 8 * RPB - 1) / (8 * RPB);
  const uint32_t row_b = (uint32_t)p.hidden * 2u;
  // The lookups below are branch-free (selects, a fixed unrolled scan): a branch inside the copy
  // loop made the compiler drain every outstanding DMA (vmcnt(0)) before each batch's LDS reads,
  // as it could no longer tell that they read the other slot.
  auto row_at = [&](int r) -> int2 {  // list entry of window row r, or (-1, -1)
    int j = 0;
#pragma unroll
    for (int k = 1; k < MOE_WAVES; ++k) j += (k < n_win && sh.pre[k] <= r) ? 1 : 0;
    const int idx = min(j * stride + sh.lo[j] + (r - sh.pre[j]), MOE_LIST - 1);
    const int2 e = list[idx];
    return r < R ? e : make_int2(-1, -1);
  };
  auto src_of = [&](int t) {
    const int tt = t < 0 ? 0 : t;
    const int r = tt / p.t_local, i = tt - r * p.t_local;
    const uint16_t* row = p.tokens[r] + (size_t)i * p.hidden;
    return make_rsrc(t < 0 ? (const uint16_t*)p.x_seg : row, t < 0 ? 0u : row_b);
  };
  auto dst_of = [&](int slot) {
    const bool ok = slot >= 0 && slot < p.capacity;
    return make_rsrc(p.x_seg + (ok ? (size_t)slot * p.hidden : (size_t)0), ok ? row_b : 0u);
  };
  // this wave's 8 KiB of a ring slot
  char* const w0 = (wave < 4 ? lo0 : hi0) + (wave & 3) * 8192;
  char* const w1 = (wave < 4 ? lo1 : hi1) + (wave & 3) * 8192;
  auto dma = [&](int b, char* base) {
#pragma unroll
    for (int i = 0; i < RPB; ++i) {
      const int2 e = row_at((b * 8 + wave) * RPB + i);
      const auto src = src_of(__builtin_amdgcn_readfirstlane(e.x));
#pragma unroll
      for (int q = 0; q < IPR; ++q)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            src, (__attribute__((address_space(3))) void*)(base + (i * IPR + q) * 1024), 16,
            (uint32_t)(q * 64 + lane) * 16u, 0, 0, 0);
    }
  };
  auto store = [&](int b, const char* wbase) {
    const char* base = wbase + lane * 16;
#pragma unroll
    for (int i = 0; i < RPB; ++i) {
      const int2 e = row_at((b * 8 + wave) * RPB + i);
      const auto dst = dst_of(__builtin_amdgcn_readfirstlane(e.y));
#pragma unroll
      for (int q = 0; q < IPR; ++q)
        bstore16_sc1(dst, (uint32_t)(q * 64 + lane) * 16u,
                     *reinterpret_cast<const u32x4*>(base + (i * IPR + q) * 1024));
    }
  };
  auto step = [&](int b, char* slot) {
    if (b >= nb) return;
    if (b == 0) wait_vm<8>();
    else wait_vm<16>();
    barrier_only();  // no LDS data crosses waves; the barrier keeps the waves in step
    store(b, slot);
    dma(b + 2, slot);  // this wave's LDS reads of the slot completed with the stores above
  };
  if (nb > 0) {
    dma(0, w0);
    dma(1, w1);
    for (int b = 0; b < nb; b += 2) {
      step(b, w0);
      step(b + 1, w1);
    }
  }
  wait_vm<0>();
  __syncthreads();
  if (wave == 0)
    for (int j = 0; j < n_win; ++j) moe_raise_chunk(p, sh, j, lane);
  __syncthreads();  // the next window rewrites the lists and chunk tables
}

// Copy workgroup cid takes rows [R cid / n_copy, R (cid + 1) / n_copy) of the routed rows taken
// in the caller's arrival order of chunks (R of them), so every workgroup moves the same number of
// rows whatever the chunks' sizes: it finds the arrival positions holding its first and last row
// (the scan laid out each position's first row), and takes those positions in windows of as many
// chunks as the listing waves and the LDS row list hold: every listing wave lists one chunk,
// then all waves move the window's part of the rows.  With the default role split a workgroup's
// rows span a few chunks: one window, one listing round trip and one pipeline fill and drain.
template <int IPR>
__device__ __forceinline__ void moe_dispatch(const MoeParams& p, int cid, MoeShared& sh, int2* list, char* lo0,
                                             char* hi0, char* lo1, char* hi1) {
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int stride = 64 * min(p.top_k, p.n_local);  // room for a chunk's largest row count
  const int cw = max(1, min(MOE_WAVES, MOE_LIST / stride));
  const __attribute__((address_space(4))) int32_t* order = (const __attribute__((address_space(4))) int32_t*)p.order;
  const auto pp = make_rsrc(p.counters + p.off_pos_pre, (uint32_t)(p.n_chunks + 1) * 4u);
  const int total = (int)__builtin_amdgcn_readfirstlane(bload4_sc1(pp, (uint32_t)p.n_chunks * 4u));
  const int r0 = (int)((int64_t)total * cid / p.n_copy), r1 = (int)((int64_t)total * (cid + 1) / p.n_copy);
  if (r0 >= r1) return;
  // the positions holding rows r0 and r1 - 1: position i holds rows [pre[i], pre[i + 1])
  if (tid == 0) sh.p0 = sh.p1 = -1;
  __syncthreads();
  for (int base = 0; base < p.n_chunks; base += MOE_THREADS) {
    const int i = base + tid;
    if (i < p.n_chunks) {
      const int a = (int)bload4_sc1(pp, (uint32_t)i * 4u), b = (int)bload4_sc1(pp, (uint32_t)(i + 1) * 4u);
      if (a <= r0 && r0 < b) sh.p0 = i;
      if (a < r1 && r1 <= b) sh.p1 = i;
    }
  }
  __syncthreads();
  const int p0 = __builtin_amdgcn_readfirstlane(*(volatile int*)&sh.p0);
  const int p1 = __builtin_amdgcn_readfirstlane(*(volatile int*)&sh.p1);
  if (p0 < 0 || p1 < p0) return;  // cannot happen for a consistent prefix
  for (int w0 = p0; w0 <= p1; w0 += cw) {
    const int n_win = min(cw, p1 - w0 + 1);
    if (wave < n_win) {
      const int pos = w0 + wave;
      int c = (p.emulated && order) ? order[pos] : pos;
      if (pos + 1 == p.drop_pos || c < 0 || c >= p.n_chunks) c = -1;  // testing: a dropped chunk never lands
      const int pre = (int)bload4_sc1(pp, (uint32_t)pos * 4u), nxt = (int)bload4_sc1(pp, (uint32_t)(pos + 1) * 4u);
      const int lo = max(r0, pre) - pre, hi = min(r1, nxt) - pre;
      if (c >= 0 && hi > lo) {
        moe_list_chunk(p, sh, list + wave * stride, wave, c, lane);
      } else {
        for (int el = lane; el < p.n_local; el += 64) sh.chunk_cnt[wave][el] = 0;
      }
      if (lane == 0) {  // after the listing's own n_rows: this workgroup's part of the chunk
        sh.lo[wave] = lo;
        sh.n_rows[wave] = (c >= 0 && hi > lo) ? hi - lo : 0;
      }
    }
    __syncthreads();
    if (tid == 0) {
      sh.pre[0] = 0;
      for (int j = 0; j < n_win; ++j) sh.pre[j + 1] = sh.pre[j] + sh.n_rows[j];
    }
    __syncthreads();
    moe_copy_window<IPR>(p, sh, list, stride, n_win, lo0, hi0, lo1, hi1);  // ends with a barrier
  }
}

__device__ __forceinline__ void moe_copy_role(const MoeParams& p, int cid, MoeShared& sh, int2* list, char* lo0,
                                              char* hi0, char* lo1, char* hi1) {
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // route: chunks (wave * n_copy + cid) + i * (n_copy * 8), i.e. chunk c on workgroup c % n_copy:
  // the chunks spread over every copy workgroup, at most one routing wave per SIMD while there are
  // fewer than 4 n_copy chunks (the top-k insertion is VALU work)
  const int c0 = wave * p.n_copy + cid, cs = p.n_copy * MOE_WAVES;
  switch (p.top_k) {
    case 1: moe_route_all<1>(p, c0, cs, lane); break;
    case 2: moe_route_all<2>(p, c0, cs, lane); break;
    case 3: moe_route_all<3>(p, c0, cs, lane); break;
    case 4: moe_route_all<4>(p, c0, cs, lane); break;
    case 5: moe_route_all<5>(p, c0, cs, lane); break;
    case 6: moe_route_all<6>(p, c0, cs, lane); break;
    case 7: moe_route_all<7>(p, c0, cs, lane); break;
    default: moe_route_all<8>(p, c0, cs, lane); break;
  }
  wait_mem();
  __syncthreads();
  trace_mark(p.trace, 5);
  if (tid == 0) sh.is_last = atomic_add_agent(moe_misc(p) + 0, 1u) == (uint32_t)(p.n_copy - 1);
  __syncthreads();
  if (sh.is_last) moe_scan(p, sh);

  if (tid == 0) sh.ok = spin_until_eq(&p.flags[0], p.epoch, p.timeout_ticks, p.status);
  __syncthreads();
  if (!sh.ok) return;
  trace_mark(p.trace, 6);
  moe_load_segments(p, sh);
  __syncthreads();
  // DMA instructions per row and wave, rounded up to a power of two (8 for hidden 4096)
  const int cpr = p.hidden >> 3;  // 16-byte pieces per row
  if (cpr > 256) moe_dispatch<8>(p, cid, sh, list, lo0, hi0, lo1, hi1);
  else if (cpr > 128) moe_dispatch<4>(p, cid, sh, list, lo0, hi0, lo1, hi1);
  else if (cpr > 64) moe_dispatch<2>(p, cid, sh, list, lo0, hi0, lo1, hi1);
  else moe_dispatch<1>(p, cid, sh, list, lo0, hi0, lo1, hi1);
}

// ------------------------------------------------------------------------------------------
// compute role: ragged grouped GEMM
// ------------------------------------------------------------------------------------------
// Grouped-GEMM tiles: `first` (a compute workgroup's static tile, or -1), then leftover tiles
// n_compute, n_compute + 1, ... claimed from a shared counter by every workgroup that has finished
// its own work (compute workgroups after their static tile, copy workgroups after the dispatch);
// mark_first: trace the first tile's start.  The K loop runs over five LDS slots (a0..a2: A, b0, b1: B); sh lives in b1 (see
// moe_kernel), so only sh.claim and sh.ok are used here, between K loops, and the segment table
// is read once from global memory (the scan's output).
__device__ __forceinline__ void moe_gemm_tiles(const MoeParams& p, MoeShared& sh, int first, bool mark_first,
                                               char* a0, char* a1, char* a2, char* b0, char* b1) {
  using G = MoeTile;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  G g;
  const int wm = wave / G::WN, wn = wave % G::WN;
  const int nk = p.hidden >> 6;
  const uint32_t lda_b = (uint32_t)p.hidden * 2u, ldb_b = (uint32_t)p.ffn * 2u;
  g.init(wm, wn, wave, lane, lda_b, ldb_b);
  // lane i < n_local: segment end seg_off[i + 1] and m-tile base tile_base[i + 1] (entry 0 of both
  // is 0), written by the scan before its flag
  const auto so = make_rsrc(p.seg_offsets, (uint32_t)(p.n_local + 1) * 4u);
  const auto tb = make_rsrc(moe_misc(p) + 2, (uint32_t)(p.n_local + 1) * 4u);
  // the segment table is fixed for the launch: read once
  const bool in = lane < p.n_local;
  const int seg_n = in ? (int)bload4_sc1(so, (uint32_t)(lane + 1) * 4u) : 0;
  const int tb_n = in ? (int)bload4_sc1(tb, (uint32_t)(lane + 1) * 4u) : 0;
  const int n_mt = __builtin_amdgcn_readlane(tb_n, p.n_local - 1);
  const int n_tiles = n_mt * p.tiles_n;
  int t = first;
  bool traced = !mark_first;
  while (true) {
    if (t < 0) {
      __syncthreads();  // every thread has read the last claim
      if (tid == 0) sh.claim = p.n_compute + (int)atomic_add_agent(moe_misc(p) + MISC_TILE, 1u);
      __syncthreads();
      t = sh.claim;
    }
    if (t >= n_tiles) break;
    const int gm = t / p.tiles_n, tn = t - gm * p.tiles_n;
    t = -1;
    // expert of m-tile gm: the number of experts whose tiles all come before it
    const int el = (int)__popcll(__ballot(in && tb_n <= gm));
    const int seg0 = el == 0 ? 0 : __builtin_amdgcn_readlane(seg_n, el - 1);
    const int seg1 = __builtin_amdgcn_readlane(seg_n, el);
    const int tb0 = el == 0 ? 0 : __builtin_amdgcn_readlane(tb_n, el - 1);
    const int mt = gm - tb0;
    const int row0 = seg0 + mt * G::BM;
    int rows_valid = min(G::BM, seg1 - row0);
    rows_valid = min(rows_valid, p.capacity - row0);
    if (rows_valid <= 0) continue;
    const int n0 = tn * G::BN;
    const int cols_valid = min(G::BN, p.ffn - n0);
    // wait until every row of this m-tile has landed
    if (tid == 0)
      sh.ok = spin_until_ge(p.counters + p.off_tile_cnt + gm, (uint32_t)rows_valid, p.timeout_ticks, p.status);
    __syncthreads();
    if (!sh.ok) return;
    if (!traced) trace_mark(p.trace, 5);  // a compute workgroup's static tile is ready
    traced = true;
    const char* a_tile = reinterpret_cast<const char*>(p.x_seg + (size_t)row0 * p.hidden);
    const uint32_t a_tile_bytes = (uint32_t)rows_valid * lda_b;
    const char* b_col = reinterpret_cast<const char*>(p.w_up + (size_t)el * p.hidden * p.ffn + n0);
    const uint32_t b_col_bytes = ((uint32_t)p.hidden * (uint32_t)p.ffn - (uint32_t)n0) * 2u;
    auto dma_a = [&](int ks, char* dst) {
      const uint32_t ca = (uint32_t)ks * 128u;
      g.dma_a(a_tile + ca, a_tile_bytes - ca, lda_b, dst, wave);
    };
    auto dma_b = [&](int ks, char* dst) {
      const uint32_t rb = (uint32_t)ks * 64u * ldb_b;
      g.dma_b(b_col + rb, b_col_bytes - rb, dst, wave);
    };
    auto prologue = [&](char* pa0, char* pb0, char* pa1) {
      dma_a(0, pa0);
      dma_b(0, pb0);
      if (nk > 1) dma_a(1, pa1);
    };
    auto none = [](int, auto) {};
    g.zero();
    k_loop_a3b2(g, nk, a0, a1, a2, b0, b1, prologue, dma_a, dma_b, none, none, none, [] { return true; });
    g.epilogue(G::epi_buf(wave, a0, a1, a2), wm, wn, lane, [&](int row, int col, f32x4 v) {
      if (row < rows_valid && col < cols_valid)
        __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p.y + (size_t)(row0 + row) * p.ffn + (n0 + col)));
    });
    __syncthreads();  // the next tile's prologue reuses the LDS
  }
}

__device__ __forceinline__ void moe_compute_role(const MoeParams& p, int slot, char* a0, char* a1, char* a2, char* b0,
                                                 char* b1, MoeShared& sh) {
  const int tid = threadIdx.x;
  if (tid == 0) sh.ok = spin_until_eq(&p.flags[0], p.epoch, p.timeout_ticks, p.status);
  __syncthreads();
  if (!sh.ok) return;
  // XCD-aware static tile: workgroup w runs on XCD w % 8, consecutive tiles (same expert and
  // m-tile, so the same A rows) go to one XCD
  const int C = p.n_compute;
  const int rs = ((C & 7) == 0) ? (slot & 7) * (C >> 3) + (slot >> 3) : slot;
  moe_gemm_tiles(p, sh, rs, true, a0, a1, a2, b0, b1);
}

// The five GEMM slots fill the 160 KiB of LDS: the copy role's row list and the shared block sit in
// the last B slot, which only the K loop uses (copy workgroups finish the dispatch before their
// first tile; during a K loop no code touches sh).
constexpr int MOE_SH = MOE_LIST * (int)sizeof(int2);
static_assert(MOE_SH + (int)sizeof(MoeShared) <= MoeTile::SLOT_B, "row list and shared block fit one B slot");
static_assert(MOE_THREADS == 512, "ring slots: 8 waves x 8 KiB");

__global__ __launch_bounds__(MOE_THREADS, 1) void moe_kernel(MoeParams p) {
  // 256-byte aligned: the swizzled B reads XOR bits 5-7 of the address
  __shared__ __attribute__((aligned(256))) char a0[MoeTile::SLOT_A];
  __shared__ __attribute__((aligned(256))) char a1[MoeTile::SLOT_A];
  __shared__ __attribute__((aligned(256))) char a2[MoeTile::SLOT_A];
  __shared__ __attribute__((aligned(256))) char b0[MoeTile::SLOT_B];
  __shared__ __attribute__((aligned(256))) char b1[MoeTile::SLOT_B];
  int2* list = reinterpret_cast<int2*>(b1);
  MoeShared& sh = *reinterpret_cast<MoeShared*>(b1 + MOE_SH);
  const int wg = blockIdx.x;
  if (wg < p.n_copy) {
    trace_begin(p.trace, ROLE_COPY);
    moe_copy_role(p, wg, sh, list, a0, a1, a2, b0);  // ring slots: a0 + a1 and a2 + b0
    trace_mark(p.trace, 7);
    // Leftover GEMM tiles only once every copy workgroup has finished its dispatch: the m-tiles of
    // the smallest experts complete early, and K loops started on them beside the dispatch slowed
    // the dispatch of their XCDs' other copy workgroups (dispatch end 73 -> 61 us without them).
    // Copy workgroups wait only on each other's dispatch, which waits on nothing but the scan.
    if (sh.ok) {
      if (threadIdx.x == 0) {
        atomic_add_agent(moe_misc(p) + MISC_DISP_DONE, 1u);
        sh.ok = spin_until_ge(moe_misc(p) + MISC_DISP_DONE, (uint32_t)p.n_copy, p.timeout_ticks, p.status);
      }
      __syncthreads();
    }
    if (sh.ok) moe_gemm_tiles(p, sh, -1, false, a0, a1, a2, b0, b1);  // then help with leftover tiles
  } else {
    trace_begin(p.trace, ROLE_COMPUTE);
    if (wg - p.n_copy < p.n_compute) moe_compute_role(p, wg - p.n_copy, a0, a1, a2, b0, b1, sh);
  }
  trace_end(p.trace);
  // exit accounting: the last workgroup out re-zeroes the counters for the next call
  wait_mem();
  __syncthreads();
  if (threadIdx.x == 0) sh.is_last = atomic_add_agent(moe_misc(p) + 1, 1u) == (uint32_t)(gridDim.x - 1);
  __syncthreads();
  if (sh.is_last) {
    // Every counter this call wrote goes back to zero, not only the ones it needs zeroed itself:
    // the per-chunk tables and m-tile counters share the context counters with other operations
    // (the RS band counters, the MLP row-block counters), which start from zero.  The tables are
    // contiguous, from the per-chunk counts to the end of the arrival-position prefix.
    const int end = p.off_pos_pre + p.n_chunks + 1;
    for (int i = p.off_chunk_cnt + threadIdx.x; i < end; i += MOE_THREADS)
      __hip_atomic_store(p.counters + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // misc: route-done, exits, the m-tile base per expert, the leftover-tile claim
    for (int i = threadIdx.x; i < 2 + p.n_local + 1; i += MOE_THREADS)
      __hip_atomic_store(moe_misc(p) + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (threadIdx.x == 0) __hip_atomic_store(moe_misc(p) + MISC_TILE, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (threadIdx.x == 0) __hip_atomic_store(moe_misc(p) + MISC_DISP_DONE, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

hipError_t launch_moe(const MoeParams& p, int grid, hipStream_t s) {
  hipLaunchKernelGGL(moe_kernel, dim3(grid), dim3(MOE_THREADS), 0, s, p);
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
