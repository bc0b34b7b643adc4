// Host-side planning for the C ABI: argument validation, arrival-unit geometry, role split
// and workspace layout.  Pure C++ with no HIP dependency, so the same code is compiled into
// the GPU library and into a host-only check library that runs on machines without a GPU.
#pragma once
#include <stddef.h>
#include <stdint.h>
#include <string.h>
#include <math.h>

#ifndef MK_OK
#define MK_OK 0
#define MK_ERR_INVALID_ARG (-1)
#define MK_ERR_UNSUPPORTED (-2)
#define MK_ERR_WORKSPACE (-3)
#define MK_ERR_HIP (-4)
#define MK_ERR_TIMEOUT (-5)
#define MK_ERR_CAPACITY (-6)
#define MK_ARRIVAL_RESIDENT 1
#define MK_ARRIVAL_EMULATED 2
#endif

namespace mkh {

constexpr int kMaxWorld = 8;
constexpr uint64_t k4G = 1ull << 32;
constexpr int kCtrBand0 = 128;  // first RS band counter in the context counters (CTR_RED_BAND0)
constexpr int kCtrHready0 = 4096;  // first MLP row-block counter of H (CTR_MLP_HREADY0)

struct Opts {  // mk_opts with defaults applied by the caller's struct (0 = default)
  int n_copy_wg, n_compute_wg, n_reduce_wg, arrival_mode;
  const void* arrival_order;
  int arrival_len, arrival_unit_rows, arrival_unit_cols, arrival_chunk_tokens;
  int64_t timeout_us;
  int test_drop_unit;
  double arrival_gbps;
};

struct Ws {  // workspace capacities of a context
  size_t n_flags, n_counters, inbox_bytes;
  int grid;  // co-resident workgroups of the persistent launch
};

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline bool mult64(int v) { return v > 0 && (v & 63) == 0; }

// Role split: copy workgroups first (a multiple of 8 so they spread over the 8 XCDs), then
// reduce, then compute.  Requested counts are clamped so at least 8 compute workgroups remain.
inline int split_roles(int grid, int want_copy, int want_reduce, int want_compute, int* n_copy, int* n_reduce,
                       int* n_compute) {
  if (want_copy < 0 || want_reduce < 0 || want_compute < 0) return MK_ERR_INVALID_ARG;
  if (want_copy + want_reduce + 8 > grid) return MK_ERR_UNSUPPORTED;
  *n_copy = want_copy;
  *n_reduce = want_reduce;
  int rest = grid - want_copy - want_reduce;
  *n_compute = (want_compute > 0 && want_compute < rest) ? want_compute : rest;
  return MK_OK;
}

// A compute role larger than the tile count leaves workgroups idle; with the XCD-contiguous tile
// order those idle slots would all fall on the last XCDs.  Unless a count was requested, keep just
// enough compute workgroups for one tile each, rounded up to whole XCD rounds.
inline int fit_compute(int n_compute, int tiles, const Opts* o) {
  if (o && o->n_compute_wg > 0) return n_compute;
  const int need = (tiles + 7) & ~7;
  return need < n_compute ? need : n_compute;
}

// ---- AllGather + GEMM ---------------------------------------------------------------------
struct AgPlan {
  int m, unit_rows, unit_cols, n_urows, n_ucols, n_order, local_in_place, emulated, drop_pos;
  int n_copy, n_compute, tiles_m, tiles_n;
  uint64_t pace_q16;  // link-rate pacing: wall-clock ticks per arrival position, Q16 (0: unpaced)
};

// Link-rate pacing of a copy role (mk_opts.arrival_gbps): arrival position i is not copied before
// i * unit_bytes / rate after the copy workgroup starts.  The device wall clock runs at 100 MHz,
// so a position takes unit_bytes / (gbps * 1e9) * 1e8 ticks, kept in Q16 fixed point.  The whole
// order must land well inside the watchdog, or a consumer would time out waiting for it.
inline int plan_pace(const Opts* o, bool emulated, int n_order, long unit_bytes, uint64_t* pace_q16) {
  *pace_q16 = 0;
  const double g = o ? o->arrival_gbps : 0.0;
  if (g == 0.0) return MK_OK;
  if (!(g > 0.0) || !(g < 1e9)) return MK_ERR_INVALID_ARG;  // negative, NaN or infinite
  if (!emulated || n_order == 0) return MK_OK;                // nothing arrives
  const double ticks = (double)unit_bytes / (g * 1e9) * 1e8;
  const int64_t timeout_us = (o->timeout_us > 0) ? o->timeout_us : 2000000;
  if (ticks * n_order / 100.0 > 0.5 * (double)timeout_us) return MK_ERR_INVALID_ARG;
  *pace_q16 = (uint64_t)(ticks * 65536.0 + 0.5);
  return MK_OK;
}

inline int plan_ag(const Ws& ws, const Opts* o, const void* const* a_shards, int world, int rank, int m_shard, int k,
                   const void* b, int n, const void* a_gathered, const void* c, int tile_m, int tile_n, AgPlan* P) {
  if (!b || !a_gathered || !c) return MK_ERR_INVALID_ARG;
  if (world < 1 || world > kMaxWorld || rank < 0 || rank >= world) return MK_ERR_INVALID_ARG;
  if (m_shard <= 0 || k <= 0 || n <= 0) return MK_ERR_INVALID_ARG;
  const int mode = (o && o->arrival_mode) ? o->arrival_mode : MK_ARRIVAL_EMULATED;
  if (mode != MK_ARRIVAL_RESIDENT && mode != MK_ARRIVAL_EMULATED) return MK_ERR_INVALID_ARG;
  if (!mult64(m_shard) || !mult64(k) || !mult64(n)) return MK_ERR_UNSUPPORTED;
  if (!aligned16(b) || !aligned16(a_gathered) || !aligned16(c)) return MK_ERR_UNSUPPORTED;
  const uint64_t m = (uint64_t)world * (uint64_t)m_shard;
  if (m * (uint64_t)k * 2 >= k4G || (uint64_t)k * n * 2 >= k4G || m * (uint64_t)n * 4 >= k4G) return MK_ERR_UNSUPPORTED;
  int ur = o && o->arrival_unit_rows ? o->arrival_unit_rows : ((m_shard % 128 == 0 && k % 128 == 0) ? 128 : 64);
  int uc = o && o->arrival_unit_cols ? o->arrival_unit_cols : ((m_shard % 128 == 0 && k % 128 == 0) ? 128 : 64);
  if ((ur != 64 && ur != 128) || (uc != 64 && uc != 128)) return MK_ERR_UNSUPPORTED;
  if (m_shard % ur || k % uc) return MK_ERR_UNSUPPORTED;
  if (k / uc > 64) return MK_ERR_UNSUPPORTED;  // K-unit masks are 64 bits wide
  if (tile_m % ur) return MK_ERR_UNSUPPORTED;
  P->m = (int)m;
  P->unit_rows = ur;
  P->unit_cols = uc;
  P->n_urows = (int)(m / ur);
  P->n_ucols = k / uc;
  P->emulated = mode == MK_ARRIVAL_EMULATED;
  P->tiles_m = (int)((m + tile_m - 1) / tile_m);
  P->tiles_n = (n + tile_n - 1) / tile_n;
  if ((size_t)P->n_urows * (size_t)P->n_ucols > ws.n_flags) return MK_ERR_WORKSPACE;
  const void* own_rows = (const char*)a_gathered + (size_t)rank * m_shard * k * 2;
  P->local_in_place = 1;
  P->n_order = 0;
  P->drop_pos = 0;
  if (P->emulated) {
    if (!a_shards) return MK_ERR_INVALID_ARG;
    for (int r = 0; r < world; ++r) {
      if (r == rank && (a_shards[r] == nullptr || a_shards[r] == own_rows)) continue;
      if (!a_shards[r]) return MK_ERR_INVALID_ARG;
      if (!aligned16(a_shards[r])) return MK_ERR_UNSUPPORTED;
    }
    P->local_in_place = (a_shards[rank] == nullptr || a_shards[rank] == own_rows) ? 1 : 0;
    const int spr = m_shard / ur;
    P->n_order = (world - P->local_in_place) * spr * P->n_ucols;
    if (o && o->arrival_order && o->arrival_len != P->n_order) return MK_ERR_INVALID_ARG;
    if (o && o->arrival_order && !aligned16(o->arrival_order) && ((uintptr_t)o->arrival_order & 3u)) return MK_ERR_UNSUPPORTED;
    P->drop_pos = (o && o->test_drop_unit > 0) ? o->test_drop_unit : 0;
  }
  // Default role split.  Every workgroup owns one tile and the copy workgroups start theirs once
  // they have copied.  Unpaced, the compute workgroups are as many as the tiles whose rows are the
  // local shard (rounded up to whole XCD rounds): they take those tiles and start at once, and every
  // other workgroup copies, so the shards land as soon as the HBM allows.  Paced at a link rate, 160
  // copy workgroups (the tuner finds the best split per shape).
  int want_copy = 0;
  if (P->emulated) {
    if (o && o->n_copy_wg) {
      want_copy = o->n_copy_wg;
    } else if (o && o->arrival_gbps > 0.0) {
      want_copy = 160;
    } else {
      long lt0 = 0, lt1 = 0;
      if (P->local_in_place) {
        lt0 = ((long)rank * m_shard + tile_m - 1) / tile_m;
        lt1 = ((long)rank * m_shard + m_shard) / tile_m;
        if (lt1 < lt0) lt1 = lt0;
      }
      long nc = ((lt1 - lt0) * P->tiles_n + 7) & ~7L;
      if (nc < 8) nc = 8;
      want_copy = ws.grid - nc >= 8 ? (int)(ws.grid - nc) : 8;
    }
  }
  if (P->emulated && P->n_order > 0 && want_copy == 0) return MK_ERR_INVALID_ARG;
  int nr = 0;
  int code = split_roles(ws.grid, P->emulated ? want_copy : 0, 0, o ? o->n_compute_wg : 0, &P->n_copy, &nr, &P->n_compute);
  if (code != MK_OK) return code;
  if (P->emulated && P->n_order == 0) P->n_copy = 0;
  P->n_compute = fit_compute(P->n_compute, P->tiles_m * P->tiles_n, o);
  return plan_pace(o, P->emulated, P->n_order, (long)ur * uc * 2, &P->pace_q16);
}

// ---- GEMM + ReduceScatter / AllReduce -----------------------------------------------------------
struct RedPlan {
  int m_slice, p_rows, unit_rows, unit_cols, n_ucols, units_per_peer, n_units, emulated, n_order, drop_pos;
  int n_copy, n_reduce, n_compute, tiles_m, tiles_n, own_tile_begin, own_tile_end;
  int assist;  // RS with peers and no reduce workgroups: compute workgroups pre-sum owned tiles
  size_t inbox_need;
  uint64_t pace_q16;  // link-rate pacing, as AgPlan::pace_q16
};

inline int plan_reduce(const Ws& ws, const Opts* o, int is_rs, const void* a, const void* b, int m, int n, int k,
                       int world, int rank, const void* const* peers, const void* out, void* const* outbox,
                       int tile_m, int tile_n, int tile_waves, int ring_kib, RedPlan* P) {
  if (!a || !b || !out) return MK_ERR_INVALID_ARG;
  if (world < 1 || world > kMaxWorld || rank < 0 || rank >= world) return MK_ERR_INVALID_ARG;
  if (m <= 0 || n <= 0 || k <= 0) return MK_ERR_INVALID_ARG;
  if (is_rs && (m % world)) return MK_ERR_INVALID_ARG;
  const int mode = (o && o->arrival_mode) ? o->arrival_mode : MK_ARRIVAL_EMULATED;
  if (mode != MK_ARRIVAL_RESIDENT && mode != MK_ARRIVAL_EMULATED) return MK_ERR_INVALID_ARG;
  if (world > 1 && !peers) return MK_ERR_INVALID_ARG;
  if (is_rs && world > 1 && !outbox) return MK_ERR_INVALID_ARG;
  for (int j = 0; j < world; ++j) {
    if (j == rank) continue;
    if (!peers[j]) return MK_ERR_INVALID_ARG;
    if (is_rs && !outbox[j]) return MK_ERR_INVALID_ARG;
  }
  if (!mult64(m) || !mult64(n) || !mult64(k)) return MK_ERR_UNSUPPORTED;
  P->m_slice = is_rs ? m / world : m;
  if (is_rs && !mult64(P->m_slice)) return MK_ERR_UNSUPPORTED;
  if (!aligned16(a) || !aligned16(b) || !aligned16(out)) return MK_ERR_UNSUPPORTED;
  for (int j = 0; j < world; ++j) {
    if (j == rank) continue;
    if (!aligned16(peers[j])) return MK_ERR_UNSUPPORTED;
    if (is_rs && !aligned16(outbox[j])) return MK_ERR_UNSUPPORTED;
  }
  if ((uint64_t)m * k * 2 >= k4G || (uint64_t)k * n * 2 >= k4G || (uint64_t)m * n * 4 >= k4G) return MK_ERR_UNSUPPORTED;
  P->p_rows = is_rs ? P->m_slice : m;
  // The copy ring moves at most ring_kib KiB of a unit per wave and batch: the largest unit that
  // fits the kernel's ring and divides the partial.
  if (tile_waves <= 0 || ring_kib <= 0) return MK_ERR_INVALID_ARG;
  const long max_unit = 1024L * ring_kib * tile_waves;
  int ur_d = 64, uc_d = 64;
  if (P->p_rows % 128 == 0 && n % 128 == 0 && 128 * 128 * 4 <= max_unit) ur_d = uc_d = 128;
  else if (n % 128 == 0 && 64 * 128 * 4 <= max_unit) uc_d = 128;
  int ur = o && o->arrival_unit_rows ? o->arrival_unit_rows : ur_d;
  int uc = o && o->arrival_unit_cols ? o->arrival_unit_cols : uc_d;
  if ((ur != 64 && ur != 128) || (uc != 64 && uc != 128)) return MK_ERR_UNSUPPORTED;
  if ((long)ur * uc * 4 > max_unit) return MK_ERR_UNSUPPORTED;
  if (P->p_rows % ur || n % uc) return MK_ERR_UNSUPPORTED;
  P->unit_rows = ur;
  P->unit_cols = uc;
  P->n_ucols = n / uc;
  P->units_per_peer = (P->p_rows / ur) * P->n_ucols;
  P->n_units = (world - 1) * P->units_per_peer;
  P->emulated = (mode == MK_ARRIVAL_EMULATED) && world > 1;
  P->tiles_m = (m + tile_m - 1) / tile_m;
  P->tiles_n = (n + tile_n - 1) / tile_n;
  if (is_rs) {
    const int o0 = rank * P->m_slice, o1 = o0 + P->m_slice;
    P->own_tile_begin = o0 / tile_m;
    P->own_tile_end = (o1 + tile_m - 1) / tile_m;
  } else {
    P->own_tile_begin = 0;
    P->own_tile_end = P->tiles_m;
  }
  P->n_order = P->emulated ? P->n_units : 0;
  P->drop_pos = (P->emulated && o && o->test_drop_unit > 0) ? o->test_drop_unit : 0;
  P->inbox_need = P->emulated ? (size_t)(world - 1) * P->p_rows * (size_t)n * 4 : 0;
  if (P->inbox_need > ws.inbox_bytes) return MK_ERR_WORKSPACE;
  if ((size_t)P->n_units + (size_t)P->tiles_m * P->tiles_n > ws.n_flags) return MK_ERR_WORKSPACE;
  if (P->emulated && o && o->arrival_order && o->arrival_len != P->n_order) return MK_ERR_INVALID_ARG;
  // copy workgroups join the compute role on leftover tiles once their units have landed, so by
  // default 7/8 of the workgroups not asked to reduce land units (a multiple of 8; measured:
  // landing ends sooner and the leftover tiles spread over more workgroups)
  const int want_reduce = (world > 1 && o) ? o->n_reduce_wg : 0;
  const int copy_q = ((ws.grid - want_reduce) * 7 / 8) & ~7;
  const int copy_d = copy_q > 8 ? copy_q : 8;
  const int want_copy = P->emulated ? ((o && o->n_copy_wg) ? o->n_copy_wg : copy_d) : 0;
  int code = split_roles(ws.grid, want_copy, want_reduce, o ? o->n_compute_wg : 0, &P->n_copy, &P->n_reduce,
                         &P->n_compute);
  if (code != MK_OK) return code;
  if (world == 1) P->n_reduce = 0;
  // Without reduce workgroups, RS compute workgroups pre-sum the owned tiles' peer partials in
  // 64-row bands between their tiles, one band counter per owned tile after the fixed counters.
  P->assist = (is_rs && world > 1 && P->n_reduce == 0) ? 1 : 0;
  const size_t n_own = (size_t)(P->own_tile_end - P->own_tile_begin) * P->tiles_n;
  if (P->assist && kCtrBand0 + n_own > ws.n_counters) return MK_ERR_WORKSPACE;
  return plan_pace(o, P->emulated, P->n_order, (long)ur * uc * 4, &P->pace_q16);
}

// ---- MLP block: AllGather + up-projection, gelu, down-projection + ReduceScatter ----------------
// The first phase is planned as mk_ag_gemm over [world*m_shard, k] @ [k, n_up] (its arrival mode,
// units and role split as given), the second as a resident mk_gemm_rs over H [world*m_shard, n_up]
// @ [n_up, n_out] on every workgroup; both use 256-row tiles, so a tile row of the second phase is
// one row block of H.
struct MlpPlan {
  AgPlan ag;
  RedPlan red;
};

inline int plan_mlp(const Ws& ws, const Opts* o, const void* const* a_shards, int world, int rank, int m_shard, int k,
                    const void* b_up, int n_up, const void* b_down, int n_out, const void* const* peers,
                    const void* a_gathered, const void* h, const void* out, void* const* outbox, int ag_tile_m,
                    int ag_tile_n, int red_tile_m, int red_tile_n, int red_tile_waves, MlpPlan* P) {
  if (!h || !b_down) return MK_ERR_INVALID_ARG;
  int code = plan_ag(ws, o, a_shards, world, rank, m_shard, k, b_up, n_up, a_gathered, h, ag_tile_m, ag_tile_n, &P->ag);
  if (code != MK_OK) return code;
  // workgroups beyond the up-projection's roles go straight to the down-projection
  if (P->ag.n_copy + P->ag.n_compute > ws.grid) return MK_ERR_UNSUPPORTED;
  Opts r;
  memset(&r, 0, sizeof(r));
  r.arrival_mode = MK_ARRIVAL_RESIDENT;  // the peers' partials of the down-projection are resident
  r.timeout_us = o ? o->timeout_us : 0;
  // (resident: no unit moves, so the ring size only bounds unit sizes nobody asked for)
  code = plan_reduce(ws, &r, 1, h, b_down, world * m_shard, n_out, n_up, world, rank, peers, out, outbox, red_tile_m,
                     red_tile_n, red_tile_waves, 8, &P->red);
  if (code != MK_OK) return code;
  if (red_tile_m != ag_tile_m || red_tile_waves * 64 != 512) return MK_ERR_UNSUPPORTED;  // one H block per tile row
  if (P->red.n_copy || P->red.n_reduce || P->red.n_compute != ws.grid) return MK_ERR_UNSUPPORTED;
  const size_t n_own = (size_t)(P->red.own_tile_end - P->red.own_tile_begin) * P->red.tiles_n;
  if (kCtrBand0 + n_own > (size_t)kCtrHready0 || kCtrHready0 + (size_t)P->ag.tiles_m > ws.n_counters)
    return MK_ERR_WORKSPACE;
  return MK_OK;
}

// ---- Ring attention -----------------------------------------------------------------------------
// Items are (head, 128-query tile); K/V move in 64-key blocks of 16 KiB, one flag each for K and V
// of every (rank, head, block).  Only head dimension 128 is implemented.
struct RaPlan {
  int n_blk, n_qt, n_items, n_units, emulated, n_order, drop_pos, n_copy, n_compute;
  float scale;
  uint64_t pace_q16;
};

constexpr int kRaHeadDim = 128;

inline int plan_ring_attn(const Ws& ws, const Opts* o, const void* q, const void* const* k_shards,
                          const void* const* v_shards, int world, int rank, int heads, int s_local, int head_dim,
                          float scale, const void* k_ring, const void* v_ring, const void* out, const void* lse,
                          RaPlan* P) {
  if (!q || !k_shards || !v_shards || !out) return MK_ERR_INVALID_ARG;
  if (world < 1 || world > kMaxWorld || rank < 0 || rank >= world) return MK_ERR_INVALID_ARG;
  if (heads <= 0 || s_local <= 0 || head_dim <= 0) return MK_ERR_INVALID_ARG;
  if (!(scale >= 0.f) || !(scale < 3.0e38f)) return MK_ERR_INVALID_ARG;  // negative, NaN or infinite
  const int mode = (o && o->arrival_mode) ? o->arrival_mode : MK_ARRIVAL_EMULATED;
  if (mode != MK_ARRIVAL_RESIDENT && mode != MK_ARRIVAL_EMULATED) return MK_ERR_INVALID_ARG;
  for (int r = 0; r < world; ++r)
    if (!k_shards[r] || !v_shards[r]) return MK_ERR_INVALID_ARG;
  if (head_dim != kRaHeadDim || s_local % 128) return MK_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(out) || ((uintptr_t)lse & 3u)) return MK_ERR_UNSUPPORTED;
  for (int r = 0; r < world; ++r)
    if (!aligned16(k_shards[r]) || !aligned16(v_shards[r])) return MK_ERR_UNSUPPORTED;
  const uint64_t shard = (uint64_t)heads * (uint64_t)s_local * head_dim * 2;
  if (shard * (uint64_t)world >= k4G) return MK_ERR_UNSUPPORTED;
  P->scale = scale > 0.f ? scale : 1.f / sqrtf((float)head_dim);
  P->n_blk = s_local / 64;
  P->n_qt = s_local / 128;
  P->n_items = heads * P->n_qt;
  P->n_units = world * heads * P->n_blk * 2;
  P->emulated = mode == MK_ARRIVAL_EMULATED && world > 1;
  if ((size_t)P->n_units > ws.n_flags) return MK_ERR_WORKSPACE;
  P->n_order = 0;
  P->drop_pos = 0;
  if (P->emulated) {
    if (!k_ring || !v_ring) return MK_ERR_INVALID_ARG;
    if (!aligned16(k_ring) || !aligned16(v_ring)) return MK_ERR_UNSUPPORTED;
    P->n_order = (world - 1) * heads * P->n_blk * 2;
    if (o && o->arrival_order && o->arrival_len != P->n_order) return MK_ERR_INVALID_ARG;
    if (o && o->arrival_order && ((uintptr_t)o->arrival_order & 3u)) return MK_ERR_UNSUPPORTED;
    P->drop_pos = (o && o->test_drop_unit > 0) ? o->test_drop_unit : 0;
  }
  // The ring moves world-1 shards of K and V (117 MB at 8 ranks x 8 heads x 4096 keys).  Copy
  // workgroups land it and then take the items left over past the compute workgroups; a CU copies
  // fresh HBM data at only a few tens of GB/s, so many copy workgroups land it soonest and start
  // their items earliest: 192 measured best (1.048 ms against 1.173 ms with 32 at the full
  // workload; 128 and 248 within 1 %).
  const int want_copy = P->emulated ? ((o && o->n_copy_wg) ? o->n_copy_wg : 192) : 0;
  int nr = 0;
  int code = split_roles(ws.grid, want_copy, 0, o ? o->n_compute_wg : 0, &P->n_copy, &nr, &P->n_compute);
  if (code != MK_OK) return code;
  P->n_compute = fit_compute(P->n_compute, P->n_items, o);
  return plan_pace(o, P->emulated, P->n_order, 64L * head_dim * 2, &P->pace_q16);
}

// ---- MoE dispatch + grouped GEMM ----------------------------------------------------------------
struct MoePlan {
  int n_tokens, n_chunks, emulated, drop_pos, n_copy, n_compute, tiles_n, max_mtiles;
  int off_misc, off_chunk_cnt, off_tile_cnt, off_chunk_rows, off_pos_pre;
  size_t counters_need;
};

inline int plan_moe(const Ws& ws, const Opts* o, const void* const* tokens, int world, int t_local, int hidden,
                    const void* logits, const void* bias, int n_experts, int top_k, int expert_begin, int n_local,
                    const void* w_up, int ffn, const void* topk_idx, const void* seg_offsets, const void* seg_token,
                    const void* x_seg, const void* y, int capacity, int tile_m, int tile_n, MoePlan* P) {
  if (!tokens || !logits || !bias || !w_up || !topk_idx || !seg_offsets) return MK_ERR_INVALID_ARG;
  if (world < 1 || world > kMaxWorld || t_local <= 0 || hidden <= 0 || ffn <= 0) return MK_ERR_INVALID_ARG;
  if (n_experts <= 0 || top_k <= 0 || top_k > n_experts) return MK_ERR_INVALID_ARG;
  if (n_local <= 0 || expert_begin < 0 || expert_begin + n_local > n_experts) return MK_ERR_INVALID_ARG;
  if (capacity < 0) return MK_ERR_INVALID_ARG;
  if (capacity > 0 && (!seg_token || !x_seg || !y)) return MK_ERR_INVALID_ARG;
  for (int r = 0; r < world; ++r)
    if (!tokens[r]) return MK_ERR_INVALID_ARG;
  const int mode = (o && o->arrival_mode) ? o->arrival_mode : MK_ARRIVAL_EMULATED;
  if (mode != MK_ARRIVAL_RESIDENT && mode != MK_ARRIVAL_EMULATED) return MK_ERR_INVALID_ARG;
  if (top_k > 8 || n_experts > 1024 || (n_experts & 3) || n_local > 64) return MK_ERR_UNSUPPORTED;
  if (hidden > 4096) return MK_ERR_UNSUPPORTED;  // the dispatch copy moves at most 8 KiB per token row
  if (!mult64(t_local) || !mult64(hidden) || !mult64(ffn)) return MK_ERR_UNSUPPORTED;
  if (o && o->arrival_chunk_tokens && o->arrival_chunk_tokens != 64) return MK_ERR_UNSUPPORTED;
  if (!aligned16(logits) || !aligned16(bias) || !aligned16(w_up) || ((uintptr_t)topk_idx & 3u) ||
      ((uintptr_t)seg_offsets & 3u))
    return MK_ERR_UNSUPPORTED;
  if (capacity > 0 && (!aligned16(x_seg) || !aligned16(y) || ((uintptr_t)seg_token & 3u))) return MK_ERR_UNSUPPORTED;
  for (int r = 0; r < world; ++r)
    if (!aligned16(tokens[r])) return MK_ERR_UNSUPPORTED;
  const uint64_t T = (uint64_t)world * t_local;
  if ((uint64_t)t_local * hidden * 2 >= k4G || T * n_experts * 4 >= k4G || (uint64_t)capacity * hidden * 2 >= k4G ||
      (uint64_t)capacity * ffn * 4 >= k4G || (uint64_t)n_local * hidden * ffn * 2 >= k4G || T * top_k * 4 >= k4G)
    return MK_ERR_UNSUPPORTED;
  P->n_tokens = (int)T;
  P->n_chunks = (int)(T / 64);
  P->emulated = mode == MK_ARRIVAL_EMULATED;
  if (P->emulated && o && o->arrival_order && o->arrival_len != P->n_chunks) return MK_ERR_INVALID_ARG;
  P->drop_pos = (P->emulated && o && o->test_drop_unit > 0) ? o->test_drop_unit : 0;
  P->tiles_n = (ffn + tile_n - 1) / tile_n;
  P->max_mtiles = capacity / tile_m + n_local + 1;
  P->off_misc = 0;
  P->off_chunk_cnt = 128;
  P->off_tile_cnt = P->off_chunk_cnt + P->n_chunks * n_local;
  P->off_chunk_rows = P->off_tile_cnt + P->max_mtiles;
  P->off_pos_pre = P->off_chunk_rows + P->n_chunks;
  P->counters_need = (size_t)P->off_pos_pre + (size_t)P->n_chunks + 1;
  if (P->counters_need > ws.n_counters || ws.n_flags < 1) return MK_ERR_WORKSPACE;
  // 15/16 of the workgroups route and dispatch, then take grouped-GEMM tiles with the rest: the
  // m-tiles complete only near the end of the dispatch (token-ordered segments), so the compute
  // workgroups mostly wait until then, and the dispatch, bound by HBM with a tail of slow
  // workgroups, ends sooner the fewer rows each moves (measured at 256 workgroups: 192 copy
  // 171.3 us, 224 167.7-168.2, 232 167.5, 240 165.3, 248 165.5-165.8)
  const int copy_q = (ws.grid * 15 / 16) & ~7;
  const int want_copy = (o && o->n_copy_wg) ? o->n_copy_wg : (copy_q > 8 ? copy_q : 8);
  int nr = 0;
  int code = split_roles(ws.grid, want_copy, 0, o ? o->n_compute_wg : 0, &P->n_copy, &nr, &P->n_compute);
  if (code != MK_OK) return code;
  if (P->n_copy < 1) return MK_ERR_INVALID_ARG;
  return MK_OK;
}

}  // namespace mkh
