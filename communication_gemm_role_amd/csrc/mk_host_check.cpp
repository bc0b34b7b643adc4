// Host-only build of the C-ABI planning logic (no HIP), so argument validation, unit geometry,
// role split and workspace layout can be checked on machines without a GPU.  Each function
// returns the status code the matching mk_* entry point would return before launching, and
// fills `out` with the plan fields in declaration order.
#include "mk_host_logic.h"
#include "mk_tiles.h"

extern "C" {

int mkh_plan_ag(size_t n_flags, size_t n_counters, size_t inbox_bytes, int grid, const mkh::Opts* o,
                const void* const* a_shards, int world, int rank, int m_shard, int k, const void* b, int n,
                const void* a_gathered, const void* c, int tile_m, int tile_n, long long* out) {
  mkh::Ws ws{n_flags, n_counters, inbox_bytes, grid};
  mkh::AgPlan P{};
  const int code = mkh::plan_ag(ws, o, a_shards, world, rank, m_shard, k, b, n, a_gathered, c, tile_m, tile_n, &P);
  const long long v[] = {P.m, P.unit_rows, P.unit_cols, P.n_urows, P.n_ucols, P.n_order, P.local_in_place,
                         P.emulated, P.drop_pos, P.n_copy, P.n_compute, P.tiles_m, P.tiles_n,
                         (long long)P.pace_q16};
  for (unsigned i = 0; i < sizeof(v) / sizeof(v[0]); ++i) out[i] = v[i];
  return code;
}

int mkh_plan_reduce(size_t n_flags, size_t n_counters, size_t inbox_bytes, int grid, const mkh::Opts* o, int is_rs,
                    const void* a, const void* b, int m, int n, int k, int world, int rank, const void* const* peers,
                    const void* out_buf, void* const* outbox, int tile_m, int tile_n, int tile_waves,
                    int ring_kib, long long* out) {
  mkh::Ws ws{n_flags, n_counters, inbox_bytes, grid};
  mkh::RedPlan P{};
  const int code = mkh::plan_reduce(ws, o, is_rs, a, b, m, n, k, world, rank, peers, out_buf, outbox, tile_m, tile_n,
                                    tile_waves, ring_kib, &P);
  const long long v[] = {P.m_slice, P.p_rows, P.unit_rows, P.unit_cols, P.n_ucols, P.units_per_peer, P.n_units,
                         P.emulated, P.n_order, P.drop_pos, P.n_copy, P.n_reduce, P.n_compute, P.tiles_m, P.tiles_n,
                         P.own_tile_begin, P.own_tile_end, (long long)P.inbox_need, P.assist,
                         (long long)P.pace_q16};
  for (unsigned i = 0; i < sizeof(v) / sizeof(v[0]); ++i) out[i] = v[i];
  return code;
}

int mkh_plan_mlp(size_t n_flags, size_t n_counters, size_t inbox_bytes, int grid, const mkh::Opts* o,
                 const void* const* a_shards, int world, int rank, int m_shard, int k, const void* b_up, int n_up,
                 const void* b_down, int n_out, const void* const* peers, const void* a_gathered, const void* h,
                 const void* out, void* const* outbox, long long* out_fields) {
  mkh::Ws ws{n_flags, n_counters, inbox_bytes, grid};
  mkh::MlpPlan P{};
  const long long rows = (long long)world * m_shard;  // the kernels' tiles for this many output rows
  const mk_tiles::Shape& red = rows <= mk_tiles::kRedSkinnyMaxRows ? mk_tiles::kRedSkinny : mk_tiles::kRedBig;
  const int code = mkh::plan_mlp(ws, o, a_shards, world, rank, m_shard, k, b_up, n_up, b_down, n_out, peers,
                                 a_gathered, h, out, outbox, mk_tiles::kAg16.bm, mk_tiles::kAg16.bn, red.bm, red.bn,
                                 red.waves(), &P);
  const long long v[] = {P.ag.n_copy, P.ag.n_compute, P.ag.tiles_m, P.ag.tiles_n, P.red.n_compute, P.red.tiles_m,
                         P.red.tiles_n, P.red.own_tile_begin, P.red.own_tile_end, P.red.assist};
  for (unsigned i = 0; i < sizeof(v) / sizeof(v[0]); ++i) out_fields[i] = v[i];
  return code;
}

int mkh_plan_ring_attn(size_t n_flags, size_t n_counters, size_t inbox_bytes, int grid, const mkh::Opts* o,
                       const void* q, const void* const* k_shards, const void* const* v_shards, int world, int rank,
                       int heads, int s_local, int head_dim, float scale, const void* k_ring, const void* v_ring,
                       const void* out, const void* lse, long long* out_fields, float* scale_out) {
  mkh::Ws ws{n_flags, n_counters, inbox_bytes, grid};
  mkh::RaPlan P{};
  const int code = mkh::plan_ring_attn(ws, o, q, k_shards, v_shards, world, rank, heads, s_local, head_dim, scale,
                                       k_ring, v_ring, out, lse, &P);
  const long long v[] = {P.n_blk, P.n_qt, P.n_items, P.n_units, P.emulated, P.n_order, P.drop_pos, P.n_copy,
                         P.n_compute, (long long)P.pace_q16};
  for (unsigned i = 0; i < sizeof(v) / sizeof(v[0]); ++i) out_fields[i] = v[i];
  *scale_out = P.scale;
  return code;
}

int mkh_plan_moe(size_t n_flags, size_t n_counters, size_t inbox_bytes, int grid, const mkh::Opts* o,
                 const void* const* tokens, int world, int t_local, int hidden, const void* logits, const void* bias,
                 int n_experts, int top_k, int expert_begin, int n_local, const void* w_up, int ffn,
                 const void* topk_idx, const void* seg_offsets, const void* seg_token, const void* x_seg,
                 const void* y, int capacity, int tile_m, int tile_n, long long* out) {
  mkh::Ws ws{n_flags, n_counters, inbox_bytes, grid};
  mkh::MoePlan P{};
  const int code = mkh::plan_moe(ws, o, tokens, world, t_local, hidden, logits, bias, n_experts, top_k, expert_begin,
                                 n_local, w_up, ffn, topk_idx, seg_offsets, seg_token, x_seg, y, capacity, tile_m,
                                 tile_n, &P);
  const long long v[] = {P.n_tokens, P.n_chunks, P.emulated, P.drop_pos, P.n_copy, P.n_compute, P.tiles_n,
                         P.max_mtiles, P.off_misc, P.off_chunk_cnt, P.off_tile_cnt, (long long)P.counters_need};
  for (unsigned i = 0; i < sizeof(v) / sizeof(v[0]); ++i) out[i] = v[i];
  return code;
}

}  // extern "C"
