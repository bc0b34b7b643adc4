// C ABI of the fused communication+GEMM library (declared in include/mk.h).
// Every entry point validates and plans on the host (mk_host_logic.h), then enqueues exactly
// one persistent kernel on the caller's stream; nothing here allocates or synchronises after
// mk_ctx_create, except mk_ctx_status which is documented to synchronise.
#include <hip/hip_runtime.h>
#include <string.h>

#include <mutex>
#include <new>

#include "mk.h"
#include "mk_host_logic.h"
#include "mk_internal.h"

namespace {

constexpr size_t kDefaultWs = 512ull << 20;
constexpr size_t kStatusBytes = 256;
constexpr size_t kCounters = 1u << 20;  // 4 MiB of u32 counters
constexpr size_t kFlags = 1u << 20;     // 4 MiB of u32 flags
static_assert(mkh::kCtrBand0 == mk::CTR_RED_BAND0, "host and kernel agree on the RS band counters");
static_assert(mkh::kCtrHready0 == mk::CTR_MLP_HREADY0, "host and kernel agree on the MLP row-block counters");

struct DeviceGuard {  // make ctx->device current for the duration of a call
  int prev = -1;
  bool ok = false;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) return;
    ok = (prev == dev) || hipSetDevice(dev) == hipSuccess;
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

mkh::Opts to_opts(const mk_opts* o) {
  mkh::Opts r;
  memset(&r, 0, sizeof(r));
  if (!o) return r;
  r.n_copy_wg = o->n_copy_wg;
  r.n_compute_wg = o->n_compute_wg;
  r.n_reduce_wg = o->n_reduce_wg;
  r.arrival_mode = o->arrival_mode;
  r.arrival_order = o->arrival_order;
  r.arrival_len = o->arrival_len;
  r.arrival_unit_rows = o->arrival_unit_rows;
  r.arrival_unit_cols = o->arrival_unit_cols;
  r.arrival_chunk_tokens = o->arrival_chunk_tokens;
  r.timeout_us = o->timeout_us;
  r.test_drop_unit = o->test_drop_unit;
  r.arrival_gbps = o->arrival_gbps;
  return r;
}

mkh::Ws ws_of(const mk_ctx* c) {
  mkh::Ws w;
  w.n_flags = c->n_flags;
  w.n_counters = c->n_counters;
  w.inbox_bytes = c->inbox_bytes;
  w.grid = c->n_cu;
  return w;
}

uint64_t timeout_ticks(const mk_opts* o) {
  const int64_t us = (o && o->timeout_us > 0) ? o->timeout_us : 2000000;
  return (uint64_t)us * 100ull;  // the device wall clock runs at 100 MHz
}

// Next epoch; restart from 1 after clearing the flags if the counter would wrap.
int next_epoch(mk_ctx* c, hipStream_t s) {
  if (c->epoch >= 0xFFFFFF00u) {
    if (mk::launch_fill_u32(c->flags, 0u, c->n_flags, s) != hipSuccess) return MK_ERR_HIP;
    c->epoch = 0;
  }
  ++c->epoch;
  return MK_OK;
}

// Kernel parameters of an AllGather + GEMM call from its plan; the workspace (flags, counters,
// status word) and the epoch are the caller's: a context's, or the static scratch array's.
mk::AgParams ag_params(const mkh::AgPlan& P, const uint16_t* const* a_shards, int world, int rank, int m_shard, int k,
                       const uint16_t* b, int n, uint16_t* a_gathered, float* c, const mk_opts* opts, uint32_t* flags,
                       uint32_t* counters, int* status, uint32_t epoch, int* status_out) {
  mk::AgParams p;
  memset(&p, 0, sizeof(p));
  for (int r = 0; r < world; ++r) p.shards[r] = a_shards ? a_shards[r] : nullptr;
  p.b = b;
  p.ag = a_gathered;
  p.c = c;
  p.order = (P.emulated && opts) ? (const int32_t*)opts->arrival_order : nullptr;
  p.flags = flags;
  p.status = status;
  p.world = world;
  p.rank = rank;
  p.m_shard = m_shard;
  p.m = P.m;
  p.n = n;
  p.k = k;
  p.unit_rows = P.unit_rows;
  p.unit_cols = P.unit_cols;
  p.n_ucols = P.n_ucols;
  p.n_urows = P.n_urows;
  p.n_copy = P.n_copy;
  p.n_compute = P.n_compute;
  p.emulated = P.emulated;
  p.pace_q16 = P.pace_q16;
  p.local_in_place = P.local_in_place;
  p.n_order = P.n_order;
  p.drop_pos = P.drop_pos;
  p.tiles_m = P.tiles_m;
  p.tiles_n = P.tiles_n;
  p.epoch = epoch;
  p.timeout_ticks = timeout_ticks(opts);
  p.trace = opts ? opts->trace : nullptr;
  p.counters = counters;
  p.status_out = status_out;
  return p;
}

}  // namespace

extern "C" {

const char* mk_strerror(int code) {
  switch (code) {
    case MK_OK: return "ok";
    case MK_ERR_INVALID_ARG: return "invalid argument";
    case MK_ERR_UNSUPPORTED: return "unsupported size, alignment or option";
    case MK_ERR_WORKSPACE: return "context workspace too small";
    case MK_ERR_HIP: return "HIP runtime error";
    case MK_ERR_TIMEOUT: return "device wait timed out";
    case MK_ERR_CAPACITY: return "routed rows exceed capacity";
    default: return "unknown error";
  }
}

int mk_ctx_create(int device, size_t workspace_bytes, mk_ctx** out) {
  if (!out) return MK_ERR_INVALID_ARG;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess) return MK_ERR_HIP;
  if (device < 0 || device >= ndev) return MK_ERR_INVALID_ARG;
  if (workspace_bytes == 0) workspace_bytes = kDefaultWs;
  const size_t fixed = kStatusBytes + (kCounters + kFlags) * 4;
  if (workspace_bytes < fixed) return MK_ERR_WORKSPACE;
  DeviceGuard g(device);
  if (!g.ok) return MK_ERR_HIP;
  mk_ctx* c = new (std::nothrow) mk_ctx();
  if (!c) return MK_ERR_HIP;
  c->device = device;
  if (hipDeviceGetAttribute(&c->n_cu, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess) {
    delete c;
    return MK_ERR_HIP;
  }
  void* ws = nullptr;
  if (hipMalloc(&ws, workspace_bytes) != hipSuccess) {
    delete c;
    return MK_ERR_HIP;
  }
  c->ws = (char*)ws;
  c->ws_bytes = workspace_bytes;
  c->status = (int*)c->ws;
  c->counters = (uint32_t*)(c->ws + kStatusBytes);
  c->n_counters = kCounters;
  c->flags = c->counters + kCounters;
  c->n_flags = kFlags;
  c->inbox = (char*)(c->flags + kFlags);
  c->inbox_bytes = workspace_bytes - fixed;
  c->epoch = 0;
  if (hipMemset(c->ws, 0, fixed) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
    (void)hipFree(ws);
    delete c;
    return MK_ERR_HIP;
  }
  *out = c;
  return MK_OK;
}

int mk_ctx_destroy(mk_ctx* ctx) {
  if (!ctx) return MK_ERR_INVALID_ARG;
  DeviceGuard g(ctx->device);
  const hipError_t e = hipFree(ctx->ws);
  delete ctx;
  return e == hipSuccess ? MK_OK : MK_ERR_HIP;
}

int mk_ctx_grid(mk_ctx* ctx) { return ctx ? ctx->n_cu : MK_ERR_INVALID_ARG; }

int mk_ctx_status(mk_ctx* ctx, void* stream) {
  if (!ctx) return MK_ERR_INVALID_ARG;
  DeviceGuard g(ctx->device);
  if (!g.ok) return MK_ERR_HIP;
  hipStream_t s = (hipStream_t)stream;
  if (hipStreamSynchronize(s) != hipSuccess) return MK_ERR_HIP;
  int v = 0;
  if (hipMemcpy(&v, ctx->status, sizeof(int), hipMemcpyDeviceToHost) != hipSuccess) return MK_ERR_HIP;
  if (v != 0) {
    const int zero = 0;
    if (hipMemcpy(ctx->status, &zero, sizeof(int), hipMemcpyHostToDevice) != hipSuccess) return MK_ERR_HIP;
  }
  return v;
}

int mk_ctx_reset(mk_ctx* ctx, void* stream) {
  if (!ctx) return MK_ERR_INVALID_ARG;
  DeviceGuard g(ctx->device);
  if (!g.ok) return MK_ERR_HIP;
  hipStream_t s = (hipStream_t)stream;
  if (mk::launch_fill_u32((uint32_t*)ctx->status, 0u, kStatusBytes / 4, s) != hipSuccess) return MK_ERR_HIP;
  if (mk::launch_fill_u32(ctx->counters, 0u, ctx->n_counters, s) != hipSuccess) return MK_ERR_HIP;
  if (mk::launch_fill_u32(ctx->flags, 0u, ctx->n_flags, s) != hipSuccess) return MK_ERR_HIP;
  ctx->epoch = 0;
  return MK_OK;
}

int mk_ag_gemm(mk_ctx* ctx, void* stream, const uint16_t* const* a_shards, int world, int rank, int m_shard, int k,
               const uint16_t* b, int n, uint16_t* a_gathered, float* c, const mk_opts* opts) {
  if (!ctx) return MK_ERR_INVALID_ARG;
  const mkh::Opts o = to_opts(opts);
  mkh::AgPlan P;
  int code = mkh::plan_ag(ws_of(ctx), opts ? &o : nullptr, (const void* const*)a_shards, world, rank, m_shard, k, b, n,
                          a_gathered, c, mk::ag_tile_m(), mk::ag_tile_n(), &P);
  if (code != MK_OK) return code;
  DeviceGuard g(ctx->device);
  if (!g.ok) return MK_ERR_HIP;
  hipStream_t s = (hipStream_t)stream;
  if ((code = next_epoch(ctx, s)) != MK_OK) return code;
  const mk::AgParams p = ag_params(P, a_shards, world, rank, m_shard, k, b, n, a_gathered, c, opts, ctx->flags,
                                   ctx->counters, ctx->status, ctx->epoch, nullptr);
  return mk::launch_ag_gemm(p, P.n_copy + P.n_compute, s) == hipSuccess ? MK_OK : MK_ERR_HIP;
}

static int gemm_reduce(int is_rs, mk_ctx* ctx, void* stream, const uint16_t* a, const uint16_t* b, int m, int n,
                       int k, int world, int rank, const float* const* peers, float* out, float* const* outbox,
                       const mk_opts* opts) {
  if (!ctx) return MK_ERR_INVALID_ARG;
  const mkh::Opts o = to_opts(opts);
  mkh::RedPlan P;
  int code = mkh::plan_reduce(ws_of(ctx), opts ? &o : nullptr, is_rs, a, b, m, n, k, world, rank,
                              (const void* const*)peers, out, (void* const*)outbox, mk::red_tile_m(m, n),
                              mk::red_tile_n(m, n), mk::red_tile_waves(m, n), mk::red_ring_kib(m, n), &P);
  if (code != MK_OK) return code;
  DeviceGuard g(ctx->device);
  if (!g.ok) return MK_ERR_HIP;
  hipStream_t s = (hipStream_t)stream;
  if ((code = next_epoch(ctx, s)) != MK_OK) return code;
  mk::RedParams p;
  memset(&p, 0, sizeof(p));
  p.a = a;
  p.b = b;
  for (int j = 0; j < world; ++j) {
    p.peers[j] = (j == rank || !peers) ? nullptr : peers[j];
    p.outbox[j] = (j == rank || !outbox) ? nullptr : outbox[j];
  }
  p.out = out;
  p.inbox = (float*)ctx->inbox;
  p.order = (P.emulated && opts) ? (const int32_t*)opts->arrival_order : nullptr;
  p.flags = ctx->flags;
  p.presum_flags = ctx->flags + P.n_units;
  p.status = ctx->status;
  p.is_rs = is_rs;
  p.m = m;
  p.n = n;
  p.k = k;
  p.world = world;
  p.rank = rank;
  p.m_slice = P.m_slice;
  p.p_rows = P.p_rows;
  p.unit_rows = P.unit_rows;
  p.unit_cols = P.unit_cols;
  p.n_ucols = P.n_ucols;
  p.units_per_peer = P.units_per_peer;
  p.n_copy = P.n_copy;
  p.n_reduce = P.n_reduce;
  p.assist = P.assist;
  p.n_compute = P.n_compute;
  p.emulated = P.emulated;
  p.pace_q16 = P.pace_q16;
  p.n_order = P.n_order;
  p.drop_pos = P.drop_pos;
  p.tiles_m = P.tiles_m;
  p.tiles_n = P.tiles_n;
  p.own_tile_begin = P.own_tile_begin;
  p.own_tile_end = P.own_tile_end;
  p.epoch = ctx->epoch;
  p.timeout_ticks = timeout_ticks(opts);
  p.trace = opts ? opts->trace : nullptr;
  p.counters = ctx->counters;
  return mk::launch_gemm_reduce(p, P.n_copy + P.n_reduce + P.n_compute, s) == hipSuccess ? MK_OK : MK_ERR_HIP;
}

int mk_gemm_rs(mk_ctx* ctx, void* stream, const uint16_t* a, const uint16_t* b, int m, int n, int k, int world,
               int rank, const float* const* peer_partials, float* owned_out, float* const* outbox,
               const mk_opts* opts) {
  return gemm_reduce(1, ctx, stream, a, b, m, n, k, world, rank, peer_partials, owned_out, outbox, opts);
}

int mk_gemm_ar(mk_ctx* ctx, void* stream, const uint16_t* a, const uint16_t* b, int m, int n, int k, int world,
               int rank, const float* const* peer_partials, float* out, const mk_opts* opts) {
  return gemm_reduce(0, ctx, stream, a, b, m, n, k, world, rank, peer_partials, out, nullptr, opts);
}

int mk_mlp_ag_rs(mk_ctx* ctx, void* stream, const uint16_t* const* a_shards, int world, int rank, int m_shard, int k,
                 const uint16_t* b_up, int n_up, const uint16_t* b_down, int n_out, const float* const* peer_partials,
                 uint16_t* a_gathered, uint16_t* h, float* owned_out, float* const* outbox, const mk_opts* opts) {
  if (!ctx) return MK_ERR_INVALID_ARG;
  const mkh::Opts o = to_opts(opts);
  // only picks the tile shapes here (the plan validates the sizes); widened so that no argument
  // can overflow it
  const long long m_all = (long long)world * (long long)m_shard;
  const int M = m_all > 0x7fffffffLL ? 0x7fffffff : (int)m_all;
  mkh::MlpPlan P;
  int code = mkh::plan_mlp(ws_of(ctx), opts ? &o : nullptr, (const void* const*)a_shards, world, rank, m_shard, k,
                           b_up, n_up, b_down, n_out, (const void* const*)peer_partials, a_gathered, h, owned_out,
                           (void* const*)outbox, mk::mlp_tile_m(), mk::mlp_tile_n(), mk::red_tile_m(M, n_out),
                           mk::red_tile_n(M, n_out), mk::red_tile_waves(M, n_out), &P);
  if (code != MK_OK) return code;
  DeviceGuard g(ctx->device);
  if (!g.ok) return MK_ERR_HIP;
  hipStream_t s = (hipStream_t)stream;
  if ((code = next_epoch(ctx, s)) != MK_OK) return code;
  mk::MlpParams p;
  memset(&p, 0, sizeof(p));
  mk::AgParams& a = p.ag;
  for (int r = 0; r < world; ++r) a.shards[r] = a_shards ? a_shards[r] : nullptr;
  a.b = b_up;
  a.ag = a_gathered;
  a.c = nullptr;
  a.h = h;
  a.h_ready = ctx->counters + mk::CTR_MLP_HREADY0;
  a.order = (P.ag.emulated && opts) ? (const int32_t*)opts->arrival_order : nullptr;
  a.flags = ctx->flags;
  a.status = ctx->status;
  a.world = world;
  a.rank = rank;
  a.m_shard = m_shard;
  a.m = P.ag.m;
  a.n = n_up;
  a.k = k;
  a.unit_rows = P.ag.unit_rows;
  a.unit_cols = P.ag.unit_cols;
  a.n_ucols = P.ag.n_ucols;
  a.n_urows = P.ag.n_urows;
  a.n_copy = P.ag.n_copy;
  a.n_compute = P.ag.n_compute;
  a.emulated = P.ag.emulated;
  a.pace_q16 = P.ag.pace_q16;
  a.local_in_place = P.ag.local_in_place;
  a.n_order = P.ag.n_order;
  a.drop_pos = P.ag.drop_pos;
  a.tiles_m = P.ag.tiles_m;
  a.tiles_n = P.ag.tiles_n;
  a.epoch = ctx->epoch;
  a.timeout_ticks = timeout_ticks(opts);
  a.trace = opts ? opts->trace : nullptr;
  a.counters = ctx->counters;
  mk::RedParams& d = p.red;
  d.a = h;
  d.b = b_down;
  for (int j = 0; j < world; ++j) {
    d.peers[j] = (j == rank || !peer_partials) ? nullptr : peer_partials[j];
    d.outbox[j] = (j == rank || !outbox) ? nullptr : outbox[j];
  }
  d.out = owned_out;
  d.inbox = (float*)ctx->inbox;
  d.flags = ctx->flags;
  d.presum_flags = ctx->flags + P.ag.n_urows * P.ag.n_ucols;
  d.status = ctx->status;
  d.is_rs = 1;
  d.m = M;
  d.n = n_out;
  d.k = n_up;
  d.world = world;
  d.rank = rank;
  d.m_slice = P.red.m_slice;
  d.p_rows = P.red.p_rows;
  d.unit_rows = P.red.unit_rows;
  d.unit_cols = P.red.unit_cols;
  d.n_ucols = P.red.n_ucols;
  d.units_per_peer = P.red.units_per_peer;
  d.n_compute = P.red.n_compute;
  d.assist = P.red.assist;
  d.tiles_m = P.red.tiles_m;
  d.tiles_n = P.red.tiles_n;
  d.own_tile_begin = P.red.own_tile_begin;
  d.own_tile_end = P.red.own_tile_end;
  d.epoch = ctx->epoch;
  d.timeout_ticks = timeout_ticks(opts);
  d.trace = nullptr;  // the trace records keep phase 1's marks
  d.counters = ctx->counters;
  d.a_ready = ctx->counters + mk::CTR_MLP_HREADY0;
  d.a_ready_need = (uint32_t)P.ag.tiles_n;
  return mk::launch_mlp(p, ws_of(ctx).grid, s) == hipSuccess ? MK_OK : MK_ERR_HIP;
}

int mk_moe_dispatch_gemm(mk_ctx* ctx, void* stream, const uint16_t* const* tokens, int world, int t_local,
                         int hidden, const float* logits, const float* bias, int n_experts, int top_k,
                         int expert_begin, int n_local_experts, const uint16_t* w_up, int ffn, int32_t* topk_idx,
                         int32_t* seg_offsets, int32_t* seg_token, uint16_t* x_seg, float* y, int capacity_rows,
                         const mk_opts* opts) {
  if (!ctx) return MK_ERR_INVALID_ARG;
  const mkh::Opts o = to_opts(opts);
  mkh::MoePlan P;
  int code = mkh::plan_moe(ws_of(ctx), opts ? &o : nullptr, (const void* const*)tokens, world, t_local, hidden, logits,
                           bias, n_experts, top_k, expert_begin, n_local_experts, w_up, ffn, topk_idx, seg_offsets,
                           seg_token, x_seg, y, capacity_rows, mk::moe_tile_m(), mk::moe_tile_n(), &P);
  if (code != MK_OK) return code;
  DeviceGuard g(ctx->device);
  if (!g.ok) return MK_ERR_HIP;
  hipStream_t s = (hipStream_t)stream;
  if ((code = next_epoch(ctx, s)) != MK_OK) return code;
  mk::MoeParams p;
  memset(&p, 0, sizeof(p));
  for (int r = 0; r < world; ++r) p.tokens[r] = tokens[r];
  p.logits = logits;
  p.bias = bias;
  p.w_up = w_up;
  p.topk_idx = topk_idx;
  p.seg_offsets = seg_offsets;
  p.seg_token = seg_token;
  p.x_seg = x_seg;
  p.y = y;
  p.order = (P.emulated && opts) ? (const int32_t*)opts->arrival_order : nullptr;
  p.counters = ctx->counters;
  p.flags = ctx->flags;
  p.status = ctx->status;
  p.world = world;
  p.t_local = t_local;
  p.hidden = hidden;
  p.n_experts = n_experts;
  p.top_k = top_k;
  p.expert_begin = expert_begin;
  p.n_local = n_local_experts;
  p.ffn = ffn;
  p.capacity = capacity_rows;
  p.n_tokens = P.n_tokens;
  p.n_chunks = P.n_chunks;
  p.n_route = P.n_copy;
  p.n_copy = P.n_copy;
  p.n_compute = P.n_compute;
  p.emulated = P.emulated;
  p.drop_pos = P.drop_pos;
  p.tiles_n = P.tiles_n;
  p.max_mtiles = P.max_mtiles;
  p.epoch = ctx->epoch;
  p.timeout_ticks = timeout_ticks(opts);
  p.trace = opts ? opts->trace : nullptr;
  p.off_chunk_cnt = P.off_chunk_cnt;
  p.off_tile_cnt = P.off_tile_cnt;
  p.off_chunk_rows = P.off_chunk_rows;
  p.off_pos_pre = P.off_pos_pre;
  p.off_misc = P.off_misc;
  return mk::launch_moe(p, P.n_copy + P.n_compute, s) == hipSuccess ? MK_OK : MK_ERR_HIP;
}

int mk_ring_attention(mk_ctx* ctx, void* stream, const uint16_t* q, const uint16_t* const* k_shards,
                      const uint16_t* const* v_shards, int world, int rank, int heads, int s_local, int head_dim,
                      float softmax_scale, uint16_t* k_ring, uint16_t* v_ring, float* out, float* lse,
                      const mk_opts* opts) {
  if (!ctx) return MK_ERR_INVALID_ARG;
  const mkh::Opts o = to_opts(opts);
  mkh::RaPlan P;
  int code = mkh::plan_ring_attn(ws_of(ctx), opts ? &o : nullptr, q, (const void* const*)k_shards,
                                 (const void* const*)v_shards, world, rank, heads, s_local, head_dim, softmax_scale,
                                 k_ring, v_ring, out, lse, &P);
  if (code != MK_OK) return code;
  DeviceGuard g(ctx->device);
  if (!g.ok) return MK_ERR_HIP;
  hipStream_t s = (hipStream_t)stream;
  if ((code = next_epoch(ctx, s)) != MK_OK) return code;
  mk::RaParams p;
  memset(&p, 0, sizeof(p));
  p.q = q;
  for (int r = 0; r < world; ++r) {
    p.k_src[r] = k_shards[r];
    p.v_src[r] = v_shards[r];
  }
  p.k_ring = k_ring;
  p.v_ring = v_ring;
  p.out = out;
  p.lse = lse;
  p.order = (P.emulated && opts) ? (const int32_t*)opts->arrival_order : nullptr;
  p.flags = ctx->flags;
  p.counters = ctx->counters;
  p.status = ctx->status;
  p.scale_log2 = P.scale * 1.4426950408889634f;
  p.world = world;
  p.rank = rank;
  p.heads = heads;
  p.s_local = s_local;
  p.n_blk = P.n_blk;
  p.n_qt = P.n_qt;
  p.n_items = P.n_items;
  p.n_units = P.n_units;
  p.n_copy = P.n_copy;
  p.n_compute = P.n_compute;
  p.emulated = P.emulated;
  p.n_order = P.n_order;
  p.drop_pos = P.drop_pos;
  p.epoch = ctx->epoch;
  p.timeout_ticks = timeout_ticks(opts);
  p.trace = opts ? opts->trace : nullptr;
  p.pace_q16 = P.pace_q16;
  return mk::launch_ring_attn(p, ws_of(ctx).grid, s) == hipSuccess ? MK_OK : MK_ERR_HIP;
}

}  // extern "C"

// ---- role-split tuning ------------------------------------------------------------------------------
namespace {

// Times call(n_copy) for each candidate on the stream: two untimed calls, then `reps` calls between
// two events.  us_out[i] is the mean time per call in microseconds, or -1 where the planner rejects
// that split (MK_ERR_INVALID_ARG / MK_ERR_UNSUPPORTED: the candidate does not fit, which is not an
// error of the tuning).  Stops at the first HIP error or device-side status (watchdog, ...).
template <class Call>
int tune_split(mk_ctx* ctx, void* stream, const int* cand, int n_cand, int reps, float* us_out, int* best,
               Call&& call) {
  if (!ctx || !cand || n_cand <= 0 || reps <= 0 || !us_out || !best) return MK_ERR_INVALID_ARG;
  DeviceGuard g(ctx->device);
  if (!g.ok) return MK_ERR_HIP;
  hipStream_t s = (hipStream_t)stream;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess) return MK_ERR_HIP;
  if (hipEventCreate(&e1) != hipSuccess) {
    (void)hipEventDestroy(e0);
    return MK_ERR_HIP;
  }
  int code = MK_OK, rejected = MK_OK, found = 0;
  float best_us = 0.f;
  for (int i = 0; i < n_cand; ++i) us_out[i] = -1.f;
  for (int i = 0; i < n_cand && code == MK_OK; ++i) {
    int c = call(cand[i]);
    if (c == MK_ERR_INVALID_ARG || c == MK_ERR_UNSUPPORTED) {
      if (rejected == MK_OK) rejected = c;
      continue;
    }
    if (c == MK_OK) c = call(cand[i]);
    if (c == MK_OK && hipEventRecord(e0, s) != hipSuccess) c = MK_ERR_HIP;
    for (int r = 0; r < reps && c == MK_OK; ++r) c = call(cand[i]);
    if (c == MK_OK && (hipEventRecord(e1, s) != hipSuccess || hipEventSynchronize(e1) != hipSuccess)) c = MK_ERR_HIP;
    if (c == MK_OK) c = mk_ctx_status(ctx, stream);
    float ms = 0.f;
    if (c == MK_OK && hipEventElapsedTime(&ms, e0, e1) != hipSuccess) c = MK_ERR_HIP;
    if (c != MK_OK) {
      code = c;
      break;
    }
    us_out[i] = ms * 1000.f / (float)reps;
    if (!found || us_out[i] < best_us) {
      best_us = us_out[i];
      *best = cand[i];
      found = 1;
    }
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (code == MK_OK && !found) code = rejected;
  return code;
}

mk_opts opts_copy(const mk_opts* o) {
  mk_opts r;
  if (o) r = *o;
  else memset(&r, 0, sizeof(r));
  return r;
}

}  // namespace

extern "C" {

int mk_ag_gemm_tune(mk_ctx* ctx, void* stream, const uint16_t* const* a_shards, int world, int rank, int m_shard,
                    int k, const uint16_t* b, int n, uint16_t* a_gathered, float* c, const mk_opts* opts,
                    const int* n_copy_candidates, int n_candidates, int reps, float* us_per_call, int* best_n_copy) {
  mk_opts o = opts_copy(opts);
  return tune_split(ctx, stream, n_copy_candidates, n_candidates, reps, us_per_call, best_n_copy, [&](int nc) {
    o.n_copy_wg = nc;
    return mk_ag_gemm(ctx, stream, a_shards, world, rank, m_shard, k, b, n, a_gathered, c, &o);
  });
}

int mk_gemm_rs_tune(mk_ctx* ctx, void* stream, const uint16_t* a, const uint16_t* b, int m, int n, int k, int world,
                    int rank, const float* const* peer_partials, float* owned_out, float* const* outbox,
                    const mk_opts* opts, const int* n_copy_candidates, int n_candidates, int reps,
                    float* us_per_call, int* best_n_copy) {
  mk_opts o = opts_copy(opts);
  return tune_split(ctx, stream, n_copy_candidates, n_candidates, reps, us_per_call, best_n_copy, [&](int nc) {
    o.n_copy_wg = nc;
    return mk_gemm_rs(ctx, stream, a, b, m, n, k, world, rank, peer_partials, owned_out, outbox, &o);
  });
}

int mk_gemm_ar_tune(mk_ctx* ctx, void* stream, const uint16_t* a, const uint16_t* b, int m, int n, int k, int world,
                    int rank, const float* const* peer_partials, float* out, const mk_opts* opts,
                    const int* n_copy_candidates, int n_candidates, int reps, float* us_per_call, int* best_n_copy) {
  mk_opts o = opts_copy(opts);
  return tune_split(ctx, stream, n_copy_candidates, n_candidates, reps, us_per_call, best_n_copy, [&](int nc) {
    o.n_copy_wg = nc;
    return mk_gemm_ar(ctx, stream, a, b, m, n, k, world, rank, peer_partials, out, &o);
  });
}

}  // extern "C"

// ---- AllGather + GEMM without allocation ------------------------------------------------------------
// The ready flags, counters and status word live in a static device array instead of a context's
// workspace.  In host code `scratch` names a host-side stand-in, not the device array: its device
// address is taken once per device with hipGetSymbolAddress and only that address is used.
namespace {

constexpr size_t kScratchStatusWords = 64;  // the status word, padded to 256 bytes
constexpr size_t kScratchCounters = 128;    // the AllGather + GEMM claim and exit counters sit at 110, 111
constexpr size_t kScratchFlags = 16384;     // one epoch flag per arrival unit
constexpr size_t kScratchWords = kScratchStatusWords + kScratchCounters + kScratchFlags;
static_assert(mk::CTR_AG_EXIT < (int)kScratchCounters, "the AllGather + GEMM counters fit the static counters");
constexpr int kMaxDevices = 64;

struct ScratchDev {
  uint32_t* ptr;   // device address of `scratch` on this device (null until set up)
  uint32_t epoch;  // call number on this device; a flag is up when it equals the current epoch
  int n_cu;
};
ScratchDev g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

}  // namespace

static __device__ __align__(256) uint32_t scratch[kScratchWords];

namespace {

// Once per device, with that device current: the array's device address, the grid size, and a
// zero fill of the array on `s` (a fill kernel, not a memset).  Nothing here allocates.
int scratch_setup(int dev, hipStream_t s, ScratchDev** out) {
  if (dev < 0 || dev >= kMaxDevices) return MK_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ScratchDev& d = g_scratch[dev];
  if (!d.ptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MK_ERR_HIP;
    int n_cu = 0;
    if (hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu <= 0)
      return MK_ERR_HIP;
    if (mk::launch_fill_u32((uint32_t*)ptr, 0u, kScratchWords, s) != hipSuccess) return MK_ERR_HIP;
    d.ptr = (uint32_t*)ptr;
    d.n_cu = n_cu;
    d.epoch = 0;
  }
  *out = &d;
  return MK_OK;
}

}  // namespace

extern "C" int mk_ag_gemm_noalloc(void* stream, const uint16_t* const* a_shards, int world, int rank, int m_shard,
                                  int k, const uint16_t* b, int n, uint16_t* a_gathered, float* c, int* status,
                                  const mk_opts* opts) {
  if (!status || ((uintptr_t)status & 3u)) return MK_ERR_INVALID_ARG;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MK_ERR_HIP;
  hipStream_t s = (hipStream_t)stream;
  ScratchDev* d = nullptr;
  int code = scratch_setup(dev, s, &d);
  if (code != MK_OK) return code;
  uint32_t* status_word = d->ptr;
  uint32_t* counters = d->ptr + kScratchStatusWords;
  uint32_t* flags = counters + kScratchCounters;
  const mkh::Ws ws{kScratchFlags, kScratchCounters, 0, d->n_cu};
  const mkh::Opts o = to_opts(opts);
  mkh::AgPlan P;
  code = mkh::plan_ag(ws, opts ? &o : nullptr, (const void* const*)a_shards, world, rank, m_shard, k, b, n, a_gathered,
                      c, mk::ag_tile_m(), mk::ag_tile_n(), &P);
  if (code != MK_OK) return code;  // MK_ERR_WORKSPACE: more arrival units than static flags
  uint32_t epoch;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (d->epoch >= 0xFFFFFF00u) {  // restart the epochs on cleared flags
      if (mk::launch_fill_u32(flags, 0u, kScratchFlags, s) != hipSuccess) return MK_ERR_HIP;
      d->epoch = 0;
    }
    epoch = ++d->epoch;
  }
  const mk::AgParams p = ag_params(P, a_shards, world, rank, m_shard, k, b, n, a_gathered, c, opts, flags, counters,
                                   (int*)status_word, epoch, status);
  return mk::launch_ag_gemm(p, P.n_copy + P.n_compute, s) == hipSuccess ? MK_OK : MK_ERR_HIP;
}
