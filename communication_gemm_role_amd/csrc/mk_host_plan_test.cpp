// CPU test driver over the host planning code (mk_host_logic.h), meant to be built with
// AddressSanitizer and UndefinedBehaviorSanitizer (g++ -fsanitize=address,undefined
// -fno-sanitize-recover=all): it calls every mkh::plan_* function on a sweep of hand-picked and
// pseudo-random arguments -- valid shapes, zeros, negatives, values near INT_MAX, null and
// misaligned pointers, bad options -- and checks, for every plan it accepts, the invariants the
// kernels rely on (role counts fit the grid, every tile and arrival unit is covered, flag, counter
// and inbox needs fit the workspace).  Any signed overflow, out-of-bounds access or failed
// invariant aborts the run with a message; a clean run prints the number of calls and "ok".
//
//   mk_host_plan_test [n_random]     (default 200000 random calls per planner)
#include <limits.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "mk_host_logic.h"
#include "mk_tiles.h"

#include <initializer_list>

namespace {

long long g_calls = 0, g_ok = 0;

#define CHECK(cond)                                                                   \
  do {                                                                                \
    if (!(cond)) {                                                                    \
      fprintf(stderr, "%s:%d: invariant failed: %s\n", __FILE__, __LINE__, #cond);    \
      abort();                                                                        \
    }                                                                                 \
  } while (0)

// splitmix64: a counter-based generator, so every run sweeps the same arguments
struct Rng {
  uint64_t s;
  uint64_t next() {
    uint64_t z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
  int below(int n) { return (int)(next() % (uint64_t)n); }
  // a size: usually a small multiple of 64, sometimes ragged, zero, negative or huge
  int size() {
    switch (below(10)) {
      case 0: return 0;
      case 1: return -64 * (1 + below(4));
      case 2: return INT_MAX - below(3);
      case 3: return 64 * below(2000000) + 64;
      case 4: return 1 + below(1000);
      default: return 64 * (1 + below(160));
    }
  }
  int small(int lo, int hi) { return lo + below(hi - lo + 1); }
  // a size the kernels take: a multiple of 64 (often of 128) up to 16384
  int good() { return below(2) ? 128 * (1 + below(128)) : 64 * (1 + below(256)); }
};

const void* P(uintptr_t v) { return (const void*)v; }

mkh::Opts random_opts(Rng& r, bool* use) {
  mkh::Opts o{};
  *use = r.below(4) != 0;
  if (!*use) return o;
  const int modes[] = {0, MK_ARRIVAL_RESIDENT, MK_ARRIVAL_EMULATED, 3, -1};
  o.arrival_mode = modes[r.below(5)];
  o.n_copy_wg = r.below(3) ? 0 : r.small(-8, 300);
  o.n_compute_wg = r.below(3) ? 0 : r.small(-8, 300);
  o.n_reduce_wg = r.below(3) ? 0 : r.small(-8, 300);
  const int units[] = {0, 64, 128, 32, 256};
  o.arrival_unit_rows = units[r.below(5)];
  o.arrival_unit_cols = units[r.below(5)];
  o.arrival_chunk_tokens = r.below(4) ? 0 : 64 * r.below(3);
  o.timeout_us = r.below(3) ? 0 : (int64_t)r.small(-5, 5000000);
  o.test_drop_unit = r.below(3) ? 0 : r.small(-2, 100);
  const double rates[] = {0.0, 0.0, 1071.0, 1.0, 0.001, -3.0, 1e12};
  o.arrival_gbps = rates[r.below(7)];
  if (r.below(3) == 0) {
    o.arrival_order = P(r.below(8) ? 0x90000 : 0x90002);
    o.arrival_len = r.below(2) ? r.small(0, 4096) : 1792;
  }
  return o;
}

mkh::Ws random_ws(Rng& r) {
  mkh::Ws w;
  w.n_flags = r.below(8) ? (1u << 20) : (size_t)r.small(0, 4096);
  w.n_counters = r.below(8) ? (1u << 20) : (size_t)r.small(0, 8192);
  w.inbox_bytes = r.below(6) ? (512ull << 20) : (size_t)r.small(0, 1 << 24);
  w.grid = r.below(8) ? 256 : r.small(1, 512);
  return w;
}

void check_roles(const mkh::Ws& ws, int n_copy, int n_reduce, int n_compute) {
  CHECK(n_copy >= 0 && n_reduce >= 0 && n_compute >= 1);
  CHECK((long long)n_copy + n_reduce + n_compute <= ws.grid);
}

// ---- AllGather + GEMM -----------------------------------------------------------------------
void ag_case(const mkh::Ws& ws, const mkh::Opts* o, int world, int rank, int m_shard, int k, int n, int shards_kind,
             int tm, int tn) {
  const void* shards[mkh::kMaxWorld];
  const uintptr_t ag = 0x10000000;
  for (int r = 0; r < mkh::kMaxWorld; ++r) shards[r] = P(0x20000000 + 0x100000 * (uintptr_t)r);
  if (shards_kind == 1 && rank >= 0 && rank < mkh::kMaxWorld && m_shard > 0 && k > 0 && world > 0)
    shards[rank] = P(ag + (uintptr_t)rank * (uintptr_t)m_shard * (uintptr_t)k * 2);
  if (shards_kind == 2 && world > 1 && world <= mkh::kMaxWorld) shards[world - 1] = nullptr;
  if (shards_kind == 3) shards[0] = P(0x20000008);
  mkh::AgPlan A{};
  ++g_calls;
  const int code = mkh::plan_ag(ws, o, shards_kind == 4 ? nullptr : shards, world, rank, m_shard, k, P(0x30000000), n,
                                P(ag), P(0x40000000), tm, tn, &A);
  if (code != MK_OK) return;
  ++g_ok;
  CHECK(world >= 1 && world <= mkh::kMaxWorld && rank >= 0 && rank < world);
  CHECK(m_shard % A.unit_rows == 0 && k % A.unit_cols == 0);
  CHECK((long long)A.m == (long long)world * m_shard);
  CHECK((long long)A.n_urows * A.unit_rows == A.m && (long long)A.n_ucols * A.unit_cols == k);
  CHECK(A.n_ucols <= 64);
  CHECK((size_t)A.n_urows * (size_t)A.n_ucols <= ws.n_flags);
  CHECK((long long)A.tiles_m * tm >= A.m && (long long)(A.tiles_m - 1) * tm < A.m);
  CHECK((long long)A.tiles_n * tn >= n && (long long)(A.tiles_n - 1) * tn < n);
  check_roles(ws, A.n_copy, 0, A.n_compute);
  if (A.emulated) {
    const long long spr = m_shard / A.unit_rows;
    CHECK((long long)A.n_order == (long long)(world - A.local_in_place) * spr * A.n_ucols);
    CHECK(A.n_order == 0 || A.n_copy > 0);
  } else {
    CHECK(A.n_copy == 0 && A.n_order == 0);
  }
}

// ---- GEMM + RS / AR ---------------------------------------------------------------------------
void red_case(const mkh::Ws& ws, const mkh::Opts* o, int is_rs, int m, int n, int k, int world, int rank,
              int ptr_kind) {
  const void* peers[mkh::kMaxWorld];
  void* outbox[mkh::kMaxWorld];
  for (int j = 0; j < mkh::kMaxWorld; ++j) {
    peers[j] = P(0x50000000 + 0x100000 * (uintptr_t)j);
    outbox[j] = (void*)(0x60000000 + 0x100000 * (uintptr_t)j);
  }
  if (ptr_kind == 1 && world > 1 && world <= mkh::kMaxWorld && rank >= 0) peers[(rank + 1) % world] = nullptr;
  if (ptr_kind == 2 && world > 1 && world <= mkh::kMaxWorld && rank >= 0) outbox[(rank + 1) % world] = (void*)0x60000004;
  const mk_tiles::Shape& t = (m > 0 && m <= mk_tiles::kRedSkinnyMaxRows) ? mk_tiles::kRedSkinny : mk_tiles::kRedBig;
  mkh::RedPlan R{};
  ++g_calls;
  const int code = mkh::plan_reduce(ws, o, is_rs, P(0x70000000), P(0x71000000), m, n, k, world, rank,
                                    ptr_kind == 3 ? nullptr : peers, P(0x72000000), ptr_kind == 4 ? nullptr : outbox,
                                    t.bm, t.bn, t.waves(), t.ring_kib, &R);
  if (code != MK_OK) return;
  ++g_ok;
  CHECK(world >= 1 && world <= mkh::kMaxWorld && rank >= 0 && rank < world);
  CHECK(R.p_rows == (is_rs ? m / world : m) && R.p_rows % R.unit_rows == 0 && n % R.unit_cols == 0);
  CHECK((long long)R.unit_rows * R.unit_cols * 4 <= 1024LL * t.ring_kib * t.waves());
  CHECK((long long)R.n_units == (long long)(world - 1) * R.units_per_peer);
  CHECK(R.inbox_need <= ws.inbox_bytes);
  CHECK((size_t)R.n_units + (size_t)R.tiles_m * R.tiles_n <= ws.n_flags);
  CHECK((long long)R.tiles_m * t.bm >= m && (long long)R.tiles_n * t.bn >= n);
  CHECK(0 <= R.own_tile_begin && R.own_tile_begin < R.own_tile_end && R.own_tile_end <= R.tiles_m);
  check_roles(ws, R.n_copy, R.n_reduce, R.n_compute);
  if (R.assist) CHECK((size_t)mkh::kCtrBand0 + (size_t)(R.own_tile_end - R.own_tile_begin) * R.tiles_n <= ws.n_counters);
  CHECK(R.emulated ? R.n_order == R.n_units : R.n_order == 0);
}

// ---- MLP block --------------------------------------------------------------------------------
void mlp_case(const mkh::Ws& ws, const mkh::Opts* o, int world, int rank, int m_shard, int k, int n_up, int n_out) {
  const void* shards[mkh::kMaxWorld];
  const void* peers[mkh::kMaxWorld];
  void* outbox[mkh::kMaxWorld];
  for (int j = 0; j < mkh::kMaxWorld; ++j) {
    shards[j] = P(0x20000000 + 0x100000 * (uintptr_t)j);
    peers[j] = P(0x50000000 + 0x100000 * (uintptr_t)j);
    outbox[j] = (void*)(0x60000000 + 0x100000 * (uintptr_t)j);
  }
  const long long rows = (long long)world * m_shard;
  const mk_tiles::Shape& t = rows <= mk_tiles::kRedSkinnyMaxRows ? mk_tiles::kRedSkinny : mk_tiles::kRedBig;
  mkh::MlpPlan M{};
  ++g_calls;
  const int code = mkh::plan_mlp(ws, o, shards, world, rank, m_shard, k, P(0x30000000), n_up, P(0x31000000), n_out,
                                 peers, P(0x10000000), P(0x11000000), P(0x12000000), outbox, mk_tiles::kAg16.bm,
                                 mk_tiles::kAg16.bn, t.bm, t.bn, t.waves(), &M);
  if (code != MK_OK) return;
  ++g_ok;
  CHECK(M.ag.n_copy + M.ag.n_compute <= ws.grid && M.red.n_compute == ws.grid);
  CHECK(M.red.tiles_m == M.ag.tiles_m);  // a tile row of the down-projection is one row block of H
  CHECK((size_t)mkh::kCtrHready0 + (size_t)M.ag.tiles_m <= ws.n_counters);
  CHECK((size_t)mkh::kCtrBand0 + (size_t)(M.red.own_tile_end - M.red.own_tile_begin) * M.red.tiles_n <=
        (size_t)mkh::kCtrHready0);
}

// ---- ring attention ---------------------------------------------------------------------------
void ring_case(const mkh::Ws& ws, const mkh::Opts* o, int world, int rank, int heads, int s_local, int d, float scale,
               bool rings) {
  const void* ks[mkh::kMaxWorld];
  const void* vs[mkh::kMaxWorld];
  for (int j = 0; j < mkh::kMaxWorld; ++j) {
    ks[j] = P(0x20000000 + 0x100000 * (uintptr_t)j);
    vs[j] = P(0x30000000 + 0x100000 * (uintptr_t)j);
  }
  mkh::RaPlan A{};
  ++g_calls;
  const int code = mkh::plan_ring_attn(ws, o, P(0x10000000), ks, vs, world, rank, heads, s_local, d, scale,
                                       rings ? P(0x40000000) : nullptr, rings ? P(0x41000000) : nullptr,
                                       P(0x42000000), P(0x43000000), &A);
  if (code != MK_OK) return;
  ++g_ok;
  CHECK(d == mkh::kRaHeadDim && s_local % 128 == 0);
  CHECK((long long)A.n_items == (long long)heads * (s_local / 128));
  CHECK((size_t)A.n_units <= ws.n_flags);
  CHECK(A.scale > 0.f);
  check_roles(ws, A.n_copy, 0, A.n_compute);
  CHECK(A.emulated ? (long long)A.n_order == (long long)(world - 1) * heads * A.n_blk * 2 : A.n_order == 0);
}

// ---- MoE --------------------------------------------------------------------------------------
void moe_case(const mkh::Ws& ws, const mkh::Opts* o, int world, int t_local, int hidden, int n_experts, int top_k,
              int expert_begin, int n_local, int ffn, int capacity) {
  const void* toks[mkh::kMaxWorld];
  for (int j = 0; j < mkh::kMaxWorld; ++j) toks[j] = P(0x20000000 + 0x100000 * (uintptr_t)j);
  mkh::MoePlan M{};
  ++g_calls;
  const int code = mkh::plan_moe(ws, o, toks, world, t_local, hidden, P(0x30000000), P(0x31000000), n_experts, top_k,
                                 expert_begin, n_local, P(0x32000000), ffn, P(0x33000000), P(0x34000000),
                                 P(0x35000000), P(0x36000000), P(0x37000000), capacity, mk_tiles::kMoe.bm,
                                 mk_tiles::kMoe.bn, &M);
  if (code != MK_OK) return;
  ++g_ok;
  CHECK(top_k >= 1 && top_k <= 8 && n_local >= 1 && n_local <= 64);
  CHECK(expert_begin >= 0 && expert_begin + n_local <= n_experts);
  CHECK((long long)M.n_chunks * 64 == (long long)world * t_local);
  CHECK(2 + n_local + 1 <= 100);  // the misc counters stay below the other ops' fixed counters
  CHECK(M.off_chunk_cnt >= 128 && M.off_tile_cnt >= M.off_chunk_cnt + M.n_chunks * n_local);
  CHECK(M.counters_need <= ws.n_counters);
  CHECK((long long)M.max_mtiles * mk_tiles::kMoe.bm >= capacity);
  check_roles(ws, M.n_copy, 0, M.n_compute);
  CHECK(M.n_copy >= 1);
}

void edge_cases() {
  mkh::Ws ws{1u << 20, 1u << 20, 512ull << 20, 256};
  const int sizes[] = {0, -1, 1, 63, 64, 128, 192, 4096, 8192, 1 << 20, INT_MAX - 63, INT_MAX};
  for (int a : sizes)
    for (int b : sizes)
      for (int c : sizes) {
        for (int world : {0, 1, 3, 8, 9})
          for (int kind = 0; kind < 5; ++kind) ag_case(ws, nullptr, world, world > 1 ? 1 : 0, a, b, c, kind, 256, 256);
        for (int world : {1, 2, 8})
          for (int is_rs = 0; is_rs < 2; ++is_rs) red_case(ws, nullptr, is_rs, a, b, c, world, 0, 0);
        mlp_case(ws, nullptr, 8, 0, a, b, c, 4096);
        ring_case(ws, nullptr, 8, 0, a > 0 && a < 64 ? a : 8, b, 128, 0.f, true);
        moe_case(ws, nullptr, 8, a, b, 64, 2, 0, 8, c, a > 0 && a < (1 << 24) ? 2 * a : 4096);
      }
  // the workloads the bench times
  mkh::Opts o{};
  o.arrival_mode = MK_ARRIVAL_EMULATED;
  ag_case(ws, &o, 8, 0, 1024, 4096, 1792, 1, 256, 256);
  red_case(ws, &o, 1, 8192, 4096, 1792, 8, 0, 0);
  red_case(ws, &o, 0, 256, 8192, 1024, 8, 0, 0);
  mlp_case(ws, &o, 8, 0, 1024, 4096, 1792, 4096);
  ring_case(ws, &o, 8, 0, 8, 4096, 128, 0.f, true);
  moe_case(ws, &o, 8, 4096, 4096, 64, 2, 0, 8, 1536, 65536);
  CHECK(g_ok >= 6);
}

// Half the calls draw every argument from the wide distributions above (mostly rejected: they
// exercise validation); the other half draw sizes the kernels take and default workspaces (mostly
// accepted: they exercise the plans' invariants).
void random_cases(long long n) {
  Rng r{12345};
  for (long long i = 0; i < n; ++i) {
    const bool plausible = (i & 1) != 0;
    mkh::Ws ws = plausible ? mkh::Ws{1u << 20, 1u << 20, 512ull << 20, r.below(4) ? 256 : r.small(16, 304)}
                           : random_ws(r);
    bool use = false;
    mkh::Opts o = random_opts(r, &use);
    if (plausible && r.below(2)) use = false;
    const mkh::Opts* po = use ? &o : nullptr;
    const int world = plausible ? r.small(1, 8) : r.small(-1, 9);
    const int rank = plausible ? r.below(world) : r.small(-1, 8);
    auto sz = [&]() { return plausible ? r.good() : r.size(); };
    ag_case(ws, po, world, rank, sz(), sz(), sz(), plausible ? r.below(2) : r.below(5), r.below(4) ? 256 : 128, 256);
    red_case(ws, po, r.below(2), plausible ? world * r.good() : r.size(), sz(), sz(), world, rank,
             plausible ? 0 : r.below(5));
    mlp_case(ws, po, world, rank, sz(), sz(), sz(), sz());
    const float scales[] = {0.f, 0.125f, -1.f, 1e30f, INFINITY, NAN};
    ring_case(ws, po, world, rank, plausible ? r.small(1, 16) : r.small(-1, 64), sz(),
              plausible || r.below(4) ? 128 : r.size(), scales[plausible ? r.below(2) : r.below(6)], r.below(4) != 0);
    const int ne = plausible ? 4 * r.small(1, 64) : (r.below(4) ? 64 : r.small(-4, 1100));
    const int nl = plausible ? r.small(1, ne < 64 ? ne : 64) : r.small(-1, 70);
    const int eb = plausible ? r.below(ne - nl + 1) : r.small(-2, 70);
    const int tl = plausible ? 64 * r.small(1, 128) : r.size();
    moe_case(ws, po, world, tl, plausible ? 64 * r.small(1, 64) : r.size(), ne,
             plausible ? r.small(1, ne < 8 ? ne : 8) : r.small(-1, 9), eb, nl, sz(),
             plausible ? world * tl * 2 : (r.below(3) ? r.size() : r.small(-5, 70000)));
  }
}

}  // namespace

int main(int argc, char** argv) {
  const long long n = argc > 1 ? atoll(argv[1]) : 200000;
  edge_cases();
  random_cases(n);
  printf("%lld planner calls, %lld accepted: ok\n", g_calls, g_ok);
  return 0;
}
