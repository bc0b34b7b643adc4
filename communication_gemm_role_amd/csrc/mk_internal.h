// Internal interface between the C-ABI host layer and the kernel translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#define MK_MAX_WORLD 8

struct mk_ctx {
  int device;
  int n_cu;
  char* ws;         // one device allocation, carved below
  size_t ws_bytes;
  int* status;      // device status word (first fault wins)
  uint32_t* counters;  // zero-initialised counters, left zeroed by every kernel that uses them
  size_t n_counters;
  uint32_t* flags;  // epoch-tagged ready flags
  size_t n_flags;
  char* inbox;      // landing buffer for emulated peer partials (RS/AR)
  size_t inbox_bytes;
  uint32_t epoch;   // call number; a flag is up when it equals the current epoch
};

namespace mk {

// Context counters: every kernel leaves each counter it wrote at zero when its last workgroup
// exits, so operations can share one context without a reset in between.  Layout:
//   [0, 2 + n_local]   MoE: route-done, exits, m-tile base per local expert (n_local <= 64)
//   [101]              MoE: next leftover grouped-GEMM tile
//   [110, 125]         AllGather+GEMM, RS/AR, MLP and ring-attention claims and exit counts (below)
//   [128, ...)         per-call tables: RS band counters (one per owned tile); MoE per-chunk counts,
//                      m-tile row counters, chunk row totals and arrival-position prefix
//   [4096, ...)        MLP: tiles stored per 256-row block of H
constexpr int CTR_AG_TILE = 110;   // next leftover AG tile
constexpr int CTR_AG_EXIT = 111;   // AG workgroups that have exited
constexpr int CTR_RED_TILE = 112;  // next leftover RS/AR tile
constexpr int CTR_RED_EXIT = 113;  // RS/AR workgroups that have exited
constexpr int CTR_RED_PRESUM = 114;  // next RS pre-sum job (64-row band of an owned tile)
constexpr int CTR_RED_BAND0 = 128;   // RS: bands pre-summed per owned tile, [own tiles] from here
constexpr int CTR_MLP_EXIT = 115;    // MLP workgroups that have exited
constexpr int CTR_MLP_HREADY0 = 4096;  // MLP: up-projection tiles stored per 256-row block of H
constexpr int CTR_RA_XITEM0 = 118;  // next leftover ring-attention item of each XCD's block, [8] from here
constexpr int CTR_RA_EXIT = 117;  // ring-attention workgroups that have exited
constexpr int CTR_RA_LANDED = 126;  // ring-attention copy workgroups that have landed all their blocks
constexpr int RA_D = 128;         // ring attention: head dimension

struct AgParams {
  const uint16_t* shards[MK_MAX_WORLD];
  const uint16_t* b;
  uint16_t* ag;
  float* c;
  const int32_t* order;
  uint32_t* flags;
  uint32_t* counters;  // context counters (CTR_AG_*)
  int* status;
  int world, rank, m_shard, m, n, k;
  int unit_rows, unit_cols, n_ucols, n_urows;
  int n_copy, n_compute;
  int emulated, local_in_place;
  int n_order, drop_pos;
  int tiles_m, tiles_n;
  uint32_t epoch;
  uint64_t timeout_ticks;
  uint64_t* trace;  // per-workgroup trace records, or nullptr
  uint64_t pace_q16;  // copy role: wall-clock ticks per arrival position, Q16 (0: unpaced)
  // MLP up-projection (the MLP kernel only): the epilogue stores H = bf16(gelu(acc)) instead of
  // C and adds one to h_ready[tile row] once a tile's stores have completed
  uint16_t* h;
  uint32_t* h_ready;
  // when set, the last workgroup out moves the status word here and clears it (the call without a
  // context reports device faults through a caller-owned output instead of mk_ctx_status)
  int* status_out;
};

struct RedParams {
  const uint16_t* a;
  const uint16_t* b;
  const float* peers[MK_MAX_WORLD];  // resident peer partials (indexed by rank)
  float* outbox[MK_MAX_WORLD];       // RS only (indexed by rank)
  float* out;                        // RS: owned slice; AR: full output
  float* inbox;                      // EMULATED: landing area, (world-1) partials back to back
  const int32_t* order;
  uint32_t* flags;                   // landing flags [n_units], then presum flags [tiles]
  uint32_t* presum_flags;
  uint32_t* counters;                // context counters (CTR_RED_*)
  int* status;
  int is_rs;
  int m, n, k, world, rank, m_slice;
  int p_rows;                        // rows of one peer partial (RS: m_slice, AR: m)
  int unit_rows, unit_cols, n_ucols, units_per_peer;
  int n_copy, n_reduce, n_compute;
  int assist;                        // RS without reduce workgroups: compute workgroups pre-sum
  int emulated, n_order, drop_pos;
  int tiles_m, tiles_n;
  int own_tile_begin, own_tile_end;  // tile rows overlapping the owned slice (RS) or all (AR)
  uint32_t epoch;
  uint64_t timeout_ticks;
  uint64_t* trace;  // per-workgroup trace records, or nullptr
  uint64_t pace_q16;  // copy role: wall-clock ticks per arrival position, Q16 (0: unpaced)
  // A produced in the same launch (the MLP kernel's H): a tile of tile row tm waits until
  // a_ready[tm] >= a_ready_need before its K loop; nullptr when A is an input
  const uint32_t* a_ready;
  uint32_t a_ready_need;
};

// MLP block (up-projection with AllGather, activation, down-projection with ReduceScatter) in one
// launch: the AllGather+GEMM roles produce H, then every workgroup runs the GEMM+RS compute role
// on it.
struct MlpParams {
  AgParams ag;
  RedParams red;
};

struct MoeParams {
  const uint16_t* tokens[MK_MAX_WORLD];
  const float* logits;
  const float* bias;
  const uint16_t* w_up;
  int32_t* topk_idx;
  int32_t* seg_offsets;
  int32_t* seg_token;
  uint16_t* x_seg;
  float* y;
  const int32_t* order;
  uint32_t* counters;  // [0] route-done, [1] exit count, [2..] per-chunk counts and m-tile counts
  uint32_t* flags;     // [0] scan-ready flag
  int* status;
  int world, t_local, hidden, n_experts, top_k, expert_begin, n_local, ffn, capacity;
  int n_tokens, n_chunks;
  int n_route, n_copy, n_compute;  // roles (route is done by every workgroup first)
  int emulated, drop_pos;
  int tiles_n, max_mtiles;         // grouped-GEMM tiling: n-tiles per expert, bound on m-tiles
  uint32_t epoch;
  uint64_t timeout_ticks;
  uint64_t* trace;  // per-workgroup trace records, or nullptr
  // counter layout (offsets into `counters`)
  int off_chunk_cnt;   // [n_chunks * n_local] per-chunk routed counts
  int off_tile_cnt;    // [max_mtiles] rows landed per global m-tile
  int off_chunk_rows;  // [n_chunks] routed rows (all local experts) per chunk
  int off_pos_pre;     // [n_chunks + 1] rows of the arrival positions before each, in arrival order
  int off_misc;        // [0] route done, [1] exit count
};

// Ring attention, one rank's share: queries [heads, s_local, 128] against every rank's K/V shard.
struct RaParams {
  const uint16_t* q;                     // [heads, s_local, d]
  const uint16_t* k_src[MK_MAX_WORLD];   // rank j's K shard [heads, s_local, d] (peers: copy sources)
  const uint16_t* v_src[MK_MAX_WORLD];
  uint16_t* k_ring;                      // EMULATED: landing buffers [world, heads, s_local, d]
  uint16_t* v_ring;
  float* out;                            // [heads, s_local, d]
  float* lse;                            // [heads, s_local] or nullptr
  const int32_t* order;
  uint32_t* flags;                       // one per K or V block of every rank: [world * heads * n_blk * 2]
  uint32_t* counters;
  int* status;
  float scale_log2;                      // softmax scale times log2(e)
  int world, rank, heads, s_local;
  int n_blk, n_qt, n_items, n_units;     // 64-key blocks per shard, 128-query tiles, items, flag slots
  int n_copy, n_compute, emulated, n_order, drop_pos;
  uint32_t epoch;
  uint64_t timeout_ticks;
  uint64_t* trace;
  uint64_t pace_q16;
};

// Launchers (stream-ordered; return hipError_t of the launch)
hipError_t launch_ag_gemm(const AgParams& p, int grid, hipStream_t s);
hipError_t launch_gemm_reduce(const RedParams& p, int grid, hipStream_t s);
hipError_t launch_moe(const MoeParams& p, int grid, hipStream_t s);
hipError_t launch_mlp(const MlpParams& p, int grid, hipStream_t s);
hipError_t launch_ring_attn(const RaParams& p, int grid, hipStream_t s);
hipError_t launch_fill_u32(uint32_t* p, uint32_t v, size_t n, hipStream_t s);

// Tile sizes the host needs for scheduling and validation
int ag_tile_m();
int ag_tile_n();
int mlp_tile_m();  // the MLP block's up-projection tile
int mlp_tile_n();
int red_tile_m(int m, int n);
int red_tile_n(int m, int n);
int red_tile_waves(int m, int n);
int red_ring_kib(int m, int n);  // KiB per wave and batch of the copy ring (bounds the landing unit)
int moe_tile_m();
int moe_tile_n();

}  // namespace mk
