/*
 * mk.h — C ABI of the fused communication+GEMM library for one MI355X (gfx950).
 *
 * One GPU's share of four persistent, role-specialised fused ops, as the mKernel
 * write-up describes them (page "mKernel：多GPU、多节点融合内核库，实现GPU驱动通信",
 * news.chathome.org; section "五种融合内核", the five-fused-kernels table, and
 * section "mKernel的功能" on persistent kernels whose CTAs self-assign the roles
 * compute / intra-node comm / send / reduce, with a per-shape number of SMs per role):
 *
 *   mk_ag_gemm            AllGather + GEMM
 *   mk_gemm_rs            GEMM + ReduceScatter
 *   mk_gemm_ar            GEMM + AllReduce
 *   mk_moe_dispatch_gemm  MoE token dispatch + per-expert grouped GEMM
 *
 * the fifth row of the same table (Ring Attention):
 *
 *   mk_ring_attention     ring K/V exchange + FlashAttention (sequence parallel)
 *
 * from the same page's roadmap section (the transformer-layer megakernel as the next step), the
 * MLP block built from two of the fused ops in one launch:
 *
 *   mk_mlp_ag_rs          AllGather + up-projection GEMM, gelu, down-projection GEMM + ReduceScatter
 *
 * and, from section "mKernel的功能" (the number of SMs per role is chosen per shape), the tuners:
 *
 *   mk_*_tune             time candidate role splits of an operation and report the fastest
 *
 * Each call is ONE kernel launch.  Inside it, workgroups take a role from their
 * id and a per-shape split: copy (lands peer data in a given order and raises a
 * per-unit ready flag), compute (bf16 MFMA tiles with fp32 accumulation, which
 * consume a unit the moment its flag is up) and reduce (folds peer partials into
 * output tiles).  Peers are emulated on the one GPU: their shards and partials
 * are ordinary device buffers, and "arrival" is the copy role writing them into
 * the landing buffers in the caller's order.
 *
 * Conventions
 *   - bf16 travels as uint16_t raw bits; fp32 as float.  All matrices are dense,
 *     row-major, with the leading dimension equal to the column count.
 *   - Every matrix pointer is a DEVICE pointer, 16-byte aligned.  Per-rank pointer
 *     arrays (a_shards, peer_partials, outbox, tokens) are HOST arrays of length
 *     `world`, indexed by rank; the entry at `rank` is unused for peer-only arrays.
 *   - `stream` is a hipStream_t (NULL = the default stream).
 *   - The caller owns every buffer; the library never allocates or frees caller
 *     memory.  Buffers must stay alive until the stream work has completed.
 *   - Outputs must not alias inputs, except that a_shards[rank] may point at its
 *     own rows inside a_gathered (then the local shard is already in place).
 *   - Calls are asynchronous: argument errors return synchronously; faults seen
 *     on the device (a wait that timed out, a capacity overflow) are recorded in
 *     the context and returned by mk_ctx_status().
 *   - A context is bound to one device and is not thread-safe; calls that share a
 *     context must be issued to one stream (they share flags and counters).
 */
#ifndef MK_H_
#define MK_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes ---------------------------------------------------------------- */
#define MK_OK 0
#define MK_ERR_INVALID_ARG (-1)  /* null pointer, size <= 0, world not in [1,8], rank not in [0,world),
                                    rows not divisible by world (RS), top_k > n_experts, bad expert range */
#define MK_ERR_UNSUPPORTED (-2)  /* a dimension not a multiple of 64 (hidden/ffn/k/n/m as stated per call),
                                    a pointer not 16-byte aligned, a unit size the kernels do not take */
#define MK_ERR_WORKSPACE (-3)    /* the context workspace is too small for this call */
#define MK_ERR_HIP (-4)          /* a HIP runtime call or kernel launch failed */
#define MK_ERR_TIMEOUT (-5)      /* device: a wait for a flag or counter exceeded opts.timeout_us */
#define MK_ERR_CAPACITY (-6)     /* device: routed rows exceeded capacity_rows (nothing past it was written) */

/* ---- arrival emulation --------------------------------------------------------- */
#define MK_ARRIVAL_RESIDENT 1 /* every operand is already in place; no copy role runs */
#define MK_ARRIVAL_EMULATED 2 /* copy-role workgroups land peer data in `arrival_order` */

typedef struct mk_ctx mk_ctx;

/* Options; pass NULL for defaults.  Zero in any field means "default". */
typedef struct mk_opts {
  int n_copy_wg;      /* workgroups that start in the copy role (0: per-shape default) */
  int n_compute_wg;   /* workgroups in the compute role (0: all the rest)             */
  int n_reduce_wg;    /* workgroups in the reduce role, RS/AR only (0: per-shape default) */
  int arrival_mode;   /* MK_ARRIVAL_RESIDENT or MK_ARRIVAL_EMULATED (0: EMULATED)         */
  const int32_t* arrival_order; /* DEVICE int32 array, the order in which units land (see each
                                   call); NULL in EMULATED mode = identity order              */
  int arrival_len;    /* number of entries in arrival_order (must equal the call's unit count) */
  int arrival_unit_rows; /* AG and RS/AR landing unit, rows (64 or 128; 0: per-shape default)  */
  int arrival_unit_cols; /* AG and RS/AR landing unit, cols (64 or 128; 0: per-shape default)  */
  int arrival_chunk_tokens; /* MoE: tokens per arrival chunk; only 64 is supported (0: 64)    */
  int64_t timeout_us; /* bound on every device-side wait (0: 2 000 000 us)                     */
  int test_drop_unit; /* testing: position in arrival_order that the copy role skips, so the
                         consumer of that unit must time out (-1 or 0 = none; values are
                         1-based positions)                                                   */
  uint64_t* trace;    /* DEVICE array of mk_ctx_grid(ctx) * 8 uint64, or NULL (no tracing).
                         When set, thread 0 of every workgroup of the call writes its record
                         i * 8 + [0..7] (i = workgroup id; workgroups the call does not launch
                         are left untouched):
                           [0] wall-clock ticks (100 MHz) at start  [1] shader cycles at start
                           [2] wall-clock ticks at end             [3] shader cycles at end
                           [4] role: 0 copy, 1 compute, 2 reduce
                           [5] [6] [7] phase marks in wall-clock ticks, 0 when not reached:
                             AG, RS/AR copy: [5] its last unit's flag raised
                             AG, RS/AR compute: [5] first tile's first operands ready;
                               RS/AR also [6] first tile's K loop done (its epilogue follows)
                               and [7] first leftover tile claimed (after any pre-sum jobs)
                             RS/AR reduce: [5] its last pre-sum flag raised
                             MoE copy: [5] routing done, [6] scan flag seen, [7] its last
                               dispatched rows counted (before it joins the leftover tiles)
                             MoE compute: [5] first tile's rows all landed
                         The caller owns the array; it must stay alive until the call's
                         stream work completes.                                               */
  double arrival_gbps; /* EMULATED AG, RS/AR and MLP landing: the rank's total inbound link rate
                         in GB/s (1e9 bytes/s).  Arrival position i of the order (i = 0, 1, ...)
                         is not copied before i * unit_bytes / rate after the copy workgroup
                         starts, so units land at that rate instead of as fast as the copy
                         role can move them (a copy workgroup moves 8 KiB per wave at a time,
                         e.g. two 128x128 bf16 units; such a batch starts at its later unit's
                         time, so its earlier unit lands up to n_copy positions late); 7 links x 153 GB/s = 1071 models one MI355X's
                         xGMI links (section "mKernel的功能" of the news.chathome.org page: the
                         intra-node leg runs over the peer links while the GEMM computes).
                         0: unpaced.  Negative, non-finite, or so low that the whole order would
                         take more than half of timeout_us: MK_ERR_INVALID_ARG.  Ignored in
                         RESIDENT mode and by MoE.  Ring attention: unit_bytes = 16 KiB.       */
} mk_opts;

/* ---- context ------------------------------------------------------------------------ */
/* Creates a context on `device` with a workspace of `workspace_bytes` device bytes (0: 512 MiB),
 * allocated once here; no later call allocates.  The workspace holds ready flags, counters, the
 * status word and, in EMULATED RS/AR, the landing inbox for peer partials.
 * Returns MK_OK and sets *out, or an error code (*out untouched). */
int mk_ctx_create(int device, size_t workspace_bytes, mk_ctx** out);
/* Frees the workspace.  The caller must have synchronised every stream that used the context. */
int mk_ctx_destroy(mk_ctx* ctx);
/* Synchronises `stream`, then returns and clears the device status word: MK_OK, MK_ERR_TIMEOUT
 * or MK_ERR_CAPACITY (the first fault recorded since the last call of mk_ctx_status). */
int mk_ctx_status(mk_ctx* ctx, void* stream);
/* After a fault: clears flags, counters and the status word on `stream` and restarts the epoch. */
int mk_ctx_reset(mk_ctx* ctx, void* stream);
/* Co-resident workgroup count the persistent kernels launch with on this device. */
int mk_ctx_grid(mk_ctx* ctx);
const char* mk_strerror(int code);

/* Self-test of the cross-workgroup handshake every role relies on: producer workgroups write a
 * payload with write-through stores and then raise a relaxed agent-scope flag; consumer workgroups
 * on other XCDs poll the flag and read the payload.  `pairs` producer/consumer pairs exchange
 * `rounds` payloads.  mode 0: fresh payload addresses every round, ordinary consumer loads (the
 * kernels' pattern: a payload is written once per launch and never read before its flag);
 * mode 1: the same addresses every round, device-coherent consumer loads; mode 2: the same
 * addresses with ordinary loads (diagnostic only: another XCD's L2 may hold a stale copy).
 * Modes 3-5 use fresh addresses and the kernels' own load paths: mode 3, the consumer reads the
 * payload by a buffer load straight into LDS (as the compute role stages its operands); mode 4,
 * the producer also lands it as the copy role does (non-temporal buffer load of a source unit
 * into LDS, then write-through stores); mode 5, the producer publishes by a counter increment
 * and the consumer waits for the count before its LDS load (the MoE m-tile handshake).
 * Allocates and frees its own device memory and synchronises the device.  Returns MK_OK with
 * *mismatches = payload words that did not match and *timeouts = 1 if a wait hit the 2 s watchdog;
 * MK_ERR_INVALID_ARG for mode not in [0,5], pairs not in [1,128], rounds < 1, or
 * pairs*rounds > 262144 with fresh addresses (131072 in mode 4); MK_ERR_HIP on a runtime failure. */
int mk_selftest_flags(int device, int mode, int pairs, int rounds, int64_t* mismatches, int64_t* timeouts);

/* ---- AllGather + GEMM ----------------------------------------------------------------
 * Five-fused-kernels table, AllGather + GEMM row: c = [A_0; ...; A_{world-1}] @ b with A_r the row
 * shard of rank r; a K-unit of a tile's rows is multiplied as soon as it has landed.
 *   a_shards[r]  [m_shard, k] bf16, r in [0, world)     (host array of device pointers)
 *   b            [k, n] bf16 (the local, fully resident operand)
 *   a_gathered   [world*m_shard, k] bf16, OUT: shard r lands at rows [r*m_shard, (r+1)*m_shard)
 *   c            [world*m_shard, n] fp32, OUT: c = a_gathered @ b
 * Arrival units are unit_rows x unit_cols blocks of a_gathered, numbered row-major over the unit
 * grid (id = unit_row * (k/unit_cols) + unit_col).  In EMULATED mode arrival_order lists the ids
 * of every unit that must be copied: all units of the peers' shards, plus those of the local
 * shard when a_shards[rank] is not already in place.  In RESIDENT mode a_gathered must already
 * hold every shard and a_shards may be NULL.
 * Sizes: m_shard, k, n multiples of 64; m_shard a multiple of unit_rows, k of unit_cols. */
int mk_ag_gemm(mk_ctx* ctx, void* stream, const uint16_t* const* a_shards, int world, int rank, int m_shard,
               int k, const uint16_t* b, int n, uint16_t* a_gathered, float* c, const mk_opts* opts);

/* ---- AllGather + GEMM without allocation ------------------------------------------------
 * For callers that cannot allocate device memory or create a context: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same operation, arguments
 * and options as mk_ag_gemm, on the CURRENT device, with no context: the ready flags, counters and
 * status word live in a static device array of the library (66 KiB per device, held until the
 * process ends), set up on the first call on a device.  No call allocates or frees memory.
 *   status   DEVICE int, OUT (4-byte aligned, not NULL): when the kernel ends it holds MK_OK,
 *            MK_ERR_TIMEOUT (a wait hit opts.timeout_us) -- the codes mk_ctx_status would return
 * Limits: at most 16384 arrival units ((world*m_shard/unit_rows) * (k/unit_cols)); more return
 * MK_ERR_WORKSPACE.  Every call on a device shares that device's array: calls must be ordered on
 * one stream (or synchronised); calls that overlap on one GPU race.  Argument errors return
 * synchronously as for mk_ag_gemm; MK_ERR_HIP if the device array cannot be set up or the launch
 * fails. */
int mk_ag_gemm_noalloc(void* stream, const uint16_t* const* a_shards, int world, int rank, int m_shard, int k,
                       const uint16_t* b, int n, uint16_t* a_gathered, float* c, int* status, const mk_opts* opts);

/* ---- GEMM + ReduceScatter -------------------------------------------------------------
 * Five-fused-kernels table, GEMM + ReduceScatter row: the sum over ranks of the partials A_j @ B_j,
 * each rank receiving only its own row slice of it; a tile of this rank's partial is added in or
 * sent on right after its K loop.  Rank j owns rows
 * [j*m/world, (j+1)*m/world).  This call is rank `rank`'s share:
 *   a [m, k] bf16, b [k, n] bf16                 local operands; P = a @ b is this rank's partial
 *   peer_partials[j] [m/world, n] fp32, j != rank  peer j's partial of THIS rank's slice
 *   owned_out [m/world, n] fp32, OUT            P[own slice] + sum_j peer_partials[j]
 *   outbox[j] [m/world, n] fp32, j != rank, OUT  P[slice j] (this rank's unreduced partial of
 *                                               j's slice, for owner j to sum)
 * EMULATED mode: peer partials first land, unit by unit in arrival_order, in an inbox inside the
 * context workspace (units are unit_rows x unit_cols blocks of one peer partial; id =
 * peer_index * units_per_partial + unit, peers indexed 0..world-2 in ascending rank skipping
 * `rank`); the reduction consumes each unit once its flag is up.  RESIDENT mode reads them in place.
 * Sizes: m, n, k multiples of 64; m/world a multiple of 64 and of unit_rows; n of unit_cols. */
int mk_gemm_rs(mk_ctx* ctx, void* stream, const uint16_t* a, const uint16_t* b, int m, int n, int k, int world,
               int rank, const float* const* peer_partials, float* owned_out, float* const* outbox,
               const mk_opts* opts);

/* ---- GEMM + AllReduce -----------------------------------------------------------------
 * Five-fused-kernels table, GEMM + AllReduce row: every rank receives the whole sum over ranks of
 * the partials A_j @ B_j; a tile of this rank's partial is added in right after its K loop.
 *   a [m, k] bf16, b [k, n] bf16; peer_partials[j] [m, n] fp32 for j != rank
 *   out [m, n] fp32, OUT: a @ b + sum_j peer_partials[j]
 * Landing units and modes as in mk_gemm_rs, over [m, n] partials.
 * Sizes: m, n, k multiples of 64; m a multiple of unit_rows, n of unit_cols. */
int mk_gemm_ar(mk_ctx* ctx, void* stream, const uint16_t* a, const uint16_t* b, int m, int n, int k, int world,
               int rank, const float* const* peer_partials, float* out, const mk_opts* opts);

/* ---- MoE dispatch + grouped GEMM ------------------------------------------------------
 * Five-fused-kernels table, MoE Dispatch + GEMM row: route every token to its top_k experts, gather
 * the rows routed to each local expert into one segment and multiply the segment by that
 * expert's weight, in one launch (each token row lands directly in its final slot).  This call is the share of the
 * rank that owns experts [expert_begin, expert_begin + n_local_experts):
 *   tokens[r] [t_local, hidden] bf16, r in [0, world); global token id g = r*t_local + i
 *   logits [world*t_local, n_experts] fp32; bias [n_experts] fp32
 *   score = fp32(logit + bias); each token picks the top_k experts by descending score, equal
 *   scores going to the lower expert id.
 *   w_up [n_local_experts, hidden, ffn] bf16
 *   topk_idx [world*t_local, top_k] int32, OUT: every token's experts, in descending score
 *   seg_offsets [n_local_experts+1] int32, OUT: exclusive prefix sum of the local experts' row
 *               counts; seg_offsets[n_local_experts] = R, the routed row count
 *   seg_token [capacity_rows] int32, OUT: rows [seg_offsets[e], seg_offsets[e+1]) list, in
 *               ascending global id, the tokens routed to local expert e
 *   x_seg [capacity_rows, hidden] bf16, OUT: x_seg[i] = token seg_token[i] (bitwise)
 *   y [capacity_rows, ffn] fp32, OUT: y[segment e] = x_seg[segment e] @ w_up[e]
 * Rows at and past R are not written.  EMULATED mode lands tokens by 64-token chunks (chunk id =
 * g / 64) in arrival_order (length world*t_local/64); RESIDENT mode has no order (the same copy
 * runs in identity order).  If R > capacity_rows, the status becomes MK_ERR_CAPACITY and rows
 * past capacity_rows are dropped.
 * Sizes: t_local a multiple of 64, hidden and ffn multiples of 64, top_k in [1, 8],
 * n_experts <= 1024, n_local_experts <= 64. */
int mk_moe_dispatch_gemm(mk_ctx* ctx, void* stream, const uint16_t* const* tokens, int world, int t_local,
                         int hidden, const float* logits, const float* bias, int n_experts, int top_k,
                         int expert_begin, int n_local_experts, const uint16_t* w_up, int ffn, int32_t* topk_idx,
                         int32_t* seg_offsets, int32_t* seg_token, uint16_t* x_seg, float* y, int capacity_rows,
                         const mk_opts* opts);

/* ---- MLP block: AllGather + GEMM, gelu, GEMM + ReduceScatter ---------------------------
 * Roadmap section of the same page (the transformer-layer megakernel) built from the AllGather +
 * GEMM and GEMM + ReduceScatter rows of the five-fused-kernels table, in ONE launch: the
 * column-parallel up-projection consumes A tiles as they land, its epilogue applies the
 * activation, and the row-parallel down-projection starts on each 256-row block of H as soon as
 * that block is complete, reducing each output tile with the peers' partials.  Rank `rank`'s share:
 *   a_shards[r] [m_shard, k] bf16, a_gathered [world*m_shard, k] bf16 OUT   as in mk_ag_gemm
 *   b_up [k, n_up] bf16, b_down [n_up, n_out] bf16      the local weights
 *   h [world*m_shard, n_up] bf16, OUT                   h = bf16(gelu(a_gathered @ b_up)), gelu(x) =
 *                                                       x * Phi(x) = x (1 + erf(x / sqrt 2)) / 2, in
 *                                                       fp32, rounded to nearest even
 *   peer_partials[j] [m_shard, n_out] fp32, j != rank   peer j's partial of THIS rank's rows of the
 *                                                       down-projection, resident
 *   owned_out [m_shard, n_out] fp32, OUT                (h @ b_down)[own rows] + sum_j peer_partials[j]
 *   outbox[j] [m_shard, n_out] fp32, j != rank, OUT     (h @ b_down)[rows of rank j]
 * The arrival mode, order and units apply to A as in mk_ag_gemm; the role split (n_copy_wg,
 * n_compute_wg) to the up-projection, after which every workgroup works on the down-projection.
 * Sizes: as mk_ag_gemm for (m_shard, k, n_up) and as mk_gemm_rs for (world*m_shard, n_out, n_up),
 * with world*m_shard > 512 (256-row tiles in both phases).  Trace records: marks [5] as
 * mk_ag_gemm, [6] the workgroup's up-projection work done. */
int mk_mlp_ag_rs(mk_ctx* ctx, void* stream, const uint16_t* const* a_shards, int world, int rank, int m_shard, int k,
                 const uint16_t* b_up, int n_up, const uint16_t* b_down, int n_out, const float* const* peer_partials,
                 uint16_t* a_gathered, uint16_t* h, float* owned_out, float* const* outbox, const mk_opts* opts);

/* ---- Ring attention ------------------------------------------------------------------
 * Five-fused-kernels table, Ring Attention row: sequence-parallel attention of this rank's queries
 * over every rank's keys and values, the peers' K/V blocks travelling round the ring and each
 * block attended to once it is present, in one launch.  Rank `rank`'s share, no mask:
 *   q [heads, s_local, head_dim] bf16                  this rank's queries
 *   k_shards[j], v_shards[j] [heads, s_local, head_dim] bf16, j in [0, world): every rank's keys
 *                         and values (entry `rank` is this rank's own, read in place)
 *   out [heads, s_local, head_dim] fp32, OUT           out[h,i] = sum_t softmax_t(scale * q[h,i].k[h,t]) v[h,t]
 *                         over the world*s_local keys t of all ranks (rank order; the order does
 *                         not change the result beyond fp32 rounding)
 *   lse [heads, s_local] fp32, OUT or NULL             natural log of sum_t exp(scale * q[h,i].k[h,t])
 *   softmax_scale                                       0: 1/sqrt(head_dim); otherwise finite, > 0
 *   k_ring, v_ring [world, heads, s_local, head_dim] bf16, OUT (EMULATED, world > 1): the ring's
 *                         landing buffers; slot j receives rank j's shard (slot `rank` untouched)
 * EMULATED mode lands peers' blocks of 64 keys (K and V separately, 16 KiB each): unit id
 * ((j*heads + h)*(s_local/64) + b)*2 + (0 for K, 1 for V) for rank j != rank; arrival_order, if
 * given, lists those (world-1)*heads*(s_local/64)*2 ids; NULL = the ring's order (step t = 1,
 * 2, ... brings rank (rank - t) mod world, each step head by head, block by block, K before V).
 * RESIDENT mode reads every shard in place.  arrival_gbps paces the ring (see mk_opts).
 * Sizes: head_dim 128, s_local a multiple of 128; world*heads*s_local*head_dim*2 < 4 GiB.
 * Trace records: copy [5] as mk_ag_gemm; compute [5] first item started. */
int mk_ring_attention(mk_ctx* ctx, void* stream, const uint16_t* q, const uint16_t* const* k_shards,
                      const uint16_t* const* v_shards, int world, int rank, int heads, int s_local, int head_dim,
                      float softmax_scale, uint16_t* k_ring, uint16_t* v_ring, float* out, float* lse,
                      const mk_opts* opts);

/* ---- role-split tuning -------------------------------------------------------------------
 * Section "mKernel的功能" of the news.chathome.org page: the number of SMs given to each role is
 * chosen per shape.  These calls time the matching operation once per candidate number of copy
 * workgroups (mk_opts.n_copy_wg; 0 = the per-shape default) with every other option as given --
 * in particular arrival_mode, arrival_order and arrival_gbps, since the best split depends on the
 * link rate -- and report the fastest.  Arguments before `opts` are those of the operation; its
 * outputs are overwritten by the timed calls (they end holding the last candidate's result).
 *   n_copy_candidates[n_candidates]  host array of splits to try
 *   reps                             timed calls per candidate, after two untimed ones
 *   us_per_call[n_candidates]        host array, OUT: mean microseconds per call between two events
 *                                    on `stream`; -1 where the planner rejects the candidate
 *   best_n_copy                      host, OUT: the fastest candidate
 * Returns MK_OK if at least one candidate ran; the planner's code if every candidate was rejected;
 * the first HIP error or device status (e.g. MK_ERR_TIMEOUT) otherwise, after which the results
 * are undefined.  Synchronises `stream` once per candidate. */
int mk_ag_gemm_tune(mk_ctx* ctx, void* stream, const uint16_t* const* a_shards, int world, int rank, int m_shard,
                    int k, const uint16_t* b, int n, uint16_t* a_gathered, float* c, const mk_opts* opts,
                    const int* n_copy_candidates, int n_candidates, int reps, float* us_per_call, int* best_n_copy);
int mk_gemm_rs_tune(mk_ctx* ctx, void* stream, const uint16_t* a, const uint16_t* b, int m, int n, int k, int world,
                    int rank, const float* const* peer_partials, float* owned_out, float* const* outbox,
                    const mk_opts* opts, const int* n_copy_candidates, int n_candidates, int reps,
                    float* us_per_call, int* best_n_copy);
int mk_gemm_ar_tune(mk_ctx* ctx, void* stream, const uint16_t* a, const uint16_t* b, int m, int n, int k, int world,
                    int rank, const float* const* peer_partials, float* out, const mk_opts* opts,
                    const int* n_copy_candidates, int n_candidates, int reps, float* us_per_call, int* best_n_copy);

#ifdef __cplusplus
}
#endif
#endif /* MK_H_ */
