// GEMM + ReduceScatter and GEMM + AllReduce, one rank's share, as one persistent launch (roles in
// mk_red_roles.hpp).
//
// Operations (mKernel write-up, news.chathome.org page, five-fused-kernels table, GEMM +
// AllReduce and GEMM + ReduceScatter rows): rank j holds a partial P_j = A_j @ B_j of the same
// [M, N] output.  AllReduce: every rank ends with sum_j P_j.  ReduceScatter: rank r ends with
// sum_j P_j on its own row slice only.  A tile of P enters the reduction right after its K loop,
// inside the same launch.
#include <type_traits>
#include "mk_red_roles.hpp"

namespace mk {

int red_tile_m(int m, int n) { return red_skinny(m, n) ? RedSkinny::BM : RedBig::BM; }
int red_tile_n(int m, int n) { return red_skinny(m, n) ? RedSkinny::BN : RedBig::BN; }
int red_tile_waves(int m, int n) { return red_skinny(m, n) ? RedSkinny::NW : RedBig::NW; }
int red_ring_kib(int m, int n) { return red_skinny(m, n) ? red_ring_kib<RedSkinny>() : red_ring_kib<RedBig>(); }

// The roles of one launch over stage buffers st0..st4 (16 x 16 x 32 core: A slots st0..st2, B slots
// st3, st4) and three workgroup-shared ints.
template <class T>
__device__ __forceinline__ void gemm_reduce_body(const RedParams& p, char* st0, char* st1, char* st2, char* st3,
                                                 char* st4, int* s_ok, int* s_claim, int* s_last) {
  const int wg = blockIdx.x;
  if (wg >= p.n_copy && wg < p.n_copy + p.n_reduce) {
    trace_begin(p.trace, ROLE_REDUCE);
    red_reduce_role<T>(p, wg - p.n_copy, s_ok);
    trace_mark(p.trace, 5);
  } else {
    // one call site of the compute role (one inlined copy of its K loop): copy workgroups join it
    // on leftover tiles (slot -1) once their units have landed
    int slot = wg - p.n_copy - p.n_reduce;
    if (wg < p.n_copy) {
      trace_begin(p.trace, ROLE_COPY);
      red_copy_role<T>(p, wg, st0, st1);
      trace_mark(p.trace, 5);
      __syncthreads();  // the ring's LDS slots become the GEMM's stage buffers
      slot = -1;
    } else {
      trace_begin(p.trace, ROLE_COMPUTE);
    }
    if (slot < p.n_compute) red_compute_role<T>(p, slot, st0, st1, st2, st3, st4, s_ok, s_claim);
  }
  trace_end(p.trace);
  // exit accounting: the last workgroup out re-zeroes the claim and band counters for the next
  // call (every workgroup's last claim returned, and its last band count or band wait finished,
  // before it counts its exit)
  __syncthreads();
  if (threadIdx.x == 0) *s_last = atomic_add_agent(p.counters + CTR_RED_EXIT, 1u) == gridDim.x - 1;
  __syncthreads();
  if (*s_last) {
    if (p.assist) {
      const int n_own = (p.own_tile_end - p.own_tile_begin) * p.tiles_n;
      for (int i = threadIdx.x; i < n_own; i += T::NW * 64)
        __hip_atomic_store(p.counters + CTR_RED_BAND0 + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (threadIdx.x == 0) {
      __hip_atomic_store(p.counters + CTR_RED_TILE, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(p.counters + CTR_RED_PRESUM, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(p.counters + CTR_RED_EXIT, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <class T>
__global__ __launch_bounds__(T::NW * 64, 1) void gemm_reduce_kernel(RedParams p) {
  __shared__ __attribute__((aligned(16))) char st0[red_stage_bytes<T>()];
  __shared__ __attribute__((aligned(16))) char st1[red_stage_bytes<T>()];
  __shared__ __attribute__((aligned(16))) char st2[k_stages<T>() >= 3 ? T::STAGE : 16];
  __shared__ __attribute__((aligned(16))) char st3[k_stages<T>() >= 5 ? T::STAGE : 16];
  __shared__ __attribute__((aligned(16))) char st4[k_stages<T>() >= 5 ? T::STAGE : 16];
  __shared__ int s_ok, s_claim, s_last;
  gemm_reduce_body<T>(p, st0, st1, st2, st3, st4, &s_ok, &s_claim, &s_last);
}

// Wide outputs: 3 A slots + 2 B slots fill the 160 KiB of LDS, so the three shared ints live in the
// first words of the last B slot.  No K loop runs while they are used: tile claims and pre-sum jobs
// come between tiles, the owned-tile wait after the K loop has drained its DMA, the reduce role runs
// no K loop, and the exit count comes after every tile.
__global__ __launch_bounds__(RedBig::NW * 64, 1) void gemm_reduce_kernel16(RedParams p) {
  // 256-byte aligned: the swizzled B reads XOR a fragment's offset into bits 5-7 of the address
  __shared__ __attribute__((aligned(256))) char a0[RedBig::SLOT_A];
  __shared__ __attribute__((aligned(256))) char a1[RedBig::SLOT_A];
  __shared__ __attribute__((aligned(256))) char a2[RedBig::SLOT_A];
  __shared__ __attribute__((aligned(256))) char b0[RedBig::SLOT_B];
  __shared__ __attribute__((aligned(256))) char b1[RedBig::SLOT_B];
  static_assert(3 * RedBig::SLOT_A + 2 * RedBig::SLOT_B <= 160 * 1024, "LDS");
  int* s = reinterpret_cast<int*>(b1);
  gemm_reduce_body<RedBig>(p, a0, a1, a2, b0, b1, s, s + 1, s + 2);
}

// GEMM + AllReduce with resident peer partials on the four-wave tile, one tile per workgroup, in
// eight waves: waves 0-3 run the tile's K loop and waves 4-7 stream the peers' partials of the same
// tile beside it, wave 4 + w summing exactly the values that compute wave w holds in its epilogue
// (one 32-row slab, SLAB_Q values of 4 per lane).  Every wave passes the same barriers, one per
// step (the loop's trip count and conditions depend only on nk and the peer count), so the peer
// stream and the K loop pace each other; the barriers carry no memory fence, so each wave's loads stay in flight
// across them (each wave waits for its own with vmcnt).  Peer q's values go in two halves
// ("pairs" 2q and 2q + 1); pair j is requested AR_PEER_AHEAD steps before it is added, into
// register buffer j % 4.  After the loop the sums reach the compute waves through the idle stage
// buffers.
constexpr int AR_SPLIT_STAGES = 4, AR_PEER_AHEAD = 3;
__global__ __launch_bounds__(2 * RedSkinny::NW * 64, 1) void gemm_ar_split_kernel(RedParams p) {
  using T = RedSkinny;
  static_assert(T::NW == 4 && T::FM == 1 && T::WN == 1 && T::WM == 4, "one 32-row slab per compute wave");
  constexpr int S = AR_SPLIT_STAGES, D = T::A_INSTR + T::B_INSTR, Q = T::SLAB_Q, H = Q / 2, C4 = T::WTN / 4;
  static_assert(Q == 8 && S * T::STAGE <= 160 * 1024, "layout");
  __shared__ __attribute__((aligned(16))) char st0[T::STAGE];
  __shared__ __attribute__((aligned(16))) char st1[T::STAGE];
  __shared__ __attribute__((aligned(16))) char st2[T::STAGE];
  __shared__ __attribute__((aligned(16))) char st3[T::STAGE];
  static_assert(2 * Q * 64 * 16 <= T::STAGE, "two waves' sums fit one stage buffer");
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool comp = wave < T::NW;
  const int cw = comp ? wave : wave - T::NW;  // the compute wave (slab) this wave works for
  const int n_tiles = p.tiles_m * p.tiles_n, C = p.n_compute, slot = blockIdx.x;
  const int rs = ((C & 7) == 0) ? (slot & 7) * (C >> 3) + (slot >> 3) : slot;
  if (slot >= C || rs >= n_tiles) return;  // the whole workgroup (the launch gives every tile one)
  trace_begin(p.trace, ROLE_COMPUTE);
  // tiles in column order: an XCD's workgroups (consecutive rs) hold every tile row of their
  // columns, so each B column block is read from memory once, by one XCD, at the same time
  const int tn = rs / p.tiles_m, tm = rs - tn * p.tiles_m;
  const int m0 = tm * T::BM, n0 = tn * T::BN;
  const int rows_valid = min(T::BM, p.m - m0), cols_valid = min(T::BN, p.n - n0);
  const int nk = p.k >> 6;
  const uint32_t lda_b = (uint32_t)p.k * 2u, ldb_b = (uint32_t)p.n * 2u;
  T g;
  g.init(cw, 0, lane, lda_b, ldb_b);
  g.zero();
  const char* a_tile = reinterpret_cast<const char*>(p.a + (size_t)m0 * p.k);
  const uint32_t a_tile_bytes = (uint32_t)rows_valid * lda_b;
  const char* b_col = reinterpret_cast<const char*>(p.b + n0);
  const uint32_t b_col_bytes = ((uint32_t)p.k * (uint32_t)p.n - (uint32_t)n0) * 2u;
  auto load = [&](int ks, char* st) {  // compute waves only
    const uint32_t ca = (uint32_t)ks * 128u, rb = (uint32_t)ks * 64u * ldb_b;
    g.dma_a(a_tile + ca, a_tile_bytes - ca, lda_b, st, cw);
    g.dma_b(b_col + rb, b_col_bytes - rb, ldb_b, st, cw);
  };
  // the peers: value v of this lane is tile row 32 cw + (64 v + lane) / C4, column 4 ((64 v + lane) % C4)
  const int n_pairs = 2 * (p.world - 1);
  const size_t base = (size_t)m0 * p.n + n0;
  constexpr int LA = AR_PEER_AHEAD;
  static_assert(LA >= 1 && LA <= 3, "pairs in flight fit the four buffers beside the one being added");
  f32x4 sum[Q], buf[4][H];
#pragma unroll
  for (int v = 0; v < Q; ++v) sum[v] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto issue = [&](int j, int half, f32x4(&b)[H]) {  // reduce waves: request pair j (half = j & 1)
    const float* src = peer_src(p, j >> 1) + base;
#pragma unroll
    for (int i = 0; i < H; ++i) {
      const int idx = (half * H + i) * 64 + lane, row = T::WTM * cw + idx / C4, col = (idx % C4) * 4;
      b[i] = (row < rows_valid && col < cols_valid)
                 ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src + (size_t)row * p.n + col))
                 : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  auto add = [&](int half, const f32x4(&b)[H]) {
#pragma unroll
    for (int i = 0; i < H; ++i) sum[half * H + i] += b[i];
  };
  // wait until pair q has landed while the pairs requested after it (at most LA) stay in flight
  auto wait_pair = [&](int q) {
    const int after = min(LA, n_pairs - 1 - q);
    if (LA >= 3 && after >= 3) wait_vm<3 * H>();
    else if (LA >= 2 && after == 2) wait_vm<2 * H>();
    else if (after == 1) wait_vm<H>();
    else wait_vm<0>();
  };
  // prologue: steps 0 .. S-2 requested, step 0 landed; pairs 0 .. LA-1 requested
  if (comp) {
#pragma unroll
    for (int i = 0; i < S - 1; ++i)
      if (i < nk) load(i, i == 0 ? st0 : i == 1 ? st1 : st2);
    wait_steps<D>(min(S - 1, nk) - 1);
  } else {
#pragma unroll
    for (int j = 0; j < LA; ++j)
      if (j < n_pairs) issue(j, j & 1, buf[j]);
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);
  barrier_only();
  trace_mark(p.trace, 5);
  // step q (R = q % 4): compute waves request step q + S - 1 into the buffer step q - 1 read and
  // run step q's MFMAs; reduce waves request pair q + LA and add pair q.  The loop runs
  // max(nk, n_pairs) steps, so a short K loop leaves no pair behind (every buffer index stays a
  // constant: the buffers stay in registers).
  const int n_steps = max(nk, n_pairs);
  auto sub = [&](int q, auto r, char* cur, char* pf) {
    constexpr int R = decltype(r)::value, RN = (R + LA) & 3;
    if (q >= n_steps) return;
    if (comp) {
      if (q < nk) {  // (past the K loop the compute waves only pass the barrier)
        if (q + S - 1 < nk) load(q + S - 1, pf);
        g.mma(cur);
        wait_steps<D>(max(0, min(S - 2, nk - 2 - q)));
      }
    } else {
      if (q + LA < n_pairs) issue(q + LA, RN & 1, buf[RN]);
      if (q < n_pairs) {
        wait_pair(q);
        add(R & 1, buf[R]);
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    barrier_only();
  };
  static_assert(S == 4, "the stage buffers and the peer buffers rotate together");
  for (int q = 0; q < n_steps; q += S) {
    sub(q, std::integral_constant<int, 0>{}, st0, st3);
    sub(q + 1, std::integral_constant<int, 1>{}, st1, st0);
    sub(q + 2, std::integral_constant<int, 2>{}, st2, st1);
    sub(q + 3, std::integral_constant<int, 3>{}, st3, st2);
  }
  trace_mark(p.trace, 6);  // the K loop is done
  if (!comp) {
    // hand the sums to compute wave cw: (v, lane) at 16 (64 v + lane) of its area
    float* area = reinterpret_cast<float*>((cw < 2 ? st2 : st3) + (cw & 1) * (Q * 64 * 16));
#pragma unroll
    for (int v = 0; v < Q; ++v) *reinterpret_cast<f32x4*>(area + (v * 64 + lane) * 4) = sum[v];
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);
  barrier_only();
  if (comp) {
    const float* area = reinterpret_cast<const float*>((cw < 2 ? st2 : st3) + (cw & 1) * (Q * 64 * 16));
    g.epilogue_slab(st0, st1, cw, 0, lane, cw, [&](int srow, f32x4(&v)[Q], const int(&r)[Q], const int(&c)[Q]) {
      (void)srow;
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const f32x4 t = *reinterpret_cast<const f32x4*>(area + (q * 64 + lane) * 4);
        if (r[q] < rows_valid && c[q] < cols_valid)  // the final value: nothing reads it back here
          __builtin_nontemporal_store(v[q] + t, reinterpret_cast<f32x4*>(p.out + base + (size_t)r[q] * p.n + c[q]));
      }
    });
  }
  trace_end(p.trace);
}

template <class T>
static hipError_t launch_t(const RedParams& p, int grid, hipStream_t s) {
  hipLaunchKernelGGL(gemm_reduce_kernel<T>, dim3(grid), dim3(T::NW * 64), 0, s, p);
  return hipGetLastError();
}

// The split AllReduce kernel serves resident AllReduce on the four-wave tile when every tile has its
// own workgroup and there is no reduce role; everything else runs the role kernels.
static bool ar_split(const RedParams& p, int grid) {
  return !p.is_rs && !p.emulated && p.n_reduce == 0 && p.n_copy == 0 && !p.a_ready && p.world > 1 &&
         (p.n_compute & 7) == 0 && p.n_compute <= grid && p.tiles_m * p.tiles_n <= p.n_compute;
}

hipError_t launch_gemm_reduce(const RedParams& p, int grid, hipStream_t s) {
  if (red_skinny(p.m, p.n) && ar_split(p, grid)) {
    hipLaunchKernelGGL(gemm_ar_split_kernel, dim3(grid), dim3(2 * RedSkinny::NW * 64), 0, s, p);
    return hipGetLastError();
  }
  if (red_skinny(p.m, p.n)) return launch_t<RedSkinny>(p, grid, s);
  hipLaunchKernelGGL(gemm_reduce_kernel16, dim3(grid), dim3(RedBig::NW * 64), 0, s, p);
  return hipGetLastError();
}

}  // namespace mk
