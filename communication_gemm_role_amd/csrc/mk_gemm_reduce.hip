// GEMM + ReduceScatter and GEMM + AllReduce, one rank's share, as one persistent launch (roles in
// mk_red_roles.hpp).
//
// Operations (mKernel write-up, news.chathome.org page, five-fused-kernels table, GEMM +
// AllReduce and GEMM + ReduceScatter rows): rank j holds a partial P_j = A_j @ B_j of the same
// [M, N] output.  AllReduce: every rank ends with sum_j P_j.  ReduceScatter: rank r ends with
// sum_j P_j on its own row slice only.  A tile of P enters the reduction right after its K loop,
// inside the same launch.
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

template <class T>
static hipError_t launch_t(const RedParams& p, int grid, hipStream_t s) {
  hipLaunchKernelGGL(gemm_reduce_kernel<T>, dim3(grid), dim3(T::NW * 64), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_gemm_reduce(const RedParams& p, int grid, hipStream_t s) {
  if (red_skinny(p.m, p.n)) return launch_t<RedSkinny>(p, grid, s);
  hipLaunchKernelGGL(gemm_reduce_kernel16, dim3(grid), dim3(RedBig::NW * 64), 0, s, p);
  return hipGetLastError();
}

}  // namespace mk
