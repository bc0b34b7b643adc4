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

template <class T>
__global__ __launch_bounds__(T::NW * 64, 1) void gemm_reduce_kernel(RedParams p) {
  __shared__ __attribute__((aligned(16))) char st0[red_stage_bytes<T>()];
  __shared__ __attribute__((aligned(16))) char st1[red_stage_bytes<T>()];
  __shared__ __attribute__((aligned(16))) char st2[k_stages<T>() >= 3 ? T::STAGE : 16];
  __shared__ __attribute__((aligned(16))) char st3[k_stages<T>() >= 5 ? T::STAGE : 16];
  __shared__ __attribute__((aligned(16))) char st4[k_stages<T>() >= 5 ? T::STAGE : 16];
  __shared__ int s_ok;
  __shared__ int s_claim;
  const int wg = blockIdx.x;
  if (wg < p.n_copy) {
    trace_begin(p.trace, ROLE_COPY);
    red_copy_role<T>(p, wg, st0, st1);
    trace_mark(p.trace, 5);
    __syncthreads();  // the ring's LDS slots become the GEMM's stage buffers
    red_compute_role<T>(p, -1, st0, st1, st2, st3, st4, &s_ok, &s_claim);  // then help with leftover tiles
  } else if (wg < p.n_copy + p.n_reduce) {
    trace_begin(p.trace, ROLE_REDUCE);
    red_reduce_role<T>(p, wg - p.n_copy, &s_ok);
    trace_mark(p.trace, 5);
  } else {
    trace_begin(p.trace, ROLE_COMPUTE);
    const int slot = wg - p.n_copy - p.n_reduce;
    if (slot < p.n_compute) red_compute_role<T>(p, slot, st0, st1, st2, st3, st4, &s_ok, &s_claim);
  }
  trace_end(p.trace);
  // exit accounting: the last workgroup out re-zeroes the claim and band counters for the next
  // call (every workgroup's last claim returned, and its last band count or band wait finished,
  // before it counts its exit)
  __shared__ int s_last;
  __syncthreads();
  if (threadIdx.x == 0) s_last = atomic_add_agent(p.counters + CTR_RED_EXIT, 1u) == gridDim.x - 1;
  __syncthreads();
  if (s_last) {
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
static hipError_t launch_t(const RedParams& p, int grid, hipStream_t s) {
  hipLaunchKernelGGL(gemm_reduce_kernel<T>, dim3(grid), dim3(T::NW * 64), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_gemm_reduce(const RedParams& p, int grid, hipStream_t s) {
  return red_skinny(p.m, p.n) ? launch_t<RedSkinny>(p, grid, s) : launch_t<RedBig>(p, grid, s);
}

}  // namespace mk
