// AllGather + GEMM, one rank's share, as one persistent launch (roles in mk_ag_roles.hpp).
//
// Operation (mKernel write-up, news.chathome.org page, five-fused-kernels table,
// AllGather + GEMM row): C = [A_0; A_1; ...; A_{W-1}] @ B, rank r holding the row shard A_r
// and B being local.  The product does not wait for the gather: a K-unit of a tile's rows
// enters the tile's K loop as soon as it is present.  Here the other ranks' shards are
// device buffers and their arrival is the copy role.
#include "mk_ag_roles.hpp"

namespace mk {

int ag_tile_m() { return TileGemm16::BM; }
int ag_tile_n() { return TileGemm16::BN; }

// Roles: workgroups [0, n_copy) copy (land peer units in the caller's order), then compute; the rest
// compute from the start (static tiles: ag_static_tile, the local shard's tiles first).
__global__ __launch_bounds__(AG_THREADS, 1) void ag_gemm_kernel(AgParams p) {
  using G = TileGemm16;
  __shared__ __attribute__((aligned(16))) char a0[G::SLOT_A];
  __shared__ __attribute__((aligned(16))) char a1[G::SLOT_A];
  __shared__ __attribute__((aligned(16))) char a2[G::SLOT_A];
  __shared__ __attribute__((aligned(16))) char b0[G::SLOT_B];
  __shared__ __attribute__((aligned(16))) char b1[G::SLOT_B];
  __shared__ int s_sched[AG_SCHED_WORDS];
  __shared__ int s_claim;
  __shared__ __attribute__((aligned(16))) uint32_t s_poll[4 * 64];
  const int wg = blockIdx.x;
  const int t_static = ag_static_tile(p, wg, gridDim.x);
  if (wg < p.n_copy) {
    trace_begin(p.trace, ROLE_COPY);
    ag_copy_role<32>(p, wg, a0, a1);
    trace_mark(p.trace, 5);
    __syncthreads();  // the copy's LDS slots become the GEMM's stage buffers
  } else {
    trace_begin(p.trace, ROLE_COMPUTE);
  }
  const bool is_copy = wg < p.n_copy;
  // Unpaced, the copy lands every unit within ~20 us, and a tile that waits for its rows and then
  // runs its K loop in order ends sooner than one that starts on partial rows ready-first (whose
  // K order differs from the other tiles of its XCD, so their A and B k-slabs stop being shared in
  // L2): every workgroup waits.  Paced at a link rate the landing takes several times longer, and
  // compute workgroups consume units ready-first.
  ag_compute_role16<0>(p, t_static, !is_copy, is_copy || p.pace_q16 == 0, a0, a1, a2, b0, b1, s_sched, &s_claim,
                       s_poll);
  trace_end(p.trace);
  // exit accounting: the last workgroup out re-zeroes the tile counter for the next call (every
  // workgroup's last claim returned before it counts its exit)
  __syncthreads();
  if (threadIdx.x == 0 && atomic_add_agent(p.counters + CTR_AG_EXIT, 1u) == gridDim.x - 1) {
    __hip_atomic_store(p.counters + CTR_AG_TILE, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(p.counters + CTR_AG_EXIT, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // every other workgroup's faults were recorded before it counted its exit
    if (p.status_out)
      *p.status_out = __hip_atomic_exchange(p.status, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

hipError_t launch_ag_gemm(const AgParams& p, int grid, hipStream_t s) {
  hipLaunchKernelGGL(ag_gemm_kernel, dim3(grid), dim3(AG_THREADS), 0, s, p);
  return hipGetLastError();
}

}  // namespace mk
