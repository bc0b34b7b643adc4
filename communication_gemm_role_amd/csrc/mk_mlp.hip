// MLP block, one rank's share, as one persistent launch: the up-projection with its AllGather,
// the activation, and the down-projection with its ReduceScatter.
//
// The mKernel write-up (news.chathome.org page, section on the roadmap and key points) names
// the transformer-layer megakernel as the next step after the five fused kernels; this is its
// MLP part on one GPU, built from two of them: AllGather + GEMM (column-parallel up-projection)
// and GEMM + ReduceScatter (row-parallel down-projection), with the activation fused into the
// first one's epilogue.
//
//   phase 1  the AllGather + GEMM roles (mk_ag_roles.hpp): copy workgroups land the peer shards
//            of A, compute workgroups (and copy workgroups once they have landed their units)
//            compute 256 x 256 tiles of A @ B_up; the epilogue stores H = bf16(gelu(tile)) and
//            counts the stored tiles of each 256-row block of H.
//   phase 2  every workgroup runs the GEMM + ReduceScatter compute role (mk_red_roles.hpp) on
//            H @ B_down, peers' partials resident: a tile waits until its 256 rows of H are
//            complete, the owned tiles' peer partials are pre-summed in bands between tiles,
//            and each tile's partial goes to the owned slice or to its owner's outbox.
// Phase 1 never waits on phase 2 and a workgroup enters phase 2 only after phase 1 has no tile
// left for it, so the workgroups that phase 2 waits for are always running.
#include "mk_ag_roles.hpp"
#include "mk_red_roles.hpp"

namespace mk {

int mlp_tile_m() { return AgTile::BM; }
int mlp_tile_n() { return AgTile::BN; }

static_assert(AgTile::BM == MlpDown::BM, "a 256-row block of H is one tile row of both phases");
static_assert(AG_THREADS == MlpDown::NW * 64, "both phases run eight-wave workgroups");
static_assert(MlpDown::BM == RedBig::BM && MlpDown::BN == RedBig::BN && MlpDown::NW == RedBig::NW,
              "the planner's reduce tile (red_tile_m/n/waves) is also the down-projection's");

__global__ __launch_bounds__(AG_THREADS, 1) void mlp_kernel(MlpParams p) {
  __shared__ __attribute__((aligned(16))) char st0[AgTile::STAGE];
  __shared__ __attribute__((aligned(16))) char st1[AgTile::STAGE];
  __shared__ __attribute__((aligned(16))) char st2[16];
  __shared__ int s_sched[64];
  __shared__ int s_claim;
  __shared__ int s_ok;
  __shared__ int s_last;
  static_assert(k_stages<AgTile>() == 2 && k_stages<MlpDown>() == 2, "two 64 KiB stage buffers");
  static_assert(red_stage_bytes<MlpDown>() == AgTile::STAGE, "the stage buffers serve both phases");
  const int wg = blockIdx.x;
  // phase 1: AllGather + up-projection
  if (wg < p.ag.n_copy) {
    trace_begin(p.ag.trace, ROLE_COPY);
    ag_copy_role<64>(p.ag, wg, st0, st1);
    trace_mark(p.ag.trace, 5);
    __syncthreads();  // the copy's LDS slots become the GEMM's stage buffers
    ag_compute_role<1>(p.ag, -1, st0, st1, st2, s_sched, &s_claim);
  } else {
    trace_begin(p.ag.trace, ROLE_COMPUTE);
    const int slot = wg - p.ag.n_copy;
    if (slot < p.ag.n_compute) ag_compute_role<1>(p.ag, slot, st0, st1, st2, s_sched, &s_claim);
  }
  __syncthreads();
  trace_mark(p.ag.trace, 6);  // phase 1 done for this workgroup
  // phase 2: down-projection + ReduceScatter on H; every workgroup is a compute workgroup
  if (!status_bad(p.red.status) && wg < p.red.n_compute)
    red_compute_role<MlpDown>(p.red, wg, st0, st1, st2, st2, st2, &s_ok, &s_claim);
  trace_end(p.ag.trace);
  // exit accounting: the last workgroup out re-zeroes every counter the two phases used
  __syncthreads();
  if (threadIdx.x == 0) s_last = atomic_add_agent(p.red.counters + CTR_MLP_EXIT, 1u) == gridDim.x - 1;
  __syncthreads();
  if (s_last) {
    uint32_t* c = p.red.counters;
    const int n_own = (p.red.own_tile_end - p.red.own_tile_begin) * p.red.tiles_n;
    for (int i = threadIdx.x; i < n_own; i += AG_THREADS)
      __hip_atomic_store(c + CTR_RED_BAND0 + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int i = threadIdx.x; i < p.ag.tiles_m; i += AG_THREADS)
      __hip_atomic_store(c + CTR_MLP_HREADY0 + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (threadIdx.x == 0) {
      for (int k : {CTR_AG_TILE, CTR_RED_TILE, CTR_RED_PRESUM, CTR_MLP_EXIT})
        __hip_atomic_store(c + k, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

hipError_t launch_mlp(const MlpParams& p, int grid, hipStream_t s) {
  hipLaunchKernelGGL(mlp_kernel, dim3(grid), dim3(AG_THREADS), 0, s, p);
  return hipGetLastError();
}

}  // namespace mk
