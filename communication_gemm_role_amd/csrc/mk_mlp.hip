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
//            compute 256 x 224 tiles of A @ B_up; the epilogue stores H = bf16(gelu(tile)) and
//            counts the stored tiles of each 256-row block of H.
//   phase 2  every workgroup runs the GEMM + ReduceScatter compute role (mk_red_roles.hpp) on
//            H @ B_down in 256 x 256 tiles, peers' partials resident: a tile waits until its 256
//            rows of H are complete, the owned tiles' peer partials are pre-summed in bands
//            between tiles, and each tile's partial goes to the owned slice or to its owner's
//            outbox.
// Both phases run the 16 x 16 x 32 core over the same five LDS slots (three A slots and two B
// slots of 32 KiB; the up-projection's B rows fill 28 KiB of a B slot).
// Phase 1 never waits on phase 2 and a workgroup enters phase 2 only after phase 1 has no tile
// left for it, so the workgroups that phase 2 waits for are always running.
#include "mk_ag_roles.hpp"
#include "mk_red_roles.hpp"

namespace mk {

int mlp_tile_m() { return TileGemm16::BM; }
int mlp_tile_n() { return TileGemm16::BN; }

static_assert(TileGemm16::BM == RedBig::BM, "a 256-row block of H is one tile row of both phases");
static_assert(AG_THREADS == RedBig::NW * 64, "both phases run eight-wave workgroups");
static_assert(TileGemm16::SLOT_A == RedBig::SLOT_A && TileGemm16::SLOT_B <= RedBig::SLOT_B, "shared slots");

// Phase 1's scheduling state lives in the last B slot past the up-projection's 28 KiB of B rows;
// phase 2's three ints in its first words, used only outside phase 2's K loops (tile claims and
// pre-sum jobs between tiles, the owned-tile wait after a K loop has drained, the exit count).
constexpr int MLP_POLL = TileGemm16::SLOT_B;                // s_poll: 4 x 64 uint32
constexpr int MLP_SCHED = MLP_POLL + 4 * 64 * 4;           // s_sched: AG_SCHED_WORDS ints
constexpr int MLP_CLAIM = MLP_SCHED + AG_SCHED_WORDS * 4;  // phase 1's s_claim
static_assert(MLP_CLAIM + 4 <= RedBig::SLOT_B, "phase 1's scheduling state fits behind its B rows");

__global__ __launch_bounds__(AG_THREADS, 1) void mlp_kernel(MlpParams p) {
  // 256-byte aligned: the down-projection's swizzled B reads XOR bits 5-7 of the address
  __shared__ __attribute__((aligned(256))) char a0[RedBig::SLOT_A];
  __shared__ __attribute__((aligned(256))) char a1[RedBig::SLOT_A];
  __shared__ __attribute__((aligned(256))) char a2[RedBig::SLOT_A];
  __shared__ __attribute__((aligned(256))) char b0[RedBig::SLOT_B];
  __shared__ __attribute__((aligned(256))) char b1[RedBig::SLOT_B];
  uint32_t* s_poll = reinterpret_cast<uint32_t*>(b1 + MLP_POLL);
  int* s_sched = reinterpret_cast<int*>(b1 + MLP_SCHED);
  int* s_claim1 = reinterpret_cast<int*>(b1 + MLP_CLAIM);
  int* s2 = reinterpret_cast<int*>(b1);  // phase 2: s_ok, s_claim, s_last
  const int wg = blockIdx.x;
  // phase 1: AllGather + up-projection
  const bool is_copy = wg < p.ag.n_copy;
  if (is_copy) {
    trace_begin(p.ag.trace, ROLE_COPY);
    ag_copy_role<32>(p.ag, wg, a0, a1);
    trace_mark(p.ag.trace, 5);
    __syncthreads();  // the copy's LDS slots become the GEMM's stage buffers
  } else {
    trace_begin(p.ag.trace, ROLE_COMPUTE);
  }
  // Every workgroup starts a tile once the tile's 256-row block of A has landed and runs its K loop
  // in K order: the ready-first loop of mk_ag_gemm does not fit the register budget beside phase 2.
  ag_compute_role16<1, false>(p.ag, ag_static_tile(p.ag, wg, gridDim.x), !is_copy, true, a0, a1, a2, b0, b1,
                              s_sched, s_claim1, s_poll);
  __syncthreads();
  trace_mark(p.ag.trace, 6);  // phase 1 done for this workgroup
  // phase 2: down-projection + ReduceScatter on H; every workgroup is a compute workgroup
  if (!status_bad(p.red.status) && wg < p.red.n_compute)
    red_compute_role<RedBig>(p.red, wg, a0, a1, a2, b0, b1, s2, s2 + 1);
  trace_end(p.ag.trace);
  // exit accounting: the last workgroup out re-zeroes every counter the two phases used
  __syncthreads();
  if (threadIdx.x == 0) s2[2] = atomic_add_agent(p.red.counters + CTR_MLP_EXIT, 1u) == gridDim.x - 1;
  __syncthreads();
  if (s2[2]) {
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
