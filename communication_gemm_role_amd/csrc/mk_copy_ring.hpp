// Copy-role data mover shared by the AllGather and GEMM+ReduceScatter/AllReduce kernels: units
// of a workgroup's arrival queue go global -> LDS (DMA) -> VGPRs -> global through two LDS slots.
// A source unit is read once, so its loads are non-temporal (they should not displace the
// compute role's operands from L2).
//
// Every wave moves its own share of each unit, so no LDS data crosses waves: while one batch is
// being stored, the next is landing and the one after is requested, so up to two batches of loads
// are in flight per CU and no register holds data in flight.  A batch gives every wave IPB DMA
// instructions of 1 KiB (64 lanes x 16 bytes): UPB units of IPU instructions each.  Stores are
// write-through (the consumers sit on other XCDs and read the units once); a batch's units are
// handed to raise() by thread 0 once every wave's stores of that batch have completed.  A slot past
// the end of the queue (or a unit the caller drops) uses an empty buffer window, so every batch
// issues the same instructions and the vmcnt arithmetic below holds: per batch and wave IPB DMA
// loads and IPB stores, completing in issue order.  The two slots are distinct LDS arrays named
// statically in an unrolled loop, so the compiler can see that reads of one never alias the DMA
// into the other; barriers carry no memory fence (the waits order the stores, and a fence would
// make the compiler drain every outstanding store at each batch).
#pragma once
#include "mk_device.hpp"
#include "mk_gemm_tile.hpp"

namespace mk {

// n_units: length of this workgroup's queue.  unit_at(i): unit id of queue entry i, or -1 (never
// lands).  src_of(u) / dst_of(u): buffer windows of unit u's first byte (u < 0: any empty window).
// off[k]: this lane's byte offset inside a unit for the unit's k-th instruction (k < IPU).
// raise(u): publish unit u (called by thread 0 only, after its stores have completed).
// pace(i): called by every wave before it requests a batch, with i the batch's last queue entry
// (link-rate pacing: no unit is requested before its own arrival time, the batch's earlier units
// wait for the last one; pace only waits on the clock, so the vmcnt arithmetic below holds).
template <int IPB, int IPU, class UnitAt, class SrcOf, class DstOf, class Raise, class Pace>
__device__ __forceinline__ void copy_ring(int n_units, char* slot0, char* slot1, const uint32_t (&off)[IPU],
                                          UnitAt&& unit_at, SrcOf&& src_of, DstOf&& dst_of, Raise&& raise,
                                          Pace&& pace) {
  constexpr int UPB = IPB / IPU;  // units per batch
  static_assert(UPB * IPU == IPB && UPB >= 1, "a batch holds whole units");
  static_assert(2 * IPB <= 63, "vmcnt is 6 bits");
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nb = (n_units + UPB - 1) / UPB;
  // this wave's IPB KiB of a slot: instruction k of the batch at +1 KiB * k, lane l at +16 B * l
  auto dma = [&](int b, char* slot) {
    if (b < nb) pace(min((b + 1) * UPB, n_units) - 1);
    char* base = slot + wave * IPB * 1024;
#pragma unroll
    for (int j = 0; j < UPB; ++j) {
      const auto src = src_of(unit_at(b * UPB + j));
#pragma unroll
      for (int i = 0; i < IPU; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            src, (__attribute__((address_space(3))) void*)(base + (j * IPU + i) * 1024), 16, off[i], 0, 0, CP_NT);
    }
  };
  auto store = [&](int b, const char* slot) {
    const char* base = slot + wave * IPB * 1024 + lane * 16;
#pragma unroll
    for (int j = 0; j < UPB; ++j) {
      const auto dst = dst_of(unit_at(b * UPB + j));
#pragma unroll
      for (int i = 0; i < IPU; ++i)
        bstore16_sc1(dst, off[i], *reinterpret_cast<const u32x4*>(base + (j * IPU + i) * 1024));
    }
  };
  auto publish = [&](int b) {
    if (tid == 0)
      for (int j = 0; j < UPB; ++j) {
        const int u = unit_at(b * UPB + j);
        if (u >= 0) raise(u);
      }
  };
  // Batch b has landed once no more than the instructions issued after its DMA are outstanding:
  // the stores of b-1 and the DMA of b+1 (only the DMA of 1 for b = 0).  That also covers the
  // stores of b-2, issued before the DMA of b, whose units are published after the barrier.
  auto step = [&](int b, char* slot) {
    if (b >= nb) return;
    if (b == 0) wait_vm<IPB>();
    else wait_vm<2 * IPB>();
    barrier_only();
    if (b >= 2) publish(b - 2);
    store(b, slot);
    dma(b + 2, slot);  // this wave's LDS reads of the slot completed with the stores above
  };
  if (nb == 0) return;
  dma(0, slot0);
  dma(1, slot1);
  for (int b = 0; b < nb; b += 2) {
    step(b, slot0);
    step(b + 1, slot1);
  }
  wait_vm<0>();
  __syncthreads();
  for (int b = nb > 2 ? nb - 2 : 0; b < nb; ++b) publish(b);
}

}  // namespace mk
