// Self-test of the producer/consumer protocol the role kernels rely on (mk_device.hpp):
// producer workgroups write a payload with write-through stores, wait for the stores, then
// raise an epoch flag; consumer workgroups on other XCDs poll the flag and read the payload.
//   mode 0  every round uses fresh payload addresses and the consumer reads with ordinary
//           loads: the kernels' own pattern (a payload is written once per launch and never
//           read before its flag), which must never mismatch;
//   mode 1  every round rewrites the same addresses and the consumer reads with device-coherent
//           (SC1) loads, which must never mismatch either;
//   mode 2  same addresses with ordinary loads: a diagnostic, not a guarantee -- the consumer's
//           XCD may keep a stale L2 copy of a line another XCD rewrote, which is why no kernel
//           re-reads an address that was rewritten within the launch.
// The next modes use fresh addresses and the instruction paths the kernels actually take:
//   mode 3  the consumer reads the payload the way the compute role reads its operands: a
//           buffer load straight into LDS (16 bytes per lane, default cache policy), then
//           checks it from LDS;
//   mode 4  the producer moves the payload the way the copy role lands a unit: a non-temporal
//           buffer load of a source unit into LDS, LDS to registers, write-through stores; the
//           consumer reads as in mode 3;
//   mode 5  the producer publishes with a counter increment (atomic add, as the MoE dispatch
//           raises an m-tile's landed-row counter) and the consumer waits for the count, then
//           reads as in mode 3 (the grouped GEMM's path).
#include "mk.h"
#include "mk_device.hpp"
#include "mk_internal.h"
#include "mk_gemm_tile.hpp"

namespace mk {

// pairs producers [0, pairs), consumers [pairs, 2*pairs); consumer c reads the slot of producer
// (c + 3) % pairs (a bijection); with workgroup w on XCD w % 8 the two sides of a pair sit on
// different XCDs whenever (pairs - 3) % 8 != 0, e.g. for pairs = 64.
__device__ __forceinline__ float litmus_value(int r, int slot, int t) {
  return (float)(r * 1000 + slot) + (float)t * 0.5f;
}

// Source units of mode 4: unit (round r, slot) holds the payload the consumer expects.
__global__ __launch_bounds__(256) void litmus_fill_kernel(float* src, int pairs, int rounds) {
  const size_t n = (size_t)pairs * rounds * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const int t = (int)(i % 256);
    const size_t u = i / 256;
    src[i] = litmus_value((int)(u / pairs) + 1, (int)(u % pairs), t);
  }
}

// One wave loads the 1 KiB unit at `rs` straight into LDS (lane l: bytes [16 l, 16 l + 16)),
// waits for it, and the workgroup barrier hands it to every thread.
__device__ __forceinline__ void litmus_dma_to_lds(__amdgpu_buffer_rsrc_t rs, char* lds, int policy) {
  if (threadIdx.x < 64) {
    if (policy == CP_NT)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16,
                                               (uint32_t)threadIdx.x * 16u, 0, 0, CP_NT);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16,
                                               (uint32_t)threadIdx.x * 16u, 0, 0, CP_DEFAULT);
    wait_vm<0>();
  }
  __syncthreads();
}

__global__ __launch_bounds__(256) void litmus_kernel(float* data, const float* src, uint32_t* flag, uint32_t* ack,
                                                     uint32_t* counts, int* status, int pairs, int rounds, int mode,
                                                     uint64_t tmo) {
  __shared__ int s_ok;
  __shared__ __attribute__((aligned(16))) char s_unit[1024];
  const int b = blockIdx.x, t = threadIdx.x;
  const bool producer = b < pairs;
  const bool fresh = mode == 0 || mode >= 3;
  const int slot = producer ? b : ((b - pairs) + 3) % pairs;
  for (int r = 1; r <= rounds; ++r) {
    // payload of (slot, round): fresh per round, or one fixed slot (modes 1 and 2)
    const size_t unit = fresh ? (size_t)(r - 1) * pairs + slot : (size_t)slot;
    const auto rs = make_rsrc(data + unit * 256, 256 * 4);
    if (producer) {
      float v = litmus_value(r, slot, t);
      if (mode == 4) {  // land the source unit as the copy ring does
        litmus_dma_to_lds(make_rsrc(src + unit * 256, 256 * 4), s_unit, CP_NT);
        v = reinterpret_cast<const float*>(s_unit)[t];
      }
      bstore4_sc1(rs, (uint32_t)t * 4u, __builtin_bit_cast(uint32_t, v));
      wait_mem();
      __syncthreads();
      if (t == 0) {
        if (mode == 5) atomic_add_agent(&flag[slot], 1u);
        else flag_store(&flag[slot], (uint32_t)r);
        s_ok = spin_until_eq(&ack[slot], (uint32_t)r, tmo, status);
      }
      __syncthreads();
      if (!s_ok) break;
    } else {
      if (t == 0)
        s_ok = mode == 5 ? spin_until_ge(&flag[slot], (uint32_t)r, tmo, status)
                         : spin_until_eq(&flag[slot], (uint32_t)r, tmo, status);
      __syncthreads();
      if (!s_ok) break;
      float v;
      if (mode >= 3) {
        litmus_dma_to_lds(rs, s_unit, CP_DEFAULT);
        v = reinterpret_cast<const float*>(s_unit)[t];
      } else {
        v = mode == 1 ? __builtin_bit_cast(float, bload4_sc1(rs, (uint32_t)t * 4u)) : data[unit * 256 + t];
      }
      if (v != litmus_value(r, slot, t)) atomic_add_agent(&counts[0], 1u);
      __syncthreads();  // every thread has read the LDS unit before the next round rewrites it
      if (t == 0) flag_store(&ack[slot], (uint32_t)r);
    }
  }
}

}  // namespace mk

extern "C" int mk_selftest_flags(int device, int mode, int pairs, int rounds, int64_t* mismatches, int64_t* timeouts) {
  if (!mismatches || !timeouts || pairs < 1 || pairs > 128 || rounds < 1 || mode < 0 || mode > 5)
    return MK_ERR_INVALID_ARG;
  const bool fresh = mode == 0 || mode >= 3;
  // fresh payloads: <= 256 MiB of them (mode 4 also holds as many source units)
  if (fresh && (size_t)pairs * (size_t)rounds > (mode == 4 ? (1u << 17) : (1u << 18))) return MK_ERR_INVALID_ARG;
  int prev = -1;
  if (hipGetDevice(&prev) != hipSuccess || hipSetDevice(device) != hipSuccess) return MK_ERR_HIP;
  const size_t payload = (size_t)pairs * (fresh ? (size_t)rounds : 1u) * 1024;
  const size_t src_bytes = mode == 4 ? payload : 0;
  const size_t bytes = payload + src_bytes + (size_t)pairs * 8 + 64;
  char* mem = nullptr;
  int code = MK_OK;
  if (hipMalloc(&mem, bytes) != hipSuccess) code = MK_ERR_HIP;
  if (code == MK_OK && hipMemset(mem, 0, bytes) != hipSuccess) code = MK_ERR_HIP;
  if (code == MK_OK) {
    float* data = (float*)mem;
    float* src = (float*)(mem + payload);
    uint32_t* flag = (uint32_t*)(mem + payload + src_bytes);
    uint32_t* ack = flag + pairs;
    uint32_t* counts = ack + pairs;
    int* status = (int*)(counts + 4);
    if (mode == 4) hipLaunchKernelGGL(mk::litmus_fill_kernel, dim3(1024), dim3(256), 0, 0, src, pairs, rounds);
    hipLaunchKernelGGL(mk::litmus_kernel, dim3(2 * pairs), dim3(256), 0, 0, data, src, flag, ack, counts, status,
                       pairs, rounds, mode, (uint64_t)200000000ull /* 2 s at 100 MHz */);
    uint32_t c = 0;
    int st = 0;
    if (hipGetLastError() != hipSuccess || hipDeviceSynchronize() != hipSuccess ||
        hipMemcpy(&c, counts, 4, hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemcpy(&st, status, 4, hipMemcpyDeviceToHost) != hipSuccess)
      code = MK_ERR_HIP;
    *mismatches = c;
    *timeouts = st != 0 ? 1 : 0;
  }
  if (mem) (void)hipFree(mem);
  (void)hipSetDevice(prev);
  return code;
}
