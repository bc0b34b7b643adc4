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
#include "mk.h"
#include "mk_device.hpp"
#include "mk_internal.h"

namespace mk {

// pairs producers [0, pairs), consumers [pairs, 2*pairs); consumer c reads the slot of producer
// (c + 3) % pairs (a bijection); with workgroup w on XCD w % 8 the two sides of a pair sit on
// different XCDs whenever (pairs - 3) % 8 != 0, e.g. for pairs = 64.
__global__ __launch_bounds__(256) void litmus_kernel(float* data, uint32_t* flag, uint32_t* ack, uint32_t* counts,
                                                     int* status, int pairs, int rounds, int mode, uint64_t tmo) {
  __shared__ int s_ok;
  const int b = blockIdx.x, t = threadIdx.x;
  const bool producer = b < pairs;
  const int slot = producer ? b : ((b - pairs) + 3) % pairs;
  for (int r = 1; r <= rounds; ++r) {
    // payload of (slot, round): fresh per round in mode 0, fixed otherwise
    const size_t base = (mode == 0 ? ((size_t)(r - 1) * pairs + slot) : (size_t)slot) * 256;
    const auto rs = make_rsrc(data + base, 256 * 4);
    if (producer) {
      const float v = (float)(r * 1000 + slot) + (float)t * 0.5f;
      bstore4_sc1(rs, (uint32_t)t * 4u, __builtin_bit_cast(uint32_t, v));
      wait_mem();
      __syncthreads();
      if (t == 0) {
        flag_store(&flag[slot], (uint32_t)r);
        s_ok = spin_until_eq(&ack[slot], (uint32_t)r, tmo, status);
      }
      __syncthreads();
      if (!s_ok) break;
    } else {
      if (t == 0) s_ok = spin_until_eq(&flag[slot], (uint32_t)r, tmo, status);
      __syncthreads();
      if (!s_ok) break;
      const float v = mode == 1 ? __builtin_bit_cast(float, bload4_sc1(rs, (uint32_t)t * 4u)) : data[base + t];
      const float expect = (float)(r * 1000 + slot) + (float)t * 0.5f;
      if (v != expect) atomic_add_agent(&counts[0], 1u);
      __syncthreads();
      if (t == 0) flag_store(&ack[slot], (uint32_t)r);
    }
  }
}

}  // namespace mk

extern "C" int mk_selftest_flags(int device, int mode, int pairs, int rounds, int64_t* mismatches, int64_t* timeouts) {
  if (!mismatches || !timeouts || pairs < 1 || pairs > 128 || rounds < 1 || mode < 0 || mode > 2)
    return MK_ERR_INVALID_ARG;
  if (mode == 0 && (size_t)pairs * (size_t)rounds > (1u << 18)) return MK_ERR_INVALID_ARG;  // <= 256 MiB payload
  int prev = -1;
  if (hipGetDevice(&prev) != hipSuccess || hipSetDevice(device) != hipSuccess) return MK_ERR_HIP;
  const size_t payload = (size_t)pairs * (mode == 0 ? (size_t)rounds : 1u) * 1024;
  const size_t bytes = payload + (size_t)pairs * 8 + 64;
  char* mem = nullptr;
  int code = MK_OK;
  if (hipMalloc(&mem, bytes) != hipSuccess) code = MK_ERR_HIP;
  if (code == MK_OK && hipMemset(mem, 0, bytes) != hipSuccess) code = MK_ERR_HIP;
  if (code == MK_OK) {
    float* data = (float*)mem;
    uint32_t* flag = (uint32_t*)(mem + payload);
    uint32_t* ack = flag + pairs;
    uint32_t* counts = ack + pairs;
    int* status = (int*)(counts + 4);
    hipLaunchKernelGGL(mk::litmus_kernel, dim3(2 * pairs), dim3(256), 0, 0, data, flag, ack, counts, status, pairs,
                       rounds, mode, (uint64_t)200000000ull /* 2 s at 100 MHz */);
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
