// Device-side primitives shared by the persistent role kernels (gfx950 only).
//
// Producer/consumer protocol between workgroups that may sit on different XCDs
// (each XCD has its own L2):
//   producer: writes the payload with write-through stores (cache policy SC1, so the
//             data reaches the device coherence point instead of staying dirty in the
//             producer's L2), waits for its stores to be acknowledged (vmcnt 0), then
//             a workgroup barrier, then one lane stores the ready flag (relaxed,
//             agent scope, itself SC1).
//   consumer: one lane polls the flag with relaxed agent-scope loads (SC1, served from
//             the coherence point) under a wall-clock watchdog; a workgroup barrier
//             hands the result to the other lanes; payload loads are issued after it.
// No L2 writeback or invalidate is issued on the hot path: measured on MI355X, an
// agent-scope acquire/release fence costs several microseconds when every CU issues
// it, while the write-through + relaxed-flag protocol passes the cross-XCD litmus test
// (tests/test_litmus_gpu.py).  The payload a consumer reads after a flag is only ever
// written once per launch and is never read before its flag, so no consumer L2 can
// hold a stale copy of it (kernel boundaries invalidate caches).
//
// Flags carry an epoch (the call number of the context), so they never need clearing
// between calls: a flag is "up" when it equals the current epoch.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// cache-policy immediates for buffer instructions on gfx950
constexpr int CP_DEFAULT = 0;
constexpr int CP_SC1 = 16;  // device-scope coherent (write-through / coherent read)
constexpr int CP_NT = 2;    // non-temporal (streaming)

// status codes written to the device status word (same values as the C ABI)
constexpr int ST_TIMEOUT = -5;
constexpr int ST_CAPACITY = -6;

// Raw buffer resource over [base, base + bytes).  Accesses outside the range read 0 and
// drop stores, which bounds every access of a tile to its own operand.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, CP_DEFAULT);
}
__device__ __forceinline__ u32x4 bload16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, CP_NT);
}
__device__ __forceinline__ u32x4 bload16_sc1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, CP_SC1);
}
__device__ __forceinline__ uint32_t bload4_sc1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, CP_SC1);
}
__device__ __forceinline__ void bstore16(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, CP_DEFAULT);
}
__device__ __forceinline__ void bstore16_sc1(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, CP_SC1);
}
__device__ __forceinline__ void bstore8_sc1(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, CP_SC1);
}
__device__ __forceinline__ void bstore4(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, CP_DEFAULT);
}
__device__ __forceinline__ void bstore4_sc1(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, CP_SC1);
}

// Wait until every memory operation this lane issued has completed (stores acknowledged).
__device__ __forceinline__ void wait_mem() { __builtin_amdgcn_s_waitcnt(0); }

__device__ __forceinline__ uint64_t wall_ticks() { return __builtin_readsteadycounter(); }  // 100 MHz

// Every lane of a wave: sleep until the wall clock reaches `deadline` (link-rate pacing of a copy
// role; the host bounds the deadline well inside the watchdog).
__device__ __forceinline__ void wait_wall_until(uint64_t deadline) {
  while ((int64_t)(wall_ticks() - deadline) < 0) __builtin_amdgcn_s_sleep(2);
}

__device__ __forceinline__ uint32_t flag_load(const uint32_t* f) {
  return __hip_atomic_load(const_cast<uint32_t*>(f), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Per-workgroup trace record (8 uint64 per workgroup, slots as documented for mk_opts.trace),
// written by thread 0 with ordinary vector stores when the caller asked for one.
__device__ __forceinline__ void trace_put(uint64_t* tr, int slot, uint64_t v) {
  if (tr && threadIdx.x == 0) tr[(size_t)blockIdx.x * 8 + slot] = v;
}
__device__ __forceinline__ void trace_mark(uint64_t* tr, int slot) { trace_put(tr, slot, wall_ticks()); }
__device__ __forceinline__ void trace_begin(uint64_t* tr, int role) {
  if (tr && threadIdx.x == 0) {
    uint64_t* r = tr + (size_t)blockIdx.x * 8;
    r[0] = wall_ticks();
    r[1] = __builtin_readcyclecounter();
    r[4] = (uint64_t)role;
    r[5] = r[6] = r[7] = 0;
  }
}
__device__ __forceinline__ void trace_end(uint64_t* tr) {
  if (tr && threadIdx.x == 0) {
    uint64_t* r = tr + (size_t)blockIdx.x * 8;
    r[2] = wall_ticks();
    r[3] = __builtin_readcyclecounter();
  }
}
constexpr int ROLE_COPY = 0, ROLE_COMPUTE = 1, ROLE_REDUCE = 2;

// Workgroup barrier without the memory fence of __syncthreads.  The fence of a workgroup-scope
// release makes the compiler wait for every outstanding vector-memory operation, stores included,
// which would drain a copy pipeline at each barrier.  Callers order memory themselves with explicit
// vmcnt waits before the barrier; the empty asm with a memory clobber keeps the compiler from
// moving loads or stores across it.
__device__ __forceinline__ void barrier_only() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ void flag_store(uint32_t* f, uint32_t v) {
  __hip_atomic_store(f, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t atomic_add_agent(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Device status word: first fault wins.
__device__ __forceinline__ void raise_status(int* status, int code) {
  int expected = 0;
  __hip_atomic_compare_exchange_strong(status, &expected, code, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool status_bad(const int* status) {
  return __hip_atomic_load(const_cast<int*>(status), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
}

// Spin (one lane) until *f == want.  Returns false on timeout or when another workgroup has
// already recorded a fault (then every waiter drains instead of spinning on).
__device__ __forceinline__ bool spin_until_eq(const uint32_t* f, uint32_t want, uint64_t timeout_ticks,
                                              int* status) {
  if (flag_load(f) == want) return true;
  const uint64_t t0 = wall_ticks();
  int n = 0;
  while (true) {
    __builtin_amdgcn_s_sleep(1);
    if (flag_load(f) == want) return true;
    if ((++n & 15) == 0) {
      if (status_bad(status)) return false;
      if (wall_ticks() - t0 > timeout_ticks) {
        raise_status(status, ST_TIMEOUT);
        return false;
      }
    }
  }
}

// Spin (one lane) until *c >= want (counters).  Counter waits (a grouped-GEMM m-tile's landed
// rows, an RS owned tile's pre-summed bands) expect a large count and many workgroups wait on the
// same few counters, so the poll backs off about a microsecond: polling as fast as the flag waits
// measurably slowed the MoE dispatch's own stores and loads.
__device__ __forceinline__ bool spin_until_ge(const uint32_t* c, uint32_t want, uint64_t timeout_ticks,
                                              int* status) {
  if (flag_load(c) >= want) return true;
  const uint64_t t0 = wall_ticks();
  int n = 0;
  while (true) {
    __builtin_amdgcn_s_sleep(32);
    if (flag_load(c) >= want) return true;
    if ((++n & 15) == 0) {
      if (status_bad(status)) return false;
      if (wall_ticks() - t0 > timeout_ticks) {
        raise_status(status, ST_TIMEOUT);
        return false;
      }
    }
  }
}

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

}  // namespace mk
