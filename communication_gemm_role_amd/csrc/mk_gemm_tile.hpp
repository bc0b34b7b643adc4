// Compute role core: one BM x BN fp32 output tile of C = A @ B with bf16 operands on gfx950
// MFMA (v_mfma_f32_32x32x16_bf16), the operands staged in LDS over K steps of BK = 64.
//
// NW = WM x WN waves (4 or 8); wave (wm, wn) owns a (BM/WM) x (BN/WN) sub-tile made of 32 x 32
// MFMA fragments.  MFMA lane layout (checked on the device): for the A operand lane l holds row
// l%32, k = 8*(l/32) .. +7 of a 32 x 16 slab; the B operand holds column l%32 with the same k;
// accumulator element r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l%32 of the fragment.
//
// Operands go global -> LDS by buffer_load ... lds (16 bytes per lane, no staging registers,
// out-of-range reads land as zeros), and B stays row-major in LDS.  The B operand is read with
// ds_read_b64_tr_b16: inside each 16-lane group, lane i receives element i%4 of the 8-byte pieces
// addressed by lanes 4j + i/4 (j = 0..3), so when those four lanes point at consecutive 4-column
// pieces of rows k0..k0+3, lane i gets column i of that 4 x 16 block (lane semantics checked on
// the device).  Two such reads give a lane the 8 consecutive k of its column that the MFMA B
// operand needs.
//
// LDS per stage: A [BM][64] bf16 (128-byte rows), B [64][BN] bf16 (2*BN-byte rows), both with
// 16-byte chunks XOR-swizzled so that 16 lanes reading the same logical chunk of 16 consecutive
// rows hit distinct 16-byte groups of the 64 four-byte banks.  The DMA writes each wave's 1 KiB
// contiguously, so the swizzle is applied on the global side: LDS chunk p of row r receives
// global chunk p ^ swz(r).
//
// BK stays 64: each A row then gives a whole 128-byte line per step.  A CU's operand load rate is
// bounded by the lines it has in flight, so BK = 32 (four stages in the same LDS, three steps in
// flight) measured slower, its A rows giving half lines.
#pragma once
#include "mk_device.hpp"
#include "mk_tiles.h"

namespace mk {

// Position of logical 16-byte chunk `c` (0..7) of A row `row` (rows are 128 bytes).  Two rows fill
// the 64 four-byte banks, so pairs of rows share a pattern: any 16 consecutive rows read at the
// same logical chunk hit 16 distinct 16-byte bank groups.
__device__ __forceinline__ int swz(int row, int c) { return c ^ ((row >> 1) & 7); }

typedef short i16x4 __attribute__((ext_vector_type(4)));

template <int BN>
__device__ __forceinline__ int swz_b(int k) {
  constexpr int CPR = BN / 8;  // 16-byte chunks per B row
  if constexpr (CPR >= 16) return 4 * (k & 3);
  else if constexpr (CPR == 8) return 4 * ((k >> 1) & 1);
  else return 0;
}

// Scalar rebase of a buffer window: the window [base + off, base + bytes) (empty if off >= bytes),
// so per-instruction row offsets live in scalar registers instead of per-lane offsets.
// The size goes through readfirstlane: a saturating subtract would otherwise be done on the
// vector ALU and drag the whole resource into VGPRs (a waterfall loop around every DMA).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_at(const char* base, uint32_t bytes, uint32_t off) {
  const uint32_t n = __builtin_amdgcn_readfirstlane(bytes - (off < bytes ? off : bytes));
  return make_rsrc(base + off, n);
}

template <int BM_, int BN_, int WM_, int WN_>
struct TileGemmDma {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int BK = 64;
  static constexpr int NW = WM * WN;  // waves per workgroup
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static_assert(FM * 32 == WTM && FN * 32 == WTN, "wave tile must be a multiple of 32");
  static constexpr int STAGE_A = BM * BK * 2;
  static constexpr int STAGE_B = BN * BK * 2;
  static constexpr int STAGE = STAGE_A + STAGE_B;
  static constexpr int LDS_BYTES = 2 * STAGE;
  static constexpr int A_INSTR = STAGE_A / NW / 1024;  // 1 KiB DMA instructions per wave
  static constexpr int B_INSTR = STAGE_B / NW / 1024;
  static_assert(A_INSTR * NW * 1024 == STAGE_A && B_INSTR * NW * 1024 == STAGE_B,
                "stage must split into 1 KiB per wave");
  static_assert((BM / NW) % 8 == 0, "each wave's A rows form whole 8-row groups");
  static constexpr int ROW_B = BN * 2;  // bytes per B row in LDS
  static_assert(ROW_B <= 1024 && 1024 % ROW_B == 0, "a DMA instruction covers whole B rows");

  f32x16 acc[FM][FN];
  // per-lane address parts, computed once (init): everything else is scalar or an immediate
  uint32_t a_dma[2];   // A DMA byte offset inside an 8-row group (two swizzle phases)
  uint32_t b_dma[4];   // B DMA byte offset inside an instruction's rows (phase = first row & 3)
  uint32_t a_rd[4];    // A operand LDS offset per 16-wide k sub-step
  uint32_t b_rd[FN];   // B operand LDS offset per 32-column fragment

  __device__ __forceinline__ void init(int wm, int wn, int lane, uint32_t lda_b, uint32_t ldb_b) {
    // A DMA: lane -> row lane>>3 of an 8-row group, LDS chunk lane&7 <- global chunk p ^ ((r>>1)&7);
    // the group's first row is a multiple of 8, so the swizzle is ((lane>>4) + 4*(group&1)) & 7.
#pragma unroll
    for (int ph = 0; ph < 2; ++ph) {
      const int x = ((lane >> 4) + 4 * ph) & 7;
      a_dma[ph] = (uint32_t)(lane >> 3) * lda_b + (uint32_t)((lane & 7) ^ x) * 16u;
    }
    // B DMA: lane -> row (lane*16)/ROW_B of the instruction's rows, chunk ((lane*16)%ROW_B)/16.
#pragma unroll
    for (int ph = 0; ph < 4; ++ph) {
      const int kr = (lane * 16) / ROW_B, p = ((lane * 16) % ROW_B) >> 4;
      b_dma[ph] = (uint32_t)kr * ldb_b + (uint32_t)(p ^ swz_b<BN>(ph + kr)) * 16u;
    }
    // A operand: row = wm*WTM + i*32 + (lane&31); the row base is a multiple of 32, so the swizzle
    // term is ((lane&31)>>1)&7; logical chunk 2*kk + (lane>>5).
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int l32 = lane & 31;
      const int kc = 2 * kk + (lane >> 5);
      a_rd[kk] = (uint32_t)(wm * WTM + l32) * 128u + (uint32_t)(swz(l32, kc) * 16);
    }
    // B operand (transposed reads): group g = lane>>4; in-group s: row jr = s>>2 of the 4-row block,
    // 4-column piece q = s&3.  k = kk*16 + 8*(g>>1) + 4*hh + jr, so k&3 = jr.
    {
      const int g = lane >> 4, sidx = lane & 15, jr = sidx >> 2, q = sidx & 3;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int nb = wn * WTN + j * 32 + 16 * (g & 1) + 4 * q;
        b_rd[j] = (uint32_t)(8 * (g >> 1) + jr) * ROW_B + (uint32_t)(((nb >> 3) ^ swz_b<BN>(jr)) << 4) +
                  (uint32_t)((nb & 7) << 1);
      }
    }
  }

  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  }

  // A k-step into stage `lds`: abase points at (row m0, first column of the k-step); a_bytes =
  // bytes from there to the end of the valid rows.
  __device__ __forceinline__ void dma_a(const char* abase, uint32_t a_bytes, uint32_t lda_b, char* lds, int wave) {
#pragma unroll
    for (int i = 0; i < A_INSTR; ++i) {
      const int r0 = wave * (BM / NW) + i * 8;
      const auto rs = rsrc_at(abase, a_bytes, (uint32_t)r0 * lda_b);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(lds + r0 * 128), 16,
                                               a_dma[i & 1], 0, 0, 0);
    }
  }
  // B k-step: bbase points at (row k0, column n0); b_bytes = bytes to the window end.
  __device__ __forceinline__ void dma_b(const char* bbase, uint32_t b_bytes, uint32_t ldb_b, char* lds, int wave) {
#pragma unroll
    for (int i = 0; i < B_INSTR; ++i) {
      const int byte0 = wave * (STAGE_B / NW) + i * 1024;
      const int k0 = byte0 / ROW_B;
      const auto rs = rsrc_at(bbase, b_bytes, (uint32_t)k0 * ldb_b);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(lds + STAGE_A + byte0),
                                               16, b_dma[k0 & 3], 0, 0, 0);
    }
  }

  // One BK = 64 stage of MFMAs for this wave from stage `lds`.  Operand fragments are double
  // buffered across the four 16-wide k sub-steps (reads for sub-step kk+1 are issued before the
  // MFMAs of kk), and a scheduling fence after each sub-step keeps the compiler from hoisting all
  // four sub-steps' reads at once, which would need 128 extra VGPRs.
  __device__ __forceinline__ void load_frags(const char* lds, int kk, bf16x8* af, bf16x8* bfr) {
    const char* lb = lds + STAGE_A;
#pragma unroll
    for (int i = 0; i < FM; ++i) af[i] = *reinterpret_cast<const bf16x8*>(lds + a_rd[kk] + i * 32 * 128);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const i16x4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(const_cast<char*>(lb) + b_rd[j] + (kk * 16 + 0) * ROW_B));
      const i16x4 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(const_cast<char*>(lb) + b_rd[j] + (kk * 16 + 4) * ROW_B));
      bfr[j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  }
  __device__ __forceinline__ void mma(const char* lds) {
    bf16x8 af[2][FM], bfr[2][FN];
    load_frags(lds, 0, af[0], bfr[0]);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (kk + 1 < 4) load_frags(lds, kk + 1, af[(kk + 1) & 1], bfr[(kk + 1) & 1]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[kk & 1][i], bfr[kk & 1][j], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Epilogue through LDS: each wave stages one 32-row slab of its sub-tile at a time (rows of
  // WTN + 8 floats, so row pairs 4 apart land 128 bytes apart) and hands out row-contiguous
  // float4s, f(row_in_tile, col_in_tile, value), so the caller issues 16-byte coalesced global
  // accesses.  The first half of the waves stage in `st_lo`, the second half in `st_hi` (each a
  // different stage buffer, so the slabs fit after the mainloop).  The caller must have passed a
  // barrier after the last mma() and must barrier again before the stage buffers are reused.
  static constexpr int EPI_STRIDE = WTN + 8;
  static constexpr int EPI_WAVE = 32 * EPI_STRIDE * 4;
  static_assert((NW / 2) * EPI_WAVE <= STAGE, "half the waves' staging must fit in one stage buffer");
  template <class F>
  __device__ __forceinline__ void epilogue(char* st_lo, char* st_hi, int wm, int wn, int lane_in, int wave, F&& f) {
    // The staging addresses do not depend on the tile; an opaque copy of the lane id stops the
    // compiler from hoisting all of them out of the persistent tile loop (64+ live registers).
    int lane = lane_in;
    asm volatile("" : "+v"(lane));
    float* wl = reinterpret_cast<float*>((wave < NW / 2 ? st_lo : st_hi) + (wave % (NW / 2)) * EPI_WAVE);
    constexpr int C4 = WTN / 4;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          wl[(8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * EPI_STRIDE + j * 32 + (lane & 31)] = acc[i][j][r];
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int q = 0; q < (32 * C4) / 64; ++q) {
        const int idx = q * 64 + lane;
        const int row = idx / C4, c4 = idx - row * C4;
        const f32x4 v = *reinterpret_cast<const f32x4*>(wl + row * EPI_STRIDE + c4 * 4);
        f(wm * WTM + i * 32 + row, wn * WTN + c4 * 4, v);
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_wave_barrier();
    }
  }

  // As epilogue(), but hands `f` all of this lane's values of one 32-row slab at once, so an
  // epilogue that loads other data per value (peer partials) can have all those loads in flight
  // together: f(slab_row0, v, rows, cols) with SLAB_Q values; rows and cols are tile-relative and
  // slab_row0 is the slab's first row.
  static constexpr int SLAB_Q = (32 * (WTN / 4)) / 64;
  template <class F>
  __device__ __forceinline__ void epilogue_slab(char* st_lo, char* st_hi, int wm, int wn, int lane_in, int wave,
                                                F&& f) {
    int lane = lane_in;
    asm volatile("" : "+v"(lane));
    float* wl = reinterpret_cast<float*>((wave < NW / 2 ? st_lo : st_hi) + (wave % (NW / 2)) * EPI_WAVE);
    constexpr int C4 = WTN / 4;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          wl[(8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * EPI_STRIDE + j * 32 + (lane & 31)] = acc[i][j][r];
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_wave_barrier();
      f32x4 v[SLAB_Q];
      int rows[SLAB_Q], cols[SLAB_Q];
#pragma unroll
      for (int q = 0; q < SLAB_Q; ++q) {
        const int idx = q * 64 + lane;
        const int row = idx / C4, c4 = idx - row * C4;
        v[q] = *reinterpret_cast<const f32x4*>(wl + row * EPI_STRIDE + c4 * 4);
        rows[q] = wm * WTM + i * 32 + row;
        cols[q] = wn * WTN + c4 * 4;
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_wave_barrier();
      f(wm * WTM + i * 32, v, rows, cols);
    }
  }
};

// s_waitcnt immediate that waits until at most `n` vector-memory operations of this wave are
// outstanding (expcnt / lgkmcnt left unconstrained).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N <= 63, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Three-stage K loop over static stage buffers st0..st2: the DMA for step q+2 is issued before
// the MFMAs of step q, and the end-of-step wait leaves that newest step's loads in flight, so
// every load has two steps of MFMA work to land.  `load(step, stage)` issues one step's DMA
// (DMA_PER_STEP instructions per wave); `before_wait(q)` runs after the MFMAs of step q.
template <class G, class Load, class After>
__device__ __forceinline__ void k_loop3(G& g, int nk, char* st0, char* st1, char* st2, Load&& load,
                                        After&& before_wait) {
  k_loop3(g, nk, st0, st1, st2, [](int) {}, load, before_wait);
}

// As above, with `before_load(q)` run at the start of step q, before the step's DMA is issued.
template <class G, class Pre, class Load, class After>
__device__ __forceinline__ void k_loop3(G& g, int nk, char* st0, char* st1, char* st2, Pre&& before_load,
                                        Load&& load, After&& before_wait) {
  constexpr int D = G::A_INSTR + G::B_INSTR;
  load(0, st0);
  if (nk > 1) {
    load(1, st1);
    wait_vm<D>();
  } else {
    wait_vm<0>();
  }
  __syncthreads();
  auto sub = [&](int q, char* cur, char* pf) {
    if (q >= nk) return;
    const bool more = q + 2 < nk;
    before_load(q);
    if (more) load(q + 2, pf);
    g.mma(cur);
    before_wait(q);
    if (more) wait_vm<D>();
    else wait_vm<0>();
    __syncthreads();
  };
  for (int q = 0; q < nk; q += 3) {
    sub(q, st0, st2);
    sub(q + 1, st1, st0);
    sub(q + 2, st2, st1);
  }
}

// Two-stage K loop for tiles whose stage is too large for three buffers: the DMA for step q+1 is
// issued before the MFMAs of step q and must land by the end of that step.
template <class G, class Pre, class Load, class After>
__device__ __forceinline__ void k_loop2(G& g, int nk, char* st0, char* st1, Pre&& before_load, Load&& load,
                                        After&& before_wait) {
  load(0, st0);
  wait_vm<0>();
  __syncthreads();
  auto sub = [&](int q, char* cur, char* pf) {
    if (q >= nk) return;
    before_load(q);
    if (q + 1 < nk) load(q + 1, pf);
    g.mma(cur);
    before_wait(q);
    wait_vm<0>();
    __syncthreads();
  };
  for (int q = 0; q < nk; q += 2) {
    sub(q, st0, st1);
    sub(q + 1, st1, st0);
  }
}

// Waits until at most n steps' DMA (D instructions each) of this wave are outstanding, n in [0, 3].
template <int D>
__device__ __forceinline__ void wait_steps(int n) {
  switch (n) {
    case 3: wait_vm<3 * D>(); break;
    case 2: wait_vm<2 * D>(); break;
    case 1: wait_vm<D>(); break;
    default: wait_vm<0>(); break;
  }
}

// Five-stage K loop over static stage buffers st0..st4, for tiles whose stages are small: the DMA
// for step q+4 is issued before the MFMAs of step q (into the buffer step q-1 read, which every
// wave left at the previous barrier), and the end-of-step wait leaves the three newest steps'
// loads in flight, so a CU has four steps of loads outstanding at the top of each step.
template <class G, class Pre, class Load, class After>
__device__ __forceinline__ void k_loop5(G& g, int nk, char* st0, char* st1, char* st2, char* st3, char* st4,
                                        Pre&& before_load, Load&& load, After&& before_wait) {
  constexpr int S = 5, D = G::A_INSTR + G::B_INSTR;
  static_assert((S - 2) * D <= 63, "vmcnt is 6 bits");
  load(0, st0);
  if (nk > 1) load(1, st1);
  if (nk > 2) load(2, st2);
  if (nk > 3) load(3, st3);
  wait_steps<D>(min(S - 1, nk) - 1);  // step 0 has landed
  __syncthreads();
  auto sub = [&](int q, char* cur, char* pf) {
    if (q >= nk) return;
    before_load(q);
    if (q + S - 1 < nk) load(q + S - 1, pf);
    g.mma(cur);
    before_wait(q);
    // step q+1 must have landed: the steps issued after it may stay in flight
    wait_steps<D>(max(0, min(S - 2, nk - 2 - q)));
    __syncthreads();
  };
  for (int q = 0; q < nk; q += S) {
    sub(q, st0, st4);
    sub(q + 1, st1, st0);
    sub(q + 2, st2, st1);
    sub(q + 3, st3, st2);
    sub(q + 4, st4, st3);
  }
}

// Stage buffers a tile's K loop uses: five when they fit in 120 KiB (small tiles, whose loads
// would otherwise be latency-bound), else three when they fit in the 160 KiB of LDS beside a few
// KiB of bookkeeping, else two.
template <class G>
constexpr int k_stages() {
  return 5 * G::STAGE <= 120 * 1024 ? 5 : 3 * G::STAGE <= 150 * 1024 ? 3 : 2;
}

// The K loop for tile G on its stage count (buffers past that count are unused).
template <class G, class Pre, class Load, class After>
__device__ __forceinline__ void k_loop(G& g, int nk, char* st0, char* st1, char* st2, char* st3, char* st4,
                                       Pre&& before_load, Load&& load, After&& before_wait) {
  if constexpr (k_stages<G>() == 5)
    k_loop5(g, nk, st0, st1, st2, st3, st4, before_load, load, before_wait);
  else if constexpr (k_stages<G>() == 3)
    k_loop3(g, nk, st0, st1, st2, before_load, load, before_wait);
  else
    k_loop2(g, nk, st0, st1, before_load, load, before_wait);
}

}  // namespace mk
