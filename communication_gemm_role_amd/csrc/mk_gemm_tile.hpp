// Compute role core: one BM x BN fp32 output tile of C = A @ B with bf16 operands on
// gfx950 MFMA (v_mfma_f32_32x32x16_bf16), LDS-staged and double-buffered over BK = 64.
//
//   A  row-major [M, K] bf16 (K contiguous)  -> LDS [BM][64], 16-byte chunks XOR-swizzled
//   B  row-major [K, N] bf16 (N contiguous)  -> LDS [BN][64] (transposed, K contiguous):
//      each thread loads an 8 (k) x 8 (n) block as eight 16-byte row pieces and transposes
//      it in registers, so both MFMA operands are read as 16-byte K-runs per lane.
//
// 256 threads = 4 waves arranged WM x WN; wave (wm, wn) owns a (BM/WM) x (BN/WN) sub-tile
// made of 32 x 32 MFMA fragments.  MFMA lane layout (checked on the device): for the
// A operand lane l holds row l%32, k = 8*(l/32) .. +7 of a 32 x 16 slab; the B operand
// holds column l%32 with the same k; accumulator element r of lane l is
// row 8*(r/4) + 4*(l/32) + r%4, column l%32 of the 32 x 32 fragment.
#pragma once
#include "mk_device.hpp"

namespace mk {

// Position of logical 16-byte chunk `c` (0..7) of LDS row `row` (rows are 128 bytes).
// Two rows fill the 64 four-byte banks, so pairs of rows share a pattern: any 16
// consecutive rows read at the same logical chunk hit 16 distinct 16-byte bank groups.
__device__ __forceinline__ int swz(int row, int c) { return c ^ ((row >> 1) & 7); }

template <int BM_, int BN_, int WM_, int WN_>
struct TileGemm {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int BK = 64;
  static constexpr int NT = 256;
  static_assert(WM * WN == 4, "4 waves");
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static_assert(FM * 32 == WTM && FN * 32 == WTN, "wave tile must be a multiple of 32");
  static constexpr int A_PER_T = (BM * 8) / NT;  // 16-byte chunks of A per thread per stage
  static_assert(A_PER_T * NT == BM * 8, "BM must be a multiple of 32");
  static constexpr int B_BLOCKS = BN;            // 8x8 blocks per stage: (64/8) * (BN/8)
  static constexpr int B_PER_T = (B_BLOCKS + NT - 1) / NT;
  static constexpr int STAGE_A = BM * BK * 2;
  static constexpr int STAGE_B = BN * BK * 2;
  static constexpr int STAGE = STAGE_A + STAGE_B;
  static constexpr int LDS_BYTES = 2 * STAGE;

  u32x4 ra[A_PER_T];
  u32x4 rb[B_PER_T][8];
  f32x16 acc[FM][FN];

  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  }

  // A: rsrc based at row m0 of A; lda_b = row stride in bytes; kb0 = byte offset of the k-step.
  __device__ __forceinline__ void load_a(__amdgpu_buffer_rsrc_t ar, uint32_t lda_b, uint32_t kb0, int tid) {
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
      const int idx = tid + i * NT;
      const int r = idx >> 3, c = idx & 7;
      ra[i] = bload16(ar, (uint32_t)r * lda_b + kb0 + (uint32_t)c * 16u);
    }
  }
  __device__ __forceinline__ void store_a(char* lds_a, int tid) {
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
      const int idx = tid + i * NT;
      const int r = idx >> 3, c = idx & 7;
      *reinterpret_cast<u32x4*>(lds_a + r * 128 + swz(r, c) * 16) = ra[i];
    }
  }
  // B: rsrc based at column n0 of B (row 0); ldb_b = row stride in bytes; k0 = first k row.
  __device__ __forceinline__ void load_b(__amdgpu_buffer_rsrc_t br, uint32_t ldb_b, int k0, int tid) {
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) {
      const int blk = tid + i * NT;
      if (B_BLOCKS % NT == 0 || blk < B_BLOCKS) {
        const int kb = blk & 7, nb = blk >> 3;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          rb[i][j] = bload16(br, (uint32_t)(k0 + kb * 8 + j) * ldb_b + (uint32_t)nb * 16u);
      }
    }
  }
  __device__ __forceinline__ void store_b(char* lds_b, int tid) {
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) {
      const int blk = tid + i * NT;
      if (B_BLOCKS % NT == 0 || blk < B_BLOCKS) {
        const int kb = blk & 7, nb = blk >> 3;
        // rb[i][j] holds k = kb*8 + j; its dword d holds n = nb*8 + 2d (low half), 2d+1 (high half)
#pragma unroll
        for (int nn = 0; nn < 8; ++nn) {
          const int d = nn >> 1;
          u32x4 o;
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const uint32_t lo = rb[i][2 * p][d], hi = rb[i][2 * p + 1][d];
            o[p] = (nn & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
          }
          const int row = nb * 8 + nn;
          *reinterpret_cast<u32x4*>(lds_b + row * 128 + swz(row, kb) * 16) = o;
        }
      }
    }
  }

  // One BK = 64 stage of MFMAs for wave (wm, wn).
  __device__ __forceinline__ void mma(const char* lds_a, const char* lds_b, int wm, int wn, int lane) {
    const int l32 = lane & 31, lh = lane >> 5;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int kc = kk * 2 + lh;
      bf16x8 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int row = wm * WTM + i * 32 + l32;
        af[i] = *reinterpret_cast<const bf16x8*>(lds_a + row * 128 + swz(row, kc) * 16);
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int row = wn * WTN + j * 32 + l32;
        bfr[j] = *reinterpret_cast<const bf16x8*>(lds_b + row * 128 + swz(row, kc) * 16);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }

  // Epilogue through LDS: each wave stages one 32-row slab of its sub-tile at a time and hands
  // out row-contiguous float4s, f(row_in_tile, col_in_tile, value), so the caller issues 16-byte
  // coalesced global accesses.  Needs EPI_LDS bytes of LDS; the caller must have passed a barrier
  // after the last mma() and must barrier again before LDS is reused.
  static constexpr int EPI_STRIDE = WTN + 8;  // floats; row pairs 4 apart land 128 bytes apart
  static constexpr int EPI_LDS = 4 * 32 * EPI_STRIDE * 4;
  static_assert(EPI_LDS <= LDS_BYTES, "epilogue staging must fit in the mainloop LDS");
  template <class F>
  __device__ __forceinline__ void epilogue(char* lds, int wm, int wn, int lane, int wave, F&& f) {
    float* wl = reinterpret_cast<float*>(lds) + wave * 32 * EPI_STRIDE;
    constexpr int C4 = WTN / 4;  // float4s per staged row
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          wl[(8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * EPI_STRIDE + j * 32 + (lane & 31)] = acc[i][j][r];
      __builtin_amdgcn_s_waitcnt(0xc07f & ~0x0f00);  // lgkmcnt(0): staged values are in LDS
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int q = 0; q < (32 * C4) / 64; ++q) {
        const int idx = q * 64 + lane;
        const int row = idx / C4, c4 = idx - row * C4;
        const f32x4 v = *reinterpret_cast<const f32x4*>(wl + row * EPI_STRIDE + c4 * 4);
        f(wm * WTM + i * 32 + row, wn * WTN + c4 * 4, v);
      }
      __builtin_amdgcn_s_waitcnt(0xc07f & ~0x0f00);
      __builtin_amdgcn_wave_barrier();
    }
  }

  // Row / column (inside the tile) of accumulator element r of fragment (i, j) for this lane.
  __device__ __forceinline__ static int acc_row(int wm, int i, int r, int lane) {
    return wm * WTM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
  }
  __device__ __forceinline__ static int acc_col(int wn, int j, int lane) { return wn * WTN + j * 32 + (lane & 31); }
};

}  // namespace mk
