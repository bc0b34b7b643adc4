// Compute role core on v_mfma_f32_16x16x32_bf16: one 256 x BN fp32 output tile of C = A @ B with
// bf16 operands, eight waves of 64 x BN/2 (4 x BN/32 fragments of 16 x 16).  BN = 224 serves the
// AllGather + GEMM kernel (at N = 1792 the 224-column tiles give 32 x 8 = 256 tiles, one per CU
// of an MI355X); BN = 256 the GEMM + ReduceScatter / AllReduce kernel on wide outputs.
//
// MFMA lane layout (16 x 16 x 32, checked on the device against the 32 x 32 x 16 core): the A
// operand of lane l is row l%16, k = 8*(l/16) .. +7; the B operand is column l%16 with the same
// k; accumulator element r of lane l is row 4*(l/16) + r, column l%16.
//
// Operands go global -> LDS by buffer_load ... lds, 16 bytes per lane.  LDS per k-step of 64:
//   A slot  256 rows x 128 B (32 KiB); 16-byte chunks XOR-swizzled by row pair (chunk p of row r
//           holds global chunk p ^ ((r >> 1) & 7)), so 16 lanes reading one logical chunk of 16
//           consecutive rows hit 64 distinct banks;
//   B slot  64 k-rows x BN * 2 bytes.  BN = 224: not swizzled; a 16-lane group of a transposed
//           read covers four consecutive k-rows, whose 448-byte rows start 48 banks apart, so the
//           group's 32 bytes per row fall in four disjoint bank ranges (measured: an XOR swizzle of
//           the chunks by k-row block changed neither the LDS bank-conflict counter nor the time),
//           and a fragment's address is one base plus 32 bytes per fragment.  BN = 256: 512-byte
//           rows start on the same bank, so chunk p of k-row r holds global chunk p ^ 2 key(r),
//           key(r) = (r & 3) | ((r >> 1) & 4): the four rows of a group land 32 bytes apart and the
//           two groups that share a read cycle in the other half of the banks; fragment j's
//           address is the lane's base XOR 32 j.
// The B operand is read with ds_read_b64_tr_b16: in each 16-lane group, lane i receives element
// i%4 of the 8-byte pieces addressed by lanes 4j + i/4 (j = 0..3); a group reading k-rows
// 8g + j, columns 4q..4q+3 (lane 4j + q) gives lane i column i of those four k-rows, and a second
// read four rows down completes the lane's 8 consecutive k.
//
// The K loop (k_loop_a3b2) keeps A in three slots loaded two steps ahead and B in two slots one
// step ahead (3 x 32 KiB + 2 x 28 or 32 KiB): the A rows of a tile row are shared by the tiles of
// one XCD and come from HBM, so they get the longer lead.
#pragma once
#include "mk_gemm_tile.hpp"

namespace mk {

template <int BN_>
struct TileGemm16T {
  static constexpr int BM = 256, BN = BN_, BK = 64;
  static constexpr int WM = 4, WN = 2, NW = WM * WN;
  static constexpr int WTM = BM / WM, WTN = BN / WN, FM = WTM / 16, FN = WTN / 16;
  static_assert(BN == 224 || BN == 256, "the layout below is written for 256 x 224 and 256 x 256");
  static constexpr int ROW_A = BK * 2, ROW_B = BN * 2;  // bytes per LDS row
  static constexpr int SLOT_A = BM * ROW_A;              // 32 KiB
  static constexpr int SLOT_B = BK * ROW_B;              // 28 or 32 KiB
  static constexpr int A_INSTR = SLOT_A / NW / 1024;     // 1 KiB DMA instructions per wave and step
  static constexpr int B_INSTR = SLOT_B / 1024;          // per step: 28 (waves 0-3 issue 4, waves 4-7
                                                         // issue 3) or 32 (4 per wave)
  static constexpr bool SWZ_B = ROW_B % 256 == 0;        // B rows start on the same bank: swizzle
  static_assert(A_INSTR == 4 && (B_INSTR == 28 || B_INSTR == 32), "A: 4 per wave; B: at most 4 per wave");

  f32x4 acc[FM][FN];
  uint32_t a_dma[2];   // A DMA byte offset inside an 8-row group (two swizzle phases)
  uint32_t b_dma[4];   // B DMA byte offset inside the step's rows, per instruction of this wave
  uint32_t a_rd[2];    // A operand LDS offset per 32-wide k sub-step
  uint32_t b_rd;       // B operand LDS offset of fragment 0's first transposed read (fragment j:
                       // + 32 j, or XOR 32 j when swizzled)

  // first LDS KiB of this wave's B instructions: 4 each, or (28 per step) waves 0-3 take 4 and
  // waves 4-7 take 3
  __device__ static int b_ins(int wave, int i) {
    return (B_INSTR == 32 || wave < 4) ? 4 * wave + i : 16 + 3 * (wave - 4) + i;
  }
  // B swizzle key of k-row r (swizzled layout only)
  __device__ static int b_key(int r) { return (r & 3) | ((r >> 1) & 4); }

  __device__ __forceinline__ void init(int wm, int wn, int wave, int lane, uint32_t lda_b, uint32_t ldb_b) {
#pragma unroll
    for (int ph = 0; ph < 2; ++ph) {
      const int x = ((lane >> 4) + 4 * ph) & 7;
      a_dma[ph] = (uint32_t)(lane >> 3) * lda_b + (uint32_t)((lane & 7) ^ x) * 16u;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int o = b_ins(wave, i) * 1024 + lane * 16;  // LDS byte of this lane's chunk
      const int r = o / ROW_B, p = (o % ROW_B) >> 4;
      b_dma[i] = (uint32_t)r * ldb_b + (uint32_t)(SWZ_B ? p ^ (2 * b_key(r)) : p) * 16u;
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int row = wm * WTM + (lane & 15);
      const int c = 4 * s + (lane >> 4);
      a_rd[s] = (uint32_t)row * ROW_A + (uint32_t)((c ^ ((row >> 1) & 7)) * 16);
    }
    const int g = lane >> 4, jr = (lane & 15) >> 2, q = lane & 3;
    // lane 4 jr + q of group g: k-row 8 g + jr (the second read four rows down, the same key),
    // columns 4q .. 4q+3; swizzled, the key sits in bits 5-7, which no other term touches
    b_rd = (uint32_t)(8 * g + jr) * ROW_B + (uint32_t)(wn * WTN + 4 * q) * 2u +
           (SWZ_B ? 32u * (uint32_t)b_key(8 * g + jr) : 0u);
  }

  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // A k-step into slot `la`: abase points at (row m0, the step's first column); a_bytes = bytes from
  // there to the end of the valid rows (rows past it read as zeros).
  __device__ __forceinline__ void dma_a(const char* abase, uint32_t a_bytes, uint32_t lda_b, char* la, int wave) {
#pragma unroll
    for (int i = 0; i < A_INSTR; ++i) {
      const int r0 = wave * (BM / NW) + i * 8;
      const auto rs = rsrc_at(abase, a_bytes, (uint32_t)r0 * lda_b);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(la + r0 * ROW_A), 16,
                                               a_dma[i & 1], 0, 0, 0);
    }
  }
  // B k-step into slot `lb`: bbase points at (the step's first k-row, column n0); b_bytes = bytes from
  // there to the end of the window (columns past the matrix read as zeros only at its very end; the
  // caller clips ragged columns at the store).
  __device__ __forceinline__ void dma_b(const char* bbase, uint32_t b_bytes, char* lb, int wave) {
    const auto rs = make_rsrc(bbase, __builtin_amdgcn_readfirstlane(b_bytes));
#pragma unroll
    for (int i = 0; i < 3; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(lb + b_ins(wave, i) * 1024),
                                               16, b_dma[i], 0, 0, 0);
    if (B_INSTR == 32 || wave < 4)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(lb + b_ins(wave, 3) * 1024),
                                               16, b_dma[3], 0, 0, 0);
  }

  // Unswizzled: fragment j at lb + b_rd + 32 j (an immediate offset).  Swizzled: at
  // (lb + b_rd) XOR 32 j, where bb = lb + b_rd is the LDS address of fragment 0 (the B slot is
  // 256-byte aligned, so the slot base leaves bits 5-7 to the key); bb is recomputed per step
  // behind an opaque copy, so the compiler does not keep eight fragment addresses per slot alive.
  __device__ static uint32_t lds_u32(const char* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
  }
  __device__ __forceinline__ void b_frag(const char* lb, uint32_t bb, int s, int j, bf16x8& bf) {
    typedef __attribute__((address_space(3))) i16x4* lp;
    i16x4 h0, h1;
    if constexpr (SWZ_B) {
      // the address as an offset from lb keeps the read's provenance (the slot), so the
      // compiler's wait insertion can see that it never aliases the DMA into the other slots
      const char* f = lb + ((bb ^ (32u * (uint32_t)j)) - lds_u32(lb));
      h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(const_cast<char*>(f) + (32 * s) * ROW_B));
      h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(const_cast<char*>(f) + (32 * s + 4) * ROW_B));
    } else {
      h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(const_cast<char*>(lb) + b_rd + 32 * j + (32 * s) * ROW_B));
      h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(const_cast<char*>(lb) + b_rd + 32 * j + (32 * s + 4) * ROW_B));
    }
    bf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7));
  }
  // One k-step of 64: two sub-steps of 32, one sub-step's fragments live at a time (the other wave
  // of the SIMD issues MFMAs while this one waits for its LDS reads; measured as fast as reading
  // the second sub-step's fragments ahead, with 44 fewer live registers).
  // BN = 256 reads B in two halves of four fragments (16 fewer live registers).
  static constexpr int FH = FN == 8 ? 4 : FN;  // B fragments per read group
  __device__ __forceinline__ void mma(const char* la, const char* lb) {
    uint32_t bb = 0;
    if constexpr (SWZ_B) {
      bb = lds_u32(lb) + b_rd;
      asm volatile("" : "+v"(bb));
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x8 af[FM];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = *reinterpret_cast<const bf16x8*>(la + a_rd[s] + i * 16 * ROW_A);
#pragma unroll
      for (int h = 0; h < FN; h += FH) {
        bf16x8 bf[FH];
#pragma unroll
        for (int j = 0; j < FH; ++j) b_frag(lb, bb, s, h + j, bf[j]);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FH; ++j)
            acc[i][h + j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf[j], acc[i][h + j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // Epilogue: each wave stages one 16-row slab of its sub-tile at a time in `wl` (16 x WTN floats,
  // rows padded by 4) and hands out row-contiguous float4s f(row_in_tile, col_in_tile, value).
  // epi_buf: a wave's staging area, three waves per A slot (the K loop has drained every slot).
  static constexpr int EPI_STRIDE = WTN + 4;
  static constexpr int EPI_WAVE = 16 * EPI_STRIDE * 4;  // 7424 or 8448 bytes
  static_assert(3 * EPI_WAVE <= SLOT_A, "three waves' staging fits one A slot");
  __device__ static float* epi_buf(int wave, char* a0, char* a1, char* a2) {
    char* slot = wave < 3 ? a0 : wave < 6 ? a1 : a2;
    return reinterpret_cast<float*>(slot + (wave % 3) * EPI_WAVE);
  }
  template <class F>
  __device__ __forceinline__ void epilogue(float* wl, int wm, int wn, int lane_in, F&& f) {
    int lane = lane_in;  // opaque copy: keeps the staging addresses out of the persistent loop
    asm volatile("" : "+v"(lane));
    constexpr int C4 = WTN / 4;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) wl[(4 * (lane >> 4) + r) * EPI_STRIDE + j * 16 + (lane & 15)] = acc[i][j][r];
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int q = 0; q < (16 * C4) / 64; ++q) {
        const int idx = q * 64 + lane;
        const int row = idx / C4, c4 = idx - row * C4;
        f(wm * WTM + i * 16 + row, wn * WTN + c4 * 4, *reinterpret_cast<const f32x4*>(wl + row * EPI_STRIDE + c4 * 4));
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_wave_barrier();
    }
  }

  // As epilogue(), but hands `f` all of this lane's values of one 16-row slab at once, so an
  // epilogue that loads other data per value (peer partials) can have all those loads in flight
  // together: f(slab_row0, v, rows, cols) with SLAB_Q values; rows and cols are tile-relative.
  static constexpr int SLAB_Q = (16 * (WTN / 4)) / 64;
  template <class F>
  __device__ __forceinline__ void epilogue_slab(float* wl, int wm, int wn, int lane_in, F&& f) {
    int lane = lane_in;
    asm volatile("" : "+v"(lane));
    constexpr int C4 = WTN / 4;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) wl[(4 * (lane >> 4) + r) * EPI_STRIDE + j * 16 + (lane & 15)] = acc[i][j][r];
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_wave_barrier();
      f32x4 v[SLAB_Q];
      int rows[SLAB_Q], cols[SLAB_Q];
#pragma unroll
      for (int q = 0; q < SLAB_Q; ++q) {
        const int idx = q * 64 + lane;
        const int row = idx / C4, c4 = idx - row * C4;
        v[q] = *reinterpret_cast<const f32x4*>(wl + row * EPI_STRIDE + c4 * 4);
        rows[q] = wm * WTM + i * 16 + row;
        cols[q] = wn * WTN + c4 * 4;
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_wave_barrier();
      f(wm * WTM + i * 16, v, rows, cols);
    }
  }
};

using TileGemm16 = TileGemm16T<mk_tiles::kAg16.bn>;  // AllGather + GEMM
static_assert(mk_tiles::kAg16.bm == 256 && mk_tiles::kAg16.wm == 4 && mk_tiles::kAg16.wn == 2, "kAg16 is this core");

// K loop over three A slots (a0..a2, loaded two steps ahead) and two B slots (b0, b1, one step
// ahead).  Step q issues B(q+1) and then A(q+2), runs the MFMAs of step q, and waits until only
// A(q+2) may still be in flight, so every A load has two steps of MFMA work to land and every B
// load one.  prologue(a0, b0, a1) issues A(0), B(0) and, when nk > 1, A(1), in that order;
// load_a(step, slot) / load_b(step, slot) issue one step's DMA.  Hooks for the emulated arrival,
// each called with a Phase tag: before_load(q, ph) runs before the step's DMA, after_load(q, ph)
// right after it (before the MFMAs), before_wait(q, ph) after the MFMAs.
// The steady state runs in groups of six steps (the slot pattern's period) with no condition
// inside a step, so the compiler's wait insertion sees straight-line code and leaves the A loads
// in flight; the last steps run with conditions.  It has two phases: groups with the hooks'
// full work (Phase<true>) while leave() is false -- evaluated between groups, uniform across the
// workgroup -- and then groups with Phase<false>, whose hooks do the light part only, so that the
// heavy part's code and registers stay out of the rest of the loop.  The last steps run with
// Phase<true>.  Barriers carry no memory fence: the explicit vmcnt wait orders the DMA, and
// lgkmcnt(0) retires this wave's LDS reads of the slot that the next step overwrites.
template <bool HEAVY>
struct Phase {
  static constexpr bool heavy = HEAVY;
};

template <class G, class Prologue, class LoadA, class LoadB, class Pre, class Post, class After, class Leave>
__device__ __forceinline__ void k_loop_a3b2(G& g, int nk, char* a0, char* a1, char* a2, char* b0, char* b1,
                                            Prologue&& prologue, LoadA&& load_a, LoadB&& load_b, Pre&& before_load,
                                            Post&& after_load, After&& before_wait, Leave&& leave) {
  constexpr int DA = G::A_INSTR;
  prologue(a0, b0, a1);
  if (nk > 1) wait_vm<DA>();
  else wait_vm<0>();
  __syncthreads();
  auto step = [&](auto ph, int q, char* ca, char* cb, char* pa, char* pb) {
    before_load(q, ph);
    load_b(q + 1, pb);
    load_a(q + 2, pa);
    after_load(q, ph);
    g.mma(ca, cb);
    before_wait(q, ph);
    wait_vm<DA>();
    __builtin_amdgcn_s_waitcnt(0xc07f);
    barrier_only();
  };
  auto group = [&](auto ph, int q) {
    step(ph, q + 0, a0, b0, a2, b1);
    step(ph, q + 1, a1, b1, a0, b0);
    step(ph, q + 2, a2, b0, a1, b1);
    step(ph, q + 3, a0, b1, a2, b0);
    step(ph, q + 4, a1, b0, a0, b1);
    step(ph, q + 5, a2, b1, a1, b0);
  };
  auto last = [&](int q, char* ca, char* cb, char* pa, char* pb) {
    if (q >= nk) return;
    before_load(q, Phase<true>{});
    if (q + 1 < nk) load_b(q + 1, pb);
    const bool more = q + 2 < nk;
    if (more) load_a(q + 2, pa);
    after_load(q, Phase<true>{});
    g.mma(ca, cb);
    before_wait(q, Phase<true>{});
    if (more) wait_vm<DA>();
    else wait_vm<0>();
    __builtin_amdgcn_s_waitcnt(0xc07f);
    barrier_only();
  };
  int q = 0;
  for (; q + 8 <= nk && !leave(); q += 6) group(Phase<true>{}, q);
  for (; q + 8 <= nk; q += 6) group(Phase<false>{}, q);
  // at most seven steps remain, starting at slot phase 0
  last(q + 0, a0, b0, a2, b1);
  last(q + 1, a1, b1, a0, b0);
  last(q + 2, a2, b0, a1, b1);
  last(q + 3, a0, b1, a2, b0);
  last(q + 4, a1, b0, a0, b1);
  last(q + 5, a2, b1, a1, b0);
  last(q + 6, a0, b0, a2, b1);
  wait_vm<0>();
  __syncthreads();
}

}  // namespace mk
