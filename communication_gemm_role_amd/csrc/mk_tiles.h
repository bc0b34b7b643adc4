// Tile geometry of the compute roles, shared by the kernels (TileGemmDma instantiations) and by the
// host-only build of the planning checks, so the two cannot drift apart.  Plain C++, no HIP.
#pragma once

namespace mk_tiles {

struct Shape {
  int bm, bn;    // output tile rows, columns
  int wm, wn;    // waves along rows, columns (bm / wm and bn / wn are multiples of 16)
  int ring_kib;  // copy ring: KiB per wave and batch (its slots are the first two stage buffers)
  constexpr int waves() const { return wm * wn; }
};

constexpr Shape kAg16{256, 224, 4, 2, 4};       // AllGather + GEMM and the MLP up-projection (16 x 16 x 32 core)
constexpr Shape kRedBig{256, 256, 4, 2, 4};     // GEMM + RS / AR with wide outputs, MLP down-projection
constexpr Shape kRedSkinny{128, 64, 4, 1, 8};   // GEMM + RS / AR with few output rows (decode-like)
constexpr int kRedSkinnyMaxRows = 512;       // outputs of at most this many rows take the skinny tile
constexpr Shape kMoe{256, 256, 4, 2, 8};        // MoE grouped GEMM (16 x 16 x 32 core; ring: 8 KiB per wave)

constexpr bool red_skinny(int m) { return m <= kRedSkinnyMaxRows; }
constexpr const Shape& red_shape(int m) { return red_skinny(m) ? kRedSkinny : kRedBig; }

}  // namespace mk_tiles
