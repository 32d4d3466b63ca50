// Tile constants shared by the host planner (plain C++) and the gfx950 kernels.
#pragma once

namespace convfwd {

// Tile shape of the generic implicit GEMM kernel.
constexpr int IG_TILE_P = 64;   // output pixels per workgroup
constexpr int IG_TILE_C = 64;   // output channels per workgroup
constexpr int IG_KSTEP_BYTES = 64;  // k-block: 32 halves or 16 floats

// Halo kernel (f16): LDS bytes per pipeline buffer (input tile + weight tile);
// two buffers are allocated statically.
constexpr int HALO_BUF_BYTES = 40 * 1024;
constexpr int HALO_MAXT = 8;  // 16x16 MFMA output tiles per wave
constexpr int HALO_MAXI = 8;  // staged (position, octet) input items per thread

}  // namespace convfwd
