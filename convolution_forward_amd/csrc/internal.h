// Internal interface between the host planner (conv_host.cpp) and the gfx950
// kernels (*.hip).  Not part of the public ABI.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

#include "tiles.h"

namespace convfwd {

enum Dtype { F32 = 0, F16 = 1, BF16 = 2 };

// Output modes of the matrix kernels.
enum OutMode {
  OUT_FUSED = 0,  // bias, residual, activation, store y in the operand dtype
  OUT_RAW = 1     // raw float32 sums into a plane of the scratch (split k, ConvT columns)
};

// Division by a launch constant d >= 1 as multiply-high, add and shift
// (Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994, with l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1):
// floor(n / d) = (umulhi(m, n) + n) >> l, exact for every 0 <= n < 2^31.
struct Magic {
  unsigned m;
  int s;
};

inline Magic make_magic(unsigned d) {
  int l = 0;
  while ((1ull << l) < d) ++l;
  Magic g;
  g.m = (unsigned)(((1ull << 32) * ((1ull << l) - d)) / d + 1);
  g.s = l;
  return g;
}

// Geometry and operands of one implicit-GEMM launch (one image chunk).
// Element pointers already include the problem's element offsets.
struct IgemmArgs {
  const void* x;
  const void* wt;      // weights
  const void* bias;      // nullptr when absent
  const void* res;       // nullptr when absent
  void* y;               // OUT_FUSED target
  float* planes;         // OUT_RAW target: plane r at planes + r * plane_stride
  int n, c_in, h, w;     // input (n = images in this chunk)
  int c_out, kh, kw, groups;
  int sh, sw, dh, dw, pt, pl;
  int ho, wo;
  int cig, cog;          // channels per group (cog = GEMM columns per group)
  int kg;                // reduction length per group
  int pix;               // n * ho * wo
  int ksteps;            // k-blocks per group
  int steps_per_split;   // k-blocks per split range
  int splits;            // R
  int wtrans;            // 1: weight element (k, col) at w[(g*cig + k) * cog + col]
  int wvec;              // 1: weight rows may be read 16 bytes at a time
  int mode;              // OutMode
  int act;
  float alpha, beta;
  long long plane_stride;  // elements per raw plane
};

struct HaloArgs {
  const void* x;
  const void* wt;        // weights
  const void* bias;
  const void* res;
  void* y;
  int n, c_in, h, w, c_out, kh, kw, groups;
  int sh, sw, dh, dw, pt, pl;
  int ho, wo;
  int cig, cog;
  int oct;               // channel octets per chunk (chunk = 8*oct channels)
  int tr;                // output rows per workgroup
  int tcb;               // 16-column blocks per output row (covers the full width)
  int cb;                // 16-channel blocks per workgroup (1 or 2)
  int tih, tiw;          // staged input tile (rows, cols)
  int n_ct, n_rt;        // channel tiles per group, row tiles per image
  int wvec;              // weight rows may be read 16 bytes at a time
  int xvec;              // input planes may be read 8 bytes at a time
  int ovec;              // output / residual planes may be written / read 8 bytes at a time
  int o2;                // row-shift kernel: y and residual 4-byte aligned, wo even
  int oflat;             // row-shift kernel: y and residual 16-byte aligned at every
                         // 32-channel tile, wo even, ho * wo >= 8
  Magic mg_w, mg_g4;     // row-shift kernel: divisors w and (h w + 3) / 4
  Magic mg_nct, mg_n;    // row-shift kernel: divisors n_ct and n
  int act;
  float alpha, beta;
  // row-shift split k: `splits` ranges of `sps` 64-channel stages, range r
  // writing float32 plane r at planes + r * plane_stride
  int splits, sps;
  float* planes;
  long long plane_stride;
  Magic mg_ng;           // divisor n * groups
};

// Grouped convolution, 8 input channels per group: one workgroup per (image,
// group) with the padded input planes staged whole.
struct GroupedArgs {
  const void* x;
  const void* wt;
  const void* bias;
  const void* res;
  void* y;
  int n, c_in, h, w, c_out, groups, cog;
  int kh, kw, sh, sw, dh, dw, pt, pl;
  int ho, wo;
  int hp, wp;            // padded plane: h + pt + pb rows, w + pl + pr columns
  int xs_bytes;          // LDS bytes of the staged plane (16 per position)
  int vec;               // x 8-byte aligned and h * w % 4 == 0
  Magic mg_w, mg_wo, mg_kw;  // divisors w, wo and kw
  Magic mg_taps;             // divisor kh * kw
  int act;
  float alpha, beta;
};

// Pointwise (1x1, stride 1, no padding, one group) GEMM on x as it lies.
struct PwArgs {
  const void* x;         // [n][c_in][hw]
  const void* wt;        // [c_out][c_in], or [c_in][c_out] with ct
  const void* bias;      // nullptr when absent
  const void* res;       // nullptr when absent (always with ct)
  void* y;
  int n, c_in, hw, c_out;  // c_out: GEMM rows (4 output channels each with ct)
  int n_pt, n_ct;        // pixel tiles per image, row tiles
  int ntiles, nchunks;   // tiles in this chunk of images, 64-channel chunks of c_in
  int vec;               // x 8-byte, w 16-byte (ct: 8-byte), y 16-byte, residual
                         // 8-byte aligned and hw % 8 == 0 (ct: w_in % 4 == 0)
  int tc;                // GEMM rows per tile: 64 or 128
  int tp;                // pixels per tile (<= 128)
  int ct;                // ConvTranspose, kernel = stride = 2, no padding: GEMM rows are
                         // (co, kh, kw), weights [c_in][c_out], outputs scattered into y
  int w_in;              // ct: input row width (the tile holds whole input rows)
  int ct_rows;           // ct: input rows per tile, tp / w_in
  Magic mg_vpr, mg_rows; // ct: divisions by w_in / 4 and by ct_rows
  Magic mg_hw;           // f32 kernel: division by h * w (pixel indexes < 2^31)
  Magic mg_nch, mg_nct, mg_npt;  // f16 kernel: divisions by nchunks, n_ct and n_pt
  int act;
  float alpha, beta;
};

// Row-band implicit GEMM for stride-2 layers with few input channels.
struct RowbandArgs {
  const void* x;
  const void* wt;
  const void* bias;
  const void* res;
  void* y;
  int n, c_in, h, w, c_out, kh, kw;
  int sh, pt, pl, ho, wo;
  int n_ct, n_band, band_rows;  // 64-channel tiles, bands of output rows per image
  int rpitch;                   // halves per LDS ring row (even)
  int ring_bytes;               // c_in * 16 rows * rpitch * 2
  int vec;                      // x, y 16-byte aligned, w % 8 == 0 and wo % 8 == 0
  int wvec;                     // weights 16-byte aligned, tile runs whole vectors
  int two_rows;                 // two output rows per step (eight waves, whole vectors)
  Magic mg_nv;                  // division by the 8-half vectors per input row
  Magic mg_cin;                 // division by c_in
  Magic mg_vpr;                 // division by the 8-output vectors per output row
  Magic mg_vpr2;                // ... and by those of two output rows
  int act;
  float alpha, beta;
};

struct DepthwiseArgs {
  const void* x;
  const void* wt;      // weights
  const void* bias;
  const void* res;
  void* y;
  int n, c_in, h, w, c_out, kh, kw;
  int mult;              // c_out / c_in
  int sh, sw, dh, dw, pt, pl;
  int ho, wo;
  int toh, tow;          // output tile
  int tih, tiw;          // staged input tile (with halo)
  int tiles_w, tiles;    // tiles per plane along w, total per plane
  // whole-plane path
  int planes;            // input planes per group (P)
  int ngroups;           // groups of P planes in this chunk
  int bh;                // outputs per thread (one column, BH rows)
  int nrb;               // row blocks per plane: ceil(ho / bh)
  int tpp;               // LDS floats per staged plane (tih * tiw)
  int oofs, wofs, bofs, sofs;  // LDS float offsets: output tile, weights, bias, sink
  int lm;                // one-wave path: LDS column of input column 0 (a multiple of 4)
  int xvec;              // x may be read 16 (f32) / 8 (f16) bytes at a time, h * w % 4 == 0
  int ovec;              // y and residual 16 / 8-byte aligned and ho * wo % 4 == 0
  Magic mg_hw, mg_w, mg_pu, mg_wo, mg_howo;  // h*w, w, nrb*wo, wo, ho*wo
  int act;
  float alpha, beta;
};

// Split-k reduction and epilogue: y = act(sum_r planes[r] + bias + res).
struct ReduceArgs {
  const float* planes;
  long long plane_stride;
  int splits;
  const void* bias;
  const void* res;
  void* y;
  long long total;       // output elements in this chunk
  int hw;                // ho * wo
  int c_out;
  int vec;               // total and plane_stride multiples of 4 (planes 16-byte aligned)
  int act;
  float alpha, beta;
};

// Gathering col2im + epilogue for ConvTranspose.
struct Col2imArgs {
  const float* cols;     // [n][groups * cog * kh * kw][h][w]
  const void* bias;
  const void* res;
  void* y;
  int n, h, w, c_out, cog, kh, kw;
  int sh, sw, dh, dw, pt, pl;
  int ho, wo;
  long long total;
  int act;
  float alpha, beta;
};


// Winograd F(2x2, 3x3): 16-bit operands, 3x3, stride 1, dilation 1.
struct WinoArgs {
  const void* x;
  const void* wt;
  const void* bias;
  const void* res;
  void* y;
  void* u;               // scratch: transformed weights [16][c_out][cig], 16-bit
  int n, c_in, h, w, c_out, groups, cig, cog, pt, pl, ho, wo;
  int th, tw;            // 2x2 output tiles per column / row of an image
  int tr, tc;            // a workgroup's band: tr tile rows x tc tile columns (tr tc <= 32)
  int nbr, nbc;          // bands per image column / row
  int cb;                // 32-channel blocks per workgroup (1 or 2)
  int nsi;               // staging items per thread and step: 10 or 17
  Magic mg_nb, mg_nbc;   // divisions by nbr * nbc and by nbc
  Magic mg_tc, mg_rc, mg_c;  // by tc, by the staged positions (2 tr + 2)(2 tc + 2), by 2 tc + 2
  int act;
  float alpha, beta;
};

hipError_t launch_igemm(Dtype dt, const IgemmArgs& a, hipStream_t s);
hipError_t launch_winograd(Dtype dt, const WinoArgs& a, hipStream_t s);

// ConvInteger on the row-shift kernel (3x3, stride 1, rows of at most 14
// outputs, channels per group a multiple of 128).  Pointers include the
// problem's offsets; xzp / wzp may be null (zero).
struct ConvIntRsArgs {
  const unsigned char* x;
  const unsigned char* wt;
  const unsigned char* xzp;
  const unsigned char* wzp;
  int wz_per_channel;
  int* y;
  int n, c_in, h, w, c_out, groups, cig, cog, pt, pl, ho, wo;
  int n_ct;              // 32-channel tiles per group
  int xvec, wvec, yvec;  // x planes of whole 4-byte groups; weights 16-byte aligned; y tiles of whole 16-byte vectors
  Magic mg_nct, mg_n, mg_g4, mg_w, mg_howo, mg_wo;
};
hipError_t launch_convint_rowshift(const ConvIntRsArgs& a, bool xu, bool wu, hipStream_t s);
hipError_t launch_halo(Dtype dt, const HaloArgs& a, hipStream_t s);
hipError_t launch_pointwise(Dtype dt, const PwArgs& a, int cus, hipStream_t s);
hipError_t launch_pointwise_f32(const PwArgs& a, hipStream_t s);
hipError_t launch_pointwise_f32_strip(const PwArgs& a, hipStream_t s);
hipError_t launch_rowband(Dtype dt, const RowbandArgs& a, hipStream_t s);
hipError_t launch_grouped(Dtype dt, const GroupedArgs& a, hipStream_t s);
hipError_t launch_rowshift(Dtype dt, const HaloArgs& a, hipStream_t s);
hipError_t launch_depthwise(Dtype dt, const DepthwiseArgs& a, hipStream_t s);
hipError_t launch_depthwise_plane(Dtype dt, const DepthwiseArgs& a, int grid, size_t lds,
                                  hipStream_t s);
hipError_t launch_depthwise_wave(Dtype dt, const DepthwiseArgs& a, long long planes, int cus,
                                 size_t lds, hipStream_t s);
hipError_t launch_reduce(Dtype dt, const ReduceArgs& a, hipStream_t s);
hipError_t launch_col2im(Dtype dt, const Col2imArgs& a, hipStream_t s);

}  // namespace convfwd
