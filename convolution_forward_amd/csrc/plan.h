// Shape-only planner of the convolution forward: problem validation with
// checked int64 arithmetic, the variant / tile / split / chunk plan and the
// overlap rules.  Plain C++ with no HIP include: the plan cannot depend on the
// device a call later runs on, only on the problem's shape, element type and
// the variant and split overrides.
//
// "Convolution, pooling and resize" (OneGpu docs), "Layout and operands":
// sizes are checked before anything is recorded; Scratch(problem, half) is a
// function of the shape; "Variants": DescribeVariant names what runs, and the
// split-k cut depends only on the shape.
#pragma once

#include <stdint.h>

#include "conv.h"
#include "tiles.h"

namespace convfwd {

// Compute units the plan is made for (gfx950: 256).  A fixed figure, not the
// running device's count, so that describe / scratch / check are shape-only and
// every device runs the same variant, tile and sum order for a shape.
constexpr int kPlanCUs = 256;

struct Geo {
  int64_t n, ci, h, w, co, kh, kw, g, sh, sw, dh, dw, pt, pl, pb, pr, oph, opw;
  int64_t ho, wo, cig, cog;
  int64_t x_elems, w_elems, y_elems;
  bool transpose;
};

struct HaloShape {
  int oct, tr, tcb, cb, tih, tiw, n_ct, n_rt;
  bool rowshift;  // the 3x3 stride-1 narrow-image kernel
};

struct Plan {
  int variant;
  HaloShape halo;
  int splits;          // implicit GEMM split-k ranges
  int ksteps;
  int steps_per_split;
  uint64_t scratch_per_image;
  uint64_t scratch_whole;
  // depthwise tiling
  int toh, tow, tih, tiw, tiles_w, tiles;
  int dw_planes;  // > 0: whole-plane path with this many planes per group
  int dw_bh;      // whole-plane path: outputs per thread along a column
  int dw_wave;    // whole-plane path: one wave per plane
  int dw_lm;      // one-wave path: LDS column of input column 0
  int pw_tc;      // pointwise: output channels per tile
  int pw_strip;   // float32 pointwise: 16-channel x 256-pixel strips, x straight to registers
  int rb_band_rows;  // row band: output rows per workgroup
  int ct_fused;      // transpose: kernel = stride = 2 taps gathered by the GEMM epilogue
  int scratch_fixed; // scratch does not grow with the batch (Winograd weights): no chunks
  int wino_cb;       // Winograd: 32-channel blocks per workgroup
  int wino_tr, wino_tc;  // Winograd: tile rows x tile columns of a workgroup's band (at most 32 tiles)
};

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// LDS floats of the whole-plane depthwise kernel.
int64_t dw_lds_floats(int64_t P, int64_t tpp, int64_t mult, int64_t howo, int64_t k);

// Checks the problem and fills the geometry (CONV_OK or a CONV_ERR_* status).
int validate(const conv_problem* p, int dtype, Geo* g);

// The plan for a validated geometry: variant, tiles, split count, scratch.
int make_plan(const conv_problem* p, int dtype, const Geo& g, Plan* pl);

// Every host-side check of a forward call (shape, enums, pointers, overlap,
// scratch); fills the geometry, the plan and the image chunk size.
int check_call(const conv_problem* p, int dtype, bool transpose, const void* x, const void* w,
               const void* bias, const void* residual, const void* y, const void* scratch,
               uint64_t scratch_bytes, Geo* gout, Plan* plout, int64_t* chunk_out);

// Bytes per element of a conv_dtype.
inline int64_t dtype_size(int dtype) { return dtype == CONV_F32 ? 4 : 2; }

// A 16-bit floating operand type (float16 or bfloat16): the matrix kernels
// that move 16-bit elements serve both, with the MFMA of that type.
inline bool half16(int dtype) { return dtype == CONV_F16 || dtype == CONV_BF16; }

}  // namespace convfwd
