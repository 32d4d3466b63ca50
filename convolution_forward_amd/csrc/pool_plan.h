// Shape-only planner of the pooling forward (include/pool.h): validation with
// checked int64 arithmetic, output extents, the kernel choice and its tiling.
// Plain C++ with no HIP include, like the convolution's planner.
#pragma once

#include <stdint.h>

#include "pool.h"

namespace convfwd {

struct PoolGeo {
  int64_t n, c, h, w, kh, kw, sh, sw, dh, dw, pt, pl, pb, pr;
  int64_t ho, wo;
  int64_t x_elems, y_elems;
  int kind, ceil_mode, cip;
  int es;  // element size in bytes
};

enum PoolVariant { POOLV_BAND = 0, POOLV_DIRECT = 1, POOLV_GLOBAL = 2, POOLV_ROWVEC = 3 };

struct PoolPlan {
  int variant;
  int band_rows;   // band: output rows per workgroup
  int in_rows;     // band: staged input rows (the band's window reach)
  int n_band;      // band: bands per plane
  int planes_wg;   // global: planes per workgroup (planes of at most 4096 elements)
  int chunks;      // global: 4096-element chunks per plane (planes above 4096)
  int tpr;         // row vector: threads per output row (each 16 / es input columns)
  int64_t threads; // row vector: planes x output rows x tpr
};

// Row-vector kernel limits: windows of 2 or 3 taps per axis, horizontal
// stride 1 or 2, no dilation, rows of whole 16-byte vectors, and a window
// reach beyond a thread's own vector of at most one 32-bit word on each side.
bool pool_rowvec_applies(const PoolGeo& g);

// LDS budget of the band kernel (staged input rows as float32).
constexpr int64_t kPoolBandLds = 64 * 1024;
// Elements per tree chunk of the global kernel.
constexpr int64_t kPoolChunk = 4096;

int pool_validate(const pool_problem* p, int dtype, PoolGeo* g);
int pool_make_plan(const PoolGeo& g, PoolPlan* pl);

}  // namespace convfwd
