// Host half of the pooling ABI (include/pool.h) that never touches the device:
// validation, output extents, auto_pad, the shape-only plan, describe and check.
//
// "Convolution, pooling and resize" (OneGpu docs), "Layout and operands": sizes
// are checked with checked arithmetic before anything is recorded; "Pooling and
// resize": ceil_mode drops a last window that starts inside the end padding.
#include <stdio.h>
#include <string.h>

#include <algorithm>

#include "conv.h"
#include "plan.h"
#include "pool_plan.h"

namespace convfwd {

namespace {

constexpr int64_t kLim = 2147483647LL;

bool mulok(int64_t a, int64_t b, int64_t* r) { return !__builtin_mul_overflow(a, b, r); }
bool addok(int64_t a, int64_t b, int64_t* r) { return !__builtin_add_overflow(a, b, r); }

// Output size along one axis, or -1 (no window fits, or overflow).  Floor mode:
// floor(span / s) + 1 with span = in + pb + pe - d(k-1) - 1; ceil mode rounds the
// division up and drops a last window whose first tap is at or beyond the end
// of the input.
int64_t pool_axis(int64_t in, int64_t k, int64_t s, int64_t d, int64_t pb, int64_t pe,
                  bool ceil_mode) {
  int64_t dk, span;
  if (!mulok(d, k - 1, &dk) || !addok(in, pb, &span) || !addok(span, pe, &span)) return -1;
  span = span - dk - 1;
  if (span < 0) return -1;
  int64_t o = ceil_mode ? (span + s - 1) / s + 1 : span / s + 1;
  int64_t last;
  if (ceil_mode && mulok(o - 1, s, &last) && last - pb >= in) o -= 1;
  return o >= 1 ? o : -1;
}

}  // namespace

int pool_validate(const pool_problem* p, int dtype, PoolGeo* out) {
  if (!p) return CONV_ERR_ARG;
  if (dtype != CONV_F32 && dtype != CONV_F16 && dtype != CONV_BF16) return CONV_ERR_ARG;
  if (p->kind < POOL_MAX || p->kind > POOL_GLOBAL_AVERAGE) return CONV_ERR_ARG;
  if ((p->ceil_mode != 0 && p->ceil_mode != 1) ||
      (p->count_include_pad != 0 && p->count_include_pad != 1) || p->reserved != 0)
    return CONV_ERR_ARG;
  if (p->x_off < 0 || p->y_off < 0) return CONV_ERR_ARG;
  PoolGeo g{};
  g.n = p->n; g.c = p->c; g.h = p->h; g.w = p->w;
  g.kind = p->kind; g.ceil_mode = p->ceil_mode; g.cip = p->count_include_pad;
  g.es = (int)dtype_size(dtype);
  if (g.n < 1 || g.c < 1 || g.h < 1 || g.w < 1) return CONV_ERR_SHAPE;
  if (g.n > kLim || g.c > kLim || g.h > kLim || g.w > kLim) return CONV_ERR_SHAPE;
  const bool global = g.kind == POOL_GLOBAL_MAX || g.kind == POOL_GLOBAL_AVERAGE;
  if (global) {
    g.kh = g.kw = g.sh = g.sw = g.dh = g.dw = 1;
    g.ho = g.wo = 1;
  } else {
    g.kh = p->kh; g.kw = p->kw; g.sh = p->stride_h; g.sw = p->stride_w;
    g.dh = p->dil_h; g.dw = p->dil_w;
    g.pt = p->pad_top; g.pl = p->pad_left; g.pb = p->pad_bottom; g.pr = p->pad_right;
    if (g.kh < 1 || g.kw < 1 || g.sh < 1 || g.sw < 1 || g.dh < 1 || g.dw < 1) return CONV_ERR_SHAPE;
    if (g.pt < 0 || g.pl < 0 || g.pb < 0 || g.pr < 0) return CONV_ERR_SHAPE;
    if (g.kh > kLim || g.kw > kLim || g.sh > kLim || g.sw > kLim || g.dh > kLim || g.dw > kLim ||
        g.pt > kLim || g.pl > kLim || g.pb > kLim || g.pr > kLim)
      return CONV_ERR_SHAPE;
    g.ho = pool_axis(g.h, g.kh, g.sh, g.dh, g.pt, g.pb, g.ceil_mode == 1);
    g.wo = pool_axis(g.w, g.kw, g.sw, g.dw, g.pl, g.pr, g.ceil_mode == 1);
    if (g.ho < 1 || g.wo < 1) return CONV_ERR_SHAPE;
    // every tap index fits int32 in the kernels
    int64_t t;
    if (!mulok(g.ho, g.sh, &t) || !addok(t, g.kh * g.dh, &t) || t > kLim ||
        !mulok(g.wo, g.sw, &t) || !addok(t, g.kw * g.dw, &t) || t > kLim)
      return CONV_ERR_SHAPE;
  }
  int64_t t;
  if (!mulok(g.n, g.c, &t) || !mulok(t, g.h, &t) || !mulok(t, g.w, &t) || t > kLim)
    return CONV_ERR_SHAPE;
  g.x_elems = t;
  if (!mulok(g.n, g.c, &t) || !mulok(t, g.ho, &t) || !mulok(t, g.wo, &t) || t > kLim)
    return CONV_ERR_SHAPE;
  g.y_elems = t;
  const int64_t es = dtype_size(dtype);
  int64_t end, bytes;
  if (!addok(p->x_off, g.x_elems, &end) || !mulok(end, es, &bytes)) return CONV_ERR_SHAPE;
  if (!addok(p->y_off, g.y_elems, &end) || !mulok(end, es, &bytes)) return CONV_ERR_SHAPE;
  *out = g;
  return CONV_OK;
}

bool pool_rowvec_applies(const PoolGeo& g) {
  if (g.kind != POOL_MAX && g.kind != POOL_AVERAGE) return false;
  if (g.kh < 2 || g.kh > 3 || g.kw < 2 || g.kw > 3 || g.sw < 1 || g.sw > 2) return false;
  if (g.dh != 1 || g.dw != 1) return false;
  const int64_t v = 16 / g.es, word = 4 / g.es;  // elements per vector and per 32-bit word
  if (g.w % v != 0) return false;
  // left reach pl, right reach kw - sw - pl beyond the thread's vector
  if (g.pl > word || g.kw - g.sw - g.pl > word) return false;
  const int64_t opt = v / g.sw, tpr = ceil_div(g.wo, opt);
  return tpr * v >= g.w;  // every real column belongs to some thread of the row
}

int pool_make_plan(const PoolGeo& g, PoolPlan* pl) {
  memset(pl, 0, sizeof *pl);
  if (g.kind == POOL_GLOBAL_MAX || g.kind == POOL_GLOBAL_AVERAGE) {
    pl->variant = POOLV_GLOBAL;
    const int64_t hw = g.h * g.w, planes = g.n * g.c;
    if (hw <= kPoolChunk) {
      // 256 / P lanes per plane (a power of two, at most 64): about 32 pairs
      // per lane on the first level, then fewer planes per workgroup until
      // the grid has about 1024 workgroups; the LDS holds P planes
      int64_t lanes = 1;
      while (lanes < 64 && lanes * 32 < hw) lanes *= 2;
      while (lanes < 64 && ceil_div(planes, 256 / lanes) < 1024) lanes *= 2;
      int64_t P = 256 / lanes;
      while (P > 1 && P * hw > kPoolChunk) P /= 2;
      pl->planes_wg = (int)P;
      pl->chunks = 1;
    } else {
      pl->planes_wg = 1;
      const int64_t ch = ceil_div(hw, kPoolChunk);
      if (ch > kPoolChunk) return CONV_ERR_SHAPE;  // chunk sums must fit one tree
      pl->chunks = (int)ch;
    }
    return CONV_OK;
  }
  if (pool_rowvec_applies(g)) {
    const int64_t opt = 16 / g.es / g.sw;
    int64_t t;
    if (mulok(g.n * g.c, g.ho, &t) && mulok(t, ceil_div(g.wo, opt), &t) && t <= kLim) {
      pl->variant = POOLV_ROWVEC;
      pl->tpr = (int)ceil_div(g.wo, opt);
      pl->threads = t;
      return CONV_OK;
    }
  }
  // band: output rows per workgroup such that the staged input rows fit the
  // LDS budget as float32 and each workgroup has a few hundred outputs
  const int64_t reach = (g.kh - 1) * g.dh + 1;
  int64_t best = 0;
  for (int64_t tb = std::min<int64_t>(g.ho, 64); tb >= 1; --tb) {
    const int64_t rows = (tb - 1) * g.sh + reach;
    if (rows * g.w * 4 <= kPoolBandLds) {
      best = tb;
      break;
    }
  }
  if (best == 0) {
    pl->variant = POOLV_DIRECT;
    return CONV_OK;
  }
  // keep at least ~256 outputs per band but no more bands than needed
  int64_t tb = std::min<int64_t>(best, std::max<int64_t>(1, ceil_div(1024, g.wo)));
  pl->variant = POOLV_BAND;
  pl->band_rows = (int)tb;
  pl->in_rows = (int)((tb - 1) * g.sh + reach);
  pl->n_band = (int)ceil_div(g.ho, tb);
  int64_t grid;
  if (!mulok(g.n * g.c, pl->n_band, &grid) || grid > kLim) return CONV_ERR_SHAPE;
  return CONV_OK;
}

}  // namespace convfwd

using namespace convfwd;

extern "C" {

int pool_output_extent(const pool_problem* p, int64_t* ho, int64_t* wo) {
  if (!p || !ho || !wo) return CONV_ERR_ARG;
  PoolGeo g;
  const int st = pool_validate(p, CONV_F32, &g);
  if (st) return st;
  *ho = g.ho;
  *wo = g.wo;
  return CONV_OK;
}

int pool_resolve_auto_pad(pool_problem* p, int auto_pad) {
  if (!p) return CONV_ERR_ARG;
  if (auto_pad < CONV_AUTO_PAD_NOTSET || auto_pad > CONV_AUTO_PAD_VALID) return CONV_ERR_ARG;
  const int64_t in[2] = {p->h, p->w}, k[2] = {p->kh, p->kw}, s[2] = {p->stride_h, p->stride_w},
                d[2] = {p->dil_h, p->dil_w};
  for (int i = 0; i < 2; ++i)
    if (in[i] < 1 || k[i] < 1 || s[i] < 1 || d[i] < 1 || in[i] > kLim || k[i] > kLim ||
        s[i] > kLim || d[i] > kLim)
      return CONV_ERR_SHAPE;
  int64_t b[2] = {p->pad_top, p->pad_left}, e[2] = {p->pad_bottom, p->pad_right};
  for (int i = 0; i < 2; ++i) {
    if (auto_pad == CONV_AUTO_PAD_NOTSET) continue;
    if (auto_pad == CONV_AUTO_PAD_VALID) { b[i] = e[i] = 0; continue; }
    const int64_t out = (in[i] + s[i] - 1) / s[i];
    int64_t total = (out - 1) * s[i] + d[i] * (k[i] - 1) + 1 - in[i];
    if (total < 0) total = 0;
    const int64_t lo = total / 2, hi = total - lo;
    b[i] = auto_pad == CONV_AUTO_PAD_SAME_UPPER ? lo : hi;
    e[i] = auto_pad == CONV_AUTO_PAD_SAME_UPPER ? hi : lo;
  }
  p->pad_top = b[0]; p->pad_left = b[1]; p->pad_bottom = e[0]; p->pad_right = e[1];
  return CONV_OK;
}

int pool_describe_variant(const pool_problem* p, int dtype, char* buf, uint64_t len) {
  if (!buf) return CONV_ERR_ARG;
  PoolGeo g;
  int st = pool_validate(p, dtype, &g);
  if (st) return st;
  PoolPlan pl;
  st = pool_make_plan(g, &pl);
  if (st) return st;
  static const char* kinds[] = {"max", "average", "global_max", "global_average"};
  const char* dn = dtype == CONV_F16 ? "f16" : dtype == CONV_BF16 ? "bf16" : "f32";
  char tmp[96];
  if (pl.variant == POOLV_BAND)
    snprintf(tmp, sizeof tmp, "pool.%s.%s.band%d", kinds[g.kind], dn, pl.band_rows);
  else if (pl.variant == POOLV_ROWVEC)
    snprintf(tmp, sizeof tmp, "pool.%s.%s.rowvec%d", kinds[g.kind], dn, (int)(16 / g.es / g.sw));
  else if (pl.variant == POOLV_DIRECT)
    snprintf(tmp, sizeof tmp, "pool.%s.%s.direct", kinds[g.kind], dn);
  else if (pl.chunks > 1)
    snprintf(tmp, sizeof tmp, "pool.%s.%s.tree.chunks%d", kinds[g.kind], dn, pl.chunks);
  else
    snprintf(tmp, sizeof tmp, "pool.%s.%s.tree.planes%d", kinds[g.kind], dn, pl.planes_wg);
  const size_t need = strlen(tmp) + 1;
  if (len < need) return CONV_ERR_ARG;
  memcpy(buf, tmp, need);
  return CONV_OK;
}

int pool_check(const pool_problem* p, int dtype, const void* x, const void* y) {
  PoolGeo g;
  int st = pool_validate(p, dtype, &g);
  if (st) return st;
  PoolPlan pl;
  st = pool_make_plan(g, &pl);
  if (st) return st;
  if (!x || !y) return CONV_ERR_ARG;
  const uint64_t es = (uint64_t)dtype_size(dtype);
  const uintptr_t x0 = (uintptr_t)x + (uintptr_t)p->x_off * es, x1 = x0 + (uintptr_t)g.x_elems * es;
  const uintptr_t y0 = (uintptr_t)y + (uintptr_t)p->y_off * es, y1 = y0 + (uintptr_t)g.y_elems * es;
  if (x0 < y1 && y0 < x1) return CONV_ERR_OVERLAP;
  return CONV_OK;
}

}  // extern "C"
