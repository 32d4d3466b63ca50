// Host half of the C ABI (include/conv.h) that never touches the device:
// problem validation with checked int64 arithmetic, auto_pad resolution, the
// shape-only variant planner, scratch sizing, the overlap rules and the status
// strings.  The launch sequence lives in conv_host.cpp.
//
// "Convolution, pooling and resize" (OneGpu docs), "Layout and operands": sizes
// are checked before anything is recorded; scratch is caller-supplied, reported
// for the whole batch and for one image, and a smaller buffer runs the batch in
// chunks of whole images without changing a bit; scratch may share an arena with
// the operands as long as its range overlaps none of them.  "Variants": the
// variant depends on the layer class; the split-k cut depends only on the shape.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>

#include "conv.h"
#include "plan.h"

namespace convfwd {

constexpr int64_t kMaxElems = 2147483647LL;  // every operand indexable with int32
constexpr int kMaxSplits = 16;

bool mul_ok(int64_t a, int64_t b, int64_t* r) { return !__builtin_mul_overflow(a, b, r); }
bool add_ok(int64_t a, int64_t b, int64_t* r) { return !__builtin_add_overflow(a, b, r); }

// floor((in + pb + pe - d(k-1) - 1)/s) + 1, or -1 when no window fits / overflow.
int64_t conv_extent(int64_t in, int64_t k, int64_t s, int64_t d, int64_t pb, int64_t pe) {
  int64_t span, dk;
  if (!mul_ok(d, k - 1, &dk)) return -1;
  if (!add_ok(in, pb, &span) || !add_ok(span, pe, &span)) return -1;
  span = span - dk - 1;
  if (span < 0) return -1;
  return span / s + 1;
}

// s(in-1) + op + d(k-1) + 1 - pb - pe, or -1.
int64_t convt_extent(int64_t in, int64_t k, int64_t s, int64_t d, int64_t pb, int64_t pe,
                     int64_t op) {
  int64_t a, dk, o;
  if (!mul_ok(s, in - 1, &a) || !mul_ok(d, k - 1, &dk)) return -1;
  if (!add_ok(a, op, &o) || !add_ok(o, dk + 1, &o)) return -1;
  o = o - pb - pe;
  return o >= 1 ? o : -1;
}


int validate(const conv_problem* p, int dtype, Geo* g) {
  if (!p) return CONV_ERR_ARG;
  if (dtype != CONV_F32 && dtype != CONV_F16 && dtype != CONV_BF16) return CONV_ERR_ARG;
  if (p->transpose != 0 && p->transpose != 1) return CONV_ERR_ARG;
  if (p->activation < CONV_ACT_IDENTITY || p->activation > CONV_ACT_LEAKY_RELU)
    return CONV_ERR_ARG;
  if ((p->has_bias != 0 && p->has_bias != 1) || (p->has_residual != 0 && p->has_residual != 1))
    return CONV_ERR_ARG;
  if (p->variant_override < CONV_VARIANT_AUTO || p->variant_override > CONV_VARIANT_WINOGRAD)
    return CONV_ERR_ARG;
  if (p->split_override < 0 || p->split_override > kMaxSplits) return CONV_ERR_ARG;
  if (p->x_off < 0 || p->w_off < 0 || p->b_off < 0 || p->r_off < 0 || p->y_off < 0)
    return CONV_ERR_ARG;

  Geo q{};
  q.n = p->n; q.ci = p->c_in; q.h = p->h; q.w = p->w; q.co = p->c_out;
  q.kh = p->kh; q.kw = p->kw; q.g = p->groups;
  q.sh = p->stride_h; q.sw = p->stride_w; q.dh = p->dil_h; q.dw = p->dil_w;
  q.pt = p->pad_top; q.pl = p->pad_left; q.pb = p->pad_bottom; q.pr = p->pad_right;
  q.oph = p->out_pad_h; q.opw = p->out_pad_w;
  q.transpose = p->transpose == 1;
  if (q.n < 1 || q.ci < 1 || q.h < 1 || q.w < 1 || q.co < 1 || q.kh < 1 || q.kw < 1 || q.g < 1)
    return CONV_ERR_SHAPE;
  if (q.ci % q.g || q.co % q.g) return CONV_ERR_SHAPE;
  if (q.sh < 1 || q.sw < 1 || q.dh < 1 || q.dw < 1) return CONV_ERR_SHAPE;
  if (q.pt < 0 || q.pl < 0 || q.pb < 0 || q.pr < 0) return CONV_ERR_SHAPE;
  const int64_t lim = kMaxElems;
  if (q.n > lim || q.ci > lim || q.h > lim || q.w > lim || q.co > lim || q.kh > lim ||
      q.kw > lim || q.sh > lim || q.sw > lim || q.dh > lim || q.dw > lim || q.pt > lim ||
      q.pl > lim || q.pb > lim || q.pr > lim)
    return CONV_ERR_SHAPE;
  if (q.transpose) {
    if (q.oph < 0 || q.oph >= q.sh || q.opw < 0 || q.opw >= q.sw) return CONV_ERR_SHAPE;
    q.ho = convt_extent(q.h, q.kh, q.sh, q.dh, q.pt, q.pb, q.oph);
    q.wo = convt_extent(q.w, q.kw, q.sw, q.dw, q.pl, q.pr, q.opw);
  } else {
    if (q.oph != 0 || q.opw != 0) return CONV_ERR_SHAPE;
    q.ho = conv_extent(q.h, q.kh, q.sh, q.dh, q.pt, q.pb);
    q.wo = conv_extent(q.w, q.kw, q.sw, q.dw, q.pl, q.pr);
  }
  if (q.ho < 1 || q.wo < 1) return CONV_ERR_SHAPE;
  q.cig = q.ci / q.g;
  q.cog = q.co / q.g;
  int64_t t;
  if (!mul_ok(q.n, q.ci, &t) || !mul_ok(t, q.h, &t) || !mul_ok(t, q.w, &t) || t > lim)
    return CONV_ERR_SHAPE;
  q.x_elems = t;
  if (!mul_ok(q.transpose ? q.ci : q.co, q.transpose ? q.cog : q.cig, &t) ||
      !mul_ok(t, q.kh, &t) || !mul_ok(t, q.kw, &t) || t > lim)
    return CONV_ERR_SHAPE;
  q.w_elems = t;
  if (!mul_ok(q.n, q.co, &t) || !mul_ok(t, q.ho, &t) || !mul_ok(t, q.wo, &t) || t > lim)
    return CONV_ERR_SHAPE;
  q.y_elems = t;
  if (q.transpose) {  // float32 columns of one image must be indexable too
    if (!mul_ok(q.co, q.kh, &t) || !mul_ok(t, q.kw, &t) || !mul_ok(t, q.h, &t) ||
        !mul_ok(t, q.w, &t) || t > lim)
      return CONV_ERR_SHAPE;
  }
  // pointer arithmetic on offsets must not overflow: every operand's byte
  // range (offset + extent, times the element size) fits int64
  const int64_t es = dtype_size(dtype);
  const int64_t offs[5] = {p->x_off, p->w_off, p->y_off, p->b_off, p->r_off};
  const int64_t lens[5] = {q.x_elems, q.w_elems, q.y_elems, q.co, q.y_elems};
  for (int i = 0; i < 5; ++i) {
    int64_t end, bytes;
    if (!add_ok(offs[i], lens[i], &end) || !mul_ok(end, es, &bytes)) return CONV_ERR_SHAPE;
  }
  *g = q;
  return CONV_OK;
}




// LDS floats of the whole-plane depthwise kernel: P staged planes, output tile
// (16-byte aligned), weights, double-buffered bias, one sink float.
int64_t dw_lds_floats(int64_t P, int64_t tpp, int64_t mult, int64_t howo, int64_t k) {
  const int64_t out0 = (P * tpp + 3) / 4 * 4;
  return out0 + P * mult * howo + P * mult * k * k + 2 * P * mult + 1;
}


bool depthwise_applicable(const Geo& g) { return !g.transpose && g.cig == 1; }

// Row-band implicit GEMM: float16, one group, stride 2 both ways, no dilation,
// kernel rows of at most 8 taps, at most 24 (ci, kh) groups, output rows of at
// most 128; the new input rows of one output row fit one 16-byte item per
// thread, the first KH rows four, and the ring holds KH rows plus three rows'
// worth of prefetched ones; an image's input planes and a 64-channel tile of
// its output planes are below 2 GiB (32-bit byte offsets).
bool rowband_applicable(const Geo& g, int dtype) {
  return !g.transpose && half16(dtype) && g.g == 1 && g.sh == 2 && g.sw == 2 && g.dh == 1 &&
         g.dw == 1 && g.kw <= 8 && g.ci * g.kh <= 24 && g.kh + 4 * g.sh <= 16 && g.wo <= 128 &&
         g.sh * g.ci * ceil_div(g.w, 8) <= 256 && g.kh * g.ci * ceil_div(g.w, 8) <= 1024 &&
         g.ci * g.h * g.w * 2 < 2147483648LL && 64 * g.ho * g.wo * 2 < 2147483648LL;
}

// Grouped implicit GEMM: float16, 8 input channels per group, at most 32 output
// channels per group, at most 10 taps, planes of at most 4096 pixels whose
// padded copy (16 bytes per position) fits 48 KiB of LDS.
bool grouped_applicable(const Geo& g, int dtype) {
  return !g.transpose && half16(dtype) && g.g > 1 && g.cig == 8 && g.cog <= 32 &&
         g.kh * g.kw <= 10 && g.h * g.w <= 4096 &&
         (g.h + g.pt + g.pb) * (g.w + g.pl + g.pr) * 16 <= 48 * 1024 && g.n * g.g <= 2147483647LL;
}

// Work items (tile, 64-channel chunk) of the pointwise kernel; its int item
// arithmetic needs them well below 2^31.
int64_t pw_items(int64_t n, int64_t pixel_tiles, int64_t channel_tiles, int64_t ci) {
  int64_t t;
  if (!mul_ok(n, pixel_tiles, &t) || !mul_ok(t, channel_tiles, &t) ||
      !mul_ok(t, ceil_div(ci, 64), &t))
    return INT64_MAX;
  return t;
}

// x, w and y (elements) of the float16 pointwise kernel below 2 GiB each: its
// loads and stores take 32-bit byte offsets.
bool pw_bytes_ok(int64_t x_elems, int64_t w_elems, int64_t y_elems) {
  const int64_t lim = (1LL << 30) - 1024;  // elements of 2 bytes, with slack for a tile past the end
  return x_elems < lim && w_elems < lim && y_elems < lim;
}

// Pointwise GEMM on x as it lies: 1x1, stride 1, no padding, one group, float16,
// whole channel octets and planes of whole 4-pixel groups.
bool pointwise_applicable(const Geo& g, int dtype) {
  if (dtype == CONV_F32)  // float32: planes and weight rows of whole float4 groups
    return !g.transpose && g.kh == 1 && g.kw == 1 && g.sh == 1 && g.sw == 1 && g.pt == 0 &&
           g.pl == 0 && g.pb == 0 && g.pr == 0 && g.g == 1 && g.ci % 4 == 0 &&
           (g.h * g.w) % 4 == 0 && ceil_div(g.n * g.h * g.w, 64) * ceil_div(g.co, 80) < (1LL << 31) &&
           g.n * g.ci * g.h * g.w < (1LL << 29) && g.co * g.ci < (1LL << 29) &&
           g.n * g.co * g.h * g.w < (1LL << 29);  // 32-bit byte offsets
  return !g.transpose && half16(dtype) && g.kh == 1 && g.kw == 1 && g.sh == 1 && g.sw == 1 &&
         g.pt == 0 && g.pl == 0 && g.pb == 0 && g.pr == 0 && g.g == 1 && g.ci % 8 == 0 &&
         (g.h * g.w) % 4 == 0 && g.h * g.w >= 4 &&
         pw_items(g.n, ceil_div(g.h * g.w, 128), ceil_div(g.co, 64), g.ci) < (1LL << 30) &&
         pw_bytes_ok(g.n * g.ci * g.h * g.w, g.co * g.ci, g.n * g.co * g.h * g.w);
}

// ConvTranspose whose kernel equals its stride of 2 with no padding: each output
// takes exactly one tap, so the GEMM's epilogue can scatter its tile straight
// into y (float16, one group, no residual, input rows of whole 4-pixel groups
// that fit a 128-pixel tile).
bool transpose_fused_applicable(const Geo& g, int dtype, bool residual) {
  return g.transpose && half16(dtype) && g.g == 1 && g.kh == 2 && g.kw == 2 && g.sh == 2 &&
         g.sw == 2 && g.dh == 1 && g.dw == 1 && g.pt == 0 && g.pl == 0 && g.pb == 0 &&
         g.pr == 0 && g.oph == 0 && g.opw == 0 && !residual && g.w % 4 == 0 && g.w <= 128 &&
         pw_items(g.n, ceil_div(g.h * g.w, (128 / g.w) * g.w), ceil_div(4 * g.co, 128), g.ci) < (1LL << 30) &&
         pw_bytes_ok(g.n * g.ci * g.h * g.w, 4 * g.co * g.ci, 4 * g.n * g.co * g.h * g.w);
}

// Winograd F(2x2, 3x3): 16-bit operands, 3x3, stride 1, dilation 1, input
// channels per group in whole steps of 16 (16-byte weight fragments), tile and
// channel-tile counts inside the grid limits, and x, y and the transformed
// weights below 2 GiB (the kernels address them with 32-bit byte offsets).
bool winograd_applicable(const Geo& g, int dtype) {
  if (g.transpose || !half16(dtype) || g.kh != 3 || g.kw != 3 || g.sh != 1 || g.sw != 1 ||
      g.dh != 1 || g.dw != 1 || g.cig % 16)
    return false;
  int64_t tiles, t;
  if (!mul_ok(g.n, ceil_div(g.ho, 2), &tiles) || !mul_ok(tiles, ceil_div(g.wo, 2), &tiles))
    return false;
  return tiles < (1LL << 31) - 64 && ceil_div(g.cog, 32) <= 65535 && g.g <= 65535 &&
         mul_ok(16 * g.co, g.cig, &t) && t < (1LL << 30) && g.x_elems < (1LL << 30) &&
         g.y_elems < (1LL << 30) &&
         g.co * g.cig / 8 < (1LL << 31) - 64;
}

// Depthwise output tile: whole plane when the staged input fits, else smaller
// tiles; the staged region stays under 48 KiB of LDS.  Kernel/stride pairs with a
// compiled register-blocked path and whole planes of at most 16 KiB take the
// whole-plane kernel: several planes per workgroup, enough 2x2 output blocks to
// give every thread a few.
bool plan_depthwise(const Geo& g, Plan* pl) {
  pl->dw_planes = 0;
  const bool compiled = g.dh == 1 && g.dw == 1 && g.sh == g.sw && g.kh == g.kw &&
                        ((g.sh == 1 && (g.kh == 3 || g.kh == 5 || g.kh == 7)) ||
                         (g.sh == 2 && (g.kh == 3 || g.kh == 5))) &&
                        (g.h * g.w) % 4 == 0;
  if (compiled) {
    const int64_t mult = g.co / g.ci;
    const int64_t hw = g.h * g.w, howo = g.ho * g.wo;
    // one wave per plane: small planes, at most 64 output columns per row block
    {
      const int64_t bh = g.sh == 1 ? 14 : 4;
      const int64_t nrb = ceil_div(g.ho, bh);
      if (hw <= 1024 && mult * howo <= 1024 && mult * g.kh * g.kw <= 64 && g.wo <= 64) {
        const int64_t lm = (g.pl + 3) / 4 * 4;
        int64_t tiw = std::max<int64_t>(lm + g.w, lm - g.pl + (g.wo - 1) * g.sw + g.kw);
        tiw = (tiw + 3) / 4 * 4;
        // two row blocks 32 banks apart when the pitch allows it
        for (int64_t t = tiw; t < tiw + 64; t += 4)
          if ((bh * g.sh * t) % 64 == 32) { tiw = t; break; }
        const int64_t tih = std::max<int64_t>(g.h + g.pt, (nrb * bh - 1) * g.sh + g.kh);
        pl->dw_wave = 1;
        pl->dw_planes = 1;
        pl->dw_bh = (int)bh;
        pl->dw_lm = (int)lm;
        pl->tih = (int)tih;
        pl->tiw = (int)tiw;
        pl->toh = (int)g.ho;
        pl->tow = (int)g.wo;
        pl->tiles = 1;
        pl->tiles_w = 1;
        return true;
      }
    }
    const int64_t bh = g.sh == 1 ? 4 : 2;
    const int64_t nrb = ceil_div(g.ho, bh);
    const int64_t tih = std::max<int64_t>(g.h + g.pt, (nrb * bh - 1) * g.sh + g.kh);
    const int64_t tiw = std::max<int64_t>(g.w + g.pl, (g.wo - 1) * g.sw + g.kw);
    // whole planes per group: every thread stages at most 4 items of 4 inputs,
    // 2 weights and 1 bias, and finishes at most 4 items of 4 outputs; the
    // group's LDS stays under 64 KiB
    int64_t P = std::min<int64_t>({4096 / hw, 4096 / (mult * howo), 256 / mult,
                                   512 / (mult * g.kh * g.kw), g.n * g.ci});
    for (; P >= 1; --P) {
      const int64_t lds = dw_lds_floats(P, tih * tiw, mult, howo, g.kh) * 4;
      if (lds <= 64 * 1024) break;
    }
    if (P >= 1) {
      pl->dw_planes = (int)P;
      pl->dw_bh = (int)bh;
      pl->tih = (int)tih;
      pl->tiw = (int)tiw;
      pl->toh = (int)g.ho;
      pl->tow = (int)g.wo;
      pl->tiles = 1;
      pl->tiles_w = 1;
      return true;
    }
  }
  int64_t toh = std::min<int64_t>(g.ho, 64), tow = std::min<int64_t>(g.wo, 64);
  for (;;) {
    int64_t tih = (toh - 1) * g.sh + (g.kh - 1) * g.dh + 1;
    int64_t tiw = (tow - 1) * g.sw + (g.kw - 1) * g.dw + 1;
    if (tih * tiw * 4 <= 48 * 1024) {
      pl->toh = (int)toh; pl->tow = (int)tow; pl->tih = (int)tih; pl->tiw = (int)tiw;
      pl->tiles_w = (int)ceil_div(g.wo, tow);
      int64_t tiles = ceil_div(g.ho, toh) * pl->tiles_w;
      if (tiles > 65535) return false;
      pl->tiles = (int)tiles;
      return true;
    }
    if (toh == 1 && tow == 1) return false;  // window alone exceeds LDS
    if (toh >= tow && toh > 1) toh = (toh + 1) / 2; else tow = (tow + 1) / 2;
  }
}

// Halo implicit GEMM (float16): kernel 3x3 or 1x1, channels per group a multiple
// of 8, output rows at most 64 wide.  Picks the chunk width, the channel tile and
// the rows per workgroup so that the staged tile fits one LDS buffer, every wave
// owns at most HALO_MAXT MFMA tiles and every thread stages at most HALO_MAXI
// items.  Shape-only.
bool plan_halo(const Geo& g, int dtype, HaloShape* hs) {
  if (!half16(dtype) || g.transpose) return false;
  // 3x3, stride 1, dilation 1, whole image of at most 14 x 14 outputs per
  // workgroup, chunk pairs of 64 channels: the row-shift kernel.
  if (g.kh == 3 && g.kw == 3 && g.sh == 1 && g.sw == 1 && g.dh == 1 && g.dw == 1 &&
      g.cig % 64 == 0 && g.ho <= 14 && g.wo <= 14) {
    HaloShape s{};
    s.rowshift = true;
    s.oct = 4;
    s.cb = 2;
    s.tcb = 1;
    s.tr = g.ho <= 8 ? 8 : 14;
    s.tih = s.tr + 2;
    s.tiw = 16;
    s.n_ct = (int)ceil_div(g.cog, 32);
    s.n_rt = 1;
    if ((int64_t)s.n_ct * g.n * g.g > 2147483647LL) return false;
    *hs = s;
    return true;
  }
  if (!((g.kh == 3 && g.kw == 3) || (g.kh == 1 && g.kw == 1))) return false;
  if (g.cig % 8 || g.wo > 64) return false;
  HaloShape s{};
  s.oct = g.cig % 32 == 0 ? 4 : (g.cig % 16 == 0 ? 2 : 1);
  s.cb = g.cog > 16 ? 2 : 1;
  s.tcb = (int)ceil_div(g.wo, 16);
  s.n_ct = (int)ceil_div(g.cog, 16 * s.cb);
  // Largest row tile that fits, then halve it while the grid is under two
  // workgroups per CU (256 CUs): a second resident workgroup hides the first's
  // staging latency.
  // MFMA tiles per wave: the 3x3 kernels with 16- or 32-channel chunks would
  // spill registers beyond 4 (resp. 7) tiles at two waves per SIMD.
  const int64_t max_tiles = (g.kh * g.kw == 9 && s.oct == 4) ? 4
                          : (g.kh * g.kw == 9 && s.oct == 2) ? 7 : HALO_MAXT;
  int64_t best = 0;
  for (int64_t tr = g.ho; tr >= 1; --tr) {
    const int64_t rb = tr * s.tcb;
    const int64_t per_wave = s.cb == 2 ? ceil_div(rb, 2) : ceil_div(rb, 4);
    if (per_wave > max_tiles) continue;
    const int64_t tih = (tr - 1) * g.sh + (g.kh - 1) * g.dh + 1;
    const int64_t tiw = (s.tcb * 16 - 1) * g.sw + (g.kw - 1) * g.dw + 1;
    const int64_t items = tih * tiw * s.oct;
    if (items > 256 * HALO_MAXI) continue;
    const int64_t bytes = items * 16 + g.kh * g.kw * 16 * s.cb * s.oct * 16;
    if (bytes > HALO_BUF_BYTES) continue;
    best = tr;
    break;
  }
  if (best == 0) return false;
  while (best > 1 && (int64_t)s.n_ct * ceil_div(g.ho, best) * g.n * g.g < 512) {
    const int64_t half = ceil_div(best, 2);
    if (ceil_div(g.ho, half) == ceil_div(g.ho, best)) break;
    best = half;
  }
  s.tr = (int)best;
  s.tih = (int)((best - 1) * g.sh + (g.kh - 1) * g.dh + 1);
  s.tiw = (int)((s.tcb * 16 - 1) * g.sw + (g.kw - 1) * g.dw + 1);
  s.n_rt = (int)ceil_div(g.ho, best);
  const int64_t grid = (int64_t)s.n_ct * s.n_rt * g.n * g.g;
  if (grid > 2147483647LL) return false;
  *hs = s;
  return true;
}

int make_plan(const conv_problem* p, int dtype, const Geo& g, Plan* pl) {
  memset(pl, 0, sizeof(*pl));
  pl->splits = 1;
  int v = p->variant_override;
  if (g.transpose) {
    if (v != CONV_VARIANT_AUTO && v != CONV_VARIANT_TRANSPOSE_GEMM_COL2IM) return CONV_ERR_ARG;
    pl->variant = CONV_VARIANT_TRANSPOSE_GEMM_COL2IM;
    if (p->split_override > 1) return CONV_ERR_ARG;
    if (transpose_fused_applicable(g, dtype, p->has_residual == 1)) {
      pl->ct_fused = 1;
      // 64-row tiles when 128-row ones would leave compute units idle
      const int64_t tiles128 =
          g.n * ceil_div(g.h * g.w, (128 / g.w) * g.w) * ceil_div(4 * g.co, 128);
      pl->pw_tc = tiles128 < kPlanCUs ? 64 : 128;
      pl->scratch_whole = 0;
      return CONV_OK;
    }
    pl->scratch_per_image = (uint64_t)(g.co * g.kh * g.kw * g.h * g.w) * 4u;
    const int ept = half16(dtype) ? 8 : 4;
    pl->ksteps = (int)ceil_div(g.cig, 4 * ept);
    pl->steps_per_split = pl->ksteps;
    if (ceil_div(g.co * g.kh * g.kw / g.g, IG_TILE_C) > 65535 || g.g > 65535) return CONV_ERR_SHAPE;
  } else {
    if (v == CONV_VARIANT_TRANSPOSE_GEMM_COL2IM) return CONV_ERR_ARG;
    if (v == CONV_VARIANT_WINOGRAD) {  // only when asked for (see conv.h)
      if (!winograd_applicable(g, dtype) || p->split_override > 1) return CONV_ERR_ARG;
      pl->variant = v;
      // a workgroup's tiles: a band of whole tile rows of one image (a row of
      // at most 32 tiles), else 32 tiles of one tile row
      const int64_t th = ceil_div(g.ho, 2), tw = ceil_div(g.wo, 2);
      pl->wino_tc = (int)std::min<int64_t>(tw, 32);
      pl->wino_tr = (int)std::min<int64_t>(32 / pl->wino_tc, th);
      const int64_t bands = g.n * ceil_div(th, pl->wino_tr) * ceil_div(tw, pl->wino_tc);
      pl->wino_cb = bands * ceil_div(g.cog, 64) * g.g >= kPlanCUs ? 2 : 1;
      pl->scratch_per_image = (uint64_t)(16 * g.co * g.cig) * 2u;
      pl->scratch_whole = pl->scratch_per_image;
      pl->scratch_fixed = 1;
      return CONV_OK;
    }
    const bool pw_ok = pointwise_applicable(g, dtype);
    if (v == CONV_VARIANT_POINTWISE_GEMM && !pw_ok) return CONV_ERR_ARG;
    if (v == CONV_VARIANT_AUTO && pw_ok && p->split_override <= 1) v = CONV_VARIANT_POINTWISE_GEMM;
    const bool gc_ok = grouped_applicable(g, dtype);
    if (v == CONV_VARIANT_IMPLICIT_GEMM_GROUPED && !gc_ok) return CONV_ERR_ARG;
    if (v == CONV_VARIANT_AUTO && gc_ok && p->split_override <= 1) v = CONV_VARIANT_IMPLICIT_GEMM_GROUPED;
    if (v == CONV_VARIANT_IMPLICIT_GEMM_GROUPED) {
      if (p->split_override > 1) return CONV_ERR_ARG;
      pl->variant = v;
      pl->scratch_whole = 0;
      return CONV_OK;
    }
    const bool rb_ok = rowband_applicable(g, dtype);
    if (v == CONV_VARIANT_IMPLICIT_GEMM_ROWBAND && !rb_ok) return CONV_ERR_ARG;
    if (v == CONV_VARIANT_AUTO && rb_ok && p->split_override <= 1) v = CONV_VARIANT_IMPLICIT_GEMM_ROWBAND;
    if (v == CONV_VARIANT_IMPLICIT_GEMM_ROWBAND) {
      if (p->split_override > 1) return CONV_ERR_ARG;
      pl->variant = v;
      // bands of output rows: one round of workgroups at full size (the ring
      // refill per band costs KH rows)
      const int64_t tiles = g.n * ceil_div(g.co, 64);
      int64_t bands = std::max<int64_t>(1, std::min<int64_t>(g.ho, ceil_div(256, tiles)));
      pl->rb_band_rows = (int)ceil_div(g.ho, bands);
      pl->scratch_whole = 0;
      return CONV_OK;
    }
    if (v == CONV_VARIANT_POINTWISE_GEMM) {
      if (p->split_override > 1) return CONV_ERR_ARG;
      pl->variant = v;
      pl->pw_tc = dtype == CONV_F32 ? 80 : g.co > 64 ? 128 : 64;
      // float32 with a short pixel axis: the 64 x 80 tiles would not fill two
      // workgroups per CU, so each tile's chunked loads would wait with nothing
      // to hide them; strips of 16 channels x 256 pixels keep a window of steps
      // in flight in registers instead (x is read once per 16 channels: at most
      // 8 times)
      pl->pw_strip = dtype == CONV_F32 && g.ci % 16 == 0 && g.co <= 128 &&
                     ceil_div(g.n * g.h * g.w, 64) * ceil_div(g.co, 80) <= 2 * kPlanCUs;
      pl->scratch_whole = 0;
      return CONV_OK;
    }
    HaloShape hs{};
    const bool halo_ok = plan_halo(g, dtype, &hs);
    if (v == CONV_VARIANT_IMPLICIT_GEMM_HALO && !halo_ok) return CONV_ERR_ARG;
    // row-shift split k (grids that fill at most half the CUs): the largest
    // count of equal ranges of 64-channel stages that keeps the grid at most
    // one workgroup per CU
    const int64_t rs_grid = (int64_t)hs.n_ct * g.n * g.g;
    const int64_t rs_stages = g.cig / 64;
    int64_t rs_split = 1;
    if (halo_ok && hs.rowshift) {
      if (p->split_override >= 1) {
        rs_split = p->split_override;
      } else if (rs_grid * 2 <= kPlanCUs) {
        for (int64_t r = std::min<int64_t>(rs_stages, kMaxSplits); r >= 2; --r)
          if (rs_stages % r == 0 && rs_grid * r <= kPlanCUs) { rs_split = r; break; }
      }
    }
    if (v == CONV_VARIANT_AUTO) {
      if (depthwise_applicable(g)) v = CONV_VARIANT_DEPTHWISE_DIRECT;
      else if (halo_ok && hs.rowshift && rs_split > 1 && rs_stages % rs_split == 0)
        v = CONV_VARIANT_IMPLICIT_GEMM_HALO;
      else if (halo_ok && p->split_override <= 1 &&
               (int64_t)hs.n_ct * hs.n_rt * g.n * g.g >= (hs.rowshift ? 32 : 128))
        v = CONV_VARIANT_IMPLICIT_GEMM_HALO;
      else v = CONV_VARIANT_IMPLICIT_GEMM;
    }
    if (v == CONV_VARIANT_IMPLICIT_GEMM_HALO) {
      if (p->split_override > 1 && !hs.rowshift) return CONV_ERR_ARG;
      pl->halo = hs;
      if (rs_split > 1) {
        // ranges of whole stages only; the row-shift kernel alone splits
        if (!hs.rowshift || rs_stages % rs_split != 0 || rs_grid * rs_split > 2147483647LL)
          return CONV_ERR_ARG;
        pl->splits = (int)rs_split;
        pl->ksteps = (int)rs_stages;
        pl->steps_per_split = (int)(rs_stages / rs_split);
        pl->scratch_per_image = (uint64_t)(rs_split * g.co * g.ho * g.wo) * 4u;
      }
    } else if (v == CONV_VARIANT_DEPTHWISE_DIRECT) {
      if (!depthwise_applicable(g)) return CONV_ERR_ARG;
      if (p->split_override > 1) return CONV_ERR_ARG;
      if (!plan_depthwise(g, pl)) return CONV_ERR_SHAPE;
    } else {
      // implicit GEMM: k-blocks of 64 bytes; split only small grids with long k
      const int ept = half16(dtype) ? 8 : 4;
      const int64_t kg = g.cig * g.kh * g.kw;
      const int64_t steps = ceil_div(kg, 4 * ept);
      const int64_t tiles = ceil_div(g.n * g.ho * g.wo, IG_TILE_P) * ceil_div(g.cog, IG_TILE_C) * g.g;
      int64_t r = 1;
      if (p->split_override >= 1) {
        r = std::min<int64_t>(p->split_override, steps);
      } else if (tiles < 256 && steps >= 8) {
        r = std::min<int64_t>({(int64_t)kMaxSplits, ceil_div(512, tiles), steps / 4});
        if (r < 2) r = 1;
      }
      const int64_t per = ceil_div(steps, r);
      r = ceil_div(steps, per);
      pl->splits = (int)r;
      pl->ksteps = (int)steps;
      pl->steps_per_split = (int)per;
      if (ceil_div(g.cog, IG_TILE_C) > 65535 || g.g * r > 65535) return CONV_ERR_SHAPE;
      if (r > 1) pl->scratch_per_image = (uint64_t)(r * g.co * g.ho * g.wo) * 4u;
    }
    pl->variant = v;
  }
  pl->scratch_whole = pl->scratch_per_image * (uint64_t)g.n;
  return CONV_OK;
}

const char* variant_name(int v) {
  switch (v) {
    case CONV_VARIANT_IMPLICIT_GEMM: return "implicit_gemm";
    case CONV_VARIANT_POINTWISE_GEMM: return "pointwise_gemm";
    case CONV_VARIANT_DEPTHWISE_DIRECT: return "depthwise_direct";
    case CONV_VARIANT_TRANSPOSE_GEMM_COL2IM: return "transpose_gemm_col2im";
    case CONV_VARIANT_IMPLICIT_GEMM_HALO: return "implicit_gemm_halo";
    case CONV_VARIANT_IMPLICIT_GEMM_ROWBAND: return "implicit_gemm_rowband";
    case CONV_VARIANT_IMPLICIT_GEMM_GROUPED: return "implicit_gemm_grouped";
    case CONV_VARIANT_WINOGRAD: return "winograd_f2x2_3x3";
    default: return "unknown";
  }
}

struct Range {
  uintptr_t lo, hi;
};
bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.lo < a.hi && b.lo < b.hi; }

// Every host-side check of a forward call; fills the geometry, the plan and the
// image chunk size.  Nothing is enqueued.
int check_call(const conv_problem* p, int dtype, bool transpose, const void* x, const void* w,
               const void* bias, const void* residual, const void* y, const void* scratch,
               uint64_t scratch_bytes, Geo* gout, Plan* plout, int64_t* chunk_out) {
  Geo g;
  if (!p) return CONV_ERR_ARG;
  if ((p->transpose == 1) != transpose) return CONV_ERR_ARG;
  int st = validate(p, dtype, &g);
  if (st) return st;
  Plan pl;
  st = make_plan(p, dtype, g, &pl);
  if (st) return st;
  if (!x || !w || !y) return CONV_ERR_ARG;
  if (p->has_bias && !bias) return CONV_ERR_ARG;
  if (p->has_residual && !residual) return CONV_ERR_ARG;

  const size_t es = (size_t)dtype_size(dtype);
  int64_t chunk = g.n;
  if (pl.scratch_per_image > 0) {
    if (!scratch) return CONV_ERR_SCRATCH;
    if (reinterpret_cast<uintptr_t>(scratch) % 16) return CONV_ERR_ARG;
    if (scratch_bytes < pl.scratch_per_image) return CONV_ERR_SCRATCH;
    if (!pl.scratch_fixed)
      chunk = std::min<int64_t>(g.n, (int64_t)(scratch_bytes / pl.scratch_per_image));
  }

  const char* xb = static_cast<const char*>(x) + p->x_off * es;
  const char* wb = static_cast<const char*>(w) + p->w_off * es;
  const char* bb = p->has_bias ? static_cast<const char*>(bias) + p->b_off * es : nullptr;
  const char* rb = p->has_residual ? static_cast<const char*>(residual) + p->r_off * es : nullptr;
  const char* yb = static_cast<const char*>(y) + p->y_off * es;

  // overlap rules ("Layout and operands": the scratch may live in the operands'
  // arena as long as its range overlaps no operand)
  Range rx{(uintptr_t)xb, (uintptr_t)xb + g.x_elems * es};
  Range rw{(uintptr_t)wb, (uintptr_t)wb + g.w_elems * es};
  Range rbias{(uintptr_t)bb, bb ? (uintptr_t)bb + g.co * es : (uintptr_t)bb};
  Range rr{(uintptr_t)rb, rb ? (uintptr_t)rb + g.y_elems * es : (uintptr_t)rb};
  Range ry{(uintptr_t)yb, (uintptr_t)yb + g.y_elems * es};
  if (overlaps(ry, rx) || overlaps(ry, rw) || (bb && overlaps(ry, rbias))) return CONV_ERR_OVERLAP;
  if (rb && overlaps(ry, rr) && !(ry.lo == rr.lo && ry.hi == rr.hi)) return CONV_ERR_OVERLAP;
  if (pl.scratch_per_image > 0) {
    const uint64_t used = pl.scratch_fixed ? pl.scratch_whole : (uint64_t)chunk * pl.scratch_per_image;
    Range rs{(uintptr_t)scratch, (uintptr_t)scratch + used};
    if (overlaps(rs, rx) || overlaps(rs, rw) || (bb && overlaps(rs, rbias)) ||
        (rb && overlaps(rs, rr)) || overlaps(rs, ry))
      return CONV_ERR_OVERLAP;
  }

  *gout = g;
  *plout = pl;
  *chunk_out = chunk;
  return CONV_OK;
}

}  // namespace convfwd

using namespace convfwd;

extern "C" {

int conv_output_extent(const conv_problem* p, int64_t* ho, int64_t* wo) {
  if (!p || !ho || !wo) return CONV_ERR_ARG;
  Geo g;
  int st = validate(p, CONV_F32, &g);
  if (st) return st;
  *ho = g.ho;
  *wo = g.wo;
  return CONV_OK;
}

int conv_resolve_auto_pad(conv_problem* p, int auto_pad, const int64_t* output_shape_hw) {
  if (!p) return CONV_ERR_ARG;
  if (auto_pad < CONV_AUTO_PAD_NOTSET || auto_pad > CONV_AUTO_PAD_VALID) return CONV_ERR_ARG;
  const int64_t in[2] = {p->h, p->w}, k[2] = {p->kh, p->kw}, s[2] = {p->stride_h, p->stride_w},
                d[2] = {p->dil_h, p->dil_w}, op[2] = {p->out_pad_h, p->out_pad_w};
  for (int i = 0; i < 2; ++i)
    if (in[i] < 1 || k[i] < 1 || s[i] < 1 || d[i] < 1 || in[i] > kMaxElems || k[i] > kMaxElems ||
        s[i] > kMaxElems || d[i] > kMaxElems)
      return CONV_ERR_SHAPE;
  int64_t pb[2] = {p->pad_top, p->pad_left}, pe[2] = {p->pad_bottom, p->pad_right};
  for (int i = 0; i < 2; ++i) {
    const int64_t keff = d[i] * (k[i] - 1) + 1;
    if (!p->transpose) {
      if (auto_pad == CONV_AUTO_PAD_NOTSET) continue;
      if (auto_pad == CONV_AUTO_PAD_VALID) { pb[i] = pe[i] = 0; continue; }
      const int64_t out = (in[i] + s[i] - 1) / s[i];
      int64_t total = (out - 1) * s[i] + keff - in[i];
      if (total < 0) total = 0;
      const int64_t lo = total / 2, hi = total - total / 2;
      pb[i] = auto_pad == CONV_AUTO_PAD_SAME_UPPER ? lo : hi;
      pe[i] = auto_pad == CONV_AUTO_PAD_SAME_UPPER ? hi : lo;
    } else {
      if (auto_pad == CONV_AUTO_PAD_VALID) { pb[i] = pe[i] = 0; continue; }
      int64_t out;
      if (output_shape_hw) out = output_shape_hw[i];
      else if (auto_pad == CONV_AUTO_PAD_NOTSET) continue;
      else out = s[i] * in[i];
      if (op[i] < 0 || op[i] >= s[i] || out < 1) return CONV_ERR_SHAPE;
      const int64_t total = s[i] * (in[i] - 1) + op[i] + keff - out;
      if (total < 0) return CONV_ERR_SHAPE;
      const int64_t lo = total / 2, hi = total - total / 2;
      pb[i] = auto_pad == CONV_AUTO_PAD_SAME_UPPER ? lo : hi;
      pe[i] = auto_pad == CONV_AUTO_PAD_SAME_UPPER ? hi : lo;
    }
  }
  p->pad_top = pb[0]; p->pad_left = pb[1]; p->pad_bottom = pe[0]; p->pad_right = pe[1];
  return CONV_OK;
}

int conv_scratch_size(const conv_problem* p, int dtype, uint64_t* whole, uint64_t* per_image) {
  if (!whole || !per_image) return CONV_ERR_ARG;
  Geo g;
  int st = validate(p, dtype, &g);
  if (st) return st;
  Plan pl;
  st = make_plan(p, dtype, g, &pl);
  if (st) return st;
  *whole = pl.scratch_whole;
  *per_image = pl.scratch_per_image;
  return CONV_OK;
}

int conv_describe_variant(const conv_problem* p, int dtype, char* buf, uint64_t len) {
  if (!buf) return CONV_ERR_ARG;
  Geo g;
  int st = validate(p, dtype, &g);
  if (st) return st;
  Plan pl;
  st = make_plan(p, dtype, g, &pl);
  if (st) return st;
  const char* dn = dtype == CONV_F16 ? "f16" : dtype == CONV_BF16 ? "bf16" : "f32";
  char tmp[128];
  switch (pl.variant) {
    case CONV_VARIANT_IMPLICIT_GEMM:
      snprintf(tmp, sizeof tmp, "implicit_gemm.%s.t%dx%d.split%d", dn, IG_TILE_P, IG_TILE_C,
               pl.splits);
      break;
    case CONV_VARIANT_POINTWISE_GEMM:
      if (pl.pw_strip)
        snprintf(tmp, sizeof tmp, "pointwise_gemm.%s.t256x16.strip", dn);
      else
        snprintf(tmp, sizeof tmp, "pointwise_gemm.%s.t%dx%d.k64", dn, dtype == CONV_F32 ? 64 : 128, pl.pw_tc);
      break;
    case CONV_VARIANT_IMPLICIT_GEMM_ROWBAND:
      snprintf(tmp, sizeof tmp, "implicit_gemm_rowband.%s.rows%d", dn, pl.rb_band_rows);
      break;
    case CONV_VARIANT_IMPLICIT_GEMM_GROUPED:
      snprintf(tmp, sizeof tmp, "implicit_gemm_grouped.%s.c8.n%d", dn, (int)std::min<int64_t>(32, g.cog));
      break;
    case CONV_VARIANT_TRANSPOSE_GEMM_COL2IM:
      if (pl.ct_fused)
        snprintf(tmp, sizeof tmp, "transpose_gemm_col2im.%s.fused_k2s2.t128x%d", dn, pl.pw_tc);
      else
        snprintf(tmp, sizeof tmp, "transpose_gemm_col2im.%s", dn);
      break;
    case CONV_VARIANT_DEPTHWISE_DIRECT:
      if (pl.dw_wave)
        snprintf(tmp, sizeof tmp, "depthwise_direct.%s.wave.col%d", dn, pl.dw_bh);
      else if (pl.dw_planes > 0)
        snprintf(tmp, sizeof tmp, "depthwise_direct.%s.planes%d.col%d", dn, pl.dw_planes,
                 pl.dw_bh);
      else
        snprintf(tmp, sizeof tmp, "depthwise_direct.%s.t%dx%d", dn, pl.toh, pl.tow);
      break;
    case CONV_VARIANT_WINOGRAD:
      snprintf(tmp, sizeof tmp, "winograd_f2x2_3x3.%s.band%dx%d.c%d", dn, pl.wino_tr, pl.wino_tc,
               32 * pl.wino_cb);
      break;
    case CONV_VARIANT_IMPLICIT_GEMM_HALO:
      if (pl.halo.rowshift && pl.splits > 1)
        snprintf(tmp, sizeof tmp, "implicit_gemm_halo.%s.rowshift.r%d.n32.split%d", dn, pl.halo.tr,
                 pl.splits);
      else if (pl.halo.rowshift)
        snprintf(tmp, sizeof tmp, "implicit_gemm_halo.%s.rowshift.r%d.n32", dn, pl.halo.tr);
      else
        snprintf(tmp, sizeof tmp, "implicit_gemm_halo.%s.r%dx%d.n%d.c%d", dn, pl.halo.tr,
                 pl.halo.tcb * 16, pl.halo.cb * 16, pl.halo.oct * 8);
      break;
    default:
      snprintf(tmp, sizeof tmp, "%s.%s", variant_name(pl.variant), dn);
  }
  const size_t need = strlen(tmp) + 1;
  if (len < need) return CONV_ERR_ARG;
  memcpy(buf, tmp, need);
  return CONV_OK;
}

int conv_check(const conv_problem* p, int dtype, const void* x, const void* w,
               const void* bias, const void* residual, const void* y, const void* scratch,
               uint64_t scratch_bytes) {
  if (!p) return CONV_ERR_ARG;
  Geo g;
  Plan pl;
  int64_t chunk;
  return check_call(p, dtype, p->transpose == 1, x, w, bias, residual, y, scratch, scratch_bytes,
                    &g, &pl, &chunk);
}

const char* conv_status_string(int status) {
  switch (status) {
    case CONV_OK: return "ok";
    case CONV_ERR_ARG: return "invalid argument";
    case CONV_ERR_SHAPE: return "invalid shape or size limit exceeded";
    case CONV_ERR_OVERLAP: return "operand or scratch ranges overlap";
    case CONV_ERR_SCRATCH: return "scratch buffer too small for one image";
    case CONV_ERR_DEVICE: return "HIP launch failed";
    default: return "unknown status";
  }
}

}  // extern "C"
