// Launch half of the C ABI (include/conv.h): runs the shape-only plan of
// conv_plan.cpp as a sequence of gfx950 kernel launches over chunks of whole
// images, on the caller's stream.  Nothing here allocates, frees or
// synchronises.
//
// "Convolution, pooling and resize" (OneGpu docs), "Layout and operands": a
// scratch buffer smaller than the whole batch's need runs the batch in chunks
// of whole images, which changes no bit of the result.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "conv.h"
#include "internal.h"
#include "plan.h"

using namespace convfwd;

namespace {

// Compute units of the current device (cached per device).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

int run(const conv_problem* p, int dtype, bool transpose, const void* x, const void* w,
        const void* bias, const void* residual, void* y, void* scratch, uint64_t scratch_bytes,
        void* stream) {
  Geo g;
  Plan pl;
  int64_t chunk;
  const int st = check_call(p, dtype, transpose, x, w, bias, residual, y, scratch, scratch_bytes,
                            &g, &pl, &chunk);
  if (st) return st;
  const size_t es = (size_t)dtype_size(dtype);
  const char* xb = static_cast<const char*>(x) + p->x_off * es;
  const char* wb = static_cast<const char*>(w) + p->w_off * es;
  const char* bb = p->has_bias ? static_cast<const char*>(bias) + p->b_off * es : nullptr;
  const char* rb = p->has_residual ? static_cast<const char*>(residual) + p->r_off * es : nullptr;
  char* yb = static_cast<char*>(y) + p->y_off * es;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Dtype dt = dtype == CONV_F16 ? F16 : dtype == CONV_BF16 ? BF16 : F32;
  const int64_t x_img = g.ci * g.h * g.w, y_img = g.co * g.ho * g.wo;

  for (int64_t i0 = 0; i0 < g.n; i0 += chunk) {
    const int cn = (int)std::min<int64_t>(chunk, g.n - i0);
    const char* xc = xb + i0 * x_img * es;
    const char* rc = rb ? rb + i0 * y_img * es : nullptr;
    char* yc = yb + i0 * y_img * es;
    hipError_t e = hipSuccess;
    if (pl.variant == CONV_VARIANT_DEPTHWISE_DIRECT) {
      DepthwiseArgs a{};
      a.x = xc; a.wt = wb; a.bias = bb; a.res = rc; a.y = yc;
      a.n = cn; a.c_in = (int)g.ci; a.h = (int)g.h; a.w = (int)g.w; a.c_out = (int)g.co;
      a.kh = (int)g.kh; a.kw = (int)g.kw; a.mult = (int)(g.co / g.ci);
      a.sh = (int)g.sh; a.sw = (int)g.sw; a.dh = (int)g.dh; a.dw = (int)g.dw;
      a.pt = (int)g.pt; a.pl = (int)g.pl; a.ho = (int)g.ho; a.wo = (int)g.wo;
      a.toh = pl.toh; a.tow = pl.tow; a.tih = pl.tih; a.tiw = pl.tiw;
      a.tiles_w = pl.tiles_w; a.tiles = pl.tiles;
      a.act = p->activation; a.alpha = p->act_alpha; a.beta = p->act_beta;
      const int vb = dt == F32 ? 16 : 8;
      // the whole-plane kernel reads x with vector loads only; a misaligned x
      // runs the tiled kernel (same sums in the same order)
      if (pl.dw_wave && reinterpret_cast<uintptr_t>(xc) % vb == 0) {
        const int64_t mult = g.co / g.ci, howo = g.ho * g.wo;
        a.planes = 1;
        a.bh = pl.dw_bh;
        a.nrb = (int)ceil_div(g.ho, pl.dw_bh);
        a.lm = pl.dw_lm;
        a.tpp = pl.tih * pl.tiw;
        a.oofs = a.tpp;  // tiw % 4 == 0
        a.bofs = (int)(a.oofs + (mult * howo + 3) / 4 * 4);
        a.wofs = (int)(a.bofs + (mult + 3) / 4 * 4);
        a.sofs = (int)(a.wofs + mult * ((g.kh * g.kw + 3) / 4 * 4));
        a.xvec = 1;
        a.ovec = reinterpret_cast<uintptr_t>(yc) % vb == 0 &&
                 (rc == nullptr || reinterpret_cast<uintptr_t>(rc) % vb == 0) && howo % 4 == 0;
        a.mg_w = make_magic((unsigned)g.w);
        a.mg_wo = make_magic((unsigned)g.wo);
        a.mg_howo = make_magic((unsigned)howo);
        const size_t lds = (size_t)(a.sofs + 4) * 4;
        e = launch_depthwise_wave(dt, a, cn * g.ci, device_cus(), lds, s);
      } else if (pl.dw_planes > 0 && !pl.dw_wave && reinterpret_cast<uintptr_t>(xc) % vb == 0) {
        const int64_t P = pl.dw_planes, mult = g.co / g.ci, howo = g.ho * g.wo;
        a.planes = (int)P;
        a.ngroups = (int)ceil_div(cn * g.ci, P);
        a.bh = pl.dw_bh;
        a.nrb = (int)ceil_div(g.ho, pl.dw_bh);
        a.tpp = pl.tih * pl.tiw;
        a.oofs = (int)((P * a.tpp + 3) / 4 * 4);
        a.wofs = (int)(a.oofs + P * mult * howo);
        a.bofs = (int)(a.wofs + P * mult * g.kh * g.kw);
        a.sofs = (int)(a.bofs + 2 * P * mult);
        a.xvec = 1;
        a.ovec = reinterpret_cast<uintptr_t>(yc) % vb == 0 &&
                 (rc == nullptr || reinterpret_cast<uintptr_t>(rc) % vb == 0) && howo % 4 == 0;
        a.mg_hw = make_magic((unsigned)(g.h * g.w));
        a.mg_w = make_magic((unsigned)g.w);
        a.mg_pu = make_magic((unsigned)(a.nrb * g.wo));
        a.mg_wo = make_magic((unsigned)g.wo);
        a.mg_howo = make_magic((unsigned)howo);
        const size_t lds = (size_t)dw_lds_floats(P, a.tpp, mult, howo, g.kh) * 4;
        // persistent grid: as many workgroups as fit the chip, each taking an
        // equal number of groups
        const int64_t per_cu = std::max<int64_t>(1, std::min<int64_t>(8, (160 * 1024) / (int64_t)lds));
        const int64_t slots = (int64_t)device_cus() * per_cu;
        const int64_t rounds = ceil_div(a.ngroups, slots);
        const int grid = (int)ceil_div(a.ngroups, rounds);
        e = launch_depthwise_plane(dt, a, grid, lds, s);
      } else {
        e = launch_depthwise(dt, a, s);
      }
    } else if (pl.variant == CONV_VARIANT_IMPLICIT_GEMM_ROWBAND) {
      RowbandArgs a{};
      a.x = xc; a.wt = wb; a.bias = bb; a.res = rc; a.y = yc;
      a.n = cn; a.c_in = (int)g.ci; a.h = (int)g.h; a.w = (int)g.w; a.c_out = (int)g.co;
      a.kh = (int)g.kh; a.kw = (int)g.kw; a.sh = (int)g.sh; a.pt = (int)g.pt; a.pl = (int)g.pl;
      a.ho = (int)g.ho; a.wo = (int)g.wo;
      a.n_ct = (int)ceil_div(g.co, 64);
      a.mg_nv = make_magic((unsigned)((g.w + 7) / 8));
      a.mg_cin = make_magic((unsigned)g.ci);
      a.mg_vpr = make_magic((unsigned)((g.wo + 7) / 8));
      a.mg_vpr2 = make_magic((unsigned)(2 * ((g.wo + 7) / 8)));
      a.band_rows = pl.rb_band_rows;
      a.n_band = (int)ceil_div(g.ho, a.band_rows);
      const int64_t need = std::max<int64_t>(g.pl + g.w, 2 * (g.wo - 1) + 8);
      a.rpitch = (int)((need + 1) / 2 * 2);
      // the ring area also stages the tile's weights once at the start
      a.ring_bytes = (int)((std::max<int64_t>((int64_t)g.ci * 16 * a.rpitch, 64 * g.ci * g.kh * g.kw) * 2 +
                            15) / 16 * 16);
      a.vec = reinterpret_cast<uintptr_t>(xc) % 16 == 0 && reinterpret_cast<uintptr_t>(yc) % 16 == 0 &&
              g.w % 8 == 0 && g.wo % 8 == 0;
      {
        // two output rows per step: 64-channel tiles on the vector path, the new
        // rows of two output rows one item per thread of 512, the first step's
        // KH + SH rows at most the fill's item count
        const int64_t nv = ceil_div(g.w, 8);
        a.two_rows = a.vec && g.co > 32 && 2 * g.sh * g.ci * nv <= 512 && (g.kh + g.sh) * g.ci * nv <= 1024;
      }
      {
        const int64_t per_co = g.ci * g.kh * g.kw;
        // every tile's run starts at a multiple of 64 channels: whole vectors when
        // the base is aligned and each tile's length is a multiple of 8 halves
        a.wvec = reinterpret_cast<uintptr_t>(wb) % 16 == 0 &&
                 (std::min<int64_t>(64, g.co) * per_co) % 8 == 0 && ((g.co % 64) * per_co) % 8 == 0;
      }
      a.act = p->activation; a.alpha = p->act_alpha; a.beta = p->act_beta;
      e = launch_rowband(dt, a, s);
    } else if (pl.variant == CONV_VARIANT_POINTWISE_GEMM) {
      if (dt == F32 && pl.pw_strip) {
        PwArgs a{};
        a.x = xc; a.wt = wb; a.bias = bb; a.res = rc; a.y = yc;
        a.n = cn; a.c_in = (int)g.ci; a.hw = (int)(g.h * g.w); a.c_out = (int)g.co;
        a.mg_hw = make_magic((unsigned)a.hw);
        a.n_pt = (int)ceil_div((int64_t)cn * g.h * g.w, 256);
        a.n_ct = (int)ceil_div(g.co, 16);
        a.ntiles = a.n_pt * a.n_ct;
        a.vec = reinterpret_cast<uintptr_t>(xc) % 16 == 0 && reinterpret_cast<uintptr_t>(wb) % 16 == 0 &&
                reinterpret_cast<uintptr_t>(yc) % 16 == 0 &&
                (rc == nullptr || reinterpret_cast<uintptr_t>(rc) % 16 == 0);
        a.act = p->activation; a.alpha = p->act_alpha; a.beta = p->act_beta;
        e = launch_pointwise_f32_strip(a, s);
      } else if (dt == F32) {
        PwArgs a{};
        a.x = xc; a.wt = wb; a.bias = bb; a.res = rc; a.y = yc;
        a.n = cn; a.c_in = (int)g.ci; a.hw = (int)(g.h * g.w); a.c_out = (int)g.co;
        a.mg_hw = make_magic((unsigned)a.hw);
        a.n_pt = (int)ceil_div((int64_t)cn * g.h * g.w, 64);
        a.n_ct = (int)ceil_div(g.co, 80);
        a.nchunks = (int)ceil_div(g.ci, 64);
        a.vec = reinterpret_cast<uintptr_t>(xc) % 16 == 0 && reinterpret_cast<uintptr_t>(wb) % 16 == 0;
        a.act = p->activation; a.alpha = p->act_alpha; a.beta = p->act_beta;
        e = launch_pointwise_f32(a, s);
      } else {
      PwArgs a{};
      a.x = xc; a.wt = wb; a.bias = bb; a.res = rc; a.y = yc;
      a.n = cn; a.c_in = (int)g.ci; a.hw = (int)(g.h * g.w); a.c_out = (int)g.co;
      a.n_pt = (int)ceil_div(g.h * g.w, 128);
      a.tp = 128;
      a.tc = pl.pw_tc;
      a.n_ct = (int)ceil_div(g.co, a.tc);
      a.ntiles = (int)((int64_t)cn * a.n_pt * a.n_ct);
      a.nchunks = (int)ceil_div(g.ci, 64);
      a.vec = reinterpret_cast<uintptr_t>(xc) % 8 == 0 && reinterpret_cast<uintptr_t>(wb) % 16 == 0 &&
              reinterpret_cast<uintptr_t>(yc) % 16 == 0 &&
              (rc == nullptr || reinterpret_cast<uintptr_t>(rc) % 8 == 0) && (g.h * g.w) % 8 == 0;
      a.act = p->activation; a.alpha = p->act_alpha; a.beta = p->act_beta;
      a.mg_nch = make_magic((unsigned)a.nchunks);
      a.mg_nct = make_magic((unsigned)a.n_ct);
      a.mg_npt = make_magic((unsigned)a.n_pt);
      e = launch_pointwise(dt, a, device_cus(), s);
      }
    } else if (pl.variant == CONV_VARIANT_IMPLICIT_GEMM_HALO) {
      HaloArgs a{};
      a.x = xc; a.wt = wb; a.bias = bb; a.res = rc; a.y = yc;
      a.n = cn; a.c_in = (int)g.ci; a.h = (int)g.h; a.w = (int)g.w; a.c_out = (int)g.co;
      a.kh = (int)g.kh; a.kw = (int)g.kw; a.groups = (int)g.g;
      a.sh = (int)g.sh; a.sw = (int)g.sw; a.dh = (int)g.dh; a.dw = (int)g.dw;
      a.pt = (int)g.pt; a.pl = (int)g.pl; a.ho = (int)g.ho; a.wo = (int)g.wo;
      a.cig = (int)g.cig; a.cog = (int)g.cog;
      a.oct = pl.halo.oct; a.tr = pl.halo.tr; a.tcb = pl.halo.tcb; a.cb = pl.halo.cb;
      a.tih = pl.halo.tih; a.tiw = pl.halo.tiw; a.n_ct = pl.halo.n_ct; a.n_rt = pl.halo.n_rt;
      a.wvec = reinterpret_cast<uintptr_t>(wb) % 16 == 0;
      a.xvec = reinterpret_cast<uintptr_t>(xc) % 8 == 0 && (g.h * g.w) % 4 == 0 && g.h * g.w >= 8;
      a.ovec = reinterpret_cast<uintptr_t>(yc) % 8 == 0 && (!rc || reinterpret_cast<uintptr_t>(rc) % 8 == 0) &&
               (g.ho * g.wo) % 4 == 0;
      a.o2 = reinterpret_cast<uintptr_t>(yc) % 4 == 0 && (!rc || reinterpret_cast<uintptr_t>(rc) % 4 == 0) &&
             g.wo % 2 == 0;
      // every 32-channel tile of y starts 16-byte aligned: (image, channel)
      // plane offsets n c_out + g cog + 32 k times ho wo are multiples of 8
      a.oflat = reinterpret_cast<uintptr_t>(yc) % 16 == 0 && (!rc || reinterpret_cast<uintptr_t>(rc) % 16 == 0) &&
                g.wo % 2 == 0 && g.ho * g.wo >= 8 && (g.co * g.ho * g.wo) % 8 == 0 &&
                (g.cog * g.ho * g.wo) % 8 == 0;
      a.mg_w = make_magic((unsigned)g.w);
      a.mg_g4 = make_magic((unsigned)((g.h * g.w + 3) / 4));
      a.mg_nct = make_magic((unsigned)a.n_ct);
      a.mg_n = make_magic((unsigned)cn);
      a.act = p->activation; a.alpha = p->act_alpha; a.beta = p->act_beta;
      a.splits = 1;
      a.sps = (int)(g.cig / 64);
      if (pl.splits > 1) {  // row-shift split k: raw planes, then the ordered reduce
        a.splits = pl.splits;
        a.sps = pl.steps_per_split;
        a.planes = static_cast<float*>(scratch);
        a.plane_stride = (long long)cn * y_img;
        a.mg_ng = make_magic((unsigned)(cn * g.g));
        a.bias = nullptr; a.res = nullptr;
        a.oflat = 0; a.o2 = 0;
        a.act = CONV_ACT_IDENTITY;
      }
      e = pl.halo.rowshift ? launch_rowshift(dt, a, s) : launch_halo(dt, a, s);
      if (e == hipSuccess && pl.splits > 1) {
        ReduceArgs r{};
        r.planes = static_cast<const float*>(scratch);
        r.plane_stride = (long long)cn * y_img;
        r.splits = pl.splits;
        r.bias = bb; r.res = rc; r.y = yc;
        r.total = (long long)cn * y_img;
        r.hw = (int)(g.ho * g.wo); r.c_out = (int)g.co;
        r.vec = r.total % 4 == 0 && r.plane_stride % 4 == 0;
        r.act = p->activation; r.alpha = p->act_alpha; r.beta = p->act_beta;
        e = launch_reduce(dt, r, s);
      }
    } else if (pl.variant == CONV_VARIANT_IMPLICIT_GEMM) {
      IgemmArgs a{};
      a.x = xc; a.wt = wb; a.bias = bb; a.res = rc; a.y = yc;
      a.planes = static_cast<float*>(scratch);
      a.n = cn; a.c_in = (int)g.ci; a.h = (int)g.h; a.w = (int)g.w; a.c_out = (int)g.co;
      a.kh = (int)g.kh; a.kw = (int)g.kw; a.groups = (int)g.g;
      a.sh = (int)g.sh; a.sw = (int)g.sw; a.dh = (int)g.dh; a.dw = (int)g.dw;
      a.pt = (int)g.pt; a.pl = (int)g.pl; a.ho = (int)g.ho; a.wo = (int)g.wo;
      a.cig = (int)g.cig; a.cog = (int)g.cog; a.kg = (int)(g.cig * g.kh * g.kw);
      a.pix = (int)(cn * g.ho * g.wo);
      a.ksteps = pl.ksteps; a.steps_per_split = pl.steps_per_split; a.splits = pl.splits;
      a.wtrans = 0;
      const int ept = dt == F32 ? 4 : 8;
      a.wvec = (a.kg % ept == 0) && (reinterpret_cast<uintptr_t>(wb) % 16 == 0);
      a.mode = pl.splits > 1 ? OUT_RAW : OUT_FUSED;
      a.act = p->activation; a.alpha = p->act_alpha; a.beta = p->act_beta;
      a.plane_stride = (long long)cn * y_img;
      e = launch_igemm(dt, a, s);
      if (e == hipSuccess && pl.splits > 1) {
        ReduceArgs r{};
        r.planes = static_cast<const float*>(scratch);
        r.plane_stride = (long long)cn * y_img;
        r.splits = pl.splits;
        r.bias = bb; r.res = rc; r.y = yc;
        r.total = (long long)cn * y_img;
        r.hw = (int)(g.ho * g.wo); r.c_out = (int)g.co;
        r.vec = r.total % 4 == 0 && r.plane_stride % 4 == 0;
        r.act = p->activation; r.alpha = p->act_alpha; r.beta = p->act_beta;
        e = launch_reduce(dt, r, s);
      }
    } else if (pl.variant == CONV_VARIANT_WINOGRAD) {
      WinoArgs a{};
      a.x = xc; a.wt = wb; a.bias = bb; a.res = rc; a.y = yc; a.u = scratch;
      a.n = cn; a.c_in = (int)g.ci; a.h = (int)g.h; a.w = (int)g.w; a.c_out = (int)g.co;
      a.groups = (int)g.g; a.cig = (int)g.cig; a.cog = (int)g.cog;
      a.pt = (int)g.pt; a.pl = (int)g.pl; a.ho = (int)g.ho; a.wo = (int)g.wo;
      a.th = (int)ceil_div(g.ho, 2); a.tw = (int)ceil_div(g.wo, 2);
      a.tr = pl.wino_tr; a.tc = pl.wino_tc;
      a.nbr = (int)ceil_div(a.th, a.tr); a.nbc = (int)ceil_div(a.tw, a.tc);
      a.cb = pl.wino_cb;
      const int rc = (2 * a.tr + 2) * (2 * a.tc + 2);
      a.nsi = 16 * rc <= 256 * 10 ? 10 : 17;
      a.mg_nb = make_magic((unsigned)(a.nbr * a.nbc));
      a.mg_nbc = make_magic((unsigned)a.nbc);
      a.mg_tc = make_magic((unsigned)a.tc);
      a.mg_rc = make_magic((unsigned)rc);
      a.mg_c = make_magic((unsigned)(2 * a.tc + 2));
      a.act = p->activation; a.alpha = p->act_alpha; a.beta = p->act_beta;
      e = launch_winograd(dt, a, s);
    } else if (pl.variant == CONV_VARIANT_IMPLICIT_GEMM_GROUPED) {
      GroupedArgs a{};
      a.x = xc; a.wt = wb; a.bias = bb; a.res = rc; a.y = yc;
      a.n = cn; a.c_in = (int)g.ci; a.h = (int)g.h; a.w = (int)g.w; a.c_out = (int)g.co;
      a.groups = (int)g.g; a.cog = (int)g.cog;
      a.kh = (int)g.kh; a.kw = (int)g.kw; a.sh = (int)g.sh; a.sw = (int)g.sw;
      a.dh = (int)g.dh; a.dw = (int)g.dw; a.pt = (int)g.pt; a.pl = (int)g.pl;
      a.ho = (int)g.ho; a.wo = (int)g.wo;
      a.hp = (int)(g.h + g.pt + g.pb); a.wp = (int)(g.w + g.pl + g.pr);
      a.xs_bytes = a.hp * a.wp * 16;
      a.vec = reinterpret_cast<uintptr_t>(xc) % 8 == 0 && (g.h * g.w) % 4 == 0;
      a.mg_w = make_magic((unsigned)g.w);
      a.mg_wo = make_magic((unsigned)g.wo);
      a.mg_kw = make_magic((unsigned)g.kw);
      a.mg_taps = make_magic((unsigned)(g.kh * g.kw));
      a.act = p->activation; a.alpha = p->act_alpha; a.beta = p->act_beta;
      e = launch_grouped(dt, a, s);
    } else if (pl.variant == CONV_VARIANT_TRANSPOSE_GEMM_COL2IM && pl.ct_fused) {
      // GEMM rows m = 4 co + 2 kh + kw over whole input rows of one image; the
      // epilogue writes y[n][co][2h + kh][2w + kw] directly
      PwArgs a{};
      a.x = xc; a.wt = wb; a.bias = bb; a.res = nullptr; a.y = yc;
      a.n = cn; a.c_in = (int)g.ci; a.hw = (int)(g.h * g.w); a.c_out = (int)(4 * g.co);
      a.ct = 1; a.w_in = (int)g.w;
      a.ct_rows = (int)(128 / g.w);
      a.tp = a.ct_rows * (int)g.w;
      a.mg_vpr = make_magic((unsigned)(g.w / 4));
      a.mg_rows = make_magic((unsigned)a.ct_rows);
      a.n_pt = (int)ceil_div(g.h * g.w, a.tp);
      a.tc = pl.pw_tc;
      a.n_ct = (int)ceil_div(4 * g.co, a.tc);
      a.ntiles = (int)((int64_t)cn * a.n_pt * a.n_ct);
      a.nchunks = (int)ceil_div(g.ci, 64);
      a.vec = reinterpret_cast<uintptr_t>(xc) % 8 == 0 && reinterpret_cast<uintptr_t>(wb) % 8 == 0 &&
              reinterpret_cast<uintptr_t>(yc) % 16 == 0;
      a.act = p->activation; a.alpha = p->act_alpha; a.beta = p->act_beta;
      a.mg_nch = make_magic((unsigned)a.nchunks);
      a.mg_nct = make_magic((unsigned)a.n_ct);
      a.mg_npt = make_magic((unsigned)a.n_pt);
      e = launch_pointwise(dt, a, device_cus(), s);
    } else if (pl.variant == CONV_VARIANT_TRANSPOSE_GEMM_COL2IM) {
      // GEMM: cols[n][g*M + m][h][w] = sum_ci w[g*cig + ci][m] * x[n][g*cig + ci][h][w],
      // M = (Cout/G)*KH*KW; the matrix kernel runs it as a 1x1 conv with transposed
      // weight rows into raw float32 planes.
      const int64_t M = g.cog * g.kh * g.kw;
      IgemmArgs a{};
      a.x = xc; a.wt = wb; a.bias = nullptr; a.res = nullptr; a.y = nullptr;
      a.planes = static_cast<float*>(scratch);
      a.n = cn; a.c_in = (int)g.ci; a.h = (int)g.h; a.w = (int)g.w;
      a.c_out = (int)(M * g.g); a.kh = 1; a.kw = 1; a.groups = (int)g.g;
      a.sh = 1; a.sw = 1; a.dh = 1; a.dw = 1; a.pt = 0; a.pl = 0;
      a.ho = (int)g.h; a.wo = (int)g.w;
      a.cig = (int)g.cig; a.cog = (int)M; a.kg = (int)g.cig;
      a.pix = (int)(cn * g.h * g.w);
      a.ksteps = pl.ksteps; a.steps_per_split = pl.steps_per_split; a.splits = 1;
      a.wtrans = 1; a.wvec = 0; a.mode = OUT_RAW;
      a.plane_stride = 0;
      e = launch_igemm(dt, a, s);
      if (e == hipSuccess) {
        Col2imArgs c{};
        c.cols = static_cast<const float*>(scratch);
        c.bias = bb; c.res = rc; c.y = yc;
        c.n = cn; c.h = (int)g.h; c.w = (int)g.w; c.c_out = (int)g.co; c.cog = (int)g.cog;
        c.kh = (int)g.kh; c.kw = (int)g.kw; c.sh = (int)g.sh; c.sw = (int)g.sw;
        c.dh = (int)g.dh; c.dw = (int)g.dw; c.pt = (int)g.pt; c.pl = (int)g.pl;
        c.ho = (int)g.ho; c.wo = (int)g.wo;
        c.total = (long long)cn * y_img;
        c.act = p->activation; c.alpha = p->act_alpha; c.beta = p->act_beta;
        e = launch_col2im(dt, c, s);
      }
    } else {
      return CONV_ERR_ARG;
    }
    if (e != hipSuccess) return CONV_ERR_DEVICE;
  }
  return CONV_OK;
}


// Scratch held by the library for conv_forward_noalloc: split-k planes and
// ConvTranspose float32 columns, for callers that cannot allocate.  The array
// is a device global, one copy per GPU, kept until the process ends.  Host code
// never uses its name as an address: the device address of each GPU's copy is
// taken once per device with hipGetSymbolAddress and cached below.
constexpr uint64_t kNoallocScratchBytes = 64ull << 20;
__device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's copy of `scratch`, or nullptr.
void* noalloc_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr) return ptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (!ptr) {
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev].store(ptr, std::memory_order_release);
  }
  return ptr;
}

}  // namespace

extern "C" {

int conv_forward_noalloc(const conv_problem* p, int dtype, const void* x, const void* w,
                         const void* bias, const void* residual, void* y, void* stream) {
  if (!p) return CONV_ERR_ARG;
  const bool tr = p->transpose == 1;
  uint64_t whole = 0, per = 0;
  const int st = conv_scratch_size(p, dtype, &whole, &per);
  if (st) return st;
  if (per > kNoallocScratchBytes) return CONV_ERR_SCRATCH;  // one image needs more than the array
  if (per == 0) return run(p, dtype, tr, x, w, bias, residual, y, nullptr, 0, stream);
  void* sp = noalloc_scratch();
  if (!sp) return CONV_ERR_DEVICE;
  // the largest whole number of images that fits; run() chunks the batch by it
  const uint64_t bytes = std::min<uint64_t>(whole, kNoallocScratchBytes / per * per);
  return run(p, dtype, tr, x, w, bias, residual, y, sp, bytes, stream);
}

int conv_forward(const conv_problem* p, int dtype, const void* x, const void* w,
                 const void* bias, const void* residual, void* y, void* scratch,
                 uint64_t scratch_bytes, void* stream) {
  return run(p, dtype, false, x, w, bias, residual, y, scratch, scratch_bytes, stream);
}

int conv_transpose_forward(const conv_problem* p, int dtype, const void* x, const void* w,
                           const void* bias, const void* residual, void* y, void* scratch,
                           uint64_t scratch_bytes, void* stream) {
  return run(p, dtype, true, x, w, bias, residual, y, scratch, scratch_bytes, stream);
}

}  // extern "C"
