// ConvInteger for gfx950 ("Convolution, pooling and resize", section
// "ConvInteger"; include/conv_integer.h states the operation): y = sum over the
// real taps of (x - xz) * (w - wz[co]) in int32 with wrap-around, uint8 or int8
// x and w in any mix.
//
// Each operand is shifted to a signed byte: a uint8 value v becomes v - 128 (its
// top bit flipped), an int8 value stays, so x - xz = xs + a and w - wz = ws + b
// with a = 128 - xz (uint8) or -xz (int8), and b likewise per output channel.
// A padded tap is the value xz, staged as its own shifted byte -a, so its
// factor xs + a is exactly 0.  Over the K = cin/groups * kh * kw taps of a
// window (padded ones included, taps beyond K staged as 0 on both sides):
//
//   y = sum xs*ws + b * sum xs + a * sum ws + K * a * b        (mod 2^32)
//
// sum xs*ws is the implicit GEMM on v_mfma_i32_16x16x64_i8, with the window
// gathered into LDS while the tile is staged (no column matrix), as the float
// kernel does; the byte sums Sx (per pixel) and Sw (per channel) come from the
// staged bytes with v_dot4 against ones; the rest is uint32 arithmetic, which
// wraps exactly as the int32 result must.  The MFMA accumulator holds at most
// 1024 k-blocks of 64 taps (|sum| <= 2^30) before it is added into uint32
// totals, so no partial sum leaves the int32 range.
//
// Tile: 64 pixels x 64 output channels, 4 waves of 32 x 32 (2 x 2 blocks of
// 16 x 16), k-blocks of 64 taps double-buffered through registers and LDS.
// 3x3 stride-1 layers on narrow images take the row-shift kernel instead
// (k_convint_rs.hip).
#include <stdio.h>
#include <string.h>

#include <type_traits>

#include "conv.h"
#include "conv_integer.h"
#include "internal.h"
#include "plan.h"

namespace convfwd {

namespace {

typedef int i32x4_t __attribute__((ext_vector_type(4)));

constexpr int CI_TILE = 64;        // pixels and channels per workgroup tile
constexpr int CI_K = 64;           // taps per k-block
constexpr int CI_ROW = CI_K + 16;  // LDS row pitch in bytes
constexpr int CI_FLUSH = 1024;     // k-blocks per MFMA accumulation run

struct ConvIntArgs {
  const unsigned char* x;
  const unsigned char* w;
  const unsigned char* xzp;  // nullable: zero
  const unsigned char* wzp;  // nullable: zero
  int wz_per_channel;
  int* y;
  int n, c_in, h, w_in, c_out, kh, kw, groups;
  int sh, sw, dh, dw, pt, pl;
  int ho, wo, cig, cog, kg, pix;
  int ksteps;
  int wvec;  // weight rows start 16-byte aligned and kg % 16 == 0
};

template <bool U>
__device__ __forceinline__ int zero_value(const unsigned char* p, int i) {
  if (!p) return 0;
  return U ? (int)p[i] : (int)(signed char)p[i];
}

template <bool XU, bool WU>
__global__ __launch_bounds__(256) void convint_kernel(const ConvIntArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char As[2][CI_TILE * CI_ROW];
  __shared__ __attribute__((aligned(16))) unsigned char Bs[2][CI_TILE * CI_ROW];
  __shared__ int sx_part[4][CI_TILE];
  __shared__ int sw_part[4][CI_TILE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tile_p0 = blockIdx.x * CI_TILE, tile_c0 = blockIdx.y * CI_TILE;
  const int grp = blockIdx.z;
  const int srow = tid & 63, squart = tid >> 6;  // staged row, 16-tap quarter

  const int xz = zero_value<XU>(a.xzp, 0);
  const unsigned char xpad = (unsigned char)((XU ? (xz ^ 0x80) : xz) & 0xFF);  // shifted xz
  const unsigned char xflip = XU ? 0x80 : 0x00, wflip = WU ? 0x80 : 0x00;

  // A side: the output pixel this thread gathers for
  const int hw_out = a.ho * a.wo;
  const int p = tile_p0 + srow;
  const bool p_ok = p < a.pix;
  int n_img = 0, oh = 0, ow = 0;
  if (p_ok) {
    n_img = p / hw_out;
    const int rem = p - n_img * hw_out;
    oh = rem / a.wo;
    ow = rem - oh * a.wo;
  }
  const int ih0 = oh * a.sh - a.pt, iw0 = ow * a.sw - a.pl;
  const unsigned char* __restrict__ xg =
      a.x + ((long long)n_img * a.c_in + (long long)grp * a.cig) * a.h * a.w_in;
  const int khw = a.kh * a.kw;
  // B side: the output channel (within the group) this thread loads
  const int bcol = tile_c0 + srow;
  const bool c_ok = bcol < a.cog;
  const unsigned char* __restrict__ wrow = a.w + ((long long)grp * a.cog + (c_ok ? bcol : 0)) * a.kg;

  i32x4_t ra, rb;
  int sx = 0, sw = 0;  // this thread's share of the byte sums

  auto gather = [&](int step) __attribute__((always_inline)) {
    const int k0 = step * CI_K + squart * 16;
    unsigned char va[16];
    int ci = k0 / khw;
    int rr = k0 - ci * khw;
    int kh = rr / a.kw;
    int kw = rr - kh * a.kw;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      unsigned char v = 0;  // beyond K (or beyond the pixels): 0 on the A side
      if (p_ok && k0 + j < a.kg) {
        const int ih = ih0 + kh * a.dh, iw = iw0 + kw * a.dw;
        v = ((unsigned)ih < (unsigned)a.h && (unsigned)iw < (unsigned)a.w_in)
                ? (unsigned char)(xg[((long long)ci * a.h + ih) * a.w_in + iw] ^ xflip)
                : xpad;
      }
      va[j] = v;
      if (++kw == a.kw) {
        kw = 0;
        if (++kh == a.kh) {
          kh = 0;
          ++ci;
        }
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
      ra[q] = (int)((unsigned)va[4 * q] | ((unsigned)va[4 * q + 1] << 8) |
                    ((unsigned)va[4 * q + 2] << 16) | ((unsigned)va[4 * q + 3] << 24));
    if (a.wvec && c_ok && k0 + 16 <= a.kg) {
      rb = *reinterpret_cast<const i32x4_t*>(wrow + k0);
      const int f = WU ? (int)0x80808080u : 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) rb[q] ^= f;
    } else {
      unsigned char vb[16];
#pragma unroll
      for (int j = 0; j < 16; ++j)
        vb[j] = (c_ok && k0 + j < a.kg) ? (unsigned char)(wrow[k0 + j] ^ wflip) : 0;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        rb[q] = (int)((unsigned)vb[4 * q] | ((unsigned)vb[4 * q + 1] << 8) |
                      ((unsigned)vb[4 * q + 2] << 16) | ((unsigned)vb[4 * q + 3] << 24));
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      sx = __builtin_amdgcn_sdot4(ra[q], 0x01010101, sx, false);
      sw = __builtin_amdgcn_sdot4(rb[q], 0x01010101, sw, false);
    }
  };

  auto stash = [&](int buf) __attribute__((always_inline)) {
    *reinterpret_cast<i32x4_t*>(&As[buf][srow * CI_ROW + squart * 16]) = ra;
    *reinterpret_cast<i32x4_t*>(&Bs[buf][srow * CI_ROW + squart * 16]) = rb;
  };

  i32x4_t acc[2][2];
  unsigned tot[2][2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      acc[i][j] = i32x4_t{0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 4; ++e) tot[i][j][e] = 0u;
    }
  const int wr = wave & 1, wc = wave >> 1;
  const int frow = lane & 15, fk = (lane >> 4) * 16;

  gather(0);
  stash(0);
  __syncthreads();
  for (int s = 0; s < a.ksteps; ++s) {
    const int buf = s & 1;
    const bool more = s + 1 < a.ksteps;
    if (more) gather(s + 1);
    i32x4_t fa[2], fb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
      fa[i] = *reinterpret_cast<const i32x4_t*>(&As[buf][(wr * 32 + i * 16 + frow) * CI_ROW + fk]);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      fb[j] = *reinterpret_cast<const i32x4_t*>(&Bs[buf][(wc * 32 + j * 16 + frow) * CI_ROW + fk]);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
    if ((s + 1) % CI_FLUSH == 0) {  // keep every accumulator far inside int32
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
          for (int e = 0; e < 4; ++e) tot[i][j][e] += (unsigned)acc[i][j][e];
          acc[i][j] = i32x4_t{0, 0, 0, 0};
        }
    }
    if (more) stash(buf ^ 1);
    __syncthreads();
  }

  // byte sums of the tile's pixels and channels, added over the 4 quarters
  sx_part[squart][srow] = sx;
  sw_part[squart][srow] = sw;
  __syncthreads();

  const int ka = XU ? 128 - xz : -xz;  // x - xz = xs + ka
  const unsigned K = (unsigned)a.kg;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int col = tile_c0 + wc * 32 + j * 16 + (lane & 15);
    if (col >= a.cog) continue;
    const int co = grp * a.cog + col;
    const int wz = zero_value<WU>(a.wzp, a.wz_per_channel ? co : 0);
    const int kb = WU ? 128 - wz : -wz;  // w - wz = ws + kb
    const int lc = col - tile_c0;
    const unsigned swsum = (unsigned)sw_part[0][lc] + (unsigned)sw_part[1][lc] +
                           (unsigned)sw_part[2][lc] + (unsigned)sw_part[3][lc];
    const unsigned base = (unsigned)ka * swsum + K * (unsigned)ka * (unsigned)kb;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int lp = wr * 32 + i * 16 + (lane >> 4) * 4 + e;
        const int pp = tile_p0 + lp;
        if (pp >= a.pix) continue;
        const unsigned sxsum = (unsigned)sx_part[0][lp] + (unsigned)sx_part[1][lp] +
                               (unsigned)sx_part[2][lp] + (unsigned)sx_part[3][lp];
        const unsigned v = tot[i][j][e] + (unsigned)acc[i][j][e] + (unsigned)kb * sxsum + base;
        const int n_o = pp / hw_out, rem = pp - n_o * hw_out;
        a.y[((long long)n_o * a.c_out + co) * hw_out + rem] = (int)v;
      }
  }
}

}  // namespace

}  // namespace convfwd

using namespace convfwd;

namespace {

int convint_validate(const conv_problem* p, int x_type, int w_type, Geo* g) {
  if (!p) return CONV_ERR_ARG;
  if ((x_type != CONVI_U8 && x_type != CONVI_I8) || (w_type != CONVI_U8 && w_type != CONVI_I8))
    return CONV_ERR_ARG;
  if (p->transpose != 0 || p->activation != CONV_ACT_IDENTITY || p->has_bias != 0 ||
      p->has_residual != 0 || p->variant_override != 0 || p->split_override != 0)
    return CONV_ERR_ARG;
  // 4-byte elements for the offset checks: exact for y (int32), safe for x, w
  const int st = validate(p, CONV_F32, g);
  if (st) return st;
  if (ceil_div(g->cog, CI_TILE) > 65535 || g->g > 65535) return CONV_ERR_SHAPE;
  const int64_t taps = g->cig * g->kh * g->kw;
  if (taps > 2147483647LL - CI_K) return CONV_ERR_SHAPE;
  return CONV_OK;
}

// The row-shift kernel: 3x3, stride 1, no dilation, output rows and columns
// at most 14, channels per group a multiple of 128 (one stage: 4 waves x 32)
// and at most 14563 (the MFMA sums stay inside int32: 9 * 14563 * 2^14 < 2^31).
bool convint_rowshift_applies(const Geo& g) {
  return g.kh == 3 && g.kw == 3 && g.sh == 1 && g.sw == 1 && g.dh == 1 && g.dw == 1 &&
         g.cig % 128 == 0 && g.cig <= 14563 && g.ho <= 14 && g.wo <= 14 &&
         ceil_div(g.cog, 32) * g.n * g.g <= 2147483647LL;
}

}  // namespace

extern "C" {

int conv_integer_describe_variant(const conv_problem* p, int x_type, int w_type, char* buf,
                                  uint64_t len) {
  if (!buf) return CONV_ERR_ARG;
  Geo g;
  const int st = convint_validate(p, x_type, w_type, &g);
  if (st) return st;
  char tmp[64];
  if (convint_rowshift_applies(g))
    snprintf(tmp, sizeof tmp, "conv_integer.%s%s.rowshift.r%d.i8mfma32",
             x_type == CONVI_U8 ? "u8" : "i8", w_type == CONVI_U8 ? "u8" : "i8", g.ho <= 8 ? 8 : 14);
  else
    snprintf(tmp, sizeof tmp, "conv_integer.%s%s.implicit_gemm.i8mfma.t64x64",
             x_type == CONVI_U8 ? "u8" : "i8", w_type == CONVI_U8 ? "u8" : "i8");
  const size_t need = strlen(tmp) + 1;
  if (len < need) return CONV_ERR_ARG;
  memcpy(buf, tmp, need);
  return CONV_OK;
}

int conv_integer_check(const conv_problem* p, int x_type, int w_type, const void* x,
                       const void* w, const void* x_zero, const void* w_zero,
                       int w_zero_per_channel, const void* y) {
  Geo g;
  const int st = convint_validate(p, x_type, w_type, &g);
  if (st) return st;
  if (!x || !w || !y) return CONV_ERR_ARG;
  if (w_zero_per_channel != 0 && w_zero_per_channel != 1) return CONV_ERR_ARG;
  const uintptr_t x0 = (uintptr_t)x + (uintptr_t)p->x_off, x1 = x0 + (uintptr_t)g.x_elems;
  const uintptr_t w0 = (uintptr_t)w + (uintptr_t)p->w_off, w1 = w0 + (uintptr_t)g.w_elems;
  const uintptr_t y0 = (uintptr_t)y + (uintptr_t)p->y_off * 4, y1 = y0 + (uintptr_t)g.y_elems * 4;
  if ((y0 < x1 && x0 < y1) || (y0 < w1 && w0 < y1)) return CONV_ERR_OVERLAP;
  const uintptr_t zx = (uintptr_t)x_zero, zw = (uintptr_t)w_zero;
  const uintptr_t zw1 = zw + (w_zero_per_channel ? (uintptr_t)g.co : 1);
  if (x_zero && zx >= y0 && zx < y1) return CONV_ERR_OVERLAP;
  if (w_zero && zw < y1 && y0 < zw1) return CONV_ERR_OVERLAP;
  return CONV_OK;
}

int conv_integer_forward(const conv_problem* p, int x_type, int w_type, const void* x,
                         const void* w, const void* x_zero, const void* w_zero,
                         int w_zero_per_channel, void* y, void* stream) {
  const int st = conv_integer_check(p, x_type, w_type, x, w, x_zero, w_zero, w_zero_per_channel, y);
  if (st) return st;
  Geo g;
  convint_validate(p, x_type, w_type, &g);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool xu = x_type == CONVI_U8, wu = w_type == CONVI_U8;
  if (convint_rowshift_applies(g)) {
    ConvIntRsArgs r{};
    r.x = static_cast<const unsigned char*>(x) + p->x_off;
    r.wt = static_cast<const unsigned char*>(w) + p->w_off;
    r.xzp = static_cast<const unsigned char*>(x_zero);
    r.wzp = static_cast<const unsigned char*>(w_zero);
    r.wz_per_channel = w_zero_per_channel;
    r.y = static_cast<int*>(y) + p->y_off;
    r.n = (int)g.n; r.c_in = (int)g.ci; r.h = (int)g.h; r.w = (int)g.w; r.c_out = (int)g.co;
    r.groups = (int)g.g; r.cig = (int)g.cig; r.cog = (int)g.cog;
    r.pt = (int)g.pt; r.pl = (int)g.pl; r.ho = (int)g.ho; r.wo = (int)g.wo;
    r.n_ct = (int)ceil_div(g.cog, 32);
    const int64_t hw = g.h * g.w, howo = g.ho * g.wo;
    // 8-byte loads of 8-pixel groups at 4-byte aligned plane offsets, planes of
    // at least 8 pixels
    r.xvec = reinterpret_cast<uintptr_t>(r.x) % 4 == 0 && hw % 4 == 0 && hw >= 8;
    r.wvec = reinterpret_cast<uintptr_t>(r.wt) % 16 == 0;  // rows of cig * 9, a multiple of 16
    // every tile starts 16-byte aligned and holds whole 4-int vectors
    r.yvec = reinterpret_cast<uintptr_t>(r.y) % 16 == 0 &&
             (howo % 4 == 0 || (g.cog % 4 == 0 && g.co % 4 == 0));
    r.mg_nct = make_magic((unsigned)r.n_ct);
    r.mg_n = make_magic((unsigned)g.n);
    r.mg_g4 = make_magic((unsigned)((hw + 3) / 4));
    r.mg_w = make_magic((unsigned)g.w);
    r.mg_howo = make_magic((unsigned)howo);
    r.mg_wo = make_magic((unsigned)g.wo);
    return launch_convint_rowshift(r, xu, wu, s) == hipSuccess ? CONV_OK : CONV_ERR_DEVICE;
  }
  ConvIntArgs a{};
  a.x = static_cast<const unsigned char*>(x) + p->x_off;
  a.w = static_cast<const unsigned char*>(w) + p->w_off;
  a.xzp = static_cast<const unsigned char*>(x_zero);
  a.wzp = static_cast<const unsigned char*>(w_zero);
  a.wz_per_channel = w_zero_per_channel;
  a.y = static_cast<int*>(y) + p->y_off;
  a.n = (int)g.n; a.c_in = (int)g.ci; a.h = (int)g.h; a.w_in = (int)g.w; a.c_out = (int)g.co;
  a.kh = (int)g.kh; a.kw = (int)g.kw; a.groups = (int)g.g;
  a.sh = (int)g.sh; a.sw = (int)g.sw; a.dh = (int)g.dh; a.dw = (int)g.dw;
  a.pt = (int)g.pt; a.pl = (int)g.pl; a.ho = (int)g.ho; a.wo = (int)g.wo;
  a.cig = (int)g.cig; a.cog = (int)g.cog; a.kg = (int)(g.cig * g.kh * g.kw);
  a.pix = (int)(g.n * g.ho * g.wo);
  a.ksteps = (int)ceil_div(a.kg, CI_K);
  a.wvec = reinterpret_cast<uintptr_t>(a.w) % 16 == 0 && a.kg % 16 == 0;
  const dim3 grid((unsigned)ceil_div(a.pix, CI_TILE), (unsigned)ceil_div(a.cog, CI_TILE),
                  (unsigned)a.groups);
  if (xu && wu) hipLaunchKernelGGL((convint_kernel<true, true>), grid, dim3(256), 0, s, a);
  else if (xu) hipLaunchKernelGGL((convint_kernel<true, false>), grid, dim3(256), 0, s, a);
  else if (wu) hipLaunchKernelGGL((convint_kernel<false, true>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((convint_kernel<false, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess ? CONV_OK : CONV_ERR_DEVICE;
}

}  // extern "C"
