// Test driver for the host-only code, built with AddressSanitizer and
// UndefinedBehaviorSanitizer (tests/test_sanitizers.py compiles it with g++ and
// runs it; there is no GPU code in it).  It links the shape-only planner of the
// library (conv_plan.cpp: validation, auto_pad, plan, describe, scratch, check,
// and the pooling / ConvInteger planners when present) and the fp64 oracle
// (oracle/oracle.c), and drives both over seeded random problems, including
// sizes at and beyond the int64 and 2^31-element limits, so that an overflow,
// an out-of-bounds access or a signed-arithmetic wrap anywhere in them aborts
// the run.  Each check also compares the library's integer results (extents,
// pads) with the oracle's, as the Python CPU tier does.
#include <inttypes.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "conv.h"
#include "pool.h"

extern "C" {
typedef struct {
  int64_t n, c_in, h, w, c_out, kh, kw, groups;
  int64_t sh, sw, dh, dw;
  int64_t pt, pl, pb, pr;
  int64_t oph, opw;
  int32_t act;
  int32_t pad_;
  double alpha, beta;
} oracle_geom;
int oracle_conv_extent(int64_t in, int64_t k, int64_t s, int64_t d, int64_t pb, int64_t pe,
                       int64_t* out);
int oracle_convt_extent(int64_t in, int64_t k, int64_t s, int64_t d, int64_t pb, int64_t pe,
                        int64_t op, int64_t* out);
int oracle_auto_pad(int transpose, int mode, int64_t in, int64_t k, int64_t s, int64_t d,
                    int64_t op, int64_t out_req, int64_t* pb, int64_t* pe);
int oracle_conv2d(const oracle_geom* g, const double* x, const double* w, const double* b,
                  const double* r, double* y, double* s, int threads);
int oracle_conv2d_im2col(const oracle_geom* g, const double* x, const double* w,
                         const double* b, const double* r, double* y, int threads);
int oracle_conv_transpose2d(const oracle_geom* g, const double* x, const double* w,
                            const double* b, const double* r, double* y, double* s,
                            int threads);
int oracle_pool_extent(int64_t in, int64_t k, int64_t s, int64_t d, int64_t pb, int64_t pe,
                       int ceil_mode, int64_t* out);
int oracle_conv_transpose2d_gather(const oracle_geom* g, const double* x, const double* w,
                                   const double* b, const double* r, double* y, int threads);
}

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64() {  // xorshift64*
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return rng_state * 2685821657736338717ull;
}
static int64_t pick(int64_t lo, int64_t hi) { return lo + (int64_t)(next_u64() % (uint64_t)(hi - lo + 1)); }

// A size drawn mostly small, sometimes at the limits.
static int64_t dim(int64_t small_hi) {
  switch (next_u64() % 16) {
    case 0: return 0;
    case 1: return -pick(1, 3);
    case 2: return (int64_t)1 << pick(20, 40);
    case 3: return INT64_MAX - pick(0, 3);
    case 4: return 2147483647LL + pick(-1, 1);
    default: return pick(1, small_hi);
  }
}

static int fails = 0;
#define EXPECT(c, ...)                                   \
  do {                                                   \
    if (!(c)) {                                          \
      fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      fprintf(stderr, __VA_ARGS__);                      \
      fprintf(stderr, "\n");                             \
      ++fails;                                           \
    }                                                    \
  } while (0)

static void random_problem(conv_problem* p) {
  memset(p, 0, sizeof *p);
  p->n = dim(4); p->c_in = dim(64); p->h = dim(40); p->w = dim(40);
  p->c_out = dim(64); p->kh = dim(7); p->kw = dim(7);
  p->groups = next_u64() % 3 == 0 ? p->c_in : dim(4);
  p->stride_h = dim(3); p->stride_w = dim(3); p->dil_h = dim(3); p->dil_w = dim(3);
  p->pad_top = pick(-1, 3); p->pad_left = pick(0, 3); p->pad_bottom = pick(0, 3);
  p->pad_right = next_u64() % 20 == 0 ? INT64_MAX : pick(0, 3);
  p->transpose = (int)(next_u64() % 3 == 0);
  p->out_pad_h = pick(0, 2); p->out_pad_w = pick(0, 2);
  p->activation = (int)pick(-1, 9);
  p->has_bias = (int)pick(0, 1); p->has_residual = (int)pick(0, 1);
  p->variant_override = (int)pick(0, 8);
  if (next_u64() % 2) p->variant_override = 0;
  p->split_override = (int)pick(0, 17);
  if (next_u64() % 2) p->split_override = 0;
  const int64_t big = next_u64() % 10 == 0 ? ((int64_t)1 << pick(40, 62)) : 0;
  p->x_off = pick(0, 9) + big; p->w_off = pick(0, 9); p->b_off = pick(0, 9);
  p->r_off = pick(0, 9); p->y_off = pick(0, 9);
}

static void check_planner(int iters) {
  char buf[256];
  for (int it = 0; it < iters; ++it) {
    conv_problem p;
    random_problem(&p);
    const int dtype = (int)pick(-1, 3);
    int64_t ho = -7, wo = -7;
    const int st = conv_output_extent(&p, &ho, &wo);
    if (st == CONV_OK && p.transpose == 0) {
      int64_t oh, ow;
      const int a = oracle_conv_extent(p.h, p.kh, p.stride_h, p.dil_h, p.pad_top, p.pad_bottom, &oh);
      const int b = oracle_conv_extent(p.w, p.kw, p.stride_w, p.dil_w, p.pad_left, p.pad_right, &ow);
      if (p.h < 100000 && p.w < 100000 && p.kh < 100 && p.kw < 100 && p.pad_right < 100)
        EXPECT(a == 0 && b == 0 && oh == ho && ow == wo, "conv extent %" PRId64 " vs %" PRId64, ho, oh);
    } else if (st == CONV_OK) {
      int64_t oh, ow;
      const int a = oracle_convt_extent(p.h, p.kh, p.stride_h, p.dil_h, p.pad_top, p.pad_bottom,
                                        p.out_pad_h, &oh);
      const int b = oracle_convt_extent(p.w, p.kw, p.stride_w, p.dil_w, p.pad_left, p.pad_right,
                                        p.out_pad_w, &ow);
      if (p.h < 100000 && p.w < 100000 && p.kh < 100 && p.kw < 100 && p.pad_right < 100)
        EXPECT(a == 0 && b == 0 && oh == ho && ow == wo, "convT extent %" PRId64 " vs %" PRId64, ho, oh);
    }
    uint64_t whole = 0, per = 0;
    const int s1 = conv_scratch_size(&p, dtype, &whole, &per);
    const int s2 = conv_describe_variant(&p, dtype, buf, sizeof buf);
    EXPECT(s1 == s2, "scratch status %d vs describe status %d", s1, s2);
    if (s2 == CONV_OK) EXPECT(strlen(buf) > 0 && strlen(buf) < sizeof buf, "describe text");
    if (s1 == CONV_OK) EXPECT(whole >= per, "whole < per image");
    // fake, never dereferenced device addresses: the check does range
    // arithmetic only
    const uintptr_t base = (uintptr_t)1 << 44;
    const void* x = (const void*)(base);
    const void* w = (const void*)(base + ((uintptr_t)1 << 40));
    const void* b = (const void*)(base + ((uintptr_t)2 << 40));
    const void* r = (const void*)(base + ((uintptr_t)3 << 40));
    const void* y = next_u64() % 8 == 0 ? x : (const void*)(base + ((uintptr_t)4 << 40));
    void* sc = (void*)(base + ((uintptr_t)5 << 40) + (next_u64() % 4 == 0 ? 4 : 0));
    const int c = conv_check(&p, dtype, x, w, p.has_bias ? b : nullptr, p.has_residual ? r : nullptr,
                             y, per ? sc : nullptr, whole);
    EXPECT(c >= CONV_OK && c <= CONV_ERR_DEVICE, "check status %d", c);
    if (s1 == CONV_OK && c == CONV_OK && per) EXPECT(whole > 0, "scratch");
    (void)conv_status_string(c);
    // auto_pad against the oracle on plain sizes
    conv_problem q = p;
    for (int mode = 0; mode < 4; ++mode) {
      if (q.h < 1 || q.h > 100000 || q.kh < 1 || q.kh > 100 || q.stride_h < 1 || q.stride_h > 100 ||
          q.dil_h < 1 || q.dil_h > 100 || q.w < 1 || q.w > 100000 || q.kw < 1 || q.kw > 100 ||
          q.stride_w < 1 || q.stride_w > 100 || q.dil_w < 1 || q.dil_w > 100)
        break;
      conv_problem t = q;
      t.pad_top = t.pad_left = t.pad_bottom = t.pad_right = 1;
      const int ra = conv_resolve_auto_pad(&t, mode, nullptr);
      int64_t pb = 1, pe = 1;
      const int rb = oracle_auto_pad(t.transpose, mode, t.h, t.kh, t.stride_h, t.dil_h, t.out_pad_h,
                                     -1, &pb, &pe);
      if (ra == CONV_OK && rb == 0 && !(t.transpose && (t.out_pad_h >= t.stride_h)))
        EXPECT(pb == t.pad_top && pe == t.pad_bottom, "auto_pad mode %d: %" PRId64 ",%" PRId64
               " vs %" PRId64 ",%" PRId64, mode, t.pad_top, t.pad_bottom, pb, pe);
    }
  }
}

static void check_oracle(int iters) {
  for (int it = 0; it < iters; ++it) {
    oracle_geom g;
    memset(&g, 0, sizeof g);
    g.groups = pick(1, 3);
    g.n = pick(1, 2); g.c_in = g.groups * pick(1, 3); g.c_out = g.groups * pick(1, 3);
    g.h = pick(1, 9); g.w = pick(1, 9); g.kh = pick(1, 4); g.kw = pick(1, 4);
    g.sh = pick(1, 3); g.sw = pick(1, 3); g.dh = pick(1, 2); g.dw = pick(1, 2);
    g.pt = pick(0, 2); g.pl = pick(0, 2); g.pb = pick(0, 2); g.pr = pick(0, 2);
    g.act = (int)pick(0, 8); g.alpha = 0.1; g.beta = 0.6;
    const bool tr = next_u64() % 2;
    int64_t ho, wo;
    if (tr) {
      g.oph = pick(0, g.sh - 1); g.opw = pick(0, g.sw - 1);
      if (oracle_convt_extent(g.h, g.kh, g.sh, g.dh, g.pt, g.pb, g.oph, &ho) ||
          oracle_convt_extent(g.w, g.kw, g.sw, g.dw, g.pl, g.pr, g.opw, &wo))
        continue;
    } else if (oracle_conv_extent(g.h, g.kh, g.sh, g.dh, g.pt, g.pb, &ho) ||
               oracle_conv_extent(g.w, g.kw, g.sw, g.dw, g.pl, g.pr, &wo)) {
      continue;
    }
    const int64_t nx = g.n * g.c_in * g.h * g.w;
    const int64_t nw = tr ? g.c_in * (g.c_out / g.groups) * g.kh * g.kw
                          : g.c_out * (g.c_in / g.groups) * g.kh * g.kw;
    const int64_t ny = g.n * g.c_out * ho * wo;
    // exact-size heap arrays: any stray index is an ASan report
    std::vector<double> x(nx), w(nw), b(g.c_out), r(ny), y1(ny), y2(ny), s(ny);
    for (auto& v : x) v = (double)pick(-3, 3);
    for (auto& v : w) v = (double)pick(-3, 3);
    for (auto& v : b) v = (double)pick(-3, 3);
    for (auto& v : r) v = (double)pick(-3, 3);
    int a, c;
    if (tr) {
      a = oracle_conv_transpose2d(&g, x.data(), w.data(), b.data(), r.data(), y1.data(), s.data(), 1);
      c = oracle_conv_transpose2d_gather(&g, x.data(), w.data(), b.data(), r.data(), y2.data(), 1);
    } else {
      a = oracle_conv2d(&g, x.data(), w.data(), b.data(), r.data(), y1.data(), s.data(), 1);
      c = oracle_conv2d_im2col(&g, x.data(), w.data(), b.data(), r.data(), y2.data(), 1);
    }
    EXPECT(a == 0 && c == 0, "oracle status %d %d", a, c);
    for (int64_t i = 0; i < ny; ++i) {
      const double d = fabs(y1[i] - y2[i]);
      EXPECT(d <= 1e-9 * (1.0 + fabs(y1[i])) || (std::isnan(y1[i]) && std::isnan(y2[i])),
             "oracle formulations differ at %" PRId64 ": %g vs %g", i, y1[i], y2[i]);
    }
  }
}

// A valid problem with one field at a time pushed to an extreme.
static void check_edges() {
  const int64_t ext[] = {0, -1, 1, 2, 3, 1LL << 31, (1LL << 31) - 1, 1LL << 40, 1LL << 61,
                         1LL << 62, INT64_MAX - 1, INT64_MAX, INT64_MIN};
  char buf[256];
  for (int field = 0; field < 23; ++field) {
    for (int64_t v : ext) {
      for (int tr = 0; tr < 2; ++tr) {
        for (int dtype = 0; dtype < 3; ++dtype) {
          conv_problem p;
          memset(&p, 0, sizeof p);
          p.n = 2; p.c_in = 8; p.h = 9; p.w = 9; p.c_out = 8; p.kh = 3; p.kw = 3; p.groups = 1;
          p.stride_h = p.stride_w = p.dil_h = p.dil_w = 1;
          p.pad_top = p.pad_left = p.pad_bottom = p.pad_right = 1;
          p.transpose = tr; p.has_bias = 1; p.has_residual = 1;
          int64_t* f[] = {&p.n, &p.c_in, &p.h, &p.w, &p.c_out, &p.kh, &p.kw, &p.groups,
                          &p.stride_h, &p.stride_w, &p.dil_h, &p.dil_w, &p.pad_top, &p.pad_left,
                          &p.pad_bottom, &p.pad_right, &p.out_pad_h, &p.out_pad_w, &p.x_off,
                          &p.w_off, &p.b_off, &p.r_off, &p.y_off};
          *f[field] = v;
          int64_t ho, wo;
          (void)conv_output_extent(&p, &ho, &wo);
          uint64_t whole, per;
          (void)conv_scratch_size(&p, dtype, &whole, &per);
          (void)conv_describe_variant(&p, dtype, buf, sizeof buf);
          const uintptr_t base = (uintptr_t)1 << 44;
          const int c = conv_check(&p, dtype, (const void*)base, (const void*)(base + (1ull << 40)),
                                   (const void*)(base + (2ull << 40)), (const void*)(base + (3ull << 40)),
                                   (const void*)(base + (4ull << 40)), (void*)(base + (5ull << 40)),
                                   ~0ull);
          EXPECT(c >= CONV_OK && c <= CONV_ERR_DEVICE, "check status %d", c);
          conv_problem q = p;
          (void)conv_resolve_auto_pad(&q, 1, nullptr);
          q = p;
          const int64_t os[2] = {v, v};
          (void)conv_resolve_auto_pad(&q, 2, os);
        }
      }
    }
  }
}

// Pooling problems, random and at the limits, through extent / auto_pad /
// describe / check, the extents compared with the oracle's.
static void check_pool(int iters) {
  char buf[256];
  for (int it = 0; it < iters; ++it) {
    pool_problem p;
    memset(&p, 0, sizeof p);
    p.n = dim(3); p.c = dim(8); p.h = dim(30); p.w = dim(30);
    p.kh = dim(5); p.kw = dim(5); p.stride_h = dim(3); p.stride_w = dim(3);
    p.dil_h = dim(2); p.dil_w = dim(2);
    p.pad_top = pick(-1, 4); p.pad_left = pick(0, 4); p.pad_bottom = pick(0, 4);
    p.pad_right = next_u64() % 20 == 0 ? INT64_MAX : pick(0, 4);
    p.kind = (int)pick(-1, 4); p.ceil_mode = (int)pick(0, 2); p.count_include_pad = (int)pick(0, 1);
    p.reserved = next_u64() % 20 == 0;
    p.x_off = next_u64() % 10 == 0 ? ((int64_t)1 << pick(40, 62)) : pick(0, 9);
    p.y_off = pick(0, 9);
    const int dtype = (int)pick(-1, 3);
    int64_t ho = 0, wo = 0;
    const int st = pool_output_extent(&p, &ho, &wo);
    if (st == CONV_OK && p.kind < 2 && p.h < 1000 && p.w < 1000 && p.kh < 100 && p.kw < 100 &&
        p.pad_right < 100 && p.stride_h < 100 && p.stride_w < 100 && p.dil_h < 100 && p.dil_w < 100) {
      int64_t oh, ow;
      const int a = oracle_pool_extent(p.h, p.kh, p.stride_h, p.dil_h, p.pad_top, p.pad_bottom,
                                       p.ceil_mode, &oh);
      const int b = oracle_pool_extent(p.w, p.kw, p.stride_w, p.dil_w, p.pad_left, p.pad_right,
                                       p.ceil_mode, &ow);
      EXPECT(a == 0 && b == 0 && oh == ho && ow == wo, "pool extent %" PRId64 " vs %" PRId64, ho, oh);
    }
    (void)pool_describe_variant(&p, dtype, buf, sizeof buf);
    const uintptr_t base = (uintptr_t)1 << 44;
    const int c = pool_check(&p, dtype, (const void*)base, (const void*)(base + ((uintptr_t)1 << 42)));
    EXPECT(c >= CONV_OK && c <= CONV_ERR_DEVICE, "pool check status %d", c);
    pool_problem q = p;
    (void)pool_resolve_auto_pad(&q, (int)pick(-1, 4));
  }
}

int main(int argc, char** argv) {
  check_edges();
  check_pool(argc > 1 ? atoi(argv[1]) : 20000);
  const int iters = argc > 1 ? atoi(argv[1]) : 20000;
  check_planner(iters);
  check_oracle(iters / 20);
  if (fails) {
    fprintf(stderr, "%d failure(s)\n", fails);
    return 1;
  }
  printf("sanitize driver: %d planner problems, %d oracle problems, no failures\n", iters,
         iters / 20);
  return 0;
}
