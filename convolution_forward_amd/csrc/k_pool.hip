// Pooling forward for gfx950 ("Convolution, pooling and resize", section
// "Pooling and resize"; include/pool.h states the operations):
//
//  * Windowed MaxPool / AveragePool, band kernel: one workgroup per (plane,
//    band of output rows).  The band's input rows (its windows' reach, clipped
//    to the input) are staged in LDS as float32 with coalesced loads (16-byte
//    vectors when rows allow), then consecutive threads take consecutive
//    outputs of a row, read their taps from LDS and store coalesced.  Rows
//    outside the input are never touched: a tap is tested against the input
//    (real), the pads (padding) or neither (beyond the padding, ceil mode).
//  * Row-vector kernel (windows of 2 or 3 taps per axis, horizontal stride 1
//    or 2, rows of whole 16-byte vectors): a thread owns one 16-byte vector
//    of each input row its output row reads and the outputs whose windows
//    start in it; the one or two elements a window reaches into the vectors
//    beside it come from the neighbouring lanes (which own those vectors)
//    through a lane shuffle, or from memory at the wave's two ends.  Every
//    load of a thread is issued before any arithmetic, so a wave keeps its
//    whole input in flight, and the outputs leave as one 8- or 16-byte
//    nontemporal store per thread.
//  * Direct kernel: the same per-output arithmetic with the taps read from
//    global memory, for rows too wide to stage.
//  * Global pools: a workgroup loads the values of up to 4096 elements (whole
//    planes, or a 4096-element chunk of a larger plane) into LDS and reduces
//    each plane with a fixed halving tree (pairs i and i + ceil(m/2) while
//    m > 1); larger planes reduce their chunk results the same way.  The order
//    depends on the plane size only: the planes per workgroup (chosen for
//    about 1024 workgroups) change which thread adds a pair, not the pairs.
//
// Max is taken over integer keys of the float32 bits (the sign-magnitude
// order turned into two's complement order), which orders -0 below +0 and
// makes the result independent of the order; NaN taps get the lowest key so
// that they are skipped, and a result still at that key is NaN if the window
// had a real tap, else the element type's lowest finite value.  Every value
// of the three element types is exact in float32, so the max is bit-exact.
// The average sums the real taps in float32 in (kh, kw) order and divides by
// the count the geometry gives (real taps, plus padding taps with
// count_include_pad).
#include <climits>
#include <type_traits>

#include "conv.h"
#include "epilogue.h"
#include "internal.h"
#include "plan.h"
#include "pool.h"
#include "pool_plan.h"

namespace convfwd {

namespace {

__device__ __forceinline__ int max_key(float v) {
  const int s = __float_as_int(v);
  return v != v ? INT_MIN : (s >= 0 ? s : s ^ 0x7FFFFFFF);
}

__device__ __forceinline__ float key_value(int k) {
  return __int_as_float(k >= 0 ? k : k ^ 0x7FFFFFFF);
}

template <typename T>
__device__ __forceinline__ float lowest_finite() {
  if constexpr (std::is_same_v<T, float>) return -3.4028234663852886e38f;
  else if constexpr (std::is_same_v<T, _Float16>) return -65504.0f;
  else return -3.3895313892515355e38f;  // bfloat16 0xff7f
}

struct PoolArgs {
  const void* x;
  void* y;
  int planes, h, w, ho, wo;
  int kh, kw, sh, sw, dh, dw, pt, pl, pb, pr;
  int cip;
  int band_rows, in_rows, n_band;
  int planes_wg, chunks;
  int vec;      // x 16-byte aligned and w % (16 / sizeof(T)) == 0: rows in 16-byte items
  int yvec;     // row vector: y aligned to a thread's outputs and wo a multiple of them
  int tpr, threads;
  Magic mg_wo, mg_w, mg_tpr, mg_ho;
  Magic mg_pairs[14];  // global tree: division by each level's pair count
};

// Taps of one window along an axis: [k0, k1) real, count_pad = taps inside
// the padded axis.  o*s - p + k*d in [0, n) for real taps, [-p, n + pe) for
// padding ones.
__device__ __forceinline__ void axis_taps(int o, int s, int p, int pe, int d, int k, int n,
                                          int& real, int& padded) {
  real = 0;
  padded = 0;
  const int st = o * s - p;
  for (int t = 0; t < k; ++t) {
    const int i = st + t * d;
    real += (i >= 0 && i < n);
    padded += (i >= -p && i < n + pe);
  }
}

// One output: LOAD(ih, iw) returns the float value of a real tap.
template <typename T, bool AVG, typename Load>
__device__ __forceinline__ T pool_one(const PoolArgs& a, int oh, int ow, Load load) {
  const int ih0 = oh * a.sh - a.pt, iw0 = ow * a.sw - a.pl;
  int rh, ph, rw, pw;
  axis_taps(oh, a.sh, a.pt, a.pb, a.dh, a.kh, a.h, rh, ph);
  axis_taps(ow, a.sw, a.pl, a.pr, a.dw, a.kw, a.w, rw, pw);
  if constexpr (AVG) {
    float sum = 0.0f;
    for (int kh = 0; kh < a.kh; ++kh) {
      const int ih = ih0 + kh * a.dh;
      if ((unsigned)ih >= (unsigned)a.h) continue;
      for (int kw = 0; kw < a.kw; ++kw) {
        const int iw = iw0 + kw * a.dw;
        if ((unsigned)iw < (unsigned)a.w) sum += load(ih, iw);
      }
    }
    const int cnt = a.cip ? ph * pw : rh * rw;
    return from_f32<T>(sum / (float)cnt);
  } else {
    int m = INT_MIN;
    for (int kh = 0; kh < a.kh; ++kh) {
      const int ih = ih0 + kh * a.dh;
      if ((unsigned)ih >= (unsigned)a.h) continue;
      for (int kw = 0; kw < a.kw; ++kw) {
        const int iw = iw0 + kw * a.dw;
        if ((unsigned)iw < (unsigned)a.w) m = max(m, max_key(load(ih, iw)));
      }
    }
    float v;
    if (m != INT_MIN) v = key_value(m);
    else v = rh * rw > 0 ? __int_as_float(0x7FC00000) : lowest_finite<T>();
    return from_f32<T>(v);
  }
}

// One output of a KH x KW window read from the staged rows: every tap's LDS
// address is clamped into the staged block, so all reads can issue at once,
// and a tap outside the input is masked out (max: the NaN key; sum: 0).
template <typename T, bool AVG, int KH, int KW>
__device__ __forceinline__ T pool_one_fixed(const PoolArgs& a, const float* rows, int ih_lo,
                                            int oh, int ow) {
  const int ih0 = oh * a.sh - a.pt, iw0 = ow * a.sw - a.pl;
  bool vh[KH], vw[KW];
  int ro[KH], co[KW];
  int rh = 0, rw = 0, ph = 0, pw = 0;
#pragma unroll
  for (int k = 0; k < KH; ++k) {
    const int ih = ih0 + k * a.dh;
    vh[k] = (unsigned)ih < (unsigned)a.h;
    rh += vh[k];
    ph += (ih >= -a.pt && ih < a.h + a.pb);
    ro[k] = (min(max(ih, ih_lo), ih_lo + a.in_rows - 1) - ih_lo) * a.w;
  }
#pragma unroll
  for (int k = 0; k < KW; ++k) {
    const int iw = iw0 + k * a.dw;
    vw[k] = (unsigned)iw < (unsigned)a.w;
    rw += vw[k];
    pw += (iw >= -a.pl && iw < a.w + a.pr);
    co[k] = min(max(iw, 0), a.w - 1);
  }
  float v[KH * KW];
#pragma unroll
  for (int kh = 0; kh < KH; ++kh)
#pragma unroll
    for (int kw = 0; kw < KW; ++kw) v[kh * KW + kw] = rows[ro[kh] + co[kw]];
  if constexpr (AVG) {
    float sum = 0.0f;
#pragma unroll
    for (int kh = 0; kh < KH; ++kh)
#pragma unroll
      for (int kw = 0; kw < KW; ++kw) sum += (vh[kh] && vw[kw]) ? v[kh * KW + kw] : 0.0f;
    const int cnt = a.cip ? ph * pw : rh * rw;
    return from_f32<T>(sum / (float)cnt);
  } else {
    int m = INT_MIN;
#pragma unroll
    for (int kh = 0; kh < KH; ++kh)
#pragma unroll
      for (int kw = 0; kw < KW; ++kw)
        m = max(m, (vh[kh] && vw[kw]) ? max_key(v[kh * KW + kw]) : INT_MIN);
    float r;
    if (m != INT_MIN) r = key_value(m);
    else r = rh * rw > 0 ? __int_as_float(0x7FC00000) : lowest_finite<T>();
    return from_f32<T>(r);
  }
}

template <typename T, bool AVG, int KF>
__global__ __launch_bounds__(256) void pool_band_kernel(const PoolArgs a) {
  extern __shared__ float rows[];  // in_rows x w
  const int plane = blockIdx.x / a.n_band;
  const int band = blockIdx.x - plane * a.n_band;
  const int oh0 = band * a.band_rows;
  const int nrow = min(a.band_rows, a.ho - oh0);
  const int ih_lo = oh0 * a.sh - a.pt;  // input row of LDS row 0 (may be < 0)
  const long long hw = (long long)a.h * a.w;
  const T* __restrict__ xp = static_cast<const T*>(a.x) + (long long)plane * hw;
  // stage the input rows of the band that exist
  const int r0 = max(0, -ih_lo), r1 = min(a.in_rows, a.h - ih_lo);
  if (r1 > r0) {
    const int n_el = (r1 - r0) * a.w;
    const T* src = xp + (long long)(ih_lo + r0) * a.w;
    float* dst = rows + r0 * a.w;
    constexpr int V = 16 / sizeof(T);
    if (a.vec) {  // rows start on 16-byte boundaries: whole-vector items
      typedef T tv __attribute__((ext_vector_type(V)));
      for (int i = threadIdx.x; i < n_el / V; i += 256) {
        const tv v = *reinterpret_cast<const tv*>(src + (long long)i * V);
#pragma unroll
        for (int e = 0; e < V; e += 4)
          *reinterpret_cast<float4*>(dst + i * V + e) =
              float4{to_f32(v[e]), to_f32(v[e + 1]), to_f32(v[e + 2]), to_f32(v[e + 3])};
      }
    } else {
      for (int i = threadIdx.x; i < n_el; i += 256) dst[i] = to_f32(src[i]);
    }
  }
  __syncthreads();
  T* __restrict__ yp = static_cast<T*>(a.y) + (long long)plane * a.ho * a.wo + (long long)oh0 * a.wo;
  const int n_out = nrow * a.wo;
  for (int i = threadIdx.x; i < n_out; i += 256) {
    const int r = (int)mdiv((unsigned)i, a.mg_wo);
    const int ow = i - r * a.wo;
    if constexpr (KF > 0)
      yp[i] = pool_one_fixed<T, AVG, KF, KF>(a, rows, ih_lo, oh0 + r, ow);
    else
      yp[i] = pool_one<T, AVG>(a, oh0 + r, ow, [&](int ih, int iw) {
        return rows[(ih - ih_lo) * a.w + iw];
      });
  }
}

// Row-vector kernel helpers.  Bits of element i of a thread's stretch of one
// input row, i in [-WE, V + WE): the last word of the left neighbour's
// vector, the thread's own four words, the first word of the right
// neighbour's.
template <typename T>
__device__ __forceinline__ unsigned stretch_bits(const unsigned (&d)[4], unsigned lw, unsigned rw,
                                                 int i) {
  constexpr int V = 16 / sizeof(T), WE = 4 / sizeof(T);
  unsigned w;
  int k;
  if (i < 0) { w = lw; k = i + WE; }
  else if (i < V) { w = d[i / WE]; k = i % WE; }
  else { w = rw; k = i - V; }
  return sizeof(T) == 4 ? w : (w >> (16 * k)) & 0xFFFFu;
}

// Max key of an element's bits: the sign-magnitude order as two's complement
// (-0 below +0); NaN, like a tap outside the input, gets INT_MIN.
template <typename T>
__device__ __forceinline__ int bits_key(unsigned b, bool ok) {
  if constexpr (sizeof(T) == 4) {
    const int s = (int)b;
    const bool nan = (b & 0x7FFFFFFFu) > 0x7F800000u;
    return ok && !nan ? s ^ ((s >> 31) & 0x7FFFFFFF) : INT_MIN;
  } else {
    constexpr unsigned kInf = std::is_same_v<T, _Float16> ? 0x7C00u : 0x7F80u;
    const int s = (int)(short)b;
    const bool nan = (b & 0x7FFFu) > kInf;
    return ok && !nan ? s ^ ((s >> 31) & 0x7FFF) : INT_MIN;
  }
}

// Bits of the max from its key; m == INT_MIN: NaN if the window had a real
// tap (all of them NaN), else the type's lowest finite value.
template <typename T>
__device__ __forceinline__ unsigned key_bits(int m, bool real) {
  if constexpr (sizeof(T) == 4) {
    return m != INT_MIN ? (unsigned)(m ^ ((m >> 31) & 0x7FFFFFFF))
                        : (real ? 0x7FC00000u : 0xFF7FFFFFu);
  } else {
    constexpr bool F16 = std::is_same_v<T, _Float16>;
    return m != INT_MIN ? (unsigned)(m ^ ((m >> 31) & 0x7FFF)) & 0xFFFFu
                        : (real ? (F16 ? 0x7E00u : 0x7FC0u) : (F16 ? 0xFBFFu : 0xFF7Fu));
  }
}

template <typename T>
__device__ __forceinline__ float bits_f32(unsigned b) {
  if constexpr (sizeof(T) == 4) return __uint_as_float(b);
  else return to_f32(__builtin_bit_cast(T, (unsigned short)b));
}

// PL: the left pad (the window of output o starts at element o * SW - PL of
// the thread's stretch).  Branch-free apart from the loads at the wave's ends:
// every load reads a clamped, valid address and taps outside the input are
// masked when the keys or terms are formed.
template <typename T, bool AVG, int KH, int KW, int SW, int PL>
__global__ __launch_bounds__(256) void pool_rowvec_kernel(const PoolArgs a) {
  constexpr int V = 16 / sizeof(T);   // elements per vector
  constexpr int WE = 4 / sizeof(T);   // elements per 32-bit word
  constexpr int OPT = V / SW;         // outputs per thread
  constexpr int NC = (OPT - 1) * SW + KW;  // columns the thread's windows cover
  static_assert(PL <= WE && NC - PL <= V + WE, "window reach beyond the neighbour words");
  const int lane = threadIdx.x & 63;
  const int t_raw = blockIdx.x * 256 + threadIdx.x;
  const bool live = t_raw < a.threads;
  const int t = live ? t_raw : a.threads - 1;  // dead lanes repeat the last thread
  const int row = (int)mdiv((unsigned)t, a.mg_tpr);
  const int j = t - row * a.tpr;
  const int plane = (int)mdiv((unsigned)row, a.mg_ho);
  const int oh = row - plane * a.ho;
  const int col0 = j * V;
  const int colc = min(col0, a.w - V);  // clamped: a valid vector of the row
  const int ih0 = oh * a.sh - a.pt;
  const T* __restrict__ xp = static_cast<const T*>(a.x) + (long long)plane * a.h * a.w;

  unsigned d[KH][4], lw[KH], rw[KH];
  bool rok[KH];
#pragma unroll
  for (int kh = 0; kh < KH; ++kh) rok[kh] = (unsigned)(ih0 + kh) < (unsigned)a.h;
  if (a.vec) {
    typedef unsigned u4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int kh = 0; kh < KH; ++kh) {
      const int ihc = min(max(ih0 + kh, 0), a.h - 1);
      const u4 v = *reinterpret_cast<const u4*>(xp + (long long)ihc * a.w + colc);
      d[kh][0] = v[0]; d[kh][1] = v[1]; d[kh][2] = v[2]; d[kh][3] = v[3];
    }
#pragma unroll
    for (int kh = 0; kh < KH; ++kh) {
      lw[kh] = __shfl_up(d[kh][3], 1);
      rw[kh] = __shfl_down(d[kh][0], 1);
    }
    // at the wave's two ends the neighbouring vector of the row is another
    // wave's: its word comes from memory (a clamped address; columns outside
    // the row are masked below)
    if (lane == 0 || lane == 63) {
      const int cw = min(max(lane == 0 ? col0 - WE : col0 + V, 0), a.w - WE);
#pragma unroll
      for (int kh = 0; kh < KH; ++kh) {
        const int ihc = min(max(ih0 + kh, 0), a.h - 1);
        const unsigned v = *reinterpret_cast<const unsigned*>(xp + (long long)ihc * a.w + cw);
        if (lane == 0) lw[kh] = v;
        else rw[kh] = v;
      }
    }
  } else {  // rows not 16-byte aligned: element loads at clamped addresses
    typedef std::conditional_t<sizeof(T) == 4, unsigned, unsigned short> bits_t;
    const bits_t* xb = reinterpret_cast<const bits_t*>(xp);
#pragma unroll
    for (int kh = 0; kh < KH; ++kh) {
      const long long rb = (long long)min(max(ih0 + kh, 0), a.h - 1) * a.w;
      unsigned e[V + 2 * WE];
#pragma unroll
      for (int i = 0; i < V + 2 * WE; ++i)
        e[i] = xb[rb + min(max(col0 - WE + i, 0), a.w - 1)];
      if constexpr (WE == 1) {
        lw[kh] = e[0];
        for (int k = 0; k < 4; ++k) d[kh][k] = e[1 + k];
        rw[kh] = e[V + 1];
      } else {
        lw[kh] = e[0] | (e[1] << 16);
#pragma unroll
        for (int k = 0; k < 4; ++k) d[kh][k] = e[2 + 2 * k] | (e[3 + 2 * k] << 16);
        rw[kh] = e[V + 2] | (e[V + 3] << 16);
      }
    }
  }

  // columns: real (inside the row) and inside the padded extent
  bool vc[NC], pc[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int iw = col0 + c - PL;
    vc[c] = (unsigned)iw < (unsigned)a.w;
    pc[c] = iw >= -a.pl && iw < a.w + a.pr;
  }
  int rh = 0, ph = 0;
#pragma unroll
  for (int kh = 0; kh < KH; ++kh) {
    rh += rok[kh];
    ph += (ih0 + kh >= -a.pt && ih0 + kh < a.h + a.pb);
  }
  unsigned ob[OPT];  // output bits
  if constexpr (AVG) {
    float cs[NC];  // column sums over the window's rows, in row order
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      cs[c] = 0.0f;
#pragma unroll
      for (int kh = 0; kh < KH; ++kh) {
        const float v = bits_f32<T>(stretch_bits<T>(d[kh], lw[kh], rw[kh], c - PL));
        cs[c] += rok[kh] & vc[c] ? v : 0.0f;
      }
    }
#pragma unroll
    for (int o = 0; o < OPT; ++o) {
      float sum = 0.0f;
      int rwn = 0, pwn = 0;
#pragma unroll
      for (int kw = 0; kw < KW; ++kw) {
        sum += cs[o * SW + kw];
        rwn += vc[o * SW + kw];
        pwn += pc[o * SW + kw];
      }
      const int cnt = a.cip ? ph * pwn : rh * rwn;
      const T r = from_f32<T>(sum / (float)cnt);
      if constexpr (sizeof(T) == 4) ob[o] = __float_as_uint(r);
      else ob[o] = __builtin_bit_cast(unsigned short, r);
    }
  } else if constexpr (sizeof(T) == 2) {
    // 16-bit max, two keys per 32-bit word.  A window with a real tap keeps
    // its max when its taps outside the input repeat one of its real taps:
    // rows outside the input were loaded as the nearest edge row (which the
    // window then contains), and the words past the row's ends are made
    // copies of its edge columns here (the element path loaded them so).
    // Keys are formed without the NaN test: a NaN tap shows in the result as
    // a key above +inf or below -inf, and only then is the output recomputed
    // with NaN taps skipped (the exact rule, rarely taken).
    typedef short s2 __attribute__((ext_vector_type(2)));
    constexpr int NWD = V / 2 + 2;  // words: left, home 0..3, right
    constexpr int KINF = std::is_same_v<T, _Float16> ? 0x7C00 : 0x7F80;
    const bool left_out = j == 0;                 // columns col0 - 2, col0 - 1
    const bool home_out = col0 >= a.w;            // the whole vector past the row
    const bool right_out = col0 + V >= a.w;       // columns col0 + V, col0 + V + 1
    s2 cm[NWD];  // per word, the column maxima over the window's rows (keys)
#pragma unroll
    for (int kh = 0; kh < KH; ++kh) {
      unsigned wd[NWD] = {lw[kh], d[kh][0], d[kh][1], d[kh][2], d[kh][3], rw[kh]};
      if (a.vec) {  // uniform
        const unsigned first = (wd[1] & 0xFFFFu) * 0x10001u;
        const unsigned last = (home_out ? wd[0] >> 16 : wd[4] >> 16) * 0x10001u;
        wd[0] = left_out ? first : wd[0];
#pragma unroll
        for (int q = 1; q < NWD - 1; ++q) wd[q] = home_out ? last : wd[q];
        wd[NWD - 1] = right_out ? last : wd[NWD - 1];
      }
#pragma unroll
      for (int q = 0; q < NWD; ++q) {
        const s2 x = __builtin_bit_cast(s2, wd[q]);
        const s2 k = x ^ ((x >> (short)15) & (short)0x7FFF);
        cm[q] = kh == 0 ? k : (cm[q] > k ? cm[q] : k);
      }
    }
#pragma unroll
    for (int o = 0; o < OPT; ++o) {
      int m = INT_MIN, rwn = 0;
#pragma unroll
      for (int kw = 0; kw < KW; ++kw) {
        const int e = o * SW + kw - PL + 2;  // element of the stretch, from -2
        m = max(m, (int)cm[e >> 1][e & 1]);
        rwn += vc[o * SW + kw];
      }
      const bool real = rh * rwn > 0;
      if (__builtin_expect(real && (m > KINF || m < -KINF - 1), 0)) {
        // a NaN tap: the exact rule over this output's taps
        m = INT_MIN;
#pragma unroll
        for (int kh = 0; kh < KH; ++kh)
#pragma unroll
          for (int kw = 0; kw < KW; ++kw) {
            const int c = o * SW + kw;
            m = max(m, bits_key<T>(stretch_bits<T>(d[kh], lw[kh], rw[kh], c - PL), rok[kh] & vc[c]));
          }
        ob[o] = key_bits<T>(m, true);
      } else {
        ob[o] = real ? (unsigned)(m ^ ((m >> 31) & 0x7FFF)) & 0xFFFFu : key_bits<T>(INT_MIN, false);
      }
    }
  } else {
    int cm[NC];  // column maxima over the window's rows
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      cm[c] = INT_MIN;
#pragma unroll
      for (int kh = 0; kh < KH; ++kh)
        cm[c] = max(cm[c], bits_key<T>(stretch_bits<T>(d[kh], lw[kh], rw[kh], c - PL),
                                       rok[kh] & vc[c]));
    }
#pragma unroll
    for (int o = 0; o < OPT; ++o) {
      int m = INT_MIN, rwn = 0;
#pragma unroll
      for (int kw = 0; kw < KW; ++kw) {
        m = max(m, cm[o * SW + kw]);
        rwn += vc[o * SW + kw];
      }
      ob[o] = key_bits<T>(m, rh * rwn > 0);
    }
  }
  if (!live) return;
  T* __restrict__ yp = static_cast<T*>(a.y) + (long long)row * a.wo + j * OPT;
  if (a.yvec) {  // wo a multiple of OPT and y aligned: one store of OPT outputs
    constexpr int NW = OPT * sizeof(T) / 4;
    typedef unsigned uw __attribute__((ext_vector_type(NW)));
    uw v;
#pragma unroll
    for (int k = 0; k < NW; ++k) v[k] = sizeof(T) == 4 ? ob[k] : ob[2 * k] | (ob[2 * k + 1] << 16);
    __builtin_nontemporal_store(v, reinterpret_cast<uw*>(yp));
  } else {
#pragma unroll
    for (int o = 0; o < OPT; ++o)
      if (j * OPT + o < a.wo) {
        if constexpr (sizeof(T) == 4) yp[o] = __uint_as_float(ob[o]);
        else yp[o] = __builtin_bit_cast(T, (unsigned short)ob[o]);
      }
  }
}

template <typename T, bool AVG>
__global__ __launch_bounds__(256) void pool_direct_kernel(const PoolArgs a) {
  const long long total = (long long)a.planes * a.ho * a.wo;
  const long long o = (long long)blockIdx.x * 256 + threadIdx.x;
  if (o >= total) return;
  const long long plane = o / ((long long)a.ho * a.wo);
  const int rem = (int)(o - plane * a.ho * a.wo);
  const int oh = (int)mdiv((unsigned)rem, a.mg_wo);
  const int ow = rem - oh * a.wo;
  const T* __restrict__ xp = static_cast<const T*>(a.x) + plane * a.h * a.w;
  static_cast<T*>(a.y)[o] = pool_one<T, AVG>(a, oh, ow, [&](int ih, int iw) {
    return to_f32(xp[(long long)ih * a.w + iw]);
  });
}

// Halving tree over `planes` runs of m 32-bit words each, in LDS: float32
// sums (AVG) or max keys.  Level l's pair count divides by mg[l].
template <bool AVG>
__device__ __forceinline__ unsigned tree_op(unsigned x, unsigned y) {
  if constexpr (AVG) return __float_as_uint(__uint_as_float(x) + __uint_as_float(y));
  else return (unsigned)max((int)x, (int)y);
}

template <bool AVG>
__device__ __forceinline__ void tree(unsigned* v, int planes, int stride, int m, const Magic* mg) {
  for (int l = 0; m > 1; ++l) {
    const int half = (m + 1) >> 1, pairs = m - half;
    for (int i = threadIdx.x; i < planes * pairs; i += 256) {
      const int q = (int)mdiv((unsigned)i, mg[l]), j = i - q * pairs;
      unsigned* p = v + q * stride + j;
      p[0] = tree_op<AVG>(p[0], p[half]);
    }
    __syncthreads();
    m = half;
  }
}

// The same tree over one run, by one thread.
template <bool AVG>
__device__ __forceinline__ unsigned tree_serial(unsigned* v, int m) {
  while (m > 1) {
    const int half = (m + 1) >> 1, pairs = m - half;
    for (int j = 0; j < pairs; ++j) v[j] = tree_op<AVG>(v[j], v[j + half]);
    m = half;
  }
  return v[0];
}

// Loads n values at src into LDS words: float32 bits (AVG) or max keys.
template <typename T, bool AVG>
__device__ __forceinline__ void load_run(const T* __restrict__ src, unsigned* dst, int n) {
  constexpr int V = 16 / sizeof(T);
  const bool vec = (reinterpret_cast<uintptr_t>(src) % 16) == 0;  // uniform
  auto put = [&](int i, float f) {
    if constexpr (AVG) dst[i] = __float_as_uint(f);
    else dst[i] = (unsigned)max_key(f);
  };
  if (vec) {
    typedef T tv __attribute__((ext_vector_type(V)));
    for (int i = threadIdx.x; i < n / V; i += 256) {
      const tv v = *reinterpret_cast<const tv*>(src + (long long)i * V);
#pragma unroll
      for (int e = 0; e < V; ++e) put(i * V + e, to_f32(v[e]));
    }
    for (int i = n / V * V + threadIdx.x; i < n; i += 256) put(i, to_f32(src[i]));
  } else {
    for (int i = threadIdx.x; i < n; i += 256) put(i, to_f32(src[i]));
  }
}

template <typename T, bool AVG>
__device__ __forceinline__ T global_result(unsigned v, float inv_hw) {
  if constexpr (AVG) {
    return from_f32<T>(__uint_as_float(v) * inv_hw);
  } else {
    const int k = (int)v;
    return from_f32<T>(k == INT_MIN ? __int_as_float(0x7FC00000) : key_value(k));
  }
}

template <typename T, bool AVG>
__global__ __launch_bounds__(256) void pool_global_kernel(const PoolArgs a) {
  extern __shared__ unsigned gsm[];  // planes_wg * hw words (small planes) or 2 chunks
  const int hw = a.h * a.w;
  const float inv_hw = 1.0f / (float)hw;
  const T* __restrict__ x = static_cast<const T*>(a.x);
  T* __restrict__ y = static_cast<T*>(a.y);
  if (a.chunks == 1) {
    const int p0 = blockIdx.x * a.planes_wg;
    const int np = min(a.planes_wg, a.planes - p0);
    load_run<T, AVG>(x + (long long)p0 * hw, gsm, np * hw);
    __syncthreads();
    tree<AVG>(gsm, np, hw, hw, a.mg_pairs);
    if ((int)threadIdx.x < np) y[p0 + threadIdx.x] = global_result<T, AVG>(gsm[threadIdx.x * hw], inv_hw);
    return;
  }
  unsigned* vals = gsm;
  unsigned* part = gsm + kPoolChunk;
  const long long plane = blockIdx.x;
  for (int c = 0; c < a.chunks; ++c) {
    const int first = c * (int)kPoolChunk;
    const int n = min((int)kPoolChunk, hw - first);
    load_run<T, AVG>(x + plane * hw + first, vals, n);
    __syncthreads();
    if (n == (int)kPoolChunk) {
      tree<AVG>(vals, 1, n, n, a.mg_pairs);
    } else {  // the last, shorter chunk: its own levels
      if (threadIdx.x == 0) tree_serial<AVG>(vals, n);
      __syncthreads();
    }
    if (threadIdx.x == 0) part[c] = vals[0];
    __syncthreads();
  }
  if (threadIdx.x == 0) y[plane] = global_result<T, AVG>(tree_serial<AVG>(part, a.chunks), inv_hw);
}

template <typename T, bool AVG>
void launch_band(const PoolArgs& a, dim3 grid, size_t lds, hipStream_t s) {
  if (a.kh == 3 && a.kw == 3)
    hipLaunchKernelGGL((pool_band_kernel<T, AVG, 3>), grid, dim3(256), lds, s, a);
  else if (a.kh == 2 && a.kw == 2)
    hipLaunchKernelGGL((pool_band_kernel<T, AVG, 2>), grid, dim3(256), lds, s, a);
  else
    hipLaunchKernelGGL((pool_band_kernel<T, AVG, 0>), grid, dim3(256), lds, s, a);
}

// The planner takes the row-vector kernel only where the window's reach
// beyond the thread's vector is at most one word on each side, which is
// exactly the set of instantiations below; anything else is refused.
template <typename T, int KW, int SW, int PL>
constexpr bool rowvec_fits() {
  constexpr int V = 16 / sizeof(T), WE = 4 / sizeof(T);
  return PL <= WE && KW - SW - PL <= WE && V % SW == 0;
}

template <typename T, bool AVG, int KH, int KW, int SW, int PL>
bool launch_rowvec_p(const PoolArgs& a, dim3 grid, hipStream_t s) {
  if constexpr (rowvec_fits<T, KW, SW, PL>()) {
    hipLaunchKernelGGL((pool_rowvec_kernel<T, AVG, KH, KW, SW, PL>), grid, dim3(256), 0, s, a);
    return true;
  }
  return false;
}

template <typename T, bool AVG, int KH, int KW, int SW>
bool launch_rowvec_s(const PoolArgs& a, dim3 grid, hipStream_t s) {
  if (a.pl == 0) return launch_rowvec_p<T, AVG, KH, KW, SW, 0>(a, grid, s);
  if (a.pl == 1) return launch_rowvec_p<T, AVG, KH, KW, SW, 1>(a, grid, s);
  if (a.pl == 2) return launch_rowvec_p<T, AVG, KH, KW, SW, 2>(a, grid, s);
  return false;
}

template <typename T, bool AVG, int KH, int KW>
bool launch_rowvec_k(const PoolArgs& a, dim3 grid, hipStream_t s) {
  if (a.sw == 1) return launch_rowvec_s<T, AVG, KH, KW, 1>(a, grid, s);
  if (a.sw == 2) return launch_rowvec_s<T, AVG, KH, KW, 2>(a, grid, s);
  return false;
}

template <typename T, bool AVG>
bool launch_rowvec(const PoolArgs& a, dim3 grid, hipStream_t s) {
  if (a.kh == 3 && a.kw == 3) return launch_rowvec_k<T, AVG, 3, 3>(a, grid, s);
  if (a.kh == 2 && a.kw == 2) return launch_rowvec_k<T, AVG, 2, 2>(a, grid, s);
  if (a.kh == 3 && a.kw == 2) return launch_rowvec_k<T, AVG, 3, 2>(a, grid, s);
  if (a.kh == 2 && a.kw == 3) return launch_rowvec_k<T, AVG, 2, 3>(a, grid, s);
  return false;
}

template <typename T>
hipError_t launch_pool_t(const PoolGeo& g, const PoolPlan& pl, const PoolArgs& a, hipStream_t s) {
  const bool avg = g.kind == POOL_AVERAGE || g.kind == POOL_GLOBAL_AVERAGE;
  if (pl.variant == POOLV_GLOBAL) {
    const unsigned grid = pl.chunks > 1 ? (unsigned)a.planes
                                        : (unsigned)((a.planes + a.planes_wg - 1) / a.planes_wg);
    const size_t lds = pl.chunks > 1 ? 2 * kPoolChunk * 4 : (size_t)a.planes_wg * g.h * g.w * 4;
    if (avg) hipLaunchKernelGGL((pool_global_kernel<T, true>), dim3(grid), dim3(256), lds, s, a);
    else hipLaunchKernelGGL((pool_global_kernel<T, false>), dim3(grid), dim3(256), lds, s, a);
  } else if (pl.variant == POOLV_ROWVEC) {
    const dim3 grid((unsigned)((a.threads + 255) / 256));
    const bool ok = avg ? launch_rowvec<T, true>(a, grid, s) : launch_rowvec<T, false>(a, grid, s);
    if (!ok) return hipErrorInvalidValue;
  } else if (pl.variant == POOLV_BAND) {
    const dim3 grid((unsigned)((long long)a.planes * a.n_band));
    const size_t lds = (size_t)a.in_rows * a.w * sizeof(float);
    if (avg) launch_band<T, true>(a, grid, lds, s);
    else launch_band<T, false>(a, grid, lds, s);
  } else {
    const long long total = (long long)a.planes * a.ho * a.wo;
    const unsigned grid = (unsigned)((total + 255) / 256);
    if (avg) hipLaunchKernelGGL((pool_direct_kernel<T, true>), dim3(grid), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((pool_direct_kernel<T, false>), dim3(grid), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

}  // namespace convfwd

using namespace convfwd;

extern "C" int pool_forward(const pool_problem* p, int dtype, const void* x, void* y,
                            void* stream) {
  int st = pool_check(p, dtype, x, y);
  if (st) return st;
  PoolGeo g;
  pool_validate(p, dtype, &g);
  PoolPlan pl;
  pool_make_plan(g, &pl);
  const int64_t es = dtype_size(dtype);
  PoolArgs a{};
  a.x = static_cast<const char*>(x) + p->x_off * es;
  a.y = static_cast<char*>(y) + p->y_off * es;
  a.planes = (int)(g.n * g.c);
  a.h = (int)g.h; a.w = (int)g.w; a.ho = (int)g.ho; a.wo = (int)g.wo;
  a.kh = (int)g.kh; a.kw = (int)g.kw; a.sh = (int)g.sh; a.sw = (int)g.sw;
  a.dh = (int)g.dh; a.dw = (int)g.dw;
  a.pt = (int)g.pt; a.pl = (int)g.pl; a.pb = (int)g.pb; a.pr = (int)g.pr;
  a.cip = g.cip;
  a.band_rows = pl.band_rows; a.in_rows = pl.in_rows; a.n_band = pl.n_band;
  a.planes_wg = pl.planes_wg; a.chunks = pl.chunks;
  a.vec = reinterpret_cast<uintptr_t>(a.x) % 16 == 0 && (g.w * es) % 16 == 0;
  a.mg_wo = make_magic((unsigned)g.wo);
  a.mg_w = make_magic((unsigned)g.w);
  if (pl.variant == POOLV_ROWVEC) {
    const int64_t opt = 16 / es / g.sw;
    a.tpr = pl.tpr;
    a.threads = (int)pl.threads;
    a.mg_tpr = make_magic((unsigned)pl.tpr);
    a.mg_ho = make_magic((unsigned)g.ho);
    a.yvec = reinterpret_cast<uintptr_t>(a.y) % (uintptr_t)(opt * es) == 0 && g.wo % opt == 0;
  }
  {  // the tree's levels over a full run (a plane, or a 4096-element chunk)
    int m = (int)(pl.chunks > 1 ? kPoolChunk : g.h * g.w), l = 0;
    while (m > 1 && l < 14) {
      const int half = (m + 1) >> 1;
      a.mg_pairs[l++] = make_magic((unsigned)(m - half));
      m = half;
    }
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (dtype == CONV_F16) e = launch_pool_t<_Float16>(g, pl, a, s);
  else if (dtype == CONV_BF16) e = launch_pool_t<__bf16>(g, pl, a, s);
  else e = launch_pool_t<float>(g, pl, a, s);
  return e == hipSuccess ? CONV_OK : CONV_ERR_DEVICE;
}
