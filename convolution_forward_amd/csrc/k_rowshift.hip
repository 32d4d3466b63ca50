// Implicit-GEMM 3x3 stride-1 convolution for narrow images (output rows of at
// most 14 columns), gfx950, float16 operands, float32 accumulation.
//
// Same operation as the other implicit-GEMM kernels ("Convolution, pooling and
// resize", "Variants": the input window is gathered while the tile is staged, no
// column matrix; the reduction is summed in an order fixed by the shape).  What
// is specific to gfx950 here is how the window is gathered and multiplied:
//
//  * MFMA v_mfma_f32_32x32x16_f16 (the gfx950 instruction with the highest
//    measured f16 rate): 32 A rows = two output rows of 16 columns, 32 B columns
//    = the workgroup's 32 output channels, k = 16 input channels of one tap.
//  * A workgroup (4 wave64s) owns one whole image (R >= Ho output rows, in row
//    pairs) and 32 output channels.  The reduction runs in stages of 64 input
//    channels; wave w takes channels 16w..16w+15 of every stage, holds the
//    accumulators of all the image's row pairs, and the four waves' float32
//    partial sums are added in wave order (((w0 + w1) + w2) + w3) at the end.
//  * The stage's input (every row plus the padding border, 16 columns, 64
//    channels) is staged channel-innermost in LDS: a 16-byte octet of channels per
//    position, so one b128 read gives an A fragment (lane l: 8 channels of pixel
//    l % 32 of a row pair).  A row pair starting at input row t serves tap row kh
//    for output row pair (t - kh) / 2; the kw = 1, 2 taps are the same fragment
//    moved 1 and 2 lanes down inside each 16-lane DPP row (row_shl), which holds
//    one image row: a 14-wide output row plus its 2-column reach fits 16 lanes, so
//    the lanes that shift in zeros only feed output columns >= Wo, never stored.
//  * The stage's weights are copied as they lie (64 channels x 9 taps contiguous
//    per output channel in OIHW) with coalesced 16-byte reads into padded LDS
//    rows; a lane's B data for all 9 taps (8 channels x 9 taps, 144 contiguous
//    bytes) is read once per stage and regrouped per tap in registers.
//  * Input planes are read as they lie: 4 consecutive pixels of 8 channel planes
//    (8 bytes each), regrouped in registers into 4 channel octets.  Tile positions
//    that no pixel maps to (the padding border) are zeroed once.
// Per output the taps of a 16-channel slice are accumulated in (kh, kw) row-major
// order, slices in increasing channel order within each wave.
#include "epilogue.h"
#include "internal.h"

namespace convfwd {

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

constexpr int RS_COLS = 16;                  // tile columns = lanes of a DPP row
constexpr int RS_CH = 64;                    // input channels per stage
constexpr int RS_WROW = RS_CH * 9 * 2 + 16;  // LDS bytes per output channel's weights (padded)
constexpr int RS_WBYTES = 32 * RS_WROW;

template <int R>
struct RsLayout {
  static constexpr int NP = (R + 1) / 2;             // output row pairs
  static constexpr int TROWS = 2 * NP + 2;           // staged input rows
  static constexpr int NPOS = TROWS * RS_COLS;
  static constexpr int IN_BYTES = NPOS * RS_CH * 2;  // 8 octets of 16 bytes per position
  static constexpr int STAGE = IN_BYTES + RS_WBYTES;
  static constexpr int TOTAL = 2 * STAGE;            // double buffer
  static constexpr int MAX_GROUPS = 16 * 16 / 4;     // 4-pixel groups of an input plane
  static constexpr int NI = (8 * MAX_GROUPS + 255) / 256;
  static constexpr int NW = (32 * 72 + 255) / 256;   // 16-byte weight vectors per thread
};

// slot of octet o (0..7) at position p: spreads 16 lanes on 16 consecutive
// positions (128 bytes apart) over all 64 banks
__device__ __forceinline__ int slot8(int p, int o) { return o ^ ((p >> 1) & 7); }

template <int K>
__device__ __forceinline__ u32x4_t row_shift(u32x4_t v) {
  u32x4_t r;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r[i] = (unsigned)__builtin_amdgcn_mov_dpp((int)v[i], 0x100 + K, 0xF, 0xF, true);
  return r;
}

__device__ __forceinline__ floatx16_t mfma32(u32x4_t a, u32x4_t b, floatx16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, a),
                                                __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
}

}  // namespace

template <int R>
__global__ __launch_bounds__(256) void rowshift_kernel(const HaloArgs a) {
  typedef RsLayout<R> L;
  constexpr int NP = L::NP;
  __shared__ __attribute__((aligned(16))) unsigned char smem[L::TOTAL];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  int bid = blockIdx.x;
  const int ct = bid % a.n_ct;
  bid /= a.n_ct;
  const int n = bid % a.n;
  const int g = bid / a.n;
  const int co0 = ct * 32;
  const int hw = a.h * a.w;

  const _Float16* __restrict__ ximg =
      static_cast<const _Float16*>(a.x) + ((long long)n * a.c_in + (long long)g * a.cig) * hw;
  const _Float16* __restrict__ wg =
      static_cast<const _Float16*>(a.wt) + (long long)g * a.cog * a.cig * 9;

  // ---- input staging items: (octet of the stage's 64 channels, 4-pixel group) ----
  const int groups4 = (hw + 3) / 4;
  const int in_items = 8 * groups4;
  int in_off[L::NI];
  int in_lds[L::NI][4];
  bool in_live[L::NI];
#pragma unroll
  for (int i = 0; i < L::NI; ++i) {
    const int q = tid + i * 256;
    in_live[i] = q < in_items;
    const int qq = in_live[i] ? q : 0;
    const int o = qq / groups4;
    const int grp4 = qq - o * groups4;
    in_off[i] = 8 * o * hw + 4 * grp4;
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4) {
      const int f = 4 * grp4 + k4;  // pixels past the plane's end (hw % 4 != 0) are skipped
      const int ih = f / a.w, iw = f - (f / a.w) * a.w;
      const int pos = (ih + a.pt) * RS_COLS + iw + a.pl;
      in_lds[i][k4] = f < hw ? (pos * 8 + slot8(pos, o)) * 16 : -1;
    }
  }
  // ---- weight staging vectors: (output channel, 16-byte piece of its 1152 bytes) ----
  int w_off[L::NW];
  int w_lds[L::NW];
  bool w_ok[L::NW], w_live[L::NW];
#pragma unroll
  for (int i = 0; i < L::NW; ++i) {
    const int q = tid + i * 256;
    w_live[i] = q < 32 * 72;
    const int qq = w_live[i] ? q : 0;
    const int col = qq / 72, piece = qq - (qq / 72) * 72;
    w_ok[i] = w_live[i] && co0 + col < a.cog;
    w_off[i] = w_ok[i] ? (int)((long long)(co0 + col) * a.cig * 9 + piece * 8) : 0;
    w_lds[i] = L::IN_BYTES + col * RS_WROW + piece * 16;
  }

  u32x2_t rin[L::NI][8];  // [item][channel]: 4 pixels
  u32x4_t rwv[L::NW];
  const int nstages = a.cig / RS_CH;

  auto load_stage = [&](int s) {
    const long long xoff = (long long)s * RS_CH * hw;
    const long long woff = (long long)s * RS_CH * 9;
    if (a.xvec) {
#pragma unroll
      for (int i = 0; i < L::NI; ++i) {
        const _Float16* src = ximg + xoff + in_off[i];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          rin[i][e] = *reinterpret_cast<const u32x2_t*>(src + (long long)e * hw);
      }
    } else {  // input not 8-byte aligned or planes not a multiple of 4: element loads
#pragma unroll
      for (int i = 0; i < L::NI; ++i) {
        const _Float16* src = ximg + xoff + in_off[i];
        const int left = hw - 1 - (in_off[i] % hw);  // last valid pixel of this group
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          half4_t h;
#pragma unroll
          for (int k4 = 0; k4 < 4; ++k4) h[k4] = src[(long long)e * hw + min(k4, left)];
          rin[i][e] = __builtin_bit_cast(u32x2_t, h);
        }
      }
    }
    if (a.wvec) {
#pragma unroll
      for (int i = 0; i < L::NW; ++i)
        rwv[i] = *reinterpret_cast<const u32x4_t*>(wg + woff + w_off[i]);
    } else {
#pragma unroll
      for (int i = 0; i < L::NW; ++i) {
        half8_t h;
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = wg[woff + w_off[i] + e];
        rwv[i] = __builtin_bit_cast(u32x4_t, h);
      }
    }
  };

  auto store_stage = [&](int buf) {
    unsigned char* base = smem + buf * L::STAGE;
#pragma unroll
    for (int i = 0; i < L::NI; ++i) {
      if (!in_live[i]) continue;
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) {
        half8_t v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = __builtin_bit_cast(half4_t, rin[i][e])[k4];
        if (in_lds[i][k4] >= 0) *reinterpret_cast<half8_t*>(base + in_lds[i][k4]) = v;
      }
    }
#pragma unroll
    for (int i = 0; i < L::NW; ++i) {
      const u32x4_t v = w_ok[i] ? rwv[i] : u32x4_t{0, 0, 0, 0};
      if (w_live[i]) *reinterpret_cast<u32x4_t*>(base + w_lds[i]) = v;
    }
  };

  floatx16_t acc[NP];
#pragma unroll
  for (int q = 0; q < NP; ++q)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[q][i] = 0.f;

  const int grp = lane >> 5;         // k group: channels 8*grp..8*grp+7 of the wave's slice
  const int prow = (lane >> 4) & 1;  // row of the pair this lane's pixel sits in
  const int pcol = lane & 15;
  const int oct = 2 * wave + grp;    // octet of the stage's 64 channels

  auto compute = [&](int buf) {
    const unsigned char* in = smem + buf * L::STAGE;
    // B: this lane's 8 channels x 9 taps (144 contiguous bytes of output channel lane % 32)
    const unsigned char* wb =
        in + L::IN_BYTES + (lane & 31) * RS_WROW + (16 * wave + 8 * grp) * 18;
    u32x4_t raw[9];
#pragma unroll
    for (int v = 0; v < 9; ++v) raw[v] = *reinterpret_cast<const u32x4_t*>(wb + 16 * v);
    u32x4_t bf[9];
    {
      const _Float16* h = reinterpret_cast<const _Float16*>(raw);
#pragma unroll
      for (int t = 0; t < 9; ++t) {
        half8_t v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = h[e * 9 + t];
        bf[t] = __builtin_bit_cast(u32x4_t, v);
      }
    }
    // A: the row pair starting at input row t feeds output row pair (t - kh) / 2 at tap row kh
#pragma unroll
    for (int t = 0; t < 2 * NP + 1; ++t) {
      const int pos = (t + prow) * RS_COLS + pcol;
      const u32x4_t f0 = *reinterpret_cast<const u32x4_t*>(in + (pos * 8 + slot8(pos, oct)) * 16);
      const u32x4_t f1 = row_shift<1>(f0);
      const u32x4_t f2 = row_shift<2>(f0);
#pragma unroll
      for (int kh = 0; kh < 3; ++kh) {
        if ((t - kh) < 0 || ((t - kh) & 1)) continue;  // compile-time
        const int q = (t - kh) >> 1;
        if (q >= NP) continue;
        acc[q] = mfma32(f0, bf[kh * 3 + 0], acc[q]);
        acc[q] = mfma32(f1, bf[kh * 3 + 1], acc[q]);
        acc[q] = mfma32(f2, bf[kh * 3 + 2], acc[q]);
      }
    }
  };

  // zero both stages' input regions once: padding positions are never written
  for (int q = tid; q < 2 * (L::IN_BYTES / 16); q += 256) {
    const int st = q / (L::IN_BYTES / 16), off = q - st * (L::IN_BYTES / 16);
    *reinterpret_cast<u32x4_t*>(smem + st * L::STAGE + off * 16) = u32x4_t{0, 0, 0, 0};
  }
  __syncthreads();
  load_stage(0);
  store_stage(0);
  __syncthreads();
  for (int s = 0; s < nstages; ++s) {
    const bool more = s + 1 < nstages;
    load_stage(more ? s + 1 : s);  // the last iteration re-reads harmlessly
    compute(s & 1);
    if (more) store_stage((s + 1) & 1);
    __syncthreads();
  }

  // ---- the four waves' partial sums, added in wave order per row pair ----
  floatx16_t* red = reinterpret_cast<floatx16_t*>(smem);  // [wave][NP][64 lanes]
#pragma unroll
  for (int q = 0; q < NP; ++q) red[(wave * NP + q) * 64 + lane] = acc[q];
  __syncthreads();

  const _Float16* bias = static_cast<const _Float16*>(a.bias);
  const _Float16* res = static_cast<const _Float16*>(a.res);
  _Float16* y = static_cast<_Float16*>(a.y);
  const int col_l = co0 + (lane & 31);
  const int co = g * a.cog + col_l;
  const long long hw_out = (long long)a.ho * a.wo;
  const long long ybase = ((long long)n * a.c_out + co) * hw_out;
  for (int q = wave; q < NP; q += 4) {
    floatx16_t v = red[q * 64 + lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      const floatx16_t o = red[(w * NP + q) * 64 + lane];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = v[i] + o[i];
    }
    if (col_l >= a.cog) continue;
    // Residuals are read for the whole tile before any store: y may alias the
    // residual exactly, and each element is read and written by this lane only,
    // so hoisting the reads keeps the result and lets them overlap.
    long long oidx[16];
    bool ok[16];
    float rv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int p = 8 * (i / 4) + 4 * (lane >> 5) + (i % 4);  // pixel of the row pair
      const int oh = 2 * q + p / 16, ow = p % 16;
      ok[i] = oh < a.ho && ow < a.wo;
      oidx[i] = ybase + (long long)(ok[i] ? oh : 0) * a.wo + (ok[i] ? ow : 0);
      rv[i] = (res && ok[i]) ? (float)res[oidx[i]] : 0.f;
    }
    const float bv = bias ? (float)bias[co] : 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (!ok[i]) continue;
      float v2 = v[i];
      if (bias) v2 = v2 + bv;
      if (res) v2 = v2 + rv[i];
      y[oidx[i]] = (_Float16)apply_act(v2, a.act, a.alpha, a.beta);
    }
  }
}

hipError_t launch_rowshift(const HaloArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((long long)a.n_ct * a.n * a.groups));
  if (a.ho <= 8)
    hipLaunchKernelGGL(rowshift_kernel<8>, grid, dim3(256), 0, s, a);
  else if (a.ho <= 14)
    hipLaunchKernelGGL(rowshift_kernel<14>, grid, dim3(256), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace convfwd
