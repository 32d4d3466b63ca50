// ConvInteger, 3x3 stride-1 layers on narrow images (output rows of at most
// 14 columns), gfx950: the row-shift implicit GEMM on v_mfma_i32_32x32x32_i8.
//
// Same operation as the generic ConvInteger kernel ("Convolution, pooling and
// resize", section "ConvInteger"): y = sum over the window of (x - xz) *
// (w - wz[co]) in int32 with wrap-around.  The operands are shifted to signed
// bytes (uint8: top bit flipped), x - xz = xs + a and w - wz = ws + b, and a
// padded tap is staged as the shifted xz, -a, so that its factor is 0:
//
//   y = sum xs*ws + b * Sx + a * Sw + K * a * b        (mod 2^32)
//
// with K = cin/groups * 9, Sx the window's byte sum and Sw the channel's.
//
//  * A workgroup (4 wave64s) owns one image and 32 output channels, as the
//    float16 row-shift kernel does: 32 A rows = two output rows of 16 columns,
//    32 B columns = the 32 channels, k = 32 input channels of one tap per MFMA.
//    The reduction runs in stages of 128 input channels; wave w takes channels
//    32w..32w+31 of every stage and holds the accumulators of all the image's
//    row pairs; the four waves' int32 partial sums are added at the end (exact
//    in any order).
//  * The stage's input is staged channel-innermost in LDS, a 16-byte run of 16
//    channels per position (one A fragment per b128 read); the kw = 1, 2 taps
//    are the kw = 0 fragment moved 1 and 2 lanes inside each 16-lane DPP row.
//    The planes are read as they lie, 4 pixels of 16 channel planes per item
//    (4-byte loads), and transposed in registers with byte permutes.
//  * The stage's weights are copied as they lie (128 channels x 9 taps per
//    output channel, contiguous in OIHW) into padded LDS rows; a lane's 16
//    channels x 9 taps (144 bytes) are read once per stage and regrouped per
//    tap with byte permutes.
//  * Sx: while staging, each lane adds the bytes of its positions over its 16
//    channels (v_dot4 against ones) and keeps the totals over the stages; the
//    positions' totals meet in LDS (integer adds), the padding positions hold
//    cin/groups copies of the staged pad byte, and Sx of an output is the sum
//    of its 3 x 3 window of positions.  Sw: each lane adds the bytes of its B
//    data (one output channel's weights of its channels) over the stages; the
//    lanes' sums meet per channel in LDS.
//  * The MFMA sums stay inside int32 (|xs ws| <= 2^14 and K <= 14563 * 9 is
//    checked by the host), the corrections are uint32 arithmetic, which wraps
//    as the int32 result must.
#include <type_traits>

#include "epilogue.h"
#include "internal.h"

namespace convfwd {

namespace {

typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

constexpr int CR_COLS = 16;                 // tile columns = lanes of a DPP row
constexpr int CR_CH = 128;                  // input channels per stage
constexpr int CR_WROW = CR_CH * 9 + 16;     // LDS bytes per output channel's weights (padded)
constexpr int CR_WBYTES = 32 * CR_WROW;

template <int R>
struct CrLayout {
  static constexpr int NP = R / 2;                   // output row pairs
  static constexpr int TROWS = 2 * NP + 2;           // staged input rows
  static constexpr int NPOS = TROWS * CR_COLS;
  static constexpr int IN_BYTES = NPOS * CR_CH;      // 8 runs of 16 bytes per position
  static constexpr int STAGE = IN_BYTES + CR_WBYTES;
  static constexpr int SINK = 2 * STAGE;             // 16 bytes that dead staging writes hit
  static constexpr int PSUM = SINK + 16;             // NPOS ints: byte sums per position
  static constexpr int SX = PSUM + NPOS * 4;         // R x 16 ints: Sx per output position
  static constexpr int SW = SX + R * CR_COLS * 4;    // 32 ints: Sw per channel
  static constexpr int KB = SW + 32 * 4;             // 32 ints: b per channel
  static constexpr int BASE = KB + 32 * 4;           // 32 ints: a Sw + K a b per channel
  static constexpr int TOTAL = BASE + 32 * 4;
  static constexpr int PITCH = R * CR_COLS + 4;      // ints per channel in a partial-sum copy
  static constexpr int COPY = 32 * PITCH;            // ints per wave's copy
  static constexpr int MAX_GROUPS = 16 * 16 / 8;     // 8-pixel groups of a plane
  static constexpr int NI = (2 * MAX_GROUPS + 63) / 64;  // input items per lane (two runs per wave)
  static constexpr int NW = (32 * 18 + 63) / 64;     // 16-byte weight pieces per lane
  static_assert(4 * COPY * 4 <= SINK, "partial sums do not fit the stage buffers");
  static_assert(TOTAL <= 160 * 1024, "LDS");
};

// slot of run o (0..7) at position p: 16 consecutive positions (128 bytes
// apart) spread over all 64 banks
__device__ __forceinline__ int slot8(int p, int o) { return o ^ ((p >> 1) & 7); }

template <int K>
__device__ __forceinline__ u32x4_t row_shift(u32x4_t v) {
  u32x4_t r;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r[i] = (unsigned)__builtin_amdgcn_mov_dpp((int)v[i], 0x100 + K, 0xF, 0xF, true);
  return r;
}

__device__ __forceinline__ unsigned byte_of(const unsigned* raw, int b) {
  return (raw[b >> 2] >> (8 * (b & 3))) & 0xFFu;
}

// 4x4 byte transpose: out[p] byte k = in[k] byte p
__device__ __forceinline__ void transpose4(const unsigned (&in)[4], unsigned (&out)[4]) {
  // pairs: t0 = (in0.b0, in1.b0, in0.b1, in1.b1), t1 = (in0.b2, in1.b2, in0.b3, in1.b3),
  // likewise t2, t3 from in2, in3; then out0 = (t0.lo16, t2.lo16), ...
  const unsigned t0 = __builtin_amdgcn_perm(in[1], in[0], 0x05010400u);
  const unsigned t1 = __builtin_amdgcn_perm(in[1], in[0], 0x07030602u);
  const unsigned t2 = __builtin_amdgcn_perm(in[3], in[2], 0x05010400u);
  const unsigned t3 = __builtin_amdgcn_perm(in[3], in[2], 0x07030602u);
  out[0] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
  out[1] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
  out[2] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
  out[3] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
}

__device__ __forceinline__ int dot_ones(unsigned v, int acc) {
  return __builtin_amdgcn_sdot4((int)v, 0x01010101, acc, false);
}

// Raw buffer descriptor (gfx9 format word 0x00020000) over [p, p + bytes), its
// operands made wave-uniform so that it lives in scalar registers: a load's
// per-lane part is a 32-bit offset, the stage and plane parts scalar offsets.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* p, int bytes) {
  const unsigned long long v = reinterpret_cast<unsigned long long>(p);
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((unsigned long long)hi << 32) | lo),
                                           (short)0, __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

}  // namespace

template <bool XU, bool WU, int R, bool XV, bool WV>
__global__ __launch_bounds__(256) void convint_rowshift_kernel(const ConvIntRsArgs a) {
  typedef CrLayout<R> L;
  constexpr int NP = L::NP;
  __shared__ __attribute__((aligned(16))) unsigned char smem[L::TOTAL];
  int* psum = reinterpret_cast<int*>(smem + L::PSUM);
  int* sxs = reinterpret_cast<int*>(smem + L::SX);
  int* sws = reinterpret_cast<int*>(smem + L::SW);
  int* kbs = reinterpret_cast<int*>(smem + L::KB);
  int* bases = reinterpret_cast<int*>(smem + L::BASE);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // logical tile: channel tile fastest, so an image's channel tiles share an XCD
  const int bid = xcd_logical(blockIdx.x, gridDim.x);
  const int bq = (int)mdiv((unsigned)bid, a.mg_nct);
  const int ct = bid - bq * a.n_ct;
  const int g = (int)mdiv((unsigned)bq, a.mg_n);
  const int n = bq - g * a.n;
  const int co0 = ct * 32;
  const int hw = a.h * a.w;

  const unsigned char* __restrict__ ximg =
      a.x + ((long long)n * a.c_in + (long long)g * a.cig) * hw;
  const unsigned char* __restrict__ wg = a.wt + (long long)g * a.cog * a.cig * 9;

  // zero points: x - xz = xs + ka with xs the staged byte
  const int xz = a.xzp ? (XU ? (int)a.xzp[0] : (int)(signed char)a.xzp[0]) : 0;
  const unsigned xpad = (unsigned)((XU ? (xz ^ 0x80) : xz) & 0xFF);  // shifted xz
  const int ka = XU ? 128 - xz : -xz;
  const unsigned xflip = XU ? 0x80808080u : 0u, wflip = WU ? 0x80808080u : 0u;

  // ---- staging items of this wave: (one of its two 16-channel runs, 8-pixel
  // group); each covers 16 channel planes x 8 pixels.  A group's first pixel is
  // clamped so that its 8 pixels stay inside the plane (the last group of a
  // plane whose size is not a multiple of 8 overlaps the one before and stores
  // the same bytes again; its byte sums count only the pixels it owns). ----
  static_assert(L::NI == 1, "one input item per lane");
  const int groups8 = (hw + 7) / 8;
  const bool in_live = lane < 2 * groups8;
  const int in_run = 2 * wave + (lane >= groups8 ? 1 : 0);
  const int in_grp = lane - (lane >= groups8 ? groups8 : 0);
  const int in_f0 = max(0, min(8 * in_grp, hw - 8));
  const int in_own = 8 * in_grp;  // first pixel this item owns (sums)
  const int in_off = 16 * in_run * hw + in_f0;
  // weight pieces: (output channel, 16-byte piece of the wave's 32 channels x
  // 9 taps, 288 contiguous bytes of the channel's 1152 in the stage).  Channels
  // past the group's last read its last one: they feed only output channels
  // (and weight sums) that are never used.
  int w_off[L::NW];
  static_assert(L::NW * 64 == 32 * 18, "one piece per lane and vector");
#pragma unroll
  for (int i = 0; i < L::NW; ++i) {
    const unsigned q = (unsigned)(lane + i * 64);
    const unsigned col = __umul24(q, 3641u) >> 16;  // q / 18, exact for q < 576
    w_off[i] = (int)__umul24((unsigned)min(co0 + (int)col, a.cog - 1), (unsigned)(a.cig * 9)) +
               288 * wave + 16 * ((int)q - 18 * (int)col);
  }

  u32x2_t rin[16];          // the next stage's input bytes: [plane], 8 pixels
  u32x4_t rwv[L::NW];
  int pacc[8];              // byte sums of the item's positions over its channels
  int sacc = 0;             // byte sum of this lane's B data (its channel's weights)
#pragma unroll
  for (int k8 = 0; k8 < 8; ++k8) pacc[k8] = 0;
  const int nstages = a.cig / CR_CH;
  const __amdgpu_buffer_rsrc_t x_rsrc = uniform_rsrc(ximg, nstages * CR_CH * hw);
  const __amdgpu_buffer_rsrc_t w_rsrc = uniform_rsrc(wg, a.cog * a.cig * 9);

  auto load_stage = [&](int s) __attribute__((always_inline)) {
    const long long xoff = (long long)s * CR_CH * hw;
    const long long woff = (long long)s * CR_CH * 9;
    if constexpr (WV) {  // 16-byte aligned weights
#pragma unroll
      for (int i = 0; i < L::NW; ++i)
        rwv[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                 w_rsrc, w_off[i], (int)woff, 0));
    } else {
#pragma unroll
      for (int i = 0; i < L::NW; ++i) {
        const unsigned char* src = wg + woff + w_off[i];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          rwv[i][q] = (unsigned)src[4 * q] | ((unsigned)src[4 * q + 1] << 8) |
                      ((unsigned)src[4 * q + 2] << 16) | ((unsigned)src[4 * q + 3] << 24);
      }
    }
    // a dead item's offset is a valid one, so every load is unconditional
    if constexpr (XV) {  // 4-byte aligned planes of at least 8 pixels, a multiple of 4
#pragma unroll
      for (int e = 0; e < 16; ++e)
        rin[e] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(
                                                 x_rsrc, in_off, (int)xoff + e * hw, 0));
    } else {  // byte loads, clamped to the plane's last pixel
      const unsigned char* src = ximg + xoff + in_off;
      const int left = hw - 1 - in_f0;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        unsigned v[2] = {0u, 0u};
#pragma unroll
        for (int k8 = 0; k8 < 8; ++k8)
          v[k8 >> 2] |= (unsigned)src[(long long)e * hw + min(k8, left)] << (8 * (k8 & 3));
        rin[e] = u32x2_t{v[0], v[1]};
      }
    }
  };
  // only the first stage is loaded before anything else is computed
  load_stage(0);
  __builtin_amdgcn_sched_barrier(0);
  // LDS byte address of the item's pixels (position p: (8 p + slot) 16), -1 for
  // none; weight pieces into the output channel's padded row
  int in_lds[8];
#pragma unroll
  for (int k8 = 0; k8 < 8; ++k8) {
    const int f = in_f0 + k8;
    const int ih = (int)mdiv((unsigned)f, a.mg_w), iw = f - ih * a.w;
    const int pos = (ih + a.pt) * CR_COLS + iw + a.pl;
    const bool ok = in_live && f < hw;
    in_lds[k8] = ok ? (pos * 8 + slot8(pos, in_run)) * 16 : -1;
  }
  int w_lds[L::NW];
#pragma unroll
  for (int i = 0; i < L::NW; ++i) {
    const unsigned q = (unsigned)(lane + i * 64);
    const unsigned col = __umul24(q, 3641u) >> 16;
    w_lds[i] = L::IN_BYTES + (int)col * CR_WROW + 288 * wave + 16 * ((int)q - 18 * (int)col);
  }

  // Branch-free: dead items and pixels past the plane write the sink.
  auto store_stage = [&](int buf) __attribute__((always_inline)) {
    unsigned char* base = smem + buf * L::STAGE;
#pragma unroll
    for (int h = 0; h < 2; ++h) {  // pixels 4h .. 4h + 3
      unsigned px[4][4];  // [pixel][word]: 16 channels of each of the 4 pixels
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const unsigned in4[4] = {rin[4 * q][h] ^ xflip, rin[4 * q + 1][h] ^ xflip,
                                 rin[4 * q + 2][h] ^ xflip, rin[4 * q + 3][h] ^ xflip};
        unsigned t4[4];
        transpose4(in4, t4);
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) px[k4][q] = t4[k4];
      }
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) {
        const int k8 = 4 * h + k4;
#pragma unroll
        for (int q = 0; q < 4; ++q) pacc[k8] = dot_ones(px[k4][q], pacc[k8]);
        unsigned char* dst = in_lds[k8] >= 0 ? base + in_lds[k8] : smem + L::SINK;
        *reinterpret_cast<u32x4_t*>(dst) = u32x4_t{px[k4][0], px[k4][1], px[k4][2], px[k4][3]};
      }
    }
#pragma unroll
    for (int i = 0; i < L::NW; ++i) {
      u32x4_t v = rwv[i];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = v[q] ^ wflip;
      *reinterpret_cast<u32x4_t*>(base + w_lds[i]) = v;
    }
  };

  i32x16_t acc[NP];
#pragma unroll
  for (int q = 0; q < NP; ++q)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[q][i] = 0;

  const int grp = lane >> 5;         // k group: channels 16 grp .. 16 grp + 15 of the wave's 32
  const int prow = (lane >> 4) & 1;  // row of the pair this lane's pixel sits in
  const int pcol = lane & 15;
  const int run = 2 * wave + grp;    // 16-channel run of the stage's 128 channels

  auto compute = [&](int buf) __attribute__((always_inline)) {
    const unsigned char* in = smem + buf * L::STAGE;
    // B: this lane's 16 channels x 9 taps (144 contiguous bytes of output channel lane % 32)
    const unsigned char* wb = in + L::IN_BYTES + (lane & 31) * CR_WROW + 288 * wave + 144 * grp;
    unsigned raw[36];
#pragma unroll
    for (int v = 0; v < 9; ++v) {
      const u32x4_t t = *reinterpret_cast<const u32x4_t*>(wb + 16 * v);
      raw[4 * v] = t[0]; raw[4 * v + 1] = t[1]; raw[4 * v + 2] = t[2]; raw[4 * v + 3] = t[3];
    }
    // Sw: each (channel, input channel, tap) of the stage is in exactly one
    // lane's B data, so the lanes' sums add up to the channels' byte sums
#pragma unroll
    for (int v = 0; v < 36; ++v) sacc = dot_ones(raw[v], sacc);
#pragma unroll
    for (int kh = 0; kh < 3; ++kh) {
      u32x4_t bf[3];  // the tap row's three B fragments, regrouped from the raw bytes
#pragma unroll
      for (int kw = 0; kw < 3; ++kw)
#pragma unroll
        for (int q = 0; q < 4; ++q) {  // channels 4q..4q+3 of the run at tap t: bytes c * 9 + t
          const int t = kh * 3 + kw;
          bf[kw][q] = byte_of(raw, (4 * q) * 9 + t) | (byte_of(raw, (4 * q + 1) * 9 + t) << 8) |
                      (byte_of(raw, (4 * q + 2) * 9 + t) << 16) | (byte_of(raw, (4 * q + 3) * 9 + t) << 24);
        }
      u32x4_t fr[NP];  // row pair 2q + kh of every output row pair q
#pragma unroll
      for (int q = 0; q < NP; ++q) {
        const int pos = (2 * q + kh + prow) * CR_COLS + pcol;
        fr[q] = *reinterpret_cast<const u32x4_t*>(in + (pos * 8 + slot8(pos, run)) * 16);
      }
#pragma unroll
      for (int kw = 0; kw < 3; ++kw)
#pragma unroll
        for (int q = 0; q < NP; ++q) {
          const u32x4_t f = kw == 0 ? fr[q] : kw == 1 ? row_shift<1>(fr[q]) : row_shift<2>(fr[q]);
          acc[q] = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4_t, f),
                                                         __builtin_bit_cast(i32x4_t, bf[kw]),
                                                         acc[q], 0, 0, 0);
        }
    }
  };

  // ---- prologue: (the first stage's loads are out) the padding positions of
  // both buffers (the pad byte, never rewritten), the sums' initial values ----
  const unsigned pad4 = xpad * 0x01010101u;
  for (int q = tid; q < 2 * L::NPOS; q += 256) {
    const int st = q / L::NPOS, pos = q - st * L::NPOS;
    const int r = pos / CR_COLS - a.pt, c = pos % CR_COLS - a.pl;
    if (r < 0 || r >= a.h || c < 0 || c >= a.w) {
#pragma unroll
      for (int o = 0; o < 8; ++o)
        *reinterpret_cast<u32x4_t*>(smem + st * L::STAGE + (pos * 8 + o) * 16) =
            u32x4_t{pad4, pad4, pad4, pad4};
    }
  }
  for (int pos = tid; pos < L::NPOS; pos += 256) {
    const int r = pos / CR_COLS - a.pt, c = pos % CR_COLS - a.pl;
    const bool border = r < 0 || r >= a.h || c < 0 || c >= a.w;
    psum[pos] = border ? (int)((unsigned)a.cig * (unsigned)(int)(signed char)xpad) : 0;
  }
  if (tid < 32) sws[tid] = 0;
  __syncthreads();
  store_stage(0);
  // Each wave stages and reads only its own channels: no barrier between stages.
  for (int s = 0; s < nstages; ++s) {
    const bool more = s + 1 < nstages;  // uniform
    if (more) load_stage(s + 1);
    compute(s & 1);
    if (more) store_stage((s + 1) & 1);
  }

  // ---- epilogue ----
  __syncthreads();  // every wave is done with the stage buffers the copies overwrite
  // the byte sums meet in LDS (integer adds: any order)
#pragma unroll
  for (int k8 = 0; k8 < 8; ++k8)
    if (in_lds[k8] >= 0 && in_f0 + k8 >= in_own) atomicAdd(&psum[in_lds[k8] >> 7], pacc[k8]);
  atomicAdd(&sws[lane & 31], sacc);
  // each wave's partial sums as a copy [channel][row][16 columns]: accumulator
  // elements 4 i4 .. 4 i4 + 3 of row pair q are pixels 8 i4 + 4 (l / 32) + 0..3
  // of the pair, 4 consecutive columns of one row
  int* cp = reinterpret_cast<int*>(smem);
  {
    const int co = lane & 31, h4 = 4 * (lane >> 5);
#pragma unroll
    for (int q = 0; q < NP; ++q)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int p = 8 * i4 + h4;
        const int idx = wave * L::COPY + co * L::PITCH + (2 * q + (p >> 4)) * CR_COLS + (p & 15);
        *reinterpret_cast<i32x4_t*>(cp + idx) =
            i32x4_t{acc[q][4 * i4], acc[q][4 * i4 + 1], acc[q][4 * i4 + 2], acc[q][4 * i4 + 3]};
      }
  }
  __syncthreads();
  // Sx per output position (3 x 3 window of position sums), and per channel
  // b and a Sw + K a b
  for (int o = tid; o < R * CR_COLS; o += 256) {
    const int oh = o / CR_COLS, ow = o % CR_COLS;
    int sx = 0;
    if (ow < a.wo && oh < a.ho) {
#pragma unroll
      for (int kh = 0; kh < 3; ++kh)
#pragma unroll
        for (int kw = 0; kw < 3; ++kw) sx += psum[(oh + kh) * CR_COLS + ow + kw];
    }
    sxs[o] = sx;
  }
  if (tid < 32) {
    const int co = g * a.cog + min(co0 + tid, a.cog - 1);
    const int wz = a.wzp ? (WU ? (int)a.wzp[a.wz_per_channel ? co : 0]
                               : (int)(signed char)a.wzp[a.wz_per_channel ? co : 0])
                         : 0;
    const int kb = WU ? 128 - wz : -wz;
    const unsigned K = (unsigned)a.cig * 9u;
    kbs[tid] = kb;
    bases[tid] = (int)((unsigned)ka * (unsigned)sws[tid] + K * (unsigned)ka * (unsigned)kb);
  }
  __syncthreads();

  // ---- outputs: item (channel co, output row oh, column quad), quad fastest,
  // then the row, then the channel; thread t takes items t + 256 k.  An item's
  // four partial-sum vectors and Sx are 16-byte LDS reads at the copy layout's
  // (channel, row, 4 columns); its outputs are 4 consecutive columns of one row
  // of y, stored as int pairs when wo is even (8-byte aligned), else singly. ----
  static_assert(R % 2 == 0, "items per thread");
  constexpr int KI = R / 2;  // 32 x R x 4 items over 256 threads
  const int howo = a.ho * a.wo;
  int* yt = a.y + ((long long)n * a.c_out + (long long)g * a.cog + co0) * howo;
  const i32x4_t* cp4 = reinterpret_cast<const i32x4_t*>(cp);
  const i32x4_t* sx4 = reinterpret_cast<const i32x4_t*>(sxs);
  const bool even = (a.wo & 1) == 0 && (reinterpret_cast<uintptr_t>(a.y) & 7) == 0;  // uniform
  const int quad = tid & 3;            // 256 k % 4 == 0: the same quad for every k
#pragma unroll
  for (int k = 0; k < KI; ++k) {
    const int rest = (tid + 256 * k) >> 2;
    const int co = rest / R, oh = rest - (rest / R) * R;
    const int li = (co * L::PITCH + oh * CR_COLS + 4 * quad) >> 2;  // 16-byte aligned
    const i32x4_t t = cp4[li] + cp4[L::COPY / 4 + li] + cp4[2 * L::COPY / 4 + li] + cp4[3 * L::COPY / 4 + li];
    const i32x4_t sx = sx4[(oh * CR_COLS + 4 * quad) >> 2];
    const unsigned kb = (unsigned)kbs[co], bs = (unsigned)bases[co];
    int v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = (int)((unsigned)t[j] + kb * (unsigned)sx[j] + bs);
    if (co0 + co < a.cog && oh < a.ho) {
      int* dst = yt + co * howo + oh * a.wo + 4 * quad;
      if (even) {
#pragma unroll
        for (int j2 = 0; j2 < 2; ++j2)
          if (4 * quad + 2 * j2 < a.wo)
            __builtin_nontemporal_store(i32x2_t{v[2 * j2], v[2 * j2 + 1]}, reinterpret_cast<i32x2_t*>(dst) + j2);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (4 * quad + j < a.wo) __builtin_nontemporal_store(v[j], dst + j);
      }
    }
  }
}

hipError_t launch_convint_rowshift(const ConvIntRsArgs& a, bool xu, bool wu, hipStream_t s) {
  const dim3 grid((unsigned)((long long)a.n_ct * a.n * a.groups));
#define CR_LAUNCH(XU_, WU_, R_)                                                                          \
  {                                                                                                      \
    if (a.xvec && a.wvec)                                                                                \
      hipLaunchKernelGGL((convint_rowshift_kernel<XU_, WU_, R_, true, true>), grid, dim3(256), 0, s, a);   \
    else if (a.xvec)                                                                                     \
      hipLaunchKernelGGL((convint_rowshift_kernel<XU_, WU_, R_, true, false>), grid, dim3(256), 0, s, a);  \
    else if (a.wvec)                                                                                     \
      hipLaunchKernelGGL((convint_rowshift_kernel<XU_, WU_, R_, false, true>), grid, dim3(256), 0, s, a);  \
    else                                                                                                 \
      hipLaunchKernelGGL((convint_rowshift_kernel<XU_, WU_, R_, false, false>), grid, dim3(256), 0, s, a); \
  }
#define CR_R(XU_, WU_)        \
  {                           \
    if (a.ho <= 8)            \
      CR_LAUNCH(XU_, WU_, 8)  \
    else                      \
      CR_LAUNCH(XU_, WU_, 14) \
  }
  if (a.ho > 14 || a.wo > 14) return hipErrorInvalidValue;
  if (xu && wu) CR_R(true, true)
  else if (xu) CR_R(true, false)
  else if (wu) CR_R(false, true)
  else CR_R(false, false)
#undef CR_R
#undef CR_LAUNCH
  return hipGetLastError();
}

}  // namespace convfwd
