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
//    The MFMAs run taps outermost and row pairs innermost, so back-to-back MFMAs
//    accumulate into different row pairs.
//  * The stage's weights are copied as they lie (64 channels x 9 taps contiguous
//    per output channel in OIHW) with coalesced 16-byte reads into padded LDS
//    rows; a lane's B data for all 9 taps (8 channels x 9 taps, 144 contiguous
//    bytes) is read once per stage and regrouped per tap in registers.
//  * Input planes are read as they lie: 4 consecutive pixels of 8 channel planes
//    (8 bytes each), regrouped in registers into 4 channel octets.  Tile positions
//    that no pixel maps to (the padding border) are zeroed once.
//  * Pipeline: only the first stage is loaded before the multiplications start;
//    afterwards every tap row's MFMAs carry a third of the global loads of the
//    stage two ahead and a third of the LDS stores of the next stage, so a load
//    whose issue stalls (memory pipeline full) leaves the matrix unit busy.
//  * Epilogue: the waves' partial sums meet in LDS.  When y and the residual are
//    16-byte aligned at every 32-channel tile, the copies are laid out like y
//    and each thread finishes 8 consecutive outputs with one 16-byte residual
//    load and one 16-byte store; otherwise 4 outputs of one row per item.
// Per output the taps of a 16-channel slice are accumulated in (kh, kw) row-major
// order, slices in increasing channel order within each wave.
#include <type_traits>

#include "epilogue.h"
#include "internal.h"

namespace convfwd {

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
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
  static constexpr int SINK = 2 * STAGE;             // 16 bytes that dead staging writes hit
  static constexpr int BIAS = 2 * STAGE + 16;        // 32 bias floats
  static constexpr int TOTAL = BIAS + 32 * 4;         // double buffer + sink + bias
  static constexpr int MAX_GROUPS = 16 * 16 / 8;     // 8-pixel groups of an input plane
  static constexpr int NI = (2 * MAX_GROUPS + 63) / 64;  // input items per lane (two octets per wave)
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

// Raw buffer descriptor (gfx9 format word 0x00020000) over [p, p + bytes); the
// operands are made wave-uniform so the descriptor lives in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* p, int bytes) {
  const unsigned long long v = reinterpret_cast<unsigned long long>(p);
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((unsigned long long)hi << 32) | lo),
                                           (short)0, __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// v_mfma_f32_32x32x16_f16 or _bf16: the operands are the same 16 bytes.
template <typename E>
__device__ __forceinline__ floatx16_t mfma32(u32x4_t a, u32x4_t b, floatx16_t c) {
  typedef E e8 __attribute__((ext_vector_type(8)));
  if constexpr (std::is_same_v<E, __bf16>)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(e8, a),
                                                   __builtin_bit_cast(e8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(e8, a),
                                                  __builtin_bit_cast(e8, b), c, 0, 0, 0);
}

}  // namespace

// RAW: split k.  Workgroup range r multiplies stages [r sps, (r + 1) sps) and
// writes its float32 sums (no bias, residual or activation) to plane r of the
// scratch; the reduce kernel adds the planes in range order and finishes.
// NS: the number of 64-channel stages when it is 1..4, at least 5 when NS = 5,
// any (read from the arguments) when NS = -1.  With the count known the
// prologue and the last steps have no branches on it, so the wait before each
// LDS store counts exactly the loads issued after its data (a branch around a
// group of loads makes the compiler wait for every load at the join).
template <typename E, int R, bool XV, bool WV, int AK = -1, bool RAW = false, int NS = -1>
__global__ __launch_bounds__(256) void rowshift_kernel(const HaloArgs a) {
  typedef E half8_t __attribute__((ext_vector_type(8)));
  typedef E half4_t __attribute__((ext_vector_type(4)));
  typedef E half2_t __attribute__((ext_vector_type(2)));

  typedef RsLayout<R> L;
  constexpr int NP = L::NP;
  // the epilogue's partial sums (4 waves x NP row pairs x 16 floats x 64 lanes)
  // reuse the two stage buffers
  static_assert(4 * NP * 16 * 64 * 4 <= L::SINK, "epilogue does not fit");
  static_assert(4 * 32 * R * (RS_COLS - 2) * 4 <= L::SINK, "flat epilogue does not fit");
  __shared__ __attribute__((aligned(16))) unsigned char smem[L::TOTAL];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // logical tile: co tile fastest, so an image's co tiles run on one XCD
  // (divisions by the host's multiply-shift constants: the tile's first loads
  // wait on this index arithmetic)
  const int bid = xcd_logical(blockIdx.x, gridDim.x);
  const int bq2 = (int)mdiv((unsigned)bid, a.mg_nct);
  const int ct = bid - bq2 * a.n_ct;
  int r = 0, bq = bq2;  // split range (slowest), then (group, image)
  if constexpr (RAW) {
    r = (int)mdiv((unsigned)bq2, a.mg_ng);
    bq = bq2 - r * a.n * a.groups;
  }
  const int g = (int)mdiv((unsigned)bq, a.mg_n);
  const int n = bq - g * a.n;
  const int co0 = ct * 32;
  const int hw = a.h * a.w;
  const int ch0 = RAW ? r * a.sps * RS_CH : 0;  // first input channel of the range

  const E* __restrict__ ximg =
      static_cast<const E*>(a.x) + ((long long)n * a.c_in + (long long)g * a.cig + ch0) * hw;
  const E* __restrict__ wg =
      static_cast<const E*>(a.wt) + (long long)g * a.cog * a.cig * 9 + (long long)ch0 * 9;

  // ---- each wave stages only its own 16 channels of every stage (octets
  // 2 wave, 2 wave + 1) and its own 16-channel slice of the weights, which are
  // all its multiplications read: the waves need no barrier between stages and
  // drift freely, one's loads overlapping another's multiplications.  Only the
  // global offsets are computed before the first stage's loads go out; the LDS
  // positions follow while those loads fly (at one wave per SIMD every
  // instruction ahead of the first load delays the whole tile). ----
  // input staging items: (one of the wave's two octets, 8-pixel group); a
  // group's first pixel is clamped so that its 8 pixels stay inside the plane
  // (the last group of a plane whose size is not a multiple of 8 overlaps the
  // one before and stores the same values again)
  static_assert(L::NI == 1, "one input item per lane");
  const int groups8 = (hw + 7) / 8;
  const bool in_live = lane < 2 * groups8;
  const int in_oct = 2 * wave + (lane >= groups8 ? 1 : 0);
  const int in_f0 = max(0, min(8 * (lane - (lane >= groups8 ? groups8 : 0)), hw - 8));
  const int in_off = 8 * in_oct * hw + in_f0;
  // weight staging vectors: (output channel, 16-byte piece of the wave's 16
  // channels x 9 taps, 288 contiguous bytes of the channel's 1152).  Channels
  // past the group's last read its last one: their sums feed only output
  // channels that are never stored.
  int w_off[L::NW];
  static_assert(L::NW * 64 == 32 * 18, "one weight vector per lane and step");
#pragma unroll
  for (int i = 0; i < L::NW; ++i) {
    const unsigned q = (unsigned)(lane + i * 64);
    const unsigned col = __umul24(q, 3641u) >> 16;  // q / 18, exact for q < 576
    w_off[i] = (int)__umul24((unsigned)min(co0 + (int)col, a.cog - 1), (unsigned)(a.cig * 9)) +
               144 * wave + 8 * ((int)q - 18 * (int)col);
  }

  u32x4_t rin[2][8];  // two staged stages in flight: [set][channel], 8 pixels
  u32x4_t rwv[2][L::NW];
  const int nstages = NS >= 1 && NS <= 4 ? NS : RAW ? a.sps : a.cig / RS_CH;
  if constexpr (NS == 5) __builtin_assume(nstages >= 5);

  // the loads of one stage in three parts (part 0 and 1: the input's channels
  // 0-3 and 4-7 of the octet, part 2: the weights), so that each tap row's
  // multiplications can carry one part
  // buffer descriptors over the image's group of planes and the group's
  // weights: the per-lane part of every address is a 32-bit item offset and the
  // stage and plane parts are scalar offsets, so the loads need no vector
  // address arithmetic between the multiplications they are issued with
  const __amdgpu_buffer_rsrc_t x_rsrc = uniform_rsrc(ximg, nstages * RS_CH * hw * 2);
  const __amdgpu_buffer_rsrc_t w_rsrc = uniform_rsrc(wg, (a.cog * a.cig - ch0) * 9 * 2);
  auto load_part = [&](int s, int set, int part) __attribute__((always_inline)) {
    const long long xoff = (long long)s * RS_CH * hw;
    const long long woff = (long long)s * RS_CH * 9;
    const int e0 = part == 1 ? 4 : 0;
    if (part == 2) {
      if constexpr (WV) {  // 16-byte aligned weights
#pragma unroll
        for (int i = 0; i < L::NW; ++i)
          rwv[set][i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                        w_rsrc, 2 * w_off[i], 2 * (int)woff, 0));
      } else {
#pragma unroll
        for (int i = 0; i < L::NW; ++i) {
          half8_t h;
#pragma unroll
          for (int e = 0; e < 8; ++e) h[e] = wg[woff + w_off[i] + e];
          rwv[set][i] = __builtin_bit_cast(u32x4_t, h);
        }
      }
    } else if constexpr (XV) {  // 8-byte aligned planes of at least 8 pixels, a multiple of 4
#pragma unroll
      for (int e = e0; e < e0 + 4; ++e)
        rin[set][e] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                      x_rsrc, 2 * in_off, 2 * (int)(xoff + e * hw), 0));
    } else {  // input not 8-byte aligned, or planes not a multiple of 4 or below 8: element loads
      const E* src = ximg + xoff + in_off;
      const int left = hw - 1 - in_f0;  // last valid pixel of this group
#pragma unroll
      for (int e = e0; e < e0 + 4; ++e) {
        half8_t h;
#pragma unroll
        for (int k8 = 0; k8 < 8; ++k8) h[k8] = src[(long long)e * hw + min(k8, left)];
        rin[set][e] = __builtin_bit_cast(u32x4_t, h);
      }
    }
  };
  auto load_stage = [&](int s, int set) __attribute__((always_inline)) {
    load_part(s, set, 0);
    load_part(s, set, 1);
    load_part(s, set, 2);
  };
  // only stage 0 is loaded before the first multiplications: stages 1 and 2
  // are issued with stage 0's multiplications, so that the multiplications
  // start as soon as the first stage has arrived
  load_stage(0, 0);
  // the tile's biases (any valid address without bias), kept in LDS for the
  // epilogue
  const E* __restrict__ bias = static_cast<const E*>(a.bias);
  const E b_in = *(bias ? bias + g * a.cog + min(co0 + (tid & 31), a.cog - 1) : ximg);
  __builtin_amdgcn_sched_barrier(0);

  // LDS positions of the staging items: input octets channel-innermost at
  // their padded tile position (pixels past the plane's end, hw % 4 != 0, go
  // nowhere), weight vectors into the output channel's padded row
  int in_lds[8];
#pragma unroll
  for (int k8 = 0; k8 < 8; ++k8) {
    const int f = in_f0 + k8;
    const int ih = (int)mdiv((unsigned)f, a.mg_w), iw = f - ih * a.w;
    const int pos = (ih + a.pt) * RS_COLS + iw + a.pl;
    in_lds[k8] = f < hw ? (pos * 8 + slot8(pos, in_oct)) * 16 : -1;
  }
  int w_lds[L::NW];
#pragma unroll
  for (int i = 0; i < L::NW; ++i) {
    const unsigned q = (unsigned)(lane + i * 64);
    const unsigned col = __umul24(q, 3641u) >> 16;
    w_lds[i] = L::IN_BYTES + (int)col * RS_WROW + 288 * wave + 16 * ((int)q - 18 * (int)col);
  }

  // Branch-free: dead items and pixels past the plane write the sink, so no
  // store sits behind a branch (which would make the compiler wait for every
  // outstanding load there, including the stage just prefetched).
  auto store_part = [&](int buf, int set, int part) __attribute__((always_inline)) {
    unsigned char* base = smem + buf * L::STAGE;
    if (part < 2) {  // pixels 0-3 or 4-7 of the group: all 8 channels of the octet
      const int k0 = part == 1 ? 4 : 0;
#pragma unroll
      for (int k8 = k0; k8 < k0 + 4; ++k8) {
        half8_t v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = __builtin_bit_cast(half8_t, rin[set][e])[k8];
        const bool live = in_live && in_lds[k8] >= 0;
        unsigned char* dst = live ? base + in_lds[k8] : smem + L::SINK;
        *reinterpret_cast<half8_t*>(dst) = v;
      }
    }
    if (part == 2) {
#pragma unroll
      for (int i = 0; i < L::NW; ++i) {
        *reinterpret_cast<u32x4_t*>(base + w_lds[i]) = rwv[set][i];
      }
    }
  };
  auto store_stage = [&](int buf, int set) __attribute__((always_inline)) {
    store_part(buf, set, 0);
    store_part(buf, set, 1);
    store_part(buf, set, 2);
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

  // hook(kh): issued with tap row kh's multiplications (the next stages' loads
  // and stores)
  auto compute = [&](int buf, auto hook) __attribute__((always_inline)) {
    const unsigned char* in = smem + buf * L::STAGE;
    // B: this lane's 8 channels x 9 taps (144 contiguous bytes of output channel lane % 32)
    const unsigned char* wb =
        in + L::IN_BYTES + (lane & 31) * RS_WROW + (16 * wave + 8 * grp) * 18;
    u32x4_t raw[9];
#pragma unroll
    for (int v = 0; v < 9; ++v) raw[v] = *reinterpret_cast<const u32x4_t*>(wb + 16 * v);
    u32x4_t bf[9];
#pragma unroll
    for (int t = 0; t < 9; ++t) {
      half8_t v;
#pragma unroll
      for (int e = 0; e < 8; ++e)  // element e*9+t of the 72 halves (compile-time index)
        v[e] = __builtin_bit_cast(half8_t, raw[(e * 9 + t) / 8])[(e * 9 + t) % 8];
      bf[t] = __builtin_bit_cast(u32x4_t, v);
    }
    // A: the row pair starting at input row t; output row pair q takes it at
    // tap row kh = t - 2q.  Taps outermost, row pairs innermost: consecutive
    // MFMAs go to NP different accumulators, so none waits for its previous
    // result, and every output still sees its taps in (kh, kw) row-major order.
#pragma unroll
    for (int kh = 0; kh < 3; ++kh) {
      u32x4_t fr[NP];  // row pair 2q + kh of every output row pair q
#pragma unroll
      for (int q = 0; q < NP; ++q) {
        const int pos = (2 * q + kh + prow) * RS_COLS + pcol;
        fr[q] = *reinterpret_cast<const u32x4_t*>(in + (pos * 8 + slot8(pos, oct)) * 16);
      }
      hook(kh);
#pragma unroll
      for (int kw = 0; kw < 3; ++kw)
#pragma unroll
        for (int q = 0; q < NP; ++q) {
          const u32x4_t f = kw == 0 ? fr[q] : kw == 1 ? row_shift<1>(fr[q]) : row_shift<2>(fr[q]);
          acc[q] = mfma32<E>(f, bf[kh * 3 + kw], acc[q]);
        }
      // the loads go out between the multiplications: a load whose issue
      // stalls (memory pipeline full) then leaves the matrix unit busy
#pragma unroll
      for (int j = 0; j < 9; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // 2 MFMA
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // 1 VMEM read
        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // 1 DS write
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 3 * NP - 18, 0);
      __builtin_amdgcn_sched_barrier(0);  // one tap row's fragments live at a time
    }
  };
  auto no_hook = [](int) __attribute__((always_inline)) {};

  // ---- epilogue items: item it = (channel co, output row oh, column quad) with
  // the quad fastest, then the row (R rows), then the channel; thread t takes
  // items t + 256 k, k < R / 2.  An item's outputs are columns 4 quad .. 4 quad + 3
  // of one output row: consecutive lanes cover consecutive 8-byte pieces of y. ----
  static_assert(R % 2 == 0, "items per thread");
  constexpr int KI = R / 2;  // 32 x R x 4 items over 256 threads
  const int howo = a.ho * a.wo;
  const long long obase = ((long long)n * a.c_out + g * a.cog + co0) * howo;
  const E* res = static_cast<const E*>(a.res);
  float* bsm = reinterpret_cast<float*>(smem + L::BIAS);  // the tile's 32 biases
  const bool pairs = !RAW && a.o2;  // y / residual 4-byte aligned, wo even (uniform)
  auto it_co = [&](int k) __attribute__((always_inline)) { return ((tid + 256 * k) >> 2) / R; };
  auto it_oh = [&](int k) __attribute__((always_inline)) { return ((tid + 256 * k) >> 2) % R; };
  const int it_ow = 4 * (tid & 3);  // 256 k % 4 == 0: the same quad for every k
  auto e_index = [&](int k, int j) __attribute__((always_inline)) {  // flat index in the tile
    return it_co(k) * howo + it_oh(k) * a.wo + it_ow + j;
  };
  auto e_valid = [&](int k, int j) __attribute__((always_inline)) {
    return co0 + it_co(k) < a.cog && it_oh(k) < a.ho && it_ow + j < a.wo;
  };
  // the nearest output (pair: back = 2) inside the tile, by clamped
  // coordinates: loads of items past the tile stay unconditional and in bounds
  // (24-bit products: small operands, and no 64-bit multiply-add whose unused
  // high half could land on a register still being loaded)
  auto e_clamped = [&](int k, int j, int back) __attribute__((always_inline)) {
    return (int)(__umul24((unsigned)min(it_co(k), a.cog - 1 - co0), (unsigned)howo) +
                 __umul24((unsigned)min(it_oh(k), a.ho - 1), (unsigned)a.wo)) +
           min(it_ow + j, a.wo - back);
  };
  // flat path: the tile's outputs (its channels' planes, contiguous in y) as
  // vectors of 8; thread t takes vectors t + 256 k, k < KV, clamped to the last
  constexpr int KV = (32 * R * (RS_COLS - 2) / 8 + 255) / 256;
  const bool flat = !RAW && a.oflat;  // uniform
  const int ftot = min(32, a.cog - co0) * howo;  // a multiple of 8 on the flat path
  const int nvec = ftot >> 3;
  u32x4_t rv[KV];  // the residual (flat path), prefetched during the last step
  auto load_epilogue_operands = [&]() __attribute__((always_inline)) {
    if (res && flat) {  // uniform
      const __amdgpu_buffer_rsrc_t rr = uniform_rsrc(res + obase, ftot * 2);
#pragma unroll
      for (int k = 0; k < KV; ++k)
        rv[k] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                rr, 16 * min(tid + 256 * k, nvec - 1), 0, 0));
    }
  };

  // Prefetch distance 2: loads for stage s+2 are issued while stage s multiplies
  // and reach LDS one step later, after stage s+1 has multiplied.  Register set
  // and LDS buffer follow the stage's parity, fixed at compile time in a loop
  // unrolled by two; the last steps load (M = 1) or also store (M = 2) nothing.
  auto step = [&](int s, auto parity, auto mode) __attribute__((always_inline)) {
    constexpr int P = decltype(parity)::value;
    constexpr int M = decltype(mode)::value;
    if constexpr (M == 2) load_epilogue_operands();  // bias and residual
    // the scheduler must not hoist the regrouping of set P^1 into the
    // multiplications (which waits for that set early)
    __builtin_amdgcn_sched_barrier(0);
    // buffer P holds stage s; stage s+2 is loaded into set P (stored last
    // step) and stage s+1 (set P^1) is stored into buffer P^1, a third of each
    // with every tap row
    if constexpr (M == 0)
      compute(P, [&](int kh) __attribute__((always_inline)) {
        load_part(s + 2, P, kh);
        store_part(P ^ 1, P ^ 1, kh);
      });
    else if constexpr (M == 1)
      compute(P, [&](int kh) __attribute__((always_inline)) { store_part(P ^ 1, P ^ 1, kh); });
    else
      compute(P, no_hook);
    __builtin_amdgcn_sched_barrier(0);
    // no barrier: the wave's next multiplications read only what it stored
  };
  typedef std::integral_constant<int, 0> P0;
  typedef std::integral_constant<int, 1> P1;
  typedef std::integral_constant<int, 0> LOAD;
  typedef std::integral_constant<int, 1> STORE_ONLY;
  typedef std::integral_constant<int, 2> LAST;
  // zero the padding positions of both stages' input regions (rows and
  // columns outside the image) while the first loads fly: staging writes only
  // image positions, so these stay zero
  for (int q = tid; q < 2 * L::NPOS; q += 256) {
    const int st = q / L::NPOS, pos = q - st * L::NPOS;
    const int r = pos / RS_COLS - a.pt, c = pos % RS_COLS - a.pl;
    if (r < 0 || r >= a.h || c < 0 || c >= a.w) {
#pragma unroll
      for (int o = 0; o < 8; ++o)
        *reinterpret_cast<u32x4_t*>(smem + st * L::STAGE + (pos * 8 + o) * 16) = u32x4_t{0, 0, 0, 0};
    }
  }
  __syncthreads();
  store_stage(0, 0);
  // without a bias the slot holds -0.0, whose addition is exact for every
  // value (a zero keeps its sign), so the epilogue adds it unconditionally
  if (tid < 32) bsm[tid] = bias ? (float)b_in : -0.0f;
  __syncthreads();
  // step 0: stage 1 into set 1 with the multiplications, then stage 2 into
  // set 0, then stage 1 into buffer 1; stages that do not exist are not
  // loaded (the kernel cannot end before every load it issued has returned)
  __builtin_amdgcn_sched_barrier(0);
  if (nstages == 1) {  // uniform
    load_epilogue_operands();
    compute(0, no_hook);
  } else if constexpr (NS >= 3) {
    compute(0, [&](int kh) __attribute__((always_inline)) {
      if (kh == 0) { load_part(1, 1, 0); load_part(1, 1, 1); }
      else if (kh == 1) { load_part(1, 1, 2); load_part(2, 0, 0); }
      else { load_part(2, 0, 1); load_part(2, 0, 2); }
    });
  } else {
    compute(0, [&](int kh) __attribute__((always_inline)) { load_part(1, 1, kh); });
  }
  __builtin_amdgcn_sched_barrier(0);
  if (NS < 3 && nstages > 2) load_stage(2, 0);
  if (nstages > 1) store_stage(1, 1);
  int s = 1;
  for (; s + 3 < nstages; s += 2) {  // both steps prefetch a stage
    step(s, P1{}, LOAD{});
    step(s + 1, P0{}, LOAD{});
  }
  if (nstages - s == 3) {
    step(s, P1{}, LOAD{});
    step(s + 1, P0{}, STORE_ONLY{});
    step(s + 2, P1{}, LAST{});
  } else if (nstages - s == 2) {
    step(s, P1{}, STORE_ONLY{});
    step(s + 1, P0{}, LAST{});
  } else if (nstages - s == 1) {
    step(s, P1{}, LAST{});
  }

  typedef float floatx4_t __attribute__((ext_vector_type(4)));
  if (flat) {
    // ---- flat epilogue (y and residual 16-byte aligned at the tile, wo even,
    // planes of at least 8 outputs): wave w writes its partial sums as float
    // pairs into its own float32 copy of the tile, laid out like y (channel
    // planes of Ho x Wo); each thread then takes 8 consecutive outputs (at most
    // two channels), adds the four waves' partials in wave order
    // (((w0 + w1) + w2) + w3), the bias and the residual, applies the
    // activation and writes 16 bytes. ----
    typedef float floatx2_t __attribute__((ext_vector_type(2)));
    float* ft = reinterpret_cast<float*>(smem);
    const int FT = 32 * howo;  // floats per wave copy
    const int fco = lane & 31, fh = lane >> 5;
    __syncthreads();  // every wave is done with the stage buffers the copies overwrite
#pragma unroll
    for (int q = 0; q < NP; ++q)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
#pragma unroll
        for (int j2 = 0; j2 < 2; ++j2) {
          const int p = 8 * i4 + 4 * fh + 2 * j2;  // pixel of the row pair (accumulator element 4 i4 + 2 j2)
          const int row = 2 * q + (p >> 4), col = p & 15;
          const bool ok = row < a.ho && col < a.wo;  // wo even: the pair is whole
          float* dst = ok ? ft + wave * FT + fco * howo + row * a.wo + col : reinterpret_cast<float*>(smem + L::SINK);
          *reinterpret_cast<floatx2_t*>(dst) = floatx2_t{acc[q][4 * i4 + 2 * j2], acc[q][4 * i4 + 2 * j2 + 1]};
        }
    __syncthreads();
    E* yt = static_cast<E*>(a.y) + obase;
    const float rhowo = 1.0f / (float)howo;
#pragma unroll
    for (int k = 0; k < KV; ++k) {
      // vectors past the tile repeat the last one (same value, same address):
      // the store count is fixed
      const int e0 = 8 * min(tid + 256 * k, nvec - 1);
      const floatx4_t* src = reinterpret_cast<const floatx4_t*>(ft + e0);
      floatx4_t lo = src[0] + src[FT / 4], hi = src[1] + src[FT / 4 + 1];
      lo = lo + src[FT / 2];
      hi = hi + src[FT / 2 + 1];
      lo = lo + src[3 * FT / 4];
      hi = hi + src[3 * FT / 4 + 1];
      // channel of the first output, and the start of the next: (e0 + 1/2) / howo
      // lies at least 1 / (2 howo) from an integer, far beyond the float error
      // for tiles of at most 32 x 14 x 14 outputs, so the truncation is exact
      const int c0 = (int)(((float)e0 + 0.5f) * rhowo), cb = (c0 + 1) * howo;
      const float b0 = bsm[c0], b1 = bsm[min(c0 + 1, 31)];
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float t = j < 4 ? lo[j] : hi[j - 4];
        const float bv = e0 + j < cb ? b0 : b1;
        v[j] = t + bv;
      }
      if (res) {
        const half8_t r8 = __builtin_bit_cast(half8_t, rv[k]);
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = v[j] + (float)r8[j];
      }
      act_apply<AK>(v, a.act, a.alpha, a.beta);
      half8_t h;
#pragma unroll
      for (int j = 0; j < 8; ++j) h[j] = (E)v[j];
      *reinterpret_cast<half8_t*>(yt + e0) = h;
    }
    return;
  }

  // ---- the four waves' partial sums are added through LDS.  Wave w writes its
  // 16 floats of row pair q as 4 float4 slot groups i4 (accumulator elements
  // 4 i4 .. 4 i4 + 3: pixels 8 i4 + 4 (l / 32) + 0..3 of the pair, one output
  // row, 4 consecutive columns); slot S = (4 q + i4) * 64 + l sits at S ^ h,
  // h = (2 (4 q + i4) + l / 32) % 16, so that both the writes (one slot group,
  // 64 lanes) and the item reads (one channel, 16 consecutive items) hit
  // distinct banks.  Each item adds its four waves' float4 in wave order,
  // ((w0 + w1) + w2) + w3. ----
  floatx4_t* part = reinterpret_cast<floatx4_t*>(smem);
  auto slot = [](int q, int i4, int l) __attribute__((always_inline)) {
    const int sg = 4 * q + i4;
    return (sg * 64 + l) ^ ((2 * sg + (l >> 5)) & 15);
  };
  __syncthreads();  // every wave is done with the stage buffers the partials overwrite
#pragma unroll
  for (int q = 0; q < NP; ++q)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4)
      part[wave * (NP * 256) + slot(q, i4, lane)] =
          floatx4_t{acc[q][4 * i4], acc[q][4 * i4 + 1], acc[q][4 * i4 + 2], acc[q][4 * i4 + 3]};
  __syncthreads();

  E* y = static_cast<E*>(a.y);
  float v[KI * 4];
#pragma unroll
  for (int k = 0; k < KI; ++k) {
    // item (co, oh, quad): row pair oh / 2, slot group 2 (oh % 2) + quad / 2,
    // lane 32 (quad % 2) + co
    const int oh = it_oh(k), quad = tid & 3;
    const int sl = slot(oh >> 1, 2 * (oh & 1) + (quad >> 1), 32 * (quad & 1) + it_co(k));
    floatx4_t t = part[sl];
    t = t + part[NP * 256 + sl];
    t = t + part[2 * NP * 256 + sl];
    t = t + part[3 * NP * 256 + sl];
    const float bv = bsm[it_co(k)];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[4 * k + j] = t[j] + bv;
  }
  if (res) {
    if (pairs) {  // every residual read before any store (y may alias it)
      unsigned rq[KI][2];
#pragma unroll
      for (int k = 0; k < KI; ++k)
#pragma unroll
        for (int j2 = 0; j2 < 2; ++j2)
          rq[k][j2] = *reinterpret_cast<const unsigned*>(res + obase + e_clamped(k, 2 * j2, 2));
#pragma unroll
      for (int k = 0; k < KI; ++k)
#pragma unroll
        for (int j2 = 0; j2 < 2; ++j2) {
          const half2_t h = __builtin_bit_cast(half2_t, rq[k][j2]);
          v[4 * k + 2 * j2] = v[4 * k + 2 * j2] + (float)h[0];
          v[4 * k + 2 * j2 + 1] = v[4 * k + 2 * j2 + 1] + (float)h[1];
        }
    } else {  // every residual read before any store (y may alias it)
#pragma unroll
      for (int k = 0; k < KI; ++k)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          v[4 * k + j] = v[4 * k + j] + (float)res[obase + e_clamped(k, j, 1)];
    }
  }
  act_apply<AK>(v, a.act, a.alpha, a.beta);
#pragma unroll
  for (int k = 0; k < KI; ++k) {
    if (pairs) {
#pragma unroll
      for (int j2 = 0; j2 < 2; ++j2)
        if (e_valid(k, 2 * j2)) {  // wo even: both of the pair exist
          const half2_t h = {(E)v[4 * k + 2 * j2], (E)v[4 * k + 2 * j2 + 1]};
          *reinterpret_cast<half2_t*>(y + obase + e_index(k, 2 * j2)) = h;
        }
    } else if constexpr (RAW) {
      float* pl = a.planes + r * a.plane_stride + obase;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (e_valid(k, j)) pl[e_index(k, j)] = v[4 * k + j];
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (e_valid(k, j)) y[obase + e_index(k, j)] = (E)v[4 * k + j];
    }
  }
}

// Launches one instance; the aligned paths take the instance of their stage
// count (1..4, or 5 for five and more), the others the run-time count.
template <typename E, int R, bool XV, bool WV, int AK, bool RAW>
static void launch_rs(const HaloArgs& a, dim3 grid, hipStream_t s) {
  if constexpr (XV && WV) {
    const int ns = RAW ? a.sps : a.cig / RS_CH;
    switch (ns < 5 ? ns : 5) {
      case 1: hipLaunchKernelGGL((rowshift_kernel<E, R, true, true, AK, RAW, 1>), grid, dim3(256), 0, s, a); break;
      case 2: hipLaunchKernelGGL((rowshift_kernel<E, R, true, true, AK, RAW, 2>), grid, dim3(256), 0, s, a); break;
      case 3: hipLaunchKernelGGL((rowshift_kernel<E, R, true, true, AK, RAW, 3>), grid, dim3(256), 0, s, a); break;
      case 4: hipLaunchKernelGGL((rowshift_kernel<E, R, true, true, AK, RAW, 4>), grid, dim3(256), 0, s, a); break;
      default: hipLaunchKernelGGL((rowshift_kernel<E, R, true, true, AK, RAW, 5>), grid, dim3(256), 0, s, a); break;
    }
  } else {
    hipLaunchKernelGGL((rowshift_kernel<E, R, XV, WV, AK, RAW>), grid, dim3(256), 0, s, a);
  }
}

template <typename E, int R, int AK, bool RAW>
static void launch_rs_aligned(const HaloArgs& a, dim3 grid, hipStream_t s) {
  if (a.xvec && a.wvec) launch_rs<E, R, true, true, AK, RAW>(a, grid, s);
  else if (a.xvec) launch_rs<E, R, true, false, -1, RAW>(a, grid, s);
  else if (a.wvec) launch_rs<E, R, false, true, -1, RAW>(a, grid, s);
  else launch_rs<E, R, false, false, -1, RAW>(a, grid, s);
}

template <typename E, int R>
static void launch_rs_r(const HaloArgs& a, dim3 grid, hipStream_t s) {
  if (a.splits > 1) launch_rs_aligned<E, R, -1, true>(a, grid, s);
  else if (a.act == 1) launch_rs_aligned<E, R, 1, false>(a, grid, s);  // ReLU fixed at compile time
  else launch_rs_aligned<E, R, -1, false>(a, grid, s);
}

template <typename E>
static hipError_t launch_rowshift_t(const HaloArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((long long)a.n_ct * a.n * a.groups * a.splits));
  if (a.ho <= 8) launch_rs_r<E, 8>(a, grid, s);
  else if (a.ho <= 14) launch_rs_r<E, 14>(a, grid, s);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_rowshift(Dtype dt, const HaloArgs& a, hipStream_t s) {
  return dt == BF16 ? launch_rowshift_t<__bf16>(a, s) : launch_rowshift_t<_Float16>(a, s);
}

}  // namespace convfwd
