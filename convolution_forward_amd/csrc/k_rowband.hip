// Implicit-GEMM convolution for stride-2 layers with few input channels (the
// stem of an image network: 3 channels, 7x7, stride 2), gfx950, float16
// operands, float32 accumulation ("Convolution, pooling and resize", "Variants":
// the input window is gathered while the tile is staged; no column matrix).
//
// The reduction index is k = (ci, kh, kw) with kw padded to 8: for one (ci, kh)
// the 8 taps of output column ow read input columns 2*ow - pl + 0..7, which are 8
// consecutive halves of one staged input row.  So an MFMA operand fragment (8
// consecutive k of one output pixel) is four 4-byte LDS reads of a row, with no
// column matrix and no per-element gather.  The weight matrix, laid out the same
// way (tap kw = 7 is zero), is loaded once into registers.
//
//  * A workgroup owns a band of output rows of one image and up to 64 output
//    channels.  Input rows live in a ring of LDS rows per channel; output row oh
//    needs input rows 2*oh - pt .. 2*oh - pt + KH - 1, so each new output row
//    brings in only 2 new input rows, loaded (16-byte reads) while the previous
//    row multiplies.  Rows above or below the image are zero rows; columns
//    outside it stay zero from the start.
//  * MFMA v_mfma_f32_32x32x16_f16: A = 32 output pixels x 16 k (two (ci, kh)
//    groups), B = 16 k x 32 output channels.  With 64 channels eight waves
//    (two per SIMD) each own one 32-channel block and one 32-pixel block of the
//    row; with 32 channels four waves own one pixel block each (rows of at most
//    128 outputs).
//  * Epilogue: bias and activation in float32, float16 into an LDS row tile
//    [channel][pixel], then whole output rows leave with 16-byte stores.
// Per output the sum runs over (ci, kh) groups in pairs, each pair inside one
// MFMA; the order is fixed by the shape.
#include <type_traits>

#include "epilogue.h"
#include "internal.h"
#include "mfma16.h"

namespace convfwd {

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

constexpr int RB_RING = 16;        // input rows kept per channel (power of two)
constexpr int RB_MAXST = 12;       // MFMA k-steps (pairs of (ci, kh) groups) at most
constexpr int RB_OPITCH = 128 * 2 + 16;  // LDS bytes per output-tile row (float16)
constexpr int RB_FILLI = 1024;     // items of the first KH rows at most

// Raw buffer descriptor (gfx9 format word 0x00020000) over [p, p + bytes), its
// operands made wave-uniform so that it lives in scalar registers: every access
// is a 32-bit byte offset, with no 64-bit address arithmetic per load or store.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rb_rsrc(const void* p, int bytes) {
  const unsigned long long v = reinterpret_cast<unsigned long long>(p);
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((unsigned long long)hi << 32) | lo),
                                           (short)0, __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

}  // namespace

// NST: MFMA k-steps, ceil(Cin * KH / 2) <= RB_MAXST; WV: waves (8: two
// 32-channel blocks x four 32-pixel blocks; 4: one channel block); VEC: whole
// 16-byte input and output vectors; TWO: two output rows per step (one barrier
// pair per two rows, two independent accumulator chains per wave; the output
// tile holds two rows).
template <typename E, int NST, int WV, bool VEC, int AK = -1, bool TWO = false>
__global__ __launch_bounds__(64 * WV) void rowband_kernel(const RowbandArgs a) {
  typedef E half8_t __attribute__((ext_vector_type(8)));
  typedef E half4_t __attribute__((ext_vector_type(4)));
  typedef E half2_t __attribute__((ext_vector_type(2)));

  constexpr int NT = 64 * WV;
  constexpr int RB_FILL = (RB_FILLI + NT - 1) / NT;  // items per thread for the first KH rows
  constexpr int RB_NSTV = 64 * 16 / NT;              // output vectors per thread and row
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_rb[];
  // ring: [ci][slot][rp halves]; output tile [64 (two rows: 128)][RB_OPITCH bytes]; bias [64]
  E* ring = reinterpret_cast<E*>(smem_rb);
  unsigned char* otile = smem_rb + a.ring_bytes;
  float* bsm = reinterpret_cast<float*>(otile + (TWO ? 128 : 64) * RB_OPITCH);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int rp = a.rpitch;  // halves per ring row (even)

  // work: (image, channel tile, band of output rows)
  int bid = blockIdx.x;
  const int band = bid % a.n_band;
  bid /= a.n_band;
  const int ct = bid % a.n_ct;
  const int n = bid / a.n_ct;
  const int co0 = ct * 64;
  const int r0 = band * a.band_rows;
  const int r1 = min(r0 + a.band_rows, a.ho);

  const E* __restrict__ x = static_cast<const E*>(a.x) + (long long)n * a.c_in * a.h * a.w;
  const __amdgpu_buffer_rsrc_t x_rsrc = rb_rsrc(x, a.c_in * a.h * a.w * 2);
  const E* __restrict__ w = static_cast<const E*>(a.wt);
  static_assert(64 * 2 * RB_MAXST * 8 <= 64 * 1024, "weights staging");

  // ---- wave roles: channel block cbw, pixel block pb0 of 32 ----
  constexpr int CB = 1;
  const int cbw = WV == 8 ? (wave & 1) : 0;
  const int pb0 = WV == 8 ? (wave >> 1) : wave;
  // ---- weights: B fragment of k-step st: lane l holds the 8 taps of group
  // g = 2 st + l / 32 for output channel co0 + 32 cbw + l % 32 ----
  const int groups = a.c_in * a.kh;  // (ci, kh) groups
  const int nv = (a.w + 7) / 8;  // vectors per input row
  // item q of a batch of rows: vector v of row r of channel ci (the batch's
  // rows are consecutive input rows); decomposed once per thread, since every
  // row step uses the same items
  struct Item {
    int v, ci, r;
    bool live;
  };
  auto decomp = [&](int q, int items) __attribute__((always_inline)) {
    Item it;
    const int qc = min(q, items - 1);
    const int rc = (int)mdiv((unsigned)qc, a.mg_nv);
    it.v = qc - rc * nv;
    it.r = (int)mdiv((unsigned)rc, a.mg_cin);
    it.ci = rc - it.r * a.c_in;
    it.live = q < items;
    return it;
  };
  // one item of the batch of rows starting at input row ir0 (clamped into the
  // batch and the image; rows outside the image read as zero)
  auto load_item = [&](int ir0, const Item& it) __attribute__((always_inline)) {
    const int v = it.v, ci = it.ci;
    const int ir = ir0 + it.r;
    // element offset of the item's vector in the clamped row (32-bit: the
    // image's planes are below 2 GiB)
    const int off = (int)__umul24((unsigned)(ci * a.h + min(max(ir, 0), a.h - 1)), (unsigned)a.w) + 8 * v;
    u32x4_t d;
    if constexpr (VEC) {  // w % 8 == 0, 16-byte aligned rows
      d = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(x_rsrc, 2 * off, 0, 0));
    } else {
      const E* src = x + off;
      half8_t h;
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = src[min(e, a.w - 1 - 8 * v)];
      d = __builtin_bit_cast(u32x4_t, h);
    }
    return (ir >= 0 && ir < a.h) ? d : u32x4_t{0, 0, 0, 0};
  };
  // ...and its store into the ring (input column c at ring column c + pl)
  auto store_item = [&](int ir0, const Item& it, u32x4_t d) __attribute__((always_inline)) {
    if (it.live) {
      const int v = it.v, ci = it.ci;
      const int slot = (ir0 + it.r) & (RB_RING - 1);
      E* dst = ring + (ci * RB_RING + slot) * rp + a.pl + 8 * v;
      const half8_t h = __builtin_bit_cast(half8_t, d);
      if constexpr (VEC) {  // w % 8 == 0: whole vectors (the ring column offset is odd-aligned)
#pragma unroll
        for (int e = 0; e < 8; ++e) dst[e] = h[e];
      } else {
        const int cnt = min(8, a.w - 8 * v);  // the row's last vector may be partial
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (e < cnt) dst[e] = h[e];
      }
    }
  };
  // first input row of the sh new rows that output row o brings in
  auto new_rows = [&](int o) __attribute__((always_inline)) { return o * a.sh - a.pt + a.kh - a.sh; };
  const int step_items = a.sh * a.c_in * nv;  // <= 256: one item per thread

  // ---- prologue: every load first (the band's first KH input rows, the next
  // three output rows' new input rows, the tile's weights and biases), so their
  // latencies overlap; then the weights pass through the ring area into
  // registers, the ring is zeroed and the first rows are stored ----
  const int first = r0 * a.sh - a.pt;
  // the first step's rows: KH input rows, and SH more for a second output row
  const int fill_items = (a.kh + (TWO ? a.sh : 0)) * a.c_in * nv;
  u32x4_t t[RB_FILL];
  Item fit[RB_FILL];
#pragma unroll
  for (int k = 0; k < RB_FILL; ++k) {
    fit[k] = decomp(tid + NT * k, fill_items);
    t[k] = load_item(first, fit[k]);
  }
  // prefetch ring of three: the new rows of output row o sit in lr[(o - r0) % 3]
  const Item sit = decomp(tid, TWO ? 2 * step_items : step_items);
  u32x4_t lr[3];
  if constexpr (TWO) {  // step k's new rows sit in lr[k % 2]; step 1's are loaded here
    lr[1] = load_item(new_rows(r0 + 2), sit);
  } else {
    lr[1] = load_item(new_rows(r0 + 1), sit);
    lr[2] = load_item(new_rows(r0 + 2), sit);
    lr[0] = load_item(new_rows(r0 + 3), sit);
  }
  // the tile's weights ([<= 64 channels][groups * kw] contiguous): 16-byte reads
  // when aligned (at most RB_WV per thread), element reads otherwise
  const int per_co = groups * a.kw;
  const int wtotal = min(64, a.c_out - co0) * per_co;  // halves
  const E* wsrc = w + (long long)co0 * per_co;
  constexpr int RB_WV = (64 * 2 * RB_MAXST * 8 / 8 + NT - 1) / NT;
  u32x4_t wv[RB_WV];
  if (a.wvec) {  // uniform: w 16-byte aligned and the tile's run a whole number of vectors
#pragma unroll
    for (int k = 0; k < RB_WV; ++k)
      wv[k] = *reinterpret_cast<const u32x4_t*>(wsrc + 8 * min(tid + NT * k, wtotal / 8 - 1));
  }
  // without a bias the slot holds -0.0, whose addition is exact for every
  // value (a zero keeps its sign), so the epilogue adds it unconditionally
  const float bv_in = (a.bias && co0 + (tid & 63) < a.c_out)
                          ? (float)static_cast<const E*>(a.bias)[co0 + (tid & 63)] : -0.0f;
  {
    E* wl = ring;
    if (a.wvec) {
#pragma unroll
      for (int k = 0; k < RB_WV; ++k) {
        const int q = tid + NT * k;
        if (q < wtotal / 8) reinterpret_cast<u32x4_t*>(wl)[q] = wv[k];
      }
    } else {
      for (int q = tid; q < wtotal; q += NT) wl[q] = wsrc[q];
    }
  }
  __syncthreads();
  // fragment st: the a.kw taps of group g start at half h0 = cl * per_co +
  // g * kw of the staged weights; five dwords from dword h0 / 2, funnel-shifted
  // by 16 bits when h0 is odd, hold halves h0 .. h0 + 7; taps past a.kw and
  // padded groups or channels are masked to zero.  The reads run ahead of any
  // use at clamped addresses (the few halves past the weights are other LDS
  // data, masked off).
  u32x4_t wf[NST];
  {
    const int cl = 32 * cbw + (lane & 31);  // channel within the tile
    const bool okc = co0 + cl < a.c_out;
    const int hc = min(cl, a.c_out - co0 - 1) * per_co;
    unsigned dw[NST][5];
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      const int h0 = hc + min(2 * st + (lane >> 5), groups - 1) * a.kw;
      const unsigned* src = reinterpret_cast<const unsigned*>(ring) + (h0 >> 1);
#pragma unroll
      for (int i = 0; i < 5; ++i) dw[st][i] = src[i];
    }
    // an empty asm that takes the values: the reads stay unconditional (the
    // compiler would otherwise put reads behind the masking branches)
#pragma unroll
    for (int st = 0; st < NST; ++st)
      asm volatile("" : "+v"(dw[st][0]), "+v"(dw[st][1]), "+v"(dw[st][2]), "+v"(dw[st][3]), "+v"(dw[st][4]));
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      const int g = 2 * st + (lane >> 5);
      const int h0 = hc + min(g, groups - 1) * a.kw;
      const unsigned sh = (unsigned)(h0 & 1) * 16u;
      const bool okg = okc && g < groups;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const unsigned keep = (2 * i + 1 < a.kw ? 0xFFFF0000u : 0u) | (2 * i < a.kw ? 0x0000FFFFu : 0u);
        const unsigned f = __builtin_amdgcn_alignbit(dw[st][i + 1], dw[st][i], sh);
        wf[st][i] = okg ? (f & keep) : 0u;
      }
    }
  }
  __syncthreads();  // the ring area is zeroed next
  if (tid < 64) bsm[tid] = bv_in;
  // zero the ring: columns outside the image are never written again
  for (int i = tid; i < a.ring_bytes / 16; i += NT)
    reinterpret_cast<u32x4_t*>(smem_rb)[i] = u32x4_t{0, 0, 0, 0};
  __syncthreads();
#pragma unroll
  for (int k = 0; k < RB_FILL; ++k) store_item(first, fit[k], t[k]);

  const int half = lane >> 5;  // k-group parity of this lane
  // per k-step: this lane's (ci, kh) group as a ring row base and a tap row
  int gbase[NST], gkh[NST];
  // g / kh as (g * m) >> 16 with m = ceil(65536 / kh): exact for g < 4096 / kh
  const unsigned mkh = (65536u + (unsigned)a.kh - 1) / (unsigned)a.kh;
#pragma unroll
  for (int st = 0; st < NST; ++st) {
    const int g = min(2 * st + half, groups - 1);  // the padded group multiplies zero weights
    const int ci = (int)(__umul24((unsigned)g, mkh) >> 16);
    gkh[st] = g - ci * a.kh;
    gbase[st] = ci * RB_RING * rp;
  }
  int pxo[CB];  // ring column offset of this lane's output column in each pixel block
#pragma unroll
  for (int j = 0; j < CB; ++j) pxo[j] = 2 * min(32 * (pb0 + j) + (lane & 31), a.wo - 1);
  const E* __restrict__ res = static_cast<const E*>(a.res);
  E* y = static_cast<E*>(a.y);
  const long long ybase = ((long long)n * a.c_out + co0) * a.ho * a.wo;
  // the tile's output planes (and the residual's) from channel co0 on; the
  // offsets below stay under 64 ho wo elements
  const int howo = a.ho * a.wo;
  const int tile_bytes = (int)min(2147483647LL, (long long)(a.c_out - co0) * howo * 2);
  const __amdgpu_buffer_rsrc_t y_rsrc = rb_rsrc(y + ybase, tile_bytes);
  const __amdgpu_buffer_rsrc_t r_rsrc = rb_rsrc(res ? res + ybase : x, res ? tile_bytes : 2);
  const int cn = min(WV == 8 ? 64 : 32, a.c_out - co0);  // channels of the tile
  const int vpr = (a.wo + 7) / 8;
  // this thread's output vectors of a row (fixed count, past the end the last
  // one repeats): tile element offset at output row 0
  int so[RB_NSTV], sv[RB_NSTV], sc[RB_NSTV];
#pragma unroll
  for (int k = 0; k < RB_NSTV; ++k) {
    const int q = min(tid + NT * k, cn * vpr - 1);
    sc[k] = (int)mdiv((unsigned)q, a.mg_vpr);
    sv[k] = q - sc[k] * vpr;
    so[k] = (int)__umul24((unsigned)sc[k], (unsigned)howo) + 8 * sv[k];
  }

  // two-row steps: vector q of a channel's two output rows (2 vpr vectors,
  // contiguous in y), channels in turn, so that the lanes of a store
  // instruction cover whole runs of 2 wo outputs per channel (fixed count:
  // past the end the last vector repeats)
  constexpr int RB_NST2 = TWO ? (64 * 32 + NT - 1) / NT : 1;
  int c2[RB_NST2], v2[RB_NST2];
#pragma unroll
  for (int k = 0; k < RB_NST2; ++k) {
    const int q = min(tid + NT * k, cn * 2 * vpr - 1);
    c2[k] = (int)mdiv((unsigned)q, a.mg_vpr2);
    v2[k] = q - c2[k] * 2 * vpr;
  }

  // one output row; J = (oh - r0) % 3 at compile time picks the prefetch registers
  auto row = [&](int oh, auto jc) __attribute__((always_inline)) {
    constexpr int J = decltype(jc)::value;
    // the next output row's new input rows go to ring slots this row does not use
    store_item(new_rows(oh + 1), sit, lr[(J + 1) % 3]);
    __syncthreads();  // rows of oh present; the previous row's tile has left
    // those registers now take the rows of output row oh + 4 (three rows ahead)
    lr[(J + 1) % 3] = load_item(new_rows(oh + 4), sit);

    // ---- MFMA: k-step st covers groups 2 st (lanes 0-31) and 2 st + 1 (32-63) ----
    floatx16_t acc[CB];
#pragma unroll
    for (int j = 0; j < CB; ++j)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[j][i] = 0.f;
    const int ir_base = oh * a.sh - a.pt;
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      const int slot = (ir_base + gkh[st]) & (RB_RING - 1);
#pragma unroll
      for (int j = 0; j < CB; ++j) {
        const unsigned int* src =
            reinterpret_cast<const unsigned int*>(ring + gbase[st] + slot * rp + pxo[j]);
        u32x4_t f;
#pragma unroll
        for (int e = 0; e < 4; ++e) f[e] = src[e];
        acc[j] = mfma_32x32x16<E>(f, wf[st], acc[j]);
      }
    }

    // ---- epilogue: lane l holds channel 32 cbw + l % 32 and, in pixel block
    // pb0 + j, output columns 32 (pb0 + j) + 8 (i / 4) + 4 (l / 32) + i % 4 ----
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      const int c = 32 * cbw + (lane & 31);
      const int pxb = 32 * (pb0 + j);
      // the bias is read once, outside any branch (a read under the per-value
      // condition became one branch and one LDS round trip per value)
      const float bv = bsm[c];
      float v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = acc[j][i] + bv;
      if (res) {  // residual read in the fragment layout (clamped, before any store)
        const int rrow = (int)__umul24((unsigned)min(c, a.c_out - co0 - 1), (unsigned)howo) + oh * a.wo;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int ow = min(pxb + 8 * (i / 4) + 4 * half + (i % 4), a.wo - 1);
          const unsigned short r16 = __builtin_amdgcn_raw_buffer_load_b16(r_rsrc, 2 * (rrow + ow), 0, 0);
          v[i] = v[i] + (float)__builtin_bit_cast(E, r16);
        }
      }
      act_apply<AK>(v, a.act, a.alpha, a.beta);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        half4_t h;
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = (E)v[4 * q + i];
        *reinterpret_cast<half4_t*>(otile + c * RB_OPITCH + 2 * (pxb + 8 * q + 4 * half)) = h;
      }
    }
    __syncthreads();
    // ---- whole rows of the tile: 16-byte vectors of 8 output columns ----
    if constexpr (VEC) {  // wo % 8 == 0: whole vectors; past the end the last one
      // repeats (same value, same address), so the store count is fixed
      const int orow = oh * a.wo;
#pragma unroll
      for (int k = 0; k < RB_NSTV; ++k) {
        const u32x4_t d = *reinterpret_cast<const u32x4_t*>(otile + sc[k] * RB_OPITCH + 16 * sv[k]);
        // nontemporal (the output is not read back)
        __builtin_amdgcn_raw_buffer_store_b128(d, y_rsrc, 2 * (so[k] + orow), 0, 2);
      }
    } else {
      for (int q = tid; q < cn * vpr; q += NT) {
        const int c = (int)mdiv((unsigned)q, a.mg_vpr), v = q - c * vpr;
        const half8_t h = __builtin_bit_cast(half8_t, *reinterpret_cast<const u32x4_t*>(
                                                          otile + c * RB_OPITCH + 16 * v));
        E* dst = y + ybase + ((long long)c * a.ho + oh) * a.wo + 8 * v;
        const int cnt = min(8, a.wo - 8 * v);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (e < cnt) dst[e] = h[e];
      }
    }
  };

  // two output rows oh, oh + 1 (the second is computed but not stored past the
  // band); J = step % 2 at compile time picks the prefetch registers
  auto row2 = [&](int oh, auto jc) __attribute__((always_inline)) {
    constexpr int J = decltype(jc)::value;
    __syncthreads();  // rows of this step present; the previous step's tile has left
    // the next step's new rows go to ring slots this step does not read (the
    // ring spans KH + 3 SH rows from this step's first), then those registers
    // take the rows of the step after
    store_item(new_rows(oh + 2), sit, lr[(J + 1) % 2]);
    lr[J] = load_item(new_rows(oh + 4), sit);

    floatx16_t acc[2];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[r][i] = 0.f;
    const int ir_base = oh * a.sh - a.pt;
#pragma unroll
    for (int st = 0; st < NST; ++st) {
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int slot = (ir_base + r * a.sh + gkh[st]) & (RB_RING - 1);
        const unsigned int* src = reinterpret_cast<const unsigned int*>(ring + gbase[st] + slot * rp + pxo[0]);
        u32x4_t f;
#pragma unroll
        for (int e = 0; e < 4; ++e) f[e] = src[e];
        acc[r] = mfma_32x32x16<E>(f, wf[st], acc[r]);
      }
    }
    const int c = 32 * cbw + (lane & 31);
    const int pxb = 32 * pb0;
    const float bv = bsm[c];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      float v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = acc[r][i] + bv;
      if (res) {  // residual read in the fragment layout (clamped, before any store)
        const int rrow = (int)__umul24((unsigned)min(c, a.c_out - co0 - 1), (unsigned)howo) +
                         min(oh + r, a.ho - 1) * a.wo;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int ow = min(pxb + 8 * (i / 4) + 4 * half + (i % 4), a.wo - 1);
          const unsigned short r16 = __builtin_amdgcn_raw_buffer_load_b16(r_rsrc, 2 * (rrow + ow), 0, 0);
          v[i] = v[i] + (float)__builtin_bit_cast(E, r16);
        }
      }
      act_apply<AK>(v, a.act, a.alpha, a.beta);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        half4_t h;
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = (E)v[4 * q + i];
        *reinterpret_cast<half4_t*>(otile + (r * 64 + c) * RB_OPITCH + 2 * (pxb + 8 * q + 4 * half)) = h;
      }
    }
    __syncthreads();
    // ---- the tile's two rows per channel as one run of 16-byte vectors (the
    // vector path: wo % 8 == 0, so row oh + 1 follows row oh in y); a row past
    // the band gets the descriptor's size as its offset (store dropped).
    // Whole runs per store instruction write faster than row-by-row stores
    // (w3a 25.7 -> 23.6 us). ----
    const int orow = oh * a.wo;
    const int rows = min(2, r1 - oh);
#pragma unroll
    for (int k = 0; k < RB_NST2; ++k) {
      const int r = v2[k] >= vpr ? 1 : 0, sv2 = v2[k] - r * vpr;
      const u32x4_t d = *reinterpret_cast<const u32x4_t*>(otile + (r * 64 + c2[k]) * RB_OPITCH + 16 * sv2);
      __builtin_amdgcn_raw_buffer_store_b128(
          d, y_rsrc, r < rows ? 2 * ((int)__umul24((unsigned)c2[k], (unsigned)howo) + orow + 8 * v2[k]) : tile_bytes,
          0, 2);
    }
  };

  if constexpr (TWO) {
    static_assert(WV == 8 && VEC, "two-row steps: eight waves, whole vectors");
    for (int oh = r0; oh < r1; oh += 4) {  // unrolled by two: prefetch sets at compile time
      row2(oh, std::integral_constant<int, 0>{});
      if (oh + 2 >= r1) break;
      row2(oh + 2, std::integral_constant<int, 1>{});
    }
  } else {
    for (int oh = r0; oh < r1; oh += 3) {  // unrolled by three: prefetch sets at compile time
      row(oh, std::integral_constant<int, 0>{});
      if (oh + 1 >= r1) break;
      row(oh + 1, std::integral_constant<int, 1>{});
      if (oh + 2 >= r1) break;
      row(oh + 2, std::integral_constant<int, 2>{});
    }
  }
}

template <typename E, int NST>
static void launch_rb_nst(const RowbandArgs& a, dim3 grid, size_t lds, hipStream_t s) {
  const bool two = a.c_out > 32;
  if (a.two_rows) {  // eight waves, whole vectors: two output rows per step
    lds += 64 * RB_OPITCH;
    if (a.act == 1) hipLaunchKernelGGL((rowband_kernel<E, NST, 8, true, 1, true>), grid, dim3(512), lds, s, a);
    else hipLaunchKernelGGL((rowband_kernel<E, NST, 8, true, -1, true>), grid, dim3(512), lds, s, a);
  } else if (a.vec && a.act == 1) {  // ReLU, the common case, fixed at compile time
    if (two) hipLaunchKernelGGL((rowband_kernel<E, NST, 8, true, 1>), grid, dim3(512), lds, s, a);
    else hipLaunchKernelGGL((rowband_kernel<E, NST, 4, true, 1>), grid, dim3(256), lds, s, a);
  } else if (a.vec) {
    if (two) hipLaunchKernelGGL((rowband_kernel<E, NST, 8, true>), grid, dim3(512), lds, s, a);
    else hipLaunchKernelGGL((rowband_kernel<E, NST, 4, true>), grid, dim3(256), lds, s, a);
  } else {
    if (two) hipLaunchKernelGGL((rowband_kernel<E, NST, 8, false>), grid, dim3(512), lds, s, a);
    else hipLaunchKernelGGL((rowband_kernel<E, NST, 4, false>), grid, dim3(256), lds, s, a);
  }
}

hipError_t launch_rowband(Dtype dt, const RowbandArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((long long)a.n * a.n_ct * a.n_band));
  const size_t lds = (size_t)a.ring_bytes + 64 * RB_OPITCH + 64 * 4;
  // k-steps: exact for the 3-channel 7x7 stem, else the maximum (padded steps
  // multiply zero weights)
  const int nst = (a.c_in * a.kh + 1) / 2;
  if (nst > RB_MAXST) return hipErrorInvalidValue;
  if (dt == BF16) {
    if (nst == 11) launch_rb_nst<__bf16, 11>(a, grid, lds, s);
    else launch_rb_nst<__bf16, RB_MAXST>(a, grid, lds, s);
  } else {
    if (nst == 11) launch_rb_nst<_Float16, 11>(a, grid, lds, s);
    else launch_rb_nst<_Float16, RB_MAXST>(a, grid, lds, s);
  }
  return hipGetLastError();
}

}  // namespace convfwd
