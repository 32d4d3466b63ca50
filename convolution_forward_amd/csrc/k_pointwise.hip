// Pointwise (1x1, stride 1, no padding, one group) convolution as a GEMM on the
// input as it lies ("Convolution, pooling and resize", "Variants": the 1x1 case
// multiplies the weight matrix by x without any gathering; "Convolutions",
// section 2.4: a 1x1 convolution is a per-pixel linear map), gfx950, float16
// operands, float32 accumulation:
//
//   y[n, co, p] = act( sum_ci w[co, ci] * x[n, ci, p]  + bias[co] + res[n, co, p] )
//
// for every image n and pixel p of the H*W plane.  The same kernel runs the
// ConvTranspose whose kernel equals its stride of 2 with no padding
// ("Convolutions", section 2.5, transposed convolution: with kernel = stride the
// copies of the kernel do not overlap, so each output takes exactly one tap):
// GEMM rows m = 4 co + 2 kh + kw, weights [ci][m] as they lie, and the epilogue
// scatters row m, pixel (h, w) to y[n, co, 2h + kh, 2w + kw].
//
//  * Tile: 128 pixels of one image x TC (64 or 128) GEMM rows; the input
//    channels are consumed in chunks of 64.  Four waves, each 16 PB pixels x 64
//    rows as PB x 4 MFMA blocks of v_mfma_f32_16x16x32_f16 (A = x transposed:
//    pixel rows, channel k; B = w transposed: channel k, GEMM-row columns).
//  * x is read as it lies: a thread loads 4 consecutive pixels of 8 channels
//    (8 bytes per channel plane) and regroups them in registers into 4 channel
//    octets, stored pixel-major in LDS (16 bytes per pixel and octet, swizzled so
//    the 16 pixels of an MFMA block hit distinct banks).  Weight rows (64
//    channels, 128 bytes per GEMM row) go to LDS rows padded to 144 bytes: as
//    16-byte copies for [co][ci] weights, regrouped in registers from 8-byte
//    pieces of 4 rows for [ci][m] weights.
//  * Persistent workgroups walk (tile, chunk) work items, PF of them in flight:
//    after an item is staged its registers are refilled with the item PF later,
//    so the loads of PF items overlap the multiplies.  Every step issues the
//    same loads, and the last PF items run without refills.
//  * Epilogue: a lane holds 4 consecutive pixels of one GEMM row; bias, residual
//    and activation run in float32 on them, the float16 results go to an LDS
//    output tile [row][pixel] in the freed staging area, and leave from there
//    with 16-byte stores (whole 256-byte rows, or the ConvTranspose scatter).
// Per output the sum runs over the channels in increasing order in steps of 32
// (the MFMA's internal order within a step).
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "epilogue.h"
#include "internal.h"
#include "mfma16.h"

namespace convfwd {

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

constexpr int PW_TP = 128;                 // pixels per tile
constexpr int PW_KC = 64;                  // input channels per chunk
constexpr int PW_XBYTES = PW_TP * PW_KC * 2;
constexpr int PW_WROW = PW_KC * 2 + 16;    // padded LDS bytes per GEMM row
constexpr int PW_OROW = PW_TP * 2 + 16;    // LDS bytes per output-tile row (float16)

// octet slot at pixel row p: the 16 rows of an MFMA block land on distinct banks
__device__ __forceinline__ int pw_slot(int p, int o) { return o ^ ((p >> 1) & 7); }

// Raw buffer descriptor (gfx9 format word 0x00020000) over [p, p + bytes), its
// operands made wave-uniform.  Accesses take a per-lane 32-bit byte offset and a
// uniform one; an access past the range reads 0 (a store is dropped).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t pw_rsrc(const void* p, int bytes) {
  const unsigned long long v = reinterpret_cast<unsigned long long>(p);
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((unsigned long long)hi << 32) | lo),
                                           (short)0, __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

}  // namespace

// VEC: x 8-byte, w 16-byte (8-byte for ConvTranspose), y 16-byte and residual
// 8-byte aligned, planes of whole 8-pixel vectors; otherwise every access is
// element-wise.  PF divides the chunk count, so a group of PF items never
// straddles two tiles.
// AK: the activation fixed at compile time (the ONNX code), or -1 for the
// launch's code chosen at run time.
template <typename E, int PW_TC, bool CT, int PF, bool VEC, int AK = -1>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(PF > 2 ? 2 : PW_TC == 128 || PF > 1 ? 3 : 4)))
void pointwise_f16_kernel(const PwArgs a) {
  typedef E half8_t __attribute__((ext_vector_type(8)));
  typedef E half4_t __attribute__((ext_vector_type(4)));
  typedef E half2_t __attribute__((ext_vector_type(2)));

  constexpr int PW_WBYTES = PW_TC * PW_WROW;
  constexpr int PW_NW = PW_TC * (PW_KC / 8) / 256;  // 16-byte weight vectors per thread
  static_assert(PW_TC * PW_OROW <= PW_XBYTES + PW_WBYTES, "output tile reuses the staging area");
  constexpr int WCN = PW_TC / 64;  // waves along the GEMM rows (64 each)
  constexpr int WPN = 4 / WCN;     // waves along the pixels
  constexpr int PB = PW_TP / WPN / 16;  // 16-pixel MFMA blocks per wave
  __shared__ __attribute__((aligned(16))) unsigned char smem[PW_XBYTES + PW_WBYTES + PW_TC * 4];
  unsigned char* xs = smem;
  unsigned char* ws = smem + PW_XBYTES;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hw = a.hw;
  const E* __restrict__ x = static_cast<const E*>(a.x);
  const E* __restrict__ w = static_cast<const E*>(a.wt);
  const E* bias = static_cast<const E*>(a.bias);
  const E* res = static_cast<const E*>(a.res);
  E* y = static_cast<E*>(a.y);

  // staging item of this thread: channel octet so, 4-pixel group sg of the tile
  const int so = tid >> 5, sg = tid & 31;
  // ConvTranspose weight item of this thread: KG input channels from kg * KG on,
  // GEMM rows 4 mq .. 4 mq + 3 (256 items per chunk)
  constexpr int KG = PW_KC * PW_TC / 4 / 256;
  const int kg = tid % (PW_KC / KG), mq = tid / (PW_KC / KG);

  // Vector path: every load's byte offset is a per-thread part fixed for the
  // launch plus a uniform per-item part, added into the per-lane offset of a
  // buffer access (tensors below 2 GiB).  Nothing is clamped: channels past
  // c_in are zeroed when staged, pixels past the plane or rows past c_out only
  // feed outputs that are never stored, and an offset past a tensor's end
  // reads 0.  The range check covers the per-lane offset only, so no part of
  // an offset goes in the scalar operand.
  const __amdgpu_buffer_rsrc_t x_rsrc = pw_rsrc(x, a.n * a.c_in * hw * 2);
  const __amdgpu_buffer_rsrc_t w_rsrc = pw_rsrc(w, a.c_out * a.c_in * 2);
  const __amdgpu_buffer_rsrc_t b_rsrc = pw_rsrc(bias ? bias : x, bias ? (CT ? a.c_out / 4 : a.c_out) * 2 : 0);
  const __amdgpu_buffer_rsrc_t y_rsrc = pw_rsrc(y, a.n * a.c_out * hw * 2);
  const __amdgpu_buffer_rsrc_t r_rsrc = pw_rsrc(res ? res : x, res ? a.n * a.c_out * hw * 2 : 0);
  const int x_lane = 2 * (8 * so * hw + 4 * sg);
  const int wt_lane = 2 * (KG * kg * a.c_out + 4 * mq);
  const int b_lane = 2 * (CT ? (tid % PW_TC) / 4 : tid % PW_TC);
  int w_lane[PW_NW];
#pragma unroll
  for (int i = 0; i < PW_NW; ++i) {
    const int q = tid + 256 * i;
    w_lane[i] = 2 * ((q >> 3) * a.c_in + 8 * (q & 7));
  }

  // operand registers of PF work items in flight (slot = compile-time index)
  u32x2_t xr[PF][8];       // 8 channels x 4 pixels
  u32x4_t wr[PF][PW_NW];   // weight vectors
  u32x2_t wt[PF][KG];      // ConvTranspose weights: KG input channels x 4 GEMM rows
  E br[PF];         // bias of tile row tid (tid < TC), converted when staged
  float* bsm = reinterpret_cast<float*>(smem + PW_XBYTES + PW_WBYTES);

  // work item = tile * nchunks + chunk; tile = (image, pixel tile, row tile),
  // row tile fastest
  auto decode = [&](int item, int& n, int& p0, int& co0, int& c0) __attribute__((always_inline)) {
    // (divisions by the host's multiply-shift constants)
    const int t = (int)mdiv((unsigned)item, a.mg_nch);
    c0 = (item - t * a.nchunks) * PW_KC;
    const int r = (int)mdiv((unsigned)t, a.mg_nct);
    const int ct = t - r * a.n_ct;
    n = (int)mdiv((unsigned)r, a.mg_npt);
    const int pt = r - n * a.n_pt;
    p0 = pt * a.tp;
    co0 = ct * PW_TC;
  };
  // Every load of a step is unconditional (clamped addresses), so the waits
  // before staging count exactly the younger loads.
  auto load = [&](auto S, int item) __attribute__((always_inline)) {
    int n, p0, co0, c0;
    decode(item, n, p0, co0, c0);
    if constexpr (VEC) {
      const int xoff = x_lane + 2 * ((n * a.c_in + c0) * hw + p0);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        xr[S][e] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(x_rsrc, xoff + 2 * e * hw, 0, 0));
      br[S] = __builtin_bit_cast(E, __builtin_amdgcn_raw_buffer_load_b16(b_rsrc, b_lane + 2 * (CT ? co0 / 4 : co0), 0, 0));
      if constexpr (CT) {  // weights lie [ci][m]: 4 rows m of KG input channels
        const int woff = wt_lane + 2 * (c0 * a.c_out + co0);
#pragma unroll
        for (int e = 0; e < KG; ++e)
          wt[S][e] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(w_rsrc, woff + 2 * e * a.c_out, 0, 0));
      } else {  // w: row co0 + q / 8, 16-byte piece q % 8 of the chunk
        const int woff = 2 * (co0 * a.c_in + c0);
#pragma unroll
        for (int i = 0; i < PW_NW; ++i)
          wr[S][i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, w_lane[i] + woff, 0, 0));
      }
      return;
    }
    // x: channels c0 + 8 so + e, pixels p0 + 4 sg .. + 3 (clamped into the plane
    // and the channel range; out-of-range values are zeroed when staged)
    const int px = min(p0 + 4 * sg, hw - 4);
    const E* xb = x + ((long long)n * a.c_in) * hw + px;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int ci = min(c0 + 8 * so + e, a.c_in - 1);
      if constexpr (VEC) {
        xr[S][e] = *reinterpret_cast<const u32x2_t*>(xb + (long long)ci * hw);
      } else {
        half4_t h;
#pragma unroll
        for (int j = 0; j < 4; ++j) h[j] = xb[(long long)ci * hw + j];
        xr[S][e] = __builtin_bit_cast(u32x2_t, h);
      }
    }
    {  // bias of tile row tid (any valid address without bias)
      const int m = min(co0 + (tid % PW_TC), a.c_out - 1);
      const E* bp = bias ? bias + (CT ? m / 4 : m) : x;
      br[S] = *bp;
    }
    if constexpr (CT) {
      // weights lie [ci][m]: 4 consecutive rows m of KG input channels, regrouped
      // into 4 row pieces of KG channels when staged
      const int m = min(co0 + 4 * mq, a.c_out - 4);  // c_out % 4 == 0
#pragma unroll
      for (int e = 0; e < KG; ++e) {
        const int ci = min(c0 + KG * kg + e, a.c_in - 1);
        const E* src = w + (long long)ci * a.c_out + m;
        if constexpr (VEC) {
          wt[S][e] = *reinterpret_cast<const u32x2_t*>(src);
        } else {
          half4_t h;
#pragma unroll
          for (int j = 0; j < 4; ++j) h[j] = src[j];
          wt[S][e] = __builtin_bit_cast(u32x2_t, h);
        }
      }
    } else {
      // w: row co0 + q / 8, 16-byte piece q % 8 of the chunk
#pragma unroll
      for (int i = 0; i < PW_NW; ++i) {
        const int q = tid + 256 * i;
        const int co = min(co0 + (q >> 3), a.c_out - 1);
        const int ci = min(c0 + 8 * (q & 7), a.c_in - 8);  // c_in % 8 == 0
        const E* src = w + (long long)co * a.c_in + ci;
        if constexpr (VEC) {
          wr[S][i] = *reinterpret_cast<const u32x4_t*>(src);
        } else {
          half8_t h;
#pragma unroll
          for (int e = 0; e < 8; ++e) h[e] = src[e];
          wr[S][i] = __builtin_bit_cast(u32x4_t, h);
        }
      }
    }
  };
  auto stage = [&](auto S, int item) __attribute__((always_inline)) {
    int n, p0, co0, c0;
    decode(item, n, p0, co0, c0);
    if (c0 + PW_KC <= a.c_in) {  // uniform: the whole chunk exists
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        half8_t v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = __builtin_bit_cast(half4_t, xr[S][e])[j];
        const int p = 4 * sg + j;
        *reinterpret_cast<half8_t*>(xs + p * 128 + 16 * pw_slot(p, so)) = v;
      }
    } else {
      const int cvalid = a.c_in - (c0 + 8 * so);  // channels of this octet that exist
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        half8_t v;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          v[e] = e < cvalid ? __builtin_bit_cast(half4_t, xr[S][e])[j] : (E)0.0f;
        const int p = 4 * sg + j;
        *reinterpret_cast<half8_t*>(xs + p * 128 + 16 * pw_slot(p, so)) = v;
      }
    }
    if (tid < PW_TC) bsm[tid] = (float)br[S];
    if constexpr (CT) {
      const int kvalid = a.c_in - (c0 + KG * kg);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        E v __attribute__((ext_vector_type(KG)));
#pragma unroll
        for (int e = 0; e < KG; ++e)
          v[e] = e < kvalid ? __builtin_bit_cast(half4_t, wt[S][e])[j] : (E)0.0f;
        *reinterpret_cast<decltype(v)*>(ws + (4 * mq + j) * PW_WROW + 2 * KG * kg) = v;
      }
    } else {
#pragma unroll
      for (int i = 0; i < PW_NW; ++i) {
        const int q = tid + 256 * i;
        const bool ok = c0 + 8 * (q & 7) < a.c_in;  // whole octets: c_in % 8 == 0
        *reinterpret_cast<u32x4_t*>(ws + (q >> 3) * PW_WROW + 16 * (q & 7)) =
            ok ? wr[S][i] : u32x4_t{0, 0, 0, 0};
      }
    }
  };

  const int wp = wave % WPN, wc = wave / WPN;  // wave's pixel and row ranges
  floatx4_t acc[PB][4];
#pragma unroll
  for (int i = 0; i < PB; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < PW_KC / 32; ++ks) {
      const int o = 4 * ks + (lane >> 4);
      half8_t af[PB], bf[4];
#pragma unroll
      for (int pb = 0; pb < PB; ++pb) {
        const int p = 16 * PB * wp + 16 * pb + (lane & 15);
        af[pb] = *reinterpret_cast<const half8_t*>(xs + p * 128 + 16 * pw_slot(p, o));
      }
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const int c = 64 * wc + 16 * cb + (lane & 15);
        bf[cb] = *reinterpret_cast<const half8_t*>(ws + c * PW_WROW + 16 * o);
      }
#pragma unroll
      for (int pb = 0; pb < PB; ++pb)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
          acc[pb][cb] = mfma_16x16x32<E>(af[pb], bf[cb], acc[pb][cb]);
    }
  };

  // Epilogue.  Phase 1, per lane from the accumulators: bias, residual and
  // activation in float32, rounded to float16 into the LDS output tile
  // [row][pixel] (which reuses the staging area).  Phase 2: the tile leaves with
  // 16-byte stores.  Every residual read happens in phase 1, before the barrier
  // that precedes any store (y may alias the residual).
  auto epilogue = [&](int item) __attribute__((always_inline)) {
    int n, p0, co0, c0;
    decode(item, n, p0, co0, c0);
    const int pl0 = 16 * PB * wp + 4 * (lane >> 4);  // tile pixel of the lane's first value
    const int cl0 = 64 * wc + (lane & 15);      // tile row of the lane's block 0
#pragma unroll
    for (int pb = 0; pb < PB; ++pb) {
      float v[16];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const float bv = bsm[cl0 + 16 * cb];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float t = acc[pb][cb][i];
          if (bias) t = t + bv;
          v[4 * cb + i] = t;
        }
      }
      if (res && VEC) {  // never with CT; rows past c_out or pixels past the plane are never stored
        const int roff = 2 * ((n * a.c_out + co0 + cl0) * hw + p0 + pl0 + 16 * pb);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          const half4_t h = __builtin_bit_cast(half4_t, __builtin_amdgcn_raw_buffer_load_b64(r_rsrc, roff + 2 * 16 * cb * hw, 0, 0));
#pragma unroll
          for (int i = 0; i < 4; ++i) v[4 * cb + i] = v[4 * cb + i] + (float)h[i];
        }
      } else if (res) {  // never with CT
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          const int p = min(p0 + pl0 + 16 * pb, hw - 4);
          const int co = min(co0 + cl0 + 16 * cb, a.c_out - 1);
          const E* src = res + ((long long)n * a.c_out + co) * hw + p;
          half4_t h;
          if constexpr (VEC) {
            h = __builtin_bit_cast(half4_t, *reinterpret_cast<const u32x2_t*>(src));
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) h[i] = src[i];
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) v[4 * cb + i] = v[4 * cb + i] + (float)h[i];
        }
      }
      if constexpr (AK < 0) {
        act_array(v, a.act, a.alpha, a.beta);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = act_t<AK>(v[i], a.alpha, a.beta);
      }
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        half4_t h;
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = (E)v[4 * cb + i];
        *reinterpret_cast<half4_t*>(smem + (cl0 + 16 * cb) * PW_OROW + 2 * (pl0 + 16 * pb)) = h;
      }
    }
#pragma unroll
    for (int i = 0; i < PB; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    __syncthreads();
    const int pvalid = min(a.tp, hw - p0);  // a multiple of 4 (of 8 with VEC)
    if constexpr (CT) {
      // output (co, 2h + kh, 2w + kw) is tile row 4 co + 2 kh + kw at pixel
      // (h, w): the scatter is a permutation of the tile.  A vector is 8
      // consecutive outputs of one output row: input columns 4v .. 4v + 3 of rows
      // kw = 0 and kw = 1, interleaved.  The tile holds whole input rows.  Vectors
      // past the valid ones repeat the last one (same value, same address): the
      // store count is fixed.
      // Vectors are numbered over a full tile of R input rows; those of rows past
      // a ragged last tile repeat its last row.
      const int win = a.w_in, R = a.ct_rows;
      const int vpr = win >> 2;  // vectors per output row
      const int rvalid = (int)mdiv((unsigned)(pvalid >> 2), a.mg_vpr);  // rows in this tile
      const int cvalid = min(PW_TC / 4, (a.c_out - co0) / 4);
      const int nvec = cvalid * R * 2 * vpr;
      const int h0 = (int)mdiv((unsigned)(p0 >> 2), a.mg_vpr), cl0 = co0 / 4;
      const int wo = 2 * win, ho = 2 * (int)mdiv((unsigned)(hw >> 2), a.mg_vpr);
#pragma unroll
      for (int k = 0; k < PW_TC / 16; ++k) {
        const int q = min(tid + 256 * k, nvec - 1);
        const int r2 = (int)mdiv((unsigned)q, a.mg_vpr), v = q - r2 * vpr;
        const int kh = r2 & 1, r3 = r2 >> 1;
        const int c = (int)mdiv((unsigned)r3, a.mg_rows), hl = min(r3 - c * R, rvalid - 1);
        const unsigned char* rp = smem + (4 * c + 2 * kh) * PW_OROW + 2 * (hl * win + 4 * v);
        const half4_t e0 = *reinterpret_cast<const half4_t*>(rp);
        const half4_t e1 = *reinterpret_cast<const half4_t*>(rp + PW_OROW);
        const half8_t hv = {e0[0], e1[0], e0[1], e1[1], e0[2], e1[2], e0[3], e1[3]};
        if constexpr (VEC) {  // nontemporal (the output is not read back)
          const int off = 2 * (((n * (a.c_out / 4) + cl0 + c) * ho + 2 * (h0 + hl) + kh) * wo + 8 * v);
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, hv), y_rsrc, off, 0, 2);
        } else {
          E* dst = y + (((long long)n * (a.c_out / 4) + cl0 + c) * ho + 2 * (h0 + hl) + kh) * wo + 8 * v;
#pragma unroll
          for (int e = 0; e < 8; ++e) dst[e] = hv[e];
        }
      }
    } else if constexpr (VEC) {
      // TC rows of 16 vectors of 8 pixels; vectors past the tile's valid rows or
      // pixels repeat the last valid vector of the tile (same value, same
      // address): the store count is fixed
      const int rlast = min(PW_TC, a.c_out - co0) - 1;
#pragma unroll
      for (int k = 0; k < PW_TC * PW_TP / 8 / 256; ++k) {
        const int q = tid + 256 * k;
        const int row = min(q >> 4, rlast), px = min(8 * (q & 15), pvalid - 8);
        const u32x4_t d = *reinterpret_cast<const u32x4_t*>(smem + row * PW_OROW + 2 * px);
        // nontemporal (the output is not read back).  The whole offset is the
        // per-lane one: with the tile's base in the scalar offset, stores of
        // lanes repeating one vector lost their first 4 bytes now and then
        // (the index probes caught it); loads take a scalar offset correctly.
        __builtin_amdgcn_raw_buffer_store_b128(d, y_rsrc, 2 * ((n * a.c_out + co0 + row) * hw + p0 + px), 0, 2);
      }
    } else {
#pragma unroll 1
      for (int k = 0; k < PW_TC * PW_TP / 8 / 256; ++k) {
        const int q = tid + 256 * k;
        const int row = q >> 4, px = 8 * (q & 15);
        const int co = co0 + row;
        if (co < a.c_out && px < pvalid) {
          const half8_t h = *reinterpret_cast<const half8_t*>(smem + row * PW_OROW + 2 * px);
          E* dst = y + ((long long)n * a.c_out + co) * hw + p0 + px;
          const int cnt = min(8, pvalid - px);
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (e < cnt) dst[e] = h[e];
        }
      }
    }
    __syncthreads();  // the next staging overwrites the output tile
  };

  // Tiles are dealt to the 8 XCDs in contiguous ranges (workgroup b runs on XCD
  // b % 8): the row tiles of one pixel tile, which read the same x, then share
  // an L2.  The grid is the tile count or a multiple of 8, so every XCD with
  // tiles has workgroups.  Workgroup j of an XCD takes tiles j, j + gx, ... of
  // its range; its work items k = 0 .. cnt - 1 are (tile, chunk) pairs.
  const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int gx = (gridDim.x >> 3) + (xcd < (int)(gridDim.x & 7));  // workgroups on this XCD
  const int tq = a.ntiles >> 3, tr = a.ntiles & 7;
  const int t_first = xcd < tr ? xcd * (tq + 1) : tr * (tq + 1) + (xcd - tr) * tq;
  const int t_count = tq + (xcd < tr);
  const int cnt = j < t_count ? (t_count - j + gx - 1) / gx * a.nchunks : 0;
  if (cnt == 0) return;
  auto item_of = [&](int k) __attribute__((always_inline)) {
    const int kt = (int)mdiv((unsigned)k, a.mg_nch);
    return (t_first + j + kt * gx) * a.nchunks + (k - kt * a.nchunks);
  };
  // one step: stage slot S (item k), refill it with item k + PF when REFILL,
  // multiply
  auto step = [&](auto S, auto REFILL, int k) __attribute__((always_inline)) {
    stage(S, item_of(k));
    __syncthreads();
    if constexpr (decltype(REFILL)::value) load(S, item_of(k + PF));
    compute();
    __syncthreads();
  };
  // a group: PF steps (one per slot), then the tile's epilogue if the group
  // ends it
  auto group = [&](auto REFILL, int k) __attribute__((always_inline)) {
    step(std::integral_constant<int, 0>{}, REFILL, k);
    if constexpr (PF > 1) step(std::integral_constant<int, 1>{}, REFILL, k + 1);
    if constexpr (PF > 2) step(std::integral_constant<int, 2>{}, REFILL, k + 2);
    if constexpr (PF > 3) step(std::integral_constant<int, 3>{}, REFILL, k + 3);
    const int last = item_of(k + PF - 1);
    if ((last % a.nchunks) == a.nchunks - 1) epilogue(last);
  };
  static_assert(PF >= 1 && PF <= 4, "prefetch depth");
  load(std::integral_constant<int, 0>{}, item_of(0));
  if constexpr (PF > 1) load(std::integral_constant<int, 1>{}, item_of(1));
  if constexpr (PF > 2) load(std::integral_constant<int, 2>{}, item_of(2));
  if constexpr (PF > 3) load(std::integral_constant<int, 3>{}, item_of(3));
  int k = 0;
  for (; k + PF < cnt; k += PF) group(std::true_type{}, k);
  group(std::false_type{}, k);  // cnt is a multiple of PF
}

template <typename E, int TC, bool CT, int PF, bool VEC, int AK = -1>
static hipError_t launch_pw_t(const PwArgs& a, int cus, hipStream_t s) {
  // persistent: one workgroup per resident slot (an uneven last round measured
  // faster than fewer workgroups with equal shares)
  static std::atomic<int> per_cu{0};
  int r = per_cu.load(std::memory_order_relaxed);
  if (r == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&r, pointwise_f16_kernel<E, TC, CT, PF, VEC, AK>, 256, 0) !=
            hipSuccess || r < 1)
      r = 1;
    per_cu.store(r, std::memory_order_relaxed);
  }
  long long grid = std::min<long long>((long long)r * cus, a.ntiles);
  if (grid < a.ntiles) grid = std::max<long long>(8, grid & ~7LL);  // whole XCD rounds
  hipLaunchKernelGGL((pointwise_f16_kernel<E, TC, CT, PF, VEC, AK>), dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename E, int TC, bool CT, int PF>
static hipError_t launch_pw_v(const PwArgs& a, int cus, hipStream_t s) {
  // ReLU and identity, the common cases, with the activation fixed at compile time
  if (a.vec && a.act == 1) return launch_pw_t<E, TC, CT, PF, true, 1>(a, cus, s);
  if (a.vec && a.act == 0) return launch_pw_t<E, TC, CT, PF, true, 0>(a, cus, s);
  return a.vec ? launch_pw_t<E, TC, CT, PF, true>(a, cus, s) : launch_pw_t<E, TC, CT, PF, false>(a, cus, s);
}

template <typename E>
static hipError_t launch_pointwise_t(const PwArgs& a, int cus, hipStream_t s) {
  // One work item in flight: deeper prefetch (2 or 4 items, fewer resident
  // workgroups) measured slower on the 1x1 and ConvTranspose workload shapes.
  if (a.ct) return a.tc == 64 ? launch_pw_v<E, 64, true, 1>(a, cus, s) : launch_pw_v<E, 128, true, 1>(a, cus, s);
  return a.tc == 64 ? launch_pw_v<E, 64, false, 1>(a, cus, s) : launch_pw_v<E, 128, false, 1>(a, cus, s);
}

hipError_t launch_pointwise(Dtype dt, const PwArgs& a, int cus, hipStream_t s) {
  return dt == BF16 ? launch_pointwise_t<__bf16>(a, cus, s) : launch_pointwise_t<_Float16>(a, cus, s);
}

}  // namespace convfwd
