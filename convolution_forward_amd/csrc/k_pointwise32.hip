// Pointwise (1x1, stride 1, no padding, one group) convolution in float32 as a
// GEMM on the input as it lies ("Convolution, pooling and resize", "Variants":
// the 1x1 case multiplies the weight matrix by x without gathering;
// "Convolutions", section 2.4: a per-pixel linear map), gfx950:
//
//   y[n, co, p] = act( sum_ci w[co, ci] * x[n, ci, p] + bias[co] + res[n, co, p] )
//
//  * The pixels of all images form one axis; a tile is 64 consecutive pixels of
//    it (planes of whole float4 groups, so a group never straddles two images)
//    x 80 output channels.  Input channels are consumed in chunks of 64, double
//    buffered in LDS and prefetched through registers one chunk ahead.
//  * v_mfma_f32_16x16x4_f32 (float32 products and sums): A = weights (16 output
//    channels x 4 k), B = x (4 k x 16 pixels).  Eight waves, two per SIMD: wave
//    w owns pixels 16 (w % 4) .. + 15 of the tile, all five 16-channel blocks,
//    and half h = w / 4 of every chunk; the two halves' sums are added at the
//    end (first half + second half).  Within a half, lane group g (lanes
//    16g..16g+15) feeds channels 32h + 8g .. + 7 to the 8 k-steps in turn, so a
//    lane's A values of four k-steps are one 16-byte LDS read.
//  * LDS layout: x rows of 64 floats rotated by 16 columns per lane group, w rows
//    padded to 68 floats, so that every fragment read hits distinct banks.
// Per output: the sum of each half runs over the chunks in order, step s of a
// half adding channels 32h + s, 32h + 8 + s, 32h + 16 + s, 32h + 24 + s (MFMA
// internal order); then first half + second half.
#include <algorithm>
#include <type_traits>

#include "epilogue.h"
#include "internal.h"

namespace convfwd {

namespace {

typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int P32_TP = 64;               // pixels per tile
constexpr int P32_TC = 80;               // output channels per tile (5 blocks)
constexpr int P32_KC = 64;               // input channels per chunk
constexpr int P32_XP = 64;               // LDS floats per channel row of x
constexpr int P32_WP = 68;               // LDS floats per output-channel row of w
constexpr int P32_XF = P32_KC * P32_XP;  // floats of one x stage
constexpr int P32_WF = P32_TC * P32_WP;  // floats of one w stage
constexpr int P32_NT = 512;              // threads: 8 waves, 2 per SIMD
constexpr int P32_NX = P32_KC * P32_TP / 4 / P32_NT;                 // x float4 per thread (2)
constexpr int P32_NW = (P32_TC * P32_KC / 4 + P32_NT - 1) / P32_NT;  // w float4 per thread (3)

// column of pixel px in the LDS row of chunk channel k: rows of the four lane
// groups (channels 8g .. 8g + 7 of each half chunk) are rotated by 16 columns
// against each other, so the groups' reads of one step hit different banks
__device__ __forceinline__ int xcol(int k, int px) { return (px + 16 * ((k >> 3) & 3)) & 63; }

// Raw buffer descriptor (gfx9 format word 0x00020000) over [p, p + bytes), its
// operands made wave-uniform.  The per-lane offset is range checked: past the
// range a load reads 0 and a store is dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t p32_rsrc(const void* p, int bytes) {
  const unsigned long long v = reinterpret_cast<unsigned long long>(p);
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((unsigned long long)hi << 32) | lo),
                                           (short)0, __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
constexpr int P32_OOB = (int)0x80000000;  // a byte offset past every descriptor's range

}  // namespace

// VEC: x and w 16-byte aligned (planes and weight rows of whole float4 groups
// are guaranteed by the planner); otherwise element loads.
template <bool VEC, int AK = -1>
__global__ __launch_bounds__(P32_NT) void pointwise_f32_kernel(const PwArgs a) {
  __shared__ __attribute__((aligned(16))) float smem[2 * (P32_XF + P32_WF) + P32_TC];
  float* bsm = smem + 2 * (P32_XF + P32_WF);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ct = blockIdx.x % a.n_ct, pt = blockIdx.x / a.n_ct;
  const int co0 = ct * P32_TC;
  const long long P0 = (long long)pt * P32_TP;  // first pixel of the flattened axis
  const long long npix = (long long)a.n * a.hw;
  const float* __restrict__ x = static_cast<const float*>(a.x);
  const float* __restrict__ w = static_cast<const float*>(a.wt);
  const float* bias = static_cast<const float*>(a.bias);
  const float* res = static_cast<const float*>(a.res);
  float* y = static_cast<float*>(a.y);

  // load items: x float4 (channel k = q / 16, pixels 4 (q % 16) ..), w float4
  // (output channel m = q / 16, channels 4 (q % 16) ..); clamped addresses, so
  // every load is unconditional; values past the ranges are zeroed when staged
  long long xoff[P32_NX];
#pragma unroll
  for (int i = 0; i < P32_NX; ++i) {
    const int q = tid + P32_NT * i;
    const long long P = min(P0 + 4 * (q & 15), npix - 4);
    const long long img = mdiv((unsigned)P, a.mg_hw);  // P < 2^31
    xoff[i] = img * a.c_in * a.hw + (P - img * a.hw);
  }
  // vector path: byte offsets through buffer descriptors (tensors below 2 GiB),
  // a per-thread part computed once plus the chunk's; channels past c_in and
  // rows past c_out read other data or 0 and are zeroed when staged
  const __amdgpu_buffer_rsrc_t x_rsrc = p32_rsrc(x, (int)min(npix * a.c_in * 4, 2147483647LL));
  const __amdgpu_buffer_rsrc_t w_rsrc = p32_rsrc(w, a.c_out * a.c_in * 4);
  int xl[P32_NX], wl[P32_NW];
#pragma unroll
  for (int i = 0; i < P32_NX; ++i) xl[i] = 4 * (int)(xoff[i] + (long long)((tid + P32_NT * i) >> 4) * a.hw);
#pragma unroll
  for (int i = 0; i < P32_NW; ++i) {
    const int q = min(tid + P32_NT * i, P32_TC * P32_KC / 4 - 1);
    wl[i] = 4 * ((co0 + (q >> 4)) * a.c_in + 4 * (q & 15));
  }
  floatx4_t xr[P32_NX], wr[P32_NW];
  auto load = [&](int c0) __attribute__((always_inline)) {
    if constexpr (VEC) {
#pragma unroll
      for (int i = 0; i < P32_NX; ++i)
        xr[i] = __builtin_bit_cast(floatx4_t, __builtin_amdgcn_raw_buffer_load_b128(x_rsrc, xl[i] + 4 * c0 * a.hw, 0, 0));
#pragma unroll
      for (int i = 0; i < P32_NW; ++i)
        wr[i] = __builtin_bit_cast(floatx4_t, __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, wl[i] + 4 * c0, 0, 0));
      return;
    }
#pragma unroll
    for (int i = 0; i < P32_NX; ++i) {
      const int q = tid + P32_NT * i;
      const int k = min(c0 + (q >> 4), a.c_in - 1);
      const float* src = x + xoff[i] + (long long)k * a.hw;
      if constexpr (VEC) {
        xr[i] = *reinterpret_cast<const floatx4_t*>(src);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) xr[i][j] = src[j];
      }
    }
#pragma unroll
    for (int i = 0; i < P32_NW; ++i) {
      const int q = min(tid + P32_NT * i, P32_TC * P32_KC / 4 - 1);
      const int m = min(co0 + (q >> 4), a.c_out - 1);
      const int k = min(c0 + 4 * (q & 15), a.c_in - 4);  // c_in % 4 == 0
      const float* src = w + (long long)m * a.c_in + k;
      if constexpr (VEC) {
        wr[i] = *reinterpret_cast<const floatx4_t*>(src);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) wr[i][j] = src[j];
      }
    }
  };
  auto stage = [&](int buf, int c0) __attribute__((always_inline)) {
    float* xs = smem + buf * (P32_XF + P32_WF);
    float* ws = xs + P32_XF;
#pragma unroll
    for (int i = 0; i < P32_NX; ++i) {
      const int q = tid + P32_NT * i;
      const int k = q >> 4, px = 4 * (q & 15);
      const bool ok = c0 + k < a.c_in && P0 + px < npix;  // whole float4 groups
      *reinterpret_cast<floatx4_t*>(xs + k * P32_XP + xcol(k, px)) = ok ? xr[i] : floatx4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int i = 0; i < P32_NW; ++i) {
      const int q = tid + P32_NT * i;
      if (P32_NT * (i + 1) <= P32_TC * P32_KC / 4 || q < P32_TC * P32_KC / 4) {  // uniform per wave
        const int m = q >> 4, k = 4 * (q & 15);
        const bool ok = co0 + m < a.c_out && c0 + k < a.c_in;
        *reinterpret_cast<floatx4_t*>(ws + m * P32_WP + k) = ok ? wr[i] : floatx4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
  };

  floatx4_t acc[5];
#pragma unroll
  for (int cb = 0; cb < 5; ++cb) acc[cb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  const int lg = lane >> 4, lc = lane & 15;
  const int pb = wave & 3, kh = wave >> 2;  // pixel block, half of each chunk
  auto compute = [&](int buf) __attribute__((always_inline)) {
    const float* xs = smem + buf * (P32_XF + P32_WF);
    const float* ws = xs + P32_XF;
#pragma unroll
    for (int s4 = 0; s4 < 2; ++s4) {  // four k-steps per 16-byte A read
      floatx4_t af[5];
#pragma unroll
      for (int cb = 0; cb < 5; ++cb)
        af[cb] = *reinterpret_cast<const floatx4_t*>(ws + (16 * cb + lc) * P32_WP + 32 * kh + 8 * lg + 4 * s4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int k = 32 * kh + 8 * lg + 4 * s4 + j;
        const float bf = xs[k * P32_XP + xcol(k, 16 * pb + lc)];
#pragma unroll
        for (int cb = 0; cb < 5; ++cb)
          acc[cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[cb][j], bf, acc[cb], 0, 0, 0);
      }
    }
  };

  // without a bias the slot holds -0.0, whose addition is exact for every
  // value (a zero keeps its sign)
  if (tid < P32_TC) bsm[tid] = bias ? bias[min(co0 + tid, a.c_out - 1)] : -0.0f;
  const int nch = a.nchunks;
  load(0);
  stage(0, 0);
  __syncthreads();
  for (int c = 0; c < nch; ++c) {
    const int buf = c & 1;
    if (c + 1 < nch) load((c + 1) * P32_KC);  // uniform
    compute(buf);
    if (c + 1 < nch) stage(buf ^ 1, (c + 1) * P32_KC);
    __syncthreads();
  }

  // the upper waves' partial sums (second half of every chunk) go through LDS
  // to the lower waves, which add them (lower + upper) and run the epilogue:
  // lane l holds pixel 16 pb + l % 16 and output channels 16 cb + 4 (l / 16) + i
  floatx4_t* part = reinterpret_cast<floatx4_t*>(smem);
  if (kh == 1) {
#pragma unroll
    for (int cb = 0; cb < 5; ++cb) part[(pb * 5 + cb) * 64 + lane] = acc[cb];
  }
  __syncthreads();
  if (kh == 1) return;
#pragma unroll
  for (int cb = 0; cb < 5; ++cb) acc[cb] = acc[cb] + part[(pb * 5 + cb) * 64 + lane];
  const long long P = P0 + 16 * pb + lc;
  if constexpr (VEC) {
    // branch-free: outputs past the pixels or channels get an offset past the
    // descriptors' range (their residual reads 0, their stores are dropped)
    const __amdgpu_buffer_rsrc_t y_rsrc = p32_rsrc(y, (int)min(npix * a.c_out * 4, 2147483647LL));
    const __amdgpu_buffer_rsrc_t r_rsrc = p32_rsrc(res ? res : x, res ? (int)min(npix * a.c_out * 4, 2147483647LL) : 0);
    const int Pc = (int)min(P, npix - 1);
    const int img = (int)mdiv((unsigned)Pc, a.mg_hw);
    const int obase = img * a.c_out * a.hw + (Pc - img * a.hw);
    auto off = [&](int m) __attribute__((always_inline)) {
      return P < npix && co0 + m < a.c_out ? 4 * (obase + (co0 + m) * a.hw) : P32_OOB;
    };
    float v[20];
#pragma unroll
    for (int cb = 0; cb < 5; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * cb + 4 * lg + i;
        float t = acc[cb][i] + bsm[m];  // the slot holds -0.0 without a bias
        if (res) t = t + __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r_rsrc, off(m), 0, 0));
        v[4 * cb + i] = t;
      }
    act_apply<AK>(v, a.act, a.alpha, a.beta);
#pragma unroll
    for (int cb = 0; cb < 5; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i)  // nontemporal: the output is not read back
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v[4 * cb + i]), y_rsrc,
                                              off(16 * cb + 4 * lg + i), 0, 2);
  } else if (P < npix) {
    const long long img = mdiv((unsigned)P, a.mg_hw), pp = P - img * a.hw;
    const long long obase = img * a.c_out * a.hw + pp;
    float v[20];
#pragma unroll
    for (int cb = 0; cb < 5; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * cb + 4 * lg + i;
        const float bv = bsm[m];  // read outside the condition: no branch per value
        float t = acc[cb][i];
        t = bias ? t + bv : t;
        if (res) t = t + res[obase + (long long)min(co0 + m, a.c_out - 1) * a.hw];
        v[4 * cb + i] = t;
      }
    act_apply<AK>(v, a.act, a.alpha, a.beta);
#pragma unroll
    for (int cb = 0; cb < 5; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * cb + 4 * lg + i;
        if (co0 + m < a.c_out) store_out(y + obase + (long long)(co0 + m) * a.hw, v[4 * cb + i]);
      }
  }
}

// Strip kernel for layers whose pixel axis is short (one round of the tiled
// kernel above leaves CUs idle and each tile waits on its loads): a tile is 16
// output channels x 256 consecutive pixels of the flattened axis, and the input
// goes from memory straight into registers, D k-steps ahead, without LDS.
//
//  * Four waves, wave w owns pixels 64 w .. 64 w + 63 of the tile as 16 groups
//    of 4 consecutive pixels (a group never straddles two images: h*w % 4 == 0).
//  * v_mfma_f32_16x16x4_f32 with A = weights (16 output channels x 4 k) and
//    B = x (4 k x 16 pixel groups).  Lane group g (lanes 16g .. 16g + 15) feeds
//    channels g c_in/4 .. (g + 1) c_in/4 - 1 to the k-steps in turn, so step s
//    multiplies channels s, c_in/4 + s, c_in/2 + s and 3 c_in/4 + s.  A lane loads
//    the 4 pixels of its group as one 16-byte vector; element j of that vector
//    is the B operand of accumulator set j (pixel 4 n + j), so the four sets
//    share every A value and cover 64 pixels.
//  * A lane's weights for 4 consecutive steps are one 16-byte load (w[co][ci]
//    rows as they lie).  D steps of x and D/4 weight vectors are in flight per
//    wave; each step refills the registers it has consumed with the step D
//    later, and the last block of D steps issues no loads.
//  * The channel tiles of one pixel range read the same x and run side by side
//    on one XCD.  Tile ct takes the k-steps in a rotated order, starting at step
//    (D ct) mod (c_in / 4) and wrapping round, so a piece of x is fetched from
//    HBM by one tile while the others find it in L2 later; taken in the same
//    order, all of them waited on the same misses.
//  * Epilogue: set j holds pixel 4 n + j of output channels 4 g + r, so a lane
//    finishes 4 consecutive pixels per channel: one 16-byte residual load and
//    one 16-byte store each.
// Per output: the k-steps in the tile's rotated order, each adding its 4
// channels in the MFMA's internal order.
constexpr int PS_TP = 256;  // pixels per tile
constexpr int PS_TC = 16;   // output channels per tile

template <bool VEC, int D, int AK = -1>
__global__ __launch_bounds__(256) void pointwise_f32_strip_kernel(const PwArgs a) {
  static_assert(D % 4 == 0, "weights come 4 steps per load");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int L = xcd_logical(blockIdx.x, a.ntiles);  // channel tiles of a pixel range share an L2
  const int pt = L / a.n_ct, ct = L - pt * a.n_ct;
  const int co0 = ct * PS_TC;
  const int g = lane >> 4, c16 = lane & 15;
  const int kq = a.c_in >> 2;  // k-steps (channels per lane group), a multiple of 4
  const long long npix = (long long)a.n * a.hw;
  const long long P = (long long)pt * PS_TP + 64 * wave + 4 * c16;  // the lane's first pixel
  const int Pc = (int)min(P, npix - 4);                              // loads stay in x
  const int img = (int)mdiv((unsigned)Pc, a.mg_hw);
  const int hwo = Pc - img * a.hw;
  const __amdgpu_buffer_rsrc_t x_rsrc = p32_rsrc(a.x, (int)(npix * a.c_in * 4));
  const __amdgpu_buffer_rsrc_t w_rsrc = p32_rsrc(a.wt, a.c_out * a.c_in * 4);
  const int xl = 4 * (img * a.c_in * a.hw + g * kq * a.hw + hwo);
  const int wl = 4 * (min(co0 + c16, a.c_out - 1) * a.c_in + g * kq);
  const int xstep = 4 * a.hw;  // bytes from one channel plane to the next

  // k-step s of x, taken at rotated position rotk(s) (clamped to the last step
  // first: a refill past the end rereads it)
  // the channel tiles of one pixel range start their k-steps D apart (mod kq)
  const int rot = (ct * D) % kq;
  auto rotk = [&](int s) __attribute__((always_inline)) {
    const int r = s + rot;
    return r >= kq ? r - kq : r;
  };
  auto ldx = [&](int s) __attribute__((always_inline)) {
    const int so = rotk(min(s, kq - 1)) * xstep;
    floatx4_t v;
    if constexpr (VEC) {
      v = __builtin_bit_cast(floatx4_t, __builtin_amdgcn_raw_buffer_load_b128(x_rsrc, xl, so, 0));
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        v[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(x_rsrc, xl + 4 * j, so, 0));
    }
    return v;
  };
  // weights of steps s .. s + 3 (s a multiple of 4, clamped likewise; rot and
  // kq are multiples of 4, so the four stay consecutive after the rotation)
  auto ldw = [&](int s) __attribute__((always_inline)) {
    const int so = 4 * rotk(min(s, kq - 4));
    floatx4_t v;
    if constexpr (VEC) {
      v = __builtin_bit_cast(floatx4_t, __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, wl, so, 0));
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        v[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(w_rsrc, wl + 4 * j, so, 0));
    }
    return v;
  };

  floatx4_t acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  floatx4_t bq[D], aq[D / 4];
#pragma unroll
  for (int i = 0; i < D; ++i) {  // in the order they are consumed
    if (i % 4 == 0) aq[i / 4] = ldw(i);
    bq[i] = ldx(i);
  }
  // D steps from s0; REFILL: load step s + D into the registers step s frees.
  // Steps at or past kq multiply a zero weight (their x is a clamped reread).
  auto block = [&](int s0, auto refill) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < D; ++i) {
      const int s = s0 + i;
      const float av = s < kq ? aq[i / 4][i % 4] : 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bq[i][j], acc[j], 0, 0, 0);
      if constexpr (decltype(refill)::value) {
        bq[i] = ldx(s + D);
        if (i % 4 == 3) aq[i / 4] = ldw(s - 3 + D);  // its four steps are done
      }
      // keep each step's loads among its own multiplies: the loads then leave in
      // the order they are consumed, and each wait counts only the later ones
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  const int nb = (kq + D - 1) / D;
  for (int b = 0; b + 1 < nb; ++b) block(b * D, std::true_type{});

  // outputs: channel co0 + 4 g + r, pixels P .. P + 3 (accumulator set j = pixel P + j);
  // out-of-range ones get an offset past the descriptors (residual reads 0, store dropped)
  const bool pv = P < npix;
  const __amdgpu_buffer_rsrc_t y_rsrc = p32_rsrc(a.y, (int)(npix * a.c_out * 4));
  const float* res = static_cast<const float*>(a.res);
  const __amdgpu_buffer_rsrc_t r_rsrc = p32_rsrc(res ? a.res : a.y, res ? (int)(npix * a.c_out * 4) : 0);
  const float* bias = static_cast<const float*>(a.bias);
  int off[4];
  float bv[4];
  floatx4_t rv[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int co = co0 + 4 * g + r;
    off[r] = pv && co < a.c_out ? 4 * (img * a.c_out * a.hw + co * a.hw + hwo) : P32_OOB;
    bv[r] = bias ? bias[min(co, a.c_out - 1)] : -0.0f;  // -0.0 adds exactly
  }
  // the residual is read during the last block's multiplications
  if (res) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (VEC) {
        rv[r] = __builtin_bit_cast(floatx4_t, __builtin_amdgcn_raw_buffer_load_b128(r_rsrc, off[r], 0, 0));
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          rv[r][j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r_rsrc, off[r] + 4 * j, 0, 0));
      }
    }
  }
  block((nb - 1) * D, std::false_type{});
  float v[16];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float t = acc[j][r] + bv[r];
      if (res) t = t + rv[r][j];
      v[4 * r + j] = t;
    }
  act_apply<AK>(v, a.act, a.alpha, a.beta);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if constexpr (VEC) {
      const floatx4_t o{v[4 * r], v[4 * r + 1], v[4 * r + 2], v[4 * r + 3]};
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, o), y_rsrc, off[r], 0, 2);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v[4 * r + j]), y_rsrc,
                                              off[r] == P32_OOB ? P32_OOB : off[r] + 4 * j, 0, 2);
    }
  }
}

template <bool VEC, int D>
static void launch_strip_act(const PwArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)a.ntiles);
  if (a.act == 0) hipLaunchKernelGGL((pointwise_f32_strip_kernel<VEC, D, 0>), grid, dim3(256), 0, s, a);
  else if (a.act == 1) hipLaunchKernelGGL((pointwise_f32_strip_kernel<VEC, D, 1>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((pointwise_f32_strip_kernel<VEC, D>), grid, dim3(256), 0, s, a);
}

hipError_t launch_pointwise_f32_strip(const PwArgs& a, hipStream_t s) {
  // 12 k-steps in flight (deeper windows measured slower: the bytes a CU pulls
  // from L2, not the latency, bound the strips)
  if (a.vec) launch_strip_act<true, 12>(a, s);
  else launch_strip_act<false, 12>(a, s);
  return hipGetLastError();
}

hipError_t launch_pointwise_f32(const PwArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((long long)a.n_pt * a.n_ct));
  // identity and ReLU with the activation fixed at compile time on the vector path
  if (a.vec && a.act == 0) hipLaunchKernelGGL((pointwise_f32_kernel<true, 0>), grid, dim3(P32_NT), 0, s, a);
  else if (a.vec && a.act == 1) hipLaunchKernelGGL((pointwise_f32_kernel<true, 1>), grid, dim3(P32_NT), 0, s, a);
  else if (a.vec) hipLaunchKernelGGL((pointwise_f32_kernel<true>), grid, dim3(P32_NT), 0, s, a);
  else hipLaunchKernelGGL((pointwise_f32_kernel<false>), grid, dim3(P32_NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace convfwd
