// Pointwise (1x1, stride 1, no padding, one group) convolution as a GEMM on the
// input as it lies ("Convolution, pooling and resize", "Variants": the 1x1 case
// multiplies the weight matrix by x without any gathering; "Convolutions",
// section 2.4: a 1x1 convolution is a per-pixel linear map), gfx950, float16
// operands, float32 accumulation:
//
//   y[n, co, p] = act( sum_ci w[co, ci] * x[n, ci, p]  + bias[co] + res[n, co, p] )
//
// for every image n and pixel p of the H*W plane.
//
//  * Tile: 128 pixels of one image x 128 output channels; the input channels are
//    consumed in chunks of 64.  Four waves, each 64 pixels x 64 channels as
//    4 x 4 MFMA blocks of v_mfma_f32_16x16x32_f16 (A = x transposed: pixel rows,
//    channel k; B = w transposed: channel k, output-channel columns).
//  * x is read as it lies: a thread loads 4 consecutive pixels of 8 channels
//    (8 bytes per channel plane) and regroups them in registers into 4 channel
//    octets, stored pixel-major in LDS (16 bytes per pixel and octet, swizzled so
//    the 16 pixels of an MFMA block hit distinct banks).  Weight rows (64
//    channels, 128 contiguous bytes per output channel) are copied with 16-byte
//    reads into rows padded to 144 bytes.
//  * Persistent workgroups walk (tile, chunk) pairs; the next pair's operands
//    are loaded into registers while the current chunk multiplies.
//  * Epilogue: a lane holds 4 consecutive pixels of one output channel; bias,
//    residual and activation run in float32 on them, the float16 results go to
//    an LDS output tile [channel][pixel] in the freed staging area, and whole
//    256-byte rows of it leave with 16-byte stores.
// Per output the sum runs over the channels in increasing order in steps of 32
// (the MFMA's internal order within a step).
#include <algorithm>
#include <atomic>

#include "epilogue.h"
#include "internal.h"

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
constexpr int PW_WROW = PW_KC * 2 + 16;    // padded LDS bytes per output channel
constexpr int PW_OROW = PW_TP * 2 + 16;    // LDS bytes per output-tile row (float16)

// octet slot at pixel row p: the 16 rows of an MFMA block land on distinct banks
__device__ __forceinline__ int pw_slot(int p, int o) { return o ^ ((p >> 1) & 7); }

}  // namespace

template <bool O16, int PW_TC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(PW_TC == 128 ? 3 : 4)))
void pointwise_f16_kernel(const PwArgs a) {
  constexpr int PW_WBYTES = PW_TC * PW_WROW;
  constexpr int PW_NW = PW_TC * (PW_KC / 8) / 256;  // 16-byte weight vectors per thread
  static_assert(PW_TC * PW_OROW <= PW_XBYTES + PW_WBYTES, "output tile reuses the staging area");
  constexpr int WCN = PW_TC / 64;  // waves along the output channels (64 each)
  constexpr int WPN = 4 / WCN;     // waves along the pixels
  constexpr int PB = PW_TP / WPN / 16;  // 16-pixel MFMA blocks per wave
  __shared__ __attribute__((aligned(16))) unsigned char smem[PW_XBYTES + PW_WBYTES + PW_TC * 4];
  unsigned char* xs = smem;
  unsigned char* ws = smem + PW_XBYTES;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hw = a.hw;
  const _Float16* __restrict__ x = static_cast<const _Float16*>(a.x);
  const _Float16* __restrict__ w = static_cast<const _Float16*>(a.wt);

  // staging item of this thread: channel octet o, 4-pixel group g of the tile
  const int so = tid >> 5, sg = tid & 31;

  u32x2_t xr[8];       // 8 channels x 4 pixels
  u32x4_t wr[PW_NW];   // weight vectors
  _Float16 br = 0.0f;  // bias of tile channel tid (tid < 128), converted when staged
  float* bsm = reinterpret_cast<float*>(smem + PW_XBYTES + PW_WBYTES);

  // work item = tile * nchunks + chunk; tile = (image, pixel tile, channel tile),
  // channel tile fastest
  auto decode = [&](int item, int& n, int& p0, int& co0, int& c0) __attribute__((always_inline)) {
    const int t = item / a.nchunks;
    c0 = (item - t * a.nchunks) * PW_KC;
    const int ct = t % a.n_ct;
    const int r = t / a.n_ct;
    const int pt = r % a.n_pt;
    n = r / a.n_pt;
    p0 = pt * PW_TP;
    co0 = ct * PW_TC;
  };
  auto load = [&](int item) __attribute__((always_inline)) {
    int n, p0, co0, c0;
    decode(item, n, p0, co0, c0);
    // x: channels c0 + 8 so + e, pixels p0 + 4 sg .. + 3 (clamped into the plane
    // and the channel range; out-of-range values are zeroed when staged)
    const int px = min(p0 + 4 * sg, hw - 4);
    const _Float16* xb = x + ((long long)n * a.c_in) * hw + px;
    if (a.xvec) {  // uniform: x 8-byte aligned
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int ci = min(c0 + 8 * so + e, a.c_in - 1);
        xr[e] = *reinterpret_cast<const u32x2_t*>(xb + (long long)ci * hw);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int ci = min(c0 + 8 * so + e, a.c_in - 1);
        half4_t h;
#pragma unroll
        for (int j = 0; j < 4; ++j) h[j] = xb[(long long)ci * hw + j];
        xr[e] = __builtin_bit_cast(u32x2_t, h);
      }
    }
    if (a.bias) br = static_cast<const _Float16*>(a.bias)[min(co0 + (tid % PW_TC), a.c_out - 1)];
    // w: row co0 + q / 8, 16-byte piece q % 8 of the chunk
#pragma unroll
    for (int i = 0; i < PW_NW; ++i) {
      const int q = tid + 256 * i;
      const int co = min(co0 + (q >> 3), a.c_out - 1);
      const int ci = min(c0 + 8 * (q & 7), a.c_in - 8);  // c_in % 8 == 0
      const _Float16* src = w + (long long)co * a.c_in + ci;
      if (a.wvec) {  // uniform: w 16-byte aligned
        wr[i] = *reinterpret_cast<const u32x4_t*>(src);
      } else {
        half8_t h;
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = src[e];
        wr[i] = __builtin_bit_cast(u32x4_t, h);
      }
    }
  };
  auto stage = [&](int item) __attribute__((always_inline)) {
    int n, p0, co0, c0;
    decode(item, n, p0, co0, c0);
    const int cvalid = a.c_in - (c0 + 8 * so);  // channels of this octet that exist
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      half8_t v;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        v[e] = e < cvalid ? __builtin_bit_cast(half4_t, xr[e])[j] : (_Float16)0.0f;
      const int p = 4 * sg + j;
      *reinterpret_cast<half8_t*>(xs + p * 128 + 16 * pw_slot(p, so)) = v;
    }
    if (tid < PW_TC) bsm[tid] = (float)br;
#pragma unroll
    for (int i = 0; i < PW_NW; ++i) {
      const int q = tid + 256 * i;
      const bool ok = c0 + 8 * (q & 7) < a.c_in;  // whole octets: c_in % 8 == 0
      *reinterpret_cast<u32x4_t*>(ws + (q >> 3) * PW_WROW + 16 * (q & 7)) =
          ok ? wr[i] : u32x4_t{0, 0, 0, 0};
    }
  };

  const int wp = wave % WPN, wc = wave / WPN;  // wave's pixel and channel ranges
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
          acc[pb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[pb], bf[cb], acc[pb][cb], 0, 0, 0);
    }
  };

  const void* bias = a.bias;
  const _Float16* res = static_cast<const _Float16*>(a.res);
  _Float16* y = static_cast<_Float16*>(a.y);
  // Epilogue.  Phase 1, per lane from the accumulators: bias, residual and
  // activation in float32, rounded to float16 into the LDS output tile
  // [channel][pixel] (which reuses the staging area).  Phase 2: full rows of the
  // tile leave with 16-byte stores.  Every residual read happens in phase 1,
  // before the barrier that precedes any store (y may alias the residual).
  auto epilogue = [&](int item) __attribute__((always_inline)) {
    int n, p0, co0, c0;
    decode(item, n, p0, co0, c0);
    const int pl0 = 16 * PB * wp + 4 * (lane >> 4);  // tile pixel of the lane's first value
    const int cl0 = 64 * wc + (lane & 15);      // tile channel of the lane's block 0
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
      if (res) {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          const int p = min(p0 + pl0 + 16 * pb, hw - 4);
          const int co = min(co0 + cl0 + 16 * cb, a.c_out - 1);
          const _Float16* src = res + ((long long)n * a.c_out + co) * hw + p;
          half4_t h;
          if (a.ovec) {  // uniform: y and residual 8-byte aligned
            h = __builtin_bit_cast(half4_t, *reinterpret_cast<const u32x2_t*>(src));
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) h[i] = src[i];
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) v[4 * cb + i] = v[4 * cb + i] + (float)h[i];
        }
      }
      act_array(v, a.act, a.alpha, a.beta);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        half4_t h;
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = (_Float16)v[4 * cb + i];
        *reinterpret_cast<half4_t*>(smem + (cl0 + 16 * cb) * PW_OROW + 2 * (pl0 + 16 * pb)) = h;
      }
    }
#pragma unroll
    for (int i = 0; i < PB; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    __syncthreads();
    // phase 2: 128 rows of 16 vectors of 8 pixels
    const int pvalid = min(PW_TP, hw - p0);  // a multiple of 4 (of 8 when O16)
    if constexpr (O16) {
      // vectors past the tile's valid rows or pixels repeat the last valid vector
      // of the tile (same value, same address): the store count is fixed, so
      // the wait before the next staging does not include these stores
      const int rlast = min(PW_TC, a.c_out - co0) - 1;
#pragma unroll
      for (int k = 0; k < PW_TC * PW_TP / 8 / 256; ++k) {
        const int q = tid + 256 * k;
        const int row = min(q >> 4, rlast), px = min(8 * (q & 15), pvalid - 8);
        const u32x4_t d = *reinterpret_cast<const u32x4_t*>(smem + row * PW_OROW + 2 * px);
        *reinterpret_cast<u32x4_t*>(y + ((long long)n * a.c_out + co0 + row) * hw + p0 + px) = d;
      }
    } else {
#pragma unroll 1
      for (int k = 0; k < PW_TC * PW_TP / 8 / 256; ++k) {
        const int q = tid + 256 * k;
        const int row = q >> 4, px = 8 * (q & 15);
        const int co = co0 + row;
        const u32x4_t d = *reinterpret_cast<const u32x4_t*>(smem + row * PW_OROW + 2 * px);
        _Float16* dst = y + ((long long)n * a.c_out + co) * hw + p0 + px;
        if (co < a.c_out && px < pvalid) {
          if (a.ovec) {
            *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{d[0], d[1]};
            if (px + 8 <= pvalid) *reinterpret_cast<u32x2_t*>(dst + 4) = u32x2_t{d[2], d[3]};
          } else {
            const half8_t h = __builtin_bit_cast(half8_t, d);
            const int cnt = min(8, pvalid - px);
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (e < cnt) dst[e] = h[e];
          }
        }
      }
    }
    __syncthreads();  // the next staging overwrites the output tile
  };

  const int nitems = a.ntiles * a.nchunks;
  int item = blockIdx.x * a.nchunks;  // workgroup b takes tiles b, b + G, ...
  const int stride = gridDim.x * a.nchunks;
  if (item < nitems) load(item);
  while (item < nitems) {
    stage(item);
    __syncthreads();
    // next work item: the next chunk of this tile, or chunk 0 of the next tile
    const bool last_chunk = (item % a.nchunks) == a.nchunks - 1;
    const int next = last_chunk ? item + stride - (a.nchunks - 1) : item + 1;
    if (next < nitems) load(next);  // uniform
    compute();
    __syncthreads();
    if (last_chunk) epilogue(item);
    item = next;
  }
}

template <bool O16, int TC>
static hipError_t launch_pw_t(const PwArgs& a, int cus, hipStream_t s) {
  // persistent: one workgroup per resident slot (an uneven last round measured
  // faster than fewer workgroups with equal shares)
  static std::atomic<int> per_cu{0};
  int r = per_cu.load(std::memory_order_relaxed);
  if (r == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&r, pointwise_f16_kernel<O16, TC>, 256, 0) !=
            hipSuccess || r < 1)
      r = 1;
    per_cu.store(r, std::memory_order_relaxed);
  }
  const int grid = (int)std::min<long long>((long long)r * cus, a.ntiles);
  hipLaunchKernelGGL((pointwise_f16_kernel<O16, TC>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_pointwise(const PwArgs& a, int cus, hipStream_t s) {
  if (a.tc == 64) return a.o16 ? launch_pw_t<true, 64>(a, cus, s) : launch_pw_t<false, 64>(a, cus, s);
  return a.o16 ? launch_pw_t<true, 128>(a, cus, s) : launch_pw_t<false, 128>(a, cus, s);
}

}  // namespace convfwd
