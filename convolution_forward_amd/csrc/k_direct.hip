// Bandwidth-bound kernels for gfx950 (VALU only, no MFMA):
//  - depthwise direct convolution ("Convolution, pooling and resize", "Variants":
//    one input channel per group, any channel multiplier, one fixed window order);
//  - the split-k reduction + epilogue (planes combined with a fixed wavefront
//    shuffle tree, then bias, residual, activation);
//  - the gathering col2im + epilogue of ConvTranspose (one thread per output
//    element, taps visited in row-major order, no atomics).
#include <mutex>
#include <type_traits>

#include "epilogue.h"
#include "internal.h"

namespace convfwd {

// ---------------------------------------------------------------------------
// Depthwise: a workgroup owns one output tile of one input plane (n, ci) and
// all `mult` output channels that read it.  The input tile plus its halo is
// staged once into LDS with zero padding (coalesced row reads), then every
// output is one f32 FMA chain over the window in (kh, kw) row-major order.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void depthwise_kernel(const DepthwiseArgs a) {
  extern __shared__ float tile[];  // tih * tiw
  const int plane = blockIdx.x;    // n * c_in + ci
  const int t = blockIdx.y;
  const int ty = t / a.tiles_w, tx = t - ty * a.tiles_w;
  const int n = plane / a.c_in, ci = plane - n * a.c_in;
  const int oh0 = ty * a.toh, ow0 = tx * a.tow;
  const int ih_base = oh0 * a.sh - a.pt, iw_base = ow0 * a.sw - a.pl;
  const T* __restrict__ xp = static_cast<const T*>(a.x) + (long long)plane * a.h * a.w;

  for (int i = threadIdx.x; i < a.tih * a.tiw; i += blockDim.x) {
    const int r = i / a.tiw, c = i - r * a.tiw;
    const int ih = ih_base + r, iw = iw_base + c;
    float v = 0.0f;
    if ((unsigned)ih < (unsigned)a.h && (unsigned)iw < (unsigned)a.w)
      v = to_f32(xp[(long long)ih * a.w + iw]);
    tile[i] = v;
  }
  __syncthreads();

  const int oh_n = min(a.toh, a.ho - oh0), ow_n = min(a.tow, a.wo - ow0);
  const T* __restrict__ wp = static_cast<const T*>(a.wt);
  const T* bias = static_cast<const T*>(a.bias);
  const T* res = static_cast<const T*>(a.res);
  T* y = static_cast<T*>(a.y);
  const int khw = a.kh * a.kw;
  for (int o = threadIdx.x; o < oh_n * ow_n; o += blockDim.x) {
    const int r = o / ow_n, c = o - r * ow_n;
    const float* src = tile + (r * a.sh) * a.tiw + c * a.sw;
    for (int j = 0; j < a.mult; ++j) {
      const int co = ci * a.mult + j;
      const T* wc = wp + (long long)co * khw;
      float acc = 0.0f;
      for (int kh = 0; kh < a.kh; ++kh)
        for (int kw = 0; kw < a.kw; ++kw)
          acc = fmaf(src[kh * a.dh * a.tiw + kw * a.dw], to_f32(wc[kh * a.kw + kw]), acc);
      const long long oidx =
          (((long long)n * a.c_out + co) * a.ho + oh0 + r) * a.wo + ow0 + c;
      y[oidx] = epilogue_one<T>(acc, bias, res, co, oidx, a.act, a.alpha, a.beta);
    }
  }
}

hipError_t launch_depthwise(Dtype dt, const DepthwiseArgs& a, hipStream_t s) {
  dim3 grid(a.n * a.c_in, a.tiles);
  const size_t lds = (size_t)a.tih * a.tiw * sizeof(float);
  if (dt == F16)
    hipLaunchKernelGGL(depthwise_kernel<_Float16>, grid, dim3(256), lds, s, a);
  else if (dt == BF16)
    hipLaunchKernelGGL(depthwise_kernel<__bf16>, grid, dim3(256), lds, s, a);
  else
    hipLaunchKernelGGL(depthwise_kernel<float>, grid, dim3(256), lds, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Depthwise, whole-plane path (dilation 1, kernel and stride fixed at compile
// time).  A persistent workgroup walks groups of P consecutive input planes
// (n, ci): P planes are one contiguous run of x, and their P * mult output
// planes one contiguous run of y.
//  * The next group's input is loaded into registers (16-byte loads in memory
//    order) while the current group is computed, so HBM reads overlap the
//    arithmetic of the previous group.
//  * The staged planes sit in zero-bordered LDS tiles; the border is written
//    once and never overwritten.
//  * A thread computes BH outputs of one output column: consecutive lanes take
//    consecutive columns, so every LDS read of the window is conflict free
//    (stride 1) or 2-way (stride 2).  Each output is one float32 FMA chain over
//    the window in (kh, kw) row-major order.
//  * Raw sums go to an LDS output tile in y's memory order; the epilogue (bias,
//    residual, activation) then runs on 4 contiguous outputs per item with
//    vector loads and stores.
// Index arithmetic divides only by launch constants, as multiply-high + shift.
// ---------------------------------------------------------------------------
constexpr int DW_NI = 4;  // 4-element input items per thread and group (P * H * W <= 4096)
constexpr int DW_NE = 4;  // 4-output epilogue items per thread and group
constexpr int DW_NW = 2;  // weights per thread and group (P * mult * K * K <= 512)

template <typename T>
struct DwVec;  // 4 elements of the operand type
template <>
struct DwVec<float> {
  typedef float4 type;
};
template <>
struct DwVec<_Float16> {
  typedef uint2 type;
};
template <>
struct DwVec<__bf16> {
  typedef uint2 type;
};

template <typename T>
__device__ __forceinline__ void dw_unpack(const typename DwVec<T>::type& v, float (&f)[4]) {
  if constexpr (sizeof(T) == 4) {
    f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w;
  } else {
    typedef T h4 __attribute__((ext_vector_type(4)));
    const h4 h = __builtin_bit_cast(h4, v);
#pragma unroll
    for (int k = 0; k < 4; ++k) f[k] = (float)h[k];
  }
}

template <typename T>
__device__ __forceinline__ typename DwVec<T>::type dw_pack(const float (&f)[4]) {
  if constexpr (sizeof(T) == 4) {
    return float4{f[0], f[1], f[2], f[3]};
  } else {
    typedef T h4 __attribute__((ext_vector_type(4)));
    h4 h;
#pragma unroll
    for (int k = 0; k < 4; ++k) h[k] = (T)f[k];
    return __builtin_bit_cast(uint2, h);
  }
}

template <typename T, int K, int S, int BH, bool RES>
__global__ __launch_bounds__(256) void depthwise_plane_kernel(const DepthwiseArgs a) {
  typedef typename DwVec<T>::type V;
  constexpr int PR = (BH - 1) * S + K;  // input rows of one thread's window column
  extern __shared__ float smem_dw[];
  const int tid = threadIdx.x;
  const int P = a.planes;
  const int hw = a.h * a.w;
  const int howo = a.ho * a.wo;
  const int mult = a.mult;
  const int nplanes = a.n * a.c_in;
  float* tile = smem_dw;           // P planes x tpp floats
  float* outt = smem_dw + a.oofs;  // P * mult * howo raw sums (16-byte aligned)
  float* wl = smem_dw + a.wofs;    // P * mult * K * K weights
  float* bl = smem_dw + a.bofs;    // 2 x P * mult bias (double buffered)
  float* sink = smem_dw + a.sofs;  // target of dead LDS writes
  const T* __restrict__ x = static_cast<const T*>(a.x);
  const T* __restrict__ wt = static_cast<const T*>(a.wt);
  const T* __restrict__ bias = static_cast<const T*>(a.bias);
  const T* res = static_cast<const T*>(a.res);
  T* y = static_cast<T*>(a.y);

  // ---- prefetched per group: input items (4 consecutive elements of the
  // group's contiguous run, one vector load each), weights and bias ----
  float xin[DW_NI][4];
  float wreg[DW_NW];
  float breg = 0.0f;
  const int mkk = mult * K * K;
  auto load = [&](int grp) __attribute__((always_inline)) {
    const int plane0 = grp * P;
    const int np = min(P, nplanes - plane0);
    const long long base = (long long)plane0 * hw;
    const int lastv = np * hw - 4;  // hw % 4 == 0: the last full vector
#pragma unroll
    for (int i = 0; i < DW_NI; ++i) {
      const int e = min(4 * (tid + 256 * i), lastv);
      dw_unpack<T>(*reinterpret_cast<const V*>(x + base + e), xin[i]);
    }
    // weights of the group's planes, indexed by each plane's channel (a group
    // may wrap from the last channel of one image to the first of the next)
#pragma unroll
    for (int i = 0; i < DW_NW; ++i) {
      const int q = min(tid + 256 * i, np * mkk - 1);
      const int pl = q / mkk, r = q - pl * mkk;
      wreg[i] = to_f32(wt[(long long)((plane0 + pl) % a.c_in) * mkk + r]);
    }
    if (bias) {
      const int q = min(tid, np * mult - 1);
      const int pl = q / mult, jm = q - pl * mult;
      breg = to_f32(bias[((plane0 + pl) % a.c_in) * mult + jm]);
    }
  };
  auto stage = [&](int grp) __attribute__((always_inline)) {
    const int cnt = min(P, nplanes - grp * P) * hw;
#pragma unroll
    for (int i = 0; i < DW_NI; ++i)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const unsigned e = 4 * (tid + 256 * i) + k;
        const unsigned pl = mdiv(e, a.mg_hw);
        const unsigned rem = e - pl * hw;
        const unsigned ih = mdiv(rem, a.mg_w);
        const unsigned iw = rem - ih * a.w;
        float* dst = (int)e < cnt ? tile + pl * a.tpp + (ih + a.pt) * a.tiw + iw + a.pl : sink;
        *dst = xin[i][k];
      }
  };

  // zero every tile once: the border (padding) is never written again
  for (int i = tid; i < P * a.tpp; i += 256) tile[i] = 0.0f;
  int grp = blockIdx.x;
  if (grp < a.ngroups) load(grp);
  __syncthreads();

  const int pu = a.nrb * a.wo;  // units (BH outputs of one column) per input plane
  for (int it = 0; grp < a.ngroups; grp += gridDim.x, ++it) {
    const int plane0 = grp * P;
    const int np = min(P, nplanes - plane0);
    stage(grp);
#pragma unroll
    for (int i = 0; i < DW_NW; ++i) {
      const int q = tid + 256 * i;
      *(q < np * mkk ? wl + q : sink) = wreg[i];
    }
    float* bcur = bl + (it & 1) * P * mult;
    *(tid < np * mult ? bcur + tid : sink) = breg;
    __syncthreads();
    if (grp + (int)gridDim.x < a.ngroups) load(grp + gridDim.x);  // prefetch (uniform)

    // ---- compute: unit = (plane, row block, output column) ----
    for (int u = tid; u < np * pu; u += 256) {
      const unsigned pl = mdiv(u, a.mg_pu);
      const unsigned r = u - pl * pu;
      const unsigned rb = mdiv(r, a.mg_wo);
      const unsigned ow = r - rb * a.wo;
      const float* src = tile + pl * a.tpp + (rb * BH * S) * a.tiw + ow * S;
      float patch[PR][K];
#pragma unroll
      for (int i = 0; i < PR; ++i)
#pragma unroll
        for (int j = 0; j < K; ++j) patch[i][j] = src[i * a.tiw + j];
      for (int jm = 0; jm < mult; ++jm) {
        const float* wv = wl + (pl * mult + jm) * K * K;
        float acc[BH];
#pragma unroll
        for (int i = 0; i < BH; ++i) acc[i] = 0.0f;
#pragma unroll
        for (int kh = 0; kh < K; ++kh)
#pragma unroll
          for (int kw = 0; kw < K; ++kw) {
            const float wk = wv[kh * K + kw];
#pragma unroll
            for (int i = 0; i < BH; ++i) acc[i] = fmaf(patch[i * S + kh][kw], wk, acc[i]);
          }
        float* o = outt + (pl * mult + jm) * howo + ow;
#pragma unroll
        for (int i = 0; i < BH; ++i) {
          const int oh = rb * BH + i;
          float* dst = oh < a.ho ? o + oh * a.wo : sink;
          *dst = acc[i];
        }
      }
    }
    __syncthreads();

    // ---- epilogue over the group's contiguous outputs ----
    const int tot = np * mult * howo;
    const long long obase = (long long)plane0 * mult * howo;
    if (a.ovec) {  // howo % 4 == 0, y / residual 16 / 8-byte aligned
      const int nq = tot / 4;
      if constexpr (RES) {
        // every residual read before any store (y may alias the residual)
        float v[DW_NE * 4];
#pragma unroll
        for (int k = 0; k < DW_NE; ++k) {
          float f[4];
          dw_unpack<T>(*reinterpret_cast<const V*>(res + obase + 4 * min(tid + 256 * k, nq - 1)), f);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[4 * k + e] = f[e];
        }
#pragma unroll
        for (int k = 0; k < DW_NE; ++k) {
          const int q = min(tid + 256 * k, nq - 1);
          const float4 s4 = *reinterpret_cast<const float4*>(outt + 4 * q);
          const float bv = bcur[mdiv(4 * q, a.mg_howo)];
          const float sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) v[4 * k + e] = (sv[e] + bv) + v[4 * k + e];
        }
        act_array(v, a.act, a.alpha, a.beta);
#pragma unroll
        for (int k = 0; k < DW_NE; ++k) {
          const int q = tid + 256 * k;
          if (q < nq) {
            const float f[4] = {v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]};
            *reinterpret_cast<V*>(y + obase + 4 * q) = dw_pack<T>(f);
          }
        }
      } else {
        for (int q = tid; q < nq; q += 256) {
          const float4 s4 = *reinterpret_cast<const float4*>(outt + 4 * q);
          const float bv = bcur[mdiv(4 * q, a.mg_howo)];
          float f[4] = {s4.x + bv, s4.y + bv, s4.z + bv, s4.w + bv};
          act_array(f, a.act, a.alpha, a.beta);
          *reinterpret_cast<V*>(y + obase + 4 * q) = dw_pack<T>(f);
        }
      }
    } else {
      if constexpr (RES) {
        float v[DW_NE * 4];
#pragma unroll
        for (int k = 0; k < DW_NE * 4; ++k) v[k] = to_f32(res[obase + min(tid + 256 * k, tot - 1)]);
#pragma unroll
        for (int k = 0; k < DW_NE * 4; ++k) {
          const int o = min(tid + 256 * k, tot - 1);
          v[k] = (outt[o] + bcur[mdiv(o, a.mg_howo)]) + v[k];
        }
        act_array(v, a.act, a.alpha, a.beta);
#pragma unroll
        for (int k = 0; k < DW_NE * 4; ++k) {
          const int o = tid + 256 * k;
          if (o < tot) store_out(y + obase + o, from_f32<T>(v[k]));
        }
      } else {
        for (int o = tid; o < tot; o += 256) {
          float f[1] = {outt[o] + bcur[mdiv(o, a.mg_howo)]};
          act_array(f, a.act, a.alpha, a.beta);
          store_out(y + obase + o, from_f32<T>(f[0]));
        }
      }
    }
    // the next group overwrites the tiles and weights only after every thread has
    // passed the barrier after the compute; the bias is double buffered
  }
}

// ---------------------------------------------------------------------------
// Depthwise, one wave per plane (planes of at most 1024 elements, at most 64
// output columns per row block).  Workgroups are single wavefronts, so nothing
// waits on other waves: each wave walks its own sequence of planes, prefetching
// the next plane into registers while it computes the current one.
//  * The plane sits in a zero-bordered LDS tile; input column 0 is placed at a
//    16-byte aligned column so a 4-element item is one LDS vector write.
//  * Lane (row block, output column) streams the PR input rows its BH outputs
//    need, reading K values per row once; row r adds to output i with tap row
//    kh = r - i * S.  Rows arrive in increasing order, so every output is still
//    one float32 FMA chain in (kh, kw) row-major order.
//  * The plane's weights are wave-uniform (scalar loads, no LDS).
//  * Raw sums go to an LDS tile in y's memory order; the epilogue runs on 4
//    contiguous outputs per item.
// ---------------------------------------------------------------------------
constexpr int DWW_NI = 4;  // 4-element input items per lane (H * W <= 1024)
constexpr int DWW_NE = 4;  // 4-output epilogue items per lane (mult * Ho * Wo <= 1024)

template <typename T, int K, int S, int BH, bool RES, bool OVEC, int AK = -1>
__global__ __launch_bounds__(64) void depthwise_wave_kernel(const DepthwiseArgs a) {
  typedef typename DwVec<T>::type V;
  constexpr int PR = (BH - 1) * S + K;  // input rows of one lane's output column
  extern __shared__ float smem_dw[];
  const int lane = threadIdx.x;
  const int hw = a.h * a.w;
  const int howo = a.ho * a.wo;
  const int mult = a.mult;
  const int nplanes = a.n * a.c_in;
  float* tile = smem_dw;           // tih x tiw; input column iw sits at column lm + iw
  float* outt = smem_dw + a.oofs;  // mult * howo raw sums (16-byte aligned)
  float* bl = smem_dw + a.bofs;    // mult bias values
  constexpr int KKP = (K * K + 3) / 4 * 4;
  float* wl = smem_dw + a.wofs;    // mult rows of K * K weights, KKP floats apart
  float* sink = smem_dw + a.sofs;  // 4 floats (16-byte aligned) that dead writes hit
  const T* __restrict__ x = static_cast<const T*>(a.x);
  const T* __restrict__ wt = static_cast<const T*>(a.wt);
  const T* __restrict__ bias = static_cast<const T*>(a.bias);
  const T* res = static_cast<const T*>(a.res);
  T* y = static_cast<T*>(a.y);

  // prefetched per plane: the input (4-element items), the bias of output
  // plane (p, lane) for lane < mult and weight `lane` of the plane's
  // mult * K * K <= 64 weights
  float xin[DWW_NI][4];
  float bin = 0.0f, win = 0.0f;
  auto load = [&](int p) __attribute__((always_inline)) {
    const long long base = (long long)p * hw;
#pragma unroll
    for (int i = 0; i < DWW_NI; ++i) {
      const int e = min(4 * (lane + 64 * i), hw - 4);  // hw % 4 == 0
      dw_unpack<T>(*reinterpret_cast<const V*>(x + base + e), xin[i]);
    }
    const int ci = p % a.c_in;
    if (bias) bin = to_f32(bias[ci * mult + min(lane, mult - 1)]);
    win = to_f32(wt[(long long)ci * (mult * K * K) + min(lane, mult * K * K - 1)]);
  };
  auto stage = [&]() __attribute__((always_inline)) {
    if (a.w % 4 == 0) {  // uniform: an item never straddles two rows
#pragma unroll
      for (int i = 0; i < DWW_NI; ++i) {
        const unsigned e = 4 * (lane + 64 * i);
        const unsigned ih = mdiv(e, a.mg_w);
        const unsigned iw = e - ih * a.w;
        float* dst = (int)e < hw ? tile + (ih + a.pt) * a.tiw + a.lm + iw : sink;
        *reinterpret_cast<float4*>(dst) = float4{xin[i][0], xin[i][1], xin[i][2], xin[i][3]};
      }
    } else {
#pragma unroll
      for (int i = 0; i < DWW_NI; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const unsigned e = 4 * (lane + 64 * i) + k;
          const unsigned ih = mdiv(e, a.mg_w);
          const unsigned iw = e - ih * a.w;
          float* dst = (int)e < hw ? tile + (ih + a.pt) * a.tiw + a.lm + iw : sink;
          *dst = xin[i][k];
        }
    }
  };

  for (int i = lane; i < a.tpp; i += 64) tile[i] = 0.0f;  // border stays zero
  int p = blockIdx.x;
  if (p < nplanes) load(p);
  __syncthreads();

  const int units = a.nrb * a.wo;
  for (; p < nplanes; p += gridDim.x) {
    stage();
    if (lane < mult) bl[lane] = bin;
    if (lane < mult * K * K) {  // weight rows padded to whole 16-byte vectors
      const int jm = lane / (K * K), t = lane - jm * (K * K);
      wl[jm * KKP + t] = win;
    }
    __syncthreads();
    if (p + (int)gridDim.x < nplanes) load(p + gridDim.x);  // prefetch (uniform)

    for (int u = lane; u < units; u += 64) {
      const unsigned rb = mdiv(u, a.mg_wo);
      const unsigned ow = u - rb * a.wo;
      const float* src = tile + (rb * BH * S) * a.tiw + ow * S + (a.lm - a.pl);
      for (int jm = 0; jm < mult; ++jm) {
        // the plane's weights: one LDS address for every lane (broadcast reads)
        float wk[KKP];
#pragma unroll
        for (int j = 0; j < KKP / 4; ++j) {
          const float4 w4 = *reinterpret_cast<const float4*>(wl + jm * KKP + 4 * j);
          wk[4 * j] = w4.x;
          wk[4 * j + 1] = w4.y;
          wk[4 * j + 2] = w4.z;
          wk[4 * j + 3] = w4.w;
        }
        float acc[BH];
#pragma unroll
        for (int i = 0; i < BH; ++i) acc[i] = 0.0f;
#pragma unroll
        for (int r = 0; r < PR; ++r) {
          float rv[K];
#pragma unroll
          for (int kw = 0; kw < K; ++kw) rv[kw] = src[r * a.tiw + kw];
#pragma unroll
          for (int i = 0; i < BH; ++i) {
            const int kh = r - i * S;
            if (kh < 0 || kh >= K) continue;  // compile time
#pragma unroll
            for (int kw = 0; kw < K; ++kw) acc[i] = fmaf(rv[kw], wk[kh * K + kw], acc[i]);
          }
        }
        float* o = outt + jm * howo + ow;
#pragma unroll
        for (int i = 0; i < BH; ++i) {
          const int oh = rb * BH + i;
          *(oh < a.ho ? o + oh * a.wo : sink) = acc[i];
        }
      }
    }
    __syncthreads();

    const int tot = mult * howo;
    const long long obase = (long long)p * tot;
    if constexpr (OVEC) {  // howo % 4 == 0, y / residual 16 / 8-byte aligned
      const int nq = tot / 4;
      if constexpr (RES) {
        float v[DWW_NE * 4];  // every residual read before any store (y may alias it)
#pragma unroll
        for (int k = 0; k < DWW_NE; ++k) {
          float f[4];
          dw_unpack<T>(*reinterpret_cast<const V*>(res + obase + 4 * min(lane + 64 * k, nq - 1)), f);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[4 * k + e] = f[e];
        }
#pragma unroll
        for (int k = 0; k < DWW_NE; ++k) {
          const int q = min(lane + 64 * k, nq - 1);
          const float4 s4 = *reinterpret_cast<const float4*>(outt + 4 * q);
          const float bv = bl[mdiv(4 * q, a.mg_howo)];
          const float sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) v[4 * k + e] = (sv[e] + bv) + v[4 * k + e];
        }
        act_apply<AK>(v, a.act, a.alpha, a.beta);
#pragma unroll
        for (int k = 0; k < DWW_NE; ++k) {
          const int q = lane + 64 * k;
          if (q < nq) {
            const float f[4] = {v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]};
            *reinterpret_cast<V*>(y + obase + 4 * q) = dw_pack<T>(f);
          }
        }
      } else {
        // items past the end repeat the last item (same value, same address):
        // a fixed number of stores lets the wait before the next staging skip them
#pragma unroll
        for (int k = 0; k < DWW_NE; ++k) {
          const int q = min(lane + 64 * k, nq - 1);
          const float4 s4 = *reinterpret_cast<const float4*>(outt + 4 * q);
          const float bv = bl[mdiv(4 * q, a.mg_howo)];
          float f[4] = {s4.x + bv, s4.y + bv, s4.z + bv, s4.w + bv};
          act_apply<AK>(f, a.act, a.alpha, a.beta);
          *reinterpret_cast<V*>(y + obase + 4 * q) = dw_pack<T>(f);
        }
      }
    } else {
      if constexpr (RES) {
        float v[DWW_NE * 4];
#pragma unroll
        for (int k = 0; k < DWW_NE * 4; ++k) v[k] = to_f32(res[obase + min(lane + 64 * k, tot - 1)]);
#pragma unroll
        for (int k = 0; k < DWW_NE * 4; ++k) {
          const int o = min(lane + 64 * k, tot - 1);
          v[k] = (outt[o] + bl[mdiv(o, a.mg_howo)]) + v[k];
        }
        act_apply<AK>(v, a.act, a.alpha, a.beta);
#pragma unroll
        for (int k = 0; k < DWW_NE * 4; ++k) {
          const int o = lane + 64 * k;
          if (o < tot) store_out(y + obase + o, from_f32<T>(v[k]));
        }
      } else {
#pragma unroll
        for (int k = 0; k < DWW_NE; ++k) {
          float f[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int o = min(lane + 64 * (4 * k + e), tot - 1);
            f[e] = outt[o] + bl[mdiv(o, a.mg_howo)];
          }
          act_apply<AK>(f, a.act, a.alpha, a.beta);
#pragma unroll
          for (int e = 0; e < 4; ++e) store_out(y + obase + min(lane + 64 * (4 * k + e), tot - 1), from_f32<T>(f[e]));
        }
      }
    }
    // one wave: its LDS accesses are ordered, so the next plane may overwrite
    // the tiles right away
  }
}

// Resident workgroups per CU of kernel f with lds bytes of dynamic LDS (cached).
static int resident_per_cu(const void* f, int threads, size_t lds) {
  struct Entry {
    const void* f;
    size_t lds;
    int n;
  };
  static Entry cache[64];
  static int used = 0;
  static std::mutex mu;
  {
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < used; ++i)
      if (cache[i].f == f && cache[i].lds == lds) return cache[i].n;
  }
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, f, threads, lds) != hipSuccess || n < 1) n = 1;
  std::lock_guard<std::mutex> lock(mu);
  if (used < 64) cache[used++] = Entry{f, lds, n};
  return n;
}

// Persistent grid over `items` work items: as many workgroups as are resident,
// each taking an equal number of items.
static int persistent_grid(long long items, int per_cu, int cus) {
  const long long slots = (long long)per_cu * cus;
  const long long rounds = (items + slots - 1) / slots;
  return (int)((items + rounds - 1) / rounds);
}

template <typename T>
static hipError_t launch_dw_wave_t(const DepthwiseArgs& a, long long planes, int cus, size_t lds,
                                   hipStream_t s) {
#define DWW_GO(...)                                                                      \
  {                                                                                      \
    const void* f = reinterpret_cast<const void*>(&depthwise_wave_kernel<__VA_ARGS__>);  \
    const int grid = persistent_grid(planes, resident_per_cu(f, 64, lds), cus);          \
    hipLaunchKernelGGL((depthwise_wave_kernel<__VA_ARGS__>), dim3(grid), dim3(64), lds, s, a); \
    return hipGetLastError();                                                            \
  }
  // identity, ReLU and hard-swish with the activation fixed at compile time on
  // the vector-output path without residual
#define DWW_LAUNCH(K_, S_, BH_, R_, O_)                                                  \
  {                                                                                      \
    if constexpr (O_ && !R_) {                                                           \
      if (a.act == 0) DWW_GO(T, K_, S_, BH_, R_, O_, 0)                                  \
      if (a.act == 1) DWW_GO(T, K_, S_, BH_, R_, O_, 1)                                  \
      if (a.act == 6) DWW_GO(T, K_, S_, BH_, R_, O_, 6)                                  \
    }                                                                                    \
    DWW_GO(T, K_, S_, BH_, R_, O_)                                                       \
  }
#define DWW_CASE(K_, S_, BH_)                                                            \
  if (a.kh == K_ && a.sh == S_ && a.bh == BH_) {                                         \
    if (a.res) {                                                                         \
      if (a.ovec) DWW_LAUNCH(K_, S_, BH_, true, true) else DWW_LAUNCH(K_, S_, BH_, true, false) \
    } else {                                                                             \
      if (a.ovec) DWW_LAUNCH(K_, S_, BH_, false, true) else DWW_LAUNCH(K_, S_, BH_, false, false) \
    }                                                                                    \
  }
  DWW_CASE(3, 1, 14)
  DWW_CASE(3, 2, 4)
  DWW_CASE(5, 1, 14)
  DWW_CASE(5, 2, 4)
  DWW_CASE(7, 1, 14)
#undef DWW_CASE
#undef DWW_LAUNCH
#undef DWW_GO
  return hipErrorInvalidValue;
}

hipError_t launch_depthwise_wave(Dtype dt, const DepthwiseArgs& a, long long planes, int cus,
                                 size_t lds, hipStream_t s) {
  return dt == F16    ? launch_dw_wave_t<_Float16>(a, planes, cus, lds, s)
         : dt == BF16 ? launch_dw_wave_t<__bf16>(a, planes, cus, lds, s)
                      : launch_dw_wave_t<float>(a, planes, cus, lds, s);
}

template <typename T>
static hipError_t launch_dw_plane_t(const DepthwiseArgs& a, int grid, size_t lds,
                                    hipStream_t s) {
#define DW_CASE(K_, S_, BH_)                                                             \
  if (a.kh == K_ && a.sh == S_ && a.bh == BH_) {                                         \
    if (a.res)                                                                           \
      hipLaunchKernelGGL((depthwise_plane_kernel<T, K_, S_, BH_, true>), dim3(grid), dim3(256), \
                         lds, s, a);                                                     \
    else                                                                                 \
      hipLaunchKernelGGL((depthwise_plane_kernel<T, K_, S_, BH_, false>), dim3(grid), dim3(256), \
                         lds, s, a);                                                     \
    return hipGetLastError();                                                            \
  }
  DW_CASE(3, 1, 4)
  DW_CASE(3, 2, 2)
  DW_CASE(5, 1, 4)
  DW_CASE(5, 2, 2)
  DW_CASE(7, 1, 4)
#undef DW_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_depthwise_plane(Dtype dt, const DepthwiseArgs& a, int grid, size_t lds,
                                  hipStream_t s) {
  return dt == F16    ? launch_dw_plane_t<_Float16>(a, grid, lds, s)
         : dt == BF16 ? launch_dw_plane_t<__bf16>(a, grid, lds, s)
                      : launch_dw_plane_t<float>(a, grid, lds, s);
}

// ---------------------------------------------------------------------------
// Split-k reduction ("Convolution, pooling and resize", split k: each range
// writes a raw plane and the epilogue pass adds the planes in range order, then
// bias, residual and activation).  Each lane owns 4 consecutive outputs, read
// as float4, so a half wave reads 512 contiguous bytes of a plane.  The two
// halves of a wave cover the same 128 outputs: the lower half adds planes
// [0, h) and the upper half planes [h, R), each in range order, h = ceil(R/2);
// one cross-half wavefront shuffle (lane xor 32) then adds the two partial
// sums.  The order depends on R alone, so two runs give the same bits.  The
// lower half applies bias, residual and activation and stores.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const ReduceArgs a) {
  const int lane = threadIdx.x & 63;
  const int upper = lane >> 5;
  const long long wave_id = ((long long)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const long long o0 = (wave_id * 32 + (lane & 31)) * 4;
  const int h = (a.splits + 1) >> 1;
  const int r0 = upper ? h : 0, r1 = upper ? a.splits : h;
  float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (o0 < a.total) {
    if (a.vec) {  // total and the plane stride are multiples of 4
      for (int r = r0; r < r1; ++r) {
        const float4 p =
            *reinterpret_cast<const float4*>(a.planes + (long long)r * a.plane_stride + o0);
        if (r == r0) {
          v[0] = p.x; v[1] = p.y; v[2] = p.z; v[3] = p.w;
        } else {
          v[0] += p.x; v[1] += p.y; v[2] += p.z; v[3] += p.w;
        }
      }
    } else {
      for (int r = r0; r < r1; ++r) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (o0 + i < a.total) {
            const float p = a.planes[(long long)r * a.plane_stride + o0 + i];
            v[i] = r == r0 ? p : v[i] + p;
          }
        }
      }
    }
  }
  // every lane reaches the shuffle (no early exit above)
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] += __shfl_xor(v[i], 32, 64);
  if (!upper) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const long long o = o0 + i;
      if (o < a.total) {
        const int co = (int)((o / a.hw) % a.c_out);
        static_cast<T*>(a.y)[o] = epilogue_one<T>(v[i], static_cast<const T*>(a.bias),
                                                  static_cast<const T*>(a.res), co, o, a.act,
                                                  a.alpha, a.beta);
      }
    }
  }
}

template <typename T>
static hipError_t launch_reduce_t(const ReduceArgs& a, hipStream_t s) {
  if (a.splits < 2) return hipErrorInvalidValue;
  const long long waves = (a.total + 127) / 128;
  dim3 grid((unsigned)((waves + 3) / 4));
  hipLaunchKernelGGL((splitk_reduce_kernel<T>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_reduce(Dtype dt, const ReduceArgs& a, hipStream_t s) {
  return dt == F16    ? launch_reduce_t<_Float16>(a, s)
         : dt == BF16 ? launch_reduce_t<__bf16>(a, s)
                      : launch_reduce_t<float>(a, s);
}

// ---------------------------------------------------------------------------
// Gathering col2im for ConvTranspose: output (n, co, oh, ow) sums, in (kh, kw)
// row-major order, the column entries of the taps whose source position
// ((oh + pt - kh*dh) / sh, (ow + pl - kw*dw) / sw) is integral and inside the
// input.  Columns: [n][groups*cog*kh*kw][h][w] float32, row g*M + (j*kh+u)*kw+v.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void col2im_kernel(const Col2imArgs a) {
  const long long o = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (o >= a.total) return;
  const int ow = (int)(o % a.wo);
  long long t = o / a.wo;
  const int oh = (int)(t % a.ho);
  t /= a.ho;
  const int co = (int)(t % a.c_out);
  const int n = (int)(t / a.c_out);
  const int g = co / a.cog, j = co - g * a.cog;
  const int m_per_g = a.cog * a.kh * a.kw;
  const long long hw = (long long)a.h * a.w;
  const float* __restrict__ cbase =
      a.cols + ((long long)n * (a.c_out * a.kh * a.kw) + (long long)g * m_per_g +
                (long long)j * a.kh * a.kw) * hw;
  float acc = 0.0f;
  for (int kh = 0; kh < a.kh; ++kh) {
    const int th = oh + a.pt - kh * a.dh;
    if (th < 0 || th % a.sh) continue;
    const int ih = th / a.sh;
    if (ih >= a.h) continue;
    for (int kw = 0; kw < a.kw; ++kw) {
      const int tw = ow + a.pl - kw * a.dw;
      if (tw < 0 || tw % a.sw) continue;
      const int iw = tw / a.sw;
      if (iw >= a.w) continue;
      acc += cbase[(long long)(kh * a.kw + kw) * hw + (long long)ih * a.w + iw];
    }
  }
  static_cast<T*>(a.y)[o] = epilogue_one<T>(acc, static_cast<const T*>(a.bias),
                                            static_cast<const T*>(a.res), co, o, a.act,
                                            a.alpha, a.beta);
}

hipError_t launch_col2im(Dtype dt, const Col2imArgs& a, hipStream_t s) {
  dim3 grid((unsigned)((a.total + 255) / 256));
  if (dt == F16)
    hipLaunchKernelGGL(col2im_kernel<_Float16>, grid, dim3(256), 0, s, a);
  else if (dt == BF16)
    hipLaunchKernelGGL(col2im_kernel<__bf16>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(col2im_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace convfwd
