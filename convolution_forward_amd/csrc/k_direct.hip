// Bandwidth-bound kernels for gfx950 (VALU only, no MFMA):
//  - depthwise direct convolution ("Convolution, pooling and resize", "Variants":
//    one input channel per group, any channel multiplier, one fixed window order);
//  - the split-k reduction + epilogue (planes combined with a fixed wavefront
//    shuffle tree, then bias, residual, activation);
//  - the gathering col2im + epilogue of ConvTranspose (one thread per output
//    element, taps visited in row-major order, no atomics).
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
  else
    hipLaunchKernelGGL(depthwise_kernel<float>, grid, dim3(256), lds, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Depthwise, whole-plane fast path (dilation 1, kernel and stride fixed at
// compile time): a workgroup stages P consecutive input planes (contiguous in
// NCHW, read with 16-byte loads) into zero-padded LDS tiles together with their
// weights, then each thread computes 2x2 output blocks from an input patch held
// in registers, so every staged value feeds several FMAs.  Each output is still
// one float32 FMA chain over the window in (kh, kw) row-major order.
// ---------------------------------------------------------------------------
template <typename T, int KH, int KW, int SH, int SW>
__global__ __launch_bounds__(256) void depthwise_plane_kernel(const DepthwiseArgs a) {
  constexpr int BH = 2, BW = 2;
  constexpr int PH = (BH - 1) * SH + KH, PW = (BW - 1) * SW + KW;  // input patch
  extern __shared__ float smem_dw[];
  const int P = a.planes;                 // input planes per workgroup
  const int tsz = a.tih * a.tiw;          // floats per plane tile (tiw = row pitch)
  float* tile = smem_dw;
  float* wl = smem_dw + P * tsz;          // P * mult * KH * KW weights
  const int plane0 = blockIdx.x * P;
  const int nplanes = a.n * a.c_in;
  const int np = min(P, nplanes - plane0);
  const int hw = a.h * a.w;
  const T* __restrict__ xp = static_cast<const T*>(a.x) + (long long)plane0 * hw;

  for (int i = threadIdx.x; i < P * tsz; i += 256) tile[i] = 0.0f;
  const int nw = np * a.mult * KH * KW;
  __syncthreads();
  for (int i = threadIdx.x; i < nw; i += 256) {
    // planes of one workgroup may wrap from the last channel of an image to the
    // first of the next: index the weights by each plane's channel
    const int pl = i / (a.mult * KH * KW), r = i - pl * (a.mult * KH * KW);
    const int ci = (plane0 + pl) % a.c_in;
    wl[i] = to_f32(static_cast<const T*>(a.wt)[(long long)ci * a.mult * KH * KW + r]);
  }
  // planes: 4 consecutive pixels per item
  const int g4 = (hw + 3) / 4;
  for (int q = threadIdx.x; q < np * g4; q += 256) {
    const int pl = q / g4, f0 = 4 * (q - pl * g4);
    float v[4];
    if (a.xvec && f0 + 4 <= hw) {
      if constexpr (sizeof(T) == 4) {
        const float4 t = *reinterpret_cast<const float4*>(xp + (long long)pl * hw + f0);
        v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
      } else {
        const uint2 t = *reinterpret_cast<const uint2*>(xp + (long long)pl * hw + f0);
        const _Float16* h = reinterpret_cast<const _Float16*>(&t);
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) v[k4] = (float)h[k4];
      }
    } else {
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4)
        v[k4] = f0 + k4 < hw ? to_f32(xp[(long long)pl * hw + f0 + k4]) : 0.0f;
    }
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4) {
      const int f = f0 + k4;
      if (f >= hw) break;
      const int ih = f / a.w, iw = f - (f / a.w) * a.w;
      const int tr = ih + a.pt, tc = iw + a.pl;
      if (tr < a.tih && tc < a.tiw - 1) tile[pl * tsz + tr * a.tiw + tc] = v[k4];
    }
  }
  __syncthreads();

  const T* __restrict__ bias = static_cast<const T*>(a.bias);
  const T* res = static_cast<const T*>(a.res);
  T* y = static_cast<T*>(a.y);
  const int nbh = (a.ho + BH - 1) / BH, nbw = (a.wo + BW - 1) / BW;
  const int per_plane = nbh * nbw;
  for (int b = threadIdx.x; b < np * per_plane; b += 256) {
    const int pl = b / per_plane, r = b - pl * per_plane;
    const int bh = r / nbw, bw = r - (r / nbw) * nbw;
    const int oh0 = bh * BH, ow0 = bw * BW;
    const float* src = tile + pl * tsz + (oh0 * SH) * a.tiw + ow0 * SW;
    float patch[PH][PW];
#pragma unroll
    for (int i = 0; i < PH; ++i)
#pragma unroll
      for (int j = 0; j < PW; ++j) {
        // the last block of a row/column may reach past the tile: clamp the read
        // (those outputs are not stored)
        const int rr = min(oh0 * SH + i, a.tih - 1) - oh0 * SH;
        const int cc = min(ow0 * SW + j, a.tiw - 1) - ow0 * SW;
        patch[i][j] = src[rr * a.tiw + cc];
      }
    const int plane = plane0 + pl;
    const int n = plane / a.c_in, ci = plane - n * a.c_in;
    for (int jm = 0; jm < a.mult; ++jm) {
      const int co = ci * a.mult + jm;
      const float* wv = wl + (pl * a.mult + jm) * KH * KW;
      float acc[BH][BW];
#pragma unroll
      for (int i = 0; i < BH; ++i)
#pragma unroll
        for (int j = 0; j < BW; ++j) acc[i][j] = 0.0f;
#pragma unroll
      for (int kh = 0; kh < KH; ++kh)
#pragma unroll
        for (int kw = 0; kw < KW; ++kw) {
          const float wk = wv[kh * KW + kw];
#pragma unroll
          for (int i = 0; i < BH; ++i)
#pragma unroll
            for (int j = 0; j < BW; ++j)
              acc[i][j] = fmaf(patch[i * SH + kh][j * SW + kw], wk, acc[i][j]);
        }
      // residuals first (y may alias the residual exactly), then the stores
      const long long obase = ((long long)n * a.c_out + co) * a.ho * a.wo;
      long long oidx[BH][BW];
      bool ok[BH][BW];
      float rv[BH][BW];
#pragma unroll
      for (int i = 0; i < BH; ++i)
#pragma unroll
        for (int j = 0; j < BW; ++j) {
          ok[i][j] = oh0 + i < a.ho && ow0 + j < a.wo;
          oidx[i][j] = obase + (ok[i][j] ? (long long)(oh0 + i) * a.wo + ow0 + j : 0);
          rv[i][j] = 0.0f;
        }
      if (res) {  // uniform; clamped indices keep every load unconditional
#pragma unroll
        for (int i = 0; i < BH; ++i)
#pragma unroll
          for (int j = 0; j < BW; ++j) rv[i][j] = to_f32(res[oidx[i][j]]);
      }
      const float bv = bias ? to_f32(bias[co]) : 0.0f;
      float v[BH * BW];
#pragma unroll
      for (int i = 0; i < BH; ++i)
#pragma unroll
        for (int j = 0; j < BW; ++j) {
          float s = acc[i][j];
          if (bias) s = s + bv;
          if (res) s = s + rv[i][j];
          v[i * BW + j] = s;
        }
      act_array(v, a.act, a.alpha, a.beta);
#pragma unroll
      for (int i = 0; i < BH; ++i)
#pragma unroll
        for (int j = 0; j < BW; ++j)
          if (ok[i][j]) y[oidx[i][j]] = from_f32<T>(v[i * BW + j]);
    }
  }
}

template <typename T>
static hipError_t launch_dw_plane_t(const DepthwiseArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((a.n * a.c_in + a.planes - 1) / a.planes));
  const size_t lds = ((size_t)a.planes * a.tih * a.tiw + (size_t)a.planes * a.mult * a.kh * a.kw) *
                     sizeof(float);
#define DW_CASE(KH_, KW_, SH_, SW_)                                                        \
  if (a.kh == KH_ && a.kw == KW_ && a.sh == SH_ && a.sw == SW_) {                          \
    hipLaunchKernelGGL((depthwise_plane_kernel<T, KH_, KW_, SH_, SW_>), grid, dim3(256), lds, s, a); \
    return hipGetLastError();                                                              \
  }
  DW_CASE(3, 3, 1, 1)
  DW_CASE(3, 3, 2, 2)
  DW_CASE(5, 5, 1, 1)
  DW_CASE(5, 5, 2, 2)
  DW_CASE(7, 7, 1, 1)
#undef DW_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_depthwise_plane(Dtype dt, const DepthwiseArgs& a, hipStream_t s) {
  return dt == F16 ? launch_dw_plane_t<_Float16>(a, s) : launch_dw_plane_t<float>(a, s);
}

// ---------------------------------------------------------------------------
// Split-k reduction.  The R raw planes hold disjoint k ranges of the same
// outputs.  Lanes are grouped R' = next_pow2(R) at a time: lane (q, r) reads
// plane r of output q, and a xor butterfly over the group adds the planes in a
// fixed tree ((p0+p1)+(p2+p3))+...; addition is commutative, so every lane of
// the group ends with bit-identical sums and the order depends only on R.
// Lane r == 0 of each group applies bias, residual, activation and stores.
// ---------------------------------------------------------------------------
template <typename T, int RP>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const ReduceArgs a) {
  constexpr int OPW = 64 / RP;  // outputs per wave
  const int lane = threadIdx.x & 63;
  const int q = lane / RP, r = lane - q * RP;
  const long long wave_id = (long long)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  const long long o = wave_id * OPW + q;
  float v = 0.0f;
  if (o < a.total && r < a.splits) v = a.planes[(long long)r * a.plane_stride + o];
#pragma unroll
  for (int off = 1; off < RP; off <<= 1) v += __shfl_xor(v, off, 64);
  if (r == 0 && o < a.total) {
    const int co = (int)((o / a.hw) % a.c_out);
    static_cast<T*>(a.y)[o] = epilogue_one<T>(v, static_cast<const T*>(a.bias),
                                              static_cast<const T*>(a.res), co, o, a.act,
                                              a.alpha, a.beta);
  }
}

template <typename T>
static hipError_t launch_reduce_t(const ReduceArgs& a, hipStream_t s) {
  int rp = 1;
  while (rp < a.splits) rp <<= 1;
  const long long opw = 64 / rp;
  const long long waves = (a.total + opw - 1) / opw;
  dim3 grid((unsigned)((waves + 3) / 4));
  switch (rp) {
    case 1: hipLaunchKernelGGL((splitk_reduce_kernel<T, 1>), grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((splitk_reduce_kernel<T, 2>), grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL((splitk_reduce_kernel<T, 4>), grid, dim3(256), 0, s, a); break;
    case 8: hipLaunchKernelGGL((splitk_reduce_kernel<T, 8>), grid, dim3(256), 0, s, a); break;
    case 16: hipLaunchKernelGGL((splitk_reduce_kernel<T, 16>), grid, dim3(256), 0, s, a); break;
    case 32: hipLaunchKernelGGL((splitk_reduce_kernel<T, 32>), grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_reduce(Dtype dt, const ReduceArgs& a, hipStream_t s) {
  return dt == F16 ? launch_reduce_t<_Float16>(a, s) : launch_reduce_t<float>(a, s);
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
  else
    hipLaunchKernelGGL(col2im_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace convfwd
