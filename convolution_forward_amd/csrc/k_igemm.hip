// Generic implicit-GEMM convolution for gfx950 (any stride, dilation, pads,
// groups, kernel size; f16, bf16 or f32 operands, f32 accumulation).
//
// Per group g the layer is the product Y_g[p, co] = sum_k A[p, k] * B[k, co]
// with p = (n, oh, ow) the output pixel, k = (ci', kh, kw) in the order of the
// OIHW weight row, A[p, k] the input value under that tap (zero in padding) and
// B[k, co] = w[co, k]  ("Convolutions", sections 1 and 2.4; "Convolution,
// pooling and resize", "Variants": implicit GEMM gathers the input window while
// it loads the tile, so no column matrix exists in memory).
//
// gfx950 mapping: a workgroup of 4 wave64s owns a 64-pixel x 64-channel tile.
// Each k-block (64 bytes of k: 32 halves or 16 floats) is gathered from global
// memory straight into LDS rows, k contiguous, double-buffered through
// registers.  Each wave multiplies a 32 x 32 sub-tile with MFMA:
//   f16 / bf16: v_mfma_f32_16x16x32_{f16,bf16}, one lane feeds 8 consecutive k
//   of one row;
//   f32: v_mfma_f32_16x16x4_f32, one lane feeds 4 consecutive k over 4 steps.
// Lane l always feeds k-slot (l / 16) of row (l % 16) of both operands with the
// same k values, so the product is exact regardless of the hardware's internal
// k order.  The result fragment holds 4 consecutive pixels of one channel per
// lane.
//
// Output modes: fused epilogue (bias, residual, activation, rounded in f32) or
// raw f32 sums into one plane per split-k range (reduced in range order of the
// shape-fixed cut by a second kernel), which also serves ConvTranspose's GEMM
// into f32 columns (wtrans: weight element (k, col) at w[(g*cig + k)*cols + col]).
#include "epilogue.h"
#include "internal.h"

namespace convfwd {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

template <typename T>
struct IgVec;
template <>
struct IgVec<_Float16> {
  static constexpr int EPT = 8;
  typedef half8_t vec;
};
template <>
struct IgVec<__bf16> {
  static constexpr int EPT = 8;
  typedef bf16x8_t vec;
};
template <>
struct IgVec<float> {
  static constexpr int EPT = 4;
  typedef floatx4_t vec;
};

constexpr int IG_ROW = IG_KSTEP_BYTES + 16;  // LDS row pitch in bytes (64 data + 16 pad)

template <typename T>
__device__ __forceinline__ void mfma_step(const typename IgVec<T>::vec& a,
                                          const typename IgVec<T>::vec& b, floatx4_t& acc);

template <>
__device__ __forceinline__ void mfma_step<_Float16>(const half8_t& a, const half8_t& b,
                                                     floatx4_t& acc) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
}

template <>
__device__ __forceinline__ void mfma_step<__bf16>(const bf16x8_t& a, const bf16x8_t& b,
                                                   floatx4_t& acc) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}

template <>
__device__ __forceinline__ void mfma_step<float>(const floatx4_t& a, const floatx4_t& b,
                                                  floatx4_t& acc) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], acc, 0, 0, 0);
}

template <typename T>
__global__ __launch_bounds__(256) void igemm_kernel(const IgemmArgs a) {
  typedef typename IgVec<T>::vec vec_t;
  constexpr int EPT = IgVec<T>::EPT;
  constexpr int KSTEP = 4 * EPT;

  __shared__ __attribute__((aligned(16))) unsigned char As[2][IG_TILE_P * IG_ROW];
  __shared__ __attribute__((aligned(16))) unsigned char Bs[2][IG_TILE_C * IG_ROW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int tile_p0 = blockIdx.x * IG_TILE_P;
  const int tile_c0 = blockIdx.y * IG_TILE_C;
  const int grp = blockIdx.z / a.splits;
  const int split = blockIdx.z - grp * a.splits;
  const int step_begin = split * a.steps_per_split;
  const int step_end = min(a.ksteps, step_begin + a.steps_per_split);
  const int nsteps = step_end - step_begin;

  // This thread stages row (tid % 64) and k-quarter (tid / 64) of both tiles.
  const int srow = tid & 63;
  const int squart = tid >> 6;

  // A side: the output pixel this thread gathers for.
  const int hw_out = a.ho * a.wo;
  const int p = tile_p0 + srow;
  const bool p_ok = p < a.pix;
  int n_img = 0, oh = 0, ow = 0;
  if (p_ok) {
    n_img = p / hw_out;
    const int rem = p - n_img * hw_out;
    oh = rem / a.wo;
    ow = rem - oh * a.wo;
  }
  const int ih0 = oh * a.sh - a.pt;
  const int iw0 = ow * a.sw - a.pl;
  const T* __restrict__ xg =
      static_cast<const T*>(a.x) + ((long long)n_img * a.c_in + (long long)grp * a.cig) *
                                       (long long)a.h * a.w;
  const int khw = a.kh * a.kw;

  // B side: the GEMM column (output channel within the group) this thread loads.
  const int bcol = tile_c0 + srow;
  const bool c_ok = bcol < a.cog;
  const T* __restrict__ wbase = static_cast<const T*>(a.wt);

  vec_t ra, rb;

  auto gather = [&](int step) __attribute__((always_inline)) {
    const int k0 = step * KSTEP + squart * EPT;
    // A: decode k0 once, then walk (ci, kh, kw) in weight-row order.
    {
      int ci = k0 / khw;
      int rr = k0 - ci * khw;
      int kh = rr / a.kw;
      int kw = rr - kh * a.kw;
#pragma unroll
      for (int j = 0; j < EPT; ++j) {
        T v = T(0);
        if (p_ok && k0 + j < a.kg) {
          const int ih = ih0 + kh * a.dh;
          const int iw = iw0 + kw * a.dw;
          if ((unsigned)ih < (unsigned)a.h && (unsigned)iw < (unsigned)a.w)
            v = xg[((long long)ci * a.h + ih) * a.w + iw];
        }
        ra[j] = v;
        if (++kw == a.kw) {
          kw = 0;
          if (++kh == a.kh) {
            kh = 0;
            ++ci;
          }
        }
      }
    }
    // B
    if (!a.wtrans) {
      const T* wr = wbase + ((long long)grp * a.cog + bcol) * a.kg;
      if (a.wvec && c_ok && k0 + EPT <= a.kg) {
        rb = *reinterpret_cast<const vec_t*>(wr + k0);
      } else {
#pragma unroll
        for (int j = 0; j < EPT; ++j) rb[j] = (c_ok && k0 + j < a.kg) ? wr[k0 + j] : T(0);
      }
    } else {
#pragma unroll
      for (int j = 0; j < EPT; ++j) {
        const int k = k0 + j;
        rb[j] = (c_ok && k < a.kg) ? wbase[((long long)grp * a.cig + k) * a.cog + bcol] : T(0);
      }
    }
  };

  auto stash = [&](int buf) __attribute__((always_inline)) {
    *reinterpret_cast<vec_t*>(&As[buf][srow * IG_ROW + squart * 16]) = ra;
    *reinterpret_cast<vec_t*>(&Bs[buf][srow * IG_ROW + squart * 16]) = rb;
  };

  floatx4_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  const int wr = wave & 1;   // pixel half of the tile
  const int wc = wave >> 1;  // channel half of the tile
  const int frow = lane & 15;
  const int fk = (lane >> 4) * 16;

  if (nsteps > 0) {
    gather(step_begin);
    stash(0);
    __syncthreads();
    for (int s = 0; s < nsteps; ++s) {
      const int buf = s & 1;
      const bool more = s + 1 < nsteps;
      if (more) gather(step_begin + s + 1);
      vec_t fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        fa[i] = *reinterpret_cast<const vec_t*>(&As[buf][(wr * 32 + i * 16 + frow) * IG_ROW + fk]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        fb[j] = *reinterpret_cast<const vec_t*>(&Bs[buf][(wc * 32 + j * 16 + frow) * IG_ROW + fk]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) mfma_step<T>(fa[i], fb[j], acc[i][j]);
      if (more) stash(buf ^ 1);
      __syncthreads();
    }
  }

  // Epilogue: lane holds pixels 4*(lane/16) + e of row block i, channel lane % 16 of
  // block j.  Every residual of the lane is read before any store: y may alias the
  // residual exactly and each element is read and written by this lane only, so
  // hoisting the reads keeps the result and lets them overlap.
  const T* bias = static_cast<const T*>(a.bias);
  const T* res = static_cast<const T*>(a.res);
  T* y = static_cast<T*>(a.y);
  long long oidx[2][2][4];
  bool ok[2][2][4];
  float rv[2][2][4];
  float bv[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int col = tile_c0 + wc * 32 + j * 16 + (lane & 15);
    const bool col_ok = col < a.cog;
    const int co = grp * a.cog + (col_ok ? col : 0);
    bv[j] = (bias && col_ok && a.mode != OUT_RAW) ? to_f32(bias[co]) : 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int pp = tile_p0 + wr * 32 + i * 16 + (lane >> 4) * 4 + e;
        ok[j][i][e] = col_ok && pp < a.pix;
        const int ppc = ok[j][i][e] ? pp : 0;
        const int n_o = ppc / hw_out;
        const int rem = ppc - n_o * hw_out;
        oidx[j][i][e] = ((long long)n_o * a.c_out + co) * hw_out + rem;
        rv[j][i][e] = 0.f;
      }
    }
  }
  if (res && a.mode != OUT_RAW) {  // uniform; every load unconditional (clamped index)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) rv[j][i][e] = to_f32(res[oidx[j][i][e]]);
  }
  if (a.mode == OUT_RAW) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (ok[j][i][e]) a.planes[(long long)split * a.plane_stride + oidx[j][i][e]] = acc[i][j][e];
    return;
  }
  float v[16];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float s = acc[i][j][e];
        if (bias) s = s + bv[j];
        if (res) s = s + rv[j][i][e];
        v[(j * 2 + i) * 4 + e] = s;
      }
  act_array(v, a.act, a.alpha, a.beta);
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (ok[j][i][e]) y[oidx[j][i][e]] = from_f32<T>(v[(j * 2 + i) * 4 + e]);
}

hipError_t launch_igemm(Dtype dt, const IgemmArgs& a, hipStream_t s) {
  dim3 grid((a.pix + IG_TILE_P - 1) / IG_TILE_P, (a.cog + IG_TILE_C - 1) / IG_TILE_C,
            a.groups * a.splits);
  if (dt == F16)
    hipLaunchKernelGGL(igemm_kernel<_Float16>, grid, dim3(256), 0, s, a);
  else if (dt == BF16)
    hipLaunchKernelGGL(igemm_kernel<__bf16>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(igemm_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace convfwd
