// Winograd F(2x2, 3x3) convolution forward for gfx950, 16-bit operands with
// float32 accumulation ("Convolutions", section 2.6: F(m, r) computes m outputs
// of an r-tap filter with m + r - 1 multiplies, 16 against 36 for 2x2 outputs of
// a 3x3 kernel, at the cost of transforms of the input tiles and the weights;
// "Convolution, pooling and resize", "Not built, with the numbers": the method
// is sixteen batched products between the transforms).  The transforms are the
// published ones of Lavin and Gray (2016):
//
//   U = G g G^T,  V = B^T d B,  M = sum over input channels of U (.) V,
//   Y = A^T M A
//   B^T = [1 0 -1 0; 0 1 1 0; 0 -1 1 0; 0 1 0 -1], G = [1 0 0; 1/2 1/2 1/2;
//   1/2 -1/2 1/2; 0 0 1], A^T = [1 1 1 0; 0 1 -1 -1].
//
// The sixteen products, one per position xi of the 4x4 transformed tile, are
// GEMMs M_xi[co][t] = sum_ci U_xi[co][ci] V_xi[ci][t] over the output tiles t
// (2x2 outputs each), run on v_mfma_f32_32x32x16_{f16,bf16}.
//
//  * Weight kernel: U for every (co, ci) into scratch, [xi][co][ci] (16-bit),
//    so each MFMA A fragment (8 consecutive input channels of one output
//    channel) is one 16-byte load.
//  * Main kernel: a workgroup owns 32 consecutive tiles (in (image, tile row,
//    tile column) order) and 32 * CB output channels; each of its 4 waves owns
//    4 of the 16 positions xi.  Per step of 16 input channels every thread
//    gathers the 4x4 input patches of 2 (tile, channel) pairs, forms V in
//    float32 (adds and subtracts only) and writes its 16 values, rounded once to
//    the 16-bit type, into LDS laid out [xi][tile][channel] (a B fragment is
//    one 16-byte read); V is double-buffered so one barrier per step suffices.
//  * Output: the accumulators go through LDS as float32 M[xi][co][t]; each
//    thread applies A^T M A to whole tiles and the fused epilogue (bias,
//    residual, activation, each rounded in float32) and stores the outputs
//    that exist (a tile past the last row or column drops them).
//
// Rounding: U and V are rounded once to the 16-bit type before the products
// (the transforms themselves run in float32), which adds cross terms' rounding
// that a direct sum does not have; the planner never picks this kernel by
// itself, a caller asks for it.
#include <type_traits>

#include "epilogue.h"
#include "internal.h"
#include "mfma16.h"

namespace convfwd {

namespace {

typedef unsigned u32x4_w __attribute__((ext_vector_type(4)));

constexpr int WN_T = 32;   // tiles per workgroup
constexpr int WN_KC = 16;  // input channels per step (the MFMA's k)
constexpr int WN_VBUF = 16 * WN_T * WN_KC;  // elements of one V buffer

// U[xi][co][ci] = (G g G^T)[xi] for every output channel co and input channel
// ci of its group (ci fastest across threads: coalesced 2-byte stores).
template <typename E>
__global__ __launch_bounds__(256) void wino_weights_kernel(const WinoArgs a) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long plane = (long long)a.c_out * a.cig;
  if (i >= plane) return;
  const E* g = static_cast<const E*>(a.wt) + i * 9;  // [co][ci][3][3]
  float w[9];
#pragma unroll
  for (int k = 0; k < 9; ++k) w[k] = to_f32(g[k]);
  float gg[4][3];
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    gg[0][j] = w[j];
    gg[1][j] = 0.5f * (w[j] + w[3 + j] + w[6 + j]);
    gg[2][j] = 0.5f * (w[j] - w[3 + j] + w[6 + j]);
    gg[3][j] = w[6 + j];
  }
  E* U = static_cast<E*>(a.u);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float u[4] = {gg[r][0], 0.5f * (gg[r][0] + gg[r][1] + gg[r][2]),
                        0.5f * (gg[r][0] - gg[r][1] + gg[r][2]), gg[r][2]};
#pragma unroll
    for (int c = 0; c < 4; ++c) U[(long long)(4 * r + c) * plane + i] = from_f32<E>(u[c]);
  }
}

template <typename E, int CB>
__global__ __launch_bounds__(256) void wino_kernel(const WinoArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[16 * WN_T * 32 * 4];  // 64 KiB
  E* vbuf = reinterpret_cast<E*>(smem);            // 2 x [16][32][16] (32 KiB)
  float* mbuf = reinterpret_cast<float*>(smem);    // [16][32][32] (64 KiB), after the loop

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * WN_T;
  const int co0 = blockIdx.y * 32 * CB;  // within the group
  const int grp = blockIdx.z;
  const int tpi = a.th * a.tw;
  const E* __restrict__ x = static_cast<const E*>(a.x);
  const E* __restrict__ U = static_cast<const E*>(a.u);
  const long long uplane = (long long)a.c_out * a.cig;

  // this thread's two staging pairs: channel ci_l = p >> 5, tile tl = p & 31
  int tl[2], cil[2], ih0[2], iw0[2];
  bool tok[2];
  const E* xp[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int p = tid + 256 * q;
    cil[q] = p >> 5;
    tl[q] = p & 31;
    const int t = t0 + tl[q];
    tok[q] = t < a.tiles;
    const int tc = tok[q] ? t : 0;
    const int n = (int)mdiv((unsigned)tc, a.mg_tpi);
    const int rem = tc - n * tpi;
    const int th = (int)mdiv((unsigned)rem, a.mg_tw);
    const int tw = rem - th * a.tw;
    ih0[q] = 2 * th - a.pt;
    iw0[q] = 2 * tw - a.pl;
    xp[q] = x + ((long long)n * a.c_in + (long long)grp * a.cig + cil[q]) * a.h * a.w;
  }
  const long long cstride = (long long)WN_KC * a.h * a.w;  // one step of 16 channels

  auto stage = [&](int step, int buf) __attribute__((always_inline)) {
    E* vb = vbuf + buf * WN_VBUF;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      float d[4][4];
      const E* src = xp[q] + step * cstride;
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int ih = ih0[q] + r, iw = iw0[q] + c;
          d[r][c] = (tok[q] && (unsigned)ih < (unsigned)a.h && (unsigned)iw < (unsigned)a.w)
                        ? to_f32(src[(long long)ih * a.w + iw])
                        : 0.0f;
        }
      float bd[4][4];  // B^T d
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        bd[0][c] = d[0][c] - d[2][c];
        bd[1][c] = d[1][c] + d[2][c];
        bd[2][c] = d[2][c] - d[1][c];
        bd[3][c] = d[1][c] - d[3][c];
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {  // (B^T d) B
        const float v[4] = {bd[r][0] - bd[r][2], bd[r][1] + bd[r][2], bd[r][2] - bd[r][1],
                            bd[r][1] - bd[r][3]};
#pragma unroll
        for (int c = 0; c < 4; ++c) vb[((4 * r + c) * WN_T + tl[q]) * WN_KC + cil[q]] = from_f32<E>(v[c]);
      }
    }
  };

  mfma_f32x16 acc[4][CB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int b = 0; b < CB; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][b][e] = 0.0f;

  // A fragments: output channel row (lane & 31) of each 32-channel block (an
  // out-of-range channel reads the last valid one; its results are dropped),
  // channels k0 + 8 * (lane >> 5) .. + 8
  const int kslot = (lane >> 5) * 8;
  long long arow[CB];
#pragma unroll
  for (int b = 0; b < CB; ++b) {
    const int co = min(co0 + 32 * b + (lane & 31), a.cog - 1);
    arow[b] = ((long long)grp * a.cog + co) * a.cig + kslot;
  }

  const int nsteps = a.cig / WN_KC;
  stage(0, 0);
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    const int buf = s & 1;
    u32x4_w af[4][CB];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int b = 0; b < CB; ++b)
        af[i][b] = *reinterpret_cast<const u32x4_w*>(U + (long long)(4 * wave + i) * uplane + arow[b] +
                                                     s * WN_KC);
    if (s + 1 < nsteps) stage(s + 1, buf ^ 1);
    const E* vb = vbuf + buf * WN_VBUF;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4_w bf =
          *reinterpret_cast<const u32x4_w*>(vb + ((4 * wave + i) * WN_T + (lane & 31)) * WN_KC + kslot);
#pragma unroll
      for (int b = 0; b < CB; ++b) acc[i][b] = mfma_32x32x16<E>(af[i][b], bf, acc[i][b]);
    }
    __syncthreads();
  }

  // output transform and epilogue, one 32-channel block at a time
  const E* bias = static_cast<const E*>(a.bias);
  const E* res = static_cast<const E*>(a.res);
  E* y = static_cast<E*>(a.y);
  const int hwo = a.ho * a.wo;
#pragma unroll
  for (int b = 0; b < CB; ++b) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int col = 8 * (e / 4) + 4 * (lane >> 5) + (e & 3);
        mbuf[((4 * wave + i) * 32 + col) * WN_T + (lane & 31)] = acc[i][b][e];
      }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = tid + 256 * q;
      const int col = idx >> 5, tt = idx & 31;
      const int co = co0 + 32 * b + col, t = t0 + tt;
      float m[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) m[k] = mbuf[(k * 32 + col) * WN_T + tt];
      if (co < a.cog && t < a.tiles) {
        float am[2][4];  // A^T M
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          am[0][c] = m[c] + m[4 + c] + m[8 + c];
          am[1][c] = m[4 + c] - m[8 + c] - m[12 + c];
        }
        const int n = (int)mdiv((unsigned)t, a.mg_tpi);
        const int rem = t - n * tpi;
        const int th = (int)mdiv((unsigned)rem, a.mg_tw);
        const int tw = rem - th * a.tw;
        const int cg = grp * a.cog + co;
        const float bv = bias ? to_f32(bias[cg]) : 0.0f;
        const long long obase = ((long long)n * a.c_out + cg) * hwo;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const float yr[2] = {am[r][0] + am[r][1] + am[r][2], am[r][1] - am[r][2] - am[r][3]};
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const int oh = 2 * th + r, ow = 2 * tw + c;
            if (oh < a.ho && ow < a.wo) {
              const long long oi = obase + (long long)oh * a.wo + ow;
              float v = yr[c];
              if (bias) v = v + bv;
              if (res) v = v + to_f32(res[oi]);
              y[oi] = from_f32<E>(apply_act(v, a.act, a.alpha, a.beta));
            }
          }
        }
      }
    }
    __syncthreads();
  }
}

template <typename E>
hipError_t launch_winograd_t(const WinoArgs& a, hipStream_t s) {
  const long long pairs = (long long)a.c_out * a.cig;
  hipLaunchKernelGGL((wino_weights_kernel<E>), dim3((unsigned)((pairs + 255) / 256)), dim3(256), 0,
                     s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned tb = (unsigned)((a.tiles + WN_T - 1) / WN_T);
  if (a.cb == 2) {
    const dim3 grid(tb, (unsigned)((a.cog + 63) / 64), (unsigned)a.groups);
    hipLaunchKernelGGL((wino_kernel<E, 2>), grid, dim3(256), 0, s, a);
  } else {
    const dim3 grid(tb, (unsigned)((a.cog + 31) / 32), (unsigned)a.groups);
    hipLaunchKernelGGL((wino_kernel<E, 1>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_winograd(Dtype dt, const WinoArgs& a, hipStream_t s) {
  if (dt == BF16) return launch_winograd_t<__bf16>(a, s);
  if (dt == F16) return launch_winograd_t<_Float16>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace convfwd
