// Grouped convolution with 8 input channels per group, float16 operands,
// float32 accumulation, gfx950 ("Convolution, pooling and resize", "Variants":
// the implicit GEMM gathers its window while staging, no column matrix; each
// group is its own GEMM, "Convolutions", section 2.3 on grouped convolution):
//
//   y[n, g*cog + co, oh, ow] = act( sum_{kh,kw,ci} w[g*cog + co, ci, kh, kw] *
//        x[n, g*8 + ci, oh*sh - pt + kh*dh, ow*sw - pl + kw*dw] + bias + res )
//
// One workgroup per (image, group).  The group's 8 input planes, zero padded,
// are staged once in LDS channel-innermost (a 16-byte octet per position), so
// every tap of every output pixel is one b128 read: the window is never
// materialised.  The GEMM per group is M = cog (<= 32 output channels) x
// N = Ho*Wo pixels x K = taps*8, run as v_mfma_f32_32x32x16_f16 with A = the
// weights (output-channel rows; k = two taps of 8 channels) held in registers
// for the whole workgroup and B = 32 output pixels (k = the same two taps).
// The sixteen waves (four per SIMD, so that one wave's latencies hide behind
// another's work) take 32-pixel blocks in turn; the epilogue runs straight from
// the accumulators (lane l: pixel l % 32, channels 4 (l / 32) + i + 8 (i / 4)).
// Per output the sum runs over the taps in pairs (k-step order), each pair in
// the MFMA's internal order.
#include <algorithm>

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

constexpr int GC_MAXTAPS = 10;  // k-steps of two taps: at most 5
constexpr int GC_NT = 1024;     // threads per workgroup: 16 waves, 4 per SIMD

// Raw buffer descriptor (gfx9 format word 0x00020000) over [p, p + bytes), its
// operands made wave-uniform: accesses are 32-bit byte offsets, and an offset
// past the range reads 0 and drops a store (so no access sits behind a branch).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t gc_rsrc(const void* p, int bytes) {
  const unsigned long long v = reinterpret_cast<unsigned long long>(p);
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((unsigned long long)hi << 32) | lo),
                                           (short)0, __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
constexpr int GC_OOB = (int)0x80000000;  // a byte offset past every descriptor's range

}  // namespace

// KS: k-steps (taps <= 2 KS).  CB: 8-channel row groups of the output
// channels (cog <= 8 CB).  VEC: x 8-byte aligned and h * w % 4 == 0.
template <typename E, int KS, int CB, bool VEC, int AK = -1>
__global__ __launch_bounds__(GC_NT) void grouped_c8_kernel(const GroupedArgs a) {
  typedef E half8_t __attribute__((ext_vector_type(8)));
  typedef E half4_t __attribute__((ext_vector_type(4)));
  typedef E half2_t __attribute__((ext_vector_type(2)));

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  u32x4_t* xs = reinterpret_cast<u32x4_t*>(smem);                      // [pos] octets
  u32x4_t* wl = reinterpret_cast<u32x4_t*>(smem + a.xs_bytes);          // [co][tap] octets
  float* bsm = reinterpret_cast<float*>(smem + a.xs_bytes + 32 * GC_MAXTAPS * 16);
  u32x4_t* sink = reinterpret_cast<u32x4_t*>(smem + a.xs_bytes + 32 * GC_MAXTAPS * 16 + 32 * 4);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = blockIdx.x / a.groups, g = blockIdx.x - n * a.groups;
  const int hw = a.h * a.w, howo = a.ho * a.wo;
  const int taps = a.kh * a.kw;
  const E* __restrict__ x = static_cast<const E*>(a.x) + ((long long)n * a.c_in + g * 8) * hw;
  const E* __restrict__ w = static_cast<const E*>(a.wt) + (long long)g * a.cog * 8 * taps;
  const E* bias = static_cast<const E*>(a.bias);
  const E* res = static_cast<const E*>(a.res);
  E* y = static_cast<E*>(a.y);
  const long long obase = ((long long)n * a.c_out + g * a.cog) * howo;

  // ---- loads: 4 consecutive pixels of the 8 planes per item (items beyond the
  // plane clamp to its last group; their LDS writes repeat that group's) ----
  const int groups4 = (hw + 3) / 4;
  constexpr int NI = 4096 / 4 / GC_NT;  // items per thread (planes up to 4096 pixels)
  static_assert(NI == 1, "one item per thread");
  // waves holding no item load and stage nothing (wave-uniform)
  const bool xwave = 64 * __builtin_amdgcn_readfirstlane(wave) < groups4;
  u32x2_t xr[NI][8];
  if (xwave) {
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int q = min(tid + GC_NT * i, groups4 - 1);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if constexpr (VEC) {
        xr[i][e] = *reinterpret_cast<const u32x2_t*>(x + (long long)e * hw + 4 * q);
      } else {
        half4_t h;
#pragma unroll
        for (int j = 0; j < 4; ++j) h[j] = x[(long long)e * hw + min(4 * q + j, hw - 1)];
        xr[i][e] = __builtin_bit_cast(u32x2_t, h);
      }
    }
  }
  }
  // weights (cog x 8 x taps halves, contiguous): thread q < cog taps gathers
  // the 8 input channels of (channel q / taps, tap q % taps), one octet
  const int nwt = a.cog * taps;  // <= 32 x 10 < GC_NT
  const bool wwave = 64 * __builtin_amdgcn_readfirstlane(wave) < nwt;  // uniform
  const int wq = min(tid, nwt - 1);
  const int wco = (int)mdiv((unsigned)wq, a.mg_taps), wt = wq - wco * taps;
  half8_t wv;
  if (wwave) {
#pragma unroll
    for (int ci = 0; ci < 8; ++ci) wv[ci] = w[(wco * 8 + ci) * taps + wt];
  }
  const E bv_in = *(bias ? bias + g * a.cog + min(tid, a.cog - 1) : x);

  // ---- zero the staged plane (padding positions stay zero) and the weight
  // octets (taps past the last and channels past cog stay zero) ----
  const int npos = a.hp * a.wp;
  for (int q = tid; q < npos; q += GC_NT) xs[q] = u32x4_t{0, 0, 0, 0};
  for (int q = tid; q < 32 * GC_MAXTAPS; q += GC_NT) wl[q] = u32x4_t{0, 0, 0, 0};
  __syncthreads();
  // branch-free within a wave: pixels past the plane and dead items write
  // the sink
  if (xwave) {
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int q = tid + GC_NT * i;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int f = 4 * q + j;
      half8_t v;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = __builtin_bit_cast(half4_t, xr[i][e])[j];
      const int fc = min(f, hw - 1);
      const int ih = (int)mdiv((unsigned)fc, a.mg_w), iw = fc - ih * a.w;
      u32x4_t* dst = q < groups4 && f < hw ? xs + (ih + a.pt) * a.wp + iw + a.pl : sink;
      *dst = __builtin_bit_cast(u32x4_t, v);
    }
  }
  }
  if (wwave) *(tid < nwt ? wl + wco * GC_MAXTAPS + wt : sink) = __builtin_bit_cast(u32x4_t, wv);
  // without a bias the slot holds -0.0, whose addition is exact for every
  // value (a zero keeps its sign), so the epilogue adds it unconditionally
  if (tid < 32) bsm[tid] = bias ? (float)bv_in : -0.0f;
  __syncthreads();

  // ---- A fragments: lane l holds output channel l % 32, taps 2 ks + l / 32 ----
  const int hi = lane >> 5;
  u32x4_t af[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) af[ks] = wl[(lane & 31) * GC_MAXTAPS + 2 * ks + hi];
  // tap offsets in the staged plane for this lane's half of each k-step
  int tofs[KS];
  bool tok[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int t = 2 * ks + hi;
    tok[ks] = t < taps;
    const int kh = (int)mdiv((unsigned)t, a.mg_kw), kw = t - kh * a.kw;
    tofs[ks] = tok[ks] ? kh * a.dh * a.wp + kw * a.dw : 0;
  }

  // NB 32-pixel blocks per pass (independent accumulators; one block for 32
  // output channels, which need all 16 accumulator elements); wave w takes
  // passes w, w + 16, ...  Lane l: pixel l % 32 of each block, output channels
  // 8 (i / 4) + 4 (l / 32) + i % 4 for accumulator element i < 4 CB.
  // the group's output (and residual) planes: cog x howo halves from obase
  const int tile_bytes = a.cog * howo * 2;
  const __amdgpu_buffer_rsrc_t y_rsrc = gc_rsrc(y + obase, tile_bytes);
  const __amdgpu_buffer_rsrc_t r_rsrc = gc_rsrc(res ? res + obase : x, res ? tile_bytes : 2);
  const int nblk = (howo + 31) / 32;
  constexpr int NB = CB >= 4 ? 1 : 2;
  for (int b0 = NB * wave; b0 < nblk; b0 += NB * (GC_NT / 64)) {
    floatx16_t acc[NB];
    int pix[NB], pbase[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      pix[u] = 32 * (b0 + u) + (lane & 31);
      const int p = min(pix[u], howo - 1);
      const int oh = (int)mdiv((unsigned)p, a.mg_wo), ow = p - oh * a.wo;
      pbase[u] = oh * a.sh * a.wp + ow * a.sw;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[u][i] = 0.f;
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const u32x4_t v = xs[pbase[u] + tofs[ks]];
        const u32x4_t bf = tok[ks] ? v : u32x4_t{0, 0, 0, 0};
        acc[u] = mfma_32x32x16<E>(af[ks], bf, acc[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      // output (co, pix) at byte offset 2 (co howo + pix); outside the tile
      // (co >= cog or pix >= howo) the offset lies past the descriptors' range
      const int pofs = 2 * (4 * hi * howo + pix[u]);
      const bool pok = pix[u] < howo;
      auto off = [&](int i) __attribute__((always_inline)) {
        const int c8 = 8 * (i / 4) + (i & 3);  // channel less 4 hi
        return pok && c8 + 4 * hi < a.cog ? pofs + 2 * howo * c8 : GC_OOB;
      };
      // at most 8 values at a time (register pressure at four waves per SIMD)
      constexpr int CH = 4 * CB > 8 ? 8 : 4 * CB;
#pragma unroll
      for (int i0 = 0; i0 < 4 * CB; i0 += CH) {
        float v[CH];
#pragma unroll
        for (int j = 0; j < CH; ++j) {
          const int i = i0 + j;
          v[j] = acc[u][i] + bsm[8 * (i / 4) + 4 * hi + (i & 3)];
        }
        if (res) {  // uniform
#pragma unroll
          for (int j = 0; j < CH; ++j)
            v[j] = v[j] + (float)__builtin_bit_cast(E, __builtin_amdgcn_raw_buffer_load_b16(r_rsrc, off(i0 + j), 0, 0));
        }
        act_apply<AK, true>(v, a.act, a.alpha, a.beta);  // 16-bit outputs: fast logistic
#pragma unroll
        for (int j = 0; j < CH; ++j)  // nontemporal: the output is not read back
          __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (E)v[j]), y_rsrc, off(i0 + j), 0, 2);
      }
    }
  }
}

template <typename E>
static hipError_t launch_grouped_t(const GroupedArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((long long)a.n * a.groups));
  const size_t lds = (size_t)a.xs_bytes + 32 * GC_MAXTAPS * 16 + 32 * 4 + 16;  // + the sink
  const int taps = a.kh * a.kw;
  if (taps > GC_MAXTAPS) return hipErrorInvalidValue;
  // ReLU and sigmoid with the activation fixed at compile time on the vector path
#define GC_CASE(KS_, CB_)                                                                      \
  if (a.vec && a.act == 1)                                                                     \
    hipLaunchKernelGGL((grouped_c8_kernel<E, KS_, CB_, true, 1>), grid, dim3(GC_NT), lds, s, a);   \
  else if (a.vec && a.act == 3)                                                                \
    hipLaunchKernelGGL((grouped_c8_kernel<E, KS_, CB_, true, 3>), grid, dim3(GC_NT), lds, s, a);   \
  else if (a.vec) hipLaunchKernelGGL((grouped_c8_kernel<E, KS_, CB_, true>), grid, dim3(GC_NT), lds, s, a); \
  else hipLaunchKernelGGL((grouped_c8_kernel<E, KS_, CB_, false>), grid, dim3(GC_NT), lds, s, a);
#define GC_KS(KS_)                          \
  if (a.cog <= 8) { GC_CASE(KS_, 1) }       \
  else if (a.cog <= 16) { GC_CASE(KS_, 2) } \
  else { GC_CASE(KS_, 4) }
  if (taps <= 2) {
    GC_KS(1)
  } else if (taps <= 4) {
    GC_KS(2)
  } else {
    GC_KS(5)
  }
#undef GC_KS
#undef GC_CASE
  return hipGetLastError();
}

hipError_t launch_grouped(Dtype dt, const GroupedArgs& a, hipStream_t s) {
  return dt == BF16 ? launch_grouped_t<__bf16>(a, s) : launch_grouped_t<_Float16>(a, s);
}

}  // namespace convfwd
