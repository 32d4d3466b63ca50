// Implicit-GEMM convolution with the input halo tile staged once per channel
// chunk (gfx950, float16 operands, float32 accumulation).
//
// "Convolution, pooling and resize" ("Variants"): the implicit GEMM gathers the
// input window while it loads the tile, so no column matrix exists; the
// WebGPU page ("El tile con halo") sizes a T x T output tile's input as the tile
// plus a border of the kernel's reach, staged once with a strided cooperative
// loop, a barrier, and the guard on the output after the barrier.
//
// gfx950 design.  A workgroup (4 wave64s) owns TR whole output rows (TCB blocks
// of 16 columns each) of one image and TN = 16*CB output channels of one group.
// The reduction runs over channel chunks of CH = 8*OCT channels.  Per chunk:
//  - the input halo region of the chunk is staged into LDS channel-innermost,
//    [row][col][CH] halves (the 8 channels of an octet are 16 contiguous bytes),
//    from coalesced NCHW reads; padding positions are written as zeros;
//  - the chunk's weights are staged as [tap][co][CH] from contiguous 16-byte
//    reads of the OIHW rows (8 channels x all taps are contiguous per row);
//  - every MFMA v_mfma_f32_16x16x32_f16 consumes 4 "k-slots" (tap, octet), one
//    per 16-lane group: lane l of group j feeds 8 channels of slot 4m+j for
//    output pixel l%16 (A) and output channel l%16 (B); each fragment is a single
//    16-byte LDS read.  Slots past the last tap carry zero weights.
// Double-buffered: the next chunk's global reads are in flight while the current
// chunk multiplies.  Sum order per output: chunks in order, within a chunk the
// MFMA k-slot order; fixed by the shape, so reruns and image chunking agree bit
// for bit.  Epilogue: bias, residual, activation in float32, float16 store.
#include "epilogue.h"
#include "internal.h"
#include "mfma16.h"

namespace convfwd {

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int MAXT = HALO_MAXT;
constexpr int MAXI = HALO_MAXI;


// LDS slot of octet o at position p.  A fragment read has 16 lanes on 16
// consecutive positions with the same octet; with positions OCT*16 bytes apart,
// OCT of those lanes would share banks, so the octet slot is XOR-ed with bits of
// the position to spread the 16 lanes' 16-byte reads over all 64 banks.
template <int OCT>
__device__ __forceinline__ int swz(int p, int o) {
  if constexpr (OCT == 4) return o ^ ((p >> 2) & 3);
  else if constexpr (OCT == 2) return o ^ ((p >> 3) & 1);
  else return o;
}

}  // namespace

template <typename E, int KH, int KW, int OCT, int NT>
__global__ __launch_bounds__(256, 2) void halo_kernel(const HaloArgs a) {
  typedef E half8_t __attribute__((ext_vector_type(8)));
  typedef E half4_t __attribute__((ext_vector_type(4)));
  typedef E half2_t __attribute__((ext_vector_type(2)));

  constexpr int KHW = KH * KW;
  constexpr int SLOTS = KHW * OCT;
  constexpr int NM = (SLOTS + 3) / 4;
  constexpr int CH = 8 * OCT;
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * HALO_BUF_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // logical tile -> (co tile, row tile, image, group); co tile varies fastest, so
  // the co tiles of one input tile run on one XCD and share its L2.
  int bid = xcd_logical(blockIdx.x, gridDim.x);
  const int ct = bid % a.n_ct;
  bid /= a.n_ct;
  const int rt = bid % a.n_rt;
  bid /= a.n_rt;
  const int n = bid % a.n;
  const int g = bid / a.n;

  const int TN = a.cb * 16;
  const int co0 = ct * TN;
  const int oh0 = rt * a.tr;
  const int ih_base = oh0 * a.sh - a.pt;
  const int iw_base = -a.pl;
  const int in_items = a.tih * a.tiw * OCT;
  const int in_bytes = in_items * 16;
  const long long hw_in = (long long)a.h * a.w;

  const E* __restrict__ x = static_cast<const E*>(a.x);
  const E* __restrict__ wt = static_cast<const E*>(a.wt);

  // ---- per-thread staging descriptors (independent of the chunk) ----
  int in_off[MAXI];    // element offset of the octet's channel 0 at this position
  int in_lds[MAXI];    // LDS byte offset inside the input region
  bool in_ok[MAXI];    // inside the image (else zero padding)
  bool in_live[MAXI];  // item exists
#pragma unroll
  for (int i = 0; i < MAXI; ++i) {
    const int q = tid + i * 256;
    in_live[i] = q < in_items;
    const int qq = in_live[i] ? q : 0;
    const int o = qq / (a.tih * a.tiw);
    const int rem = qq - o * (a.tih * a.tiw);
    const int ii = rem / a.tiw;
    const int jj = rem - ii * a.tiw;
    const int ih = ih_base + ii, iw = iw_base + jj;
    in_ok[i] = in_live[i] && (unsigned)ih < (unsigned)a.h && (unsigned)iw < (unsigned)a.w;
    in_off[i] = in_ok[i] ? (int)(((long long)(g * a.cig + 8 * o)) * hw_in + (long long)ih * a.w + iw) : 0;
    const int pos = ii * a.tiw + jj;
    in_lds[i] = (pos * OCT + swz<OCT>(pos, o)) * 16;
  }
  const E* __restrict__ ximg = x + (long long)n * a.c_in * hw_in;

  // weights: item = (co_l, octet) -> KHW contiguous 16-byte vectors
  const int w_item = tid;
  const bool w_live = w_item < TN * OCT;
  const int w_co_l = w_live ? w_item / OCT : 0;
  const int w_o = w_live ? w_item - (w_item / OCT) * OCT : 0;
  const bool w_ok = w_live && (co0 + w_co_l) < a.cog;
  const E* __restrict__ wrow =
      wt + ((long long)(g * a.cog + (w_ok ? co0 + w_co_l : 0)) * a.cig + 8 * w_o) * KHW;

  // Staging registers.  Loads are unconditional (padding items read a valid
  // address and are zeroed at the LDS store) so that no branch forces a wait on
  // memory before the chunk's multiplies are issued.
  half8_t rin[MAXI];
  u32x4_t rw[KHW];

  // items per thread (uniform across the workgroup): a scalar branch per item
  const int ni = (in_items + 255) / 256;
  auto load_chunk = [&](int c) __attribute__((always_inline)) {
    const long long coff = (long long)c * CH * hw_in;
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
      if (i < ni) {
        const E* p = ximg + coff + in_off[i];
#pragma unroll
        for (int e = 0; e < 8; ++e) rin[i][e] = p[e * hw_in];
      }
    }
    const E* pw = wrow + (long long)c * CH * KHW;
    if (a.wvec) {
      const u32x4_t* p = reinterpret_cast<const u32x4_t*>(pw);
#pragma unroll
      for (int v = 0; v < KHW; ++v) rw[v] = p[v];
    } else {  // weights not 16-byte aligned: same values, element loads
#pragma unroll
      for (int v = 0; v < KHW; ++v) {
        half8_t h;
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = pw[v * 8 + e];
        rw[v] = __builtin_bit_cast(u32x4_t, h);
      }
    }
  };

  auto store_chunk = [&](int buf) __attribute__((always_inline)) {
    unsigned char* base = smem + buf * HALO_BUF_BYTES;
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
      half8_t v;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = in_ok[i] ? rin[i][e] : E(0);
      if (i < ni && in_live[i]) *reinterpret_cast<half8_t*>(base + in_lds[i]) = v;
    }
    if (w_live) {
      // the item holds w[co][8 channels][KHW taps]; element e*KHW + t is channel e, tap t
      unsigned char* wb = base + in_bytes;
#pragma unroll
      for (int t = 0; t < KHW; ++t) {
        half8_t v;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          v[e] = w_ok ? __builtin_bit_cast(half8_t, rw[(e * KHW + t) / 8])[(e * KHW + t) % 8]
                      : E(0);
        const int pos = t * TN + w_co_l;
        *reinterpret_cast<half8_t*>(wb + (pos * OCT + swz<OCT>(pos, w_o)) * 16) = v;
      }
    }
  };

  // ---- wave tiles: (row block, co block) pairs ----
  const int RB = a.tr * a.tcb;
  const int cbw = a.cb == 2 ? (wave & 1) : 0;
  const int rb0 = a.cb == 2 ? (wave >> 1) : wave;
  const int rbs = a.cb == 2 ? 2 : 4;
  // NT tiles per wave, a compile-time count so the multiply loop has no
  // branches; tiles past the wave's share (ntile) read a valid position and are
  // dropped at the epilogue.
  int a_lane_off[NT];  // (row*sh*tiw + col*sw) for this lane's pixel in tile i
  int ntile = 0;
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int rb = rb0 + i * rbs;
    if (rb < RB) ntile = i + 1;
    const int rbc = rb < RB ? rb : rb0;
    const int r = rbc / a.tcb, cblk = rbc - (rbc / a.tcb) * a.tcb;
    const int col = cblk * 16 + (lane & 15);
    a_lane_off[i] = (r * a.sh) * a.tiw + col * a.sw;
  }

  floatx4_t acc[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) acc[i] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  const int lg = lane >> 4;
  auto compute_chunk = [&](int buf) __attribute__((always_inline)) {
    const unsigned char* base = smem + buf * HALO_BUF_BYTES;
    const unsigned char* wb = base + in_bytes;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const int s = 4 * m + lg;
      const bool sv = s < SLOTS;
      const int t = sv ? s / OCT : 0;
      const int o = sv ? s - (s / OCT) * OCT : 0;
      const int kh = t / KW, kw = t - (t / KW) * KW;
      const int wpos = t * TN + cbw * 16 + (lane & 15);
      u32x4_t bf = *reinterpret_cast<const u32x4_t*>(wb + (wpos * OCT + swz<OCT>(wpos, o)) * 16);
      if (!sv) bf = u32x4_t{0, 0, 0, 0};
      const int tap_off = (kh * a.dh) * a.tiw + kw * a.dw;
      u32x4_t af[NT];
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        const int pos = a_lane_off[i] + tap_off;
        af[i] = *reinterpret_cast<const u32x4_t*>(base + (pos * OCT + swz<OCT>(pos, o)) * 16);
      }
#pragma unroll
      for (int i = 0; i < NT; ++i)
        acc[i] = mfma_16x16x32<E>(af[i], bf, acc[i]);
    }
  };

  const int nchunks = a.cig / CH;
  load_chunk(0);
  store_chunk(0);
  __syncthreads();
  for (int c = 0; c < nchunks; ++c) {
    const bool more = c + 1 < nchunks;
    load_chunk(more ? c + 1 : c);  // the last iteration re-reads harmlessly
    compute_chunk(c & 1);
    if (more) store_chunk((c + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: the accumulators (lane: pixels 4*(lane/16)+e of a 16-column
  // block, output channel lane % 16) are laid out [channel][row][column] in LDS,
  // then every thread finishes outputs in memory order, so residual reads and
  // stores are contiguous along output rows. ----
  const int TNc = a.cb * 16;
  const int rows = min(a.tr, a.ho - oh0);
  const int tile_px = rows * a.wo;
  float* outt = reinterpret_cast<float*>(smem);  // [TNc][rows * wo]; the loop ended on a barrier
  float* bsm = reinterpret_cast<float*>(smem + 2 * HALO_BUF_BYTES) - 32;
  const E* __restrict__ bias = static_cast<const E*>(a.bias);
  if (tid < TNc) bsm[tid] = (bias && co0 + tid < a.cog) ? (float)bias[g * a.cog + co0 + tid] : 0.f;
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    if (i >= ntile) continue;
    const int rb = rb0 + i * rbs;
    const int r = rb / a.tcb, cblk = rb - (rb / a.tcb) * a.tcb;
    if (r >= rows) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int ow = cblk * 16 + 4 * lg + e;
      if (ow < a.wo) outt[(cbw * 16 + (lane & 15)) * tile_px + r * a.wo + ow] = acc[i][e];
    }
  }
  __syncthreads();
  const E* res = static_cast<const E*>(a.res);
  E* y = static_cast<E*>(a.y);
  const int cvalid = min(TNc, a.cog - co0);
  const int total = cvalid * tile_px;
  const long long hw_out = (long long)a.ho * a.wo;
  const long long cbase = ((long long)n * a.c_out + g * a.cog + co0) * hw_out + (long long)oh0 * a.wo;
  // every residual of the thread is read before its first store (y may alias the
  // residual exactly; every element is read and written by one thread only); the
  // bias went to LDS before the barrier
  constexpr int EPT = 32;  // at most 32 channels x 256 pixels per workgroup tile
  long long oidx[EPT];
  float v[EPT];
#pragma unroll
  for (int k2 = 0; k2 < EPT; ++k2) {
    const int idx = min(tid + 256 * k2, total - 1);
    const int cl = idx / tile_px, rem = idx - cl * tile_px;
    oidx[k2] = cbase + (long long)cl * hw_out + rem;
  }
  if (res) {  // uniform; loads from clamped indices so none sits behind a branch
#pragma unroll
    for (int k2 = 0; k2 < EPT; ++k2) v[k2] = (float)res[oidx[k2]];
  }
#pragma unroll
  for (int k2 = 0; k2 < EPT; ++k2) {
    const int idx = min(tid + 256 * k2, total - 1);
    float s = outt[idx];
    const float bv = bsm[idx / tile_px];  // read outside the condition
    s = a.bias ? s + bv : s;
    if (res) s = s + v[k2];
    v[k2] = s;
  }
  act_array(v, a.act, a.alpha, a.beta);
#pragma unroll
  for (int k2 = 0; k2 < EPT; ++k2)
    if (tid + 256 * k2 < total) y[oidx[k2]] = (E)v[k2];
}

template <typename E, int KH, int KW, int OCT>
static hipError_t launch_halo_o(const HaloArgs& a, hipStream_t s, dim3 grid) {
  const int rb = a.tr * a.tcb;
  const int per_wave = a.cb == 2 ? (rb + 1) / 2 : (rb + 3) / 4;
  if (per_wave <= 4)
    hipLaunchKernelGGL((halo_kernel<E, KH, KW, OCT, 4>), grid, dim3(256), 0, s, a);
  else if (per_wave == 7)
    hipLaunchKernelGGL((halo_kernel<E, KH, KW, OCT, 7>), grid, dim3(256), 0, s, a);
  else if (per_wave <= 8)
    hipLaunchKernelGGL((halo_kernel<E, KH, KW, OCT, 8>), grid, dim3(256), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <typename E, int KH, int KW>
static hipError_t launch_halo_k(const HaloArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((long long)a.n_ct * a.n_rt * a.n * a.groups));
  switch (a.oct) {
    case 4: return launch_halo_o<E, KH, KW, 4>(a, s, grid);
    case 2: return launch_halo_o<E, KH, KW, 2>(a, s, grid);
    case 1: return launch_halo_o<E, KH, KW, 1>(a, s, grid);
    default: return hipErrorInvalidValue;
  }
}

template <typename E>
static hipError_t launch_halo_t(const HaloArgs& a, hipStream_t s) {
  if (a.kh == 3 && a.kw == 3) return launch_halo_k<E, 3, 3>(a, s);
  if (a.kh == 1 && a.kw == 1) return launch_halo_k<E, 1, 1>(a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_halo(Dtype dt, const HaloArgs& a, hipStream_t s) {
  return dt == BF16 ? launch_halo_t<__bf16>(a, s) : launch_halo_t<_Float16>(a, s);
}

}  // namespace convfwd
