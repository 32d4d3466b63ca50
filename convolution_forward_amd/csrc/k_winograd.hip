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
//  * Weight kernel: U for every (co, ci) into scratch, 16-bit, laid out
//    [xi][ci / 16][co][ci % 16]: each MFMA A fragment (8 consecutive input
//    channels of one output channel) is one 16-byte load, and the 32 output
//    channels of a fragment load are 1 KiB of contiguous memory (the lines a
//    step reads are whole).  A thread transforms 8 input channels of one
//    output channel (144 contiguous bytes of weights in, one 16-byte store per
//    position out).
//  * Main kernel: a workgroup owns 32 consecutive tiles (in (image, tile row,
//    tile column) order) and 32 * CB output channels; each of its 4 waves owns
//    4 of the 16 positions xi.  Per step of 16 input channels every thread
//    gathers the 4x4 input patches of one tile for 2 adjacent channels, forms
//    V in float32 (adds and subtracts only) and writes its 16 pairs of values,
//    rounded once to the 16-bit type, into LDS laid out [xi][tile][channel]
//    (a B fragment is one 16-byte read); V is double-buffered so one barrier
//    per step suffices.  The input patches and the U fragments are loaded two
//    steps ahead through buffer descriptors: the patch offsets are fixed for
//    the launch (a tap in the padding reads 0 through an offset past the
//    descriptor's range) and a step only adds a scalar offset.
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
constexpr int WN_OOB = (int)0x80000000;     // a byte offset past every descriptor's range

// Raw buffer descriptor (gfx9 format word 0x00020000) over [p, p + bytes), its
// operands made wave-uniform; an access whose per-lane offset is past the range
// reads 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t wino_rsrc(const void* p, int bytes) {
  const unsigned long long v = reinterpret_cast<unsigned long long>(p);
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((unsigned long long)hi << 32) | lo),
                                           (short)0, __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// The 16 bits of an element as float32.
template <typename E>
__device__ __forceinline__ float bits_to_f32(unsigned b) {
  if constexpr (std::is_same_v<E, __bf16>) return __uint_as_float(b << 16);
  else return (float)__builtin_bit_cast(_Float16, (unsigned short)b);
}

// U[xi][ci / 16][co][ci % 16] = (G g G^T)[xi] for every output channel co and
// input channel ci of its group.  A thread takes one output channel and 8 consecutive input
// channels: their 72 weights are 144 contiguous bytes of the OIHW tensor, and
// each position xi receives 8 consecutive U values (one 16-byte store when the
// weights are 16-byte aligned).
template <typename E, bool VEC>
__global__ __launch_bounds__(64) void wino_weights_kernel(const WinoArgs a) {
  typedef E e8 __attribute__((ext_vector_type(8)));
  const int octs = a.cig >> 3;
  const int i = blockIdx.x * 64 + threadIdx.x;  // (co, octet), below c_out * cig / 8
  if (i >= a.c_out * octs) return;
  const int co = i / octs, ci0 = 8 * (i - co * octs);
  const long long plane = (long long)a.c_out * a.cig;
  const E* g = static_cast<const E*>(a.wt) + ((long long)co * a.cig + ci0) * 9;  // [ci][3][3]
  E wv[72];
  if constexpr (VEC) {
#pragma unroll
    for (int k = 0; k < 9; ++k) {
      const e8 v = *reinterpret_cast<const e8*>(g + 8 * k);
#pragma unroll
      for (int e = 0; e < 8; ++e) wv[8 * k + e] = v[e];
    }
  } else {
#pragma unroll
    for (int k = 0; k < 72; ++k) wv[k] = g[k];
  }
  e8 out[16];
#pragma unroll
  for (int c8 = 0; c8 < 8; ++c8) {
    float w[9];
#pragma unroll
    for (int k = 0; k < 9; ++k) w[k] = to_f32(wv[9 * c8 + k]);
    float gg[4][3];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      gg[0][j] = w[j];
      gg[1][j] = 0.5f * (w[j] + w[3 + j] + w[6 + j]);
      gg[2][j] = 0.5f * (w[j] - w[3 + j] + w[6 + j]);
      gg[3][j] = w[6 + j];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      out[4 * r + 0][c8] = from_f32<E>(gg[r][0]);
      out[4 * r + 1][c8] = from_f32<E>(0.5f * (gg[r][0] + gg[r][1] + gg[r][2]));
      out[4 * r + 2][c8] = from_f32<E>(0.5f * (gg[r][0] - gg[r][1] + gg[r][2]));
      out[4 * r + 3][c8] = from_f32<E>(gg[r][2]);
    }
  }
  // 16-byte aligned: scratch, cig % 16 == 0
  E* U = static_cast<E*>(a.u) + ((long long)(ci0 >> 4) * a.c_out + co) * 16 + (ci0 & 15);
#pragma unroll
  for (int xi = 0; xi < 16; ++xi) *reinterpret_cast<e8*>(U + xi * plane) = out[xi];
}

// Main kernel.  Workgroup: a band of tr x tc tiles of one image (tr whole tile
// rows when a tile row has at most 32 tiles, else 32 tiles of one tile row) x
// 32 CB output channels of one group; wave w multiplies the positions
// xi = 4 w .. 4 w + 3.  Per step of 16 input channels:
//  * the band's input window, (2 tr + 2) rows x (2 tc + 2) columns of the 16
//    channels, is copied into LDS laid out [position][channel] (36 bytes per
//    position: 16 channels + 4 bytes that spread the banks); each thread
//    copies up to NSI elements whose offsets are fixed for the launch (a
//    position in the padding reads 0 through an offset past the descriptor's
//    range) plus a scalar step offset, loaded one step ahead;
//  * thread (tile slot tl = tid / 8, channel pair cp = tid % 8) reads its
//    tile's 4 x 4 patch of both channels (one 32-bit LDS read per position),
//    forms V and writes each position's two values as one 32-bit word
//    [xi][tile][channel] (a wave's writes cover 8 whole tiles: 256 contiguous
//    bytes, every bank once);
//  * the U fragments (16-byte loads, two steps ahead) times the V fragments.
// Window and V are double-buffered: one barrier per step.
template <typename E, int CB, int NSI, bool PAIR>
__global__ __launch_bounds__(256) void wino_kernel(const WinoArgs a) {
  typedef E e2 __attribute__((ext_vector_type(2)));
  constexpr int PP = 36;                 // LDS bytes per staged position
  constexpr int WPOS = 264;              // at most (2 tr + 2)(2 tc + 2) positions
  constexpr int WBUF = WPOS * PP + 16;   // window buffer and its sink (items past the window)
  constexpr int VOFF = 2 * WBUF;         // V buffers after the two windows
  __shared__ __attribute__((aligned(16))) unsigned char smem[16 * WN_T * 32 * 4];  // 64 KiB
  static_assert(VOFF + 2 * WN_VBUF * 2 <= 16 * WN_T * 32 * 4, "window and V buffers fit");
  E* vbuf = reinterpret_cast<E*>(smem + VOFF);    // 2 x [16][32][16]
  float* mbuf = reinterpret_cast<float*>(smem);  // [16][32][32], after the loop

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int co0 = blockIdx.y * 32 * CB;  // within the group
  const int grp = blockIdx.z;
  const int hw = a.h * a.w;
  // band: image n, tile rows tr0 .., tile columns tc0 ..
  const int bid = blockIdx.x;
  const int n = (int)mdiv((unsigned)bid, a.mg_nb);
  const int bb = bid - n * (a.nbr * a.nbc);
  const int br = (int)mdiv((unsigned)bb, a.mg_nbc);
  const int tr0 = br * a.tr, tc0 = (bb - br * a.nbc) * a.tc;
  const int C = 2 * a.tc + 2;            // window columns
  const int RC = (2 * a.tr + 2) * C;     // window positions
  const int ih0 = 2 * tr0 - a.pt, iw0 = 2 * tc0 - a.pl;

  // window items of this thread: element (channel, position) of the step
  int gx[NSI], lx[NSI];
  {
    const int xbase = (n * a.c_in + grp * a.cig) * hw;
#pragma unroll
    for (int k = 0; k < NSI; ++k) {
      const int i = tid + 256 * k;
      const int ch = (int)mdiv((unsigned)i, a.mg_rc);
      const int pos = i - ch * RC;
      const int r = (int)mdiv((unsigned)pos, a.mg_c);
      const int ih = ih0 + r, iw = iw0 + pos - r * C;
      const bool live = ch < 16;
      const bool ok = live && (unsigned)ih < (unsigned)a.h && (unsigned)iw < (unsigned)a.w;
      gx[k] = ok ? 2 * (xbase + ch * hw + ih * a.w + iw) : WN_OOB;
      lx[k] = live ? pos * PP + 2 * ch : WPOS * PP;  // items past the window write the sink
    }
  }
  const __amdgpu_buffer_rsrc_t x_rsrc = wino_rsrc(a.x, 2 * a.n * a.c_in * hw);
  const int cstep = 2 * WN_KC * hw;  // bytes from one step's channels to the next

  // this thread's tile slot in the band (slots past the band read the last
  // tile's window; their results are dropped) and channel pair
  const int tl = tid >> 3, cp = tid & 7;
  const int tlc = min(tl, a.tr * a.tc - 1);
  const int tlr = (int)mdiv((unsigned)tlc, a.mg_tc);
  const int pbase = (2 * tlr * C + 2 * (tlc - tlr * a.tc)) * PP + 4 * cp;  // patch corner

  // U fragments: output channel row (lane & 31) of each 32-channel block (an
  // out-of-range channel reads the last valid one; its results are dropped),
  // channels k0 + 8 * (lane >> 5) .. + 8, position 4 wave + i
  const int kslot = (lane >> 5) * 8;
  const int uplane = a.c_out * a.cig;
  const __amdgpu_buffer_rsrc_t u_rsrc = wino_rsrc(a.u, 2 * 16 * uplane);
  int uoff[4][CB];
#pragma unroll
  for (int b = 0; b < CB; ++b) {
    const int co = min(co0 + 32 * b + (lane & 31), a.cog - 1);
    const int row = (grp * a.cog + co) * 16 + kslot;
#pragma unroll
    for (int i = 0; i < 4; ++i) uoff[i][b] = 2 * ((4 * wave + i) * uplane + row);
  }
  const int ustep = 2 * 16 * a.c_out;  // bytes from one step's U block to the next

  unsigned xr[NSI];         // the next step's window items, 16 bits each
  u32x4_w af[2][4][CB];    // [set][position][channel block]
  auto load_x = [&](int s) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < NSI; ++k) xr[k] = __builtin_amdgcn_raw_buffer_load_b16(x_rsrc, gx[k], s * cstep, 0);
  };
  auto put_x = [&](int set) __attribute__((always_inline)) {  // into window buffer `set`
#pragma unroll
    for (int k = 0; k < NSI; ++k)
      *reinterpret_cast<unsigned short*>(smem + set * WBUF + lx[k]) = (unsigned short)xr[k];
  };
  auto load_u = [&](int s, int set) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int b = 0; b < CB; ++b)
        af[set][i][b] = __builtin_bit_cast(
            u32x4_w, __builtin_amdgcn_raw_buffer_load_b128(u_rsrc, uoff[i][b], s * ustep, 0));
  };
  // V = B^T d B of both channels from window buffer `set`, into V buffer `set`
  auto transform = [&](int set) __attribute__((always_inline)) {
    const unsigned char* wb = smem + set * WBUF + pbase;
    float d[2][4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const unsigned w2 = *reinterpret_cast<const unsigned*>(wb + (r * C + c) * PP);
        d[0][r][c] = bits_to_f32<E>(w2 & 0xFFFFu);
        d[1][r][c] = bits_to_f32<E>(w2 >> 16);
      }
    float v[2][16];
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
      float bd[4][4];  // B^T d
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        bd[0][c] = d[ch][0][c] - d[ch][2][c];
        bd[1][c] = d[ch][1][c] + d[ch][2][c];
        bd[2][c] = d[ch][2][c] - d[ch][1][c];
        bd[3][c] = d[ch][1][c] - d[ch][3][c];
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {  // (B^T d) B
        v[ch][4 * r + 0] = bd[r][0] - bd[r][2];
        v[ch][4 * r + 1] = bd[r][1] + bd[r][2];
        v[ch][4 * r + 2] = bd[r][2] - bd[r][1];
        v[ch][4 * r + 3] = bd[r][1] - bd[r][3];
      }
    }
    E* vb = vbuf + set * WN_VBUF;
#pragma unroll
    for (int xi = 0; xi < 16; ++xi) {
      const e2 p = {from_f32<E>(v[0][xi]), from_f32<E>(v[1][xi])};
      *reinterpret_cast<e2*>(vb + (xi * WN_T + tl) * WN_KC + 2 * cp) = p;
    }
  };

  mfma_f32x16 acc[4][CB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int b = 0; b < CB; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][b][e] = 0.0f;

  auto mult = [&](int set) __attribute__((always_inline)) {
    const E* vb = vbuf + set * WN_VBUF;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4_w bf =
          *reinterpret_cast<const u32x4_w*>(vb + ((4 * wave + i) * WN_T + (lane & 31)) * WN_KC + kslot);
#pragma unroll
      for (int b = 0; b < CB; ++b) acc[i][b] = mfma_32x32x16<E>(af[set][i][b], bf, acc[i][b]);
    }
  };
  // Step s (buffers and U registers s & 1): window s + 1 from the registers
  // into LDS and the registers refilled with step s + 2; window s -> V s;
  // barrier; V s times U s and the U registers refilled with step s + 2.
  // The loads a step waits for are then always the oldest ones outstanding.
  // Refills past the last step reread it (unused).
  const int nsteps = a.cig / WN_KC;
  const int last = nsteps - 1;
  auto step = [&](int s, int set) __attribute__((always_inline)) {
    put_x(set ^ 1);
    load_x(min(s + 2, last));
    transform(set);
    __syncthreads();
    mult(set);
    load_u(min(s + 2, last), set);
  };
  load_x(0);
  load_u(0, 0);
  put_x(0);
  load_x(min(1, last));
  load_u(min(1, last), 1);  // as in the loop: the next window's items, then U
  __syncthreads();
  int s = 0;
  for (; s + 1 < nsteps; s += 2) {
    step(s, 0);
    step(s + 1, 1);
  }
  if (s < nsteps) step(s, 0);
  __syncthreads();  // every wave is done with the buffers the output tiles overwrite

  // Output transform and epilogue, one 32-channel block at a time.  A thread
  // finishes 4 (channel, tile) items per block.  The offsets and residual of
  // every block are loaded first, so the residual's latency overlaps the
  // exchange of the sums through LDS; every access is branch-free: an output
  // outside the image gets an offset past the descriptor (its residual reads
  // 0, its store is dropped).  PAIR (even output width, 4-byte aligned y and
  // residual): a tile row's two outputs move as one 32-bit word.  The stores
  // are nontemporal (y is not read back).
  const E* bias = static_cast<const E*>(a.bias);
  const int hwo = a.ho * a.wo;
  const int ybytes = 2 * a.n * a.c_out * hwo;
  const __amdgpu_buffer_rsrc_t y_rsrc = wino_rsrc(a.y, ybytes);
  const __amdgpu_buffer_rsrc_t r_rsrc = wino_rsrc(a.res ? a.res : a.y, a.res ? ybytes : 0);
  const int nslots = a.tr * a.tc;
  int off[CB][4][4];  // [block][item][2 r + c]: byte offset of output (2 th + r, 2 tw + c)
  float bv[CB][4];
#pragma unroll
  for (int b = 0; b < CB; ++b)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = tid + 256 * q;
      const int col = idx >> 5, tt = idx & 31;
      const int co = co0 + 32 * b + col;
      const int ttr = (int)mdiv((unsigned)tt, a.mg_tc);
      const int th = tr0 + ttr, tw = tc0 + tt - ttr * a.tc;
      const bool ok = co < a.cog && tt < nslots && th < a.th && tw < a.tw;
      const int cg = grp * a.cog + min(co, a.cog - 1);
      const int obase = (n * a.c_out + cg) * hwo;
      bv[b][q] = bias ? to_f32(bias[cg]) : 0.0f;
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int oh = 2 * th + r, ow = 2 * tw + c;
          off[b][q][2 * r + c] = ok && oh < a.ho && ow < a.wo ? 2 * (obase + oh * a.wo + ow) : WN_OOB;
        }
    }
  unsigned rw[CB][4][4];  // residual bits (PAIR: word 2 r holds both outputs of row r)
  if (a.res) {
#pragma unroll
    for (int b = 0; b < CB; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          if constexpr (PAIR) {
            rw[b][q][2 * r] = __builtin_amdgcn_raw_buffer_load_b32(r_rsrc, off[b][q][2 * r], 0, 0);
          } else {
#pragma unroll
            for (int c = 0; c < 2; ++c)
              rw[b][q][2 * r + c] = __builtin_amdgcn_raw_buffer_load_b16(r_rsrc, off[b][q][2 * r + c], 0, 0);
          }
        }
  }
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
    float vv[16];  // [item][2 r + c]
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = tid + 256 * q;
      const int col = idx >> 5, tt = idx & 31;
      float m[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) m[k] = mbuf[(k * 32 + col) * WN_T + tt];
      float am[2][4];  // A^T M
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        am[0][c] = m[c] + m[4 + c] + m[8 + c];
        am[1][c] = m[4 + c] - m[8 + c] - m[12 + c];
      }
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const float yr[2] = {am[r][0] + am[r][1] + am[r][2], am[r][1] - am[r][2] - am[r][3]};
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          float v = yr[c];
          if (bias) v = v + bv[b][q];
          if (a.res) {
            const unsigned bits = PAIR ? (c ? rw[b][q][2 * r] >> 16 : rw[b][q][2 * r] & 0xFFFFu) : rw[b][q][2 * r + c];
            v = v + bits_to_f32<E>(bits);
          }
          vv[4 * q + 2 * r + c] = v;
        }
      }
    }
    act_array(vv, a.act, a.alpha, a.beta);  // one uniform switch for all 16 outputs
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const unsigned short o0 = __builtin_bit_cast(unsigned short, from_f32<E>(vv[4 * q + 2 * r]));
        const unsigned short o1 = __builtin_bit_cast(unsigned short, from_f32<E>(vv[4 * q + 2 * r + 1]));
        if constexpr (PAIR) {
          __builtin_amdgcn_raw_buffer_store_b32((unsigned)o0 | ((unsigned)o1 << 16), y_rsrc, off[b][q][2 * r], 0, 2);
        } else {
          __builtin_amdgcn_raw_buffer_store_b16(o0, y_rsrc, off[b][q][2 * r], 0, 2);
          __builtin_amdgcn_raw_buffer_store_b16(o1, y_rsrc, off[b][q][2 * r + 1], 0, 2);
        }
      }
    __syncthreads();
  }
}

template <typename E, int CB, bool PAIR>
void launch_wino_main(const WinoArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.n * a.nbr * a.nbc), (unsigned)((a.cog + 32 * CB - 1) / (32 * CB)),
                  (unsigned)a.groups);
  if (a.nsi == 10) hipLaunchKernelGGL((wino_kernel<E, CB, 10, PAIR>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((wino_kernel<E, CB, 17, PAIR>), grid, dim3(256), 0, s, a);
}

template <typename E>
hipError_t launch_winograd_t(const WinoArgs& a, hipStream_t s) {
  const unsigned items = (unsigned)(a.c_out * (a.cig / 8));  // (output channel, 8 input channels)
  const dim3 wgrid((items + 63) / 64);
  if (reinterpret_cast<unsigned long long>(a.wt) % 16 == 0)
    hipLaunchKernelGGL((wino_weights_kernel<E, true>), wgrid, dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL((wino_weights_kernel<E, false>), wgrid, dim3(64), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // outputs in 32-bit pairs: even output width, y and residual 4-byte aligned
  const bool pair = a.wo % 2 == 0 &&
                    ((reinterpret_cast<unsigned long long>(a.y) | reinterpret_cast<unsigned long long>(a.res)) & 3) == 0;
  if (a.cb == 2) {
    if (pair) launch_wino_main<E, 2, true>(a, s);
    else launch_wino_main<E, 2, false>(a, s);
  } else {
    if (pair) launch_wino_main<E, 1, true>(a, s);
    else launch_wino_main<E, 1, false>(a, s);
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
