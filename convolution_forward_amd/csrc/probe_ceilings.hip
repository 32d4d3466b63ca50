// Measured ceilings of one MI355X, the yardsticks the benchmark reports next to
// the published peaks ("Convolution, pooling and resize", "Not built, with the
// numbers": a kernel moving the bytes with nothing else to do is a floor no
// implementation can beat).  Built into its own library (libconvprobe.so), used
// only by the benchmark; the convolution library does not contain it.
//
//  * probe_copy: a streaming copy, 16-byte vector loads and stores, every line
//    touched once, as many workgroups as the chip holds, grid-stride.
//  * probe_l2read: reads from the L2 into registers: every workgroup walks the
//    same 2 MiB buffer (it stays in each XCD's L2 after the first touch) with
//    16-byte loads, 8 per thread in flight, and folds what it read into one
//    value per thread; the bytes a CU can pull from L2, which bounds the
//    kernels that stage a tile per CU.
//  * probe_mfma: register-only MFMA loops (independent accumulators, operands
//    never reloaded): v_mfma_f32_32x32x16_f16 (kind 0), v_mfma_f32_16x16x32_f16
//    (kind 1), v_mfma_i32_16x16x64_i8 (kind 2).  Each thread writes one value of
//    its accumulators so that nothing is optimised away.
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src,
                                                   u32x4* __restrict__ dst, long long n) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256)
    __builtin_nontemporal_store(src[i], dst + i);
}

__global__ __launch_bounds__(256) void l2read_kernel(const u32x4* __restrict__ src, int n16, int per_wg,
                                                     unsigned* out) {
  // workgroup b starts 4 KiB * b into the buffer (mod its size); thread t reads
  // vectors start + t + 256 j, j < per_wg, eight loads in flight
  const int start = (int)(((long long)blockIdx.x * 256) % n16);
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int j = 0; j < per_wg; j += 8) {
    u32x4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = src[(start + (int)threadIdx.x + 256 * (j + k)) % n16];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc ^= v[k];
  }
  out[blockIdx.x * 256 + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

template <int KIND>
__global__ __launch_bounds__(256) void mfma_kernel(int iters, float* out) {
  const int lane = threadIdx.x & 63;
  f16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (_Float16)(0.001f * (lane + e));
    b[e] = (_Float16)(0.002f * (lane - e));
  }
  if constexpr (KIND == 0) {
    f32x16 c[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int e = 0; e < 16; ++e) c[k][e] = 0.0f;
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int k = 0; k < 4; ++k) c[k] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c[k], 0, 0, 0);
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) s += c[k][lane & 15];
    out[blockIdx.x * 256 + threadIdx.x] = s;
  } else if constexpr (KIND == 1) {
    f32x4 c[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) c[k] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int k = 0; k < 8; ++k) c[k] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c[k], 0, 0, 0);
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) s += c[k][lane & 3];
    out[blockIdx.x * 256 + threadIdx.x] = s;
  } else {
    const i32x4 ai = __builtin_bit_cast(i32x4, a), bi = __builtin_bit_cast(i32x4, b);
    i32x4 c[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) c[k] = i32x4{0, 0, 0, 0};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int k = 0; k < 8; ++k) c[k] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ai, bi, c[k], 0, 0, 0);
    int s = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) s += c[k][lane & 3];
    out[blockIdx.x * 256 + threadIdx.x] = (float)s;
  }
}

}  // namespace

extern "C" {

// Copies n16 16-byte vectors from src to dst (device pointers) on stream.
int probe_copy(const void* src, void* dst, long long n16, int blocks, void* stream) {
  if (!src || !dst || n16 < 1 || blocks < 1) return 1;
  hipLaunchKernelGGL(copy_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n16);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

// Each of blocks workgroups reads per_wg x 4 KiB (per_wg a multiple of 8) from
// the n16 16-byte vectors at buf (a power of two, at most 2^27); out holds
// blocks * 256 values.
int probe_l2read(const void* buf, int n16, int per_wg, int blocks, void* out, void* stream) {
  if (!buf || !out || n16 < 256 || (n16 & (n16 - 1)) || n16 > (1 << 27) || per_wg < 8 || per_wg % 8 ||
      blocks < 1)
    return 1;
  hipLaunchKernelGGL(l2read_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(buf), n16, per_wg, static_cast<unsigned*>(out));
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

// Runs blocks workgroups of 4 waves, each wave iters x (4 or 8) MFMAs of the
// kind; out holds blocks * 256 floats.  MACs per launch: blocks * 4 * iters *
// (4 * 32*32*16, 8 * 16*16*32 or 8 * 16*16*64).
int probe_mfma(int kind, int iters, int blocks, float* out, void* stream) {
  if (!out || iters < 1 || blocks < 1) return 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (kind == 0) hipLaunchKernelGGL(mfma_kernel<0>, dim3(blocks), dim3(256), 0, s, iters, out);
  else if (kind == 1) hipLaunchKernelGGL(mfma_kernel<1>, dim3(blocks), dim3(256), 0, s, iters, out);
  else if (kind == 2) hipLaunchKernelGGL(mfma_kernel<2>, dim3(blocks), dim3(256), 0, s, iters, out);
  else return 1;
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

}  // extern "C"
