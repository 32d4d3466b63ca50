// Fused epilogue shared by every kernel: sum -> + bias -> + residual -> activation,
// each step rounded in float32 ("Convolution, pooling and resize", "Layout and
// operands"), then the store in the operand type (float16: round to nearest even).
#pragma once

#include <hip/hip_runtime.h>

#include "internal.h"

namespace convfwd {

template <typename T>
__device__ __forceinline__ float to_f32(T v) { return static_cast<float>(v); }

// Output store marked nontemporal: y is written once and not read back by the
// kernel, so its lines need not sit dirty in the L2 until the end-of-kernel
// release writes them all back at once.
template <typename V>
__device__ __forceinline__ void store_out(V* p, V v) { __builtin_nontemporal_store(v, p); }

template <typename T>
__device__ __forceinline__ T from_f32(float v) { return static_cast<T>(v); }

// Activations in float32 (ONNX operator definitions).  The code is uniform across
// a launch, so the switch is a scalar branch.
__device__ __forceinline__ float apply_act(float v, int act, float alpha, float beta) {
  switch (act) {
    case 0: return v;
    case 1: return v > 0.0f ? v : 0.0f;
    case 2: return tanhf(v);
    case 3: return 1.0f / (1.0f + expf(-v));
    case 4: return v / (1.0f + expf(-v));
    case 5: return fminf(fmaxf(alpha * v + beta, 0.0f), 1.0f);
    case 6: return v * fminf(fmaxf(v * (1.0f / 6.0f) + 0.5f, 0.0f), 1.0f);
    case 7: return fminf(fmaxf(v, alpha), beta);
    case 8: return v >= 0.0f ? v : alpha * v;
    default: return v;
  }
}

// Logistic function from the hardware base-2 exponential and reciprocal
// (v_exp_f32 and v_rcp_f32, about 1 ulp each; scaling the argument by log2 e
// adds |v| 2^-24 relative): within about |v| + 3 float32 ulps of 1 / (1 + e^-v),
// inside a 16-bit output's rounding and the accumulation tolerance (which
// grows with the sum's magnitude, itself at least |v|).  For kernels whose
// outputs are stored in 16 bits; NaN propagates, +-inf give 1 and 0.
__device__ __forceinline__ float logistic_fast(float v) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * v));
}

// FX: sigmoid and SiLU through logistic_fast (16-bit outputs only).
template <int ACT, bool FX = false>
__device__ __forceinline__ float act_t(float v, float alpha, float beta) {
  if constexpr (ACT == 1) return v > 0.0f ? v : 0.0f;
  else if constexpr (ACT == 2) return tanhf(v);
  else if constexpr (ACT == 3 && FX) return logistic_fast(v);
  else if constexpr (ACT == 4 && FX) return v * logistic_fast(v);
  else if constexpr (ACT == 3) return 1.0f / (1.0f + expf(-v));
  else if constexpr (ACT == 4) return v / (1.0f + expf(-v));
  else if constexpr (ACT == 5) return fminf(fmaxf(alpha * v + beta, 0.0f), 1.0f);
  else if constexpr (ACT == 6) return v * fminf(fmaxf(v * (1.0f / 6.0f) + 0.5f, 0.0f), 1.0f);
  else if constexpr (ACT == 7) return fminf(fmaxf(v, alpha), beta);
  else if constexpr (ACT == 8) return v >= 0.0f ? v : alpha * v;
  else return v;
}

// Activation over a thread's whole batch of outputs: one uniform branch, then a
// branch-free loop (an activation switch per element would multiply the code by
// the batch size).
template <bool FX = false, int N>
__device__ __forceinline__ void act_array(float (&v)[N], int act, float alpha, float beta) {
  switch (act) {
#define CONVFWD_ACT_CASE(A)                                                   \
  case A:                                                                     \
    _Pragma("unroll") for (int i = 0; i < N; ++i) v[i] = act_t<A, FX>(v[i], alpha, beta); \
    break;
    CONVFWD_ACT_CASE(1)
    CONVFWD_ACT_CASE(2)
    CONVFWD_ACT_CASE(3)
    CONVFWD_ACT_CASE(4)
    CONVFWD_ACT_CASE(5)
    CONVFWD_ACT_CASE(6)
    CONVFWD_ACT_CASE(7)
    CONVFWD_ACT_CASE(8)
#undef CONVFWD_ACT_CASE
    default: break;
  }
}

// floor(n / d) for a launch-constant divisor (see make_magic); n < 2^31.
__device__ __forceinline__ unsigned mdiv(unsigned n, Magic g) {
  return (__umulhi(g.m, n) + n) >> g.s;
}

// Workgroups are handed to the 8 XCDs round robin (workgroup b runs on XCD b % 8),
// and each XCD has its own L2.  This maps the launch index to a logical index such
// that every XCD receives one contiguous range of logical indices: tiles that
// share an operand (consecutive logical indices) then share an L2 instead of
// fetching that operand once per XCD.  A bijection on [0, total).
__device__ __forceinline__ int xcd_logical(int bid, int total) {
  const int x = bid & 7, q = total >> 3, r = total & 7;
  const int first = x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q;
  return first + (bid >> 3);
}

// One output element: v is the float32 sum; idx the flat NCHW output index.
template <typename T>
__device__ __forceinline__ T epilogue_one(float v, const T* bias, const T* res, int co,
                                          long long idx, int act, float alpha, float beta) {
  if (bias) v = v + to_f32(bias[co]);
  if (res) v = v + to_f32(res[idx]);
  return from_f32<T>(apply_act(v, act, alpha, beta));
}

// The activation fixed at compile time (AK = the ONNX code), or, for AK < 0,
// the launch's code chosen at run time.  A fixed activation keeps the other
// activations' code (and its registers) out of the kernel.  FX: see act_t.
template <int AK, bool FX = false, int N>
__device__ __forceinline__ void act_apply(float (&v)[N], int act, float alpha, float beta) {
  if constexpr (AK < 0) {
    act_array<FX>(v, act, alpha, beta);
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = act_t<AK, FX>(v[i], alpha, beta);
  }
}

}  // namespace convfwd
