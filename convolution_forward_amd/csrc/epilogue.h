// Fused epilogue shared by every kernel: sum -> + bias -> + residual -> activation,
// each step rounded in float32 ("Convolution, pooling and resize", "Layout and
// operands"), then the store in the operand type (float16: round to nearest even).
#pragma once

#include <hip/hip_runtime.h>

#include "internal.h"

namespace convfwd {

template <typename T>
__device__ __forceinline__ float to_f32(T v) { return static_cast<float>(v); }

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

// One output element: v is the float32 sum; idx the flat NCHW output index.
template <typename T>
__device__ __forceinline__ T epilogue_one(float v, const T* bias, const T* res, int co,
                                          long long idx, int act, float alpha, float beta) {
  if (bias) v = v + to_f32(bias[co]);
  if (res) v = v + to_f32(res[idx]);
  return from_f32<T>(apply_act(v, act, alpha, beta));
}

}  // namespace convfwd
