// MFMA on 16-bit operands for gfx950: float16 and bfloat16 elements occupy the
// same 16 bytes per lane and the same fragment layout, so a kernel templated on
// its element type E moves the same bits and only picks the instruction here.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

namespace convfwd {

typedef float mfma_f32x4 __attribute__((ext_vector_type(4)));
typedef float mfma_f32x16 __attribute__((ext_vector_type(16)));

// v_mfma_f32_32x32x16_{f16,bf16}: a and b are any 16-byte values holding 8 E.
template <typename E, typename A, typename B>
__device__ __forceinline__ mfma_f32x16 mfma_32x32x16(A a, B b, mfma_f32x16 c) {
  static_assert(sizeof(A) == 16 && sizeof(B) == 16, "8 elements of 16 bits per lane");
  typedef E e8 __attribute__((ext_vector_type(8)));
  if constexpr (std::is_same_v<E, __bf16>)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(e8, a),
                                                   __builtin_bit_cast(e8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(e8, a),
                                                  __builtin_bit_cast(e8, b), c, 0, 0, 0);
}

// v_mfma_f32_16x16x32_{f16,bf16}.
template <typename E, typename A, typename B>
__device__ __forceinline__ mfma_f32x4 mfma_16x16x32(A a, B b, mfma_f32x4 c) {
  static_assert(sizeof(A) == 16 && sizeof(B) == 16, "8 elements of 16 bits per lane");
  typedef E e8 __attribute__((ext_vector_type(8)));
  if constexpr (std::is_same_v<E, __bf16>)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(e8, a),
                                                   __builtin_bit_cast(e8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(e8, a),
                                                  __builtin_bit_cast(e8, b), c, 0, 0, 0);
}

}  // namespace convfwd
