// float16 storage type of the float32-arithmetic kernels (the fp32 path and
// the backward pass), with its conversions.  bfloat16 storage is bf16_t.
#pragma once

#include "common.hpp"

namespace aa {

// float16 storage for the float32 kernels (bfloat16 has its own bf16_t)
struct half_t {
  uint16_t bits;
};
__device__ __forceinline__ float to_f32(half_t x) {
  return static_cast<float>(__builtin_bit_cast(_Float16, x.bits));
}
template <>
__device__ __forceinline__ half_t from_f32<half_t>(float x) {
  return half_t{__builtin_bit_cast(uint16_t, static_cast<_Float16>(x))};
}

}  // namespace aa
