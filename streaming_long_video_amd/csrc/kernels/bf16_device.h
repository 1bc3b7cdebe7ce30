// bfloat16 conversions shared by the kernels that round to bf16 themselves.
#pragma once

#include <stdint.h>

namespace skv {

__device__ inline float bf16_bits_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

// Nearest bf16 (8 significant bits, ties to even) of a finite double in the
// float normal range (or zero): round the 52-bit fraction to 7 bits as an
// integer, then the value converts to float exactly.
__device__ inline uint16_t f64_to_bf16_rne(double y) {
  uint64_t u = __builtin_bit_cast(uint64_t, y);
  u += 0xFFFFFFFFFFFull + ((u >> 45) & 1u);
  u &= ~((1ull << 45) - 1);
  const float f = (float)__builtin_bit_cast(double, u);
  return (uint16_t)(__builtin_bit_cast(uint32_t, f) >> 16);
}

}  // namespace skv
