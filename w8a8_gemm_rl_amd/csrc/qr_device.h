// Device helpers shared by the gfx950 kernels of the W8A8 linear.
//
// Number formats:
//   bf16      top half of an IEEE binary32; fp32 -> bf16 rounds to nearest,
//             ties to even.
//   E4M3FN    OCP FP8 E4M3 ("fn": no infinities, S.1111.111 is NaN): bias 7,
//             3 mantissa bits, subnormal spacing 2^-9, largest finite 448.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qr {

constexpr int kQInt8 = 0;
constexpr int kQFp8 = 1;

// Largest code magnitude: the absmax of a row maps to it.
template <int QT>
__device__ __forceinline__ constexpr float qmax() {
  return QT == kQInt8 ? 127.0f : 448.0f;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even. Finite inputs only.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// fp32 (finite) -> E4M3FN byte, saturating to +-448, round to nearest even.
// The sign of v is kept, also when the magnitude rounds to zero.
__device__ __forceinline__ uint32_t f32_to_e4m3fn_sat_rne(float v) {
  v = fminf(fmaxf(v, -448.0f), 448.0f);
  const uint32_t b = __float_as_uint(v);
  const uint32_t sign = (b >> 24) & 0x80u;
  const float av = fabsf(v);
  uint32_t mag;
  if (av < 0.015625f) {
    // Below the smallest normal 2^-6 the spacing is 2^-9: scale exactly by
    // 2^9 and round to an integer 0..8 (8 is the code of 2^-6 itself).
    mag = (uint32_t)rintf(av * 512.0f);
  } else {
    const uint32_t a = b & 0x7fffffffu;
    const uint32_t e = (a >> 23) - 120u;  // biased exponent for bias 7: 1..15
    const uint32_t m = a & 0x7fffffu;
    const uint32_t keep = m >> 20;
    const uint32_t rem = m & 0xfffffu;
    const uint32_t up = (rem > 0x80000u) | ((rem == 0x80000u) & (keep & 1u));
    mag = (e << 3) + keep + up;  // a mantissa carry moves into the exponent
  }
  return sign | mag;
}

// One quantized code from fp32 x and the row's step t (t > 0).
template <int QT>
__device__ __forceinline__ uint32_t quant_code(float x, float t) {
  const float v = x / t;  // IEEE division, correctly rounded
  if constexpr (QT == kQInt8) {
    const float r = fminf(fmaxf(rintf(v), -127.0f), 127.0f);
    return (uint32_t)(int32_t)r & 0xffu;
  } else {
    return f32_to_e4m3fn_sat_rne(v);
  }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace qr
