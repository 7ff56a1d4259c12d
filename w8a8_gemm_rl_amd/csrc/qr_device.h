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

// The GEMM epilogue: fl32(acc) * sx * sw -> bf16 bits (two roundings to fp32,
// one to bf16; no fused multiply-add).
__device__ __forceinline__ uint32_t epi_bf16(float a, float sx, float sw) {
  const float t = a * sx;
  const float y = t * sw;
  return f32_to_bf16_rne(y);
}

// Four codes from fp32 values and the row's step t (t > 0), packed
// little-endian (a -> byte 0). Each value is first divided by t with IEEE
// division (correctly rounded).
//   INT8:    round half to even, clamp to [-127, 127].
//   E4M3FN:  clamp to [-448, 448], then the gfx950 conversion
//            v_cvt_pk_fp8_f32 (OCP E4M3FN, round to nearest even; a negative
//            value that rounds to zero keeps its sign, 0x80). Checked equal
//            to a bit-level software encoder for every fp32 value in
//            [-448, 448], subnormals included.
template <int QT>
__device__ __forceinline__ uint32_t quant_codes4(float a, float b, float c, float d, float t) {
  a = a / t;
  b = b / t;
  c = c / t;
  d = d / t;
  if constexpr (QT == kQInt8) {
    auto q = [](float v) {
      return (uint32_t)(int32_t)fminf(fmaxf(rintf(v), -127.0f), 127.0f) & 0xffu;
    };
    return q(a) | (q(b) << 8) | (q(c) << 16) | (q(d) << 24);
  } else {
    auto cl = [](float v) { return fminf(fmaxf(v, -448.0f), 448.0f); };
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(cl(a), cl(b), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(cl(c), cl(d), w, true);
    return (uint32_t)w;
  }
}

// Absmax of eight bf16 values (one 16-byte chunk of a row).
__device__ __forceinline__ float absmax8_bf16(const uint4 v) {
  float m = fmaxf(fabsf(bf16_lo(v.x)), fabsf(bf16_hi(v.x)));
  m = fmaxf(m, fmaxf(fabsf(bf16_lo(v.y)), fabsf(bf16_hi(v.y))));
  m = fmaxf(m, fmaxf(fabsf(bf16_lo(v.z)), fabsf(bf16_hi(v.z))));
  m = fmaxf(m, fmaxf(fabsf(bf16_lo(v.w)), fabsf(bf16_hi(v.w))));
  return m;
}

// Eight codes of one 16-byte bf16 chunk with step t > 0.
template <int QT>
__device__ __forceinline__ uint2 codes8_bf16(const uint4 v, float t) {
  return make_uint2(quant_codes4<QT>(bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y), t),
                    quant_codes4<QT>(bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w), t));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace qr
