// Device helpers shared by the gfx950 kernels of the paged KV-cache library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace vp {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

template <typename T, typename U>
__device__ __forceinline__ T bitcast(U u) {
  static_assert(sizeof(T) == sizeof(U), "size");
  return __builtin_bit_cast(T, u);
}

// ---- 16-bit <-> fp32 ---------------------------------------------------------

// Two packed bf16 -> two fp32 (exact: bf16 is the upper half of an fp32).
__device__ __forceinline__ void bf16x2_to_f32(uint32_t w, float& lo, float& hi) {
  lo = bitcast<float>(w << 16);
  hi = bitcast<float>(w & 0xFFFF0000u);
}

// Two packed fp16 -> two fp32 (exact).
__device__ __forceinline__ void f16x2_to_f32(uint32_t w, float& lo, float& hi) {
  half2_t h = bitcast<half2_t>(w);
  lo = (float)h.x;
  hi = (float)h.y;
}

template <int F>
__device__ __forceinline__ void x2_to_f32(uint32_t w, float& lo, float& hi) {
  if constexpr (F == kBF16) bf16x2_to_f32(w, lo, hi);
  else f16x2_to_f32(w, lo, hi);
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = bitcast<uint32_t>(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// fp32 -> fp16 bits, round to nearest even (hardware conversion, default mode).
__device__ __forceinline__ uint16_t f32_to_f16_rne(float f) {
  return bitcast<uint16_t>((_Float16)f);
}

template <int F>
__device__ __forceinline__ uint16_t f32_to_16(float f) {
  if constexpr (F == kBF16) return f32_to_bf16_rne(f);
  else return f32_to_f16_rne(f);
}

// ---- OCP FP8 E4M3 -------------------------------------------------------------
//
// Encoder written from the OCP 8-bit floating point specification (E4M3:
// bias 7, 3 mantissa bits, max 448, NaN S.1111.111, no infinities) with
// integer operations on the fp32 bit pattern: saturate to +-448, round to
// nearest with ties to the even code, NaN -> 0x7F | sign, zero keeps its sign.
__device__ __forceinline__ uint32_t e4m3_from_f32(float y) {
  const uint32_t u = bitcast<uint32_t>(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7Fu;          // NaN
  if (a >= 0x43E00000u) return sign | 0x7Eu;         // >= 448 (and inf): saturate
  if (a < 0x3C800000u) {                             // below 2^-6: spacing 2^-9
    // |y| * 2^9 is exact; round it to the nearest even integer (0..8).
    float r = __builtin_rintf(bitcast<float>(a) * 512.0f);
    return sign | (uint32_t)r;                       // 8 is the code of 2^-6
  }
  const uint32_t e = (a >> 23) - 127u + 7u;          // 1 .. 15
  const uint32_t mant = a & 0x7FFFFFu;
  const uint32_t keep = mant >> 20;                  // top 3 mantissa bits
  const uint32_t rest = mant & 0xFFFFFu;             // 20 dropped bits
  uint32_t code = (e << 3) | keep;
  code += (rest > 0x80000u) || (rest == 0x80000u && (keep & 1u));
  return sign | code;                                // never reaches 0x7F below 448
}

// Encoder written from the OCP specification for E5M2 (bias 15, 2 mantissa
// bits, max finite 57344, infinities S.11111.00, NaN S.11111.xx) with the
// same rule: saturate to +-57344 (infinities included), round to nearest with
// ties to the even code, NaN -> 0x7F | sign, zero keeps its sign.
__device__ __forceinline__ uint32_t e5m2_from_f32(float y) {
  const uint32_t u = bitcast<uint32_t>(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7Fu;          // NaN
  if (a >= 0x47600000u) return sign | 0x7Bu;         // >= 57344 (and inf): saturate
  if (a < 0x38800000u) {                             // below 2^-14: spacing 2^-16
    // |y| * 2^16 is exact; round it to the nearest even integer (0..4).
    float r = __builtin_rintf(bitcast<float>(a) * 65536.0f);
    return sign | (uint32_t)r;                       // 4 is the code of 2^-14
  }
  const uint32_t e = (a >> 23) - 127u + 15u;         // 1 .. 30
  const uint32_t mant = a & 0x7FFFFFu;
  const uint32_t keep = mant >> 21;                  // top 2 mantissa bits
  const uint32_t rest = mant & 0x1FFFFFu;            // 21 dropped bits
  uint32_t code = (e << 2) | keep;
  code += (rest > 0x100000u) || (rest == 0x100000u && (keep & 1u));
  return sign | code;                                // never passes 0x7B below 57344
}

template <int KF>
__device__ __forceinline__ uint32_t fp8_from_f32(float y) {
  static_assert(KF == kE4M3 || KF == kE5M2, "FP8 format");
  if constexpr (KF == kE4M3) return e4m3_from_f32(y);
  else return e5m2_from_f32(y);
}

// Two 8-bit codes (bytes 2 HI and 2 HI + 1 of w) -> two values of q's 16-bit
// format, exactly (gfx950 conversions; both FP8 formats embed in fp16 and bf16).
template <int KF, int QF, bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_q16(uint32_t w) {
  if constexpr (KF == kE4M3 && QF == kF16)
    return bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
  else if constexpr (KF == kE4M3)
    return bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
  else if constexpr (QF == kF16)
    return bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_f16_bf8(w, 1.0f, HI));
  else
    return bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, HI));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace vp
