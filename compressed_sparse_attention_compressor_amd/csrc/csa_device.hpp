// Device-side helpers of the CSA library: bf16 and MXFP4 (E2M1 + E8M0)
// encode/decode, cross-lane reductions, MFMA operand types.  gfx950 only.
//
// MXFP4 follows the OCP Microscaling format named by [V4.1] section
// "FP4 主 KV キャッシュ": 32 contiguous channels share one E8M0 scale byte,
// elements are E2M1 codes, channel 2i in the low nibble of byte i.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

constexpr int kD = 576;       // channels per KV row
constexpr int kDNope = 512;   // MXFP4 channels
constexpr int kDRope = 64;    // bf16 channels
constexpr int kNopeBytes = kDNope / 2;
constexpr int kNopeScales = kDNope / 32;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned short v8u16 __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round to nearest even; finite inputs only.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// 2^(s - 127) for an E8M0 byte s < 255, exactly (s = 0 is an fp32 subnormal).
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  return s ? __uint_as_float(s << 23) : __uint_as_float(0x00400000u);
}

// E2M1 code (0..15) -> fp32, exactly.
__device__ __forceinline__ float e2m1_to_f32(uint32_t c) {
  uint32_t mag = c & 7u;
  uint32_t bits = mag >= 2u ? (((126u + (mag >> 1)) << 23) | ((mag & 1u) << 22)) : (mag ? 0x3F000000u : 0u);
  return __uint_as_float(bits | ((c & 8u) << 28));
}

// Block exponent X = floor(log2 amax) - 2 clamped to [-127, 127], as the
// E8M0 byte X + 127.  For a normal amax with exponent field e this is
// e - 2; subnormal and zero maxima give X = -127 (byte 0).
__device__ __forceinline__ uint32_t mx_scale_byte(float amax) {
  int e = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
  return (uint32_t)(e >= 2 ? e - 2 : 0);
}

// |v| / 2^X -> E2M1 code with sign: nearest value, ties to the even
// mantissa bit, saturating at 6.  The sign is taken from v itself.
__device__ __forceinline__ uint32_t e2m1_encode(float v, float inv_scale) {
  float a = fabsf(v) * inv_scale;  // exact: multiplication by a power of two
  uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) + (a > 5.0f);
  return c | (v < 0.0f ? 8u : 0u);
}

// 1 / 2^X for the block byte s (X = s - 127), exactly: 2^(127 - s).
__device__ __forceinline__ float mx_inv_scale(uint32_t s) { return __uint_as_float((254u - s) << 23); }

template <int W>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Order-preserving map of an fp32 score to uint32 (larger score, larger key).
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Marks a workspace score slot that holds no candidate.
constexpr uint32_t kNoScoreBits = 0xFFFFFFFFu;

}  // namespace csa
