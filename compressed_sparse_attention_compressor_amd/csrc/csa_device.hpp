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

// Round to nearest even (gfx950's v_cvt_pk_bf16_f32); finite inputs only.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
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

// MXFP8 (E4M3 elements) block exponent X = floor(log2 amax) - 8 clamped to
// [-127, 127], as the E8M0 byte X + 127: the exponent field minus 8, and 0
// for maxima below 2^-118 (subnormal and zero maxima included).
__device__ __forceinline__ uint32_t mx8_scale_byte(float amax) {
  int e = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
  return (uint32_t)(e >= 8 ? e - 8 : 0);
}

// Magnitude a >= 0 (already divided by the block scale, exactly) -> E4M3
// code 0..126: nearest value, ties to the even code, saturating at 448.
// Below 2^-6 the codes step by 2^-9 (subnormals, and 2^-6 itself as code 8);
// above, a * 2^(3 - e) in [8, 16) rounds to 8 + the mantissa, a carry to 16
// moving into the exponent.  Scaling by powers of two is exact, and rintf
// rounds half to even.
__device__ __forceinline__ uint32_t e4m3_code(float a) {
  if (a >= 448.0f) return 0x7Eu;
  if (a < 0.015625f) return (uint32_t)__builtin_rintf(a * 512.0f);
  const int e = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;  // -6 .. 8
  const float t = a * __uint_as_float((uint32_t)(130 - e) << 23);  // a * 2^(3 - e)
  return (uint32_t)((e + 7) << 3) + (uint32_t)__builtin_rintf(t) - 8u;
}

// 1 / 2^X for the block byte s (X = s - 127), exactly: 2^(127 - s).
__device__ __forceinline__ float mx_inv_scale(uint32_t s) { return __uint_as_float((254u - s) << 23); }

// Workgroup barrier that orders LDS only: global loads still in flight stay
// in flight (a __syncthreads() also waits for every outstanding global load,
// which defeats fetching ahead across it).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Cross-lane steps on DPP (data-parallel primitives): they run at VALU
// latency, where a ds_bpermute shuffle makes an LDS round trip.  Lanes
// whose DPP source lies outside their row (or rows left out by the row
// mask) read 0.
template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ int dpp_i32(int x) {
  return __builtin_amdgcn_update_dpp(0, x, kCtrl, kRowMask, 0xF, false);
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts by 1, 2, 4, 8
// within each row of 16 lanes, then the row totals carried into the rows
// above (row_bcast:15 into rows 1 and 3, row_bcast:31 into rows 2 and 3).
// acc + the number of lanes below this one whose bit is set in the wave
// mask mk (v_mbcnt_lo / v_mbcnt_hi: two instructions, the add included).
__device__ __forceinline__ int lanes_below(uint64_t mk, int acc) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mk >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mk, (uint32_t)acc));
}

__device__ __forceinline__ int wave_incl_scan(int x) {
  x += dpp_i32<0x111>(x);
  x += dpp_i32<0x112>(x);
  x += dpp_i32<0x114>(x);
  x += dpp_i32<0x118>(x);
  x += dpp_i32<0x142, 0xA>(x);
  x += dpp_i32<0x143, 0xC>(x);
  return x;
}

// Wave-uniform sum and maximum: a butterfly within each row of 16 lanes
// (quad permutes, then rotations by 4 and 8), then the four row results
// read into scalar registers.
__device__ __forceinline__ int wave_sum(int x) {
  x += dpp_i32<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_i32<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_i32<0x124>(x);  // row_ror:4
  x += dpp_i32<0x128>(x);  // row_ror:8
  return __builtin_amdgcn_readlane(x, 0) + __builtin_amdgcn_readlane(x, 16) + __builtin_amdgcn_readlane(x, 32) +
         __builtin_amdgcn_readlane(x, 48);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, (uint32_t)dpp_i32<0xB1>((int)x));
  x = max(x, (uint32_t)dpp_i32<0x4E>((int)x));
  x = max(x, (uint32_t)dpp_i32<0x124>((int)x));
  x = max(x, (uint32_t)dpp_i32<0x128>((int)x));
  const uint32_t a = max((uint32_t)__builtin_amdgcn_readlane((int)x, 0), (uint32_t)__builtin_amdgcn_readlane((int)x, 16));
  const uint32_t b = max((uint32_t)__builtin_amdgcn_readlane((int)x, 32), (uint32_t)__builtin_amdgcn_readlane((int)x, 48));
  return max(a, b);
}

// Reductions over each row of 16 lanes (lanes 16r .. 16r+15), every lane
// of the row receiving the same bits: partners at xor 1 and xor 2 (quad
// permutes), then the mirrored lane within 8 and within 16, so each step
// adds two equal-shaped partial results and the addition order is the same
// (up to commutation) in every lane.
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float x) {
  // every lane has a valid source under these controls, so the old value is
  // never used: leaving it undefined lets the move fold into the consuming
  // max/add as its DPP source operand
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), kCtrl, 0xF, 0xF, true));
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f32<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f32<0x141>(v));  // row_half_mirror
  return fmaxf(v, dpp_f32<0x140>(v));  // row_mirror
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x141>(v);
  return v + dpp_f32<0x140>(v);
}

// Order-preserving map of an fp32 score to uint32 (larger score, larger key).
// -0 and +0 are the same number and get the same key (that of +0).
__device__ __forceinline__ uint32_t score_key(float s) {
  const uint32_t u = s == 0.f ? 0u : __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Encodes the pair (v0, v1) of channels 2t, 2t+1 of a 32-channel block
// spread over 16 consecutive lanes; returns the packed byte and the block's
// scale byte (valid in every lane of the group).
__device__ __forceinline__ uint32_t encode_pair(float v0, float v1, uint32_t &sbyte) {
  float amax = row16_max(fmaxf(fabsf(v0), fabsf(v1)));
  sbyte = mx_scale_byte(amax);
  float inv = mx_inv_scale(sbyte);
  return e2m1_encode(v0, inv) | (e2m1_encode(v1, inv) << 4);
}

// Data-dependent faults: skipped on the device, recorded as bits of a device
// word that csa_read_device_flags returns (the public CSA_FLAG_* values).
constexpr uint32_t kFaultIdxRange = 1u;   // a selected index outside [-1, visible)
constexpr uint32_t kFaultIdxOrder = 2u;   // neighbouring selected indices not strictly ascending
constexpr uint32_t kFaultWindow = 4u;     // window rows of a query missing from the window buffer
constexpr uint32_t kFaultCand = 8u;       // a candidate outside [-1, visible) or not strictly ascending
constexpr uint32_t kFaultEntries = 16u;   // an entry count outside [0, N_cap]

// Sets fault bits with a global (vector-memory) atomic; the word may be absent.
__device__ __forceinline__ void raise_fault(uint32_t *flags, uint32_t bits) {
  if (flags) atomicOr(flags, bits);
}

// Top-k hint: a per-row count of scores by the top 32 - kHintShift bits of their
// order-preserving keys (score_key), written by the indexer launch that
// writes the scores and consumed (and left zero) by the top-k launch.
constexpr int kHintShift = 21;
constexpr int kHintBins = 1 << (32 - kHintShift);

// Marks a workspace score slot that holds no candidate.
constexpr uint32_t kNoScoreBits = 0xFFFFFFFFu;

}  // namespace csa
