// Sliding-window rows in FP8 ([V4.1] "FP4 主 KV キャッシュ": the window KV
// stays FP8, being sensitive to quantisation).  Each raw row of 576 bf16
// channels becomes three planes: the 512 content channels as MXFP8 (E4M3
// codes, one E8M0 scale byte per 32 channels, the OCP MX scale rule with
// the E4M3 maximum exponent 8), and the 64 positional channels unchanged in
// bf16.  One thread per 32-channel block: a workgroup of 256 threads covers
// 16 rows; the first 8 threads of a row also copy its positional channels.
#include "csa_device.hpp"
#include "csa_internal.hpp"

namespace csa {
namespace {

constexpr int kSwaThreads = 256;
constexpr int kSwaBlocks = kDNope / 32;            // 16 blocks per row
constexpr int kSwaRows = kSwaThreads / kSwaBlocks;  // 16 rows per workgroup

__global__ __launch_bounds__(kSwaThreads) void swa_encode_kernel(const uint16_t *__restrict__ x, int64_t x_stride_b,
                                                                 int S, int64_t rows, uint8_t *__restrict__ codes,
                                                                 uint8_t *__restrict__ scales,
                                                                 uint16_t *__restrict__ rope) {
  const int tid = threadIdx.x;
  const int64_t r = (int64_t)blockIdx.x * kSwaRows + tid / kSwaBlocks;
  const int blk = tid % kSwaBlocks;
  if (r >= rows) return;
  const int64_t b = r / S, s = r % S;
  const uint16_t *row = x + b * x_stride_b + s * kD;
  const uint4 *src = reinterpret_cast<const uint4 *>(row + blk * 32);
  uint32_t w[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = src[i];
    w[4 * i + 0] = v.x;
    w[4 * i + 1] = v.y;
    w[4 * i + 2] = v.z;
    w[4 * i + 3] = v.w;
  }
  float v[32];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    v[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
    v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
    amax = fmaxf(amax, fmaxf(fabsf(v[2 * i]), fabsf(v[2 * i + 1])));
  }
  const uint32_t sb = mx8_scale_byte(amax);
  const float inv = mx_inv_scale(sb);
  uint32_t out[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float x4 = v[4 * i + j];
      const uint32_t c = e4m3_code(fabsf(x4) * inv) | (x4 < 0.0f ? 0x80u : 0u);
      word |= c << (8 * j);
    }
    out[i] = word;
  }
  uint4 *dst = reinterpret_cast<uint4 *>(codes + r * kDNope + blk * 32);
  dst[0] = uint4{out[0], out[1], out[2], out[3]};
  dst[1] = uint4{out[4], out[5], out[6], out[7]};
  scales[r * kSwaBlocks + blk] = (uint8_t)sb;
  if (blk < kDRope / 8)
    reinterpret_cast<uint4 *>(rope + r * kDRope)[blk] = reinterpret_cast<const uint4 *>(row + kDNope)[blk];
}

}  // namespace

hipError_t launch_swa_encode(const uint16_t *x, int64_t x_stride_b, int B, int S, uint8_t *codes, uint8_t *scales,
                             uint16_t *rope, hipStream_t stream) {
  const int64_t rows = (int64_t)B * S;
  if (rows == 0) return hipSuccess;
  const unsigned grid = (unsigned)((rows + kSwaRows - 1) / kSwaRows);
  swa_encode_kernel<<<grid, kSwaThreads, 0, stream>>>(x, x_stride_b, S, rows, codes, scales, rope);
  return hipGetLastError();
}

}  // namespace csa
