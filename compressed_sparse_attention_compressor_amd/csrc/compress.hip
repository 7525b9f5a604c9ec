// Compressor: softmax-gated pooling of m raw rows into one cache entry
// ([V4] "ハイブリッド注意：CSAとHCA", CSA paragraph and Fig. 3; Fig. 4 for
// HCA's m = 128), then the MXFP4 main entry, the bf16 rope channels and
// the MXFP4 indexer key kI = W_IK^T c ([V4.1] CSA2 paragraph: the indexer
// key is a projection of the main entry, and entries do not overlap).
//
// One workgroup handles kEPB consecutive entries of one sequence:
//   1. pooling: each task is (entry, 4 channels); it reads the m gate
//      logits twice (max, then exp-weighted sums) and the m KV rows once,
//      with 8-byte vector loads that are contiguous across tasks;
//   2. the pooled fp32 rows sit in LDS and are encoded 2 channels per
//      thread, 16 threads per 32-channel scale block (shuffle max);
//   3. the projection runs on the fp32 pooled values: for each 32-channel
//      key block, 8 slices of 72 channels are accumulated in channel order
//      (fmaf) and then added in slice order; when there are few workgroups
//      (decode appends) the key blocks are spread over gridDim.z.
#include "csa_device.hpp"
#include "csa_internal.hpp"

namespace csa {

constexpr int kEPB = 16;
constexpr int kCompThreads = 256;
constexpr int kSmallM = 8;   // blocks up to this many rows are pooled from registers

// kPooled: the pooled fp32 rows come from `pooled` ([B][n_chunk][576], the
// hidden-state compressor's output) and only the indexer key is made.
template <bool kGateFull, bool kPooled = false>
__global__ __launch_bounds__(kCompThreads) void compress_kernel(
    const uint16_t *__restrict__ x, int64_t x_stride_b, const uint16_t *__restrict__ z, int64_t z_stride_b,
    const float *__restrict__ bias, const uint16_t *__restrict__ w_ik, int m, int n_chunk, int64_t entry0,
    uint8_t *__restrict__ nope, uint8_t *__restrict__ nscale, uint16_t *__restrict__ rope,
    uint8_t *__restrict__ ikey, uint8_t *__restrict__ iscale, int N_cap, int d_idx,
    const float *__restrict__ pooled = nullptr) {
  __shared__ float cs[kEPB][kD];
  __shared__ float ks[kEPB][32];
  __shared__ float kpart[kCompThreads / 32][kEPB][32];

  const int b = blockIdx.y;
  const int j0 = blockIdx.x * kEPB;
  const int ne = min(kEPB, n_chunk - j0);
  const int tid = threadIdx.x;
  const uint16_t *xb = x + (int64_t)b * x_stride_b;
  const uint16_t *zb = z + (int64_t)b * z_stride_b;

  // The W_IK slice of this thread's first key block is loaded before the
  // pooling, so its latency overlaps the raw-row loads.
  constexpr int kParts = kCompThreads / 32;
  constexpr int kSlice = kD / kParts;
  const int ol = tid & 31;
  const int part = tid >> 5;
  const int nkb = w_ik ? d_idx / 32 : 0;
  uint16_t wr[kSlice];
  if ((int)blockIdx.z < nkb) {
    const uint16_t *wp = w_ik + (int64_t)(part * kSlice) * d_idx + blockIdx.z * 32 + ol;
#pragma unroll
    for (int u = 0; u < kSlice; ++u) wr[u] = wp[(int64_t)u * d_idx];
  }

  if (kPooled) {
    for (int t = tid; t < ne * (kD / 4); t += kCompThreads) {
      const int e = t / (kD / 4), c = (t % (kD / 4)) * 4;
      *reinterpret_cast<float4 *>(&cs[e][c]) =
          *reinterpret_cast<const float4 *>(pooled + ((int64_t)b * n_chunk + j0 + e) * kD + c);
    }
  }
  // 1. pooling
  for (int t = tid; t < (kPooled ? 0 : ne * (kD / 4)); t += kCompThreads) {
    const int e = t / (kD / 4);
    const int c = (t % (kD / 4)) * 4;
    const int64_t row0 = (int64_t)(j0 + e) * m;
    float mx[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    float den[4] = {0.f, 0.f, 0.f, 0.f};
    float num[4] = {0.f, 0.f, 0.f, 0.f};
    if (m <= kSmallM) {
      // short blocks: every row of the block is loaded once, up front
      // unconditional loads (row index clamped to the block): loads inside
      // per-lane branches would be issued one after another
      uint2 gz[kSmallM], gx[kSmallM];
#pragma unroll
      for (int i = 0; i < kSmallM; ++i) {
        const int64_t rr = row0 + min(i, m - 1);
        gx[i] = *reinterpret_cast<const uint2 *>(xb + rr * kD + c);
        if (kGateFull) {
          gz[i] = *reinterpret_cast<const uint2 *>(zb + rr * kD + c);
        } else {
          const uint32_t h = zb[rr];
          gz[i] = uint2{h | (h << 16), h | (h << 16)};
        }
      }
      float a[kSmallM][4];
#pragma unroll
      for (int i = 0; i < kSmallM; ++i) {
        if (i < m) {
          const float bi = bias[i];
          a[i][0] = bf16_to_f32(gz[i].x & 0xFFFFu) + bi;
          a[i][1] = bf16_to_f32(gz[i].x >> 16) + bi;
          a[i][2] = bf16_to_f32(gz[i].y & 0xFFFFu) + bi;
          a[i][3] = bf16_to_f32(gz[i].y >> 16) + bi;
#pragma unroll
          for (int u = 0; u < 4; ++u) mx[u] = fmaxf(mx[u], a[i][u]);
        }
      }
#pragma unroll
      for (int i = 0; i < kSmallM; ++i) {
        if (i < m) {
          const float xv[4] = {bf16_to_f32(gx[i].x & 0xFFFFu), bf16_to_f32(gx[i].x >> 16),
                               bf16_to_f32(gx[i].y & 0xFFFFu), bf16_to_f32(gx[i].y >> 16)};
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float w = expf(a[i][u] - mx[u]);
            den[u] += w;
            num[u] = fmaf(w, xv[u], num[u]);
          }
        }
      }
    } else {
      // long blocks (HCA): two passes over the rows; unrolled so that eight
      // rows' loads are in flight at once (a runtime loop would wait for
      // each load before issuing the next)
#pragma unroll 8
      for (int i = 0; i < m; ++i) {
        const float bi = bias[i];
        if (kGateFull) {
          uint2 gg = *reinterpret_cast<const uint2 *>(zb + (row0 + i) * kD + c);
          mx[0] = fmaxf(mx[0], bf16_to_f32(gg.x & 0xFFFFu) + bi);
          mx[1] = fmaxf(mx[1], bf16_to_f32(gg.x >> 16) + bi);
          mx[2] = fmaxf(mx[2], bf16_to_f32(gg.y & 0xFFFFu) + bi);
          mx[3] = fmaxf(mx[3], bf16_to_f32(gg.y >> 16) + bi);
        } else {
          const float av = bf16_to_f32(zb[row0 + i]) + bi;
          mx[0] = fmaxf(mx[0], av);
        }
      }
      if (!kGateFull) mx[1] = mx[2] = mx[3] = mx[0];
#pragma unroll 8
      for (int i = 0; i < m; ++i) {
        const float bi = bias[i];
        float a[4];
        if (kGateFull) {
          uint2 gg = *reinterpret_cast<const uint2 *>(zb + (row0 + i) * kD + c);
          a[0] = bf16_to_f32(gg.x & 0xFFFFu) + bi;
          a[1] = bf16_to_f32(gg.x >> 16) + bi;
          a[2] = bf16_to_f32(gg.y & 0xFFFFu) + bi;
          a[3] = bf16_to_f32(gg.y >> 16) + bi;
        } else {
          a[0] = a[1] = a[2] = a[3] = bf16_to_f32(zb[row0 + i]) + bi;
        }
        uint2 v = *reinterpret_cast<const uint2 *>(xb + (row0 + i) * kD + c);
        const float xv[4] = {bf16_to_f32(v.x & 0xFFFFu), bf16_to_f32(v.x >> 16), bf16_to_f32(v.y & 0xFFFFu),
                             bf16_to_f32(v.y >> 16)};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float w = expf(a[u] - mx[u]);
          den[u] += w;
          num[u] = fmaf(w, xv[u], num[u]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) cs[e][c + u] = num[u] / den[u];
  }
  __syncthreads();

  // 2. MXFP4 main entry (bytes 0..255) and bf16 rope channels (workgroup z = 0)
  for (int e = 0; e < (blockIdx.z == 0 && !kPooled ? ne : 0); ++e) {
    const int64_t row = (int64_t)b * N_cap + entry0 + j0 + e;
    uint32_t sb;
    const uint32_t byte = encode_pair(cs[e][2 * tid], cs[e][2 * tid + 1], sb);
    nope[row * kNopeBytes + tid] = (uint8_t)byte;
    if ((tid & 15) == 0) nscale[row * kNopeScales + (tid >> 4)] = (uint8_t)sb;
  }
  for (int t = tid; t < (blockIdx.z == 0 && !kPooled ? ne * kDRope : 0); t += kCompThreads) {
    const int e = t / kDRope, c = t % kDRope;
    const int64_t row = (int64_t)b * N_cap + entry0 + j0 + e;
    rope[row * kDRope + c] = (uint16_t)f32_to_bf16(cs[e][kDNope + c]);
  }
  if (w_ik == nullptr) return;

  // 3. indexer key, one 32-channel block (= one MX block) at a time:
  //    kI[o] = sum_d c[d] * W[d][o].  Thread t owns output o = 32*kb + t%32 and
  //    the channel slice [72p, 72p+72), p = t/32; the 8 partial sums are
  //    added in slice order.  Workgroup z handles blocks z, z+gridDim.z, ...
  for (int kb = blockIdx.z; kb < nkb; kb += gridDim.z) {
    const int o = kb * 32 + ol;
    if (kb != (int)blockIdx.z) {
      // later blocks (many entries per workgroup): the whole slice at once
      const uint16_t *wp = w_ik + (int64_t)(part * kSlice) * d_idx + o;
#pragma unroll
      for (int u = 0; u < kSlice; ++u) wr[u] = wp[(int64_t)u * d_idx];
    }
    float wf[kSlice];
#pragma unroll
    for (int u = 0; u < kSlice; ++u) wf[u] = bf16_to_f32(wr[u]);
    // one entry at a time (a runtime loop: decode appends have ne = 1); the
    // pooled values of the slice are read as 16-byte LDS vectors (the 32
    // lanes of a slice read the same address)
    float acc[kEPB];
    for (int r = 0; r < ne; ++r) {
      const float4 *cp = reinterpret_cast<const float4 *>(&cs[r][part * kSlice]);
      float a = 0.f;
#pragma unroll
      for (int u4 = 0; u4 < kSlice / 4; ++u4) {
        const float4 c4 = cp[u4];
        a = fmaf(c4.x, wf[4 * u4 + 0], a);
        a = fmaf(c4.y, wf[4 * u4 + 1], a);
        a = fmaf(c4.z, wf[4 * u4 + 2], a);
        a = fmaf(c4.w, wf[4 * u4 + 3], a);
      }
      acc[r] = a;
    }
    __syncthreads();  // ks is reused across blocks
    for (int r = 0; r < ne; ++r) kpart[part][r][ol] = acc[r];
    __syncthreads();
    for (int t = tid; t < ne * 32; t += kCompThreads) {
      const int r = t >> 5;
      float s = 0.f;
#pragma unroll
      for (int pp = 0; pp < kParts; ++pp) s += kpart[pp][r][ol];
      ks[r][ol] = s;
    }
    __syncthreads();
    // encode: 16 lanes per (entry, block), two channels each
    {
      const int e = tid >> 4, t = tid & 15;
      const int ec = e < ne ? e : ne - 1;
      uint32_t sb;
      const uint32_t byte = encode_pair(ks[ec][2 * t], ks[ec][2 * t + 1], sb);
      if (e < ne) {
        const int64_t row = (int64_t)b * N_cap + entry0 + j0 + e;
        ikey[row * (d_idx / 2) + kb * 16 + t] = (uint8_t)byte;
        if (t == 0) iscale[row * nkb + kb] = (uint8_t)sb;
      }
    }
  }
}

// Long blocks without an indexer key (HCA, m = 128): one workgroup per
// (entry, sequence, 64-channel group).  Thread (row group rg, channel quad
// q) takes rows rg, rg + 16, ... of its four channels, so each pass issues
// its loads together (m / 16 rows per thread) instead of walking all m rows;
// the row groups' maxima, then their weighted sums, are combined through
// LDS (maximum, then sums in row-group order).  Each term is the same
// exp(a_i - max) as in compress_kernel; only the summation order differs.
// Group g < 8 encodes MX blocks 2g and 2g + 1 of the main entry; group 8
// holds the bf16 rope channels.
constexpr int kLongCh = 64;
constexpr int kLongQuads = kLongCh / 4;
constexpr int kLongRG = kCompThreads / kLongQuads;
static_assert(kD % kLongCh == 0 && kDNope % kLongCh == 0 && kDRope == kLongCh, "channel groups");

template <bool kGateFull>
__global__ __launch_bounds__(kCompThreads) void compress_long_kernel(
    const uint16_t *__restrict__ x, int64_t x_stride_b, const uint16_t *__restrict__ z, int64_t z_stride_b,
    const float *__restrict__ bias, int m, int64_t entry0, uint8_t *__restrict__ nope, uint8_t *__restrict__ nscale,
    uint16_t *__restrict__ rope, int N_cap) {
  __shared__ float red_a[kLongRG][kLongCh];
  __shared__ float red_b[kLongRG][kLongCh];
  __shared__ float cs[kLongCh];
  const int j = blockIdx.x, b = blockIdx.y, cg = blockIdx.z;
  const int tid = threadIdx.x, q = tid % kLongQuads, rg = tid / kLongQuads;
  const int c = cg * kLongCh + 4 * q;
  const uint16_t *xb = x + (int64_t)b * x_stride_b;
  const uint16_t *zb = z + (int64_t)b * z_stride_b;
  const int64_t row0 = (int64_t)j * m;

  // pass 1: gate maxima of this thread's rows
  float mx[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll 8
  for (int i = rg; i < m; i += kLongRG) {
    const float bi = bias[i];
    if (kGateFull) {
      const uint2 gg = *reinterpret_cast<const uint2 *>(zb + (row0 + i) * kD + c);
      mx[0] = fmaxf(mx[0], bf16_to_f32(gg.x & 0xFFFFu) + bi);
      mx[1] = fmaxf(mx[1], bf16_to_f32(gg.x >> 16) + bi);
      mx[2] = fmaxf(mx[2], bf16_to_f32(gg.y & 0xFFFFu) + bi);
      mx[3] = fmaxf(mx[3], bf16_to_f32(gg.y >> 16) + bi);
    } else {
      mx[0] = fmaxf(mx[0], bf16_to_f32(zb[row0 + i]) + bi);
    }
  }
  if (!kGateFull) mx[1] = mx[2] = mx[3] = mx[0];
#pragma unroll
  for (int u = 0; u < 4; ++u) red_a[rg][4 * q + u] = mx[u];
  __syncthreads();
  if (tid < kLongCh) {
    float v = red_a[0][tid];
    for (int r = 1; r < kLongRG; ++r) v = fmaxf(v, red_a[r][tid]);
    cs[tid] = v;
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 4; ++u) mx[u] = cs[4 * q + u];

  // pass 2: weighted sums of this thread's rows
  float den[4] = {0.f, 0.f, 0.f, 0.f};
  float num[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
  for (int i = rg; i < m; i += kLongRG) {
    const float bi = bias[i];
    float a[4];
    if (kGateFull) {
      const uint2 gg = *reinterpret_cast<const uint2 *>(zb + (row0 + i) * kD + c);
      a[0] = bf16_to_f32(gg.x & 0xFFFFu) + bi;
      a[1] = bf16_to_f32(gg.x >> 16) + bi;
      a[2] = bf16_to_f32(gg.y & 0xFFFFu) + bi;
      a[3] = bf16_to_f32(gg.y >> 16) + bi;
    } else {
      a[0] = a[1] = a[2] = a[3] = bf16_to_f32(zb[row0 + i]) + bi;
    }
    const uint2 v = *reinterpret_cast<const uint2 *>(xb + (row0 + i) * kD + c);
    const float xv[4] = {bf16_to_f32(v.x & 0xFFFFu), bf16_to_f32(v.x >> 16), bf16_to_f32(v.y & 0xFFFFu),
                         bf16_to_f32(v.y >> 16)};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float w = expf(a[u] - mx[u]);
      den[u] += w;
      num[u] = fmaf(w, xv[u], num[u]);
    }
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    red_a[rg][4 * q + u] = den[u];
    red_b[rg][4 * q + u] = num[u];
  }
  __syncthreads();
  if (tid < kLongCh) {
    float d = 0.f, n = 0.f;
    for (int r = 0; r < kLongRG; ++r) {
      d += red_a[r][tid];
      n += red_b[r][tid];
    }
    cs[tid] = n / d;
  }
  __syncthreads();

  const int64_t row = (int64_t)b * N_cap + entry0 + j;
  if (cg < kDNope / kLongCh) {
    if (tid < kLongCh / 2) {
      uint32_t sb;
      const uint32_t byte = encode_pair(cs[2 * tid], cs[2 * tid + 1], sb);
      nope[row * kNopeBytes + cg * (kLongCh / 2) + tid] = (uint8_t)byte;
      if ((tid & 15) == 0) nscale[row * kNopeScales + cg * (kLongCh / 32) + (tid >> 4)] = (uint8_t)sb;
    }
  } else if (tid < kDRope) {
    rope[row * kDRope + tid] = (uint16_t)f32_to_bf16(cs[tid]);
  }
}

hipError_t launch_compress(const uint16_t *x, int64_t x_stride_b, const uint16_t *z, int64_t z_stride_b,
                           int G, const float *bias, const uint16_t *w_ik, int64_t entry0, int n_chunk,
                           const CacheView &c, hipStream_t stream) {
  if (n_chunk <= 0 || c.B <= 0) return hipSuccess;
  if (!w_ik && c.m > kSmallM) {
    const dim3 grid((unsigned)n_chunk, c.B, kD / kLongCh);
    if (G == kD)
      compress_long_kernel<true><<<grid, kCompThreads, 0, stream>>>(x, x_stride_b, z, z_stride_b, bias, c.m, entry0,
                                                                    c.nope, c.nscale, c.rope, c.N_cap);
    else
      compress_long_kernel<false><<<grid, kCompThreads, 0, stream>>>(x, x_stride_b, z, z_stride_b, bias, c.m, entry0,
                                                                     c.nope, c.nscale, c.rope, c.N_cap);
    return hipGetLastError();
  }
  // Few workgroups (decode appends): spread the key blocks over workgroups,
  // each recomputing the pooled rows it needs; many: one workgroup per group.
  const int groups = (n_chunk + kEPB - 1) / kEPB;
  const int nkb = w_ik ? c.d_idx / 32 : 1;
  const int zsplit = (int64_t)groups * c.B < 1024 ? nkb : 1;
  dim3 grid(groups, c.B, zsplit);
  if (G == kD)
    compress_kernel<true><<<grid, kCompThreads, 0, stream>>>(x, x_stride_b, z, z_stride_b, bias, w_ik, c.m, n_chunk,
                                                             entry0, c.nope, c.nscale, c.rope, c.ikey, c.iscale,
                                                             c.N_cap, c.d_idx);
  else
    compress_kernel<false><<<grid, kCompThreads, 0, stream>>>(x, x_stride_b, z, z_stride_b, bias, w_ik, c.m, n_chunk,
                                                              entry0, c.nope, c.nscale, c.rope, c.ikey, c.iscale,
                                                              c.N_cap, c.d_idx);
  return hipGetLastError();
}

// The indexer keys of entries whose pooled fp32 rows are already made
// (the hidden-state compressor): stage 3 of compress_kernel alone.
hipError_t launch_ikey_from_pooled(const float *pooled, const uint16_t *w_ik, int64_t entry0, int n_chunk,
                                   const CacheView &c, hipStream_t stream) {
  const int groups = (n_chunk + kEPB - 1) / kEPB;
  const int nkb = c.d_idx / 32;
  const int zsplit = (int64_t)groups * c.B < 1024 ? nkb : 1;
  dim3 grid(groups, c.B, zsplit);
  compress_kernel<true, true><<<grid, kCompThreads, 0, stream>>>(nullptr, 0, nullptr, 0, nullptr, w_ik, c.m, n_chunk,
                                                                  entry0, c.nope, c.nscale, c.rope, c.ikey, c.iscale,
                                                                  c.N_cap, c.d_idx, pooled);
  return hipGetLastError();
}

}  // namespace csa
