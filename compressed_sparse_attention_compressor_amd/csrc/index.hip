// Lightning-indexer scores ([V4] "ハイブリッド注意：CSAとHCA", CSA paragraph:
// FP4 keys, ReLU-scored multi-head dot product, one score per compressed
// block and query; [V4.1] Fig. 4, Reindex mode: rescoring a candidate list).
//
//   s_j = sum_h w_h * max(0, qI_h . kI_j)
//
// The contraction runs on the gfx950 block-scaled MFMA
// v_mfma_scale_f32_16x16x128_f8f6f4: A = 16 indexer heads x 128 channels of
// E4M3 queries (unit scale byte 127), B = 128 channels x 16 entries of E2M1
// keys with the entries' own E8M0 bytes as the B scales.  For the E2M1
// operand, lane l supplies entry l%16 and channels 32(l/16)..+31 (low nibble
// first), i.e. 16 contiguous key bytes, plus that block's scale byte: a wave
// reads 16 whole 64-byte key rows per instruction (fully coalesced).  The
// E4M3 operand of lane group g holds channels 16g..16g+15 and 64+16g..+15;
// the scale of channel block b comes from lane group b for both operands
// (established with an in-bounds probe of the instruction).  E4M3 x E2M1 products are exact in fp32;
// the 16x16 result (lane l: entry l%16, heads 4(l/16)..+3) goes through
// ReLU and the head weights in registers, then two cross-lane adds finish
// the head sum.
#include "csa_device.hpp"
#include "csa_internal.hpp"

namespace csa {

constexpr int kIdxThreads = 256;     // 4 waves
constexpr int kIdxWaveEntries = 64;  // entries per wave per workgroup
constexpr int kIdxWGEntries = kIdxThreads / 64 * kIdxWaveEntries;

// HT: head tiles of 16 (H_I <= 16 * HT).  QB: queries per wave.
template <int HT, int QB, bool kCand>
__global__ __launch_bounds__(kIdxThreads) void index_scores_kernel(
    const uint8_t *__restrict__ ikey, const uint8_t *__restrict__ iscale, const int32_t *__restrict__ n_entries,
    int N_cap, int d_idx, int m, const uint8_t *__restrict__ q_idx, const float *__restrict__ w_idx, int H_I,
    const int32_t *__restrict__ q_pos, int Q, const int32_t *__restrict__ cand, int C, float *__restrict__ scores,
    int Ns) {
  const int b = blockIdx.z;
  const int q0 = blockIdx.y * QB;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;   // 32-channel block (K group)
  const int r = lane & 15;   // entry within the tile / head row within the head tile
  const int kb = d_idx / 32; // key blocks per entry (2 or 4)
  const int nE = min(n_entries[b], N_cap);

  v8i A[QB][HT];
  float wv[QB][HT][4];
  int vis[QB];
  int vis_max = 0;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int q = q0 + qb;
    const bool qv = q < Q;
    const int p = qv ? q_pos[(int64_t)b * Q + q] : -1;
    vis[qb] = qv ? max(0, min(nE, (p + 1) / m)) : 0;
    vis_max = max(vis_max, vis[qb]);
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const int h = ht * 16 + r;
      // E4M3 operand layout of the instruction: bytes 0..15 of lane group g
      // hold channels 16g..16g+15, bytes 16..31 hold channels 64+16g..+15.
      v8i a = {0, 0, 0, 0, 0, 0, 0, 0};
      if (qv && h < H_I) {
        const uint8_t *qr = q_idx + (((int64_t)b * Q + q) * H_I + h) * d_idx;
        const v4i lo = *reinterpret_cast<const v4i *>(qr + 16 * g);
        a[0] = lo[0];
        a[1] = lo[1];
        a[2] = lo[2];
        a[3] = lo[3];
        if (d_idx > 64) {
          const v4i hi = *reinterpret_cast<const v4i *>(qr + 64 + 16 * g);
          a[4] = hi[0];
          a[5] = hi[1];
          a[6] = hi[2];
          a[7] = hi[3];
        }
      }
      A[qb][ht] = a;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hh = ht * 16 + g * 4 + i;
        wv[qb][ht][i] = (qv && hh < H_I) ? w_idx[((int64_t)b * Q + q) * H_I + hh] : 0.f;
      }
    }
  }

  const int limit = kCand ? C : vis_max;
  const int base = blockIdx.x * kIdxWGEntries + wave * kIdxWaveEntries;
  for (int it = 0; it < kIdxWaveEntries / 16; ++it) {
    const int e0 = base + it * 16;
    if (e0 >= limit) break;
    const int slot = e0 + r;
    int ent = slot;
    bool valid;
    if (kCand) {
      ent = slot < C ? cand[((int64_t)b * Q + q0) * C + slot] : -1;
      valid = ent >= 0 && ent < vis[0];
    } else {
      valid = slot < nE;
    }
    v8i B = {0, 0, 0, 0, 0, 0, 0, 0};
    int sb = 127;
    if (valid && g < kb) {
      const int64_t row = (int64_t)b * N_cap + ent;
      const v4i kv = *reinterpret_cast<const v4i *>(ikey + row * (d_idx / 2) + g * 16);
      B[0] = kv[0];
      B[1] = kv[1];
      B[2] = kv[2];
      B[3] = kv[3];
      sb = iscale[row * kb + g];
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float s = 0.f;
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        v4f acc = {0.f, 0.f, 0.f, 0.f};
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[qb][ht], B, acc, 0, 4, 0, 127, 0, sb);
#pragma unroll
        for (int i = 0; i < 4; ++i) s = fmaf(fmaxf(acc[i], 0.f), wv[qb][ht][i], s);
      }
      s += __shfl_xor(s, 16);
      s += __shfl_xor(s, 32);
      const int q = q0 + qb;
      if (g == 0 && q < Q) {
        float *dst = scores + ((int64_t)b * Q + q) * Ns;
        if (kCand) {
          if (slot < C) dst[slot] = valid ? s : __uint_as_float(kNoScoreBits);
        } else if (slot < vis[qb]) {
          dst[slot] = s;
        }
      }
    }
  }
}

template <int HT, int QB, bool kCand>
static void launch_idx(dim3 grid, hipStream_t stream, const CacheView &c, const uint8_t *q_idx, const float *w_idx,
                       int H_I, const int32_t *q_pos, int Q, const int32_t *cand, int C, float *scores, int Ns) {
  index_scores_kernel<HT, QB, kCand><<<grid, kIdxThreads, 0, stream>>>(
      c.ikey, c.iscale, c.n_entries, c.N_cap, c.d_idx, c.m, q_idx, w_idx, H_I, q_pos, Q, cand, C, scores, Ns);
}

template <int HT>
static void dispatch_idx(const CacheView &c, const uint8_t *q_idx, const float *w_idx, int H_I, const int32_t *q_pos,
                         int Q, const int32_t *cand, int C, float *scores, hipStream_t stream) {
  if (cand) {
    const int Ns = C;
    dim3 grid((C + kIdxWGEntries - 1) / kIdxWGEntries, Q, c.B);
    launch_idx<HT, 1, true>(grid, stream, c, q_idx, w_idx, H_I, q_pos, Q, cand, C, scores, Ns);
  } else if (Q >= 4) {
    dim3 grid((c.N_cap + kIdxWGEntries - 1) / kIdxWGEntries, (Q + 3) / 4, c.B);
    launch_idx<HT, 4, false>(grid, stream, c, q_idx, w_idx, H_I, q_pos, Q, nullptr, 0, scores, c.N_cap);
  } else {
    dim3 grid((c.N_cap + kIdxWGEntries - 1) / kIdxWGEntries, Q, c.B);
    launch_idx<HT, 1, false>(grid, stream, c, q_idx, w_idx, H_I, q_pos, Q, nullptr, 0, scores, c.N_cap);
  }
}

hipError_t launch_index_scores(const CacheView &c, const uint8_t *q_idx, const float *w_idx, int H_I,
                               const int32_t *q_pos, int Q, const int32_t *cand, int C, float *scores,
                               hipStream_t stream) {
  if (H_I <= 16)
    dispatch_idx<1>(c, q_idx, w_idx, H_I, q_pos, Q, cand, C, scores, stream);
  else if (H_I <= 32)
    dispatch_idx<2>(c, q_idx, w_idx, H_I, q_pos, Q, cand, C, scores, stream);
  else
    dispatch_idx<4>(c, q_idx, w_idx, H_I, q_pos, Q, cand, C, scores, stream);
  return hipGetLastError();
}

}  // namespace csa
