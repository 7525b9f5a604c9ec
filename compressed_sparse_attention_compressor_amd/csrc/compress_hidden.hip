// Compressor fed from hidden states ([V4.1] "アーキテクチャ", CED paragraph,
// eq. 1: a decoder layer's KV entries are projected from the encoder's last
// hidden state, C = H W^KV and Z = H W^Z), fused: the projections never
// leave the chip.  Then the softmax-gated pooling of [V4] "ハイブリッド注意：
// CSAとHCA" (CSA paragraph, Fig. 3), the MXFP4 main entry and the bf16
// positional channels.
//
// One workgroup (4 waves) per (E consecutive entries, 64 channels,
// sequence), E = 64/m entries of up to 64 tokens for m <= 64, one entry for
// longer blocks (its tokens in sub-tiles of 64).  Per sub-tile of 64 tokens:
//   1. x and z for 64 tokens x 64 channels on v_mfma_f32_16x16x32_bf16
//      (fp32 accumulation of exact bf16 products), wave w owning tokens
//      16w..16w+15; the H and W tiles of 32 k go through double-buffered LDS,
//      the next step's global loads in flight during the MFMAs.  W is stored
//      k-major as it is in memory and read transposed with
//      ds_read_b64_tr_b16; both operands take the product's k in the order
//      that read produces (MFMA k 8g + 4h + e is tile k 16h + 4g + e).
//      One gate logit per token (G = 1) needs one extra MFMA per step: its
//      B operand repeats W^Z in every column.
//   2. x and z go through LDS to the pooling threads: per (entry, channel)
//      a maximum over the block's logits plus bias, then exp-weighted sums
//      (the stream compressor's arithmetic); blocks longer than a sub-tile
//      keep a running (max, sum, weighted sum) per quarter of the tokens,
//      combined at the end.
//   3. the pooled fp32 values are encoded (MXFP4 blocks of 32 channels, or
//      bf16 for the positional channels) and, when an indexer key follows,
//      written to the workspace for that projection (compress.hip).
#include "csa_device.hpp"
#include "csa_internal.hpp"

namespace csa {

constexpr int kHTok = 64;            // tokens per sub-tile
constexpr int kHCh = 64;             // channels per workgroup
constexpr int kHK = 32;              // k per step
constexpr int kHThreads = 256;
constexpr int kHRowH = kHK + 8;      // H tile row (bf16): 80 bytes
constexpr int kHRowW = kHCh + 16;    // W tile row (bf16): 160 bytes, as the attention key tile's 8-dword skew

struct HiddenArgs {
  const uint16_t *h;       // bf16 [B][*][d_model], row stride d_model, sequence stride h_stride_b
  int64_t h_stride_b;
  int d_model;
  const uint16_t *w_kv;    // bf16 [d_model][576]
  const uint16_t *w_z;     // bf16 [d_model][G]
  const float *bias;       // [m]
  int m;
  int n_ent;               // entries written by the call
  int64_t entry0;          // first of them (token 0 of h is its first token)
  int E;                   // entries per workgroup
  uint8_t *nope;
  uint8_t *nscale;
  uint16_t *rope;
  int N_cap;
  float *pooled;           // fp32 [B][n_ent][576] or null
  int B;                   // sequences
};

// kRB: 16-token row blocks per wave.  With kRB = 2 a sub-tile is 128
// tokens, wave w owning rows 16w..16w+15 of each 64-token half: every k-step
// issues twice the MFMAs per barrier and reuses each W operand read from
// LDS for both row blocks.  The epilogue runs half by half (pool, encode and
// write the half's entries), so the block size must divide 64; kRB = 1 takes
// every other block size, long blocks (m > 64) included.
template <bool kGateFull, int kRB>
__global__ __launch_bounds__(kHThreads) void compress_hidden_kernel(HiddenArgs a) {
  constexpr int kTok = kHTok * kRB;  // tokens per sub-tile
  // One LDS region for both phases of a sub-tile (a barrier separates
  // them): the double-buffered H / W tiles of the k loop, then x, z and the
  // pooled rows of the epilogue (one 64-token half at a time).  At about
  // 49 KB, three workgroups fit on a CU.
  constexpr int kHsB = 2 * kTok * kHRowH * 2, kWxB = 2 * kHK * kHRowW * 2;
  constexpr int kWzB = 2 * (kGateFull ? kHK * kHRowW : kHK) * 2;
  constexpr int kXsB = kHTok * (kHCh + 1) * 4, kZsB = kHTok * (kGateFull ? kHCh + 1 : 1) * 4;
  constexpr int kCsB = kHTok * kHCh * 4;
  constexpr int kLoopB = kHsB + kWxB + kWzB, kEpiB = kXsB + kZsB + kCsB;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kLoopB > kEpiB ? kLoopB : kEpiB];
  auto Hs = reinterpret_cast<uint16_t (*)[kTok * kHRowH]>(smem);
  auto Wx = reinterpret_cast<uint16_t (*)[kHK * kHRowW]>(smem + kHsB);
  auto Wz = reinterpret_cast<uint16_t (*)[kGateFull ? kHK * kHRowW : kHK]>(smem + kHsB + kWxB);
  auto xs = reinterpret_cast<float (*)[kHCh + 1]>(smem);
  auto zs = reinterpret_cast<float (*)[kGateFull ? kHCh + 1 : 1]>(smem + kXsB);
  auto cs = reinterpret_cast<float (*)[kHCh]>(smem + kXsB + kZsB);  // pooled rows of a half, then the long-block combine

  // Workgroup L runs on XCD L % 8.  The 9 channel blocks of one token tile
  // (sequence b, tile t) get ids that share that remainder and follow each
  // other on their XCD, so the tile's hidden states are read from HBM once
  // and then from that XCD's L2.
  const int L = blockIdx.x;
  const int n_tiles = (a.n_ent + a.E - 1) / a.E;
  const int sidx = L >> 3;
  const int T = 8 * (sidx / (kD / kHCh)) + (L & 7);  // sequence-major tile index
  if (T >= n_tiles * a.B) return;  // the whole workgroup, before any barrier
  const int b = T / n_tiles;
  const int c0 = (sidx % (kD / kHCh)) * kHCh;
  const int e0 = (T % n_tiles) * a.E;
  const int ne = min(a.E, a.n_ent - e0);
  const int ntok = ne * a.m;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r = lane & 15;
  const uint16_t *hb = a.h + (int64_t)b * a.h_stride_b + (int64_t)e0 * a.m * a.d_model;
  const int nk = a.d_model / kHK;
  const bool lng = a.m > kHTok;  // one entry, several sub-tiles (kRB = 1 only)
  const int e_half = kRB == 1 ? a.E : kHTok / a.m;  // entries per 64-token half

  // Staging of one k-step: H kTok tokens x 32 k (16 bytes per thread and row
  // block), W^KV 32 k x 64 channels (16 bytes per thread), W^Z likewise or
  // its 32 values.
  const int ht = tid >> 2, hk = (tid & 3) * 8;    // H: token (of a 64-token half), k offset
  const int wk = tid >> 3, wc = (tid & 7) * 8;    // W: k row, channel offset
  struct Stage { uint4 h[kRB], x, z; };
  auto load_step = [&](int st, int ks, Stage &v) __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      const int tok = st + kHTok * rb + ht;
      const uint16_t *hp = hb + (int64_t)min(tok, ntok - 1) * a.d_model + ks * kHK + hk;
      v.h[rb] = *reinterpret_cast<const uint4 *>(hp);
      if (tok >= ntok) v.h[rb] = uint4{0u, 0u, 0u, 0u};
    }
    const int64_t kr = (int64_t)ks * kHK + wk;
    v.x = *reinterpret_cast<const uint4 *>(a.w_kv + kr * kD + c0 + wc);
    if (kGateFull) v.z = *reinterpret_cast<const uint4 *>(a.w_z + kr * kD + c0 + wc);
    else v.z = *reinterpret_cast<const uint4 *>(a.w_z + (int64_t)ks * kHK + min(tid, 3) * 8);
  };
  auto store_step = [&](int buf, const Stage &v) __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb)
      *reinterpret_cast<uint4 *>(&Hs[buf][(kHTok * rb + ht) * kHRowH + hk]) = v.h[rb];
    *reinterpret_cast<uint4 *>(&Wx[buf][wk * kHRowW + wc]) = v.x;
    if (kGateFull) *reinterpret_cast<uint4 *>(&Wz[buf][wk * kHRowW + wc]) = v.z;
    else if (tid < 4) *reinterpret_cast<uint4 *>(&Wz[buf][tid * 8]) = v.z;
  };

  // long blocks: running (max, sum, weighted sum) of channel tid % 64 over
  // token quarter tid / 64 of every sub-tile
  float lmx = -INFINITY, lden = 0.f, lnum = 0.f;

  for (int st = 0; st < ntok; st += kTok) {
    v4f X[kRB][kHCh / 16], Z[kRB][kGateFull ? kHCh / 16 : 1];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
#pragma unroll
      for (int j = 0; j < kHCh / 16; ++j) X[rb][j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < (kGateFull ? kHCh / 16 : 1); ++j) Z[rb][j] = v4f{0.f, 0.f, 0.f, 0.f};
    }

    Stage v;
    load_step(st, 0, v);
    store_step(0, v);
    for (int ks = 0; ks < nk; ++ks) {
      const int buf = ks & 1;
      lds_barrier();  // step ks staged; every wave is done with step ks - 1's buffer
      if (ks + 1 < nk) load_step(st, ks + 1, v);
      // A: token 64 rb + 16 wave + r, k {4g..4g+3, 16+4g..16+4g+3}
      v8bf A[kRB];
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        const uint16_t *hr = &Hs[buf][(kHTok * rb + 16 * wave + r) * kHRowH + 4 * g];
        const uint2 a0 = *reinterpret_cast<const uint2 *>(hr), a1 = *reinterpret_cast<const uint2 *>(hr + 16);
        A[rb] = __builtin_bit_cast(v8bf, uint4{a0.x, a0.y, a1.x, a1.y});
      }
      typedef __attribute__((address_space(3))) v4s lds_v4s;
      const uint16_t *wb = &Wx[buf][(4 * g + (r >> 2)) * kHRowW + 4 * (r & 3)];
#pragma unroll
      for (int j = 0; j < kHCh / 16; ++j) {
        const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(wb + 16 * j));
        const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(wb + 16 * kHRowW + 16 * j));
        const v8bf Bx = __builtin_bit_cast(v8bf, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) X[rb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[rb], Bx, X[rb][j], 0, 0, 0);
      }
      if (kGateFull) {
        const uint16_t *zb = &Wz[buf][(4 * g + (r >> 2)) * kHRowW + 4 * (r & 3)];
#pragma unroll
        for (int j = 0; j < kHCh / 16; ++j) {
          const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(zb + 16 * j));
          const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(zb + 16 * kHRowW + 16 * j));
          const v8bf Bz = __builtin_bit_cast(v8bf, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int rb = 0; rb < kRB; ++rb)
            Z[rb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[rb], Bz, Z[rb][j], 0, 0, 0);
        }
      } else {
        // W^Z in every column: lane (g, r) takes k {4g..4g+3, 16+4g..16+4g+3}
        const uint2 z0 = *reinterpret_cast<const uint2 *>(&Wz[buf][4 * g]);
        const uint2 z1 = *reinterpret_cast<const uint2 *>(&Wz[buf][16 + 4 * g]);
        const v8bf Bz = __builtin_bit_cast(v8bf, uint4{z0.x, z0.y, z1.x, z1.y});
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) Z[rb][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[rb], Bz, Z[rb][0], 0, 0, 0);
      }
      if (ks + 1 < nk) store_step(buf ^ 1, v);
    }

#pragma unroll
    for (int hh = 0; hh < kRB; ++hh) {
      __syncthreads();  // the k loop's tiles (or the previous half) are done with: the region becomes x and z
      // x and z of this 64-token half to LDS: lane (g, r) holds tokens
      // 16 wave + 4g + i, channel 16j + r
#pragma unroll
      for (int j = 0; j < kHCh / 16; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          xs[16 * wave + 4 * g + i][16 * j + r] = X[hh][j][i];
          if (kGateFull) zs[16 * wave + 4 * g + i][16 * j + r] = Z[hh][j][i];
          else if (j == 0 && r == 0) zs[16 * wave + 4 * g + i][0] = Z[hh][0][i];
        }
      __syncthreads();

      if (!lng) {
        // the entries of this half lie in it whole
        const int eh0 = hh * e_half, neh = max(0, min(e_half, ne - eh0));
        for (int p = tid; p < neh * kHCh; p += kHThreads) {
          const int e = p / kHCh, c = p % kHCh;
          const int t0 = e * a.m;
          float mx = -INFINITY;
          for (int i = 0; i < a.m; ++i) mx = fmaxf(mx, zs[t0 + i][kGateFull ? c : 0] + a.bias[i]);
          float den = 0.f, num = 0.f;
          for (int i = 0; i < a.m; ++i) {
            const float w = expf(zs[t0 + i][kGateFull ? c : 0] + a.bias[i] - mx);
            den += w;
            num = fmaf(w, xs[t0 + i][c], num);
          }
          cs[e][c] = num / den;
        }
        __syncthreads();
        // encoding: MXFP4 blocks 2y, 2y + 1 of the main entry, or the bf16
        // positional channels; 16 lanes per 32-channel block
        for (int t = tid; t < (c0 < kDNope ? neh * 32 : 0); t += kHThreads) {
          const int e = t >> 5, half = (t >> 4) & 1, l = t & 15;
          uint32_t sb;
          const uint32_t byte = encode_pair(cs[e][32 * half + 2 * l], cs[e][32 * half + 2 * l + 1], sb);
          const int64_t row = (int64_t)b * a.N_cap + a.entry0 + e0 + eh0 + e;
          const int kb = c0 / 32 + half;
          a.nope[row * kNopeBytes + kb * 16 + l] = (uint8_t)byte;
          if (l == 0) a.nscale[row * kNopeScales + kb] = (uint8_t)sb;
        }
        for (int t = tid; t < (c0 >= kDNope ? neh * kHCh : 0); t += kHThreads) {
          const int e = t / kHCh, c = t % kHCh;
          const int64_t row = (int64_t)b * a.N_cap + a.entry0 + e0 + eh0 + e;
          a.rope[row * kDRope + c] = (uint16_t)f32_to_bf16(cs[e][c]);
        }
        if (a.pooled)
          for (int t = tid; t < neh * kHCh; t += kHThreads) {
            const int e = t / kHCh, c = t % kHCh;
            a.pooled[((int64_t)b * a.n_ent + e0 + eh0 + e) * kD + c0 + c] = cs[e][c];
          }
      } else {
        const int c = tid % kHCh, q4 = tid / kHCh;
        const int i1 = min(kHTok, ntok - st);
        for (int i = q4 * (kHTok / 4); i < min(i1, (q4 + 1) * (kHTok / 4)); ++i) {
          const float v = zs[i][kGateFull ? c : 0] + a.bias[st + i];
          if (v > lmx) {
            const float s = expf(lmx - v);  // 0 on the first token
            lden *= s;
            lnum *= s;
            lmx = v;
          }
          const float w = expf(v - lmx);
          lden += w;
          lnum = fmaf(w, xs[i][c], lnum);
        }
      }
    }
    __syncthreads();  // xs / zs / cs are rewritten by the next sub-tile
  }

  if (lng) {
    // the four token quarters of each channel, combined in quarter order
    float *part = &cs[0][0];  // [3][4][64]: max, sum, weighted sum
    part[(0 * 4 + tid / kHCh) * kHCh + tid % kHCh] = lmx;
    part[(1 * 4 + tid / kHCh) * kHCh + tid % kHCh] = lden;
    part[(2 * 4 + tid / kHCh) * kHCh + tid % kHCh] = lnum;
    __syncthreads();
    float res = 0.f;
    if (tid < kHCh) {
      float M = -INFINITY;
#pragma unroll
      for (int q = 0; q < 4; ++q) M = fmaxf(M, part[(0 * 4 + q) * kHCh + tid]);
      float den = 0.f, num = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float mq = part[(0 * 4 + q) * kHCh + tid];
        const float s = mq == -INFINITY ? 0.f : expf(mq - M);
        den = fmaf(part[(1 * 4 + q) * kHCh + tid], s, den);
        num = fmaf(part[(2 * 4 + q) * kHCh + tid], s, num);
      }
      res = num / den;
    }
    __syncthreads();
    if (tid < kHCh) cs[0][tid] = res;
    __syncthreads();
    // one entry: its encoding as above
    for (int t = tid; t < (c0 < kDNope ? 32 : 0); t += kHThreads) {
      const int half = (t >> 4) & 1, l = t & 15;
      uint32_t sb;
      const uint32_t byte = encode_pair(cs[0][32 * half + 2 * l], cs[0][32 * half + 2 * l + 1], sb);
      const int64_t row = (int64_t)b * a.N_cap + a.entry0 + e0;
      const int kb = c0 / 32 + half;
      a.nope[row * kNopeBytes + kb * 16 + l] = (uint8_t)byte;
      if (l == 0) a.nscale[row * kNopeScales + kb] = (uint8_t)sb;
    }
    for (int t = tid; t < (c0 >= kDNope ? kHCh : 0); t += kHThreads) {
      const int64_t row = (int64_t)b * a.N_cap + a.entry0 + e0;
      a.rope[row * kDRope + t] = (uint16_t)f32_to_bf16(cs[0][t]);
    }
    if (a.pooled)
      for (int t = tid; t < kHCh; t += kHThreads) a.pooled[((int64_t)b * a.n_ent + e0) * kD + c0 + t] = cs[0][t];
  }
}

size_t compress_hidden_ws_bytes(int B, int n_ent, bool has_ik) {
  return has_ik ? (size_t)B * n_ent * kD * sizeof(float) : 0;
}

hipError_t launch_compress_hidden(const uint16_t *h, int64_t h_stride_b, int d_model, const uint16_t *w_kv,
                                  const uint16_t *w_z, int G, const float *bias, const uint16_t *w_ik,
                                  int64_t entry0, int n_ent, const CacheView &c, void *ws, hipStream_t stream) {
  if (n_ent <= 0 || c.B <= 0) return hipSuccess;
  HiddenArgs a;
  a.h = h;
  a.h_stride_b = h_stride_b;
  a.d_model = d_model;
  a.w_kv = w_kv;
  a.w_z = w_z;
  a.bias = bias;
  a.m = c.m;
  a.n_ent = n_ent;
  a.entry0 = entry0;
  // 128-token sub-tiles when the block size divides 64 (the epilogue's
  // halves then hold whole blocks), else 64
  const bool wide = c.m <= kHTok && kHTok % c.m == 0;
  a.E = wide ? 2 * kHTok / c.m : (c.m <= kHTok ? kHTok / c.m : 1);
  a.nope = c.nope;
  a.nscale = c.nscale;
  a.rope = c.rope;
  a.N_cap = c.N_cap;
  a.pooled = w_ik ? reinterpret_cast<float *>(ws) : nullptr;
  a.B = c.B;
  const int64_t tiles = (int64_t)c.B * ((n_ent + a.E - 1) / a.E);
  const dim3 grid((unsigned)(8 * ((tiles + 7) / 8) * (kD / kHCh)));
  if (G == kD && wide)
    compress_hidden_kernel<true, 2><<<grid, kHThreads, 0, stream>>>(a);
  else if (G == kD)
    compress_hidden_kernel<true, 1><<<grid, kHThreads, 0, stream>>>(a);
  else if (wide)
    compress_hidden_kernel<false, 2><<<grid, kHThreads, 0, stream>>>(a);
  else
    compress_hidden_kernel<false, 1><<<grid, kHThreads, 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !w_ik) return e;
  return launch_ikey_from_pooled(a.pooled, w_ik, entry0, n_ent, c, stream);
}

}  // namespace csa
