// Lightning-indexer scores ([V4] "ハイブリッド注意：CSAとHCA", CSA paragraph:
// FP4 keys, ReLU-scored multi-head dot product, one score per compressed
// block and query; [V4.1] Fig. 4, Reindex mode: rescoring a candidate list).
//
//   s_j = sum_h w_h * max(0, qI_h . kI_j)
//
// The contraction runs on the gfx950 block-scaled MFMA
// v_mfma_scale_f32_16x16x128_f8f6f4: A = 16 indexer heads x 128 channels of
// E4M3 queries (block scales 1 or 2^-3, below), B = 128 channels x 16 entries of E2M1
// keys with the entries' own E8M0 bytes as the B scales.  For the E2M1
// operand, lane l supplies entry l%16 and channels 32(l/16)..+31 (low nibble
// first), i.e. 16 contiguous key bytes, plus that block's scale byte: a wave
// reads 16 whole 64-byte key rows per instruction (fully coalesced).  The
// E4M3 operand of lane group g holds channels 16g..16g+15 and 64+16g..+15;
// the scale of channel block b comes from lane group b for both operands
// (established with an in-bounds probe of the instruction).  E4M3 x E2M1
// products of normal E4M3 codes are exact in fp32, those of subnormal codes
// are not (the instruction keeps them to a multiple of 2^-9 before the
// scales): every query block of 32 channels whose largest magnitude is at
// most 56 is therefore multiplied by 2^3 and given the scale 2^-3, which
// turns its subnormal codes into exact normal ones;
// the 16x16 result (lane l: entry l%16, heads 4(l/16)..+3) goes through
// ReLU and the head weights in registers, then two cross-lane adds finish
// the head sum.
#include "csa_device.hpp"
#include "csa_internal.hpp"

namespace csa {

constexpr int kIdxThreads = 256;     // 4 waves
constexpr int kIdxWaveEntries = 128; // entries per wave per workgroup (groups of 64)
constexpr int kIdxWGEntries = kIdxThreads / 64 * kIdxWaveEntries;

// Sum over the four lane groups of per-lane partial sums of four 16-entry
// tiles (p_j: tile j, entry lane%16): two rounds of permlane swaps, after
// which lane l holds the total of tile l/16, entry l%16.
__device__ __forceinline__ float reduce_scatter4(float p0, float p1, float p2, float p3) {
  const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p2), false, false);
  const auto y = __builtin_amdgcn_permlane32_swap(__float_as_uint(p1), __float_as_uint(p3), false, false);
  const float k0 = __uint_as_float(x[0]) + __uint_as_float(x[1]);
  const float k1 = __uint_as_float(y[0]) + __uint_as_float(y[1]);
  const auto z = __builtin_amdgcn_permlane16_swap(__float_as_uint(k0), __float_as_uint(k1), false, false);
  return __uint_as_float(z[0]) + __uint_as_float(z[1]);
}

// --- Query block rescaling (E4M3, blocks of 32 channels) ------------------
// Nonzero when a byte of the 16 codes has a magnitude above 56 (code 0x66):
// such a block keeps scale 1.
__device__ __forceinline__ uint32_t e4m3_over56(uint4 v) {
  auto o = [](uint32_t w) { return ((w & 0x7F7F7F7Fu) + 0x19191919u) & 0x80808080u; };
  return o(v.x) | o(v.y) | o(v.z) | o(v.w);
}

// Four E4M3 codes times 2^3, exactly, for magnitudes up to 56 (the products
// stay within E4M3's range, 448, and subnormal codes m 2^-9 become the normal
// m 2^-6): decoded to fp32 times 8 and encoded again, two codes per
// conversion, four instructions for the word.
__device__ __forceinline__ uint32_t e4m3_times8(uint32_t w) {
  typedef float v2f __attribute__((ext_vector_type(2)));
  typedef short v2s __attribute__((ext_vector_type(2)));
  const v2f lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 8.0f, false);  // codes 0 and 1, times 8
  const v2f hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 8.0f, true);   // codes 2 and 3
  v2s r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v2s{0, 0}, lo.x, lo.y, 1.0f, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, hi.x, hi.y, 1.0f, true);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint4 e4m3_times8(uint4 v) {
  return uint4{e4m3_times8(v.x), e4m3_times8(v.y), e4m3_times8(v.z), e4m3_times8(v.w)};
}

constexpr int kQScale1 = 127;     // E8M0 byte of 1
constexpr int kQScaleDiv8 = 124;  // E8M0 byte of 2^-3

// A staged 16-byte piece of a query row: pieces 2j and 2j+1 of a row (block
// j) sit in neighbouring lanes.  Rescales the piece when its block allows it
// and returns the block's E8M0 byte.  Every lane of the wave must call it.
__device__ __forceinline__ int e4m3_rescale_piece(uint4 &v) {
  const int over = e4m3_over56(v) != 0u;
  const int blk_over = over | __shfl_xor(over, 1);
  if (!blk_over) v = e4m3_times8(v);
  return blk_over ? kQScale1 : kQScaleDiv8;
}

// The A fragment of lane (g, r) (head row r; channels 16g..16g+15 in words
// 0..3, 64+16g..+15 in words 4..7): blocks g/2 and 2 + g/2, each shared with
// lane group g ^ 1.  Rescales the lane's halves of the blocks that allow it
// and returns the E8M0 byte of block g, the scale this lane supplies.  Every
// lane of the wave must call it.
__device__ __forceinline__ int e4m3_rescale_fragment(v8i &A, int g, int r) {
  const uint4 lo = {(uint32_t)A[0], (uint32_t)A[1], (uint32_t)A[2], (uint32_t)A[3]};
  const uint4 hi = {(uint32_t)A[4], (uint32_t)A[5], (uint32_t)A[6], (uint32_t)A[7]};
  const uint64_t bl = __builtin_amdgcn_ballot_w64(e4m3_over56(lo) != 0u);
  const uint64_t bh = __builtin_amdgcn_ballot_w64(e4m3_over56(hi) != 0u);
  // bit 32 j + r: block j (of the low halves) resp. 2 + j (high) of head r is over
  const uint64_t fl = bl | (bl >> 16), fh = bh | (bh >> 16);
  const int sh = 32 * (g >> 1) + r;
  if (!((fl >> sh) & 1)) {
    const uint4 t = e4m3_times8(lo);
    A[0] = (int)t.x; A[1] = (int)t.y; A[2] = (int)t.z; A[3] = (int)t.w;
  }
  if (!((fh >> sh) & 1)) {
    const uint4 t = e4m3_times8(hi);
    A[4] = (int)t.x; A[5] = (int)t.y; A[6] = (int)t.z; A[7] = (int)t.w;
  }
  return (((g < 2 ? fl : fh) >> (32 * (g & 1) + r)) & 1) ? kQScale1 : kQScaleDiv8;
}

// HT: head tiles of 16 (H_I <= 16 * HT).  QB: queries per wave.  The body of
// one workgroup: entry tile bx, query block by, sequence b; the score of
// entry `skip` (-1: none) is left to another workgroup.
template <int HT, int QB, bool kCand>
__device__ __forceinline__ void index_body(
    const uint8_t *__restrict__ ikey, const uint8_t *__restrict__ iscale, const int32_t *__restrict__ n_entries,
    int N_cap, int d_idx, int m, const uint8_t *__restrict__ q_idx, const float *__restrict__ w_idx, int H_I,
    const int32_t *__restrict__ q_pos, int Q, const int32_t *__restrict__ cand, int C, float *__restrict__ scores,
    int Ns, int bx, int by, int bz, int skip, uint32_t *flags, uint32_t *hint) {
  // Indexer queries of this workgroup (QB queries x 16*HT heads x d_idx bytes),
  // staged once so that the waves read their MFMA fragments from LDS.
  __shared__ __attribute__((aligned(16))) uint8_t qs[QB * HT * 16 * 128];
  __shared__ uint8_t qsc[QB * HT * 16 * 4];  // E8M0 byte of each query block
  // One-query full scans may also count their scores by the top bits of the
  // order-preserving key for the top-k launch (kHintBins per row, added
  // into the row's global counts at the end).
  constexpr bool kHintable = QB == 1 && !kCand;
  __shared__ uint32_t hint_lds[kHintable ? kHintBins : 1];
  const bool use_hint = kHintable && hint != nullptr;
  if (use_hint)
    for (int i = threadIdx.x; i < kHintBins; i += kIdxThreads) hint_lds[i] = 0u;
  const int b = bz;
  const int q0 = by * QB;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;   // 32-channel block (K group)
  const int r = lane & 15;   // entry within the tile / head row within the head tile
  const int kb = d_idx / 32; // key blocks per entry (2 or 4)
  const int base = bx * kIdxWGEntries + wave * kIdxWaveEntries;
  constexpr int kIters = kIdxWaveEntries / 16;
  static_assert(kIters % 4 == 0, "whole groups of four 16-entry tiles");

  // Several queries per workgroup (prefill): a workgroup whose entries are
  // visible to none of its queries has nothing to score (causal prefill skips
  // about half the pairs this way; nothing reads those score slots).  One
  // query (decode) keeps its key stream free of this dependent read.
  if (QB > 1 && !kCand) {
    const int nE = min(n_entries[b], N_cap);
    int vmax = 0;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
      if (q0 + qb < Q) vmax = max(vmax, min(nE, (q_pos[(int64_t)b * Q + q0 + qb] + 1) / m));
    if (bx * kIdxWGEntries >= vmax) return;
  }

  // 1. Small, cache-resident loads first (queries for LDS staging, head
  //    weights, visibility): vector-memory counters retire in order, so
  //    what is issued before the key stream can be waited for alone.
  constexpr int kQBytes = HT * 16 * 128;
  constexpr int kQVec = (QB * kQBytes / 16 + kIdxThreads - 1) / kIdxThreads;
  uint4 qv_stage[kQVec];
#pragma unroll
  for (int u = 0; u < kQVec; ++u) {
    const int i = threadIdx.x + u * kIdxThreads;
    const int qb = i / (kQBytes / 16), rem = (i % (kQBytes / 16)) * 16;
    const int h = rem / 128, c = rem % 128;
    const int q = q0 + qb;
    const bool ok = i < QB * kQBytes / 16 && q < Q && h < H_I && c < d_idx;
    const int64_t off = ok ? (((int64_t)b * Q + q) * H_I + h) * d_idx + c : 0;
    const uint4 v = *reinterpret_cast<const uint4 *>(q_idx + off);
    qv_stage[u] = ok ? v : uint4{0u, 0u, 0u, 0u};
  }
  // Head weights of lane group g: heads 16*ht + 4g .. +3, one 16-byte load
  // per head tile when H_I is a multiple of 4 (then the four are all valid
  // or all beyond H_I) and the weights are 16-byte aligned, else one load
  // per head.
  float w_raw[QB][HT][4];
  if ((H_I & 3) == 0 && (reinterpret_cast<uintptr_t>(w_idx) & 15) == 0) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int qc = min(q0 + qb, Q - 1);
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        const int h0 = ht * 16 + g * 4;
        const float4 v =
            *reinterpret_cast<const float4 *>(w_idx + ((int64_t)b * Q + qc) * H_I + (h0 < H_I ? h0 : 0));
        w_raw[qb][ht][0] = v.x;
        w_raw[qb][ht][1] = v.y;
        w_raw[qb][ht][2] = v.z;
        w_raw[qb][ht][3] = v.w;
      }
    }
  } else {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int qc = min(q0 + qb, Q - 1);
#pragma unroll
      for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int hh = ht * 16 + g * 4 + i;
          w_raw[qb][ht][i] = w_idx[((int64_t)b * Q + qc) * H_I + (hh < H_I ? hh : 0)];
        }
    }
  }

  // 2. Key loads: their addresses depend only on the grid position
  //    (and, for candidates, on the candidate list), so the HBM stream
  //    starts before anything else is known.
  //    The loads are unconditional, from clamped (always in-bounds)
  //    addresses, and masked afterwards: loads inside per-lane branches make
  //    the compiler wait for each one before issuing the next.
  v4i kv[kIters];
  int sbv[kIters];
  int ent[kIters];
  int prv[kCand ? kIters : 1];  // the candidate before each slot (order check)
  bool use[kIters];
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const int slot = base + it * 16 + r;
    int e = slot;
    if (kCand) {
      const int32_t *cp = cand + ((int64_t)b * Q + q0) * C;
      const int sc = min(slot, C - 1);
      e = cp[sc];
      prv[it] = (slot > 0 && slot < C) ? cp[max(sc - 1, 0)] : -1;
    }
    ent[it] = (kCand && slot >= C) ? -1 : e;
    const bool inb = kCand ? (ent[it] >= 0 && ent[it] < N_cap) : (slot < N_cap);
    use[it] = inb && g < kb;
    const int64_t row = (int64_t)b * N_cap + (inb ? e : 0);
    const int gg = g < kb ? g : 0;
    kv[it] = *reinterpret_cast<const v4i *>(ikey + row * (d_idx / 2) + gg * 16);
    sbv[it] = iscale[row * kb + gg];
  }

  float wv[QB][HT][4];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const bool qv = q0 + qb < Q;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hh = ht * 16 + g * 4 + i;
        wv[qb][ht][i] = (qv && hh < H_I) ? w_raw[qb][ht][i] : 0.f;
      }
  }

  // 3. Queries into LDS (zero rows beyond H_I and beyond Q), rescaled by
  //    block, with each block's scale byte.
#pragma unroll
  for (int u = 0; u < kQVec; ++u) {
    const int i = threadIdx.x + u * kIdxThreads;
    const int sc = e4m3_rescale_piece(qv_stage[u]);
    if (i < QB * kQBytes / 16) {
      const int qb = i / (kQBytes / 16), rem = (i % (kQBytes / 16)) * 16;
      *reinterpret_cast<uint4 *>(qs + qb * kQBytes + rem) = qv_stage[u];
      if (!(i & 1)) qsc[i >> 1] = (uint8_t)sc;
    }
  }
  // LDS-only barrier: the key loads stay in flight, each MFMA below waits
  // only for its own tile.
  lds_barrier();
  // E4M3 operand layout of the instruction: bytes 0..15 of lane group g hold
  // channels 16g..16g+15, bytes 16..31 hold channels 64+16g..+15.
  v8i A[QB][HT];
  int sa[QB][HT];  // the scale of block g of head row r
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const uint8_t *qr = qs + qb * (HT * 16 * 128) + (ht * 16 + r) * 128;
      const v4i lo = *reinterpret_cast<const v4i *>(qr + 16 * g);
      const v4i hi = *reinterpret_cast<const v4i *>(qr + 64 + 16 * g);
      A[qb][ht] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      sa[qb][ht] = qsc[(qb * HT * 16 + ht * 16 + r) * 4 + g];
    }

  // 4. Visibility of this workgroup's queries (uniform loads).
  const int nE_raw = n_entries[b];
  const int nE = min(nE_raw, N_cap);
  if (threadIdx.x == 0 && bx == 0 && by == 0 && (nE_raw < 0 || nE_raw > N_cap)) raise_fault(flags, kFaultEntries);
  int vis[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int q = q0 + qb;
    vis[qb] = q < Q ? max(0, min(nE, (q_pos[(int64_t)b * Q + q] + 1) / m)) : 0;
  }

  // 5. Scores, four 16-entry tiles (64 entries) at a time: MFMA, ReLU and
  //    head weights give each lane a partial head sum (its lane group's
  //    heads) for entry r of every tile; a reduce-scatter over the lane
  //    groups (two rounds of permlane swaps, no LDS) leaves lane l with the
  //    full sum of entry l of the 64, stored with one coalesced 256-byte
  //    write per query.
#pragma unroll
  for (int grp = 0; grp < kIters / 4; ++grp) {
    float p[QB][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int it = grp * 4 + j;
      const v4i kk = use[it] ? kv[it] : v4i{0, 0, 0, 0};
      const int sbu = use[it] ? sbv[it] : 127;
      const v8i Bm = {kk[0], kk[1], kk[2], kk[3], 0, 0, 0, 0};
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float sum = 0.f;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
          v4f acc = {0.f, 0.f, 0.f, 0.f};
          acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[qb][ht], Bm, acc, 0, 4, 0, sa[qb][ht], 0, sbu);
#pragma unroll
          for (int i = 0; i < 4; ++i) sum = fmaf(fmaxf(acc[i], 0.f), wv[qb][ht][i], sum);
        }
        p[qb][j] = sum;
      }
    }
    // lane l holds tile g = l/16; its entry slot is base + 64*grp + l
    const int slot = base + grp * 64 + lane;
    int e_l = 0;
    if (kCand) {
      const int t0 = ent[grp * 4], t1 = ent[grp * 4 + 1], t2 = ent[grp * 4 + 2], t3 = ent[grp * 4 + 3];
      e_l = g == 0 ? t0 : g == 1 ? t1 : g == 2 ? t2 : t3;
      // every lane group loaded every tile's candidates: lane (g, r) checks
      // its own tile g, slot r (a candidate outside [-1, visible), or a
      // neighbour pair that is not strictly ascending: skipped / as given)
      if (slot < C) {
        const int u0 = prv[grp * 4], u1 = prv[grp * 4 + 1], u2 = prv[grp * 4 + 2], u3 = prv[grp * 4 + 3];
        const int pe = g == 0 ? u0 : g == 1 ? u1 : g == 2 ? u2 : u3;
        uint32_t f = (e_l < -1 || e_l >= vis[0]) ? kFaultCand : 0u;
        if (e_l >= 0 && pe >= 0 && e_l <= pe) f |= kFaultCand;
        if (f) raise_fault(flags, f);
      }
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float res = reduce_scatter4(p[qb][0], p[qb][1], p[qb][2], p[qb][3]);
      const int q = q0 + qb;
      if (q >= Q) continue;
      float *dst = scores + ((int64_t)b * Q + q) * Ns;
      if (kCand) {
        if (!(e_l >= 0 && e_l < vis[0])) res = __uint_as_float(kNoScoreBits);
        if (slot < C) dst[slot] = res;
      } else if (slot < vis[qb] && slot != skip) {
        dst[slot] = res;
        if (use_hint) atomicAdd(&hint_lds[score_key(res) >> kHintShift], 1u);
      }
    }
  }
  if (use_hint) {
    __syncthreads();
    uint32_t *hg = hint + ((int64_t)b * Q + q0) * kHintBins;
    for (int i = threadIdx.x; i < kHintBins; i += kIdxThreads) {
      const uint32_t c = hint_lds[i];
      if (c) atomicAdd(hg + i, c);
    }
  }
}

// zero4 / n_zero4: a side job, 16-byte words of the next launch's workspace
// that must start at zero (the radix top-k's histograms), cleared by the
// whole grid before its own work, so that the next launch needs no
// clearing launch of its own.
template <int HT, int QB, bool kCand>
__global__ __launch_bounds__(kIdxThreads) void index_scores_kernel(
    const uint8_t *__restrict__ ikey, const uint8_t *__restrict__ iscale, const int32_t *__restrict__ n_entries,
    int N_cap, int d_idx, int m, const uint8_t *__restrict__ q_idx, const float *__restrict__ w_idx, int H_I,
    const int32_t *__restrict__ q_pos, int Q, const int32_t *__restrict__ cand, int C, float *__restrict__ scores,
    int Ns, uint32_t *flags, uint32_t *hint, uint4 *zero4, int64_t n_zero4) {
  if (zero4) {
    const int64_t wg = ((int64_t)blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
    const int64_t stride = (int64_t)gridDim.x * gridDim.y * gridDim.z * kIdxThreads;
    for (int64_t i = wg * kIdxThreads + threadIdx.x; i < n_zero4; i += stride) zero4[i] = uint4{0u, 0u, 0u, 0u};
  }
  index_body<HT, QB, kCand>(ikey, iscale, n_entries, N_cap, d_idx, m, q_idx, w_idx, H_I, q_pos, Q, cand, C, scores, Ns,
                            blockIdx.x, blockIdx.y, blockIdx.z, -1, flags, hint);
}

// ---------------------------------------------------------------------------
// Decode append fused with the indexer.  When every sequence appends one
// entry (one block of m <= 8 raw rows) and then scores it with one query,
// the first B workgroups of the launch pool and encode the new entry (the
// compressor's arithmetic, step for step: the same pooling order, MXFP4
// encoding and 8-slice projection sums as compress.hip, so the cache bytes
// are identical) and score it from the codes they just produced; the other
// workgroups run the indexer body on every other visible entry.  The new
// entry's score goes through the same scaled MFMA (its column of a 16-entry
// tile, the other columns zero), the same ReLU/weight FMA order and the
// same reduce-scatter as in the indexer body, so it is identical too.  The
// indexer workgroups may read the new entry's key while it is being
// written; its score slot is the one they do not store.
struct AppendArgs {
  const uint16_t *x;
  int64_t x_stride_b;
  const uint16_t *z;
  int64_t z_stride_b;
  const float *bias;
  const uint16_t *w_ik;
  int m;
  int entry;  // the appended entry (the same index in every sequence)
  uint8_t *nope;
  uint8_t *nscale;
  uint16_t *rope;
};

constexpr int kAppSlices = kIdxThreads / 32;     // projection slices
constexpr int kAppSlice = kD / kAppSlices;       // channels per slice
constexpr int kAppMaxM = 8;

template <int HT, bool kGateFull>
__device__ __forceinline__ void append_and_score(const AppendArgs &ap, uint8_t *__restrict__ ikey,
                                                 uint8_t *__restrict__ iscale, const int32_t *__restrict__ n_entries,
                                                 int N_cap, int d_idx, const uint8_t *__restrict__ q_idx,
                                                 const float *__restrict__ w_idx, int H_I,
                                                 const int32_t *__restrict__ q_pos, int Q, float *__restrict__ scores,
                                                 int Ns, int b, uint32_t *hint) {
  __shared__ __attribute__((aligned(16))) float cs[kD];
  __shared__ float kpart[kAppSlices][128];
  __shared__ float ks[128];
  __shared__ __attribute__((aligned(16))) uint8_t kc[64];
  __shared__ uint32_t ksc[4];
  __shared__ __attribute__((aligned(16))) uint8_t qs[HT * 16 * 128];
  __shared__ uint8_t qsc[HT * 16 * 4];  // E8M0 byte of each query block
  const int tid = threadIdx.x;
  const int m = ap.m;
  const int nkb = d_idx / 32;
  const int64_t row = (int64_t)b * N_cap + ap.entry;

  // queries for LDS staging first (as in the indexer body, one query)
  constexpr int kQBytes = HT * 16 * 128;
  constexpr int kQVec = (kQBytes / 16 + kIdxThreads - 1) / kIdxThreads;
  uint4 qv_stage[kQVec];
#pragma unroll
  for (int u = 0; u < kQVec; ++u) {
    const int i = tid + u * kIdxThreads;
    const int rem = (i % (kQBytes / 16)) * 16;
    const int h = rem / 128, c = rem % 128;
    const bool ok = i < kQBytes / 16 && h < H_I && c < d_idx;
    const int64_t off = ok ? ((int64_t)b * Q * H_I + h) * d_idx + c : 0;
    const uint4 v = *reinterpret_cast<const uint4 *>(q_idx + off);
    qv_stage[u] = ok ? v : uint4{0u, 0u, 0u, 0u};
  }

  // 1. pooling: thread t < 144 owns channels 4t..4t+3; the chunk holds
  //    exactly the m raw rows of the new entry (rows 0..m-1)
  const uint16_t *xb = ap.x + (int64_t)b * ap.x_stride_b;
  const uint16_t *zb = ap.z + (int64_t)b * ap.z_stride_b;
  if (tid < kD / 4) {
    const int c = tid * 4;
    const int64_t row0 = 0;
    float mx[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    float den[4] = {0.f, 0.f, 0.f, 0.f};
    float num[4] = {0.f, 0.f, 0.f, 0.f};
    uint2 gz[kAppMaxM], gx[kAppMaxM];
#pragma unroll
    for (int i = 0; i < kAppMaxM; ++i) {
      const int64_t rr = row0 + min(i, m - 1);
      gx[i] = *reinterpret_cast<const uint2 *>(xb + rr * kD + c);
      if (kGateFull) {
        gz[i] = *reinterpret_cast<const uint2 *>(zb + rr * kD + c);
      } else {
        const uint32_t h = zb[rr];
        gz[i] = uint2{h | (h << 16), h | (h << 16)};
      }
    }
    float a[kAppMaxM][4];
#pragma unroll
    for (int i = 0; i < kAppMaxM; ++i) {
      if (i < m) {
        const float bi = ap.bias[i];
        a[i][0] = bf16_to_f32(gz[i].x & 0xFFFFu) + bi;
        a[i][1] = bf16_to_f32(gz[i].x >> 16) + bi;
        a[i][2] = bf16_to_f32(gz[i].y & 0xFFFFu) + bi;
        a[i][3] = bf16_to_f32(gz[i].y >> 16) + bi;
#pragma unroll
        for (int u = 0; u < 4; ++u) mx[u] = fmaxf(mx[u], a[i][u]);
      }
    }
#pragma unroll
    for (int i = 0; i < kAppMaxM; ++i) {
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
#pragma unroll
    for (int u = 0; u < 4; ++u) cs[c + u] = num[u] / den[u];
  }
#pragma unroll
  for (int u = 0; u < kQVec; ++u) {
    const int i = tid + u * kIdxThreads;
    const int sc = e4m3_rescale_piece(qv_stage[u]);  // as in the indexer body
    if (i < kQBytes / 16) {
      *reinterpret_cast<uint4 *>(qs + i * 16) = qv_stage[u];
      if (!(i & 1)) qsc[i >> 1] = (uint8_t)sc;
    }
  }
  // the projection's first batch of W_IK loads goes out now and stays in
  // flight across the LDS-only barrier and the main entry's encoding
  const int nq = d_idx / 4;
  const int part = tid / nq, pq = tid % nq;
  const bool projects = part < kAppSlices;
  const uint2 *wp = reinterpret_cast<const uint2 *>(ap.w_ik + (int64_t)((projects ? part : 0) * kAppSlice) * d_idx +
                                                    4 * pq);
  constexpr int kBatch = kAppSlice / 2;
  uint2 wv0[kBatch];
#pragma unroll
  for (int j = 0; j < kBatch; ++j) wv0[j] = wp[(int64_t)j * nq];
  lds_barrier();

  // 2. MXFP4 main entry and bf16 rope channels
  {
    uint32_t sb;
    const uint32_t byte = encode_pair(cs[2 * tid], cs[2 * tid + 1], sb);
    ap.nope[row * kNopeBytes + tid] = (uint8_t)byte;
    if ((tid & 15) == 0) ap.nscale[row * kNopeScales + (tid >> 4)] = (uint8_t)sb;
  }
  if (tid < kDRope) ap.rope[row * kDRope + tid] = (uint16_t)f32_to_bf16(cs[kDNope + tid]);

  // 3. indexer key: thread (slice p, output quad q) accumulates channels
  //    [72p, 72p+72) of outputs 4q..4q+3 in channel order (one 8-byte W_IK
  //    load per channel serves the four), in batches of loads issued
  //    together; the slices are added in order
  {
    const int q = pq;
    if (projects) {
      const float4 *cp = reinterpret_cast<const float4 *>(&cs[part * kAppSlice]);
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int h = 0; h < kAppSlice / kBatch; ++h) {
        uint2 wv[kBatch];
        if (h == 0) {
#pragma unroll
          for (int j = 0; j < kBatch; ++j) wv[j] = wv0[j];
        } else {
#pragma unroll
          for (int j = 0; j < kBatch; ++j) wv[j] = wp[(int64_t)(h * kBatch + j) * nq];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u4 = 0; u4 < kBatch / 4; ++u4) {
          const float4 c4 = cp[h * (kBatch / 4) + u4];
          const float cc[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint2 w2 = wv[4 * u4 + j];
            acc[0] = fmaf(cc[j], bf16_to_f32(w2.x & 0xFFFFu), acc[0]);
            acc[1] = fmaf(cc[j], bf16_to_f32(w2.x >> 16), acc[1]);
            acc[2] = fmaf(cc[j], bf16_to_f32(w2.y & 0xFFFFu), acc[2]);
            acc[3] = fmaf(cc[j], bf16_to_f32(w2.y >> 16), acc[3]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) kpart[part][4 * q + j] = acc[j];
    }
  }
  __syncthreads();
  if (tid < d_idx) {
    float s = 0.f;
#pragma unroll
    for (int pp = 0; pp < kAppSlices; ++pp) s += kpart[pp][tid];
    ks[tid] = s;
  }
  __syncthreads();
  if (tid < 64) {
    // 16 lanes per key block (a DPP row), two channels each; rows past the
    // key's blocks encode a copy of block 0 and store nothing
    const int kb = tid >> 4, t = tid & 15;
    const int kbc = kb < nkb ? kb : 0;
    uint32_t sb;
    const uint32_t byte = encode_pair(ks[kbc * 32 + 2 * t], ks[kbc * 32 + 2 * t + 1], sb);
    if (kb < nkb) {
      ikey[row * (d_idx / 2) + kb * 16 + t] = (uint8_t)byte;
      kc[kb * 16 + t] = (uint8_t)byte;
      if (t == 0) {
        iscale[row * nkb + kb] = (uint8_t)sb;
        ksc[kb] = sb;
      }
    }
  }
  __syncthreads();

  // 4. the new entry's score (one wave; one query)
  if (tid >= 64) return;
  const int lane = tid, g = lane >> 4, r = lane & 15;
  float wv[HT][4];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = ht * 16 + g * 4 + i;
      wv[ht][i] = hh < H_I ? w_idx[(int64_t)b * Q * H_I + hh] : 0.f;
    }
  const int r_new = ap.entry & 15, t_new = (ap.entry & 63) >> 4;
  const bool mine = r == r_new && g < nkb;
  const v4i kk = mine ? *reinterpret_cast<const v4i *>(&kc[g * 16]) : v4i{0, 0, 0, 0};
  const int sbu = mine ? (int)ksc[g] : 127;
  const v8i Bm = {kk[0], kk[1], kk[2], kk[3], 0, 0, 0, 0};
  float sum = 0.f;
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const uint8_t *qr = qs + (ht * 16 + r) * 128;
    const v4i lo = *reinterpret_cast<const v4i *>(qr + 16 * g);
    const v4i hi = *reinterpret_cast<const v4i *>(qr + 64 + 16 * g);
    const v8i A = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    const int sa = qsc[(ht * 16 + r) * 4 + g];
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, Bm, acc, 0, 4, 0, sa, 0, sbu);
#pragma unroll
    for (int i = 0; i < 4; ++i) sum = fmaf(fmaxf(acc[i], 0.f), wv[ht][i], sum);
  }
  const float res = reduce_scatter4(t_new == 0 ? sum : 0.f, t_new == 1 ? sum : 0.f, t_new == 2 ? sum : 0.f,
                                    t_new == 3 ? sum : 0.f);
  const int nE = min(n_entries[b], N_cap);
  const int vis = max(0, min(nE, (q_pos[(int64_t)b * Q] + 1) / m));
  if (lane == 16 * t_new + r_new && ap.entry < vis) {
    scores[(int64_t)b * Q * Ns + ap.entry] = res;
    if (hint) atomicAdd(hint + (int64_t)b * Q * kHintBins + (score_key(res) >> kHintShift), 1u);
  }
}

// Grid: B append workgroups first, then B x tiles indexer workgroups.  The
// append workgroups' dependent chain (rows, pooling, two batches of W_IK
// loads, encoding, the entry's score) ends the launch when it is slower than
// the key stream; the register bound keeps room for a whole 36-load batch
// at the indexer's own occupancy (5 waves per SIMD with 32 heads, 4 with 64).
template <int HT, bool kGateFull>
__global__ __launch_bounds__(kIdxThreads, HT >= 4 ? 4 : 5) void append_index_kernel(
    AppendArgs ap, uint8_t *__restrict__ ikey, uint8_t *__restrict__ iscale, const int32_t *__restrict__ n_entries,
    int N_cap, int d_idx, const uint8_t *__restrict__ q_idx, const float *__restrict__ w_idx, int H_I,
    const int32_t *__restrict__ q_pos, int Q, float *__restrict__ scores, int B, int tiles, uint32_t *flags,
    uint32_t *hint) {
  const int w = blockIdx.x;
  if (w < B) {
    append_and_score<HT, kGateFull>(ap, ikey, iscale, n_entries, N_cap, d_idx, q_idx, w_idx, H_I, q_pos, Q, scores,
                                    N_cap, w, hint);
    return;
  }
  const int t = w - B;
  index_body<HT, 1, false>(ikey, iscale, n_entries, N_cap, d_idx, ap.m, q_idx, w_idx, H_I, q_pos, Q, nullptr, 0,
                           scores, N_cap, t % tiles, 0, t / tiles, ap.entry, flags, hint);
}

template <int HT>
static void launch_append(const AppendArgs &ap, bool gate_full, const CacheView &c, const uint8_t *q_idx,
                          const float *w_idx, int H_I, const int32_t *q_pos, float *scores, hipStream_t stream,
                          uint32_t *hint) {
  const int tiles = (c.N_cap + kIdxWGEntries - 1) / kIdxWGEntries;
  const unsigned grid = (unsigned)(c.B + c.B * tiles);
  if (gate_full)
    append_index_kernel<HT, true><<<grid, kIdxThreads, 0, stream>>>(ap, c.ikey, c.iscale, c.n_entries, c.N_cap,
                                                                    c.d_idx, q_idx, w_idx, H_I, q_pos, 1, scores,
                                                                    c.B, tiles, c.flags, hint);
  else
    append_index_kernel<HT, false><<<grid, kIdxThreads, 0, stream>>>(ap, c.ikey, c.iscale, c.n_entries, c.N_cap,
                                                                     c.d_idx, q_idx, w_idx, H_I, q_pos, 1, scores,
                                                                     c.B, tiles, c.flags, hint);
}

bool append_index_fusable(int m, int64_t T, int Q, int G, const uint16_t *w_ik, int B) {
  return w_ik && (reinterpret_cast<uintptr_t>(w_ik) & 7) == 0 && m <= kAppMaxM && T == m && Q == 1 &&
         (G == kD || G == 1) && B > 0;
}

hipError_t launch_append_index(const uint16_t *x, int64_t x_stride_b, const uint16_t *z, int64_t z_stride_b, int G,
                               const float *bias, const uint16_t *w_ik, int64_t entry, const CacheView &c,
                               const uint8_t *q_idx, const float *w_idx, int H_I, const int32_t *q_pos,
                               float *scores, hipStream_t stream, uint32_t *hint) {
  AppendArgs ap{x, x_stride_b, z, z_stride_b, bias, w_ik, c.m, (int)entry, c.nope, c.nscale, c.rope};
  const bool full = G == kD;
  if (H_I <= 16)
    launch_append<1>(ap, full, c, q_idx, w_idx, H_I, q_pos, scores, stream, hint);
  else if (H_I <= 32)
    launch_append<2>(ap, full, c, q_idx, w_idx, H_I, q_pos, scores, stream, hint);
  else
    launch_append<4>(ap, full, c, q_idx, w_idx, H_I, q_pos, scores, stream, hint);
  return hipGetLastError();
}

template <int HT, int QB, bool kCand>
static void launch_idx(dim3 grid, hipStream_t stream, const CacheView &c, const uint8_t *q_idx, const float *w_idx,
                       int H_I, const int32_t *q_pos, int Q, const int32_t *cand, int C, float *scores, int Ns,
                       uint32_t *hint = nullptr, void *zero = nullptr, size_t zero_bytes = 0) {
  index_scores_kernel<HT, QB, kCand><<<grid, kIdxThreads, 0, stream>>>(
      c.ikey, c.iscale, c.n_entries, c.N_cap, c.d_idx, c.m, q_idx, w_idx, H_I, q_pos, Q, cand, C, scores, Ns, c.flags,
      hint, reinterpret_cast<uint4 *>(zero), (int64_t)(zero_bytes / 16));
}

// ---------------------------------------------------------------------------
// Prefill (many queries, full scan): a GEMM-shaped pass.  Each wave keeps the
// MFMA fragments of its QW queries (A operands) and head weights in registers
// for the whole launch and walks one chunk of kPfChunk entries in 64-entry
// groups; nothing goes through LDS.  Key tiles come in through range-checked
// buffer loads (reads past the cache row return zero), one group ahead.
// Per 16-entry tile and query, ReLU + head weights give each lane a partial
// head sum for one entry; the four tiles of a group are then summed across
// the four lane groups with two rounds of permlane swaps (a reduce-scatter:
// lane l ends with entry 16*(l/16) + l%16 = l of the group), so that each
// query's 64 scores leave in one coalesced 256-byte store.  Causal prefill:
// a wave stops at the last entry any of its queries can see, and chunks past
// it exit at once.
// max(x, 0) as one integer max on the bit pattern (negative floats, -0
// included, are negative integers): a float max would first quiet its
// operand, one more instruction per score term.
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

constexpr int kPfWaves = 4;
constexpr int kPfChunk = 1024;
constexpr int kPfMinQ = 64;  // from this many queries per launch on

// HT: head tiles of 16; DI: d_idx (64 or 128), fixed at compile time so that
// key addresses are a per-lane constant plus a uniform group offset plus an
// immediate per tile (no per-load address arithmetic).
template <int HT, int DI>
__global__ __launch_bounds__(kPfWaves * 64) void index_prefill_kernel(
    const uint8_t *__restrict__ ikey, const uint8_t *__restrict__ iscale, const int32_t *__restrict__ n_entries,
    int N_cap, int m, const uint8_t *__restrict__ q_idx, const float *__restrict__ w_idx, int H_I,
    const int32_t *__restrict__ q_pos, int Q, float *__restrict__ scores, int n_qblk, int n_chunk,
    uint32_t *flags) {
  constexpr int QW = 8 / HT;  // queries per wave
  constexpr int d_idx = DI;
  // Workgroup i runs on XCD i % 8: the chunks of one query block follow each
  // other on one XCD, whose L2 then serves that block's queries to all of them.
  const int L = blockIdx.x;
  const int sidx = L >> 3;
  const int c = sidx % n_chunk;
  const int qblk = (sidx / n_chunk) * 8 + (L & 7);
  if (qblk >= n_qblk) return;
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, r = lane & 15;
  const int q0 = (qblk * kPfWaves + wave) * QW;
  if (q0 >= Q) return;
  constexpr int kb = d_idx / 32;

  // Loads below are unconditional, from clamped addresses, and masked with
  // bit operations: a load under a condition (even a uniform one) is moved
  // into a branch that waits for it before the next load is issued.
  const int nE_raw = n_entries[b];
  const int nE = min(nE_raw, N_cap);
  if (L == 0 && threadIdx.x == 0 && (nE_raw < 0 || nE_raw > N_cap)) raise_fault(flags, kFaultEntries);
  int pos[QW];
#pragma unroll
  for (int qw = 0; qw < QW; ++qw) pos[qw] = q_pos[(int64_t)b * Q + min(q0 + qw, Q - 1)];
  int vis[QW];
  int vmax = 0;
#pragma unroll
  for (int qw = 0; qw < QW; ++qw) {
    vis[qw] = max(0, min(nE, (pos[qw] + 1) / m)) & -(int)(q0 + qw < Q);
    vmax = max(vmax, vis[qw]);
  }
  const int e_begin = c * kPfChunk;
  const int e_end = min(e_begin + kPfChunk, vmax);
  if (e_begin >= e_end) return;

  // Key tiles: lane (r, g) reads entry e+r's channel block g (16 bytes) and
  // its scale byte.  Blocks past d_idx (d_idx = 64) read block 0 and meet
  // zero query channels; their scale is forced to 1.
  constexpr int rowb = d_idx / 2;
  const int gg = g < kb ? g : 0;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(ikey + (int64_t)b * N_cap * rowb), 0, N_cap * rowb, 0x00020000);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(iscale + (int64_t)b * N_cap * kb), 0, N_cap * kb, 0x00020000);
  // per-lane part of the key / scale offsets; the group part is uniform
  // (scalar offset), the tile part an immediate
  const int kvo = r * rowb + gg * 16, svo = r * kb + gg;
  v4i kv[4];
  int sb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    kv[j] = __builtin_amdgcn_raw_buffer_load_b128(krs, kvo + 16 * j * rowb, e_begin * rowb, 0);
    sb[j] = __builtin_amdgcn_raw_buffer_load_b8(srs, svo + 16 * j * kb, e_begin * kb, 0);
  }

  // Query fragments (E4M3 layout: lane group g holds channels 16g..+15 and
  // 64+16g..+15 of head row r) and head weights (lane l: heads 4(l/16)..+3
  // of each 16-head tile).  Head rows past H_I and channels past d_idx are
  // zeroed in A, which zeroes their scores whatever weight they meet; rows
  // of queries past Q are never stored.
  v8i A[QW][HT];
  int sa[QW][HT];  // the scale of block g of head row r
  float w[QW][HT][4];
#pragma unroll
  for (int qw = 0; qw < QW; ++qw) {
    const int64_t qrow = ((int64_t)b * Q + min(q0 + qw, Q - 1)) * H_I;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const int h = ht * 16 + r;
      const uint8_t *qr = q_idx + (qrow + (h < H_I ? h : 0)) * d_idx;
      const v4i lo = *reinterpret_cast<const v4i *>(qr + 16 * g);
      const v4i hi = *reinterpret_cast<const v4i *>(qr + (d_idx > 64 ? 64 : 0) + 16 * g);
      const int ml = -(int)(h < H_I);
      const int mh = ml & -(int)(d_idx > 64);
      A[qw][ht] = v8i{lo[0] & ml, lo[1] & ml, lo[2] & ml, lo[3] & ml, hi[0] & mh, hi[1] & mh, hi[2] & mh, hi[3] & mh};
      sa[qw][ht] = e4m3_rescale_fragment(A[qw][ht], g, r);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hh = ht * 16 + g * 4 + i;
        w[qw][ht][i] = w_idx[qrow + (hh < H_I ? hh : 0)];
      }
    }
  }

  // Score rows: buffer stores through a range of vis[qw] floats, so that
  // the entries a query cannot see are left untouched without a branch.
  __amdgpu_buffer_rsrc_t ors[QW];
#pragma unroll
  for (int qw = 0; qw < QW; ++qw)
    ors[qw] = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(scores + ((int64_t)b * Q + min(q0 + qw, Q - 1)) * N_cap), 0, vis[qw] * 4, 0x00020000);

  for (int e64 = e_begin; e64 < e_end; e64 += 64) {
    float p[QW][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int sbu = g < kb ? sb[j] : 127;
      const v8i Bm = {kv[j][0], kv[j][1], kv[j][2], kv[j][3], 0, 0, 0, 0};
      // query by query: the MFMAs of query qw+1 run while the vector unit
      // folds the heads of query qw
      v4f acc[2][HT];
#pragma unroll
      for (int qw = 0; qw <= QW; ++qw) {
        if (qw < QW) {
#pragma unroll
          for (int ht = 0; ht < HT; ++ht)
            acc[qw & 1][ht] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                A[qw][ht], Bm, v4f{0.f, 0.f, 0.f, 0.f}, 0, 4, 0, sa[qw][ht], 0, sbu);
        }
        if (qw > 0) {
          float s = 0.f;
#pragma unroll
          for (int ht = 0; ht < HT; ++ht)
#pragma unroll
            for (int i = 0; i < 4; ++i) s = fmaf(relu_bits(acc[(qw - 1) & 1][ht][i]), w[qw - 1][ht][i], s);
          p[qw - 1][j] = s;
        }
      }
      // refill this slot with the same tile of the next group
      kv[j] = __builtin_amdgcn_raw_buffer_load_b128(krs, kvo + 16 * j * rowb, (e64 + 64) * rowb, 0);
      sb[j] = __builtin_amdgcn_raw_buffer_load_b8(srs, svo + 16 * j * kb, (e64 + 64) * kb, 0);
    }
    // Reduce-scatter over the lane groups: after the 32-lane swaps the low
    // half holds tiles 0/1 and the high half tiles 2/3 (sums over lane groups
    // g and g^2); after the 16-lane swap, row g holds tile g (all four groups).
#pragma unroll
    for (int qw = 0; qw < QW; ++qw) {
      const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[qw][0]), __float_as_uint(p[qw][2]), false,
                                                      false);
      const auto y = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[qw][1]), __float_as_uint(p[qw][3]), false,
                                                      false);
      const float k0 = __uint_as_float(x[0]) + __uint_as_float(x[1]);
      const float k1 = __uint_as_float(y[0]) + __uint_as_float(y[1]);
      const auto z = __builtin_amdgcn_permlane16_swap(__float_as_uint(k0), __float_as_uint(k1), false, false);
      const float res = __uint_as_float(z[0]) + __uint_as_float(z[1]);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(res), ors[qw], lane * 4, e64 * 4, 0);
    }
  }
}

template <int HT>
static void launch_prefill(const CacheView &c, const uint8_t *q_idx, const float *w_idx, int H_I,
                           const int32_t *q_pos, int Q, float *scores, hipStream_t stream) {
  constexpr int QW = 8 / HT;
  const int n_qblk = (Q + kPfWaves * QW - 1) / (kPfWaves * QW);
  const int n_chunk = (c.N_cap + kPfChunk - 1) / kPfChunk;
  dim3 grid(((n_qblk + 7) / 8) * 8 * n_chunk, c.B);
  if (c.d_idx == 128)
    index_prefill_kernel<HT, 128><<<grid, kPfWaves * 64, 0, stream>>>(
        c.ikey, c.iscale, c.n_entries, c.N_cap, c.m, q_idx, w_idx, H_I, q_pos, Q, scores, n_qblk, n_chunk, c.flags);
  else
    index_prefill_kernel<HT, 64><<<grid, kPfWaves * 64, 0, stream>>>(
        c.ikey, c.iscale, c.n_entries, c.N_cap, c.m, q_idx, w_idx, H_I, q_pos, Q, scores, n_qblk, n_chunk, c.flags);
}

// The launch shapes that can clear words for the next launch (one-query
// full scans; see index_scores_kernel).
bool index_can_zero(int Q, bool cand) { return !cand && Q > 0 && Q < 4; }

template <int HT>
static void dispatch_idx(const CacheView &c, const uint8_t *q_idx, const float *w_idx, int H_I, const int32_t *q_pos,
                         int Q, const int32_t *cand, int C, float *scores, hipStream_t stream, uint32_t *hint,
                         void *zero, size_t zero_bytes) {
  if (cand) {
    const int Ns = C;
    dim3 grid((C + kIdxWGEntries - 1) / kIdxWGEntries, Q, c.B);
    launch_idx<HT, 1, true>(grid, stream, c, q_idx, w_idx, H_I, q_pos, Q, cand, C, scores, Ns);
  } else if (Q >= kPfMinQ) {
    launch_prefill<HT>(c, q_idx, w_idx, H_I, q_pos, Q, scores, stream);
  } else if (Q >= 4) {
    dim3 grid((c.N_cap + kIdxWGEntries - 1) / kIdxWGEntries, (Q + 3) / 4, c.B);
    launch_idx<HT, 4, false>(grid, stream, c, q_idx, w_idx, H_I, q_pos, Q, nullptr, 0, scores, c.N_cap);
  } else {
    dim3 grid((c.N_cap + kIdxWGEntries - 1) / kIdxWGEntries, Q, c.B);
    launch_idx<HT, 1, false>(grid, stream, c, q_idx, w_idx, H_I, q_pos, Q, nullptr, 0, scores, c.N_cap, hint, zero,
                             zero_bytes);
  }
}

hipError_t launch_index_scores(const CacheView &c, const uint8_t *q_idx, const float *w_idx, int H_I,
                               const int32_t *q_pos, int Q, const int32_t *cand, int C, float *scores,
                               hipStream_t stream, uint32_t *hint, void *zero, size_t zero_bytes) {
  if (zero && (!index_can_zero(Q, cand != nullptr) || (zero_bytes & 15) != 0 ||
               (reinterpret_cast<uintptr_t>(zero) & 15) != 0))
    return hipErrorInvalidValue;
  if (H_I <= 16)
    dispatch_idx<1>(c, q_idx, w_idx, H_I, q_pos, Q, cand, C, scores, stream, hint, zero, zero_bytes);
  else if (H_I <= 32)
    dispatch_idx<2>(c, q_idx, w_idx, H_I, q_pos, Q, cand, C, scores, stream, hint, zero, zero_bytes);
  else
    dispatch_idx<4>(c, q_idx, w_idx, H_I, q_pos, Q, cand, C, scores, stream, hint, zero, zero_bytes);
  return hipGetLastError();
}

}  // namespace csa
