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
constexpr int kIdxWaveEntries = 128; // entries per wave per workgroup (groups of 64)
constexpr int kIdxWGEntries = kIdxThreads / 64 * kIdxWaveEntries;

// HT: head tiles of 16 (H_I <= 16 * HT).  QB: queries per wave.
template <int HT, int QB, bool kCand>
__global__ __launch_bounds__(kIdxThreads) void index_scores_kernel(
    const uint8_t *__restrict__ ikey, const uint8_t *__restrict__ iscale, const int32_t *__restrict__ n_entries,
    int N_cap, int d_idx, int m, const uint8_t *__restrict__ q_idx, const float *__restrict__ w_idx, int H_I,
    const int32_t *__restrict__ q_pos, int Q, const int32_t *__restrict__ cand, int C, float *__restrict__ scores,
    int Ns) {
  // Indexer queries of this workgroup (QB queries x 16*HT heads x d_idx bytes),
  // staged once so that the waves read their MFMA fragments from LDS.
  __shared__ __attribute__((aligned(16))) uint8_t qs[QB * HT * 16 * 128];
  const int b = blockIdx.z;
  const int q0 = blockIdx.y * QB;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;   // 32-channel block (K group)
  const int r = lane & 15;   // entry within the tile / head row within the head tile
  const int kb = d_idx / 32; // key blocks per entry (2 or 4)
  const int base = blockIdx.x * kIdxWGEntries + wave * kIdxWaveEntries;
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
    if ((int)blockIdx.x * kIdxWGEntries >= vmax) return;
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
  bool use[kIters];
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const int slot = base + it * 16 + r;
    int e = slot;
    if (kCand) e = cand[((int64_t)b * Q + q0) * C + min(slot, C - 1)];
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

  // 3. Queries into LDS (zero rows beyond H_I and beyond Q).
#pragma unroll
  for (int u = 0; u < kQVec; ++u) {
    const int i = threadIdx.x + u * kIdxThreads;
    if (i < QB * kQBytes / 16) {
      const int qb = i / (kQBytes / 16), rem = (i % (kQBytes / 16)) * 16;
      *reinterpret_cast<uint4 *>(qs + qb * kQBytes + rem) = qv_stage[u];
    }
  }
  // LDS-only barrier: the key loads stay in flight, each MFMA below waits
  // only for its own tile.
  lds_barrier();
  // E4M3 operand layout of the instruction: bytes 0..15 of lane group g hold
  // channels 16g..16g+15, bytes 16..31 hold channels 64+16g..+15.
  v8i A[QB][HT];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const uint8_t *qr = qs + qb * (HT * 16 * 128) + (ht * 16 + r) * 128;
      const v4i lo = *reinterpret_cast<const v4i *>(qr + 16 * g);
      const v4i hi = *reinterpret_cast<const v4i *>(qr + 64 + 16 * g);
      A[qb][ht] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }

  // 4. Visibility of this workgroup's queries (uniform loads).
  const int nE = min(n_entries[b], N_cap);
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
          acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[qb][ht], Bm, acc, 0, 4, 0, 127, 0, sbu);
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
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[qb][0]), __float_as_uint(p[qb][2]), false,
                                                      false);
      const auto y = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[qb][1]), __float_as_uint(p[qb][3]), false,
                                                      false);
      const float k0 = __uint_as_float(x[0]) + __uint_as_float(x[1]);
      const float k1 = __uint_as_float(y[0]) + __uint_as_float(y[1]);
      const auto z = __builtin_amdgcn_permlane16_swap(__float_as_uint(k0), __float_as_uint(k1), false, false);
      float res = __uint_as_float(z[0]) + __uint_as_float(z[1]);
      const int q = q0 + qb;
      if (q >= Q) continue;
      float *dst = scores + ((int64_t)b * Q + q) * Ns;
      if (kCand) {
        if (!(e_l >= 0 && e_l < vis[0])) res = __uint_as_float(kNoScoreBits);
        if (slot < C) dst[slot] = res;
      } else if (slot < vis[qb]) {
        dst[slot] = res;
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
    const int32_t *__restrict__ q_pos, int Q, float *__restrict__ scores, int n_qblk, int n_chunk) {
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
  const int nE = min(n_entries[b], N_cap);
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
                A[qw][ht], Bm, v4f{0.f, 0.f, 0.f, 0.f}, 0, 4, 0, 127, 0, sbu);
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
        c.ikey, c.iscale, c.n_entries, c.N_cap, c.m, q_idx, w_idx, H_I, q_pos, Q, scores, n_qblk, n_chunk);
  else
    index_prefill_kernel<HT, 64><<<grid, kPfWaves * 64, 0, stream>>>(
        c.ikey, c.iscale, c.n_entries, c.N_cap, c.m, q_idx, w_idx, H_I, q_pos, Q, scores, n_qblk, n_chunk);
}

template <int HT>
static void dispatch_idx(const CacheView &c, const uint8_t *q_idx, const float *w_idx, int H_I, const int32_t *q_pos,
                         int Q, const int32_t *cand, int C, float *scores, hipStream_t stream) {
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
