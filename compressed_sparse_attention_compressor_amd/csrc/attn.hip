// Attention over compressed entries plus the sliding window.
//
// [V4] "ハイブリッド注意：CSAとHCA": Fig. 3 (CSA: the query attends to its
// selected compressed blocks, and a sliding-window branch covers the
// recent raw tokens) and Fig. 4 (HCA: every compressed block, the same
// window).  One softmax runs over the union of the two key sets; the key
// and the value are the same decoded 576-channel row.
//
// Work split: one workgroup per (query, key-range split), a pair of waves
// per 16 query heads (heads are the MFMA M dimension, so a key is decoded
// once per workgroup and shared by every head); each wave of a pair owns
// half of the 576 output channels.  The logits either come from both waves
// computing the full Q K^T (kDupQK: no exchange, twice the products) or
// from each wave's half of the channels, the halves swapped through LDS.
// A query's key slots are its selected
// entries (padded to a multiple of the chunk size) followed by its window
// rows, so every chunk of 32 slots holds one kind of row and is fetched
// with the loads of that kind only.  Per chunk:
//   1. the workgroup decodes the 32 rows into a key-major bf16 LDS tile
//      (E2M1 x E8M0 -> bf16 is exact; gfx950's v_cvt_scalef32_pk_bf16_fp4
//      converts two codes per instruction); the raw bytes of the next chunk
//      are fetched into registers while the current one is computed (the
//      tile and the slot lists are multi-buffered, one barrier per chunk);
//   2. S = Q K^T on v_mfma_f32_16x16x32_bf16 (lane: key l%16, heads
//      4(l/16)..+3), online softmax in the log2 domain with DPP row
//      reductions (both waves of a pair hold bit-identical logits);
//   3. P goes through a small per-wave LDS tile to become the A operand of
//      O += P V; the V operand (keys along K) is read transposed from the
//      same key-major tile with ds_read_b64_tr_b16, so no second copy of
//      the keys is written.  With fp32 outputs P is split into two bf16
//      parts (hi + lo) so that the probabilities keep ~16 bits.
// Splits write unnormalised (O, max, sum) partials that a merge kernel
// combines; a single split writes the normalised output directly.
#include <type_traits>

#include "csa_device.hpp"
#include "csa_internal.hpp"

namespace csa {

constexpr int kKC = 32;           // key slots per chunk
// Key-major LDS row (bf16 elements).  Padding of 16 elements: with a
// 1184-byte row the Q K^T operand reads (16 rows x 16 bytes per lane group)
// run conflict-free, measured 4 LDS cycles per instruction against 8 with
// 8 elements of padding.
constexpr int kKRow = kD + 16;
constexpr int kPRow = kKC + 8;
constexpr int kHalfD = kD / 2;    // output channels per wave of a pair
constexpr int kHalfNT = kHalfD / 16;  // 18 channel tiles of 16 (P V)
constexpr int kKSteps = kD / 32;  // 18 channel steps of 32 (Q K^T)
constexpr int kFp4Tasks = kKC * (kDNope / 32);  // one MXFP4 block (16 code bytes + scale) each
constexpr int kRopeTasks = kKC * (kDRope / 8);  // 8 bf16 channels each
constexpr int kRowPieces = kD / 8;              // 16-byte pieces of a bf16 window row
constexpr int kWinTasks = kKC * kRowPieces;

struct AttnArgs {
  const uint8_t *nope;
  const uint8_t *nscale;
  const uint16_t *rope;
  const int32_t *n_entries;
  int N_cap, m;
  const uint16_t *q;
  int H;
  const int32_t *q_pos;
  int Q;
  const int32_t *idx;
  int k;
  const uint16_t *swa;
  const uint8_t *swa_codes;    // FP8 window rows (with kW8): MXFP8 codes [B][S][512],
  const uint8_t *swa_scales;   // their E8M0 scales [B][S][16],
  const uint16_t *swa_rope;    // and the bf16 positional channels [B][S][64]
  const int32_t *swa_pos0;
  int S, n_win;
  float scale_log2;
  void *out;
  float *lse;
  int out_bf16;
  float *ws_o;
  float *ws_ml;
  int nsplit, per_split;
};

// Per-thread share of one chunk's raw bytes for NT threads.
template <int NT>
struct ChunkShare {
  static constexpr int kFp4 = kFp4Tasks / NT > 0 ? kFp4Tasks / NT : 1;
  static constexpr int kRope = (kRopeTasks + NT - 1) / NT;
  static constexpr int kEnt = kFp4 + kRope;
  static constexpr int kWin = (kWinTasks + NT - 1) / NT;
  // FP8 window rows: 32-byte MXFP8 blocks (two pieces) plus rope pieces
  static constexpr int kW8 = 2 * kFp4 + kRope;
  // hold a whole chunk in registers (and fetch it ahead) when it is small
  static constexpr bool kAhead = kEnt <= 9 && kWin <= 9 && kW8 <= 9;
  static constexpr int kWinBatch = kAhead ? kWin : 9;
  static constexpr int kRaw0 = kEnt > kWinBatch ? kEnt : kWinBatch;
  static constexpr int kRaw = kRaw0 > kW8 ? kRaw0 : kW8;
};

template <int NT>
struct RawChunk {
  uint4 v[ChunkShare<NT>::kRaw];
  uint32_t s[ChunkShare<NT>::kFp4];
};

// Loads of an entry chunk: MXFP4 blocks and rope pieces.  Slots without an
// entry read row 0 (a valid address) and are zeroed when stored.
template <int NT>
__device__ __forceinline__ void load_entries(const AttnArgs &a, int b, const int *src, RawChunk<NT> &r) {
  using CS = ChunkShare<NT>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < CS::kFp4; ++u) {
    // clamped: with more threads than MXFP4 blocks in a chunk (1,024) the
    // surplus threads repeat the last block and store nothing
    const int t = min(tid + u * NT, kFp4Tasks - 1);
    const int key = t >> 4, blk = t & 15;
    const int64_t row = (int64_t)b * a.N_cap + min(max(src[key], 0), a.N_cap - 1);
    r.v[u] = *reinterpret_cast<const uint4 *>(a.nope + row * kNopeBytes + blk * 16);
    r.s[u] = a.nscale[row * kNopeScales + blk];
  }
#pragma unroll
  for (int u = 0; u < CS::kRope; ++u) {
    const int t = min(tid + u * NT, kRopeTasks - 1);
    const int key = t >> 3, part = t & 7;
    const int64_t row = (int64_t)b * a.N_cap + min(max(src[key], 0), a.N_cap - 1);
    r.v[CS::kFp4 + u] = *reinterpret_cast<const uint4 *>(a.rope + row * kDRope + part * 8);
  }
}

template <int NT>
__device__ __forceinline__ void store_entries(uint16_t *K, const int *src, const RawChunk<NT> &r) {
  using CS = ChunkShare<NT>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < CS::kFp4; ++u) {
    const int t = tid + u * NT;
    if (t >= kFp4Tasks) break;
    const int key = t >> 4, blk = t & 15;
    uint4 *dst = reinterpret_cast<uint4 *>(K + key * kKRow + blk * 32);
    if (src[key] >= 0) {
      // E2M1 x 2^(s-127) -> bf16 is exact (hardware conversion, two codes per byte)
      const float sc = e8m0_to_f32(r.s[u]);
      const uint4 c = r.v[u];
#define CSA_CVT(w, sel) __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, sel))
#define CSA_CVT4(w) uint4 { CSA_CVT(w, 0), CSA_CVT(w, 1), CSA_CVT(w, 2), CSA_CVT(w, 3) }
      // the four 16-byte quarters of the block are stored in a lane-dependent
      // order, (i + blk + blk / 4) mod 4: lanes of one key row would otherwise
      // hit the same banks (measured 8 LDS cycles per store against 32)
      const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int qi = (i + blk + (blk >> 2)) & 3;
        // the source word by value selects (no selection between array lvalues)
        const uint32_t w = qi == 0 ? cw[0] : (qi == 1 ? cw[1] : (qi == 2 ? cw[2] : cw[3]));
        dst[qi] = CSA_CVT4(w);
      }
#undef CSA_CVT4
#undef CSA_CVT
    } else {
      const uint4 z = {0u, 0u, 0u, 0u};
      dst[0] = z;
      dst[1] = z;
      dst[2] = z;
      dst[3] = z;
    }
  }
#pragma unroll
  for (int u = 0; u < CS::kRope; ++u) {
    const int t = tid + u * NT;
    if (t < kRopeTasks) {
      const int key = t >> 3, part = t & 7;
      uint4 v = r.v[CS::kFp4 + u];  // a value copy: a conditional between lvalues would pin r to memory
      if (src[key] < 0) v = uint4{0u, 0u, 0u, 0u};
      *reinterpret_cast<uint4 *>(K + key * kKRow + kDNope + part * 8) = v;
    }
  }
}

// FP8 window rows: per row 16 MXFP8 blocks (32 code bytes + one E8M0
// scale) and 8 rope pieces, laid out as the MXFP4 tasks of an entry chunk.
template <int NT>
__device__ __forceinline__ void load_win8(const AttnArgs &a, int b, const int *src, RawChunk<NT> &r) {
  using CS = ChunkShare<NT>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < CS::kFp4; ++u) {
    const int t = min(tid + u * NT, kFp4Tasks - 1);
    const int key = t >> 4, blk = t & 15;
    const int64_t row = (int64_t)b * a.S + min(max(src[key], 0), a.S - 1);
    const uint4 *cp = reinterpret_cast<const uint4 *>(a.swa_codes + row * kDNope + blk * 32);
    r.v[2 * u] = cp[0];
    r.v[2 * u + 1] = cp[1];
    r.s[u] = a.swa_scales[row * kNopeScales + blk];
  }
#pragma unroll
  for (int u = 0; u < CS::kRope; ++u) {
    const int t = min(tid + u * NT, kRopeTasks - 1);
    const int key = t >> 3, part = t & 7;
    const int64_t row = (int64_t)b * a.S + min(max(src[key], 0), a.S - 1);
    r.v[2 * CS::kFp4 + u] = *reinterpret_cast<const uint4 *>(a.swa_rope + row * kDRope + part * 8);
  }
}

template <int NT>
__device__ __forceinline__ void store_win8(uint16_t *K, const int *src, const RawChunk<NT> &r) {
  using CS = ChunkShare<NT>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < CS::kFp4; ++u) {
    const int t = tid + u * NT;
    if (t >= kFp4Tasks) break;
    const int key = t >> 4, blk = t & 15;
    uint4 *dst = reinterpret_cast<uint4 *>(K + key * kKRow + blk * 32);
    if (src[key] >= 0) {
      // E4M3 x 2^(s-127) -> bf16 (hardware conversion, two codes per call);
      // exact for the rows the encoder writes
      const float sc = e8m0_to_f32(r.s[u]);
      const uint4 c0 = r.v[2 * u], c1 = r.v[2 * u + 1];
#define CSA_CVT8(w, hi) __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, sc, hi))
      // quarter i of the 32 decoded channels = codes 8i..8i+7 = words 2i, 2i+1,
      // stored in the lane-dependent order of the MXFP4 path
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int qi = (i + blk + (blk >> 2)) & 3;
        const uint32_t w0 = qi == 0 ? c0.x : (qi == 1 ? c0.z : (qi == 2 ? c1.x : c1.z));
        const uint32_t w1 = qi == 0 ? c0.y : (qi == 1 ? c0.w : (qi == 2 ? c1.y : c1.w));
        dst[qi] = uint4{CSA_CVT8(w0, false), CSA_CVT8(w0, true), CSA_CVT8(w1, false), CSA_CVT8(w1, true)};
      }
#undef CSA_CVT8
    } else {
      const uint4 z = {0u, 0u, 0u, 0u};
      dst[0] = z;
      dst[1] = z;
      dst[2] = z;
      dst[3] = z;
    }
  }
#pragma unroll
  for (int u = 0; u < CS::kRope; ++u) {
    const int t = tid + u * NT;
    if (t < kRopeTasks) {
      const int key = t >> 3, part = t & 7;
      uint4 v = r.v[2 * CS::kFp4 + u];
      if (src[key] < 0) v = uint4{0u, 0u, 0u, 0u};
      *reinterpret_cast<uint4 *>(K + key * kKRow + kDNope + part * 8) = v;
    }
  }
}

// Window rows: `nb` 16-byte pieces per thread starting at task t0.
template <int NT, int nb>
__device__ __forceinline__ void load_window(const AttnArgs &a, int b, const int *src, int t0, RawChunk<NT> &r) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < nb; ++u) {
    const int t = min(t0 + tid + u * NT, kWinTasks - 1);
    const int key = t / kRowPieces, part = t % kRowPieces;
    const int64_t row = (int64_t)b * a.S + min(max(src[key], 0), a.S - 1);
    r.v[u] = *reinterpret_cast<const uint4 *>(a.swa + row * kD + part * 8);
  }
}

template <int NT, int nb>
__device__ __forceinline__ void store_window(uint16_t *K, const int *src, int t0, const RawChunk<NT> &r) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < nb; ++u) {
    const int t = t0 + tid + u * NT;
    if (t < kWinTasks) {
      const int key = t / kRowPieces, part = t % kRowPieces;
      uint4 v = r.v[u];
      if (src[key] < 0) v = uint4{0u, 0u, 0u, 0u};
      *reinterpret_cast<uint4 *>(K + key * kKRow + part * 8) = v;
    }
  }
}

template <int HG, bool kSplitP, bool kDense, bool kDupQK, bool kW8>
__global__ __launch_bounds__(HG * 128) void attn_kernel(AttnArgs a) {
  constexpr int NT = HG * 128;
  constexpr int kQSteps = kDupQK ? kKSteps : kKSteps / 2;  // channel steps of this wave's Q K^T
  using CS = ChunkShare<NT>;
  // Key-major bf16 tiles of the chunk (double buffered); the P V operand is
  // read transposed from the same tile with ds_read_b64_tr_b16.
  __shared__ __attribute__((aligned(16))) uint16_t Kl[2][kKC * kKRow];
  __shared__ __attribute__((aligned(16))) uint16_t Pl[2 * HG][kSplitP ? 2 : 1][16 * kPRow];
  __shared__ __attribute__((aligned(16))) float Sx[kDupQK ? 1 : 2 * HG][2 * 4 * 64];
  // Slot lists of three consecutive chunks: the list of chunk c + 1 is
  // written while a slower wave may still read that of chunk c.
  __shared__ int src_s[3][kKC];

  const int split = blockIdx.x % a.nsplit, q = blockIdx.x / a.nsplit, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r = lane & 15;
  // wave pair (2hg, 2hg+1) shares heads 16hg..16hg+15; `half` picks channels [288 half, +288)
  const int hg = wave >> 1, half = wave & 1;
  const int cbase = half * kHalfD;
  const int64_t qrow = (int64_t)b * a.Q + q;
  const int s_begin = split * a.per_split;
  // A slot's index load and its publication are split so that other loads
  // can be issued in between.
  auto fetch_slot = [&](int c0) __attribute__((always_inline)) {
    // unconditional load from a clamped address (no wait on the query's
    // position); the slot's validity is applied when it is published
    const int slot = c0 + (tid & (kKC - 1));
    if (kDense || a.k <= 0) return slot;
    return a.idx[qrow * a.k + min(slot, a.k - 1)];
  };
  const int j_first = fetch_slot(s_begin);
  const int p = a.q_pos[qrow];
  const int nE = min(a.n_entries[b], a.N_cap);
  const int V = p >= 0 ? max(0, min(nE, (p + 1) / a.m)) : 0;
  const int n_main = kDense ? V : a.k;
  const int n_main_pad = (n_main + kKC - 1) / kKC * kKC;
  int win_lo = 0, n_swa = 0, swa0 = 0;
  if (a.n_win > 0 && p >= 0) {
    swa0 = a.swa_pos0[b];
    win_lo = max(max(0, p - a.n_win + 1), swa0);
    const int win_hi = min(p, swa0 + a.S - 1);
    n_swa = max(0, win_hi - win_lo + 1);
  }
  const int n_slots = n_main_pad + n_swa;
  const int s_end = min(n_slots, s_begin + a.per_split);

  // Slot -> source row: an entry index (entry chunks) or a row of the window
  // buffer (window chunks); -1 = nothing.
  auto publish_slot = [&](int c0, int j, int sb) __attribute__((always_inline)) {
    if (tid < kKC) {
      const int slot = c0 + tid;
      int src = -1;
      if (slot < s_end) {
        if (slot < n_main_pad) {
          if (slot < n_main && j >= 0 && j < V) src = j;
        } else {
          src = win_lo + (slot - n_main_pad) - swa0;
        }
      }
      src_s[sb][tid] = src;
    }
  };

  float m2[4], lsum[4];
  v4f O[kHalfNT];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m2[i] = -INFINITY;
    lsum[i] = 0.f;
  }
#pragma unroll
  for (int j = 0; j < kHalfNT; ++j) O[j] = v4f{0.f, 0.f, 0.f, 0.f};

  v8bf Qf[kQSteps];
  if (s_begin < s_end) {
    const int j0 = j_first;  // issued before the query loads
    const uint16_t *qp = a.q + (qrow * a.H + hg * 16 + r) * kD + (kDupQK ? 0 : cbase) + 8 * g;
#pragma unroll
    for (int kk = 0; kk < kQSteps; ++kk) Qf[kk] = *reinterpret_cast<const v8bf *>(qp + 32 * kk);
    publish_slot(s_begin, j0, 0);
  }

  // S = Q K^T of one chunk for two tiles of 16 keys (two independent MFMA
  // chains), over this wave's channels.
  auto qk_part = [&](const uint16_t *K, v4f &S0, v4f &S1) __attribute__((always_inline)) {
    S0 = v4f{0.f, 0.f, 0.f, 0.f};
    S1 = v4f{0.f, 0.f, 0.f, 0.f};
    {
      const uint16_t *k0 = K + r * kKRow + (kDupQK ? 0 : cbase) + 8 * g;
      const uint16_t *k1 = k0 + 16 * kKRow;
#pragma unroll
      for (int kk = 0; kk < kQSteps; ++kk) {
        S0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Qf[kk], *reinterpret_cast<const v8bf *>(k0 + 32 * kk), S0, 0, 0,
                                                     0);
        S1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Qf[kk], *reinterpret_cast<const v8bf *>(k1 + 32 * kk), S1, 0, 0,
                                                     0);
      }
    }
  };
  // Adds the partner wave's half of the channels (one LDS-only barrier).
  auto exchange = [&](v4f &S0, v4f &S1) __attribute__((always_inline)) {
    if (!kDupQK) {
      // the partner's half of the channels, added in a fixed order of the
      // halves so that both waves of the pair agree bit for bit
      float *sx = &Sx[kDupQK ? 0 : wave][0];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sx[i * 64 + lane] = S0[i];
        sx[(4 + i) * 64 + lane] = S1[i];
      }
      lds_barrier();
      const float *so = &Sx[kDupQK ? 0 : wave ^ 1][0];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float o0 = so[i * 64 + lane], o1 = so[(4 + i) * 64 + lane];
        S0[i] = half == 0 ? S0[i] + o0 : o0 + S0[i];
        S1[i] = half == 0 ? S1[i] + o1 : o1 + S1[i];
      }
    }
  };
  // Online softmax of one chunk's logits, then O += P V with the chunk's
  // rows as V.
  auto softmax_pv = [&](const uint16_t *K, const v4f &S0, const v4f &S1, bool kv0, bool kv1)
                        __attribute__((always_inline)) {
    float alpha[4], p0[4], p1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x0 = kv0 ? S0[i] * a.scale_log2 : -INFINITY;
      const float x1 = kv1 ? S1[i] * a.scale_log2 : -INFINITY;
      const float tmax = row16_max(fmaxf(x0, x1));
      // The running maximum moves only when the chunk's maximum exceeds it by
      // more than 2^8 (or on the first keys): the result is the same for any
      // reference value, probabilities stay below 256, and the rescale of O
      // below is skipped in the common case.
      const float mn = (tmax > m2[i] + 8.f) ? tmax : m2[i];
      // branch-free: with no key yet (mn = -inf) the reference 0 gives
      // p = 0 and alpha = 0 on an empty state.  v_exp_f32 directly: results
      // below 2^-126 of the reference do not matter to these sums.
      const float mref = mn == -INFINITY ? 0.f : mn;
      alpha[i] = __builtin_amdgcn_exp2f(m2[i] - mref);
      p0[i] = __builtin_amdgcn_exp2f(x0 - mref);
      p1[i] = __builtin_amdgcn_exp2f(x1 - mref);
      lsum[i] = lsum[i] * alpha[i] + row16_sum(p0[i] + p1[i]);
      m2[i] = mn;
    }
    const bool moved = alpha[0] != 1.f || alpha[1] != 1.f || alpha[2] != 1.f || alpha[3] != 1.f;
    if (__builtin_amdgcn_ballot_w64(moved)) {
#pragma unroll
      for (int j = 0; j < kHalfNT; ++j) {
#pragma unroll
        for (int i = 0; i < 4; ++i) O[j][i] *= alpha[i];
      }
    }
    // P (bf16, or hi + lo) through this wave's LDS tile into the A layout
    // (LDS operations of one wave complete in order).  The product's key
    // order is permuted against the tile rows: MFMA key 8b + 4h + e (b < 4,
    // h, e < 4) is tile row 16h + 4b + e, so that each transposed V read
    // below covers 8 consecutive rows per 32 lanes, which a 1184-byte row
    // stride spreads over all LDS banks (measured conflict-free); tile row
    // r goes to P column 8(r/4) + r%4, tile row 16 + r to 8(r/4) + 4 + r%4.
    uint16_t *pw = &Pl[wave][0][0];
    const int pc0 = 8 * (r >> 2) + (r & 3);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t hi0 = f32_to_bf16(p0[i]), hi1 = f32_to_bf16(p1[i]);
      pw[(4 * g + i) * kPRow + pc0] = (uint16_t)hi0;
      pw[(4 * g + i) * kPRow + pc0 + 4] = (uint16_t)hi1;
      if (kSplitP) {
        uint16_t *pl = &Pl[wave][kSplitP ? 1 : 0][0];
        pl[(4 * g + i) * kPRow + pc0] = (uint16_t)f32_to_bf16(p0[i] - bf16_to_f32(hi0));
        pl[(4 * g + i) * kPRow + pc0 + 4] = (uint16_t)f32_to_bf16(p1[i] - bf16_to_f32(hi1));
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
    const v8bf Pa = *reinterpret_cast<const v8bf *>(&Pl[wave][0][r * kPRow + 8 * g]);
    v8bf Pb;
    if (kSplitP) Pb = *reinterpret_cast<const v8bf *>(&Pl[wave][kSplitP ? 1 : 0][r * kPRow + 8 * g]);
    // O += P V over this wave's 18 channel tiles; lane (g, r) needs
    // V[MFMA keys 8g..8g+7][channel c + r], i.e. tile rows 4g..4g+3 and
    // 16+4g..16+4g+3: two transposed 4x16 reads of the key-major tile.
    typedef __attribute__((address_space(3))) v4s lds_v4s;
    const uint16_t *vb = K + (4 * g + (r >> 2)) * kKRow + cbase + 4 * (r & 3);
#pragma unroll
    for (int j = 0; j < kHalfNT; ++j) {
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(vb + 16 * j));
      const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(vb + 16 * kKRow + 16 * j));
      const v8s both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      const v8bf Bv = __builtin_bit_cast(v8bf, both);
      O[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Pa, Bv, O[j], 0, 0, 0);
      if (kSplitP) O[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Pb, Bv, O[j], 0, 0, 0);
    }
  };
  // One chunk of decoded keys in K: logits, online softmax, O += P V.
  auto compute_chunk = [&](const uint16_t *K, bool kv0, bool kv1) __attribute__((always_inline)) {
    v4f S0, S1;
    qk_part(K, S0, S1);
    exchange(S0, S1);
    softmax_pv(K, S0, S1, kv0, kv1);
  };

  // Chunks of one kind in [c_lo, c_hi): decode the fetched rows into K,
  // publish the next slot list, one LDS-only barrier, fetch the next rows
  // (unconditionally: slots past the range read a clamped valid row), then
  // compute.  Buffers: K alternates between two tiles; slot lists rotate over
  // three (the list of chunk c + 1 is written while a slower wave may still
  // read that of chunk c); Sx is rewritten only after the next barrier.  The
  // list of c_lo is published and its rows fetched before the call.
  int ci = 0;
  auto run_chunks = [&](auto win_tag, int c_lo, int c_hi) __attribute__((always_inline)) {
    constexpr bool kWin = decltype(win_tag)::value;
    constexpr bool kWin16 = kWin && !kW8;   // bf16 window rows
    RawChunk<NT> raw;
    // whole-chunk loads and stores of entry chunks and FP8 window chunks
    auto ld = [&](int sb) __attribute__((always_inline)) {
      if (kWin16) load_window<NT, CS::kWinBatch>(a, b, src_s[sb], 0, raw);
      else if (kWin) load_win8<NT>(a, b, src_s[sb], raw);
      else load_entries<NT>(a, b, src_s[sb], raw);
    };
    auto st = [&](uint16_t *K, int sb) __attribute__((always_inline)) {
      if (kWin16) store_window<NT, CS::kWinBatch>(K, src_s[sb], 0, raw);
      else if (kWin) store_win8<NT>(K, src_s[sb], raw);
      else store_entries<NT>(K, src_s[sb], raw);
    };
    lds_barrier();
    if (CS::kAhead) ld(ci % 3);
    for (int c0 = c_lo; c0 < c_hi; c0 += kKC, ++ci) {
      uint16_t *K = Kl[ci & 1];
      const int sb = ci % 3, sn = (ci + 1) % 3;
      const int jn = kWin ? -1 : fetch_slot(c0 + kKC);
      if (CS::kAhead) {
        st(K, sb);
      } else if (kWin16) {
        for (int t0 = 0; t0 < kWinTasks; t0 += CS::kWinBatch * NT) {
          load_window<NT, CS::kWinBatch>(a, b, src_s[sb], t0, raw);
          store_window<NT, CS::kWinBatch>(K, src_s[sb], t0, raw);
        }
      } else {
        ld(sb);
        st(K, sb);
      }
      publish_slot(c0 + kKC, jn, sn);
      lds_barrier();
      const bool kv0 = src_s[sb][r] >= 0, kv1 = src_s[sb][16 + r] >= 0;
      if (CS::kAhead) ld(sn);
      compute_chunk(K, kv0, kv1);
    }
  };
  const int e_hi = min(s_end, n_main_pad);
  if (s_begin < e_hi) run_chunks(std::false_type{}, s_begin, e_hi);
  const int w_lo = max(s_begin, n_main_pad);
  if (w_lo < s_end) run_chunks(std::true_type{}, w_lo, s_end);  // its first list was published by the last entry chunk

  const int h0 = hg * 16;
  // bf16 results leave through LDS as 16-byte stores: the wave's 16 heads x
  // 288 channels in two halves of 144 channels, staged in the key tile no
  // wave reads any more (the one before the last chunk's: every wave passed
  // the last chunk's barrier after computing on it).  dst points at head
  // h0's row at channel cbase; rows are kD apart.
  constexpr bool kStaged = HG <= 4;  // 2*HG waves x 4,608 bytes within one key tile
  static_assert(!kStaged || 2 * HG * 16 * (kHalfD / 2) <= kKC * kKRow, "staging fits a key tile");
  auto store_bf16 = [&](uint16_t *dst, const float (&mul)[4]) __attribute__((always_inline)) {
    constexpr int kHalfCh = kHalfD / 2;  // 144
    uint16_t *stg = &Kl[ci & 1][0] + wave * (16 * kHalfCh);
#pragma unroll
    for (int hc = 0; hc < 2; ++hc) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < kHalfNT / 2; ++jj)
          stg[(4 * g + i) * kHalfCh + 16 * jj + r] = (uint16_t)f32_to_bf16(O[hc * (kHalfNT / 2) + jj][i] * mul[i]);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
#pragma unroll
      for (int it = 0; it < (16 * kHalfCh / 8 + 63) / 64; ++it) {
        const int vi = lane + 64 * it;
        if (vi < 16 * kHalfCh / 8) {
          const int row = vi / (kHalfCh / 8), c8 = (vi % (kHalfCh / 8)) * 8;
          const uint4 v = *reinterpret_cast<const uint4 *>(stg + row * kHalfCh + c8);
          *reinterpret_cast<uint4 *>(dst + (int64_t)row * kD + hc * kHalfCh + c8) = v;
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
    }
  };
  if (a.nsplit == 1 && a.out_bf16 && kStaged) {
    float inv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) inv[i] = lsum[i] > 0.f ? 1.f / lsum[i] : 0.f;
    store_bf16(reinterpret_cast<uint16_t *>(a.out) + (qrow * a.H + h0) * kD + cbase, inv);
    if (a.lse && r == 0 && half == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hh = h0 + 4 * g + i;
        a.lse[qrow * a.H + hh] = lsum[i] > 0.f ? (m2[i] + log2f(lsum[i])) * 0.69314718055994531f : -INFINITY;
      }
    }
  } else if (a.nsplit != 1 && a.out_bf16 && kStaged) {
    const float one[4] = {1.f, 1.f, 1.f, 1.f};
    store_bf16(reinterpret_cast<uint16_t *>(a.ws_o) + ((qrow * a.nsplit + split) * a.H + h0) * kD + cbase, one);
    if (r == 0 && half == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t pr = (qrow * a.nsplit + split) * a.H + h0 + 4 * g + i;
        a.ws_ml[pr * 2 + 0] = m2[i];
        a.ws_ml[pr * 2 + 1] = lsum[i];
      }
    }
  } else if (a.nsplit == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = h0 + 4 * g + i;
      const float inv = lsum[i] > 0.f ? 1.f / lsum[i] : 0.f;
      const int64_t ob = (qrow * a.H + hh) * kD + cbase;
      if (a.out_bf16) {
        uint16_t *o = reinterpret_cast<uint16_t *>(a.out) + ob;
#pragma unroll
        for (int j = 0; j < kHalfNT; ++j) o[16 * j + r] = (uint16_t)f32_to_bf16(O[j][i] * inv);
      } else {
        float *o = reinterpret_cast<float *>(a.out) + ob;
#pragma unroll
        for (int j = 0; j < kHalfNT; ++j) o[16 * j + r] = O[j][i] * inv;
      }
      if (a.lse && r == 0 && half == 0)
        a.lse[qrow * a.H + hh] = lsum[i] > 0.f ? (m2[i] + log2f(lsum[i])) * 0.69314718055994531f : -INFINITY;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = h0 + 4 * g + i;
      const int64_t pr = (qrow * a.nsplit + split) * a.H + hh;
      if (a.out_bf16) {
        // bf16 partials for a bf16 result: the merged error stays near the
        // output's own rounding (about 2^-9 of the row maximum per split)
        uint16_t *o = reinterpret_cast<uint16_t *>(a.ws_o) + pr * kD + cbase;
#pragma unroll
        for (int j = 0; j < kHalfNT; ++j) o[16 * j + r] = (uint16_t)f32_to_bf16(O[j][i]);
      } else {
        float *o = a.ws_o + pr * kD + cbase;
#pragma unroll
        for (int j = 0; j < kHalfNT; ++j) o[16 * j + r] = O[j][i];
      }
      if (r == 0 && half == 0) {
        a.ws_ml[pr * 2 + 0] = m2[i];
        a.ws_ml[pr * 2 + 1] = lsum[i];
      }
    }
  }
}

// Combines the splits: output = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s
// with M the largest m_s.  One thread per 8 channels of one (query, head):
// 16-byte loads of bf16 partials (8-byte halves of fp32 ones), the split
// weights formed once per thread, and the loads over splits issued together
// (up to kU at a time).  Partials are fp32, or bf16 when the
// result is bf16.
constexpr int kMergeThreads = 256;
// kU: splits whose loads go out together (8, or 16 / 32 for bf16 partials of
// many splits, so that the HCA step's 29 splits take one memory round).
// bf16 partials stay packed in registers until they are weighted.
template <bool kBf16, int kU>
__global__ __launch_bounds__(kMergeThreads) void attn_merge_kernel(const float *__restrict__ ws_o,
                                                                   const float *__restrict__ ws_ml, int nsplit, int H,
                                                                   int64_t n_items, void *out, float *lse) {
  const int64_t item = (int64_t)blockIdx.x * kMergeThreads + threadIdx.x;  // (qrow, head, channel group of 8)
  if (item >= n_items) return;
  constexpr int kGroups = kD / 8;
  const int64_t qh = item / kGroups;  // qrow * H + head
  const int c8 = (int)(item % kGroups) * 8;
  const int64_t qrow = qh / H, hh = qh % H;
  auto pr_of = [&](int s) { return (qrow * nsplit + s) * H + hh; };
  // One round of loads for up to kU splits: every split's (m, l) and partial
  // row are issued together and the maximum is formed from the loaded values
  // (a separate pass for the maximum would wait on memory twice).
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  float M = -INFINITY;
  for (int s0 = 0; s0 < nsplit; s0 += kU) {
    float2 ml[kU];
    uint4 raw[kBf16 ? kU : 2 * kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t pr = pr_of(min(s0 + u, nsplit - 1));
      ml[u] = *reinterpret_cast<const float2 *>(ws_ml + pr * 2);
      if (kBf16) {
        raw[u] = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(ws_o) + pr * kD + c8);
      } else {
        raw[2 * u] = *reinterpret_cast<const uint4 *>(ws_o + pr * kD + c8);
        raw[2 * u + 1] = *reinterpret_cast<const uint4 *>(ws_o + pr * kD + c8 + 4);
      }
    }
    // running maximum over the splits seen so far; earlier sums are rescaled
    // when it moves (only with more than kU splits)
    float Mn = M;
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (s0 + u < nsplit) Mn = fmaxf(Mn, ml[u].x);
    if (Mn != -INFINITY) {
      const float r = M == -INFINITY ? 0.f : exp2f(M - Mn);
      L *= r;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] *= r;
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const float wgt = (s0 + u < nsplit && ml[u].x != -INFINITY) ? exp2f(ml[u].x - Mn) : 0.f;
        L += wgt * (wgt != 0.f ? ml[u].y : 0.f);
        float v[8];
        if (kBf16) {
          const uint32_t w4[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            v[2 * j] = bf16_to_f32(w4[j] & 0xFFFFu);
            v[2 * j + 1] = bf16_to_f32(w4[j] >> 16);
          }
        } else {
          const uint4 p0 = raw[kBf16 ? 0 : 2 * u], p1 = raw[kBf16 ? 0 : 2 * u + 1];
          v[0] = __uint_as_float(p0.x); v[1] = __uint_as_float(p0.y); v[2] = __uint_as_float(p0.z);
          v[3] = __uint_as_float(p0.w); v[4] = __uint_as_float(p1.x); v[5] = __uint_as_float(p1.y);
          v[6] = __uint_as_float(p1.z); v[7] = __uint_as_float(p1.w);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = fmaf(wgt, v[j], acc[j]);
      }
      M = Mn;
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  if (kBf16) {
    uint32_t w4[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) w4[j] = f32_to_bf16(acc[2 * j] * inv) | (f32_to_bf16(acc[2 * j + 1] * inv) << 16);
    *reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(out) + qh * kD + c8) = uint4{w4[0], w4[1], w4[2], w4[3]};
  } else {
    float *o = reinterpret_cast<float *>(out) + qh * kD + c8;
    *reinterpret_cast<float4 *>(o) = float4{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
    *reinterpret_cast<float4 *>(o + 4) = float4{acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv};
  }
  if (lse && c8 == 0) lse[qh] = L > 0.f ? (M + log2f(L)) * 0.69314718055994531f : -INFINITY;
}

// Slots per query: the selected entries rounded up to whole chunks, then
// the window rows.
static int slots_max(int n_main, int n_win) { return (n_main + kKC - 1) / kKC * kKC + n_win; }

AttnShape attn_shape(int B, int Q, int n_main, int n_win) {
  const int n_slots_max = slots_max(n_main, n_win);
  const int chunks = n_slots_max > 0 ? (n_slots_max + kKC - 1) / kKC : 1;
  const int64_t rows = (int64_t)B * Q;
  int want = (int)(rows >= 256 ? 1 : (256 + rows - 1) / rows);
  want = want < chunks ? want : chunks;
  const int per_chunks = (chunks + want - 1) / want;
  const int nsplit = (chunks + per_chunks - 1) / per_chunks;
  return AttnShape{nsplit, per_chunks * kKC};
}

size_t attn_workspace_bytes(int B, int Q, int H, int n_main, int n_win) {
  const AttnShape s = attn_shape(B, Q, n_main, n_win);
  if (s.nsplit <= 1) return 0;
  return (size_t)B * Q * s.nsplit * H * (kD + 2) * sizeof(float);
}

#ifndef CSA_ATTN_DUP_QK
#define CSA_ATTN_DUP_QK 0
#endif
template <int HG, bool kSplitP>
static void launch_hg(const AttnArgs &a, bool dense, bool w8, dim3 grid, hipStream_t stream) {
  constexpr bool kDup = CSA_ATTN_DUP_QK != 0;
  if (dense && w8)
    attn_kernel<HG, kSplitP, true, kDup, true><<<grid, HG * 128, 0, stream>>>(a);
  else if (dense)
    attn_kernel<HG, kSplitP, true, kDup, false><<<grid, HG * 128, 0, stream>>>(a);
  else if (w8)
    attn_kernel<HG, kSplitP, false, kDup, true><<<grid, HG * 128, 0, stream>>>(a);
  else
    attn_kernel<HG, kSplitP, false, kDup, false><<<grid, HG * 128, 0, stream>>>(a);
}

template <bool kSplitP>
static void launch_split(const AttnArgs &a, bool dense, bool w8, dim3 grid, hipStream_t stream) {
  switch (a.H / 16) {
    case 1: launch_hg<1, kSplitP>(a, dense, w8, grid, stream); break;
    case 2: launch_hg<2, kSplitP>(a, dense, w8, grid, stream); break;
    case 4: launch_hg<4, kSplitP>(a, dense, w8, grid, stream); break;
    default: launch_hg<8, kSplitP>(a, dense, w8, grid, stream); break;
  }
}

hipError_t launch_attention(const CacheView &c, const uint16_t *q, int H, const int32_t *q_pos, int Q,
                            const int32_t *idx, int k, bool dense, const uint16_t *swa, const SwaPlanes *swa8,
                            const int32_t *swa_pos0, int S, int n_win, float scale, bool out_bf16, void *out,
                            float *lse, void *ws, hipStream_t stream) {
  const AttnShape sh = attn_shape(c.B, Q, dense ? c.N_cap : k, n_win);
  AttnArgs a;
  a.nope = c.nope;
  a.nscale = c.nscale;
  a.rope = c.rope;
  a.n_entries = c.n_entries;
  a.N_cap = c.N_cap;
  a.m = c.m;
  a.q = q;
  a.H = H;
  a.q_pos = q_pos;
  a.Q = Q;
  a.idx = idx;
  a.k = k;
  a.swa = swa;
  a.swa_codes = swa8 ? swa8->codes : nullptr;
  a.swa_scales = swa8 ? swa8->scales : nullptr;
  a.swa_rope = swa8 ? swa8->rope : nullptr;
  a.swa_pos0 = swa_pos0;
  a.S = S;
  a.n_win = n_win;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  a.out = out;
  a.lse = lse;
  a.out_bf16 = out_bf16 ? 1 : 0;
  a.nsplit = sh.nsplit;
  a.per_split = sh.per_split;
  const size_t po = (size_t)c.B * Q * sh.nsplit * H * kD;
  a.ws_o = reinterpret_cast<float *>(ws);
  a.ws_ml = a.ws_o ? a.ws_o + po : nullptr;
  dim3 grid((unsigned)(sh.nsplit * Q), c.B);
  if (out_bf16)
    launch_split<false>(a, dense, swa8 != nullptr, grid, stream);
  else
    launch_split<true>(a, dense, swa8 != nullptr, grid, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || sh.nsplit == 1) return e;
  const int64_t n_items = (int64_t)c.B * Q * H * (kD / 8);
  const unsigned nb = (unsigned)((n_items + kMergeThreads - 1) / kMergeThreads);
  if (out_bf16 && sh.nsplit > 16)
    attn_merge_kernel<true, 32><<<nb, kMergeThreads, 0, stream>>>(a.ws_o, a.ws_ml, sh.nsplit, H, n_items, out, lse);
  else if (out_bf16 && sh.nsplit > 8)
    attn_merge_kernel<true, 16><<<nb, kMergeThreads, 0, stream>>>(a.ws_o, a.ws_ml, sh.nsplit, H, n_items, out, lse);
  else if (out_bf16)
    attn_merge_kernel<true, 8><<<nb, kMergeThreads, 0, stream>>>(a.ws_o, a.ws_ml, sh.nsplit, H, n_items, out, lse);
  else
    attn_merge_kernel<false, 8><<<nb, kMergeThreads, 0, stream>>>(a.ws_o, a.ws_ml, sh.nsplit, H, n_items, out, lse);
  return hipGetLastError();
}

}  // namespace csa
