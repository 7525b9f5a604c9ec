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
// half of the 576 output channels and computes Q K^T over that half; the
// halves are swapped through LDS.  A query's key slots are its selected
// entries (padded to a multiple of the chunk size) followed by its window
// rows, so every chunk of 32 slots holds one kind of row and is fetched
// with the loads of that kind only.  Per chunk:
//   1. the workgroup decodes the 32 rows into a key-major bf16 LDS tile
//      (E2M1 x E8M0 -> bf16 is exact; gfx950's v_cvt_scalef32_pk_bf16_fp4
//      converts two codes per instruction); the raw bytes of the next chunk
//      are fetched into registers while the current one is computed (the
//      tile and the slot lists are multi-buffered, one barrier per chunk);
//   2. S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (lane (g, r): head r, keys
//      4g..4g+3 of each 16-key tile), online softmax per head in the log2
//      domain, reduced in registers and across the lane groups by permlane
//      swaps (both waves of a pair hold bit-identical logits);
//   3. the lane's 8 probabilities are its A operand of O += P V as they are
//      (the MFMA key order is permuted against the tile rows to match), so
//      P never goes through LDS; the V operand (keys along K) is read
//      transposed from the same key-major tile with ds_read_b64_tr_b16, so
//      no second copy of the keys is written.  With fp32 outputs P is split
//      into two bf16 parts (hi + lo) so that the probabilities keep ~16
//      bits.
// Splits write unnormalised (O, max, sum) partials that a merge kernel
// combines; a single split writes the normalised output directly.
#include <cmath>
#include <type_traits>

#include "csa_device.hpp"
#include "csa_internal.hpp"

namespace csa {

constexpr int kKC = 32;           // key slots per chunk
// The running maximum before any key: finite, so that it can serve as the
// exponent's reference as it is (exp2 of a logit minus it is 0 for a masked
// key, -inf, and for a real one it is replaced first), and far below every
// logit in the log2 domain.
constexpr float kNoMax = -3.0e38f;
// Key-major LDS row (bf16 elements).  Padding of 16 elements: with a
// 1184-byte row the Q K^T operand reads (16 rows x 16 bytes per lane group)
// run conflict-free, measured 4 LDS cycles per instruction against 8 with
// 8 elements of padding.
constexpr int kKRow = kD + 16;
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
  uint32_t *flags;             // device fault word (may be null)
  // Fused rotary epilogue: rot != 0 turns channel pair (2i, 2i+1) of the
  // 64 positional channels by pos * base^(-2i/64) radians; rot_turns[i] is
  // base^(-2i/64) / (2 pi), the turn per position, in fp64.
  int rot;
  double rot_turns[kDRope / 2];
  // Workgroup -> (query row, split).  With xcd != 0 (at least 8 rows) every
  // split of row r gets a linear id = r (mod 8): workgroups are dealt to the
  // 8 XCDs round-robin by linear id, so a row's query, its partials and its
  // merge stay in one XCD's L2.
  int rows, xcd;
};

// The XCD-aware order: workgroup L sits on XCD L % 8 and takes the
// (L / 8)-th (row, part) pair of that XCD's rows r = x, x + 8, ...
// Returns false for the workgroups past the last row.
__device__ __forceinline__ bool xcd_slot(int L, int per_row, int rows, int &row, int &part) {
  const int x = L & 7, sidx = L >> 3;
  row = x + 8 * (sidx / per_row);
  part = sidx % per_row;
  return row < rows;
}

// Two fp32 values as bf16 (round to nearest even) in one word, low first:
// one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float v2f_t __attribute__((ext_vector_type(2)));
  typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f_t{lo, hi}, v2bf_t));
}

// Reductions over the four lane groups g (lanes r, r + 16, r + 32, r + 48):
// a swap of the 32-lane halves, then of the 16-lane rows inside them.  Every
// lane takes the same operands in the same order, so the four groups end
// with the same bits.
__device__ __forceinline__ float allgroups_max(float v) {
  const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(x[0]), __uint_as_float(x[1]));
  const auto y = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(y[0]), __uint_as_float(y[1]));
}
__device__ __forceinline__ float allgroups_sum(float v) {
  const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(x[0]) + __uint_as_float(x[1]);
  const auto y = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(y[0]) + __uint_as_float(y[1]);
}

// cos and sin of the rotary angle of pair i at position pos: the angle in
// turns is reduced to [0, 1) in fp64 (exact to ~1e-10 turn for positions
// below 2^31), then the fp32 hardware cosine and sine (which take turns)
// are evaluated on it.
__device__ __forceinline__ float2 rope_cs(int64_t pos, double turns) {
  const double t = (double)pos * turns;
  const float r = (float)(t - floor(t));
  return float2{__builtin_amdgcn_cosf(r), __builtin_amdgcn_sinf(r)};
}

// One word of two bf16 channels (2i low, 2i+1 high) turned by the angle
// (c, s), rounded back to bf16.
__device__ __forceinline__ uint32_t rope_pair(uint32_t w, float c, float s) {
  const float x = __uint_as_float(w << 16), y = __uint_as_float(w & 0xFFFF0000u);
  return f32_to_bf16(x * c - y * s) | (f32_to_bf16(x * s + y * c) << 16);
}

// 8 positional channels 8 part .. 8 part + 7 (four pairs) of a row at
// position pos, rotated.
__device__ __forceinline__ uint4 rope_piece(const AttnArgs &a, uint4 v, int64_t pos, int part) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float2 cs = rope_cs(pos, a.rot_turns[4 * part + k]);
    w[k] = rope_pair(w[k], cs.x, cs.y);
  }
  return uint4{w[0], w[1], w[2], w[3]};
}

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

template <int NT, bool kRot>
__device__ __forceinline__ void store_entries(const AttnArgs &a, uint16_t *K, const int *src, const RawChunk<NT> &r) {
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
      // the words rotated by rot in two select stages (by 1, then by 2),
      // so that store i takes quarter (i + rot) & 3 from register i
      const int rot = (blk + (blk >> 2)) & 3;
      const bool r1 = rot & 1, r2 = rot & 2;
      const uint32_t a0 = r1 ? c.y : c.x, a1 = r1 ? c.z : c.y, a2 = r1 ? c.w : c.z, a3 = r1 ? c.x : c.w;
      const uint32_t cw[4] = {r2 ? a2 : a0, r2 ? a3 : a1, r2 ? a0 : a2, r2 ? a1 : a3};
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[(i + rot) & 3] = CSA_CVT4(cw[i]);
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
      const int j = src[key];
      // a compressed entry sits at its last raw token, (j + 1) m - 1
      if (kRot && j >= 0) v = rope_piece(a, v, (int64_t)(j + 1) * a.m - 1, part);
      if (j < 0) v = uint4{0u, 0u, 0u, 0u};
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

template <int NT, bool kRot>
__device__ __forceinline__ void store_win8(const AttnArgs &a, int swa0, uint16_t *K, const int *src,
                                           const RawChunk<NT> &r) {
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
      const int row = src[key];
      if (kRot && row >= 0) v = rope_piece(a, v, (int64_t)swa0 + row, part);  // a window row at its raw position
      if (row < 0) v = uint4{0u, 0u, 0u, 0u};
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

template <int NT, int nb, bool kRot>
__device__ __forceinline__ void store_window(const AttnArgs &a, int swa0, uint16_t *K, const int *src, int t0,
                                             const RawChunk<NT> &r) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < nb; ++u) {
    const int t = t0 + tid + u * NT;
    if (t < kWinTasks) {
      const int key = t / kRowPieces, part = t % kRowPieces;
      uint4 v = r.v[u];
      const int row = src[key];
      constexpr int kRope0 = kDNope / 8;  // first positional piece of a row
      if (kRot && row >= 0 && part >= kRope0) v = rope_piece(a, v, (int64_t)swa0 + row, part - kRope0);
      if (row < 0) v = uint4{0u, 0u, 0u, 0u};
      *reinterpret_cast<uint4 *>(K + key * kKRow + part * 8) = v;
    }
  }
}

template <int HG, bool kSplitP, bool kDense, bool kW8, bool kRot>
__global__ __launch_bounds__(HG * 128) void attn_kernel(AttnArgs a) {
  constexpr int NT = HG * 128;
  constexpr int kQSteps = kKSteps / 2;  // channel steps of this wave's Q K^T
  using CS = ChunkShare<NT>;
  // Key-major bf16 tiles of the chunk (double buffered); the P V operand is
  // read transposed from the same tile with ds_read_b64_tr_b16.
  __shared__ __attribute__((aligned(16))) uint16_t Kl[2][kKC * kKRow];
  __shared__ __attribute__((aligned(16))) float Sx[2 * HG][2 * 4 * 64];
  // Slot lists of three consecutive chunks: the list of chunk c + 1 is
  // written while a slower wave may still read that of chunk c.
  __shared__ __attribute__((aligned(16))) int src_s[3][kKC];
  // per slot of those lists: 0 for a key, -inf for none (added to the logit)
  __shared__ __attribute__((aligned(16))) float bias_s[3][kKC];

  int row_id, split;
  if (a.xcd) {
    if (!xcd_slot(blockIdx.x, a.nsplit, a.rows, row_id, split)) return;  // the whole workgroup, before any barrier
  } else {
    row_id = blockIdx.x / a.nsplit;
    split = blockIdx.x % a.nsplit;
  }
  const int q = row_id % a.Q, b = row_id / a.Q;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r = lane & 15;
  // wave pair (2hg, 2hg+1) shares heads 16hg..16hg+15; `half` picks channels [288 half, +288)
  const int hg = wave >> 1, half = wave & 1;
  const int cbase = half * kHalfD;
  const int64_t qrow = (int64_t)b * a.Q + q;
  const int s_begin = split * a.per_split;
  // A slot's index load and its publication are split so that other loads
  // can be issued in between.  The index of the slot before is loaded with
  // it (same cache lines) for the ascending-order check.
  auto fetch_slot = [&](int c0) __attribute__((always_inline)) {
    // unconditional loads from clamped addresses (no wait on the query's
    // position); the slot's validity is applied when it is published
    const int slot = c0 + (tid & (kKC - 1));
    if (kDense || a.k <= 0) return int2{slot, slot - 1};
    const int sc = min(slot, a.k - 1);
    const int32_t *ip = a.idx + qrow * a.k;
    return int2{ip[sc], ip[max(sc - 1, 0)]};
  };
  // Every load the prologue needs goes out in one round: the first slot's
  // index, the query's position, the entry count, the window's first row
  // and the query itself (valid addresses whatever the position turns out
  // to be); nothing waits on another load.
  const int2 j_first = fetch_slot(s_begin);
  const int p = a.q_pos[qrow];
  const int nE_raw = a.n_entries[b];
  const int swa0_raw = a.n_win > 0 ? a.swa_pos0[b] : 0;
  v8bf Qf[kQSteps];
  {
    const uint16_t *qp = a.q + (qrow * a.H + hg * 16 + r) * kD + cbase + 8 * g;
#pragma unroll
    for (int kk = 0; kk < kQSteps; ++kk) Qf[kk] = *reinterpret_cast<const v8bf *>(qp + 32 * kk);
  }
  const int nE = min(nE_raw, a.N_cap);
  const int V = p >= 0 ? max(0, min(nE, (p + 1) / a.m)) : 0;
  const int n_main = kDense ? V : a.k;
  const int n_main_pad = (n_main + kKC - 1) / kKC * kKC;
  int win_lo = 0, n_swa = 0, swa0 = 0;
  if (a.n_win > 0 && p >= 0) {
    swa0 = swa0_raw;
    win_lo = max(max(0, p - a.n_win + 1), swa0);
    const int win_hi = min(p, swa0 + a.S - 1);
    n_swa = max(0, win_hi - win_lo + 1);
  }
  const int n_slots = n_main_pad + n_swa;
  const int s_end = min(n_slots, s_begin + a.per_split);
  if (tid == 0 && split == 0) {
    // per (sequence, query): an entry count outside [0, N_cap], window rows
    // that the buffer does not hold (they are skipped)
    uint32_t f = (nE_raw < 0 || nE_raw > a.N_cap) ? kFaultEntries : 0u;
    if (a.n_win > 0 && p >= 0 && (swa0 > max(0, p - a.n_win + 1) || p > swa0 + a.S - 1)) f |= kFaultWindow;
    if (f) raise_fault(a.flags, f);
  }

  // Slot -> source row: an entry index (entry chunks) or a row of the window
  // buffer (window chunks); -1 = nothing.  Selected indices outside
  // [-1, V) and neighbours that are not strictly ascending raise fault bits
  // (the former are skipped, the latter attended as given).
  auto publish_slot = [&](int c0, int2 jj, int sb) __attribute__((always_inline)) {
    if (tid < kKC) {
      const int slot = c0 + tid;
      const int j = jj.x;
      int src = -1;
      if (slot < s_end) {
        if (slot < n_main_pad) {
          if (slot < n_main && j >= 0 && j < V) src = j;
          if (!kDense && slot < n_main) {
            uint32_t f = (j < -1 || j >= V) ? kFaultIdxRange : 0u;
            if (slot > 0 && j >= 0 && jj.y >= 0 && j <= jj.y) f |= kFaultIdxOrder;
            if (f) raise_fault(a.flags, f);
          }
        } else {
          src = win_lo + (slot - n_main_pad) - swa0;
        }
      }
      src_s[sb][tid] = src;
      bias_s[sb][tid] = src >= 0 ? 0.f : -INFINITY;
    }
  };

  // Softmax state of head r (lane (g, r); the four lane groups hold the same
  // bits): the running maximum in the log2 domain and the running sum.
  float hm = kNoMax, hl = 0.f;
  v4f O[kHalfNT];
#pragma unroll
  for (int j = 0; j < kHalfNT; ++j) O[j] = v4f{0.f, 0.f, 0.f, 0.f};

  if (s_begin < s_end) {
    const int2 j0 = j_first;
    if (kRot) {
      // the first rotation of the fused epilogue: the query's positional
      // channels turned by its own position (rounded to bf16 as they are
      // stored)
#pragma unroll
      for (int kk = 0; kk < kQSteps; ++kk) {
        const int c0 = cbase + 32 * kk + 8 * g;
        if (c0 >= kDNope)
          Qf[kk] = __builtin_bit_cast(v8bf, rope_piece(a, __builtin_bit_cast(uint4, Qf[kk]), p, (c0 - kDNope) / 8));
      }
    }
    publish_slot(s_begin, j0, 0);
  }

  // S^T = K Q^T of one chunk for two tiles of 16 keys (two independent MFMA
  // chains), over this wave's channels: the key tile is the A operand and
  // the query the B operand (the same registers as Q K^T, in the other
  // slots), so lane (g, r) gets head r's logits for tile rows 4g..4g+3
  // (S0) and 16+4g..16+4g+3 (S1).
  auto qk_part = [&](const uint16_t *K, v4f &S0, v4f &S1) __attribute__((always_inline)) {
    S0 = v4f{0.f, 0.f, 0.f, 0.f};
    S1 = v4f{0.f, 0.f, 0.f, 0.f};
    {
      const uint16_t *k0 = K + r * kKRow + cbase + 8 * g;
      const uint16_t *k1 = k0 + 16 * kKRow;
#pragma unroll
      for (int kk = 0; kk < kQSteps; ++kk) {
        S0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const v8bf *>(k0 + 32 * kk), Qf[kk], S0, 0, 0,
                                                     0);
        S1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const v8bf *>(k1 + 32 * kk), Qf[kk], S1, 0, 0,
                                                     0);
      }
    }
  };
  // Adds the partner wave's half of the channels (one LDS-only barrier).
  auto exchange = [&](v4f &S0, v4f &S1) __attribute__((always_inline)) {
    // the partner's half of the channels, added in a fixed order of the
    // halves so that both waves of the pair agree bit for bit
    // 8 values per lane as two 16-byte stores and loads
    float4 *sx = reinterpret_cast<float4 *>(&Sx[wave][0]) + 2 * lane;
    sx[0] = float4{S0[0], S0[1], S0[2], S0[3]};
    sx[1] = float4{S1[0], S1[1], S1[2], S1[3]};
    lds_barrier();
    const float4 *so = reinterpret_cast<const float4 *>(&Sx[wave ^ 1][0]) + 2 * lane;
    const float4 o0 = so[0], o1 = so[1];
    const float p0[4] = {o0.x, o0.y, o0.z, o0.w}, p1[4] = {o1.x, o1.y, o1.z, o1.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      S0[i] = half == 0 ? S0[i] + p0[i] : p0[i] + S0[i];
      S1[i] = half == 0 ? S1[i] + p1[i] : p1[i] + S1[i];
    }
  };
  // Online softmax of one chunk's logits, then O += P V with the chunk's
  // rows as V.
  // Online softmax of one chunk's logits for head r, then O += P V with the
  // chunk's rows as V.  bias: the chunk's slot biases (0 / -inf).
  auto softmax_pv = [&](const uint16_t *K, const v4f &S0, const v4f &S1, const float *bias)
                        __attribute__((always_inline)) {
    const float4 b0 = *reinterpret_cast<const float4 *>(bias + 4 * g);
    const float4 b1 = *reinterpret_cast<const float4 *>(bias + 16 + 4 * g);
    // raw logits, masked by adding the slot's 0 / -inf (exact either way);
    // the scale (positive) is applied to the row maximum and inside the
    // exponent (max(a c, b c) = c max(a, b) exactly)
    const float x[8] = {S0[0] + b0.x, S0[1] + b0.y, S0[2] + b0.z, S0[3] + b0.w,
                        S1[0] + b1.x, S1[1] + b1.y, S1[2] + b1.z, S1[3] + b1.w};
    // head r's maximum: the lane's 8 keys, then the four lane groups
    // (permlane swaps of the 32-lane and 16-lane halves; every group ends
    // with the same bits)
    float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
    mx = allgroups_max(mx);
    const float tmax = mx * a.scale_log2;
    // The running maximum moves only when the chunk's maximum exceeds it by
    // more than 2^8 (or on the first keys): the result is the same for any
    // reference value, probabilities stay below 256, and the rescale of O
    // below is skipped in the common case.  With no key yet the reference
    // is kNoMax and every p is 0 (masked logits are -inf); the first keys
    // move it (alpha = 0 on the empty state).  v_exp_f32 directly: results
    // below 2^-126 of the reference do not matter to these sums.
    const float mn = (tmax > hm + 8.f) ? tmax : hm;
    float pv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pv[e] = __builtin_amdgcn_exp2f(fmaf(x[e], a.scale_log2, -mn));
    if (__builtin_amdgcn_ballot_w64(mn != hm)) {
      // O rows are heads 4g..4g+3 (lane (g, r)); their factors come from
      // lanes 16g + 4g + i, whose head is 4g + i
      const float alpha = __builtin_amdgcn_exp2f(hm - mn);
      hl *= alpha;
      float al[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        al[i] = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * (20 * g + i), __float_as_int(alpha)));
#pragma unroll
      for (int j = 0; j < kHalfNT; ++j) {
#pragma unroll
        for (int i = 0; i < 4; ++i) O[j][i] *= al[i];
      }
    }
    hm = mn;
    hl += allgroups_sum(((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7])));
    // P stays in registers: lane (g, r) holds P[head r][MFMA keys 8g..8g+7],
    // exactly its A operand of P V.  The product's key order is permuted
    // against the tile rows: MFMA key 8b + 4h + e (b < 4, h, e < 4) is tile
    // row 16h + 4b + e, so that each transposed V read below covers 8
    // consecutive rows per 32 lanes, which a 1184-byte row stride spreads
    // over all LDS banks (measured conflict-free); with b = g that is tile
    // rows 4g + e (S0) and 16 + 4g + e (S1), the lane's own logits.
    uint32_t hw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) hw[e] = pack_bf16x2(pv[2 * e], pv[2 * e + 1]);
    const v8bf Pa = __builtin_bit_cast(v8bf, uint4{hw[0], hw[1], hw[2], hw[3]});
    v8bf Pb;
    if (kSplitP) {
      // fp32 outputs: the probabilities as bf16 hi + lo (about 16 bits)
      uint32_t lw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        lw[e] = pack_bf16x2(pv[2 * e] - __uint_as_float(hw[e] << 16),
                            pv[2 * e + 1] - __uint_as_float(hw[e] & 0xFFFF0000u));
      Pb = __builtin_bit_cast(v8bf, uint4{lw[0], lw[1], lw[2], lw[3]});
    }
    // O += P V over this wave's 18 channel tiles; lane (g, r) needs
    // V[MFMA keys 8g..8g+7][channel c + r], i.e. tile rows 4g..4g+3 and
    // 16+4g..16+4g+3: two transposed 4x16 reads of the key-major tile.
    typedef __attribute__((address_space(3))) v4s lds_v4s;
    const uint16_t *vb = K + (4 * g + (r >> 2)) * kKRow + cbase + 4 * (r & 3);
#pragma unroll
    for (int j = 0; j < kHalfNT; ++j) {
      const v4s lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(vb + 16 * j));
      const v4s hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(vb + 16 * kKRow + 16 * j));
      const v8s both = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
      const v8bf Bv = __builtin_bit_cast(v8bf, both);
      O[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Pa, Bv, O[j], 0, 0, 0);
      if (kSplitP) O[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Pb, Bv, O[j], 0, 0, 0);
    }
  };
  // One chunk of decoded keys in K: logits, online softmax, O += P V.
  auto compute_chunk = [&](const uint16_t *K, const float *bias) __attribute__((always_inline)) {
    v4f S0, S1;
    qk_part(K, S0, S1);
    exchange(S0, S1);
    softmax_pv(K, S0, S1, bias);
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
      if (kWin16) store_window<NT, CS::kWinBatch, kRot>(a, swa0, K, src_s[sb], 0, raw);
      else if (kWin) store_win8<NT, kRot>(a, swa0, K, src_s[sb], raw);
      else store_entries<NT, kRot>(a, K, src_s[sb], raw);
    };
    lds_barrier();
    if (CS::kAhead) ld(ci % 3);
    for (int c0 = c_lo; c0 < c_hi; c0 += kKC, ++ci) {
      uint16_t *K = Kl[ci & 1];
      const int sb = ci % 3, sn = (ci + 1) % 3;
      const int2 jn = kWin ? int2{-1, -1} : fetch_slot(c0 + kKC);
      if (CS::kAhead) {
        st(K, sb);
      } else if (kWin16) {
        for (int t0 = 0; t0 < kWinTasks; t0 += CS::kWinBatch * NT) {
          load_window<NT, CS::kWinBatch>(a, b, src_s[sb], t0, raw);
          store_window<NT, CS::kWinBatch, kRot>(a, swa0, K, src_s[sb], t0, raw);
        }
      } else {
        ld(sb);
        st(K, sb);
      }
      publish_slot(c0 + kKC, jn, sn);
      lds_barrier();
      if (CS::kAhead) ld(sn);
      compute_chunk(K, bias_s[sb]);
    }
  };
  const int e_hi = min(s_end, n_main_pad);
  if (s_begin < e_hi) run_chunks(std::false_type{}, s_begin, e_hi);
  const int w_lo = max(s_begin, n_main_pad);
  if (w_lo < s_end) run_chunks(std::true_type{}, w_lo, s_end);  // its first list was published by the last entry chunk

  // The second rotation of the fused epilogue: the output's positional
  // channels turned back by -p.  The rotation is linear, so it applies to
  // unnormalised partials too.  Lane (g, r) holds channel cbase + 16 j + r of
  // four heads; its pair partner is the neighbouring lane (r ^ 1).
  if (kRot) {
#pragma unroll
    for (int j = 0; j < kHalfNT; ++j) {
      const int c = cbase + 16 * j;  // uniform in the wave
      if (c < kDNope) continue;
      const float2 cs = rope_cs(p, a.rot_turns[(c - kDNope + r) >> 1]);
      const float sn = (r & 1) ? -cs.y : cs.y;  // (x, y) -> (x c + y s, y c - x s)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float mine = O[j][i];
        const float other = __builtin_bit_cast(
            float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, mine), 0xB1, 0xF, 0xF, false));
        O[j][i] = mine * cs.x + other * sn;
      }
    }
  }
  // The state of the output rows' heads 4g + i, from lanes 16g + 4g + i.
  float m2[4], lsum[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m2[i] = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * (20 * g + i), __float_as_int(hm)));
    lsum[i] = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * (20 * g + i), __float_as_int(hl)));
  }
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
        a.ws_ml[pr * 2 + 0] = lsum[i] > 0.f ? m2[i] : -INFINITY;  // -inf: a split without keys
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
        a.ws_ml[pr * 2 + 0] = lsum[i] > 0.f ? m2[i] : -INFINITY;  // -inf: a split without keys
        a.ws_ml[pr * 2 + 1] = lsum[i];
      }
    }
  }
}

// Combines the splits: output = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s
// with M the largest m_s.  kT adjacent lanes share one (query, head, group
// of 8 channels): lane t takes splits t, t + kT, t + 2 kT, ... and keeps its
// own (max, sum, 8 weighted channels); the kT states are then combined by
// DPP moves inside the lane quad (exchange with lane ^ 1, then lane ^ 2),
// and lane t = 0 writes.  Each lane issues the loads of up to kU of its
// splits in one round: 16-byte loads of bf16 partials (8-byte halves of
// fp32 ones) and the (max, sum) pairs, the maximum formed from the loaded
// values.  With many splits (the dense 1M step's 29) the lanes of a group
// wait on a quarter of the loads each, and the grid has kT times the
// workgroups.  Partials are fp32, or bf16 when the result is bf16.
constexpr int kMergeThreads = 256;
template <bool kBf16, int kU, int kT>
__global__ __launch_bounds__(kMergeThreads) void attn_merge_kernel(const float *__restrict__ ws_o,
                                                                   const float *__restrict__ ws_ml, int nsplit, int H,
                                                                   int64_t n_items, void *out, float *lse, int rows,
                                                                   int xcd, int wg_per_row) {
  static_assert(kT == 1 || kT == 2 || kT == 4, "lane groups within a DPP quad");
  static_assert(kMergeThreads % kT == 0, "groups never straddle a workgroup");
  constexpr int kGroups = kD / 8;
  const int t = threadIdx.x % kT;
  int64_t item;  // (qrow, head, channel group of 8); the same for the kT lanes of a group
  if (xcd) {
    // the row's splits ran on XCD row % 8 (xcd_slot): merge it there
    int row, part;
    if (!xcd_slot(blockIdx.x, wg_per_row, rows, row, part)) return;
    const int in_row = (part * kMergeThreads + threadIdx.x) / kT;
    if (in_row >= H * kGroups) return;  // whole groups only
    item = (int64_t)row * H * kGroups + in_row;
  } else {
    item = ((int64_t)blockIdx.x * kMergeThreads + threadIdx.x) / kT;
    if (item >= n_items) return;
  }
  const int64_t qh = item / kGroups;  // qrow * H + head
  const int c8 = (int)(item % kGroups) * 8;
  const int64_t qrow = qh / H, hh = qh % H;
  // Split s of this item: partial row (qrow * nsplit + s) * H + hh.  The
  // row's base is formed once in 64 bits; a split's offset from it,
  // s * H * (kD + 2) elements at most, stays far below 2^31.
  const int64_t pr0 = qrow * nsplit * H + hh;
  const float *ml_base = ws_ml + pr0 * 2;
  const uint16_t *o16_base = reinterpret_cast<const uint16_t *>(ws_o) + pr0 * kD + c8;
  const float *o32_base = ws_o + pr0 * kD + c8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  float M = -INFINITY;
  const int n_per = (nsplit + kT - 1) / kT;  // splits of the busiest lane
  for (int u0 = 0; u0 < n_per; u0 += kU) {
    float2 ml[kU];
    uint4 raw[kBf16 ? kU : 2 * kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int ds = min(t + kT * (u0 + u), nsplit - 1) * H;  // partial rows past the base
      ml[u] = *reinterpret_cast<const float2 *>(ml_base + ds * 2);
      if (kBf16) {
        raw[u] = *reinterpret_cast<const uint4 *>(o16_base + ds * kD);
      } else {
        raw[2 * u] = *reinterpret_cast<const uint4 *>(o32_base + ds * kD);
        raw[2 * u + 1] = *reinterpret_cast<const uint4 *>(o32_base + ds * kD + 4);
      }
    }
    // running maximum over the splits seen so far; earlier sums are rescaled
    // when it moves (only with more than kU splits per lane)
    float Mn = M;
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (t + kT * (u0 + u) < nsplit) Mn = fmaxf(Mn, ml[u].x);
    if (Mn != -INFINITY) {
      // v_exp_f32 directly: a weight below 2^-126 of the largest adds nothing
      const float r = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
      L *= r;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] *= r;
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const float wgt =
            (t + kT * (u0 + u) < nsplit && ml[u].x != -INFINITY) ? __builtin_amdgcn_exp2f(ml[u].x - Mn) : 0.f;
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
  // The kT lane states combined: quad_perm [1,0,3,2] (lane ^ 1), then
  // [2,3,0,1] (lane ^ 2).  A state with no key (M = -inf) weighs 0.
  auto combine = [&](auto ctrl_tag) __attribute__((always_inline)) {
    constexpr int kCtrl = decltype(ctrl_tag)::value;
    auto mv = [](float x) { return __int_as_float(dpp_i32<kCtrl>(__float_as_int(x))); };
    const float Mp = mv(M), Lp = mv(L);
    const float Mn = fmaxf(M, Mp);
    const float ws = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
    const float wp = Mp == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(Mp - Mn);
    L = L * ws + Lp * wp;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = acc[j] * ws + mv(acc[j]) * wp;
    M = Mn;
  };
  if (kT >= 2) combine(std::integral_constant<int, 0xB1>{});
  if (kT >= 4) combine(std::integral_constant<int, 0x4E>{});
  if (t != 0) return;
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

template <int HG, bool kSplitP, bool kRot>
static void launch_hg_rot(const AttnArgs &a, bool dense, bool w8, dim3 grid, hipStream_t stream) {
  if (dense && w8)
    attn_kernel<HG, kSplitP, true, true, kRot><<<grid, HG * 128, 0, stream>>>(a);
  else if (dense)
    attn_kernel<HG, kSplitP, true, false, kRot><<<grid, HG * 128, 0, stream>>>(a);
  else if (w8)
    attn_kernel<HG, kSplitP, false, true, kRot><<<grid, HG * 128, 0, stream>>>(a);
  else
    attn_kernel<HG, kSplitP, false, false, kRot><<<grid, HG * 128, 0, stream>>>(a);
}

// The rotary epilogue is a separate instantiation: its rotation sits in the
// chunk loop's decode, and the registers it needs would otherwise be held
// by the kernel without it too.
template <int HG, bool kSplitP>
static void launch_hg(const AttnArgs &a, bool dense, bool w8, dim3 grid, hipStream_t stream) {
  if (a.rot)
    launch_hg_rot<HG, kSplitP, true>(a, dense, w8, grid, stream);
  else
    launch_hg_rot<HG, kSplitP, false>(a, dense, w8, grid, stream);
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
                            const int32_t *swa_pos0, int S, int n_win, float scale, double rope_base,
                            bool out_bf16, void *out, float *lse, void *ws, hipStream_t stream) {
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
  a.flags = c.flags;
  a.rot = rope_base > 0.0 ? 1 : 0;
  for (int i = 0; i < kDRope / 2; ++i)
    a.rot_turns[i] = a.rot ? std::pow(rope_base, -2.0 * i / kDRope) / (2.0 * 3.14159265358979323846) : 0.0;
  const size_t po = (size_t)c.B * Q * sh.nsplit * H * kD;
  a.ws_o = reinterpret_cast<float *>(ws);
  a.ws_ml = a.ws_o ? a.ws_o + po : nullptr;
  a.rows = c.B * Q;
  a.xcd = a.rows >= 8 && sh.nsplit > 1 ? 1 : 0;  // fewer rows would leave XCDs idle; one split has no merge
  dim3 grid(a.xcd ? (unsigned)(8 * ((a.rows + 7) / 8) * sh.nsplit) : (unsigned)(sh.nsplit * a.rows));
  if (out_bf16)
    launch_split<false>(a, dense, swa8 != nullptr, grid, stream);
  else
    launch_split<true>(a, dense, swa8 != nullptr, grid, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || sh.nsplit == 1) return e;
  const int64_t n_items = (int64_t)c.B * Q * H * (kD / 8);
  // lanes per merged item: the splits spread over 1, 2 or 4 lanes
  const int lanes = sh.nsplit > 16 ? 4 : (sh.nsplit > 8 ? 2 : 1);
  const int wg_per_row = (H * (kD / 8) * lanes + kMergeThreads - 1) / kMergeThreads;
  const unsigned nb = a.xcd ? (unsigned)(8 * ((a.rows + 7) / 8) * wg_per_row)
                            : (unsigned)((n_items * lanes + kMergeThreads - 1) / kMergeThreads);
#define CSA_MERGE(BF, T)                                                                                       \
  attn_merge_kernel<BF, 8, T><<<nb, kMergeThreads, 0, stream>>>(a.ws_o, a.ws_ml, sh.nsplit, H, n_items, out, lse, \
                                                                a.rows, a.xcd, wg_per_row)
  if (lanes == 4) {
    if (out_bf16) CSA_MERGE(true, 4); else CSA_MERGE(false, 4);
  } else if (lanes == 2) {
    if (out_bf16) CSA_MERGE(true, 2); else CSA_MERGE(false, 2);
  } else {
    if (out_bf16) CSA_MERGE(true, 1); else CSA_MERGE(false, 1);
  }
#undef CSA_MERGE
  return hipGetLastError();
}

}  // namespace csa
