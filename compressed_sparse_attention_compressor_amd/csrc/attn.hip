// Attention over compressed entries plus the sliding window.
//
// [V4] "ハイブリッド注意：CSAとHCA": Fig. 3 (CSA: the query attends to its
// selected compressed blocks, and a sliding-window branch covers the
// recent raw tokens) and Fig. 4 (HCA: every compressed block, the same
// window).  One softmax runs over the union of the two key sets; the key
// and the value are the same decoded 576-channel row.
//
// Work split: one workgroup per (query, key-range split), one wave per 16
// query heads (heads are the MFMA M dimension, so every key is decoded once
// per workgroup and shared by all heads).  Per chunk of 32 key slots:
//   1. the slot list is resolved (selected entry, window row, or nothing);
//   2. the workgroup decodes the 32 rows into a key-major bf16 LDS tile
//      (E2M1 x E8M0 -> bf16 is exact; gfx950's v_cvt_scalef32_pk_bf16_fp4
//      converts two codes per instruction); when a chunk's loads fit one
//      register batch, the next chunk's raw bytes are fetched while the
//      current chunk is computed (the tile is double buffered);
//   3. S = Q K^T on v_mfma_f32_16x16x32_bf16 (lane: key l%16, heads
//      4(l/16)..+3), online softmax in the log2 domain;
//   4. P goes through a small per-wave LDS tile to become the A operand of
//      O += P V; the V operand (keys along K) is read transposed from the
//      same key-major tile with ds_read_b64_tr_b16, so no second copy of
//      the keys is written.  With fp32 outputs P is split into two bf16
//      parts (hi + lo) so that the probabilities keep ~16 bits.
// Splits write unnormalised (O, max, sum) partials that a merge kernel
// combines; a single split writes the normalised output directly.
#include "csa_device.hpp"
#include "csa_internal.hpp"

namespace csa {

constexpr int kKC = 32;           // key slots per chunk
constexpr int kKRow = kD + 8;     // key-major LDS row (bf16 elements)
constexpr int kPRow = kKC + 8;
constexpr int kNT = kD / 16;      // 36 channel tiles of 16
constexpr int kHalfD = kD / 2;    // channels per wave of a wave pair
constexpr int kHalfNT = kNT / 2;

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

// Raw bytes of one decode task: 16 channels of one key.
struct RawTask {
  uint4 a, b;       // bf16 rows: 32 bytes; MXFP4: a.x, a.y hold 16 codes
  uint32_t meta;    // kind (0 nothing, 1 MXFP4, 2 bf16) | E8M0 scale byte << 8
};

constexpr int kSegs = kD / 16;          // 36 tasks of 16 channels per key
constexpr int kChunkTasks = kKC * kSegs;

// Branch-free: three unconditional loads from clamped addresses (codes,
// scale byte, 32 bf16 bytes) with a known-valid stand-in address for the
// parts a task does not use; loads inside per-lane branches would make the
// compiler wait for each one before issuing the next.
__device__ __forceinline__ void load_task(const AttnArgs &a, int b, int src, int seg, const uint8_t *dummy,
                                          RawTask &t) {
  const int ch = seg * 16;
  const bool none = src < 0;
  const bool win = !none && (src & 0x40000000);
  const bool ent = !none && !win;
  const bool fp4 = ent && ch < kDNope;
  const int64_t row = (int64_t)b * a.N_cap + (ent ? src : 0);
  const uint8_t *pc = fp4 ? a.nope + row * kNopeBytes + ch / 2 : dummy;
  const uint8_t *ps = fp4 ? a.nscale + row * kNopeScales + ch / 32 : dummy;
  const uint8_t *pb = dummy;
  if (win) pb = reinterpret_cast<const uint8_t *>(a.swa + ((int64_t)b * a.S + (src & 0x3FFFFFFF)) * kD + ch);
  if (ent && !fp4) pb = reinterpret_cast<const uint8_t *>(a.rope + row * kDRope + (ch - kDNope));
  const uint2 c = *reinterpret_cast<const uint2 *>(pc);
  const uint32_t sc = *ps;
  const uint4 lo = reinterpret_cast<const uint4 *>(pb)[0];
  const uint4 hi = reinterpret_cast<const uint4 *>(pb)[1];
  t.a = fp4 ? uint4{c.x, c.y, 0u, 0u} : lo;
  t.b = hi;
  t.meta = none ? 0u : (fp4 ? (1u | (sc << 8)) : 2u);
}

// Writes the 16 decoded bf16 channels of a task (zeros for an empty slot).
__device__ __forceinline__ void store_task(uint16_t *row, const RawTask &t) {
  uint4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
  const uint32_t kind = t.meta & 0xFFu;
  if (kind == 2) {
    lo = t.a;
    hi = t.b;
  } else if (kind == 1) {
    // E2M1 x 2^(s-127) -> bf16 is exact (hardware conversion, two codes per byte)
    const float sc = e8m0_to_f32(t.meta >> 8);
#define CSA_CVT(src, sel) __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(src, sc, sel))
    lo = uint4{CSA_CVT(t.a.x, 0), CSA_CVT(t.a.x, 1), CSA_CVT(t.a.x, 2), CSA_CVT(t.a.x, 3)};
    hi = uint4{CSA_CVT(t.a.y, 0), CSA_CVT(t.a.y, 1), CSA_CVT(t.a.y, 2), CSA_CVT(t.a.y, 3)};
#undef CSA_CVT
  }
  reinterpret_cast<uint4 *>(row)[0] = lo;
  reinterpret_cast<uint4 *>(row)[1] = hi;
}

template <int HG, bool kSplitP, bool kDense>
__global__ __launch_bounds__(HG * 128) void attn_kernel(AttnArgs a) {
  // Key-major bf16 tiles of the chunk (double buffered); the P V operand is
  // read transposed from the same tile with ds_read_b64_tr_b16.
  __shared__ __attribute__((aligned(16))) uint16_t Kl[2][kKC * kKRow];
  __shared__ __attribute__((aligned(16))) uint16_t Pl[2 * HG][kSplitP ? 2 : 1][16 * kPRow];
  __shared__ __attribute__((aligned(16))) float Sx[2 * HG][2 * 4 * 64];
  __shared__ int src_s[2][kKC];

  constexpr int nthr = HG * 128;
  constexpr int kTasksPerThread = (kChunkTasks + nthr - 1) / nthr;
  constexpr int kBatch = kTasksPerThread < 5 ? kTasksPerThread : 5;
  constexpr bool kOneBatch = kBatch == kTasksPerThread;  // prefetch the next chunk in registers

  const int split = blockIdx.x % a.nsplit, q = blockIdx.x / a.nsplit, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, r = lane & 15;
  // wave pair (2hg, 2hg+1) shares heads 16hg..16hg+15; `half` picks channels [288 half, +288)
  const int hg = wave >> 1, half = wave & 1;
  const int cbase = half * kHalfD;
  const int64_t qrow = (int64_t)b * a.Q + q;
  const int p = a.q_pos[qrow];
  const int nE = min(a.n_entries[b], a.N_cap);
  const int V = p >= 0 ? max(0, min(nE, (p + 1) / a.m)) : 0;
  const int n_main = kDense ? V : a.k;
  int win_lo = 0, n_swa = 0, swa0 = 0;
  if (a.n_win > 0 && p >= 0) {
    swa0 = a.swa_pos0[b];
    win_lo = max(max(0, p - a.n_win + 1), swa0);
    const int win_hi = min(p, swa0 + a.S - 1);
    n_swa = max(0, win_hi - win_lo + 1);
  }
  const int n_slots = n_main + n_swa;
  const int s_begin = split * a.per_split;
  const int s_end = min(n_slots, s_begin + a.per_split);

  auto resolve = [&](int c0, int buf) {
    if (tid < kKC) {
      const int slot = c0 + tid;
      int src = -1;
      if (slot < s_end) {
        if (slot < n_main) {
          const int j = kDense ? slot : a.idx[qrow * a.k + slot];
          if (j >= 0 && j < V) src = j;
        } else {
          src = 0x40000000 | (win_lo + (slot - n_main) - swa0);
        }
      }
      src_s[buf][tid] = src;
    }
  };

  // a known-valid address for loads a task does not need: this query's row
  const uint8_t *dummy = reinterpret_cast<const uint8_t *>(a.q + qrow * a.H * kD);
  const int h0 = hg * 16;
  v8bf Qf[kHalfD / 32];
  {
    const uint16_t *qp = a.q + (qrow * a.H + h0 + r) * kD + cbase + 8 * g;
#pragma unroll
    for (int kk = 0; kk < kHalfD / 32; ++kk) Qf[kk] = *reinterpret_cast<const v8bf *>(qp + 32 * kk);
  }

  float m2[4], lsum[4];
  v4f O[kHalfNT];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m2[i] = -INFINITY;
    lsum[i] = 0.f;
  }
#pragma unroll
  for (int j = 0; j < kHalfNT; ++j) O[j] = v4f{0.f, 0.f, 0.f, 0.f};

  RawTask pre[kBatch];
  if (s_begin < s_end) {
    resolve(s_begin, 0);
    __syncthreads();
    if (kOneBatch) {
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int t = tid + u * nthr;
        if (t < kChunkTasks) load_task(a, b, src_s[0][t / kSegs], t % kSegs, dummy, pre[u]);
        else pre[u].meta = 0;
      }
    }
  }

  int buf = 0;
  for (int c0 = s_begin; c0 < s_end; c0 += kKC, buf ^= 1) {
    uint16_t *K = Kl[buf];
    // 1. decode this chunk into K
    if (kOneBatch) {
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int t = tid + u * nthr;
        if (t < kChunkTasks) store_task(K + (t / kSegs) * kKRow + (t % kSegs) * 16, pre[u]);
      }
    } else {
      for (int t0 = 0; t0 < kChunkTasks; t0 += kBatch * nthr) {
        RawTask tk[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int t = t0 + tid + u * nthr;
          if (t < kChunkTasks) load_task(a, b, src_s[buf][t / kSegs], t % kSegs, dummy, tk[u]);
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int t = t0 + tid + u * nthr;
          if (t < kChunkTasks) store_task(K + (t / kSegs) * kKRow + (t % kSegs) * 16, tk[u]);
        }
      }
    }
    if (c0 + kKC < s_end) resolve(c0 + kKC, buf ^ 1);
    __syncthreads();
    // key-slot flags of this chunk, read before the next barrier (the list of
    // this buffer is resolved again one iteration later)
    const bool kv0 = src_s[buf][r] >= 0, kv1 = src_s[buf][16 + r] >= 0;
    // 2. prefetch the next chunk's raw bytes while this one is computed
    if (kOneBatch && c0 + kKC < s_end) {
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int t = tid + u * nthr;
        if (t < kChunkTasks) load_task(a, b, src_s[buf ^ 1][t / kSegs], t % kSegs, dummy, pre[u]);
        else pre[u].meta = 0;
      }
    }

    // 3. half of S = Q K^T (this wave's 288 channels) for two tiles of 16 keys,
    //    then the partner's half through LDS
    v4f S2[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      v4f acc = {0.f, 0.f, 0.f, 0.f};
      const uint16_t *kp = K + (kt * 16 + r) * kKRow + cbase + 8 * g;
#pragma unroll
      for (int kk = 0; kk < kHalfD / 32; ++kk)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Qf[kk], *reinterpret_cast<const v8bf *>(kp + 32 * kk), acc, 0,
                                                      0, 0);
      S2[kt] = acc;
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) Sx[wave][(kt * 4 + i) * 64 + lane] = S2[kt][i];
    __syncthreads();
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // a fixed order of the two halves, so both waves of the pair agree bit for bit
        const float mine = S2[kt][i], other = Sx[wave ^ 1][(kt * 4 + i) * 64 + lane];
        S2[kt][i] = half == 0 ? mine + other : other + mine;
      }

    float alpha[4], p0[4], p1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x0 = kv0 ? S2[0][i] * a.scale_log2 : -INFINITY;
      const float x1 = kv1 ? S2[1][i] * a.scale_log2 : -INFINITY;
      const float tmax = row16_max(fmaxf(x0, x1));
      const float mn = fmaxf(m2[i], tmax);
      if (mn == -INFINITY) {
        alpha[i] = 1.f;
        p0[i] = p1[i] = 0.f;
      } else {
        alpha[i] = exp2f(m2[i] - mn);
        p0[i] = exp2f(x0 - mn);
        p1[i] = exp2f(x1 - mn);
      }
      lsum[i] = lsum[i] * alpha[i] + row16_sum(p0[i] + p1[i]);
      m2[i] = mn;
    }
#pragma unroll
    for (int j = 0; j < kHalfNT; ++j) {
#pragma unroll
      for (int i = 0; i < 4; ++i) O[j][i] *= alpha[i];
    }
    // 4. P (bf16, or hi + lo) through this wave's LDS tile into the A layout
    //    (LDS operations of one wave complete in order)
    uint16_t *pw = &Pl[wave][0][0];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t hi0 = f32_to_bf16(p0[i]), hi1 = f32_to_bf16(p1[i]);
      pw[(4 * g + i) * kPRow + r] = (uint16_t)hi0;
      pw[(4 * g + i) * kPRow + 16 + r] = (uint16_t)hi1;
      if (kSplitP) {
        uint16_t *pl = &Pl[wave][kSplitP ? 1 : 0][0];
        pl[(4 * g + i) * kPRow + r] = (uint16_t)f32_to_bf16(p0[i] - bf16_to_f32(hi0));
        pl[(4 * g + i) * kPRow + 16 + r] = (uint16_t)f32_to_bf16(p1[i] - bf16_to_f32(hi1));
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const v8bf Pa = *reinterpret_cast<const v8bf *>(&Pl[wave][0][r * kPRow + 8 * g]);
    v8bf Pb;
    if (kSplitP) Pb = *reinterpret_cast<const v8bf *>(&Pl[wave][kSplitP ? 1 : 0][r * kPRow + 8 * g]);
    // 5. O += P V for this wave's channels; lane (g, r) needs V[keys 8g..8g+7]
    //    [channel c + r]: two transposed 4x16 reads of the key-major tile.
    typedef __attribute__((address_space(3))) v4s lds_v4s;
    const uint16_t *vb = K + (8 * g + (r >> 2)) * kKRow + cbase + 4 * (r & 3);
#pragma unroll
    for (int j = 0; j < kHalfNT; ++j) {
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(vb + 16 * j));
      const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(vb + 4 * kKRow + 16 * j));
      const v8s both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      const v8bf Bv = __builtin_bit_cast(v8bf, both);
      O[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Pa, Bv, O[j], 0, 0, 0);
      if (kSplitP) O[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Pb, Bv, O[j], 0, 0, 0);
    }
    // The next iteration writes the other K buffer and Sx only after its own
    // barrier; the K buffer read here is rewritten two iterations later.
  }

  if (a.nsplit == 1) {
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
      float *o = a.ws_o + pr * kD + cbase;
#pragma unroll
      for (int j = 0; j < kHalfNT; ++j) o[16 * j + r] = O[j][i];
      if (r == 0 && half == 0) {
        a.ws_ml[pr * 2 + 0] = m2[i];
        a.ws_ml[pr * 2 + 1] = lsum[i];
      }
    }
  }
}

// Combines the splits of one (query, head): weights 2^(m_s - M).
__global__ __launch_bounds__(64) void attn_merge_kernel(const float *__restrict__ ws_o, const float *__restrict__ ws_ml,
                                                        int nsplit, int H, int out_bf16, void *out, float *lse) {
  const int64_t qh = blockIdx.x;           // qrow * H + h
  const int64_t qrow = qh / H, hh = qh % H;
  const int tid = threadIdx.x;
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, ws_ml[((qrow * nsplit + s) * H + hh) * 2]);
  float acc[kD / 64];
#pragma unroll
  for (int c = 0; c < kD / 64; ++c) acc[c] = 0.f;
  float L = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < nsplit; ++s) {
      const int64_t pr = (qrow * nsplit + s) * H + hh;
      const float ms = ws_ml[pr * 2];
      if (ms == -INFINITY) continue;
      const float wgt = exp2f(ms - M);
      L += wgt * ws_ml[pr * 2 + 1];
      const float *o = ws_o + pr * kD;
#pragma unroll
      for (int c = 0; c < kD / 64; ++c) acc[c] = fmaf(wgt, o[tid + 64 * c], acc[c]);
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  if (out_bf16) {
    uint16_t *o = reinterpret_cast<uint16_t *>(out) + qh * kD;
#pragma unroll
    for (int c = 0; c < kD / 64; ++c) o[tid + 64 * c] = (uint16_t)f32_to_bf16(acc[c] * inv);
  } else {
    float *o = reinterpret_cast<float *>(out) + qh * kD;
#pragma unroll
    for (int c = 0; c < kD / 64; ++c) o[tid + 64 * c] = acc[c] * inv;
  }
  if (lse && tid == 0) lse[qh] = L > 0.f ? (M + log2f(L)) * 0.69314718055994531f : -INFINITY;
}

AttnShape attn_shape(int B, int Q, int n_slots_max) {
  const int chunks = n_slots_max > 0 ? (n_slots_max + kKC - 1) / kKC : 1;
  const int64_t rows = (int64_t)B * Q;
  int want = (int)(rows >= 256 ? 1 : (256 + rows - 1) / rows);
  want = want < chunks ? want : chunks;
  const int per_chunks = (chunks + want - 1) / want;
  const int nsplit = (chunks + per_chunks - 1) / per_chunks;
  return AttnShape{nsplit, per_chunks * kKC};
}

size_t attn_workspace_bytes(int B, int Q, int H, int n_slots_max) {
  const AttnShape s = attn_shape(B, Q, n_slots_max);
  if (s.nsplit <= 1) return 0;
  return (size_t)B * Q * s.nsplit * H * (kD + 2) * sizeof(float);
}

template <int HG, bool kSplitP>
static void launch_hg(const AttnArgs &a, bool dense, dim3 grid, hipStream_t stream) {
  if (dense)
    attn_kernel<HG, kSplitP, true><<<grid, HG * 128, 0, stream>>>(a);
  else
    attn_kernel<HG, kSplitP, false><<<grid, HG * 128, 0, stream>>>(a);
}

template <bool kSplitP>
static void launch_split(const AttnArgs &a, bool dense, dim3 grid, hipStream_t stream) {
  switch (a.H / 16) {
    case 1: launch_hg<1, kSplitP>(a, dense, grid, stream); break;
    case 2: launch_hg<2, kSplitP>(a, dense, grid, stream); break;
    case 4: launch_hg<4, kSplitP>(a, dense, grid, stream); break;
    default: launch_hg<8, kSplitP>(a, dense, grid, stream); break;
  }
}

hipError_t launch_attention(const CacheView &c, const uint16_t *q, int H, const int32_t *q_pos, int Q,
                            const int32_t *idx, int k, bool dense, const uint16_t *swa, const int32_t *swa_pos0,
                            int S, int n_win, float scale, bool out_bf16, void *out, float *lse, void *ws,
                            hipStream_t stream) {
  const int n_slots_max = (dense ? c.N_cap : k) + n_win;
  const AttnShape sh = attn_shape(c.B, Q, n_slots_max);
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
    launch_split<false>(a, dense, grid, stream);
  else
    launch_split<true>(a, dense, grid, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || sh.nsplit == 1) return e;
  attn_merge_kernel<<<(unsigned)((int64_t)c.B * Q * H), 64, 0, stream>>>(a.ws_o, a.ws_ml, sh.nsplit, H, a.out_bf16,
                                                                        out, lse);
  return hipGetLastError();
}

}  // namespace csa
