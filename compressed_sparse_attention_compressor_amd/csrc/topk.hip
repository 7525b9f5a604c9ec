// Per-query top-k of the indexer scores ([V4] "ハイブリッド注意：CSAとHCA",
// CSA paragraph: the indexer picks the top-k compressed blocks of each
// query; [V4.1] "推論カーネル" names a dedicated TopK kernel).  All paths
// select exactly, on order-preserving uint32 keys, ties to the lower entry;
// topk_plan picks one per launch shape:
//   * rows of at most 32,768 scores (and candidate lists): one 512-thread
//     workgroup per row with the keys in registers (topk_select.hpp);
//   * rows with few siblings (B*Q < 256) longer than 4,096: slices whose own
//     top-k candidates a second register-resident launch reduces;
//   * few rows (B*Q < 256) of at least 65,536 scores: a radix selection
//     spread over many workgroups (launch_radix, further below);
//   * many rows longer than 32,768: the tiled LDS radix select below.
//
// Tiled LDS radix select, one 1024-thread workgroup per query:
//   * the scores of a tile (up to kTile of them) sit in LDS as keys, each
//     thread owning a contiguous run, padded one word per 32 so that the
//     strided runs do not collide on LDS banks;
//   * four passes of 8 bits, most significant first, build per-wave
//     histograms of the elements still matching the chosen prefix and fix
//     one digit of the k-th largest key T;
//   * a last pass keeps every key > T plus the first (by entry index)
//     elements equal to T, and writes them in ascending order through two
//     block-wide prefix sums.
// Rows longer than kTile are processed tile by tile in every pass.
#include "csa_device.hpp"
#include "csa_internal.hpp"
#include "topk_select.hpp"

namespace csa {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kTile = 32768;
constexpr int kTilePadded = kTile + kTile / 32;

__device__ __forceinline__ int lds_pos(int i) { return i + (i >> 5); }

// Exclusive prefix of the kW per-wave totals in sh[0..kW) (in place), total
// in sh[kW]; done by the first wave with shuffles (one LDS read per lane).
template <int kW>
__device__ __forceinline__ void scan_wave_totals(int *sh) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int v = lane < kW ? sh[lane] : 0;
    int inc = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(inc, o);
      if (lane >= o) inc += t;
    }
    if (lane < kW) sh[lane] = inc - v;
    if (lane == kW - 1) sh[kW] = inc;
  }
}

// Exclusive prefix sum over the NT threads in thread order; also returns the total.
template <int NT = kTopkThreads>
__device__ __forceinline__ int block_excl_scan(int v, int *sh, int &total) {
  constexpr int kW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(inc, o);
    if (lane >= o) inc += t;
  }
  if (lane == 63) sh[wave] = inc;
  __syncthreads();
  scan_wave_totals<kW>(sh);
  __syncthreads();
  const int res = sh[wave] + inc - v;
  total = sh[kW];
  __syncthreads();
  return res;
}

__global__ __launch_bounds__(kTopkThreads) void topk_tiled_kernel(const float *__restrict__ scores, int Ns,
                                                             const int32_t *__restrict__ n_entries, int N_cap, int m,
                                                             const int32_t *__restrict__ q_pos, int Q,
                                                             const int32_t *__restrict__ cand, int C, int k,
                                                             int32_t *__restrict__ idx_out,
                                                             float *__restrict__ score_out) {
  __shared__ uint32_t keys[kTilePadded];
  __shared__ int hist[kTopkWaves][256];
  __shared__ int scan_sh[kTopkWaves + 1];
  __shared__ uint32_t sel_prefix;
  __shared__ int sel_need;

  const int q = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = (int64_t)b * Q + q;
  const float *src = scores + row * Ns;
  int n;
  if (cand) {
    n = C;
  } else {
    const int nE = min(n_entries[b], N_cap);
    n = max(0, min(nE, (q_pos[row] + 1) / m));
  }
  const int ntiles = (n + kTile - 1) / kTile;

  auto load_tile = [&](int t0) {
    const int nt = min(kTile, n - t0);
    for (int i = tid; i < nt; i += kTopkThreads) {
      const uint32_t u = __float_as_uint(src[t0 + i]);
      keys[lds_pos(i)] = (u == kNoScoreBits) ? 0u : score_key(__uint_as_float(u));
    }
  };

  // Valid elements (candidate slots may be empty; a full scan has none empty).
  int n_valid = n;
  if (cand) {
    int cnt = 0;
    for (int t0 = 0; t0 < n; t0 += kTile) {
      const int nt = min(kTile, n - t0);
      for (int i = tid; i < nt; i += kTopkThreads) cnt += __float_as_uint(src[t0 + i]) != kNoScoreBits;
    }
    int tot;
    block_excl_scan(cnt, scan_sh, tot);
    n_valid = tot;
  }
  const int k_eff = min(k, n_valid);

  uint32_t prefix = 0;
  int need = 0;  // elements equal to the threshold that are taken
  if (k_eff > 0 && k_eff < n_valid) {
    int k_rem = k_eff;
    if (ntiles == 1) {
      load_tile(0);
      __syncthreads();
    }
    for (int shift = 24; shift >= 0; shift -= 8) {
      const uint32_t hmask = shift == 24 ? 0u : (0xFFFFFFFFu << (shift + 8));
      for (int i = tid; i < kTopkWaves * 256; i += kTopkThreads) (&hist[0][0])[i] = 0;
      __syncthreads();
      for (int t0 = 0; t0 < n; t0 += kTile) {
        if (ntiles > 1) {
          load_tile(t0);
          __syncthreads();
        }
        const int nt = min(kTile, n - t0);
        const int per = (nt + kTopkThreads - 1) / kTopkThreads;
        const int i0 = tid * per, i1 = min(nt, i0 + per);
        for (int i = i0; i < i1; ++i) {
          const uint32_t u = keys[lds_pos(i)];
          if ((u & hmask) == prefix) atomicAdd(&hist[wave][(u >> shift) & 255u], 1);
        }
        __syncthreads();
      }
      // Digit holding the k_rem-th largest remaining element.
      if (wave == 0) {
        int c[4];
        int tsum = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = 255 - (lane * 4 + j);   // lane 0 holds the top digits
          int s = 0;
          for (int w = 0; w < kTopkWaves; ++w) s += hist[w][d];
          c[j] = s;
          tsum += s;
        }
        int inc = tsum;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int t = __shfl_up(inc, o);
          if (lane >= o) inc += t;
        }
        int above = inc - tsum;  // elements in higher digits than this lane's
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (above < k_rem && k_rem <= above + c[j]) {
            sel_prefix = prefix | ((uint32_t)(255 - (lane * 4 + j)) << shift);
            sel_need = k_rem - above;
          }
          above += c[j];
        }
      }
      __syncthreads();
      prefix = sel_prefix;
      k_rem = sel_need;
      __syncthreads();
    }
    need = k_rem;
  } else if (k_eff > 0) {
    prefix = 0;  // take every valid element: keys > 0
    need = 0;
  }

  // Selection, in entry order.
  int32_t *out_i = idx_out + row * k;
  float *out_s = score_out ? score_out + row * k : nullptr;
  int out_base = 0, eq_base = 0;
  if (k_eff > 0) {
    for (int t0 = 0; t0 < n; t0 += kTile) {
      if (ntiles > 1 || !(k_eff < n_valid)) {
        __syncthreads();
        load_tile(t0);
        __syncthreads();
      }
      const int nt = min(kTile, n - t0);
      const int per = (nt + kTopkThreads - 1) / kTopkThreads;
      const int i0 = tid * per, i1 = min(nt, i0 + per);
      int gt = 0, eq = 0;
      for (int i = i0; i < i1; ++i) {
        const uint32_t u = keys[lds_pos(i)];
        gt += u > prefix;
        eq += (u == prefix) && need > 0;
      }
      int eq_tot;
      const int eq_before = eq_base + block_excl_scan(eq, scan_sh, eq_tot);
      const int take_eq = max(0, min(eq, need - eq_before));
      int sel_tot;
      int off = out_base + block_excl_scan(gt + take_eq, scan_sh, sel_tot);
      int eq_seen = 0;
      for (int i = i0; i < i1; ++i) {
        const uint32_t u = keys[lds_pos(i)];
        bool take = u > prefix;
        if (!take && u == prefix && need > 0) {
          take = eq_seen < take_eq;
          ++eq_seen;
        }
        if (take && off < k_eff) {
          const int e = cand ? cand[row * C + t0 + i] : t0 + i;
          out_i[off] = e;
          if (out_s) out_s[off] = key_score(u);
          ++off;
        }
      }
      out_base += sel_tot;
      eq_base += eq_tot;
    }
  }
  for (int j = k_eff + tid; j < k; j += kTopkThreads) {
    out_i[j] = -1;
    if (out_s) out_s[j] = __uint_as_float(kNoScoreBits);  // a NaN
  }
}


// Rows (or row slices) of at most kPer*kRegThreads scores.  Element
// i = v*(4*kRegThreads) + 4*tid + u (u < 4) is held by thread tid, so every
// load instruction is fully coalesced.
// With nsl > 1 the workgroup handles slice blockIdx.x % nsl (elements
// [slice*S, slice*S + S) of the row) and writes that slice's own top-k to
// row (row*nsl + slice) of the outputs, empty slots marked -1 and
// kNoScoreBits; a second launch in candidate mode (kCand) then selects
// among them.
template <int kPer, bool kCand>
__global__ __launch_bounds__(kRegThreads) void topk_reg_kernel(const float *__restrict__ scores, int Ns,
                                                                 const int32_t *__restrict__ n_entries, int N_cap,
                                                                 int m, const int32_t *__restrict__ q_pos, int Q,
                                                                 const int32_t *__restrict__ cand, int C, int k,
                                                                 int32_t *__restrict__ idx_out,
                                                                 float *__restrict__ score_out, int nsl, int S) {
  constexpr int NT = kRegThreads;
  constexpr int kV = kPer / 4;              // slices of 4*NT elements
  constexpr int kSlice = NT * 4;
  constexpr bool kPrefetch = kCand && kPer <= 32;  // candidate ids loaded with the scores

  const int q = blockIdx.x / nsl, sl = blockIdx.x % nsl, b = blockIdx.y;
  const int tid = threadIdx.x;
  const int64_t row = (int64_t)b * Q + q;
  const int off = sl * S;                   // first element of this slice
  const int len = nsl > 1 ? min(S, Ns - off) : Ns;
  const float *src = scores + row * Ns + off;
  const int32_t *csrc = kCand ? cand + row * C : nullptr;

  // Unconditional loads from clamped addresses first (loads inside per-lane
  // branches are serialised by the compiler); the row length is applied after.
  uint32_t key[kPer];  // key[4v + u] (raw score bits until converted); 0 = not a candidate
  int32_t cid[kPrefetch ? kPer : 1];
  auto to_key = [](uint32_t bits) { return bits != kNoScoreBits ? score_key(__uint_as_float(bits)) : 0u; };
  if (len >= 4 && ((Ns | off | len) & 3) == 0) {
#pragma unroll
    for (int v = 0; v < kV; ++v) {
      const int i0 = min(v * kSlice + 4 * tid, len - 4);
      const uint4 t4 = *reinterpret_cast<const uint4 *>(src + i0);
      key[4 * v + 0] = t4.x;
      key[4 * v + 1] = t4.y;
      key[4 * v + 2] = t4.z;
      key[4 * v + 3] = t4.w;
      if constexpr (kPrefetch) {
        const int4 c4 = *reinterpret_cast<const int4 *>(csrc + i0);
        cid[4 * v + 0] = c4.x;
        cid[4 * v + 1] = c4.y;
        cid[4 * v + 2] = c4.z;
        cid[4 * v + 3] = c4.w;
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = min((j >> 2) * kSlice + 4 * tid + (j & 3), len - 1);
      key[j] = len > 0 ? __float_as_uint(src[i]) : kNoScoreBits;
      if constexpr (kPrefetch) cid[j] = len > 0 ? csrc[i] : -1;
    }
  }
  int n;
  if (kCand) {
    n = C;
  } else {
    const int nE = min(n_entries[b], N_cap);
    n = max(0, min(nE, (q_pos[row] + 1) / m));
  }
  n = __builtin_amdgcn_readfirstlane(max(0, min(n - off, len)));  // elements of this slice
  // keys from the raw bits, per slice of 4*NT elements: slices past n are
  // empty (about half of a causal prefill row), slices before it need no
  // per-element test
#pragma unroll
  for (int v = 0; v < kV; ++v) {
    if (v * kSlice >= n) {
#pragma unroll
      for (int u = 0; u < 4; ++u) key[4 * v + u] = 0u;
    } else if ((v + 1) * kSlice <= n) {
#pragma unroll
      for (int u = 0; u < 4; ++u) key[4 * v + u] = to_key(key[4 * v + u]);
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        key[4 * v + u] = v * kSlice + 4 * tid + u < n ? to_key(key[4 * v + u]) : 0u;
    }
  }

  const int64_t orow = row * nsl + sl;
  // every slot at or past n is empty (in a causal prefill about half of a
  // row): the selection skips the 4*kRegThreads-element slices beyond it
  select_keys<kPer, kPrefetch>(key, cid, k, idx_out + orow * k, score_out ? score_out + orow * k : nullptr,
                               [&](int i) { return kCand ? csrc[i] : off + i; }, n);
}

// ---------------------------------------------------------------------------
// Rows with a histogram hint (decode: few rows of at most 32,768 scores).
// The indexer launch that wrote a row's scores also counted them by the top
// 11 bits of their order-preserving keys (kHintBins words per row).  Two
// launches, both spread over the whole GPU where the bytes are:
//   1. compaction: one workgroup per slice of 4,096 scores reads the row's
//      counts, finds the bin holding the k-th largest key (one block scan,
//      the same in every slice) and writes the slice's keys in that bin or
//      above, in entry order, with its counts above / inside the bin;
//   2. final: one workgroup per row checks the counts of all slices against
//      the hint, settles the exact threshold among the candidates of the
//      bin (a histogram of the next 11 bits, then a gather-and-rank of at
//      most 64 keys or one more radix pass) and places the selection.  It
//      leaves the row's hint zero for the next indexer launch.
// A hint that does not match the scores (a workspace that an earlier call
// did not leave zero), or a threshold bin with more candidates than one
// workgroup holds, only costs time: the final launch then selects from the
// whole row.
constexpr int kHintSlice = 4096;                      // scores per compaction workgroup
constexpr int kHintPer = kHintSlice / kRegThreads;    // 8 contiguous scores per thread
constexpr int kHintCand = 8;                          // candidates per thread in the final launch
constexpr int kHintSlot = kRegThreads * kHintCand / (kRegN / kHintSlice);  // 512 candidate slots read per slice

struct HintArgs {
  const float *scores;
  int Ns;
  const int32_t *n_entries;
  int N_cap, m;
  const int32_t *q_pos;
  int Q, k, nsl;
  uint32_t *hint;       // [rows][kHintBins]
  int32_t *cand_i;      // [rows][nsl * kHintSlice] entry of each candidate
  uint32_t *cand_k;     // [rows][nsl * kHintSlice] its key
  int32_t *slice_info;  // [rows][nsl][3]: keys above the bin, keys in it, visible keys
  int32_t *row_info;    // [rows][4]: bin, keys above it (hint), keys in it (hint), hint total
  int32_t *idx_out;
  float *score_out;
};

__device__ __forceinline__ int hint_visible(const HintArgs &a, int b, int64_t row) {
  const int nE = min(a.n_entries[b], a.N_cap);
  return max(0, min(min(nE, (a.q_pos[row] + 1) / a.m), a.Ns));
}

// The hint's block scan: thread t holds bins 2047 - 4t .. 2044 - 4t.  Returns
// the hint total and, when 0 < min(k, total) < total, the bin holding the
// min(k, total)-th largest key, the count above it and inside it (bin -1:
// every counted key is taken).  Two barriers; sh holds NT/64 + 3 ints.
__device__ __forceinline__ void hint_bin(uint4 hc, int k, int *sh, int &bin, int &above, int &inside, int &all) {
  constexpr int kW = kRegThreads / 64;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c[4] = {(int)hc.w, (int)hc.z, (int)hc.y, (int)hc.x};  // descending bins
  const int tot = c[0] + c[1] + c[2] + c[3];
  const int inc = wave_incl_scan(tot);
  if (lane == 63) sh[wave] = inc;
  __syncthreads();
  int base = 0, sum = 0;
#pragma unroll
  for (int w = 0; w < kW; ++w) {
    const int t = sh[w];
    base += w < wave ? t : 0;
    sum += t;
  }
  all = __builtin_amdgcn_readfirstlane(sum);
  const int ke = min(k, all);
  if (tid == 0) sh[kW] = -1;
  __syncthreads();
  int ab = base + inc - tot;
  if (ke > 0 && ke < all) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (ab < ke && ke <= ab + c[j]) {
        sh[kW] = kHintBins - 1 - 4 * tid - j;
        sh[kW + 1] = ab;
        sh[kW + 2] = c[j];
      }
      ab += c[j];
    }
  }
  __syncthreads();
  bin = __builtin_amdgcn_readfirstlane(sh[kW]);
  above = bin >= 0 ? __builtin_amdgcn_readfirstlane(sh[kW + 1]) : 0;
  inside = bin >= 0 ? __builtin_amdgcn_readfirstlane(sh[kW + 2]) : 0;
}

__global__ __launch_bounds__(kRegThreads) void topk_hint_compact_kernel(HintArgs a) {
  constexpr int kW = kRegThreads / 64;
  __shared__ int sh[kW + 3];
  __shared__ int wsum[3][kW];
  const int q = blockIdx.x / a.nsl, sl = blockIdx.x % a.nsl, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t row = (int64_t)b * a.Q + q;
  const uint4 hc = *reinterpret_cast<const uint4 *>(a.hint + row * kHintBins + (kHintBins - 4 - 4 * tid));
  const int off = sl * kHintSlice;
  const int e0 = off + kHintPer * tid;                     // this thread's first element
  const float *src = a.scores + row * a.Ns;
  uint32_t key[kHintPer];
  auto to_key = [](float x) { return __float_as_uint(x) != kNoScoreBits ? score_key(x) : 0u; };
  if ((a.Ns & 3) == 0) {
#pragma unroll
    for (int v = 0; v < kHintPer / 4; ++v) {
      const float4 t4 = *reinterpret_cast<const float4 *>(src + min(e0 + 4 * v, a.Ns - 4));
      key[4 * v + 0] = to_key(t4.x);
      key[4 * v + 1] = to_key(t4.y);
      key[4 * v + 2] = to_key(t4.z);
      key[4 * v + 3] = to_key(t4.w);
    }
  } else {
#pragma unroll
    for (int j = 0; j < kHintPer; ++j) key[j] = to_key(src[min(e0 + j, a.Ns - 1)]);
  }
  const int n = hint_visible(a, b, row);
#pragma unroll
  for (int j = 0; j < kHintPer; ++j)
    if (e0 + j >= n) key[j] = 0u;

  int bin, above, inside, all;
  hint_bin(hc, a.k, sh, bin, above, inside, all);
  // candidates: every visible key in the bin or above (all of them when the
  // hint takes every key)
  const uint32_t lo = bin >= 0 ? (uint32_t)bin : 0u;
  int ng = 0, ne = 0, nv = 0;
#pragma unroll
  for (int j = 0; j < kHintPer; ++j) {
    const uint32_t kk = key[j];
    const uint32_t d = kk >> kHintShift;
    nv += kk != 0u;
    ng += kk != 0u && d > lo;
    ne += kk != 0u && d == lo;
  }
  const int mine = ng + ne;
  const int inc = wave_incl_scan(mine);
  if (lane == 63) wsum[0][wave] = inc;
  const int wg = wave_sum(ng), we = wave_sum(ne), wv = wave_sum(nv);
  if (lane == 0) {
    wsum[1][wave] = wg;
    wsum[2][wave] = we * 65536 + wv;  // both below 65,536 per wave
  }
  __syncthreads();
  int base = 0, sg = 0, se = 0, sv = 0;
#pragma unroll
  for (int w = 0; w < kW; ++w) {
    base += w < wave ? wsum[0][w] : 0;
    sg += wsum[1][w];
    se += wsum[2][w] >> 16;
    sv += wsum[2][w] & 0xFFFF;
  }
  int pos = base + inc - mine;
  const int64_t cb = row * (int64_t)a.nsl * kHintSlice + off;
#pragma unroll
  for (int j = 0; j < kHintPer; ++j) {
    const uint32_t kk = key[j];
    if (kk != 0u && (kk >> kHintShift) >= lo) {
      a.cand_i[cb + pos] = e0 + j;
      a.cand_k[cb + pos] = kk;
      ++pos;
    }
  }
  if (tid == 0) {
    int32_t *si = a.slice_info + (row * a.nsl + sl) * 3;
    si[0] = sg;
    si[1] = se;
    si[2] = sv;
    if (sl == 0) {
      int32_t *ri = a.row_info + row * 4;
      ri[0] = bin;
      ri[1] = above;
      ri[2] = inside;
      ri[3] = all;
    }
  }
}

__global__ __launch_bounds__(kRegThreads) void topk_hint_final_kernel(HintArgs a) {
  constexpr int NT = kRegThreads;
  constexpr int kW = NT / 64;
  constexpr int kFullPer = kRegN / NT;  // 64: the fallback holds a whole row
  constexpr int kMaxSl = kRegN / kHintSlice;
  __shared__ int hist[kW * kBins];      // also the placement's staging area
  __shared__ int sh[kW + 3];
  __shared__ int wred[3 * kW];
  __shared__ uint32_t bin_keys[64];
  __shared__ int cnt[2 * (kFullPer / 4) * kW];
  __shared__ int n_bin;
  constexpr int kStage = kW * kBins / 2;
  int (*hist2)[kBins] = reinterpret_cast<int (*)[kBins]>(hist);
  const int q = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t row = (int64_t)b * a.Q + q;
  int32_t *out_i = a.idx_out + row * a.k;
  float *out_s = a.score_out ? a.score_out + row * a.k : nullptr;

  // The candidates in entry order, loaded before their counts are known:
  // element i = v*(4*NT) + 4*tid + u is position i % kHintSlot of slice
  // i / kHintSlot (slots past a slice's count are masked below; a slice with
  // more than kHintSlot candidates sends the row to the fallback).
  uint32_t key[kHintCand];
  int32_t cid[kHintCand];
#pragma unroll
  for (int j = 0; j < kHintCand; ++j) {
    const int i = (j >> 2) * (4 * NT) + 4 * tid + (j & 3);
    const int s = min(i / kHintSlot, a.nsl - 1);
    const int64_t at = (row * a.nsl + s) * (int64_t)kHintSlice + (i % kHintSlot);
    key[j] = a.cand_k[at];
    cid[j] = a.cand_i[at];
  }
  // counts of every slice (uniform loads), checked against the hint
  const int32_t *ri = a.row_info + row * 4;
  const int bin = ri[0], above = ri[1], inside = ri[2], all = ri[3];
  int cnt_s[kMaxSl];
  int sg = 0, se = 0, sv = 0;
  bool big = false;
#pragma unroll
  for (int s = 0; s < kMaxSl; ++s) {
    const bool in = s < a.nsl;
    const int32_t *si = a.slice_info + (row * a.nsl + (in ? s : 0)) * 3;
    const int g = in ? si[0] : 0, e = in ? si[1] : 0, v = in ? si[2] : 0;
    sg += g;
    se += e;
    sv += v;
    cnt_s[s] = g + e;
    big = big || g + e > kHintSlot;
  }
  const int n_valid = sv;
  const int k_eff = min(a.k, n_valid);
  // the hint matches when its total is the row's visible count and, with a
  // threshold bin, the counts above and inside it are the scores' own
  const bool ok = all == n_valid && !big && (bin >= 0 ? (sg == above && se == inside) : true);
  if (tid < kHintBins / 4)  // the hint is left zero for the next indexer launch
    *reinterpret_cast<uint4 *>(a.hint + row * kHintBins + 4 * tid) = uint4{0u, 0u, 0u, 0u};
  if (ok) {
    // the slice of element i is the same in the whole wave: a 4*NT-element
    // step holds whole slices, and a slice spans kHintSlot/256 waves
    static_assert((4 * NT) % kHintSlot == 0 && kHintSlot % 256 == 0, "slices of whole waves");
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
#pragma unroll
    for (int j = 0; j < kHintCand; ++j) {
      const int i = (j >> 2) * (4 * NT) + 4 * tid + (j & 3);
      const int s = (j >> 2) * (4 * NT / kHintSlot) + wave / (kHintSlot / 256);  // i / kHintSlot
      int c = 0;
#pragma unroll
      for (int t = 0; t < kMaxSl; ++t) c = s == t ? cnt_s[t] : c;
      if (s >= a.nsl || i % kHintSlot >= c) {
        key[j] = 0u;
        cid[j] = -1;
      }
    }
    for (int i = tid; i < kBins; i += NT) hist[i] = 0;
    if (tid == 0) n_bin = 0;
    __syncthreads();  // the histogram is zero before any thread adds to it
    uint32_t thr = 1u;  // every candidate (all visible keys) when there is no bin
    int need = 0, n_eq = 0;
    if (bin >= 0) {
      // the next 11 bits of the keys in the bin
#pragma unroll
      for (int j = 0; j < kHintCand; ++j)
        if (key[j] != 0u && (key[j] >> kHintShift) == (uint32_t)bin) atomicAdd(&hist[(key[j] >> 10) & 0x7FFu], 1);
      __syncthreads();
      int k_rem = k_eff - above;
      int e2, ab, c2, tt;
      find_digit<NT>(hist2, 1, kBins, k_rem, sh, e2, ab, c2, tt);
      k_rem -= ab;
      const uint32_t p12 = ((uint32_t)bin << 11) | (uint32_t)e2;
      if (c2 <= 64) {
        // gather the bin's keys: a ballot per key, and on a non-empty one an
        // LDS atomic reserves its slots
#pragma unroll
        for (int j = 0; j < kHintCand; ++j) {
          const bool in = key[j] != 0u && (key[j] >> 10) == p12;
          const uint64_t mk = __builtin_amdgcn_ballot_w64(in);
          if (mk) {
            int pos = 0;
            if (lane == 0) pos = atomicAdd(&n_bin, (int)__popcll(mk));
            pos = __builtin_amdgcn_readfirstlane(pos);
            if (in) bin_keys[lanes_below(mk, pos)] = key[j];
          }
        }
        __syncthreads();
        rank_gathered<NT>(bin_keys, c2, k_rem, sh, hist, thr, need, n_eq);  // the histogram is free now
      } else {
        // a crowded bin: one more pass over bits 9..0
        __syncthreads();
        for (int i = tid; i < kBins; i += NT) hist[i] = 0;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kHintCand; ++j)
          if (key[j] != 0u && (key[j] >> 10) == p12) atomicAdd(&hist[key[j] & 0x3FFu], 1);
        __syncthreads();
        int e3;
        find_digit<NT>(hist2, 1, 1024, k_rem, sh, e3, ab, n_eq, tt);  // every key equal to thr lies in bin e3
        k_rem -= ab;
        thr = (p12 << 10) | (uint32_t)e3;
        need = k_rem;
      }
    }
    place_selected<NT, kHintCand, true, kStage>(key, cid, thr, need, n_eq, k_eff, a.k, cnt, hist,
                                                reinterpret_cast<float *>(hist + kStage), out_i, out_s,
                                                [](int i) { return i; });
    return;
  }
  // the hint did not match: select from the whole row
  const float *src = a.scores + row * a.Ns;
  const int n = hint_visible(a, b, row);
  uint32_t fkey[kFullPer];
  auto to_key = [](float x) { return __float_as_uint(x) != kNoScoreBits ? score_key(x) : 0u; };
#pragma unroll
  for (int j = 0; j < kFullPer; ++j) {
    const int i = (j >> 2) * (4 * NT) + 4 * tid + (j & 3);
    const float x = src[min(i, max(a.Ns - 1, 0))];
    fkey[j] = i < n ? to_key(x) : 0u;
  }
  int ke, need, n_eq;
  uint32_t thr;
  linear_threshold<NT, kFullPer>(fkey, a.k, hist, sh, wred, bin_keys, &n_bin, ke, thr, need, n_eq);
  const int32_t no_cid[1] = {0};
  place_selected<NT, kFullPer, false, kStage>(fkey, no_cid, thr, need, n_eq, ke, a.k, cnt, hist,
                                              reinterpret_cast<float *>(hist + kStage), out_i, out_s,
                                              [](int i) { return i; });
}

// ---------------------------------------------------------------------------
// Few, long rows (B*Q < 256 rows of at least 65,536 scores): a radix
// selection spread over slices of 4,096 scores per workgroup, the digits of
// the order-preserving key (11, 11 and 10 bits) resolved one launch at a
// time through per-row histograms in global memory, so that every launch
// keeps the whole GPU busy however large k is (the slice-and-reduce path
// must pass k candidates per slice on, which for k = 2,048 barely shrinks
// the rows).  Launches: zero the histograms; digit-1 histogram; digit-2
// histogram of the keys in the threshold digit-1 bin; digit-3 likewise;
// per-slice counts of the keys above / equal to the threshold key T;
// placement in ascending entry order from the prefix of those counts.  Ties
// at T go to the lower entries: the first `need` keys equal to T are taken.
constexpr int kRxPer = 8;
constexpr int kRxSlice = kRegThreads * kRxPer;  // 4,096 scores per workgroup

struct RxArgs {
  const float *scores;
  int Ns;
  const int32_t *n_entries;
  int N_cap, m;
  const int32_t *q_pos;
  int Q, k, nsl;
  int *hist1;   // [rows][2048] digit 1 (key >> 21)
  int *hist2;   // [rows][2048] digit 2 ((key >> 10) & 2047) inside the digit-1 threshold bin
  int *hist3;   // [rows][1024] digit 3 (key & 1023) inside the digit-2 threshold bin
  int *counts;  // [rows][nsl][2]: keys > T, keys == T
  int *desc;    // [rows][4]: T, need, k_eff
  int32_t *idx_out;
  float *score_out;
};

// This workgroup's slice as keys (0 = not visible / no score); element
// i = v*(4*kRegThreads) + 4*tid + u is key[4v + u].
__device__ __forceinline__ void rx_load(const RxArgs &a, int64_t row, int b, int sl, uint32_t (&key)[kRxPer]) {
  constexpr int kSlice = kRegThreads * 4;
  const int tid = threadIdx.x;
  const int off = sl * kRxSlice;
  const int len = min(kRxSlice, a.Ns - off);
  const float *src = a.scores + row * a.Ns + off;
  if (len >= 4 && ((a.Ns | off | len) & 3) == 0) {
#pragma unroll
    for (int v = 0; v < kRxPer / 4; ++v) {
      const float4 t4 = *reinterpret_cast<const float4 *>(src + min(v * kSlice + 4 * tid, len - 4));
      const float t[4] = {t4.x, t4.y, t4.z, t4.w};
#pragma unroll
      for (int u = 0; u < 4; ++u)
        key[4 * v + u] = __float_as_uint(t[u]) != kNoScoreBits ? score_key(t[u]) : 0u;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kRxPer; ++j) {
      const float x = src[min((j >> 2) * kSlice + 4 * tid + (j & 3), max(len - 1, 0))];
      key[j] = len > 0 && __float_as_uint(x) != kNoScoreBits ? score_key(x) : 0u;
    }
  }
  const int nE = min(a.n_entries[b], a.N_cap);
  const int n = max(0, min(max(0, min(nE, (a.q_pos[row] + 1) / a.m)) - off, len));
#pragma unroll
  for (int j = 0; j < kRxPer; ++j)
    if ((j >> 2) * kSlice + 4 * tid + (j & 3) >= n) key[j] = 0u;
}

// The row's histogram of `nb` bins into LDS, then the digit holding the
// k_rem-th largest key.
__device__ __forceinline__ void rx_digit(const int *g, int nb, int k_rem, int (*hs)[kBins], int *sh, int &digit,
                                         int &above, int &total) {
  for (int i = threadIdx.x; i < nb; i += kRegThreads) hs[0][i] = g[i];
  __syncthreads();
  int count;
  find_digit<kRegThreads>(hs, 1, nb, k_rem, sh, digit, above, count, total);
}

// Adds this workgroup's histogram (LDS, nb bins) into the row's.
__device__ __forceinline__ void rx_flush(int (*hs)[kBins], int nb, int *g) {
  __syncthreads();
  for (int i = threadIdx.x; i < nb; i += kRegThreads) {
    const int c = hs[0][i];
    if (c) atomicAdd(g + i, c);
  }
}

__global__ void rx_zero_kernel(int *p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// Stage s: 1 = digit-1 histogram, 2 = digit 2, 3 = digit 3, 4 = counts at T.
template <int kStage>
__global__ __launch_bounds__(kRegThreads) void rx_hist_kernel(RxArgs a) {
  __shared__ int hs[1][kBins];
  __shared__ int sh[kRegThreads / 64 + 3];
  const int q = blockIdx.x / a.nsl, sl = blockIdx.x % a.nsl, b = blockIdx.y;
  const int64_t row = (int64_t)b * a.Q + q;
  uint32_t key[kRxPer];
  rx_load(a, row, b, sl, key);
  int k_eff = 0, k_rem = a.k;
  uint32_t prefix = 0;  // resolved high bits of T
  if (kStage >= 2) {
    int d1, above, total;
    rx_digit(a.hist1 + row * 2048, 2048, a.k, hs, sh, d1, above, total);
    k_eff = min(a.k, total);
    if (k_eff == total || k_eff == 0) {
      // every visible key is taken (T = 0: key > 0), or none
      if (kStage == 4) {
        const uint32_t T = k_eff == 0 ? 0xFFFFFFFFu : 0u;
        int ng = 0;
#pragma unroll
        for (int j = 0; j < kRxPer; ++j) ng += key[j] > T;
        ng = wave_sum(ng);
        if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = ng;
        __syncthreads();
        if (threadIdx.x == 0) {
          int t = 0;
          for (int w = 0; w < kRegThreads / 64; ++w) t += sh[w];
          a.counts[(row * a.nsl + sl) * 2] = t;
          a.counts[(row * a.nsl + sl) * 2 + 1] = 0;
          if (sl == 0) {
            a.desc[row * 4] = (int)T;
            a.desc[row * 4 + 1] = 0;
            a.desc[row * 4 + 2] = k_eff;
          }
        }
      }
      return;
    }
    k_rem = k_eff - above;
    prefix = (uint32_t)d1;
    if (kStage >= 3) {
      int d2;
      rx_digit(a.hist2 + row * 2048, 2048, k_rem, hs, sh, d2, above, total);
      k_rem -= above;
      prefix = (prefix << 11) | (uint32_t)d2;
      if (kStage >= 4) {
        int d3;
        rx_digit(a.hist3 + row * 1024, 1024, k_rem, hs, sh, d3, above, total);
        k_rem -= above;
        const uint32_t T = (prefix << 10) | (uint32_t)d3;
        int ng = 0, ne = 0;
#pragma unroll
        for (int j = 0; j < kRxPer; ++j) {
          ng += key[j] > T;
          ne += key[j] == T;
        }
        ng = wave_sum(ng);
        ne = wave_sum(ne);
        __syncthreads();  // sh reads of find_digit are done
        if ((threadIdx.x & 63) == 0) {
          sh[threadIdx.x >> 6] = ng;
          hs[0][threadIdx.x >> 6] = ne;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
          int tg = 0, te = 0;
          for (int w = 0; w < kRegThreads / 64; ++w) {
            tg += sh[w];
            te += hs[0][w];
          }
          a.counts[(row * a.nsl + sl) * 2] = tg;
          a.counts[(row * a.nsl + sl) * 2 + 1] = te;
          if (sl == 0) {
            a.desc[row * 4] = (int)T;
            a.desc[row * 4 + 1] = k_rem;  // keys equal to T that are taken
            a.desc[row * 4 + 2] = k_eff;
          }
        }
        return;
      }
    }
    __syncthreads();  // the histogram buffer is reused below
  }
  const int nb = kStage == 3 ? 1024 : 2048;
  for (int i = threadIdx.x; i < nb; i += kRegThreads) hs[0][i] = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kRxPer; ++j) {
    const uint32_t kk = key[j];
    if (kk == 0u) continue;
    if (kStage == 1) atomicAdd(&hs[0][kk >> 21], 1);
    if (kStage == 2 && (kk >> 21) == prefix) atomicAdd(&hs[0][(kk >> 10) & 2047u], 1);
    if (kStage == 3 && (kk >> 10) == prefix) atomicAdd(&hs[0][kk & 1023u], 1);
  }
  int *g = kStage == 1 ? a.hist1 + row * 2048 : kStage == 2 ? a.hist2 + row * 2048 : a.hist3 + row * 1024;
  rx_flush(hs, nb, g);
}

// Placement: the keys above T and the first `need` keys equal to T (in
// entry order over the whole row) go to their rank among the selected, in
// ascending entry order.
__global__ __launch_bounds__(kRegThreads) void rx_place_kernel(RxArgs a) {
  constexpr int kW = kRegThreads / 64;
  constexpr int kV = kRxPer / 4;
  constexpr int kSlice = kRegThreads * 4;
  __shared__ int cnt[2][kV * kW];
  const int q = blockIdx.x / a.nsl, sl = blockIdx.x % a.nsl, b = blockIdx.y;
  const int64_t row = (int64_t)b * a.Q + q;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint32_t key[kRxPer];
  rx_load(a, row, b, sl, key);
  const uint32_t T = (uint32_t)a.desc[row * 4];
  const int need = a.desc[row * 4 + 1], k_eff = a.desc[row * 4 + 2];
  // counts of the slices before this one (every thread sums a few)
  int bg = 0, be = 0;
  for (int s = lane; s < sl; s += 64) {
    bg += a.counts[(row * a.nsl + s) * 2];
    be += a.counts[(row * a.nsl + s) * 2 + 1];
  }
  bg = wave_sum(bg);
  be = wave_sum(be);
  const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
#pragma unroll
  for (int v = 0; v < kV; ++v) {
    int gc = 0, ec = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      gc += __popcll(__ballot(key[4 * v + u] > T));
      ec += __popcll(__ballot(key[4 * v + u] == T));
    }
    if (lane == 0) {
      cnt[0][v * kW + wave] = gc;
      cnt[1][v * kW + wave] = ec;
    }
  }
  __syncthreads();
  int32_t *oi = a.idx_out + row * a.k;
  float *os = a.score_out ? a.score_out + row * a.k : nullptr;
#pragma unroll
  for (int v = 0; v < kV; ++v) {
    int gb = bg, eb = be;
    for (int e = 0; e < v * kW + wave; ++e) {
      gb += cnt[0][e];
      eb += cnt[1][e];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      gb += __popcll(__ballot(key[4 * v + u] > T) & below);
      eb += __popcll(__ballot(key[4 * v + u] == T) & below);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t kk = key[4 * v + u];
      const bool gt = kk > T, eq = kk == T;
      if (gt || (eq && eb < need)) {
        const int p = gb + min(eb, need);
        if (p < k_eff) {
          oi[p] = sl * kRxSlice + v * kSlice + 4 * tid + u;
          if (os) os[p] = key_score(kk);
        }
      }
      gb += gt;
      eb += eq;
    }
  }
  if (sl == a.nsl - 1) {
    for (int j = k_eff + tid; j < a.k; j += kRegThreads) {
      oi[j] = -1;
      if (os) os[j] = __uint_as_float(kNoScoreBits);
    }
  }
}

static hipError_t launch_radix(const CacheView &c, const float *scores, int Ns, const int32_t *q_pos, int Q, int k,
                               int32_t *idx_out, float *score_out, void *ws, hipStream_t stream, bool prezeroed) {
  const int rows = c.B * Q;
  const int nsl = (Ns + kRxSlice - 1) / kRxSlice;
  RxArgs a;
  a.scores = scores;
  a.Ns = Ns;
  a.n_entries = c.n_entries;
  a.N_cap = c.N_cap;
  a.m = c.m;
  a.q_pos = q_pos;
  a.Q = Q;
  a.k = k;
  a.nsl = nsl;
  a.hist1 = reinterpret_cast<int *>(ws);
  a.hist2 = a.hist1 + (size_t)rows * 2048;
  a.hist3 = a.hist2 + (size_t)rows * 2048;
  a.counts = a.hist3 + (size_t)rows * 1024;
  a.desc = a.counts + (size_t)rows * nsl * 2;
  a.idx_out = idx_out;
  a.score_out = score_out;
  const int nz = rows * (2048 + 2048 + 1024);  // the histograms, topk_radix_zero_bytes()
  if (!prezeroed) rx_zero_kernel<<<(nz + 255) / 256, 256, 0, stream>>>(a.hist1, nz);
  const dim3 grid(Q * nsl, c.B);
  rx_hist_kernel<1><<<grid, kRegThreads, 0, stream>>>(a);
  rx_hist_kernel<2><<<grid, kRegThreads, 0, stream>>>(a);
  rx_hist_kernel<3><<<grid, kRegThreads, 0, stream>>>(a);
  rx_hist_kernel<4><<<grid, kRegThreads, 0, stream>>>(a);
  rx_place_kernel<<<grid, kRegThreads, 0, stream>>>(a);
  return hipGetLastError();
}

TopkPlan topk_plan(int B, int Q, int Ns, int k) {
  TopkPlan p{1, Ns, 0};
  const int64_t rows = (int64_t)B * Q;
  if (rows < 256 && Ns >= 65536 && k > 0) {
    p.radix = true;
    p.nsl = (Ns + kRxSlice - 1) / kRxSlice;
    p.S = kRxSlice;
    p.ws_bytes = (size_t)rows * (2048 + 2048 + 1024 + 2 * p.nsl + 4) * sizeof(int);
    return p;
  }
  if (rows >= 256 || Ns <= 4096 || k <= 0) return p;
  // Smallest power-of-two slice (>= 4096, >= k) whose candidates fit one
  // register-resident row in the second stage.
  for (int S = 4096; S <= kRegN; S *= 2) {
    if (S < k) continue;
    const int nsl = (Ns + S - 1) / S;
    if (nsl < 2) break;
    if ((int64_t)nsl * k <= kRegN) {
      p.nsl = nsl;
      p.S = S;
      p.ws_bytes = (size_t)rows * nsl * k * (sizeof(int32_t) + sizeof(float));
      return p;
    }
  }
  return p;
}

template <int kPer>
static void launch_reg(dim3 grid, hipStream_t stream, const float *scores, int Ns, const CacheView &c,
                       const int32_t *q_pos, int Q, const int32_t *cand, int C, int k, int32_t *idx_out,
                       float *score_out, int nsl, int S) {
  if (cand)
    topk_reg_kernel<kPer, true><<<grid, kRegThreads, 0, stream>>>(scores, Ns, c.n_entries, c.N_cap, c.m, q_pos, Q,
                                                                  cand, C, k, idx_out, score_out, nsl, S);
  else
    topk_reg_kernel<kPer, false><<<grid, kRegThreads, 0, stream>>>(scores, Ns, c.n_entries, c.N_cap, c.m, q_pos, Q,
                                                                   nullptr, 0, k, idx_out, score_out, nsl, S);
}

static void launch_one(const CacheView &c, const float *scores, int Ns, int len, const int32_t *q_pos, int Q,
                       const int32_t *cand, int C, int k, int32_t *idx_out, float *score_out, int nsl, int S,
                       hipStream_t stream) {
  dim3 grid(Q * nsl, c.B);
  if (len <= kRegThreads * 8)
    launch_reg<8>(grid, stream, scores, Ns, c, q_pos, Q, cand, C, k, idx_out, score_out, nsl, S);
  else if (len <= kRegThreads * 16)
    launch_reg<16>(grid, stream, scores, Ns, c, q_pos, Q, cand, C, k, idx_out, score_out, nsl, S);
  else if (len <= kRegThreads * 32)
    launch_reg<32>(grid, stream, scores, Ns, c, q_pos, Q, cand, C, k, idx_out, score_out, nsl, S);
  else if (len <= kRegN)
    launch_reg<64>(grid, stream, scores, Ns, c, q_pos, Q, cand, C, k, idx_out, score_out, nsl, S);
  else
    topk_tiled_kernel<<<dim3(Q, c.B), kTopkThreads, 0, stream>>>(scores, Ns, c.n_entries, c.N_cap, c.m, q_pos, Q, cand,
                                                                 C, k, idx_out, score_out);
}

size_t topk_radix_zero_bytes(int B, int Q, int Ns, int k) {
  return topk_plan(B, Q, Ns, k).radix ? (size_t)B * Q * (2048 + 2048 + 1024) * sizeof(int) : 0;
}

bool topk_hint_fits(int B, int Q, int Ns, int k) {
  return (int64_t)B * Q < 256 && Ns > 0 && Ns <= kRegN && k > 0;
}

size_t topk_hint_ws_bytes(int B, int Q, int Ns) {
  const int64_t rows = (int64_t)B * Q;
  const int nsl = (Ns + kHintSlice - 1) / kHintSlice;
  return (size_t)rows * ((size_t)kHintBins * 4 + (size_t)nsl * kHintSlice * 8 + (size_t)nsl * 3 * 4 + 4 * 4);
}

hipError_t launch_topk_hint(const CacheView &c, const float *scores, int Ns, const int32_t *q_pos, int Q, int k,
                            int32_t *idx_out, float *score_out, void *ws, hipStream_t stream) {
  const int64_t rows = (int64_t)c.B * Q;
  const int nsl = (Ns + kHintSlice - 1) / kHintSlice;
  HintArgs a;
  a.scores = scores;
  a.Ns = Ns;
  a.n_entries = c.n_entries;
  a.N_cap = c.N_cap;
  a.m = c.m;
  a.q_pos = q_pos;
  a.Q = Q;
  a.k = k;
  a.nsl = nsl;
  a.hint = reinterpret_cast<uint32_t *>(ws);
  a.cand_i = reinterpret_cast<int32_t *>(a.hint + rows * kHintBins);
  a.cand_k = reinterpret_cast<uint32_t *>(a.cand_i + rows * nsl * kHintSlice);
  a.slice_info = reinterpret_cast<int32_t *>(a.cand_k + rows * nsl * kHintSlice);
  a.row_info = a.slice_info + rows * nsl * 3;
  a.idx_out = idx_out;
  a.score_out = score_out;
  topk_hint_compact_kernel<<<dim3(Q * nsl, c.B), kRegThreads, 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  topk_hint_final_kernel<<<dim3(Q, c.B), kRegThreads, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_topk(const CacheView &c, const float *scores, int Ns, const int32_t *q_pos, int Q,
                       const int32_t *cand, int C, int k, int32_t *idx_out, float *score_out, void *ws,
                       hipStream_t stream, bool prezeroed) {
  const TopkPlan p = cand ? TopkPlan{1, Ns, 0} : topk_plan(c.B, Q, Ns, k);
  if (p.radix) return launch_radix(c, scores, Ns, q_pos, Q, k, idx_out, score_out, ws, stream, prezeroed);
  if (p.nsl == 1) {
    launch_one(c, scores, Ns, Ns, q_pos, Q, cand, C, k, idx_out, score_out, 1, Ns, stream);
    return hipGetLastError();
  }
  // stage 1: exact top-k of every slice; stage 2: top-k of the candidates
  const int Cc = p.nsl * k;
  int32_t *ci = reinterpret_cast<int32_t *>(ws);
  float *cs = reinterpret_cast<float *>(ci + (size_t)c.B * Q * Cc);
  launch_one(c, scores, Ns, p.S, q_pos, Q, nullptr, 0, k, ci, cs, p.nsl, p.S, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  launch_one(c, cs, Cc, Cc, q_pos, Q, ci, Cc, k, idx_out, score_out, 1, Cc, stream);
  return hipGetLastError();
}

}  // namespace csa
