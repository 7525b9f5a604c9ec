// Per-query top-k of the indexer scores ([V4] "ハイブリッド注意：CSAとHCA",
// CSA paragraph: the indexer picks the top-k compressed blocks of each
// query; [V4.1] "推論カーネル" names a dedicated TopK kernel).
//
// Exact radix select on order-preserving uint32 keys, one 1024-thread
// workgroup per query:
//   * the scores of a tile (up to kTile of them) sit in LDS as keys, each
//     thread owning a contiguous run, padded one word per 32 so that the
//     strided runs do not collide on LDS banks;
//   * four passes of 8 bits, most significant first, build per-wave
//     histograms of the elements still matching the chosen prefix and fix
//     one digit of the k-th largest key T;
//   * a last pass keeps every key > T plus the first (by entry index)
//     elements equal to T, and writes them in ascending order through two
//     block-wide prefix sums.
// Rows longer than kTile are processed tile by tile in every pass.  Rows of
// at most 32,768 scores take the register-resident variant further below.
#include "csa_device.hpp"
#include "csa_internal.hpp"

namespace csa {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kTile = 32768;
constexpr int kTilePadded = kTile + kTile / 32;

__device__ __forceinline__ int lds_pos(int i) { return i + (i >> 5); }

// Exclusive prefix sum over the 1024 threads in thread order; also returns the total.
__device__ __forceinline__ int block_excl_scan(int v, int *sh, int &total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(inc, o);
    if (lane >= o) inc += t;
  }
  if (lane == 63) sh[wave] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < kTopkWaves; ++w) {
      const int t = sh[w];
      sh[w] = run;
      run += t;
    }
    sh[kTopkWaves] = run;
  }
  __syncthreads();
  const int res = sh[wave] + inc - v;
  total = sh[kTopkWaves];
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
    if (out_s) out_s[j] = __uint_as_float(0x7FC00000u);
  }
}


// Rows of at most kRegN scores: every thread keeps its kRegPer consecutive
// keys in registers; digits of 11, 11 and 10 bits (the first, which every
// element takes part in, spreads over four bins per octave of the score,
// so same-bin atomics within a wave stay few); per-wave histograms in LDS.
constexpr int kRegPer = 32;
constexpr int kRegN = kTopkThreads * kRegPer;
constexpr int kBins = 2048;

// Finds the digit (of `nb` bins, nb = 2048 or 1024) holding the k_rem-th
// largest remaining element; the counts are summed over `nh` per-wave
// histograms.  Every thread returns the same (digit, elements above it).
__device__ __forceinline__ void find_digit(const int (*hist)[kBins], int nh, int nb, int k_rem, int *sh, int &digit,
                                           int &above_out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = nb / kTopkThreads;  // 2 or 1 bins per thread, in descending digit order
  int c[2] = {0, 0};
  for (int j = 0; j < per; ++j) {
    const int d = nb - 1 - (tid * per + j);
    int s = 0;
    for (int w = 0; w < nh; ++w) s += hist[w][d];
    c[j] = s;
  }
  const int tot = c[0] + c[1];
  int inc = tot;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(inc, o);
    if (lane >= o) inc += t;
  }
  if (lane == 63) sh[wave] = inc;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int w = 0; w < kTopkWaves; ++w) {
      const int t = sh[w];
      sh[w] = run;
      run += t;
    }
  }
  __syncthreads();
  int above = sh[wave] + inc - tot;
  for (int j = 0; j < per; ++j) {
    if (above < k_rem && k_rem <= above + c[j]) {
      sh[kTopkWaves + 1] = nb - 1 - (tid * per + j);
      sh[kTopkWaves + 2] = above;
    }
    above += c[j];
  }
  __syncthreads();
  digit = sh[kTopkWaves + 1];
  above_out = sh[kTopkWaves + 2];
  __syncthreads();
}

__global__ __launch_bounds__(kTopkThreads) void topk_reg_kernel(const float *__restrict__ scores, int Ns,
                                                                 const int32_t *__restrict__ n_entries, int N_cap,
                                                                 int m, const int32_t *__restrict__ q_pos, int Q,
                                                                 const int32_t *__restrict__ cand, int C, int k,
                                                                 int32_t *__restrict__ idx_out,
                                                                 float *__restrict__ score_out) {
  __shared__ int hist[kTopkWaves][kBins];
  __shared__ int sh[kTopkWaves + 4];

  const int q = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6;
  const int64_t row = (int64_t)b * Q + q;
  const float *src = scores + row * Ns;
  int n;
  if (cand) {
    n = C;
  } else {
    const int nE = min(n_entries[b], N_cap);
    n = max(0, min(nE, (q_pos[row] + 1) / m));
  }

  // keys of elements tid*kRegPer .. +kRegPer-1; 0 = not a candidate
  uint32_t key[kRegPer];
  const int i0 = tid * kRegPer;
  if (i0 + kRegPer <= n && (Ns & 3) == 0) {
#pragma unroll
    for (int v = 0; v < kRegPer / 4; ++v) {
      const float4 f = *reinterpret_cast<const float4 *>(src + i0 + 4 * v);
      const float ff[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t bits = __float_as_uint(ff[u]);
        key[4 * v + u] = bits == kNoScoreBits ? 0u : score_key(ff[u]);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < kRegPer; ++j) {
      uint32_t kk = 0;
      if (i0 + j < n) {
        const uint32_t bits = __float_as_uint(src[i0 + j]);
        kk = bits == kNoScoreBits ? 0u : score_key(__uint_as_float(bits));
      }
      key[j] = kk;
    }
  }

  int n_valid = n;
  if (cand) {
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < kRegPer; ++j) cnt += key[j] != 0u;
    int tot;
    block_excl_scan(cnt, sh, tot);
    n_valid = tot;
  }
  const int k_eff = min(k, n_valid);

  uint32_t thr = 0;   // full key of the k_eff-th largest element
  int need = 0;       // elements equal to thr that are taken
  if (k_eff > 0 && k_eff < n_valid) {
    // pass 1: bits 31..21, per-wave histograms
    for (int i = tid; i < kTopkWaves * kBins; i += kTopkThreads) (&hist[0][0])[i] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kRegPer; ++j) atomicAdd(&hist[wave][key[j] >> 21], 1);
    __syncthreads();
    int d1, above;
    find_digit(hist, kTopkWaves, kBins, k_eff, sh, d1, above);
    int k_rem = k_eff - above;
    // pass 2: bits 20..10 of the elements in bin d1
    for (int i = tid; i < kBins; i += kTopkThreads) hist[0][i] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kRegPer; ++j)
      if ((key[j] >> 21) == (uint32_t)d1) atomicAdd(&hist[0][(key[j] >> 10) & 0x7FFu], 1);
    __syncthreads();
    int d2;
    find_digit(hist, 1, kBins, k_rem, sh, d2, above);
    k_rem -= above;
    const uint32_t p12 = ((uint32_t)d1 << 11) | (uint32_t)d2;
    // pass 3: bits 9..0
    for (int i = tid; i < kBins; i += kTopkThreads) hist[0][i] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kRegPer; ++j)
      if ((key[j] >> 10) == p12) atomicAdd(&hist[0][key[j] & 0x3FFu], 1);
    __syncthreads();
    int d3;
    find_digit(hist, 1, 1024, k_rem, sh, d3, above);
    k_rem -= above;
    thr = (p12 << 10) | (uint32_t)d3;
    need = k_rem;
  }

  int32_t *out_i = idx_out + row * k;
  float *out_s = score_out ? score_out + row * k : nullptr;
  if (k_eff > 0) {
    int gt = 0, eq = 0;
#pragma unroll
    for (int j = 0; j < kRegPer; ++j) {
      gt += key[j] > thr;
      eq += need > 0 && key[j] == thr;
    }
    int eq_tot;
    const int eq_before = block_excl_scan(eq, sh, eq_tot);
    const int take_eq = max(0, min(eq, need - eq_before));
    int sel_tot;
    int off = block_excl_scan(gt + take_eq, sh, sel_tot);
    int eq_seen = 0;
#pragma unroll
    for (int j = 0; j < kRegPer; ++j) {
      bool take = key[j] > thr;
      if (!take && need > 0 && key[j] == thr) {
        take = eq_seen < take_eq;
        ++eq_seen;
      }
      if (take && off < k_eff) {
        out_i[off] = cand ? cand[row * C + i0 + j] : i0 + j;
        if (out_s) out_s[off] = key_score(key[j]);
        ++off;
      }
    }
  }
  for (int j = k_eff + tid; j < k; j += kTopkThreads) {
    out_i[j] = -1;
    if (out_s) out_s[j] = __uint_as_float(0x7FC00000u);
  }
}

hipError_t launch_topk(const CacheView &c, const float *scores, int Ns, const int32_t *q_pos, int Q,
                       const int32_t *cand, int C, int k, int32_t *idx_out, float *score_out, hipStream_t stream) {
  dim3 grid(Q, c.B);
  if (Ns <= kRegN)
    topk_reg_kernel<<<grid, kTopkThreads, 0, stream>>>(scores, Ns, c.n_entries, c.N_cap, c.m, q_pos, Q, cand, C, k,
                                                       idx_out, score_out);
  else
    topk_tiled_kernel<<<grid, kTopkThreads, 0, stream>>>(scores, Ns, c.n_entries, c.N_cap, c.m, q_pos, Q, cand, C, k,
                                                         idx_out, score_out);
  return hipGetLastError();
}

}  // namespace csa
