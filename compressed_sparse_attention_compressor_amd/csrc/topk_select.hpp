// Exact top-k selection over keys held in registers by one workgroup
// ([V4] "ハイブリッド注意：CSAとHCA", CSA paragraph: the indexer keeps the
// top-k compressed blocks of each query).  Shared by the stand-alone top-k
// kernels and the indexer kernel that selects within its own slice.
#pragma once

#include "csa_device.hpp"

namespace csa {

// Register-resident selection: a workgroup of kRegThreads threads holding
// up to kRegN keys in registers.
constexpr int kRegThreads = 512;
constexpr int kRegN = kRegThreads * 64;
constexpr int kBins = 2048;

// Finds the digit (of `nb` <= kBins bins) holding the k_rem-th largest
// remaining element; the counts are summed over `nh` per-wave histograms.
// Every thread returns the same digit, the number of elements in higher
// digits and the histogram total; when the total is below k_rem the digit
// is undefined.  Two barriers; uses sh[0 .. kW+2).
template <int NT>
__device__ __forceinline__ void find_digit(const int (*hist)[kBins], int nh, int nb, int k_rem, int *sh, int &digit,
                                           int &above_out, int &total) {
  constexpr int kW = NT / 64;
  constexpr int kMaxPer = kBins / NT;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int per = nb >= NT ? nb / NT : 1;  // bins per thread, in descending digit order
  int c[kMaxPer];
  int tot = 0;
#pragma unroll
  for (int j = 0; j < kMaxPer; ++j) {
    const int bin = tid * per + j;
    int s = 0;
    if (j < per && bin < nb)
      for (int w = 0; w < nh; ++w) s += hist[w][nb - 1 - bin];
    c[j] = s;
    tot += s;
  }
  const int inc = wave_incl_scan(tot);
  if (lane == 63) sh[wave] = inc;
  __syncthreads();
  int base = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kW; ++w) {
    const int t = sh[w];
    base += w < wave ? t : 0;
    all += t;
  }
  int above = base + inc - tot;
#pragma unroll
  for (int j = 0; j < kMaxPer; ++j) {
    if (j < per && above < k_rem && k_rem <= above + c[j]) {
      sh[kW] = nb - 1 - (tid * per + j);
      sh[kW + 1] = above;
    }
    above += c[j];
  }
  __syncthreads();
  // A later call writes sh only after its first barrier, which every thread
  // reaches after these reads.
  digit = __builtin_amdgcn_readfirstlane(sh[kW]);
  above_out = __builtin_amdgcn_readfirstlane(sh[kW + 1]);
  total = __builtin_amdgcn_readfirstlane(all);
}

// Selects, among the keys held in registers by the kRegThreads threads of
// the workgroup (key[4v + u] is element v*(4*kRegThreads) + 4*tid + u; key 0
// marks an empty slot), the k largest, exact ties to the lower element, and
// writes their ids (cid, or id_of(element)) and scores in ascending element
// order to out_i / out_s, padding with -1 and kNoScoreBits up to k.
// Selection is a short chain of block-wide steps; cross-lane work runs on
// DPP and readlane, and small scans are repeated by every wave rather than
// published through a further barrier:
//   1. row maximum, minimum and valid count;
//   2. histogram of 2,047 linear bins in score space between the extremes
//      (each key's bin kept in registers) and the bin holding the k-th
//      element;
//   3. when that bin holds at most 64 elements they are gathered (one LDS
//      atomic per wave) and every wave ranks them to fix the exact threshold
//      key T and how many elements equal to T are taken; otherwise, and when
//      the window holds fewer than k elements, radix passes over the
//      remaining bits do it;
//   4. placement in ascending entry order: per (slice, wave) ballots of
//      "key > T" and "key == T", a scan of those counts, and in-wave ranks
//      from masked popcounts.
template <int kPer, bool kPrefetch, typename IdOf>
__device__ __forceinline__ void select_keys(uint32_t (&key)[kPer], const int32_t (&cid)[kPrefetch ? kPer : 1], int k,
                                            int32_t *__restrict__ out_i, float *__restrict__ out_s, IdOf id_of) {
  constexpr int NT = kRegThreads;
  constexpr int kW = NT / 64;
  constexpr int kV = kPer / 4;              // slices of 4*NT elements
  constexpr int kSlice = NT * 4;
  constexpr int kE = kV * kW;               // (slice, wave) pairs
  static_assert(kE <= 128, "a wave scans the (slice, wave) counts two per lane");
  __shared__ int hist[kW][kBins];
  __shared__ int sh[kW + 3];
  __shared__ uint32_t wmax[kW], wmin[kW];
  __shared__ int wcnt[kW];
  __shared__ uint32_t bin_keys[64];
  __shared__ int cnt[2][kE];                // per (slice, wave): elements > T, elements == T
  __shared__ int n_bin;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  for (int i = tid; i < kBins; i += NT) hist[0][i] = 0;
  if (tid == 0) n_bin = 0;

  // 1. maximum, minimum and count of the valid keys
  {
    uint32_t mx = 0, mnc = 0;  // mnc: complement of the minimum
    int nv = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      mx = key[j] > mx ? key[j] : mx;
      const uint32_t c = key[j] ? ~key[j] : 0u;
      mnc = c > mnc ? c : mnc;
      nv += key[j] != 0u;
    }
    mx = wave_max_u32(mx);
    mnc = wave_max_u32(mnc);
    nv = wave_sum(nv);
    if (lane == 0) {
      wmax[wave] = mx;
      wmin[wave] = mnc;
      wcnt[wave] = nv;
    }
  }
  __syncthreads();
  uint32_t mx = 0, mnc = 0;
  int n_valid = 0;
#pragma unroll
  for (int w = 0; w < kW; ++w) {
    mx = max(mx, wmax[w]);
    mnc = max(mnc, wmin[w]);
    n_valid += wcnt[w];
  }
  mx = __builtin_amdgcn_readfirstlane(mx);
  mnc = __builtin_amdgcn_readfirstlane(mnc);
  n_valid = __builtin_amdgcn_readfirstlane(n_valid);
  const int k_eff = min(k, n_valid);

  // Linear bins in score space between the extremes: bin(v) = (vmax - v) * inv
  // is non-increasing in v (each rounding step is monotone), so keys in a
  // lower bin are strictly larger than keys in a higher one; the exact order
  // inside the threshold bin is settled on the keys themselves.
  const float vmax = key_score(mx), vmin = key_score(~mnc);
  float inv = (float)(kBins - 2) / (vmax - vmin);
  if (!(inv < INFINITY)) inv = 0.f;  // equal extremes, or a span beyond fp32
  auto bin_of = [&](uint32_t kk) { return (uint32_t)fminf((vmax - key_score(kk)) * inv, (float)(kBins - 2)); };

  uint32_t thr = 1u;  // full key of the k_eff-th largest element (1: every valid key)
  int need = 0;       // elements equal to thr that are taken
  int n_eq = 0;       // elements equal to thr
  if (k_eff > 0 && k_eff < n_valid) {
    // each key's bin is computed once and kept (two 16-bit bins per
    // register; 0xFFFF for an invalid key) for the threshold-bin passes
    uint32_t binp[(kPer + 1) / 2];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const uint32_t bj = key[j] != 0u ? bin_of(key[j]) : 0xFFFFu;
      if (j & 1) binp[j >> 1] |= bj << 16;
      else binp[j >> 1] = bj;
      if (key[j] != 0u) atomicAdd(&hist[0][kBins - 2 - bj], 1);
    }
    __syncthreads();
    int d1, above, tot;
    find_digit<NT>(hist, 1, kBins, k_eff, sh, d1, above, tot);
    const int c1 = __builtin_amdgcn_readfirstlane(hist[0][d1]);
    const uint32_t dhi = (uint32_t)(kBins - 2 - d1);
    auto in_dhi = [&](int j) { return ((binp[j >> 1] >> (16 * (j & 1))) & 0xFFFFu) == dhi; };
    int k_rem = k_eff - above;
    if (c1 <= 64) {
      // 2a. gather the threshold bin (one LDS atomic per wave) and rank it
      int mine = 0;
#pragma unroll
      for (int j = 0; j < kPer; ++j) mine += in_dhi(j);
      const int inc = wave_incl_scan(mine);
      const int wtot = __builtin_amdgcn_readlane(inc, 63);
      int base = 0;
      if (wtot > 0) {
        if (lane == 63) base = atomicAdd(&n_bin, wtot);
        base = __builtin_amdgcn_readlane(base, 63);
      }
      int pos = base + inc - mine;
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if (in_dhi(j)) bin_keys[pos++] = key[j];
      __syncthreads();
      // wave 0 ranks the gathered keys (lanes past c1 take no part) and
      // publishes the threshold
      if (wave == 0) {
        const uint32_t kl = lane < c1 ? bin_keys[lane] : 0u;
        int gt = 0, ge = 0;
        for (int j = 0; j < c1; ++j) {
          const uint32_t kj = (uint32_t)__builtin_amdgcn_readlane((int)kl, j);
          gt += kj > kl;
          ge += kj >= kl;
        }
        if (lane < c1 && gt < k_rem && k_rem <= ge) {  // every lane holding the threshold key agrees
          sh[kW] = (int)kl;
          sh[kW + 1] = k_rem - gt;
          sh[kW + 2] = ge - gt;
        }
      }
      __syncthreads();
      thr = (uint32_t)__builtin_amdgcn_readfirstlane(sh[kW]);
      need = __builtin_amdgcn_readfirstlane(sh[kW + 1]);
      n_eq = __builtin_amdgcn_readfirstlane(sh[kW + 2]);
    } else {
      // 2b. a crowded bin (many equal or nearly equal scores): radix passes
      //     over the keys of that bin, bits 31..21, 20..10 and 9..0
      for (int i = tid; i < kBins; i += NT) hist[0][i] = 0;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if (in_dhi(j)) atomicAdd(&hist[0][key[j] >> 21], 1);
      __syncthreads();
      int e1, ab;
      find_digit<NT>(hist, 1, kBins, k_rem, sh, e1, ab, tot);
      k_rem -= ab;
      for (int i = tid; i < kBins; i += NT) hist[0][i] = 0;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if (in_dhi(j) && (key[j] >> 21) == (uint32_t)e1)
          atomicAdd(&hist[0][(key[j] >> 10) & 0x7FFu], 1);
      __syncthreads();
      int e2;
      find_digit<NT>(hist, 1, kBins, k_rem, sh, e2, ab, tot);
      k_rem -= ab;
      const uint32_t p12 = ((uint32_t)e1 << 11) | (uint32_t)e2;
      for (int i = tid; i < kBins; i += NT) hist[0][i] = 0;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if (in_dhi(j) && (key[j] >> 10) == p12) atomicAdd(&hist[0][key[j] & 0x3FFu], 1);
      __syncthreads();
      int e3;
      find_digit<NT>(hist, 1, 1024, k_rem, sh, e3, ab, tot);
      k_rem -= ab;
      thr = (p12 << 10) | (uint32_t)e3;
      need = k_rem;
      n_eq = __builtin_amdgcn_readfirstlane(hist[0][e3]);  // every key equal to thr lies in this bin
    }
  }

  // 3. placement in ascending entry order.  When every element equal to the
  // threshold is taken the selection is simply key >= thr; otherwise the
  // elements above it and the first `need` equal ones (by entry) are taken.
  // Up to kStage selections are placed in LDS (over the histograms, whose
  // last reads precede the barrier below) and written out coalesced.
  constexpr int kStage = kW * kBins / 2;
  const bool staged = k_eff <= kStage;
  int32_t *st_i = &hist[0][0];
  float *st_s = reinterpret_cast<float *>(&hist[0][0] + kStage);
  if (k_eff > 0) {
    const bool simple = need == n_eq;
    // taken outright: key >= thr when simple, key > thr otherwise
    auto sure = [&](uint32_t kk) { return simple ? kk >= thr : kk > thr; };
    const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
#pragma unroll
    for (int v = 0; v < kV; ++v) {
      int gc = 0, ec = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        gc += __popcll(__ballot(sure(key[4 * v + u])));
        if (!simple) ec += __popcll(__ballot(key[4 * v + u] == thr));
      }
      if (lane == 0) {
        cnt[0][v * kW + wave] = gc;
        cnt[1][v * kW + wave] = ec;
      }
    }
    __syncthreads();
    // every wave scans the counts in (slice, wave) order, two per lane
    int gx[2], ex[2] = {0, 0};
    {
      const int e0 = 2 * lane, e1 = 2 * lane + 1;
      const int g0 = e0 < kE ? cnt[0][e0] : 0, g1 = e1 < kE ? cnt[0][e1] : 0;
      const int gi = wave_incl_scan(g0 + g1);
      gx[0] = gi - g0 - g1;
      gx[1] = gi - g1;
      if (!simple) {
        const int q0 = e0 < kE ? cnt[1][e0] : 0, q1 = e1 < kE ? cnt[1][e1] : 0;
        const int qi = wave_incl_scan(q0 + q1);
        ex[0] = qi - q0 - q1;
        ex[1] = qi - q1;
      }
    }
#pragma unroll
    for (int v = 0; v < kV; ++v) {
      const int e = v * kW + wave;
      int gb = (e & 1) ? __builtin_amdgcn_readlane(gx[1], e >> 1) : __builtin_amdgcn_readlane(gx[0], e >> 1);
      int eb = 0;
      if (!simple) eb = (e & 1) ? __builtin_amdgcn_readlane(ex[1], e >> 1) : __builtin_amdgcn_readlane(ex[0], e >> 1);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        gb += __popcll(__ballot(sure(key[4 * v + u])) & below);
        if (!simple) eb += __popcll(__ballot(key[4 * v + u] == thr) & below);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t kk = key[4 * v + u];
        const bool is_gt = sure(kk), is_eq = !simple && kk == thr;
        if (is_gt || (is_eq && eb < need)) {
          const int p = gb + min(eb, need);
          if (p < k_eff) {
            const int i = v * kSlice + 4 * tid + u;
            int32_t id;
            if constexpr (kPrefetch) id = cid[4 * v + u];
            else id = id_of(i);
            if (staged) {
              st_i[p] = id;
              st_s[p] = key_score(kk);
            } else {
              out_i[p] = id;
              if (out_s) out_s[p] = key_score(kk);
            }
          }
        }
        gb += is_gt;
        eb += is_eq;
      }
    }
  }
  if (staged) {
    __syncthreads();
    for (int j = tid; j < k; j += NT) {
      const bool sel = j < k_eff;
      out_i[j] = sel ? st_i[j] : -1;
      if (out_s) out_s[j] = sel ? st_s[j] : __uint_as_float(kNoScoreBits);  // a NaN marks an empty slot
    }
  } else {
    for (int j = k_eff + tid; j < k; j += NT) {
      out_i[j] = -1;
      if (out_s) out_s[j] = __uint_as_float(kNoScoreBits);
    }
  }
}

}  // namespace csa
