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
// digits, the number in the digit itself and the histogram total; when the
// total is below k_rem the digit is undefined.  Two barriers; uses
// sh[0 .. kW+3).  The histogram is read only before the first barrier, so a
// caller may rewrite it as soon as this returns.
template <int NT>
__device__ __forceinline__ void find_digit(const int (*hist)[kBins], int nh, int nb, int k_rem, int *sh, int &digit,
                                           int &above_out, int &count_out, int &total) {
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
      sh[kW + 2] = c[j];
    }
    above += c[j];
  }
  __syncthreads();
  // A later call writes sh only after its first barrier, which every thread
  // reaches after these reads.
  digit = __builtin_amdgcn_readfirstlane(sh[kW]);
  above_out = __builtin_amdgcn_readfirstlane(sh[kW + 1]);
  count_out = __builtin_amdgcn_readfirstlane(sh[kW + 2]);
  total = __builtin_amdgcn_readfirstlane(all);
}

// The waves rank the c1 (<= 64) keys gathered in bin_keys together: wave w
// compares every lane's key with keys w, w + NT/64, ..., the counts (keys
// greater, keys greater or equal; both below 2^16) meet in part (NT ints),
// and wave 0 publishes the exact threshold key (the k_rem-th largest of
// them), how many keys equal to it are taken and how many there are; every
// thread returns them.  Two barriers; uses sh[kW .. kW+3) and part, which
// no thread may read or write between the caller's last barrier and the
// return.
template <int NT>
__device__ __forceinline__ void rank_gathered(const uint32_t *bin_keys, int c1, int k_rem, int *sh, int *part,
                                              uint32_t &thr, int &need, int &n_eq) {
  constexpr int kW = NT / 64;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t kl = lane < c1 ? bin_keys[lane] : 0u;
  int gt = 0, ge = 0;
  for (int j = wave; j < c1; j += kW) {
    const uint32_t kj = (uint32_t)__builtin_amdgcn_readlane((int)kl, j);
    gt += kj > kl;
    ge += kj >= kl;
  }
  part[wave * 64 + lane] = gt | (ge << 16);
  __syncthreads();
  if (wave == 0) {
    int g = 0, e = 0;
#pragma unroll
    for (int w = 0; w < kW; ++w) {
      const int v = part[w * 64 + lane];
      g += v & 0xFFFF;
      e += v >> 16;
    }
    if (lane < c1 && g < k_rem && k_rem <= e) {  // every lane holding the threshold key agrees
      sh[kW] = (int)kl;
      sh[kW + 1] = k_rem - g;
      sh[kW + 2] = e - g;
    }
  }
  __syncthreads();
  thr = (uint32_t)__builtin_amdgcn_readfirstlane(sh[kW]);
  need = __builtin_amdgcn_readfirstlane(sh[kW + 1]);
  n_eq = __builtin_amdgcn_readfirstlane(sh[kW + 2]);
}

// Placement in ascending entry order, the last step of a selection by NT
// threads holding kPer keys each (key[4v + u] is element
// v*(4*NT) + 4*tid + u; key 0 marks an empty slot): the elements with
// key > thr, then the first `need` of the `n_eq` elements with key == thr
// (by entry), k_eff in all, as ids (cid, or id_of(element)) and scores,
// padded with -1 and kNoScoreBits up to k.  When every element equal to the
// threshold is taken the selection is simply key >= thr.  Per (slice, wave)
// ballots of "key > T" and "key == T", a scan of those counts by every wave,
// and in-wave ranks from masked popcounts.  Up to kStage selections are
// staged in LDS (st_i/st_s) and written out coalesced.  Two barriers;
// cnt holds 2 x (kPer/4)*(NT/64) ints.
template <int NT, int kPer, bool kPrefetch, int kStage, typename IdOf>
__device__ __forceinline__ void place_selected(const uint32_t (&key)[kPer], const int32_t (&cid)[kPrefetch ? kPer : 1],
                                               uint32_t thr, int need, int n_eq, int k_eff, int k, int *cnt,
                                               int32_t *st_i, float *st_s, int32_t *__restrict__ out_i,
                                               float *__restrict__ out_s, IdOf id_of, int n_live = 1 << 30) {
  constexpr int kW = NT / 64;
  constexpr int kV = kPer / 4;              // slices of 4*NT elements
  constexpr int kSlice = NT * 4;
  constexpr int kE = kV * kW;               // (slice, wave) pairs
  static_assert(kE <= 128, "a wave scans the (slice, wave) counts two per lane");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool staged = k_eff <= kStage;
  if (k_eff > 0) {
    // taken outright: key >= thr when simple, key > thr otherwise.  Each
    // case has loops of its own, so that a ballot takes one comparison.
    const bool simple = need == n_eq;
#pragma unroll
    for (int v = 0; v < kV; ++v) {
      int gc = 0, ec = 0;
      if (v * kSlice < n_live) {
        if (simple) {
#pragma unroll
          for (int u = 0; u < 4; ++u) gc += __popcll(__builtin_amdgcn_ballot_w64(key[4 * v + u] >= thr));
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            gc += __popcll(__builtin_amdgcn_ballot_w64(key[4 * v + u] > thr));
            ec += __popcll(__builtin_amdgcn_ballot_w64(key[4 * v + u] == thr));
          }
        }
      }
      if (lane == 0) {
        cnt[v * kW + wave] = gc;
        cnt[kE + v * kW + wave] = ec;
      }
    }
    __syncthreads();
    // every wave scans the counts in (slice, wave) order, two per lane
    int gx[2], ex[2] = {0, 0};
    {
      const int e0 = 2 * lane, e1 = 2 * lane + 1;
      const int g0 = e0 < kE ? cnt[e0] : 0, g1 = e1 < kE ? cnt[e1] : 0;
      const int gi = wave_incl_scan(g0 + g1);
      gx[0] = gi - g0 - g1;
      gx[1] = gi - g1;
      if (!simple) {
        const int q0 = e0 < kE ? cnt[kE + e0] : 0, q1 = e1 < kE ? cnt[kE + e1] : 0;
        const int qi = wave_incl_scan(q0 + q1);
        ex[0] = qi - q0 - q1;
        ex[1] = qi - q1;
      }
    }
    // staged selections keep their keys; the copy-out turns them into scores
    uint32_t *st_k = reinterpret_cast<uint32_t *>(st_s);
    auto put = [&](int p, int32_t id, uint32_t kk) __attribute__((always_inline)) {
      if (staged) {
        st_i[p] = id;
        st_k[p] = kk;
      } else {
        out_i[p] = id;
        if (out_s) out_s[p] = key_score(kk);
      }
    };
    if (simple) {
      // every key >= thr is taken, k_eff of them: no tie count, no bound test
#pragma unroll
      for (int v = 0; v < kV; ++v) {
        if (v * kSlice >= n_live) continue;  // a slice of empty slots selects nothing
        const int e = v * kW + wave;
        int gb = (e & 1) ? __builtin_amdgcn_readlane(gx[1], e >> 1) : __builtin_amdgcn_readlane(gx[0], e >> 1);
#pragma unroll
        for (int u = 0; u < 4; ++u) gb = lanes_below(__builtin_amdgcn_ballot_w64(key[4 * v + u] >= thr), gb);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t kk = key[4 * v + u];
          if (kk >= thr) {
            int32_t id;
            if constexpr (kPrefetch) id = cid[4 * v + u];
            else id = id_of(v * kSlice + 4 * tid + u);
            put(gb, id, kk);
            ++gb;
          }
        }
      }
    } else {
#pragma unroll
      for (int v = 0; v < kV; ++v) {
        if (v * kSlice >= n_live) continue;
        const int e = v * kW + wave;
        int gb = (e & 1) ? __builtin_amdgcn_readlane(gx[1], e >> 1) : __builtin_amdgcn_readlane(gx[0], e >> 1);
        int eb = (e & 1) ? __builtin_amdgcn_readlane(ex[1], e >> 1) : __builtin_amdgcn_readlane(ex[0], e >> 1);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          gb = lanes_below(__builtin_amdgcn_ballot_w64(key[4 * v + u] > thr), gb);
          eb = lanes_below(__builtin_amdgcn_ballot_w64(key[4 * v + u] == thr), eb);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t kk = key[4 * v + u];
          const bool is_gt = kk > thr, is_eq = kk == thr;
          if (is_gt || (is_eq && eb < need)) {
            const int p = gb + min(eb, need);
            if (p < k_eff) {
              int32_t id;
              if constexpr (kPrefetch) id = cid[4 * v + u];
              else id = id_of(v * kSlice + 4 * tid + u);
              put(p, id, kk);
            }
          }
          gb += is_gt;
          eb += is_eq;
        }
      }
    }
  }
  if (staged) {
    __syncthreads();
    const uint32_t *st_k = reinterpret_cast<const uint32_t *>(st_s);
    for (int j = tid; j < k; j += NT) {
      const bool sel = j < k_eff;
      out_i[j] = sel ? st_i[j] : -1;
      if (out_s) out_s[j] = sel ? key_score(st_k[j]) : __uint_as_float(kNoScoreBits);  // a NaN marks an empty slot
    }
  } else {
    for (int j = k_eff + tid; j < k; j += NT) {
      out_i[j] = -1;
      if (out_s) out_s[j] = __uint_as_float(kNoScoreBits);
    }
  }
}

// Exact threshold of a selection by NT threads holding kPer keys each (the
// layout of place_selected), on linear bins between the extremes: returns
// k_eff = min(k, valid keys), the full key thr of the k_eff-th largest
// element (1 when every valid key is taken), how many elements equal to
// thr are taken (need) and how many there are (n_eq).
//   1. row maximum, minimum and valid count;
//   2. histogram of 2,047 linear bins in score space between the extremes
//      (each key's bin kept in registers) and the bin holding the k-th
//      element;
//   3. when that bin holds at most 64 elements they are gathered (one LDS
//      atomic per wave) and every wave ranks them to fix the exact threshold
//      key T and how many elements equal to T are taken; otherwise radix
//      passes over the remaining bits do it.
// hist: kBins ints; sh: NT/64 + 3 ints; wred: 3 * NT/64 ints; bin_keys: 64.
template <int NT, int kPer>
__device__ __forceinline__ void linear_threshold(const uint32_t (&key)[kPer], int k, int *hist, int *sh, int *wred,
                                                 uint32_t *bin_keys, int *n_bin, int &k_eff_out, uint32_t &thr_out,
                                                 int &need_out, int &n_eq_out, int n_live = 1 << 30) {
  constexpr int kW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // key j lies in a slice of 4*NT elements that may start past n_live, the
  // bound beyond which every slot is empty: such slices are skipped whole
  auto live = [&](int j) { return (j >> 2) * (4 * NT) < n_live; };
  int (*hist2)[kBins] = reinterpret_cast<int (*)[kBins]>(hist);
  for (int i = tid; i < kBins; i += NT) hist[i] = 0;
  if (tid == 0) *n_bin = 0;
  uint32_t *wmax = reinterpret_cast<uint32_t *>(wred), *wmin = wmax + kW;
  int *wcnt = wred + 2 * kW;

  // 1. maximum, minimum and count of the valid keys (the count from the
  //    ballots of the validity test, on the scalar unit)
  {
    uint32_t mx = 0, mn = 0xFFFFFFFFu;
    int nv = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if (!live(j)) continue;
      const bool valid = key[j] != 0u;
      mx = key[j] > mx ? key[j] : mx;
      const uint32_t c = valid ? key[j] : 0xFFFFFFFFu;
      mn = c < mn ? c : mn;
      nv += __popcll(__builtin_amdgcn_ballot_w64(valid));
    }
    mx = wave_max_u32(mx);
    const uint32_t mnc = wave_max_u32(~mn);  // complement of the minimum (0: no valid key)
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
      if (!live(j)) {
        binp[j >> 1] = 0xFFFFFFFFu;
        continue;
      }
      const uint32_t bj = key[j] != 0u ? bin_of(key[j]) : 0xFFFFu;
      if (j & 1) binp[j >> 1] |= bj << 16;
      else binp[j >> 1] = bj;
      if (key[j] != 0u) atomicAdd(&hist[kBins - 2 - bj], 1);
    }
    __syncthreads();
    // (the bin's count comes from find_digit: a read of hist[d1] here would
    // race with the zeroing of the crowded-bin passes below)
    int d1, above, c1, tot;
    find_digit<NT>(hist2, 1, kBins, k_eff, sh, d1, above, c1, tot);
    const uint32_t dhi = (uint32_t)(kBins - 2 - d1);
    auto in_dhi = [&](int j) { return live(j) && ((binp[j >> 1] >> (16 * (j & 1))) & 0xFFFFu) == dhi; };
    int k_rem = k_eff - above;
    if (c1 <= 64) {
      // 2a. gather the threshold bin and rank it.  One pass: a ballot per
      //     key, and on the rare non-empty one an LDS atomic reserves its
      //     slots, each key going to its ballot's lanes below it.
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        if (!live(j)) continue;  // uniform: the ballot takes the comparison itself
        const bool in = ((binp[j >> 1] >> (16 * (j & 1))) & 0xFFFFu) == dhi;
        const uint64_t mk = __builtin_amdgcn_ballot_w64(in);
        if (mk) {
          int pos = 0;
          if (lane == 0) pos = atomicAdd(n_bin, (int)__popcll(mk));
          pos = __builtin_amdgcn_readfirstlane(pos);
          if (in) bin_keys[lanes_below(mk, pos)] = key[j];
        }
      }
      __syncthreads();
      rank_gathered<NT>(bin_keys, c1, k_rem, sh, hist, thr, need, n_eq);  // the histogram is free now
    } else {
      // 2b. a crowded bin (many equal or nearly equal scores): radix passes
      //     over the keys of that bin, bits 31..21, 20..10 and 9..0
      for (int i = tid; i < kBins; i += NT) hist[i] = 0;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if (in_dhi(j)) atomicAdd(&hist[key[j] >> 21], 1);
      __syncthreads();
      int e1, ab, ce;
      find_digit<NT>(hist2, 1, kBins, k_rem, sh, e1, ab, ce, tot);
      k_rem -= ab;
      for (int i = tid; i < kBins; i += NT) hist[i] = 0;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if (in_dhi(j) && (key[j] >> 21) == (uint32_t)e1) atomicAdd(&hist[(key[j] >> 10) & 0x7FFu], 1);
      __syncthreads();
      int e2;
      find_digit<NT>(hist2, 1, kBins, k_rem, sh, e2, ab, ce, tot);
      k_rem -= ab;
      const uint32_t p12 = ((uint32_t)e1 << 11) | (uint32_t)e2;
      for (int i = tid; i < kBins; i += NT) hist[i] = 0;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if (in_dhi(j) && (key[j] >> 10) == p12) atomicAdd(&hist[key[j] & 0x3FFu], 1);
      __syncthreads();
      int e3;
      find_digit<NT>(hist2, 1, 1024, k_rem, sh, e3, ab, n_eq, tot);  // every key equal to thr lies in bin e3
      k_rem -= ab;
      thr = (p12 << 10) | (uint32_t)e3;
      need = k_rem;
    }
  }
  k_eff_out = k_eff;
  thr_out = thr;
  need_out = need;
  n_eq_out = n_eq;
}

// Selects, among the keys held in registers by the kRegThreads threads of
// the workgroup (key[4v + u] is element v*(4*kRegThreads) + 4*tid + u; key 0
// marks an empty slot), the k largest, exact ties to the lower element, and
// writes their ids (cid, or id_of(element)) and scores in ascending element
// order to out_i / out_s, padding with -1 and kNoScoreBits up to k: the
// linear-bin threshold, then the placement.  Cross-lane work runs on DPP
// and readlane, and small scans are repeated by every wave rather than
// published through a further barrier.
template <int kPer, bool kPrefetch, typename IdOf>
__device__ __forceinline__ void select_keys(uint32_t (&key)[kPer], const int32_t (&cid)[kPrefetch ? kPer : 1], int k,
                                            int32_t *__restrict__ out_i, float *__restrict__ out_s, IdOf id_of,
                                            int n_live = 1 << 30) {
  constexpr int NT = kRegThreads;
  constexpr int kW = NT / 64;
  constexpr int kE = (kPer / 4) * kW;
  // the histogram area doubles as the staging area of the placement, sized
  // for selections of up to 2,048 (larger ones are written out directly):
  // 16 KB, so that three workgroups of 512 threads share a CU
  constexpr int kStage = 2048;
  __shared__ int hist[kBins > 2 * kStage ? kBins : 2 * kStage];
  __shared__ int sh[kW + 3];
  __shared__ int wred[3 * kW];
  __shared__ uint32_t bin_keys[64];
  __shared__ int cnt[2 * kE];
  __shared__ int n_bin;
  int k_eff, need, n_eq;
  uint32_t thr;
  linear_threshold<NT, kPer>(key, k, hist, sh, wred, bin_keys, &n_bin, k_eff, thr, need, n_eq, n_live);
  // the histogram's last reads precede the placement's first barrier
  place_selected<NT, kPer, kPrefetch, kStage>(key, cid, thr, need, n_eq, k_eff, k, cnt, hist,
                                              reinterpret_cast<float *>(hist + kStage), out_i, out_s, id_of, n_live);
}

}  // namespace csa
