// Candidate pool of the hierarchical sparse indexer ([V4.1] "Hierarchical
// Sparse Indexer" bullet and Fig. 5).  A Full layer's full-scan scores are
// reduced to one score per block of `block` consecutive entries (the
// maximum over the block's visible entries), the best `n_blocks` blocks are
// selected by the ordinary top-k launcher run over the block scores, and
// the visible entries of the kept blocks are written out, ascending, as the
// candidate list a Reindex layer rescores.
//
// The top-k launcher sees the block scores as a cache of Nb = ceil(N_cap /
// block) entries with m = 1: every sequence's entry count is Nb and each
// row's "position" is (visible blocks - 1), so its usual visibility rule,
// min(n_entries, position + 1), yields exactly the visible blocks.  Block
// scores are written for every block, the invisible ones with the no-score
// pattern.
#include "csa_device.hpp"
#include "csa_internal.hpp"

namespace csa {
namespace {

constexpr int kPoolThreads = 256;

size_t a256(size_t n) { return (n + 255) & ~(size_t)255; }

__device__ __forceinline__ int visible_entries(const int32_t *__restrict__ n_entries, int N_cap, int m,
                                               const int32_t *__restrict__ q_pos, int64_t row, int b) {
  const int nE = min(n_entries[b], N_cap);
  return max(0, min(nE, (q_pos[row] + 1) / m));
}

// One thread per block; the grid is flattened over (row, tile of blocks).
__global__ __launch_bounds__(kPoolThreads) void pool_blockmax_kernel(
    const float *__restrict__ scores, int N_cap, const int32_t *__restrict__ n_entries, int m,
    const int32_t *__restrict__ q_pos, int Q, int block, int Nb, int tiles, float *__restrict__ bscore,
    int32_t *__restrict__ vis_last, int32_t *__restrict__ nb_seq) {
  const int64_t row = blockIdx.x / tiles;
  const int tile = blockIdx.x - (int)(row * tiles);
  const int b = (int)(row / Q);
  const int V = visible_entries(n_entries, N_cap, m, q_pos, row, b);
  if (tile == 0 && threadIdx.x == 0) {
    vis_last[row] = (V + block - 1) / block - 1;
    if (row % Q == 0) nb_seq[b] = Nb;
  }
  const int blk = tile * kPoolThreads + threadIdx.x;
  if (blk >= Nb) return;
  const float *src = scores + row * (int64_t)N_cap;
  const int j0 = blk * block;
  const int j1 = min(j0 + block, V);
  float mx = __uint_as_float(kNoScoreBits);
  if (j0 < j1) {
    mx = src[j0];
    for (int j = j0 + 1; j < j1; ++j) mx = fmaxf(mx, src[j]);
  }
  bscore[row * (int64_t)Nb + blk] = mx;
}

// One thread per pool slot: slot t holds entry kept[t / block] * block +
// t % block when that block was kept and the entry is visible, else -1.
__global__ __launch_bounds__(kPoolThreads) void pool_expand_kernel(
    const int32_t *__restrict__ kept, int n_kept, int n_blocks, int block, const int32_t *__restrict__ n_entries,
    int N_cap, int m, const int32_t *__restrict__ q_pos, int Q, int tiles, int32_t *__restrict__ pool) {
  const int64_t row = blockIdx.x / tiles;
  const int t = (int)(blockIdx.x - row * tiles) * kPoolThreads + threadIdx.x;
  const int C = n_blocks * block;
  if (t >= C) return;
  const int b = (int)(row / Q);
  const int V = visible_entries(n_entries, N_cap, m, q_pos, row, b);
  const int slot = t / block;
  int out = -1;
  if (V > 0 && slot < n_kept) {
    const int kb = kept[row * (int64_t)n_kept + slot];
    const int j = kb * block + (t - slot * block);
    if (kb >= 0 && j < V) out = j;
  }
  pool[row * (int64_t)C + t] = out;
}

struct PoolLayout {
  int Nb, n_kept;
  size_t off_vis, off_nb, off_kept, off_topk, topk_bytes, total;
};

PoolLayout pool_layout(int B, int Q, int N_cap, int block, int n_blocks) {
  PoolLayout L;
  L.Nb = (N_cap + block - 1) / block;
  L.n_kept = n_blocks < L.Nb ? n_blocks : L.Nb;
  const size_t rows = (size_t)B * Q;
  L.off_vis = a256(rows * L.Nb * sizeof(float));
  L.off_nb = L.off_vis + a256(rows * sizeof(int32_t));
  L.off_kept = L.off_nb + a256((size_t)B * sizeof(int32_t));
  L.off_topk = L.off_kept + a256(rows * L.n_kept * sizeof(int32_t));
  L.topk_bytes = L.Nb > 0 && L.n_kept > 0 ? topk_plan(B, Q, L.Nb, L.n_kept).ws_bytes : 0;
  L.total = L.off_topk + L.topk_bytes;
  return L;
}

}  // namespace

size_t pool_workspace_bytes(int B, int Q, int N_cap, int block, int n_blocks) {
  if (B <= 0 || Q <= 0) return 0;
  return pool_layout(B, Q, N_cap, block, n_blocks).total;
}

hipError_t launch_index_pool(const CacheView &c, const float *scores, const int32_t *q_pos, int Q, int block,
                             int n_blocks, int32_t *pool, void *ws, hipStream_t stream) {
  const PoolLayout L = pool_layout(c.B, Q, c.N_cap, block, n_blocks);
  const int64_t rows = (int64_t)c.B * Q;
  char *w = reinterpret_cast<char *>(ws);
  float *bscore = reinterpret_cast<float *>(w);
  int32_t *vis_last = reinterpret_cast<int32_t *>(w + L.off_vis);
  int32_t *nb_seq = reinterpret_cast<int32_t *>(w + L.off_nb);
  int32_t *kept = reinterpret_cast<int32_t *>(w + L.off_kept);
  if (L.Nb > 0) {
    const int tiles = (L.Nb + kPoolThreads - 1) / kPoolThreads;
    pool_blockmax_kernel<<<(unsigned)(rows * tiles), kPoolThreads, 0, stream>>>(
        scores, c.N_cap, c.n_entries, c.m, q_pos, Q, block, L.Nb, tiles, bscore, vis_last, nb_seq);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    CacheView v = c;
    v.n_entries = nb_seq;
    v.N_cap = L.Nb;
    v.m = 1;
    e = launch_topk(v, bscore, L.Nb, vis_last, Q, nullptr, 0, L.n_kept, kept, nullptr,
                    L.topk_bytes ? w + L.off_topk : nullptr, stream);
    if (e != hipSuccess) return e;
  }
  const int C = n_blocks * block;
  const int tiles = (C + kPoolThreads - 1) / kPoolThreads;
  pool_expand_kernel<<<(unsigned)(rows * tiles), kPoolThreads, 0, stream>>>(
      kept, L.n_kept, n_blocks, block, c.n_entries, c.N_cap, c.m, q_pos, Q, tiles, pool);
  return hipGetLastError();
}

}  // namespace csa
