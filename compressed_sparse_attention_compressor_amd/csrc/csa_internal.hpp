// Host-side launchers shared between the kernel translation units and the
// C ABI (abi.hip).  Arguments are validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa {

struct CacheView {
  uint8_t *nope;
  uint8_t *nscale;
  uint16_t *rope;
  uint8_t *ikey;
  uint8_t *iscale;
  const int32_t *n_entries;
  int B, N_cap, d_idx, m;
  uint32_t *flags;  // device word of data-dependent faults (kFault* bits); may be null
};

hipError_t launch_compress(const uint16_t *x, int64_t x_stride_b, const uint16_t *z, int64_t z_stride_b,
                           int G, const float *bias, const uint16_t *w_ik, int64_t entry0, int n_chunk_entries,
                           const CacheView &c, hipStream_t stream);

// Scores of every scanned entry (full scan: [B][Q][N_cap], candidates:
// [B][Q][C]) into `scores`; slots without a candidate get kNoScoreBits.
// hint: null, or kHintBins uint32 per row (zero on entry) that a one-query
// full scan (Q < 4) fills with the row's score histogram for
// launch_topk_hint; other shapes leave it untouched.
// zero / zero_bytes: null, or 16-byte-aligned bytes (a multiple of 16) that
// the same launch clears for the next one; only the shapes index_can_zero()
// accepts (others return hipErrorInvalidValue and launch nothing).
bool index_can_zero(int Q, bool cand);
hipError_t launch_index_scores(const CacheView &c, const uint8_t *q_idx, const float *w_idx, int H_I,
                               const int32_t *q_pos, int Q, const int32_t *cand, int C, float *scores,
                               hipStream_t stream, uint32_t *hint = nullptr, void *zero = nullptr,
                               size_t zero_bytes = 0);

// Decode append fused with the indexer: csa_compress of one entry per
// sequence (entry `entry`, from rows 0..m-1 of the x/z chunk) followed by
// a full-scan csa_index_scores of one query per sequence, in
// one launch, with identical results.  Only for the shapes
// append_index_fusable() accepts.
bool append_index_fusable(int m, int64_t T, int Q, int G, const uint16_t *w_ik, int B);
hipError_t launch_append_index(const uint16_t *x, int64_t x_stride_b, const uint16_t *z, int64_t z_stride_b, int G,
                               const float *bias, const uint16_t *w_ik, int64_t entry, const CacheView &c,
                               const uint8_t *q_idx, const float *w_idx, int H_I, const int32_t *q_pos,
                               float *scores, hipStream_t stream, uint32_t *hint = nullptr);

// Top-k plan: rows with few siblings are split into `nsl` slices of S
// scores whose own top-k candidates (ws_bytes of workspace) are reduced in
// a second launch.  nsl = 1: one workgroup per row.
struct TopkPlan {
  int nsl;          // slices per row (1: one workgroup per row)
  int S;            // elements per slice
  size_t ws_bytes;  // workspace needed
  bool radix = false;  // multi-workgroup radix selection (few, long rows)
};
TopkPlan topk_plan(int B, int Q, int Ns, int k);
// Bytes at the start of a radix plan's workspace that must be zero when
// its selection starts (0 for other plans).
size_t topk_radix_zero_bytes(int B, int Q, int Ns, int k);

// prezeroed: the first topk_radix_zero_bytes() of ws are already zero (an
// earlier launch on the stream cleared them), so the radix selection skips
// its clearing launch.
hipError_t launch_topk(const CacheView &c, const float *scores, int Ns, const int32_t *q_pos, int Q,
                       const int32_t *cand, int C, int k, int32_t *idx_out, float *score_out, void *ws,
                       hipStream_t stream, bool prezeroed = false);

// Top-k of full-scan rows from their scores and the indexer's histogram
// hint, for the shapes topk_hint_fits() accepts (few rows of at most 32,768
// scores).  ws (topk_hint_ws_bytes) starts with the hint, kHintBins uint32
// per row, which the indexer launch filled and this call leaves zero; the
// rest holds the compacted candidates.
bool topk_hint_fits(int B, int Q, int Ns, int k);
size_t topk_hint_ws_bytes(int B, int Q, int Ns);
hipError_t launch_topk_hint(const CacheView &c, const float *scores, int Ns, const int32_t *q_pos, int Q, int k,
                            int32_t *idx_out, float *score_out, void *ws, hipStream_t stream);

// Hierarchical indexer pool: block maxima of full-scan scores, the best
// n_blocks blocks, and their visible entries as a candidate list
// [B][Q][n_blocks * block].
size_t pool_workspace_bytes(int B, int Q, int N_cap, int block, int n_blocks);
hipError_t launch_index_pool(const CacheView &c, const float *scores, const int32_t *q_pos, int Q, int block,
                             int n_blocks, int32_t *pool, void *ws, hipStream_t stream);

// FP8 window rows: bf16 rows [B][S][576] (row stride 576, sequence stride
// x_stride_b) -> codes [B][S][512], scales [B][S][16], rope [B][S][64].
hipError_t launch_swa_encode(const uint16_t *x, int64_t x_stride_b, int B, int S, uint8_t *codes, uint8_t *scales,
                             uint16_t *rope, hipStream_t stream);
// The planes of FP8 window rows for the attention (nullptr: bf16 rows).
struct SwaPlanes {
  const uint8_t *codes;
  const uint8_t *scales;
  const uint16_t *rope;
};

struct AttnShape {
  int nsplit;       // key-range splits per query
  int per_split;    // key slots per split (a multiple of the chunk size)
};
// n_main: selected entries per query (k), or N_cap for dense attention.
AttnShape attn_shape(int B, int Q, int n_main, int n_win);
size_t attn_workspace_bytes(int B, int Q, int H, int n_main, int n_win);

// Hidden-state compressor (compress_hidden.hip): H W^KV and H W^Z pooled
// without leaving the chip; with w_ik the pooled rows pass through `ws`
// (compress_hidden_ws_bytes) to the indexer-key projection.
size_t compress_hidden_ws_bytes(int B, int n_ent, bool has_ik);
hipError_t launch_compress_hidden(const uint16_t *h, int64_t h_stride_b, int d_model, const uint16_t *w_kv,
                                  const uint16_t *w_z, int G, const float *bias, const uint16_t *w_ik,
                                  int64_t entry0, int n_ent, const CacheView &c, void *ws, hipStream_t stream);
hipError_t launch_ikey_from_pooled(const float *pooled, const uint16_t *w_ik, int64_t entry0, int n_chunk,
                                   const CacheView &c, hipStream_t stream);

hipError_t launch_attention(const CacheView &c, const uint16_t *q, int H, const int32_t *q_pos, int Q,
                            const int32_t *idx, int k, bool dense, const uint16_t *swa, const SwaPlanes *swa8,
                            const int32_t *swa_pos0, int S, int n_win, float scale, double rope_base,
                            bool out_bf16, void *out, float *lse, void *ws, hipStream_t stream);

}  // namespace csa
