/*
 * csa.h -- C ABI of the compressed sparse attention (CSA / HCA / CSA2) path
 * for AMD Instinct MI355X (gfx950).
 *
 * Pages this interface follows (cited by title, section and figure):
 *   [V4]   "DeepSeek-V4: エージェントが実際に使える100万トークンのコンテキスト"
 *          (DeepSeek-V4 blog post, Japanese translation), section
 *          "ハイブリッド注意：CSAとHCA", Fig. 3 (CSA) and Fig. 4 (HCA).
 *   [V4.1] "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression"
 *          (digest of the V4.1-Flash technical report), section
 *          "アーキテクチャ": CSA2 paragraph and Fig. 4 (Full / Reindex / Reuse
 *          modes), "FP4 主 KV キャッシュ" (MXFP4 main KV cache).
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every pointer argument is a DEVICE pointer owned by the caller, except
 *   the csa_cache_t struct itself, which is read on the host during the
 *   call and not kept.  The library keeps no pointer after it returns.
 * - Every call is asynchronous on `stream`, allocates nothing, never
 *   synchronises, and makes no HIP call before its host-side argument
 *   checks have passed; a failed check returns a negative csa_status and
 *   launches nothing.
 * - Channels: D = 576 = d_nope 512 (MXFP4) + d_rope 64 (bf16) per KV row.
 * - bf16 values are passed as their uint16 bit patterns; E4M3 and MXFP4
 *   data as bytes.
 * - A query at raw position p (0-based) sees compressed entry j when
 *   (j + 1) * m - 1 <= p and j < n_entries[b]; its sliding window is the raw
 *   rows at positions max(0, p - n_win + 1, swa_pos0[b]) .. p that the
 *   window buffer holds.
 * - Data-dependent problems (an index outside the visible range, a window
 *   row the buffer does not hold, ...) are skipped on the device, never
 *   trapped, and recorded as bits of a per-GPU device word that
 *   csa_read_device_flags returns (see there).
 * - The calls keep no host state between calls except, per GPU, the device
 *   address of that fault word, looked up on the first call on the GPU.
 */
#ifndef CSA_H_
#define CSA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CSA_OK = 0,
  CSA_ERR_NULL = -1,        /* a required pointer is NULL                       */
  CSA_ERR_SHAPE = -2,       /* sizes inconsistent with each other               */
  CSA_ERR_ALIGN = -3,       /* a plane or tensor is not 16-byte aligned         */
  CSA_ERR_UNSUPPORTED = -4, /* sizes outside the supported envelope             */
  CSA_ERR_WORKSPACE = -5,   /* workspace smaller than csa_workspace_bytes()     */
  CSA_ERR_HIP = -6,         /* a kernel launch failed (csa_last_hip_error())    */
  CSA_ERR_SCRATCH = -7      /* more than CSA_NOALLOC_SCRATCH_BYTES needed        */
} csa_status;

typedef enum { CSA_OUT_F32 = 0, CSA_OUT_BF16 = 1 } csa_out_dtype;

/* One compressed cache: one layer's, or one shared by CSA2 layers
 * ([V4.1] CSA2 paragraph: main KV and indexer K are shared across layers).
 * Plane layouts (row-major, one row per entry, N_cap rows per sequence):
 *   nope   uint8  [B][N_cap][d_nope/2]   E2M1 codes, channel 2i in the low nibble
 *   nscale uint8  [B][N_cap][d_nope/32]  E8M0 scale of channels 32s..32s+31
 *   rope   uint16 [B][N_cap][d_rope]     bf16
 *   ikey   uint8  [B][N_cap][d_idx/2]    indexer key, MXFP4 like nope
 *   iscale uint8  [B][N_cap][d_idx/32]
 * ikey/iscale may be NULL (HCA caches, d_idx = 0).
 * n_entries: int32 [B] on the device, entries valid per sequence. */
typedef struct {
  uint8_t *nope;
  uint8_t *nscale;
  uint16_t *rope;
  uint8_t *ikey;
  uint8_t *iscale;
  const int32_t *n_entries;
  int32_t B, N_cap, d_nope, d_rope, d_idx, m;
} csa_cache_t;

/* Compressor ([V4] CSA paragraph and Fig. 3: softmax-gated pooling with a
 * learned positional bias folds every m raw tokens into one entry; Fig. 4:
 * HCA uses m = 128; [V4.1] CSA2 paragraph: no overlap between entries, the
 * indexer key is a projection of the main entry).
 *
 * For sequence b and every entry j of the chunk, per channel d:
 *   c[d] = sum_i softmax_i(z[jm+i][d or 0] + pos_bias[i]) * x[jm+i][d]
 * then c[0:512] -> MXFP4 (scale X = floor(log2 max|v|) - 2 clamped to
 * [-127,127], elements rounded to nearest E2M1 with ties to even, saturated
 * at 6), c[512:576] -> bf16 (round to nearest even), and, when w_ik is not
 * NULL, kI = W_IK^T c (fp32) -> MXFP4.
 *
 *   x        bf16 [B][*][576]; row t of sequence b at x + b*x_stride_b + t*576,
 *            t = 0..T-1 holding raw positions tok_begin + t
 *   z        bf16 [B][*][G] gate logits, G = 576 (per channel) or 1, row
 *            stride G, sequence stride z_stride_b
 *   pos_bias fp32 [m]
 *   w_ik     bf16 [576][d_idx] or NULL (then ikey/iscale are not written)
 *   tok_begin, T: multiples of cache->m; entries tok_begin/m .. (tok_begin+T)/m - 1
 *            are written and must lie below N_cap.
 * n_entries is not modified: the caller publishes new entries. */
int csa_compress(const uint16_t *x, int64_t x_stride_b, const uint16_t *z, int64_t z_stride_b, int G,
                 const float *pos_bias, const uint16_t *w_ik, int64_t tok_begin, int64_t T,
                 const csa_cache_t *cache, hipStream_t stream);

/* The compressor fed from hidden states ([V4.1] "アーキテクチャ", CED
 * paragraph, eq. 1: a decoder layer's KV entries C^l, Z^l are projected
 * from the encoder's last hidden state by W^KV_l, W^Z_l), fused: the raw
 * rows x = H W^KV and the gate logits z = H W^Z are formed on the GPU's
 * matrix cores (fp32 sums of exact bf16 products) and pooled without being
 * written out; everything after is csa_compress (same planes, same
 * pooling, same quantisation).
 *   h        bf16 [B][*][d_model] hidden states, row stride d_model,
 *            sequence stride h_stride_b (>= T*d_model when B > 1, a
 *            multiple of 8); h row 0 of each sequence is token tok_begin
 *   d_model  a multiple of 32 in [32, 16384]
 *   w_kv     bf16 [d_model][576]     w_z  bf16 [d_model][G], G = 576 or 1
 *   pos_bias, w_ik, tok_begin, T, cache: as in csa_compress
 *   ws       >= csa_compress_hidden_ws_bytes(B, T, m, w_ik != NULL) bytes,
 *            16-byte aligned (the pooled fp32 rows, on their way to the
 *            indexer-key projection); NULL when that is 0.
 * h, w_kv, w_z 16-byte aligned.  n_entries is not modified. */
int csa_compress_hidden(const uint16_t *h, int64_t h_stride_b, int d_model, const uint16_t *w_kv,
                        const uint16_t *w_z, int G, const float *pos_bias, const uint16_t *w_ik, int64_t tok_begin,
                        int64_t T, const csa_cache_t *cache, void *ws, size_t ws_bytes, hipStream_t stream);
size_t csa_compress_hidden_ws_bytes(int B, int64_t T, int m, int with_ikey);

/* Lightning indexer + per-query top-k ([V4] CSA paragraph: FP4,
 * ReLU-scored multi-head dot product; top-k compressed blocks per query.
 * [V4.1] Fig. 4, Reindex mode: with `cand`, only an earlier layer's
 * selection is rescored).
 *
 *   score(j) = sum_h w_idx[h] * max(0, q_idx[h] . kI_j)   (fp32 accumulation
 *              of exact E4M3 x E2M1 products)
 *   idx_out  = the min(k, n) highest-scoring entries, exact ties to the lower
 *              entry index, ascending, padded with -1; n = visible entries
 *              (or visible, non-negative candidates)
 *
 *   q_idx    E4M3 [B][Q][H_I][d_idx] (unit scale)      w_idx fp32 [B][Q][H_I]
 *   q_pos    int32 [B][Q] raw positions
 *   cand     int32 [B][Q][C] ascending entry indices, -1 = none, no repeats;
 *            NULL for a full scan (C ignored)
 *   idx_out  int32 [B][Q][k]      score_out fp32 [B][Q][k] or NULL (NaN in padding)
 *   ws       >= csa_workspace_bytes(CSA_WS_INDEX_TOPK, ...) bytes, 256-byte aligned
 *            (fp32 scores of every scanned entry, then the top-k workspace).
 * A full scan of one to three queries per sequence (fewer than 256 rows)
 * over at most 32,768 entries selects from a histogram hint: the indexer
 * launch also counts each row's scores by the top 11 bits of their
 * order-preserving keys into the workspace; a compaction launch over
 * slices of 4,096 scores keeps the keys in the bin of the k-th largest
 * and above, and a final launch per row settles the selection among them
 * and leaves the counts zero.  The counts are checked against the scores
 * themselves, so any workspace contents give the same result; counts that
 * do not match (a workspace that was not zero on its first use) only make
 * that one call select from the whole row, more slowly. */
int csa_index_topk(const csa_cache_t *cache, const uint8_t *q_idx, const float *w_idx, int H_I,
                   const int32_t *q_pos, int Q, const int32_t *cand, int C, int k, int32_t *idx_out,
                   float *score_out, void *ws, size_t ws_bytes, hipStream_t stream);

/* csa_index_topk for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * arguments without the workspace, the same checks and the same results.
 * The workspace is a fixed device array of CSA_NOALLOC_SCRATCH_BYTES in the
 * library, one per GPU, held from the first call on that GPU until the
 * process ends; the call itself allocates nothing.  A call whose
 * csa_workspace_bytes(CSA_WS_INDEX_TOPK, ...) exceeds that size returns
 * CSA_ERR_SCRATCH and launches nothing (the batched 128K decode, 32 rows of
 * 32,768 entries at k = 512, needs 12.9 MB).  Every call on a GPU uses that
 * GPU's one array: calls that overlap on one GPU (other streams or host
 * threads) race and must be serialised by the caller. */
#define CSA_NOALLOC_SCRATCH_BYTES (16u << 20)
int csa_index_topk_noalloc(const csa_cache_t *cache, const uint8_t *q_idx, const float *w_idx, int H_I,
                           const int32_t *q_pos, int Q, const int32_t *cand, int C, int k, int32_t *idx_out,
                           float *score_out, hipStream_t stream);

/* The two stages of csa_index_topk as separate calls (same semantics):
 * csa_index_scores writes the score of every scanned entry into
 * scores fp32 [B][Q][Ns] (Ns = N_cap for a full scan, C with `cand`;
 * entries not visible at q_pos are left unwritten in a full scan, empty
 * candidate slots get the bit pattern 0xFFFFFFFF); csa_topk selects from
 * such a score array.  scores_bytes >= B*Q*Ns*4. */
int csa_index_scores(const csa_cache_t *cache, const uint8_t *q_idx, const float *w_idx, int H_I,
                     const int32_t *q_pos, int Q, const int32_t *cand, int C, float *scores, size_t scores_bytes,
                     hipStream_t stream);
int csa_topk(const csa_cache_t *cache, const float *scores, const int32_t *q_pos, int Q, const int32_t *cand,
             int C, int k, int32_t *idx_out, float *score_out, void *ws, size_t ws_bytes, hipStream_t stream);

/* csa_compress followed by a full-scan csa_index_scores (no candidates), the
 * decode append: the same arguments as those two calls, the same checks and
 * the same results (the cache bytes written and every score, bit for bit).
 * When every sequence appends one entry (T == m, m <= 8), there is one query
 * per sequence (Q == 1) and w_ik is given and 8-byte aligned, both run in
 * one launch: the new entry is compressed and scored while the older
 * entries are scored; other shapes run the two calls one after the other.  n_entries must already
 * count the appended entry for it to be visible to the query (the caller
 * publishes it before the call). */
int csa_compress_index_scores(const uint16_t *x, int64_t x_stride_b, const uint16_t *z, int64_t z_stride_b, int G,
                              const float *pos_bias, const uint16_t *w_ik, int64_t tok_begin, int64_t T,
                              const csa_cache_t *cache, const uint8_t *q_idx, const float *w_idx, int H_I,
                              const int32_t *q_pos, int Q, float *scores, size_t scores_bytes, hipStream_t stream);

/* The decode step's front half in two launches: csa_compress_index_scores
 * followed by the top-k of csa_index_topk (full scan, no candidates), with
 * the same arguments, checks and results.  ws is the workspace of
 * csa_index_topk (csa_workspace_bytes(CSA_WS_INDEX_TOPK, B, Q, k, N_cap, 0));
 * when the append fuses with the indexer (see csa_compress_index_scores)
 * and the top-k takes the hinted path (see csa_index_topk), the whole call
 * is three launches: append + indexer, compaction, final selection. */
int csa_compress_index_topk(const uint16_t *x, int64_t x_stride_b, const uint16_t *z, int64_t z_stride_b, int G,
                            const float *pos_bias, const uint16_t *w_ik, int64_t tok_begin, int64_t T,
                            const csa_cache_t *cache, const uint8_t *q_idx, const float *w_idx, int H_I,
                            const int32_t *q_pos, int Q, int k, int32_t *idx_out, float *score_out, void *ws,
                            size_t ws_bytes, hipStream_t stream);

/* Candidate pool of the hierarchical sparse indexer ([V4.1] "Hierarchical
 * Sparse Indexer" bullet and Fig. 5: the first Full layer ranks blocks of
 * consecutive positions by their largest indexer score and hands the
 * positions of the best blocks to the Reindex layers that follow).
 *
 * For each query row, from a full scan's scores:
 *   block score(b) = max of score(j) over the visible entries j of block b
 *                    (entries b*block .. b*block+block-1; blocks without a
 *                    visible entry take no part)
 *   kept           = the min(n_blocks, visible blocks) blocks of largest block
 *                    score, exact ties to the lower block
 *   pool_out       = every visible entry of the kept blocks, ascending, then -1
 *
 *   scores   fp32 [B][Q][N_cap] as csa_index_scores writes in a full scan
 *            (slots of entries not visible at q_pos are not read)
 *   q_pos    int32 [B][Q] raw positions
 *   block    entries per block, 1..64;  n_blocks >= 1, n_blocks*block <= 2^20
 *   pool_out int32 [B][Q][n_blocks*block]: the `cand` list (C = n_blocks*block)
 *            of csa_index_topk / csa_index_scores / csa_topk for a Reindex layer
 *   ws       >= csa_workspace_bytes(CSA_WS_INDEX_POOL, B, Q, n_blocks, N_cap,
 *            block) bytes, 16-byte aligned (block scores, the kept blocks and
 *            their top-k workspace); contents need not be initialised. */
int csa_index_pool(const csa_cache_t *cache, const float *scores, const int32_t *q_pos, int Q, int block,
                   int n_blocks, int32_t *pool_out, void *ws, size_t ws_bytes, hipStream_t stream);

/* Sparse attention over selected entries plus the sliding window ([V4]
 * Fig. 3).  One softmax over the union of the entries listed in idx and the
 * window rows; key = value = the decoded 576-channel row; no rotation is
 * applied to the rope channels.
 *
 *   q        bf16 [B][Q][H][576]         q_pos int32 [B][Q]
 *   idx      int32 [B][Q][k]; -1 and entries not visible at q_pos are skipped;
 *            a repeated index is attended once per occurrence (the list is
 *            expected ascending, as csa_index_topk writes it, but order does
 *            not change the result)
 *   swa      bf16 [B][S][576] raw rows, row r of sequence b = position swa_pos0[b] + r
 *   swa_pos0 int32 [B]                   n_win >= 0 (0 = no window branch)
 *   out      [B][Q][H][576] fp32 or bf16 (out_dtype)
 *   lse      fp32 [B][Q][H] natural-log sum of exp of the scaled logits, or NULL
 *   ws       >= csa_workspace_bytes(CSA_WS_SPARSE_ATTN, ...) bytes.
 *   rope_base  0: the 64 positional channels (576 - 64 .. 575) are used as
 *            stored.  > 0 (finite): the fused RoPE-attention-RoPE-cast
 *            epilogue ([V4.1] "推論カーネル": FlashMLA's fused kernel; [V4]
 *            CSA paragraph: those channels are kept in BF16).  Channel pair
 *            (2i, 2i+1) of the positional channels is turned by
 *            pos * rope_base^(-2i/64) radians, (x, y) -> (x cos - y sin,
 *            x sin + y cos): the query at its position q_pos, compressed
 *            entry j at its last raw token (j+1)*m - 1, a window row at its
 *            raw position; the rotated channels of q and of every key are
 *            rounded to bf16 before the products, each rotated key is also
 *            the value, and the output's positional channels are turned back
 *            by -q_pos before the cast to out_dtype.  The cache and the
 *            window rows hold the unrotated channels.  Negative, NaN or
 *            infinite rope_base: CSA_ERR_SHAPE. */
int csa_sparse_attn(const csa_cache_t *cache, const uint16_t *q, int H, const int32_t *q_pos, int Q,
                    const int32_t *idx, int k, const uint16_t *swa, const int32_t *swa_pos0, int S,
                    int n_win, float softmax_scale, float rope_base, int out_dtype, void *out, float *lse,
                    void *ws, size_t ws_bytes, hipStream_t stream);

/* Dense attention over every visible entry plus the window ([V4] Fig. 4,
 * HCA: no selection; the compressed stream is short).  Arguments as in
 * csa_sparse_attn without idx/k. */
int hca_dense_attn(const csa_cache_t *cache, const uint16_t *q, int H, const int32_t *q_pos, int Q,
                   const uint16_t *swa, const int32_t *swa_pos0, int S, int n_win, float softmax_scale,
                   float rope_base, int out_dtype, void *out, float *lse, void *ws, size_t ws_bytes,
                   hipStream_t stream);

/* FP8 window rows ([V4.1] "FP4 主 KV キャッシュ": the sliding-window KV stays
 * FP8, being sensitive to quantisation).  csa_swa_encode turns bf16 raw rows
 * into three planes, per row:
 *   codes   uint8  [B][S][512]  the content channels 0..511 as OCP MXFP8
 *                               E4M3 codes, one byte per channel
 *   scales  uint8  [B][S][16]   E8M0 byte of channels 32s..32s+31:
 *                               X = floor(log2 max|v|) - 8 clamped to
 *                               [-127, 127], byte X + 127 (0 for a zero block);
 *                               codes round v / 2^X to the nearest E4M3 value,
 *                               ties to even, saturate at 448, and keep the
 *                               sign of negative values
 *   rope    uint16 [B][S][64]   channels 512..575, the bf16 bits unchanged
 *   x       bf16 [B][S][576], row stride 576, sequence stride x_stride_b
 *           (>= S*576 when B > 1, a multiple of 8); x, codes and rope 16-byte
 *           aligned.
 * Decoding (E4M3 x 2^(s-127)) is exact in bf16 for every row it writes.
 * csa_sparse_attn_w8 and hca_dense_attn_w8 are csa_sparse_attn and
 * hca_dense_attn with the window rows read from such planes (same
 * positions: row s of sequence b is raw position swa_pos0[b] + s); every
 * other argument, the workspace and the results are as there. */
int csa_swa_encode(const uint16_t *x, int64_t x_stride_b, int B, int S, uint8_t *codes, uint8_t *scales,
                   uint16_t *rope, hipStream_t stream);
int csa_sparse_attn_w8(const csa_cache_t *cache, const uint16_t *q, int H, const int32_t *q_pos, int Q,
                       const int32_t *idx, int k, const uint8_t *swa_codes, const uint8_t *swa_scales,
                       const uint16_t *swa_rope, const int32_t *swa_pos0, int S, int n_win, float softmax_scale,
                       float rope_base, int out_dtype, void *out, float *lse, void *ws, size_t ws_bytes,
                       hipStream_t stream);
int hca_dense_attn_w8(const csa_cache_t *cache, const uint16_t *q, int H, const int32_t *q_pos, int Q,
                      const uint8_t *swa_codes, const uint8_t *swa_scales, const uint16_t *swa_rope,
                      const int32_t *swa_pos0, int S, int n_win, float softmax_scale, float rope_base,
                      int out_dtype, void *out, float *lse, void *ws, size_t ws_bytes, hipStream_t stream);

/* A stack of CSA2 layers for the same query tokens ([V4.1], CSA2 paragraph
 * and Fig. 4: every layer is statically Full, Reindex or Reuse; Fig. 5: the
 * first Full layer may build the hierarchical candidate pool).  The stack is
 * walked in order on `stream`:
 *   Full     scores every visible entry of its own `cache` with q_idx/w_idx,
 *            writes its top-k to idx_out, builds the pool into pool_out when
 *            pool_blocks > 0, and attends to its selection; it becomes the
 *            cache of the layers that follow and drops any earlier pool.
 *   Reindex  scores candidates of the latest Full layer's cache with its own
 *            q_idx/w_idx and writes its own top-k to idx_out; the candidates
 *            (`cand`): CSA2_CAND_POOL the latest Full layer's pool,
 *            CSA2_CAND_SELECTION the latest Full or Reindex layer's
 *            selection, CSA2_CAND_SCAN every visible entry, CSA2_CAND_AUTO the
 *            pool when the latest Full layer built one, else the selection.
 *   Reuse    attends to the latest Full or Reindex layer's selection on the
 *            latest Full layer's cache; no indexer work.
 * Every layer attends with its own q, window rows and output buffers, as in
 * csa_sparse_attn.  The first layer must be Full.  Layer fields that a mode
 * does not use are ignored.  All checks of every layer (those of the calls
 * named above plus the stack rules) run before the first launch. */
enum { CSA2_FULL = 0, CSA2_REINDEX = 1, CSA2_REUSE = 2 };
enum { CSA2_CAND_AUTO = 0, CSA2_CAND_SCAN = 1, CSA2_CAND_SELECTION = 2, CSA2_CAND_POOL = 3 };
typedef struct {
  int32_t mode;              /* CSA2_FULL, CSA2_REINDEX or CSA2_REUSE              */
  int32_t cand;              /* Reindex: CSA2_CAND_*                                 */
  const csa_cache_t *cache;  /* Full: this layer's cache                             */
  const uint8_t *q_idx;      /* Full, Reindex: E4M3 [B][Q][H_I][d_idx]               */
  const float *w_idx;        /* Full, Reindex: fp32 [B][Q][H_I]                      */
  int32_t H_I;
  int32_t k;                 /* Full, Reindex: entries selected (>= 1)              */
  int32_t pool_block;        /* Full: entries per pool block (when pool_blocks > 0)  */
  int32_t pool_blocks;       /* Full: blocks kept; 0 = no pool                       */
  int32_t *idx_out;          /* Full, Reindex: int32 [B][Q][k]                       */
  int32_t *pool_out;         /* Full with a pool: int32 [B][Q][pool_blocks*pool_block] */
  const uint16_t *q;         /* bf16 [B][Q][H][576]                                  */
  int32_t H;
  int32_t n_win;
  const uint16_t *swa;       /* bf16 window rows [B][S][576] from raw position swa_pos0[b] */
  const int32_t *swa_pos0;
  int32_t S;
  float softmax_scale;
  int32_t out_dtype;         /* CSA_OUT_F32 or CSA_OUT_BF16                          */
  void *out;                 /* [B][Q][H][576]                                       */
  float *lse;                /* fp32 [B][Q][H] or NULL                               */
  float rope_base;           /* 0, or the rotary base of the fused epilogue          */
} csa2_layer_t;

/*   n_layers  1..256
 *   q_pos  int32 [B][Q] raw positions, shared by every layer
 *   ws     >= csa2_stack_workspace_bytes(layers, n_layers, Q) bytes, 16-byte
 *          aligned, reused by each layer in turn. */
int csa2_layer_stack(const csa2_layer_t *layers, int n_layers, const int32_t *q_pos, int Q, void *ws,
                     size_t ws_bytes, hipStream_t stream);
/* Workspace of csa2_layer_stack; 0 when the stack is not valid. */
size_t csa2_stack_workspace_bytes(const csa2_layer_t *layers, int n_layers, int Q);

enum { CSA_WS_INDEX_TOPK = 0, CSA_WS_SPARSE_ATTN = 1, CSA_WS_DENSE_ATTN = 2, CSA_WS_TOPK = 3, CSA_WS_INDEX_POOL = 4 };

/* Workspace bytes for one call (0 = none needed).
 *   CSA_WS_INDEX_TOPK: H_or_k = k, n = N_cap, C = candidate count (0 for a
 *                      full scan); scores plus the top-k workspace.
 *   CSA_WS_TOPK:       H_or_k = k, n = scores per row (N_cap or C), C unused.
 *                      Rows with few siblings are selected in two launches
 *                      (per-slice candidates, then their top-k), which uses it.
 *   CSA_WS_INDEX_POOL: H_or_k = n_blocks, n = N_cap, C = block (0 when
 *                      block or n_blocks is outside the supported range).
 *   CSA_WS_SPARSE_ATTN / CSA_WS_DENSE_ATTN: H_or_k = query heads H, n = k
 *                      (sparse) or N_cap (dense), C = n_win. */
size_t csa_workspace_bytes(int op, int B, int Q, int H_or_k, int n, int C);

const char *csa_status_str(int status);
int csa_version(void);
/* hipError_t of the last CSA_ERR_HIP on this host thread. */
int csa_last_hip_error(void);

/* Data-dependent faults seen on the device ([V4] Fig. 3 fixes what is
 * attended: the selected entries a query can see plus its window rows;
 * inputs outside that are skipped, never trapped, and leave a bit here).
 * Kernels OR these bits into one word per GPU with vector-memory atomics:
 *   CSA_FLAG_IDX_RANGE  csa_sparse_attn*: a selected index outside
 *                       [-1, visible entries) (skipped; -1 is padding)
 *   CSA_FLAG_IDX_ORDER  csa_sparse_attn*: two neighbouring selected indices
 *                       (both >= 0) not strictly ascending, e.g. a repeat
 *                       (attended as given, once per occurrence)
 *   CSA_FLAG_WINDOW     attention: a query's window positions
 *                       max(0, p - n_win + 1) .. p not all held by the window
 *                       buffer (the missing rows are skipped)
 *   CSA_FLAG_CAND       indexer with `cand`: a candidate outside
 *                       [-1, visible entries) (skipped), or two neighbouring
 *                       candidates (both >= 0) not strictly ascending
 *   CSA_FLAG_ENTRIES    n_entries[b] outside [0, N_cap] (clamped)
 * csa_read_device_flags enqueues, on `stream`, an atomic exchange of the
 * current GPU's word with 0, copies the old value to *flags (host memory)
 * and waits for the stream: unlike every other call it synchronises.  Bits
 * set by work still running on other streams are reported by a later read.
 * Returns CSA_ERR_NULL for a null `flags`, CSA_ERR_HIP on a HIP failure. */
enum {
  CSA_FLAG_IDX_RANGE = 1,
  CSA_FLAG_IDX_ORDER = 2,
  CSA_FLAG_WINDOW = 4,
  CSA_FLAG_CAND = 8,
  CSA_FLAG_ENTRIES = 16
};
int csa_read_device_flags(hipStream_t stream, uint32_t *flags);

#ifdef __cplusplus
}
#endif
#endif /* CSA_H_ */
