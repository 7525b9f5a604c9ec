// C ABI of the CSA library: argument checks on the host, then launches.
// No HIP call is made before every check has passed.
#include <math.h>

#include <atomic>
#include <mutex>

#include "../../include/csa.h"
#include "csa_device.hpp"
#include "csa_internal.hpp"

// The device word of data-dependent faults (CSA_FLAG_* bits), one per GPU,
// and the word csa_read_device_flags exchanges it into.
__device__ uint32_t g_fault_word;
__device__ uint32_t g_fault_taken;

__global__ void take_fault_word_kernel(uint32_t *word, uint32_t *taken) { *taken = atomicExch(word, 0u); }

// Fixed scratch of csa_index_topk_noalloc, one copy per GPU, held until the
// process ends.  Host code never passes this name to a kernel (on the host
// it is only a stand-in): the device address comes from hipGetSymbolAddress,
// looked up once per device.
static __device__ __align__(256) uint8_t scratch[CSA_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local int g_last_hip_error = 0;

constexpr int kMaxDevices = 64;
std::atomic<uint32_t *> g_word_ptr[kMaxDevices];
std::atomic<uint32_t *> g_taken_ptr[kMaxDevices];
std::mutex g_word_mu;

// Device addresses of the two words on the current device, looked up once
// per device (the host-side names are not device addresses).
hipError_t fault_words(uint32_t **word, uint32_t **taken) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  uint32_t *w = g_word_ptr[dev].load(std::memory_order_acquire);
  if (!w) {
    std::lock_guard<std::mutex> lock(g_word_mu);
    w = g_word_ptr[dev].load(std::memory_order_acquire);
    if (!w) {
      uint32_t *t = nullptr;
      e = hipGetSymbolAddress(reinterpret_cast<void **>(&w), HIP_SYMBOL(g_fault_word));
      if (e == hipSuccess) e = hipGetSymbolAddress(reinterpret_cast<void **>(&t), HIP_SYMBOL(g_fault_taken));
      if (e != hipSuccess) return e;
      g_taken_ptr[dev].store(t, std::memory_order_release);
      g_word_ptr[dev].store(w, std::memory_order_release);
    }
  }
  *word = w;
  if (taken) *taken = g_taken_ptr[dev].load(std::memory_order_acquire);
  return hipSuccess;
}

std::atomic<void *> g_scratch_ptr[kMaxDevices];

// Device address of this GPU's scratch (the current device's), looked up on
// the first call on the device.
hipError_t scratch_address(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_word_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

// The fault word for the kernels (null when it cannot be found: faults then
// go unrecorded, results are unchanged).
uint32_t *fault_word() {
  uint32_t *w = nullptr;
  return fault_words(&w, nullptr) == hipSuccess ? w : nullptr;
}

constexpr int kMaxH = 128;
constexpr int kMaxHI = 64;
constexpr int kMaxM = 256;
constexpr int kMaxK = 1 << 20;
constexpr int kMaxWin = 1 << 20;
constexpr int kMaxPoolBlock = 64;
constexpr int kMaxStackLayers = 256;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int status_of(hipError_t e) {
  if (e == hipSuccess) return CSA_OK;
  g_last_hip_error = (int)e;
  return CSA_ERR_HIP;
}

// Checks shared by every call that reads a cache.
int check_cache(const csa_cache_t *c, bool need_ikey) {
  if (!c) return CSA_ERR_NULL;
  if (!c->nope || !c->nscale || !c->rope || !c->n_entries) return CSA_ERR_NULL;
  if (need_ikey && (!c->ikey || !c->iscale)) return CSA_ERR_NULL;
  if (c->B < 0 || c->N_cap < 0) return CSA_ERR_SHAPE;
  if (c->d_nope != csa::kDNope || c->d_rope != csa::kDRope) return CSA_ERR_UNSUPPORTED;
  if (c->m < 1 || c->m > kMaxM) return CSA_ERR_UNSUPPORTED;
  if (need_ikey && c->d_idx != 64 && c->d_idx != 128) return CSA_ERR_UNSUPPORTED;
  if (c->d_idx != 0 && c->d_idx != 64 && c->d_idx != 128) return CSA_ERR_UNSUPPORTED;
  if (!aligned16(c->nope) || !aligned16(c->nscale) || !aligned16(c->rope)) return CSA_ERR_ALIGN;
  if (c->ikey && (!aligned16(c->ikey) || !aligned16(c->iscale))) return CSA_ERR_ALIGN;
  return CSA_OK;
}

csa::CacheView view_of(const csa_cache_t *c) {
  csa::CacheView v;
  v.nope = c->nope;
  v.nscale = c->nscale;
  v.rope = c->rope;
  v.ikey = c->ikey;
  v.iscale = c->iscale;
  v.n_entries = c->n_entries;
  v.B = c->B;
  v.N_cap = c->N_cap;
  v.d_idx = c->d_idx;
  v.m = c->m;
  v.flags = fault_word();
  return v;
}

size_t index_ws_bytes(int B, int Q, int N_cap, int C) {
  const int Ns = C > 0 ? C : N_cap;
  return (size_t)B * Q * Ns * sizeof(float);
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// Top-k workspace; candidate rows are selected in one launch.
size_t topk_ws_bytes(int B, int Q, int Ns, int k, bool cand) {
  if (cand) return 0;
  return csa::topk_plan(B, Q, Ns, k).ws_bytes;
}

// Full scans of one query per workgroup (Q < 4) of at most 32,768 entries
// select in one launch from the scores and the indexer's histogram hint.
bool hint_path(int B, int Q, int N_cap, int k, bool cand) {
  return !cand && Q > 0 && Q < 4 && csa::topk_hint_fits(B, Q, N_cap, k);
}

// Workspace of csa_index_topk: the scores, then the hinted top-k's (the
// hint first) or the top-k's own.
size_t index_topk_ws_bytes(int B, int Q, int N_cap, int k, int C, bool cand) {
  const size_t s = align256(index_ws_bytes(B, Q, N_cap, cand ? C : 0));
  if (hint_path(B, Q, N_cap, k, cand)) return s + csa::topk_hint_ws_bytes(B, Q, N_cap);
  return s + topk_ws_bytes(B, Q, cand ? C : N_cap, k, cand);
}

int check_attn_common(const csa_cache_t *cache, const uint16_t *q, int H, const int32_t *q_pos, int Q,
                      const uint16_t *swa, const int32_t *swa_pos0, int S, int n_win, float scale,
                      float rope_base, int out_dtype, void *out) {
  int st = check_cache(cache, false);
  if (st) return st;
  if (!q || !q_pos || !out) return CSA_ERR_NULL;
  if (Q < 0 || S < 0 || n_win < 0) return CSA_ERR_SHAPE;
  if (n_win > 0 && (!swa || !swa_pos0)) return CSA_ERR_NULL;
  if (H < 16 || H > kMaxH || (H != 16 && H != 32 && H != 64 && H != 128)) return CSA_ERR_UNSUPPORTED;
  if (n_win > kMaxWin) return CSA_ERR_UNSUPPORTED;
  if (out_dtype != CSA_OUT_F32 && out_dtype != CSA_OUT_BF16) return CSA_ERR_UNSUPPORTED;
  if (!(scale == scale) || isinf(scale)) return CSA_ERR_SHAPE;
  if (!(rope_base >= 0.f) || isinf(rope_base)) return CSA_ERR_SHAPE;  // NaN fails the comparison
  if (!aligned16(q) || !aligned16(out) || (n_win > 0 && !aligned16(swa))) return CSA_ERR_ALIGN;
  return CSA_OK;
}

}  // namespace

extern "C" {

int csa_version(void) { return 10200; }

int csa_read_device_flags(hipStream_t stream, uint32_t *flags) {
  if (!flags) return CSA_ERR_NULL;
  uint32_t *word = nullptr, *taken = nullptr;
  hipError_t e = fault_words(&word, &taken);
  if (e != hipSuccess) return status_of(e);
  take_fault_word_kernel<<<1, 1, 0, stream>>>(word, taken);
  e = hipGetLastError();
  uint32_t v = 0;
  if (e == hipSuccess) e = hipMemcpyAsync(&v, taken, sizeof(v), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return status_of(e);
  *flags = v;
  return CSA_OK;
}

int csa_last_hip_error(void) { return g_last_hip_error; }

const char *csa_status_str(int status) {
  switch (status) {
    case CSA_OK: return "ok";
    case CSA_ERR_NULL: return "a required pointer is NULL";
    case CSA_ERR_SHAPE: return "inconsistent sizes";
    case CSA_ERR_ALIGN: return "a buffer is not 16-byte aligned";
    case CSA_ERR_UNSUPPORTED: return "sizes outside the supported envelope";
    case CSA_ERR_WORKSPACE: return "workspace too small";
    case CSA_ERR_HIP: return "HIP launch failure";
    case CSA_ERR_SCRATCH: return "the call needs more than the fixed scratch of the allocation-free entry point";
    default: return "unknown status";
  }
}

size_t csa_workspace_bytes(int op, int B, int Q, int H_or_k, int n, int C) {
  if (B <= 0 || Q <= 0) return 0;
  switch (op) {
    case CSA_WS_INDEX_TOPK: return index_topk_ws_bytes(B, Q, n, H_or_k, C, C > 0);
    case CSA_WS_TOPK: return topk_ws_bytes(B, Q, n, H_or_k, false);
    case CSA_WS_INDEX_POOL:
      if (C < 1 || C > kMaxPoolBlock || H_or_k < 1 || n < 0) return 0;
      return csa::pool_workspace_bytes(B, Q, n, C, H_or_k);
    case CSA_WS_SPARSE_ATTN:
    case CSA_WS_DENSE_ATTN: return csa::attn_workspace_bytes(B, Q, H_or_k, n, C > 0 ? C : 0);
    default: return 0;
  }
}

static int check_compress_args(const uint16_t *x, int64_t x_stride_b, const uint16_t *z, int64_t z_stride_b, int G,
                               const float *pos_bias, const uint16_t *w_ik, int64_t tok_begin, int64_t T,
                               const csa_cache_t *cache) {
  int st = check_cache(cache, w_ik != nullptr);
  if (st) return st;
  if (!x || !z || !pos_bias) return CSA_ERR_NULL;
  if (G != 1 && G != csa::kD) return CSA_ERR_UNSUPPORTED;
  if (T < 0 || tok_begin < 0) return CSA_ERR_SHAPE;
  if (tok_begin % cache->m || T % cache->m) return CSA_ERR_SHAPE;
  if ((tok_begin + T) / cache->m > cache->N_cap) return CSA_ERR_SHAPE;
  if (cache->B > 1 && (x_stride_b < T * csa::kD || z_stride_b < T * G)) return CSA_ERR_SHAPE;
  if (!aligned16(x) || (G == csa::kD && !aligned16(z))) return CSA_ERR_ALIGN;
  if (G == csa::kD && (z_stride_b % 4)) return CSA_ERR_ALIGN;
  if (x_stride_b % 4) return CSA_ERR_ALIGN;
  return CSA_OK;
}

int csa_compress(const uint16_t *x, int64_t x_stride_b, const uint16_t *z, int64_t z_stride_b, int G,
                 const float *pos_bias, const uint16_t *w_ik, int64_t tok_begin, int64_t T,
                 const csa_cache_t *cache, hipStream_t stream) {
  int st = check_compress_args(x, x_stride_b, z, z_stride_b, G, pos_bias, w_ik, tok_begin, T, cache);
  if (st) return st;
  if (T == 0 || cache->B == 0) return CSA_OK;
  const csa::CacheView v = view_of(cache);
  return status_of(csa::launch_compress(x, x_stride_b, z, z_stride_b, G, pos_bias, w_ik, tok_begin / cache->m,
                                        (int)(T / cache->m), v, stream));
}

static int check_hidden_args(const uint16_t *h, int64_t h_stride_b, int d_model, const uint16_t *w_kv,
                             const uint16_t *w_z, int G, const float *pos_bias, const uint16_t *w_ik, int64_t tok_begin,
                             int64_t T, const csa_cache_t *cache) {
  int st = check_cache(cache, w_ik != nullptr);
  if (st) return st;
  if (!h || !w_kv || !w_z || !pos_bias) return CSA_ERR_NULL;
  if (G != 1 && G != csa::kD) return CSA_ERR_UNSUPPORTED;
  if (d_model < 32 || d_model > 16384 || d_model % 32) return CSA_ERR_UNSUPPORTED;
  if (T < 0 || tok_begin < 0) return CSA_ERR_SHAPE;
  if (tok_begin % cache->m || T % cache->m) return CSA_ERR_SHAPE;
  if ((tok_begin + T) / cache->m > cache->N_cap) return CSA_ERR_SHAPE;
  if (cache->B > 1 && h_stride_b < T * d_model) return CSA_ERR_SHAPE;
  if (!aligned16(h) || !aligned16(w_kv) || !aligned16(w_z) || (h_stride_b % 8)) return CSA_ERR_ALIGN;
  return CSA_OK;
}

size_t csa_compress_hidden_ws_bytes(int B, int64_t T, int m, int with_ikey) {
  if (B < 0 || T < 0 || m < 1) return 0;
  return csa::compress_hidden_ws_bytes(B, (int)(T / m), with_ikey != 0);
}

int csa_compress_hidden(const uint16_t *h, int64_t h_stride_b, int d_model, const uint16_t *w_kv,
                        const uint16_t *w_z, int G, const float *pos_bias, const uint16_t *w_ik, int64_t tok_begin,
                        int64_t T, const csa_cache_t *cache, void *ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_hidden_args(h, h_stride_b, d_model, w_kv, w_z, G, pos_bias, w_ik, tok_begin, T, cache);
  if (st) return st;
  if (T == 0 || cache->B == 0) return CSA_OK;
  const size_t need = csa::compress_hidden_ws_bytes(cache->B, (int)(T / cache->m), w_ik != nullptr);
  if (need > 0 && !ws) return CSA_ERR_NULL;
  if (ws_bytes < need) return CSA_ERR_WORKSPACE;
  if (need > 0 && !aligned16(ws)) return CSA_ERR_ALIGN;
  const csa::CacheView v = view_of(cache);
  return status_of(csa::launch_compress_hidden(h, h_stride_b, d_model, w_kv, w_z, G, pos_bias, w_ik,
                                               tok_begin / cache->m, (int)(T / cache->m), v, ws, stream));
}

static int check_index_args(const csa_cache_t *cache, const uint8_t *q_idx, const float *w_idx, int H_I,
                            const int32_t *q_pos, int Q, const int32_t *cand, int C) {
  int st = check_cache(cache, true);
  if (st) return st;
  if (!q_idx || !w_idx || !q_pos) return CSA_ERR_NULL;
  if (Q < 0 || (cand && C < 0)) return CSA_ERR_SHAPE;
  if (H_I < 1 || H_I > kMaxHI) return CSA_ERR_UNSUPPORTED;
  if (cand && Q > 65535) return CSA_ERR_UNSUPPORTED;
  if (!aligned16(q_idx)) return CSA_ERR_ALIGN;
  return CSA_OK;
}

static int check_topk_args(const csa_cache_t *cache, const int32_t *q_pos, int Q, const int32_t *cand, int C, int k,
                           const int32_t *idx_out) {
  int st = check_cache(cache, false);
  if (st) return st;
  if (!q_pos || !idx_out) return CSA_ERR_NULL;
  if (Q < 0 || k < 0 || (cand && C < 0)) return CSA_ERR_SHAPE;
  if (k > kMaxK) return CSA_ERR_UNSUPPORTED;
  return CSA_OK;
}

int csa_index_scores(const csa_cache_t *cache, const uint8_t *q_idx, const float *w_idx, int H_I,
                     const int32_t *q_pos, int Q, const int32_t *cand, int C, float *scores, size_t scores_bytes,
                     hipStream_t stream) {
  int st = check_index_args(cache, q_idx, w_idx, H_I, q_pos, Q, cand, C);
  if (st) return st;
  if (!scores) return CSA_ERR_NULL;
  if (Q == 0 || cache->B == 0) return CSA_OK;
  if (scores_bytes < index_ws_bytes(cache->B, Q, cache->N_cap, cand ? C : 0)) return CSA_ERR_WORKSPACE;
  const int Ns = cand ? C : cache->N_cap;
  if (Ns == 0) return CSA_OK;
  return status_of(csa::launch_index_scores(view_of(cache), q_idx, w_idx, H_I, q_pos, Q, cand, C, scores, stream));
}

int csa_topk(const csa_cache_t *cache, const float *scores, const int32_t *q_pos, int Q, const int32_t *cand, int C,
             int k, int32_t *idx_out, float *score_out, void *ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_topk_args(cache, q_pos, Q, cand, C, k, idx_out);
  if (st) return st;
  if (Q == 0 || cache->B == 0 || k == 0) return CSA_OK;
  const int Ns = cand ? C : cache->N_cap;
  if (Ns > 0 && !scores) return CSA_ERR_NULL;
  const size_t need = topk_ws_bytes(cache->B, Q, Ns, k, cand != nullptr);
  if (need > 0 && !ws) return CSA_ERR_NULL;
  if (ws_bytes < need) return CSA_ERR_WORKSPACE;
  if (need > 0 && !aligned16(ws)) return CSA_ERR_ALIGN;
  return status_of(
      csa::launch_topk(view_of(cache), scores, Ns, q_pos, Q, cand, C, k, idx_out, score_out, ws, stream));
}

// A full scan's scores, then its top-k from tws (topk_ws_bytes of it).  When
// the top-k is the radix selection, the indexer launch clears the radix
// histograms as a side job and the selection skips its clearing launch.
// The caller has applied every argument and workspace check of both calls.
static hipError_t full_scan_topk(const csa_cache_t *cache, const uint8_t *q_idx, const float *w_idx, int H_I,
                                 const int32_t *q_pos, int Q, int k, float *scores, int32_t *idx_out,
                                 float *score_out, void *tws, hipStream_t stream) {
  const csa::CacheView v = view_of(cache);
  if (cache->N_cap == 0) return csa::launch_topk(v, scores, 0, q_pos, Q, nullptr, 0, k, idx_out, score_out, tws, stream);
  const size_t zb = csa::topk_radix_zero_bytes(cache->B, Q, cache->N_cap, k);
  const bool fold = zb > 0 && tws && csa::index_can_zero(Q, false);
  hipError_t e = csa::launch_index_scores(v, q_idx, w_idx, H_I, q_pos, Q, nullptr, 0, scores, stream, nullptr,
                                          fold ? tws : nullptr, fold ? zb : 0);
  if (e == hipSuccess)
    e = csa::launch_topk(v, scores, cache->N_cap, q_pos, Q, nullptr, 0, k, idx_out, score_out, tws, stream, fold);
  return e;
}

int csa_index_topk(const csa_cache_t *cache, const uint8_t *q_idx, const float *w_idx, int H_I,
                   const int32_t *q_pos, int Q, const int32_t *cand, int C, int k, int32_t *idx_out,
                   float *score_out, void *ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_index_args(cache, q_idx, w_idx, H_I, q_pos, Q, cand, C);
  if (st) return st;
  st = check_topk_args(cache, q_pos, Q, cand, C, k, idx_out);
  if (st) return st;
  if (Q == 0 || cache->B == 0 || k == 0) return CSA_OK;
  const size_t sbytes = index_ws_bytes(cache->B, Q, cache->N_cap, cand ? C : 0);
  const size_t need = index_topk_ws_bytes(cache->B, Q, cache->N_cap, k, C, cand != nullptr);
  if (need > 0 && !ws) return CSA_ERR_NULL;
  if (ws_bytes < need) return CSA_ERR_WORKSPACE;
  if (!aligned16(ws)) return CSA_ERR_ALIGN;
  float *scores = reinterpret_cast<float *>(ws);
  if (hint_path(cache->B, Q, cache->N_cap, k, cand != nullptr)) {
    uint32_t *hint = reinterpret_cast<uint32_t *>(reinterpret_cast<char *>(ws) + align256(sbytes));
    const csa::CacheView v = view_of(cache);
    hipError_t e = csa::launch_index_scores(v, q_idx, w_idx, H_I, q_pos, Q, nullptr, 0, scores, stream, hint);
    if (e == hipSuccess)
      e = csa::launch_topk_hint(v, scores, cache->N_cap, q_pos, Q, k, idx_out, score_out, hint, stream);
    return status_of(e);
  }
  const size_t tbytes = need - align256(sbytes);
  void *tws = tbytes ? reinterpret_cast<char *>(ws) + align256(sbytes) : nullptr;
  if (!cand)
    return status_of(full_scan_topk(cache, q_idx, w_idx, H_I, q_pos, Q, k, scores, idx_out, score_out, tws, stream));
  st = csa_index_scores(cache, q_idx, w_idx, H_I, q_pos, Q, cand, C, scores, sbytes, stream);
  if (st) return st;
  return csa_topk(cache, scores, q_pos, Q, cand, C, k, idx_out, score_out, tws, tbytes, stream);
}

int csa_index_topk_noalloc(const csa_cache_t *cache, const uint8_t *q_idx, const float *w_idx, int H_I,
                           const int32_t *q_pos, int Q, const int32_t *cand, int C, int k, int32_t *idx_out,
                           float *score_out, hipStream_t stream) {
  int st = check_index_args(cache, q_idx, w_idx, H_I, q_pos, Q, cand, C);
  if (st) return st;
  st = check_topk_args(cache, q_pos, Q, cand, C, k, idx_out);
  if (st) return st;
  if (Q == 0 || cache->B == 0 || k == 0) return CSA_OK;
  const size_t need = index_topk_ws_bytes(cache->B, Q, cache->N_cap, k, C, cand != nullptr);
  if (need > (size_t)CSA_NOALLOC_SCRATCH_BYTES) return CSA_ERR_SCRATCH;
  void *ws = nullptr;
  hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return status_of(e);
  // nothing in the scratch has to start at zero: the top-k hint counts are
  // checked against the scores (every call leaves them zero, and the array
  // starts zero)
  return csa_index_topk(cache, q_idx, w_idx, H_I, q_pos, Q, cand, C, k, idx_out, score_out, ws,
                        (size_t)CSA_NOALLOC_SCRATCH_BYTES, stream);
}

int csa_compress_index_scores(const uint16_t *x, int64_t x_stride_b, const uint16_t *z, int64_t z_stride_b, int G,
                              const float *pos_bias, const uint16_t *w_ik, int64_t tok_begin, int64_t T,
                              const csa_cache_t *cache, const uint8_t *q_idx, const float *w_idx, int H_I,
                              const int32_t *q_pos, int Q, float *scores, size_t scores_bytes, hipStream_t stream) {
  int st = check_compress_args(x, x_stride_b, z, z_stride_b, G, pos_bias, w_ik, tok_begin, T, cache);
  if (st) return st;
  st = check_index_args(cache, q_idx, w_idx, H_I, q_pos, Q, nullptr, 0);
  if (st) return st;
  if (!scores) return CSA_ERR_NULL;
  if (cache->B > 0 && Q > 0 && scores_bytes < index_ws_bytes(cache->B, Q, cache->N_cap, 0)) return CSA_ERR_WORKSPACE;
  if (cache->B > 0 && Q > 0 && T > 0 && cache->N_cap > 0 &&
      csa::append_index_fusable(cache->m, T, Q, G, w_ik, cache->B))
    return status_of(csa::launch_append_index(x, x_stride_b, z, z_stride_b, G, pos_bias, w_ik, tok_begin / cache->m,
                                              view_of(cache), q_idx, w_idx, H_I, q_pos, scores, stream));
  st = csa_compress(x, x_stride_b, z, z_stride_b, G, pos_bias, w_ik, tok_begin, T, cache, stream);
  if (st) return st;
  return csa_index_scores(cache, q_idx, w_idx, H_I, q_pos, Q, nullptr, 0, scores, scores_bytes, stream);
}

int csa_compress_index_topk(const uint16_t *x, int64_t x_stride_b, const uint16_t *z, int64_t z_stride_b, int G,
                            const float *pos_bias, const uint16_t *w_ik, int64_t tok_begin, int64_t T,
                            const csa_cache_t *cache, const uint8_t *q_idx, const float *w_idx, int H_I,
                            const int32_t *q_pos, int Q, int k, int32_t *idx_out, float *score_out, void *ws,
                            size_t ws_bytes, hipStream_t stream) {
  int st = check_compress_args(x, x_stride_b, z, z_stride_b, G, pos_bias, w_ik, tok_begin, T, cache);
  if (st) return st;
  st = check_index_args(cache, q_idx, w_idx, H_I, q_pos, Q, nullptr, 0);
  if (st) return st;
  st = check_topk_args(cache, q_pos, Q, nullptr, 0, k, idx_out);
  if (st) return st;
  if (cache->B > 0 && Q > 0 && k > 0) {
    const size_t need = index_topk_ws_bytes(cache->B, Q, cache->N_cap, k, 0, false);
    if (need > 0 && !ws) return CSA_ERR_NULL;
    if (ws_bytes < need) return CSA_ERR_WORKSPACE;
    if (!aligned16(ws)) return CSA_ERR_ALIGN;
  }
  if (cache->B > 0 && Q > 0 && k > 0 && T > 0 && cache->N_cap > 0 &&
      csa::append_index_fusable(cache->m, T, Q, G, w_ik, cache->B) &&
      hint_path(cache->B, Q, cache->N_cap, k, false)) {
    float *scores = reinterpret_cast<float *>(ws);
    uint32_t *hint = reinterpret_cast<uint32_t *>(reinterpret_cast<char *>(ws) +
                                                  align256(index_ws_bytes(cache->B, Q, cache->N_cap, 0)));
    const csa::CacheView v = view_of(cache);
    hipError_t e = csa::launch_append_index(x, x_stride_b, z, z_stride_b, G, pos_bias, w_ik, tok_begin / cache->m, v,
                                            q_idx, w_idx, H_I, q_pos, scores, stream, hint);
    if (e == hipSuccess)
      e = csa::launch_topk_hint(v, scores, cache->N_cap, q_pos, Q, k, idx_out, score_out, hint, stream);
    return status_of(e);
  }
  st = csa_compress(x, x_stride_b, z, z_stride_b, G, pos_bias, w_ik, tok_begin, T, cache, stream);
  if (st) return st;
  return csa_index_topk(cache, q_idx, w_idx, H_I, q_pos, Q, nullptr, 0, k, idx_out, score_out, ws, ws_bytes, stream);
}

int csa_index_pool(const csa_cache_t *cache, const float *scores, const int32_t *q_pos, int Q, int block,
                   int n_blocks, int32_t *pool_out, void *ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_cache(cache, false);
  if (st) return st;
  if (!q_pos || !pool_out) return CSA_ERR_NULL;
  if (Q < 0) return CSA_ERR_SHAPE;
  if (block < 1 || block > kMaxPoolBlock || n_blocks < 1) return CSA_ERR_UNSUPPORTED;
  if ((int64_t)n_blocks * block > kMaxK) return CSA_ERR_UNSUPPORTED;
  if (Q == 0 || cache->B == 0) return CSA_OK;
  if (cache->N_cap > 0 && !scores) return CSA_ERR_NULL;
  {
    // flattened launch grids: rows x tiles of 256 blocks / pool slots
    const int64_t rows = (int64_t)cache->B * Q;
    const int64_t nb = ((int64_t)cache->N_cap + block - 1) / block;
    const int64_t tiles = ((nb > (int64_t)n_blocks * block ? nb : (int64_t)n_blocks * block) + 255) / 256;
    if (rows * tiles > INT32_MAX) return CSA_ERR_UNSUPPORTED;
  }
  const size_t need = csa::pool_workspace_bytes(cache->B, Q, cache->N_cap, block, n_blocks);
  if (!ws) return CSA_ERR_NULL;
  if (ws_bytes < need) return CSA_ERR_WORKSPACE;
  if (!aligned16(ws)) return CSA_ERR_ALIGN;
  return status_of(
      csa::launch_index_pool(view_of(cache), scores, q_pos, Q, block, n_blocks, pool_out, ws, stream));
}

// The window rows of an attention call: bf16 rows (swa) or FP8 planes (w8).
static int check_window8(const uint8_t *codes, const uint8_t *scales, const uint16_t *rope, int n_win) {
  if (n_win <= 0) return CSA_OK;
  if (!codes || !scales || !rope) return CSA_ERR_NULL;
  if (!aligned16(codes) || !aligned16(rope)) return CSA_ERR_ALIGN;
  return CSA_OK;
}

static int sparse_attn_impl(const csa_cache_t *cache, const uint16_t *q, int H, const int32_t *q_pos, int Q,
                            const int32_t *idx, int k, const uint16_t *swa, const csa::SwaPlanes *w8,
                            const int32_t *swa_pos0, int S, int n_win, float softmax_scale, float rope_base,
                            int out_dtype, void *out, float *lse, void *ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_attn_common(cache, q, H, q_pos, Q, swa, swa_pos0, S, n_win, softmax_scale, rope_base, out_dtype,
                             out);
  if (st) return st;
  if (k < 0) return CSA_ERR_SHAPE;
  if (k > 0 && !idx) return CSA_ERR_NULL;
  if (k > kMaxK) return CSA_ERR_UNSUPPORTED;
  if (Q == 0 || cache->B == 0) return CSA_OK;
  const size_t need = csa::attn_workspace_bytes(cache->B, Q, H, k, n_win);
  if (need > 0 && !ws) return CSA_ERR_NULL;
  if (ws_bytes < need) return CSA_ERR_WORKSPACE;
  if (need > 0 && !aligned16(ws)) return CSA_ERR_ALIGN;
  const csa::CacheView v = view_of(cache);
  return status_of(csa::launch_attention(v, q, H, q_pos, Q, idx, k, false, swa, w8, swa_pos0, S, n_win,
                                         softmax_scale, rope_base, out_dtype == CSA_OUT_BF16, out, lse, ws,
                                         stream));
}

static int dense_attn_impl(const csa_cache_t *cache, const uint16_t *q, int H, const int32_t *q_pos, int Q,
                           const uint16_t *swa, const csa::SwaPlanes *w8, const int32_t *swa_pos0, int S, int n_win,
                           float softmax_scale, float rope_base, int out_dtype, void *out, float *lse, void *ws,
                           size_t ws_bytes, hipStream_t stream) {
  int st = check_attn_common(cache, q, H, q_pos, Q, swa, swa_pos0, S, n_win, softmax_scale, rope_base, out_dtype,
                             out);
  if (st) return st;
  if (Q == 0 || cache->B == 0) return CSA_OK;
  const size_t need = csa::attn_workspace_bytes(cache->B, Q, H, cache->N_cap, n_win);
  if (need > 0 && !ws) return CSA_ERR_NULL;
  if (ws_bytes < need) return CSA_ERR_WORKSPACE;
  if (need > 0 && !aligned16(ws)) return CSA_ERR_ALIGN;
  const csa::CacheView v = view_of(cache);
  return status_of(csa::launch_attention(v, q, H, q_pos, Q, nullptr, 0, true, swa, w8, swa_pos0, S, n_win,
                                         softmax_scale, rope_base, out_dtype == CSA_OUT_BF16, out, lse, ws,
                                         stream));
}

int csa_sparse_attn(const csa_cache_t *cache, const uint16_t *q, int H, const int32_t *q_pos, int Q,
                    const int32_t *idx, int k, const uint16_t *swa, const int32_t *swa_pos0, int S, int n_win,
                    float softmax_scale, float rope_base, int out_dtype, void *out, float *lse, void *ws,
                    size_t ws_bytes, hipStream_t stream) {
  return sparse_attn_impl(cache, q, H, q_pos, Q, idx, k, swa, nullptr, swa_pos0, S, n_win, softmax_scale, rope_base,
                          out_dtype, out, lse, ws, ws_bytes, stream);
}

int hca_dense_attn(const csa_cache_t *cache, const uint16_t *q, int H, const int32_t *q_pos, int Q,
                   const uint16_t *swa, const int32_t *swa_pos0, int S, int n_win, float softmax_scale,
                   float rope_base, int out_dtype, void *out, float *lse, void *ws, size_t ws_bytes,
                   hipStream_t stream) {
  return dense_attn_impl(cache, q, H, q_pos, Q, swa, nullptr, swa_pos0, S, n_win, softmax_scale, rope_base, out_dtype,
                         out, lse, ws, ws_bytes, stream);
}

int csa_sparse_attn_w8(const csa_cache_t *cache, const uint16_t *q, int H, const int32_t *q_pos, int Q,
                       const int32_t *idx, int k, const uint8_t *swa_codes, const uint8_t *swa_scales,
                       const uint16_t *swa_rope, const int32_t *swa_pos0, int S, int n_win, float softmax_scale,
                       float rope_base, int out_dtype, void *out, float *lse, void *ws, size_t ws_bytes,
                       hipStream_t stream) {
  int st = check_window8(swa_codes, swa_scales, swa_rope, n_win);
  if (st) return st;
  const csa::SwaPlanes w8{swa_codes, swa_scales, swa_rope};
  // the rope plane stands in for the bf16 rows in the shared checks
  return sparse_attn_impl(cache, q, H, q_pos, Q, idx, k, swa_rope, &w8, swa_pos0, S, n_win, softmax_scale, rope_base,
                          out_dtype, out, lse, ws, ws_bytes, stream);
}

int hca_dense_attn_w8(const csa_cache_t *cache, const uint16_t *q, int H, const int32_t *q_pos, int Q,
                      const uint8_t *swa_codes, const uint8_t *swa_scales, const uint16_t *swa_rope,
                      const int32_t *swa_pos0, int S, int n_win, float softmax_scale, float rope_base,
                      int out_dtype, void *out, float *lse, void *ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_window8(swa_codes, swa_scales, swa_rope, n_win);
  if (st) return st;
  const csa::SwaPlanes w8{swa_codes, swa_scales, swa_rope};
  return dense_attn_impl(cache, q, H, q_pos, Q, swa_rope, &w8, swa_pos0, S, n_win, softmax_scale, rope_base,
                         out_dtype, out, lse, ws, ws_bytes, stream);
}

int csa_swa_encode(const uint16_t *x, int64_t x_stride_b, int B, int S, uint8_t *codes, uint8_t *scales,
                   uint16_t *rope, hipStream_t stream) {
  if (B < 0 || S < 0) return CSA_ERR_SHAPE;
  if (B == 0 || S == 0) return CSA_OK;
  if (!x || !codes || !scales || !rope) return CSA_ERR_NULL;
  if (B > 1 && x_stride_b < (int64_t)S * csa::kD) return CSA_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(rope) || (x_stride_b % 8)) return CSA_ERR_ALIGN;
  if ((int64_t)B * S > (int64_t)INT32_MAX * 16) return CSA_ERR_UNSUPPORTED;
  return status_of(csa::launch_swa_encode(x, x_stride_b, B, S, codes, scales, rope, stream));
}

// ---------------------------------------------------------------------------
// CSA2 layer stack: host orchestration of the calls above.

static int check_pool_args(int block, int n_blocks, const int32_t *pool_out) {
  if (!pool_out) return CSA_ERR_NULL;
  if (block < 1 || block > kMaxPoolBlock || n_blocks < 1) return CSA_ERR_UNSUPPORTED;
  if ((int64_t)n_blocks * block > kMaxK) return CSA_ERR_UNSUPPORTED;
  return CSA_OK;
}

// What one layer of a stack reads: its cache, its candidates (Reindex), and
// the selection it attends to.
struct StackStep {
  const csa_cache_t *cache;
  const int32_t *cand;
  int C;
  const int32_t *sel;
  int k;
  size_t ws_scores;  // 256-byte aligned score buffer at the front of ws
  size_t ws_rest;    // top-k / pool / attention workspace behind it
};

// Walks the stack, applying every check of the calls it will make; fills
// steps[] and the workspace needed.  Launches nothing.
static int stack_plan(const csa2_layer_t *L, int n, const int32_t *q_pos, int Q, StackStep *steps, size_t *ws_need) {
  if (!L || !q_pos) return CSA_ERR_NULL;
  if (n < 1 || Q < 0) return CSA_ERR_SHAPE;
  if (n > kMaxStackLayers) return CSA_ERR_UNSUPPORTED;
  const csa_cache_t *full = nullptr;
  const int32_t *pool = nullptr;
  int pool_C = 0;
  const int32_t *sel = nullptr;
  int sel_k = 0;
  int B = -1;
  size_t need = 0;
  for (int i = 0; i < n; ++i) {
    const csa2_layer_t &l = L[i];
    StackStep st{};
    int rc;
    if (l.mode == CSA2_FULL) {
      if (!l.cache) return CSA_ERR_NULL;
      if (B >= 0 && l.cache->B != B) return CSA_ERR_SHAPE;
      B = l.cache->B;
      if (l.k < 1) return CSA_ERR_SHAPE;
      if ((rc = check_index_args(l.cache, l.q_idx, l.w_idx, l.H_I, q_pos, Q, nullptr, 0))) return rc;
      if ((rc = check_topk_args(l.cache, q_pos, Q, nullptr, 0, l.k, l.idx_out))) return rc;
      full = l.cache;
      pool = nullptr;
      pool_C = 0;
      size_t rest = topk_ws_bytes(B, Q, full->N_cap, l.k, false);
      if (l.pool_blocks > 0) {
        if ((rc = check_pool_args(l.pool_block, l.pool_blocks, l.pool_out))) return rc;
        pool = l.pool_out;
        pool_C = l.pool_blocks * l.pool_block;
        const size_t pb = csa::pool_workspace_bytes(B, Q, full->N_cap, l.pool_block, l.pool_blocks);
        rest = rest > pb ? rest : pb;
      } else if (l.pool_blocks < 0) {
        return CSA_ERR_SHAPE;
      }
      st.ws_scores = align256(index_ws_bytes(B, Q, full->N_cap, 0));
      st.ws_rest = rest;
      sel = l.idx_out;
      sel_k = l.k;
    } else if (l.mode == CSA2_REINDEX) {
      if (!full) return CSA_ERR_SHAPE;
      if (l.k < 1) return CSA_ERR_SHAPE;
      int src = l.cand;
      if (src == CSA2_CAND_AUTO) src = pool ? CSA2_CAND_POOL : CSA2_CAND_SELECTION;
      if (src == CSA2_CAND_POOL) {
        if (!pool) return CSA_ERR_SHAPE;
        st.cand = pool;
        st.C = pool_C;
      } else if (src == CSA2_CAND_SELECTION) {
        st.cand = sel;
        st.C = sel_k;
      } else if (src != CSA2_CAND_SCAN) {
        return CSA_ERR_UNSUPPORTED;
      }
      if ((rc = check_index_args(full, l.q_idx, l.w_idx, l.H_I, q_pos, Q, st.cand, st.C))) return rc;
      if ((rc = check_topk_args(full, q_pos, Q, st.cand, st.C, l.k, l.idx_out))) return rc;
      const int Ns = st.cand ? st.C : full->N_cap;
      st.ws_scores = align256(index_ws_bytes(B, Q, full->N_cap, st.cand ? st.C : 0));
      st.ws_rest = topk_ws_bytes(B, Q, Ns, l.k, st.cand != nullptr);
      sel = l.idx_out;
      sel_k = l.k;
    } else if (l.mode == CSA2_REUSE) {
      if (!full || !sel) return CSA_ERR_SHAPE;
    } else {
      return CSA_ERR_UNSUPPORTED;
    }
    st.cache = full;
    st.sel = sel;
    st.k = sel_k;
    if ((rc = check_attn_common(full, l.q, l.H, q_pos, Q, l.swa, l.swa_pos0, l.S, l.n_win, l.softmax_scale,
                                l.rope_base, l.out_dtype, l.out)))
      return rc;
    if (st.k > kMaxK) return CSA_ERR_UNSUPPORTED;
    if (Q == 0 || B == 0) {
      // nothing will be launched: no workspace
      st.ws_scores = st.ws_rest = 0;
    } else {
      const size_t aw = csa::attn_workspace_bytes(B, Q, l.H, st.k, l.n_win);
      st.ws_rest = st.ws_rest > aw ? st.ws_rest : aw;
    }
    const size_t total = st.ws_scores + st.ws_rest;
    need = need > total ? need : total;
    if (steps) steps[i] = st;
  }
  *ws_need = need;
  return CSA_OK;
}

size_t csa2_stack_workspace_bytes(const csa2_layer_t *layers, int n_layers, int Q) {
  if (!layers || n_layers < 1 || Q < 0) return 0;
  // a q_pos pointer only has to be non-null for the walk
  static const int32_t dummy = 0;
  size_t need = 0;
  if (stack_plan(layers, n_layers, &dummy, Q, nullptr, &need) != CSA_OK) return 0;
  return need;
}

int csa2_layer_stack(const csa2_layer_t *layers, int n_layers, const int32_t *q_pos, int Q, void *ws,
                     size_t ws_bytes, hipStream_t stream) {
  if (!layers) return CSA_ERR_NULL;
  if (n_layers < 1) return CSA_ERR_SHAPE;
  if (n_layers > kMaxStackLayers) return CSA_ERR_UNSUPPORTED;
  StackStep steps[kMaxStackLayers];
  size_t need = 0;
  int st = stack_plan(layers, n_layers, q_pos, Q, steps, &need);
  if (st == CSA_OK && need > 0 && !ws) st = CSA_ERR_NULL;
  if (st == CSA_OK && ws_bytes < need) st = CSA_ERR_WORKSPACE;
  if (st == CSA_OK && ws && !aligned16(ws)) st = CSA_ERR_ALIGN;
  const int B = st == CSA_OK ? steps[0].cache->B : 0;
  for (int i = 0; st == CSA_OK && i < n_layers && Q > 0 && B > 0; ++i) {
    const csa2_layer_t &l = layers[i];
    const StackStep &s = steps[i];
    float *scores = reinterpret_cast<float *>(ws);
    void *rest = s.ws_rest ? reinterpret_cast<char *>(ws) + s.ws_scores : nullptr;
    if (l.mode == CSA2_FULL) {
      st = status_of(full_scan_topk(s.cache, l.q_idx, l.w_idx, l.H_I, q_pos, Q, l.k, scores, l.idx_out, nullptr,
                                    s.ws_rest ? rest : nullptr, stream));
    } else if (l.mode != CSA2_REUSE) {
      st = csa_index_scores(s.cache, l.q_idx, l.w_idx, l.H_I, q_pos, Q, s.cand, s.C, scores, s.ws_scores, stream);
      if (st == CSA_OK)
        st = csa_topk(s.cache, scores, q_pos, Q, s.cand, s.C, l.k, l.idx_out, nullptr, rest, s.ws_rest, stream);
    }
    if (st == CSA_OK && l.mode == CSA2_FULL && l.pool_blocks > 0)
      st = csa_index_pool(s.cache, scores, q_pos, Q, l.pool_block, l.pool_blocks, l.pool_out, rest, s.ws_rest, stream);
    if (st == CSA_OK)
      st = csa_sparse_attn(s.cache, l.q, l.H, q_pos, Q, s.sel, s.k, l.swa, l.swa_pos0, l.S, l.n_win,
                           l.softmax_scale, l.rope_base, l.out_dtype, l.out, l.lse, rest, s.ws_rest, stream);
  }
  return st;
}

}  // extern "C"
