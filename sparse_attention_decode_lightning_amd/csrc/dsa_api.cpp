// C ABI of the sparse-attention decode library: argument validation, then a
// launch on the caller's stream. Validation touches no HIP API, so every
// error path can be exercised without a GPU; nothing is enqueued on error.
#include <math.h>

#include "dsa_internal.h"

namespace {

using dsa::BatchArgs;
using dsa::CacheArgs;

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

dsa_status check_batch(const dsa_batch *bt, BatchArgs *out) {
  if (bt == nullptr) return DSA_ERR_NULL;
  if (bt->batch < 0 || bt->total_q < 0 || bt->max_seq_len < 0 || bt->max_q < 0 ||
      bt->bt_stride < 0)
    return DSA_ERR_SHAPE;
  if (bt->total_q > 0) {
    if (bt->block_table == nullptr || bt->seq_lens == nullptr || bt->cu_q == nullptr)
      return DSA_ERR_NULL;
    if (!aligned(bt->block_table, 4) || !aligned(bt->seq_lens, 4) || !aligned(bt->cu_q, 4))
      return DSA_ERR_SHAPE;
    if (bt->batch < 1 || bt->max_q < 1 || bt->max_q > bt->total_q || bt->max_seq_len < 1 ||
        bt->bt_stride < 1)
      return DSA_ERR_SHAPE;
  }
  out->block_table = bt->block_table;
  out->seq_lens = bt->seq_lens;
  out->cu_q = bt->cu_q;
  out->batch = bt->batch;
  out->bt_stride = bt->bt_stride;
  out->total_q = bt->total_q;
  out->max_seq_len = bt->max_seq_len;
  out->max_q = bt->max_q;
  return DSA_OK;
}

// Element type, geometry and alignment of a paged cache.
dsa_status check_cache_geometry(const dsa_paged_cache *c, CacheArgs *out) {
  if (c->data == nullptr) return DSA_ERR_NULL;
  if (c->dtype != DSA_F32 && c->dtype != DSA_BF16 && c->dtype != DSA_FP8_E4M3)
    return DSA_ERR_DTYPE;
  if (c->dtype == DSA_FP8_E4M3 && c->scale == nullptr) return DSA_ERR_NULL;
  if (c->num_pages < 1 || c->page_size < 1 || c->row_elems < 1) return DSA_ERR_SHAPE;
  if (!aligned(c->data, 16) || (c->dtype == DSA_FP8_E4M3 && !aligned(c->scale, 4)))
    return DSA_ERR_SHAPE;
  out->data = c->data;
  out->scale = c->dtype == DSA_FP8_E4M3 ? c->scale : nullptr;
  out->num_pages = c->num_pages;
  out->page_size = c->page_size;
  out->row_elems = c->row_elems;
  out->dtype = c->dtype;
  return DSA_OK;
}

// A cache read through a batch's block table: its pages must cover max_seq_len.
dsa_status check_cache(const dsa_paged_cache *c, const BatchArgs &bt, CacheArgs *out) {
  if (c == nullptr) return DSA_ERR_NULL;
  const dsa_status st = check_cache_geometry(c, out);
  if (st != DSA_OK) return st;
  if (bt.total_q > 0 && (int64_t)bt.bt_stride < ceil_div(bt.max_seq_len, c->page_size))
    return DSA_ERR_SHAPE;
  return DSA_OK;
}

dsa_status launch_status(hipError_t e) { return e == hipSuccess ? DSA_OK : DSA_ERR_LAUNCH; }

}  // namespace

extern "C" {

const char *dsa_status_str(dsa_status status) {
  switch (status) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_NULL: return "DSA_ERR_NULL: a required pointer is NULL";
    case DSA_ERR_SHAPE: return "DSA_ERR_SHAPE: a size, stride, bound or alignment is invalid";
    case DSA_ERR_DTYPE: return "DSA_ERR_DTYPE: element type not allowed here";
    case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE: workspace missing or too small";
    case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED: no kernel for this combination";
    case DSA_ERR_LAUNCH: return "DSA_ERR_LAUNCH: the HIP runtime rejected a launch";
  }
  return "DSA_ERR_UNKNOWN";
}

int32_t dsa_abi_version(void) { return DSA_ABI_VERSION; }

dsa_status dsa_indexer_scores(const dsa_batch *batch, const void *q_idx, int32_t q_dtype,
                              const float *w, int32_t n_heads, int32_t head_dim,
                              const dsa_paged_cache *keys, float *scores, int64_t ld_scores,
                              void *stream) {
  BatchArgs bt;
  CacheArgs kc;
  dsa_status st = check_batch(batch, &bt);
  if (st != DSA_OK) return st;
  if (keys == nullptr) return DSA_ERR_NULL;
  if (bt.total_q > 0 && (q_idx == nullptr || w == nullptr || scores == nullptr)) return DSA_ERR_NULL;
  st = check_cache(keys, bt, &kc);
  if (st != DSA_OK) return st;
  if (q_dtype != DSA_F32 && q_dtype != DSA_BF16) return DSA_ERR_DTYPE;
  if (q_dtype == DSA_F32 && kc.dtype != DSA_F32) return DSA_ERR_DTYPE;
  if (q_dtype == DSA_BF16 && kc.dtype == DSA_F32) return DSA_ERR_DTYPE;
  if (n_heads < 1 || head_dim < 1 || kc.row_elems != head_dim) return DSA_ERR_SHAPE;
  if (ld_scores < bt.max_seq_len || ld_scores < 1) return DSA_ERR_SHAPE;
  if (!aligned(q_idx, 16) || !aligned(w, 4) || !aligned(scores, 4)) return DSA_ERR_SHAPE;
  if (bt.total_q == 0) return DSA_OK;
  return launch_status(dsa::launch_indexer_scores(bt, q_idx, q_dtype, w, n_heads, head_dim, kc,
                                                  scores, ld_scores,
                                                  static_cast<hipStream_t>(stream)));
}

size_t dsa_topk_workspace_size(int32_t total_q, int32_t max_seq_len, int32_t k) {
  return dsa::topk_workspace_bytes(total_q, max_seq_len, k);
}

dsa_status dsa_topk(const dsa_batch *batch, const float *scores, int64_t ld_scores, int32_t k,
                    int32_t *indices, void *workspace, size_t workspace_bytes, void *stream) {
  BatchArgs bt;
  dsa_status st = check_batch(batch, &bt);
  if (st != DSA_OK) return st;
  if (bt.total_q > 0 && (scores == nullptr || indices == nullptr)) return DSA_ERR_NULL;
  if (k < 1 || ld_scores < bt.max_seq_len || ld_scores < 1) return DSA_ERR_SHAPE;
  if (!aligned(scores, 4) || !aligned(indices, 4)) return DSA_ERR_SHAPE;
  if (!dsa::topk_supported(bt.max_seq_len, k)) return DSA_ERR_UNSUPPORTED;
  const size_t need = dsa::topk_workspace_bytes(bt.total_q, bt.max_seq_len, k);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 16)))
    return DSA_ERR_WORKSPACE;
  if (bt.total_q == 0) return DSA_OK;
  return launch_status(dsa::launch_topk(bt, scores, ld_scores, k, 1, indices, workspace,
                                        workspace_bytes, static_cast<hipStream_t>(stream)));
}

size_t dsa_sparse_mla_workspace_size(int32_t total_q, int32_t n_heads, int32_t d_latent,
                                     int32_t k) {
  if (total_q < 1 || n_heads < 1 || d_latent < 1 || k < 1) return 0;
  return dsa::mla_workspace_bytes(total_q, n_heads, d_latent, k);
}

}  // extern "C"

namespace {

// One or more attention layers over one index list: validation common to
// dsa_sparse_mla_fwd (one layer) and dsa_sparse_mla_fwd_layers.
dsa_status mla_layers(const dsa_batch *batch, int32_t n_layers, const void *const *q,
                      int32_t q_dtype, int32_t n_heads, int32_t d_latent, int32_t d_rope,
                      const dsa_paged_cache *kv, const int32_t *indices, int32_t k, float scale,
                      float *const *out, float *const *lse, void *workspace,
                      size_t workspace_bytes, void *stream, bool use_scratch = false) {
  BatchArgs bt;
  dsa_status st = check_batch(batch, &bt);
  if (st != DSA_OK) return st;
  if (n_layers < 1 || n_layers > dsa::kMlaMaxLayers) return DSA_ERR_SHAPE;
  if (kv == nullptr || q == nullptr || out == nullptr) return DSA_ERR_NULL;
  if (bt.total_q > 0 && indices == nullptr) return DSA_ERR_NULL;
  if (q_dtype != DSA_F32 && q_dtype != DSA_BF16) return DSA_ERR_DTYPE;
  if (n_heads < 1 || d_latent < 1 || d_rope < 0 || k < 1) return DSA_ERR_SHAPE;
  // a softmax scale is positive (the pages tie it to 1 / sqrt(192 + 64)); the
  // MFMA kernel takes a tile's maximum of the raw logits before scaling
  if (!isfinite(scale) || !(scale > 0.0f)) return DSA_ERR_SHAPE;
  if (!aligned(indices, 4)) return DSA_ERR_SHAPE;
  dsa::MlaLayer ly[dsa::kMlaMaxLayers];
  for (int l = 0; l < n_layers; ++l) {
    st = check_cache(&kv[l], bt, &ly[l].kv);
    if (st != DSA_OK) return st;
    if (bt.total_q > 0 && (q[l] == nullptr || out[l] == nullptr)) return DSA_ERR_NULL;
    if (ly[l].kv.dtype != q_dtype) return DSA_ERR_DTYPE;
    if ((int64_t)ly[l].kv.row_elems != (int64_t)d_latent + d_rope) return DSA_ERR_SHAPE;
    // one block table addresses every layer's cache
    if (ly[l].kv.page_size != ly[0].kv.page_size) return DSA_ERR_SHAPE;
    ly[l].q = q[l];
    ly[l].out = out[l];
    ly[l].lse = lse == nullptr ? nullptr : lse[l];
    if (!aligned(ly[l].q, 16) || !aligned(ly[l].out, 16) ||
        (ly[l].lse != nullptr && !aligned(ly[l].lse, 4)))
      return DSA_ERR_SHAPE;
  }
  const bool mfma_shape =
      q_dtype == DSA_BF16 && n_heads <= 64 && d_latent == 512 && d_rope == 64;
  if (!mfma_shape && d_latent > 1024) return DSA_ERR_UNSUPPORTED;
  if (mfma_shape && k > dsa::mla_max_k()) return DSA_ERR_UNSUPPORTED;
  const size_t need = (size_t)n_layers * dsa::mla_workspace_bytes(bt.total_q, n_heads, d_latent, k);
  if (use_scratch) {
    // the library's static scratch array stands in for the workspace
    if (need > DSA_MLA_NOALLOC_SCRATCH_BYTES) return DSA_ERR_WORKSPACE;
  } else if (need > 0 && (workspace == nullptr || workspace_bytes < need ||
                          !aligned(workspace, 16))) {
    return DSA_ERR_WORKSPACE;
  }
  if (bt.total_q == 0) return DSA_OK;
  if (use_scratch && need > 0) {
    // this device's copy of the array (found on the first call on the device)
    if (dsa::mla_scratch(&workspace) != hipSuccess) return DSA_ERR_LAUNCH;
    workspace_bytes = DSA_MLA_NOALLOC_SCRATCH_BYTES;
  }
  return launch_status(dsa::launch_sparse_mla(bt, ly, n_layers, q_dtype, n_heads, d_latent,
                                              d_rope, indices, k, scale, workspace,
                                              workspace_bytes, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

dsa_status dsa_sparse_mla_fwd(const dsa_batch *batch, const void *q, int32_t q_dtype,
                              int32_t n_heads, int32_t d_latent, int32_t d_rope,
                              const dsa_paged_cache *kv, const int32_t *indices, int32_t k,
                              float scale, float *out, float *lse, void *workspace,
                              size_t workspace_bytes, void *stream) {
  return mla_layers(batch, 1, &q, q_dtype, n_heads, d_latent, d_rope, kv, indices, k, scale, &out,
                    &lse, workspace, workspace_bytes, stream);
}

size_t dsa_sparse_mla_layers_workspace_size(int32_t n_layers, int32_t total_q, int32_t n_heads,
                                            int32_t d_latent, int32_t k) {
  if (n_layers < 1 || n_layers > dsa::kMlaMaxLayers) return 0;
  return (size_t)n_layers * dsa_sparse_mla_workspace_size(total_q, n_heads, d_latent, k);
}

dsa_status dsa_sparse_mla_fwd_layers(const dsa_batch *batch, int32_t n_layers,
                                     const void *const *q, int32_t q_dtype, int32_t n_heads,
                                     int32_t d_latent, int32_t d_rope, const dsa_paged_cache *kv,
                                     const int32_t *indices, int32_t k, float scale,
                                     float *const *out, float *const *lse, void *workspace,
                                     size_t workspace_bytes, void *stream) {
  return mla_layers(batch, n_layers, q, q_dtype, n_heads, d_latent, d_rope, kv, indices, k, scale,
                    out, lse, workspace, workspace_bytes, stream);
}

dsa_status dsa_sparse_mla_fwd_noalloc(const dsa_batch *batch, const void *q, int32_t q_dtype,
                                      int32_t n_heads, int32_t d_latent, int32_t d_rope,
                                      const dsa_paged_cache *kv, const int32_t *indices, int32_t k,
                                      float scale, float *out, float *lse, void *stream) {
  return mla_layers(batch, 1, &q, q_dtype, n_heads, d_latent, d_rope, kv, indices, k, scale, &out,
                    &lse, nullptr, 0, stream, /*use_scratch=*/true);
}

size_t dsa_sparse_mla_qblocked_workspace_size(int32_t total_q, int32_t n_heads, int32_t k) {
  return dsa::mla_qblock_workspace_bytes(total_q, n_heads, k);
}

dsa_status dsa_sparse_mla_fwd_qblocked(const dsa_batch *batch, const void *q, int32_t q_dtype,
                                       int32_t n_heads, int32_t d_latent, int32_t d_rope,
                                       const dsa_paged_cache *kv, const int32_t *indices, int32_t k,
                                       float scale, float *out, float *lse, void *workspace,
                                       size_t workspace_bytes, void *stream) {
  BatchArgs bt;
  dsa_status st = check_batch(batch, &bt);
  if (st != DSA_OK) return st;
  if (kv == nullptr) return DSA_ERR_NULL;
  if (bt.total_q > 0 && (q == nullptr || out == nullptr || indices == nullptr)) return DSA_ERR_NULL;
  if (q_dtype != DSA_F32 && q_dtype != DSA_BF16) return DSA_ERR_DTYPE;
  if (n_heads < 1 || d_latent < 1 || d_rope < 0 || k < 1) return DSA_ERR_SHAPE;
  if (!isfinite(scale) || !(scale > 0.0f)) return DSA_ERR_SHAPE;
  dsa::MlaLayer ly;
  st = check_cache(kv, bt, &ly.kv);
  if (st != DSA_OK) return st;
  if (ly.kv.dtype != q_dtype) return DSA_ERR_DTYPE;
  if ((int64_t)ly.kv.row_elems != (int64_t)d_latent + d_rope) return DSA_ERR_SHAPE;
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(indices, 4) ||
      (lse != nullptr && !aligned(lse, 4)))
    return DSA_ERR_SHAPE;
  // positions and physical rows travel as 32-bit words in the unions
  if (!dsa::mla_qblock_supported(q_dtype, n_heads, d_latent, d_rope, k) ||
      bt.max_seq_len >= (1 << 29) ||
      (uint64_t)ly.kv.num_pages * (uint64_t)ly.kv.page_size > 0xFFFFFFFFull)
    return DSA_ERR_UNSUPPORTED;
  const size_t need = dsa::mla_qblock_workspace_bytes(bt.total_q, n_heads, k);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 16)))
    return DSA_ERR_WORKSPACE;
  if (bt.total_q == 0) return DSA_OK;
  ly.q = q;
  ly.out = out;
  ly.lse = lse;
  return launch_status(dsa::launch_sparse_mla_qblocked(bt, ly, n_heads, indices, k, scale, workspace,
                                                       static_cast<hipStream_t>(stream)));
}

dsa_status dsa_indexer_page_scores(const dsa_batch *batch, const void *q_idx, int32_t q_dtype,
                                   const float *w, int32_t n_heads, int32_t head_dim,
                                   const dsa_paged_cache *keys, int32_t page_size,
                                   float *page_scores, int64_t ld_pages, void *stream) {
  BatchArgs bt;
  CacheArgs kc;
  dsa_status st = check_batch(batch, &bt);
  if (st != DSA_OK) return st;
  if (keys == nullptr) return DSA_ERR_NULL;
  if (bt.total_q > 0 && (q_idx == nullptr || w == nullptr || page_scores == nullptr))
    return DSA_ERR_NULL;
  st = check_cache(keys, bt, &kc);
  if (st != DSA_OK) return st;
  if (q_dtype != DSA_F32 && q_dtype != DSA_BF16) return DSA_ERR_DTYPE;
  if (n_heads < 1 || head_dim < 1 || kc.row_elems != head_dim || page_size < 1)
    return DSA_ERR_SHAPE;
  if (ld_pages < dsa::candidate_bound(bt.max_seq_len, page_size) || ld_pages < 1)
    return DSA_ERR_SHAPE;
  if (!aligned(q_idx, 16) || !aligned(w, 4) || !aligned(page_scores, 4)) return DSA_ERR_SHAPE;
  if (!dsa::indexer_page_max_supported(bt, q_dtype, n_heads, head_dim, kc, page_size))
    return DSA_ERR_UNSUPPORTED;
  if (bt.total_q == 0) return DSA_OK;
  return launch_status(dsa::launch_indexer_page_scores(bt, q_idx, w, n_heads, kc, page_size,
                                                       page_scores, ld_pages,
                                                       static_cast<hipStream_t>(stream)));
}

size_t dsa_indexer_topk_state_size(int32_t total_q) {
  return dsa::indexer_topk_state_bytes(total_q);
}

dsa_status dsa_indexer_topk(const dsa_batch *batch, const void *q_idx, int32_t q_dtype,
                            const float *w, int32_t n_heads, int32_t head_dim,
                            const dsa_paged_cache *keys, int32_t k, float *scores,
                            int64_t ld_scores, int32_t *indices, void *state,
                            size_t state_bytes, void *stream) {
  BatchArgs bt;
  CacheArgs kc;
  dsa_status st = check_batch(batch, &bt);
  if (st != DSA_OK) return st;
  if (keys == nullptr) return DSA_ERR_NULL;
  if (bt.total_q > 0 &&
      (q_idx == nullptr || w == nullptr || scores == nullptr || indices == nullptr))
    return DSA_ERR_NULL;
  st = check_cache(keys, bt, &kc);
  if (st != DSA_OK) return st;
  if (q_dtype != DSA_F32 && q_dtype != DSA_BF16) return DSA_ERR_DTYPE;
  if (n_heads < 1 || head_dim < 1 || kc.row_elems != head_dim || k < 1) return DSA_ERR_SHAPE;
  if (ld_scores < bt.max_seq_len || ld_scores < 1) return DSA_ERR_SHAPE;
  if (!aligned(q_idx, 16) || !aligned(w, 4) || !aligned(scores, 4) || !aligned(indices, 4))
    return DSA_ERR_SHAPE;
  if (!dsa::indexer_topk_supported(bt, q_dtype, n_heads, head_dim, kc)) return DSA_ERR_UNSUPPORTED;
  const size_t need = dsa::indexer_topk_state_bytes(bt.total_q);
  if (need > 0 && (state == nullptr || state_bytes < need || !aligned(state, 256)))
    return DSA_ERR_WORKSPACE;
  if (bt.total_q == 0) return DSA_OK;
  return launch_status(dsa::launch_indexer_topk(bt, q_idx, w, n_heads, kc, k, indices, scores,
                                                ld_scores, static_cast<uint32_t *>(state),
                                                static_cast<hipStream_t>(stream)));
}

dsa_status dsa_page_scores(const dsa_batch *batch, const float *scores, int64_t ld_scores,
                           int32_t page_size, float *page_scores, int64_t ld_pages, void *stream) {
  BatchArgs bt;
  const dsa_status st = check_batch(batch, &bt);
  if (st != DSA_OK) return st;
  if (bt.total_q > 0 && (scores == nullptr || page_scores == nullptr)) return DSA_ERR_NULL;
  if (page_size < 1 || ld_scores < bt.max_seq_len || ld_scores < 1) return DSA_ERR_SHAPE;
  if (ld_pages < dsa::candidate_bound(bt.max_seq_len, page_size) || ld_pages < 1)
    return DSA_ERR_SHAPE;
  if (!aligned(scores, 4) || !aligned(page_scores, 4)) return DSA_ERR_SHAPE;
  if (bt.total_q == 0) return DSA_OK;
  return launch_status(dsa::launch_page_scores(bt, scores, ld_scores, page_size, page_scores,
                                               ld_pages, static_cast<hipStream_t>(stream)));
}

size_t dsa_page_topk_workspace_size(int32_t total_q, int32_t max_seq_len, int32_t page_size,
                                    int32_t kp) {
  if (page_size < 1) return 0;
  return dsa::topk_workspace_bytes(total_q, dsa::candidate_bound(max_seq_len, page_size), kp);
}

dsa_status dsa_page_topk(const dsa_batch *batch, const float *page_scores, int64_t ld_pages,
                         int32_t page_size, int32_t kp, int32_t *pages, int32_t *indices,
                         void *workspace, size_t workspace_bytes, void *stream) {
  BatchArgs bt;
  const dsa_status st = check_batch(batch, &bt);
  if (st != DSA_OK) return st;
  if (bt.total_q > 0 && (page_scores == nullptr || pages == nullptr)) return DSA_ERR_NULL;
  if (page_size < 1 || kp < 1) return DSA_ERR_SHAPE;
  const int32_t max_pages = dsa::candidate_bound(bt.max_seq_len, page_size);
  if (ld_pages < max_pages || ld_pages < 1) return DSA_ERR_SHAPE;
  if ((int64_t)kp * page_size > (int64_t)0x7FFFFFFF) return DSA_ERR_SHAPE;
  if (!aligned(page_scores, 4) || !aligned(pages, 4) || (indices != nullptr && !aligned(indices, 4)))
    return DSA_ERR_SHAPE;
  if (!dsa::topk_supported(max_pages, kp)) return DSA_ERR_UNSUPPORTED;
  const size_t need = dsa::topk_workspace_bytes(bt.total_q, max_pages, kp);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 16)))
    return DSA_ERR_WORKSPACE;
  if (bt.total_q == 0) return DSA_OK;
  return launch_status(dsa::launch_page_topk(bt, page_scores, ld_pages, page_size, kp, pages,
                                             indices, workspace, workspace_bytes,
                                             static_cast<hipStream_t>(stream)));
}

dsa_status dsa_kv_append(const int32_t *slot_mapping, int32_t n_tokens, const void *latent,
                         const dsa_paged_cache *kv, const void *idx_keys, int32_t key_dtype,
                         const dsa_paged_cache *k_idx, void *stream) {
  if (n_tokens < 0) return DSA_ERR_SHAPE;
  if (kv == nullptr && k_idx == nullptr) return DSA_ERR_NULL;
  // with no tokens the row and slot arrays may be empty (NULL)
  if (n_tokens > 0 && ((kv == nullptr) != (latent == nullptr) ||
                       (k_idx == nullptr) != (idx_keys == nullptr) || slot_mapping == nullptr))
    return DSA_ERR_NULL;
  if (slot_mapping != nullptr && !aligned(slot_mapping, 4)) return DSA_ERR_SHAPE;
  CacheArgs kc, ic;
  if (kv != nullptr) {
    const dsa_status st = check_cache_geometry(kv, &kc);
    if (st != DSA_OK) return st;
    if (kc.dtype == DSA_FP8_E4M3) return DSA_ERR_DTYPE;
    if (latent != nullptr && !aligned(latent, kc.dtype == DSA_F32 ? 4 : 2)) return DSA_ERR_SHAPE;
  }
  if (k_idx != nullptr) {
    const dsa_status st = check_cache_geometry(k_idx, &ic);
    if (st != DSA_OK) return st;
    if (key_dtype != DSA_F32 && key_dtype != DSA_BF16) return DSA_ERR_DTYPE;
    if (ic.dtype != DSA_FP8_E4M3 && ic.dtype != key_dtype) return DSA_ERR_DTYPE;
    if (idx_keys != nullptr && !aligned(idx_keys, key_dtype == DSA_F32 ? 4 : 2))
      return DSA_ERR_SHAPE;
  }
  if (n_tokens == 0) return DSA_OK;
  // one wave per (token, cache): the grid must fit
  if ((int64_t)n_tokens * 2 > (int64_t)0x7FFFFFFF) return DSA_ERR_SHAPE;
  return launch_status(dsa::launch_kv_append(slot_mapping, n_tokens, latent,
                                             kv != nullptr ? &kc : nullptr, idx_keys, key_dtype,
                                             k_idx != nullptr ? &ic : nullptr,
                                             static_cast<hipStream_t>(stream)));
}

}  // extern "C"
