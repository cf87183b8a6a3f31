// Internal launcher interface between the C ABI (dsa_api.cpp) and the kernel
// translation units. Arguments have already been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dsa.h"

namespace dsa {

struct BatchArgs {
  const int32_t *block_table;
  const int32_t *seq_lens;
  const int32_t *cu_q;
  int32_t batch;
  int64_t bt_stride;
  int32_t total_q;
  int32_t max_seq_len;
  int32_t max_q;
};

struct CacheArgs {
  const void *data;
  const float *scale;
  int64_t num_pages;
  int32_t page_size;
  int32_t row_elems;
  int32_t dtype;
};

hipError_t launch_indexer_scores(const BatchArgs &bt, const void *q_idx, int32_t q_dtype,
                                 const float *w, int32_t n_heads, int32_t head_dim,
                                 const CacheArgs &keys, float *scores, int64_t ld_scores,
                                 hipStream_t stream);

// Top-k over candidates: positions (unit 1) or pages of `unit` positions;
// sizes and support are in candidates per row (candidate_bound of the batch).
int candidate_bound(int32_t max_seq_len, int32_t unit);
// Page maxima straight from the indexer (selection pages of 64 positions;
// bf16 queries of width 128; streamed key caches).
bool indexer_page_max_supported(const BatchArgs &bt, int32_t q_dtype, int32_t n_heads,
                                int32_t head_dim, const CacheArgs &keys, int32_t sel_page);
hipError_t launch_indexer_page_scores(const BatchArgs &bt, const void *q_idx, const float *w,
                                      int32_t n_heads, const CacheArgs &keys, int32_t sel_page,
                                      float *page_scores, int64_t ld_pages, hipStream_t stream);

// Indexer scores and their top-k in one launch (one query row per sequence,
// streamed keys, rows of up to 16K positions); `state` is zero between calls.
bool indexer_topk_supported(const BatchArgs &bt, int32_t q_dtype, int32_t n_heads,
                            int32_t head_dim, const CacheArgs &keys);
size_t indexer_topk_state_bytes(int32_t total_q);
hipError_t launch_indexer_topk(const BatchArgs &bt, const void *q_idx, const float *w,
                               int32_t n_heads, const CacheArgs &keys, int32_t k,
                               int32_t *indices, float *scores, int64_t ld_scores,
                               uint32_t *state, hipStream_t stream);

size_t topk_workspace_bytes(int32_t total_q, int32_t max_cands, int32_t k);
bool topk_supported(int32_t max_cands, int32_t k);
// expand (page candidates only): also write the kept pages' positions there
// when the selection kernel can; *expanded tells whether it did.
hipError_t launch_topk(const BatchArgs &bt, const float *scores, int64_t ld_scores, int32_t k,
                       int32_t unit, int32_t *indices, void *workspace, size_t ws_bytes,
                       hipStream_t stream, int32_t *expand = nullptr, bool *expanded = nullptr);

// One attention layer of a sparse MLA call: its query, latent cache and outputs.
struct MlaLayer {
  const void *q;
  CacheArgs kv;
  float *out;
  float *lse;  // may be null
};
constexpr int kMlaMaxLayers = 8;  // layers one call may take (sharing one index list)

int mla_num_splits(int32_t total_q, int32_t n_heads, int32_t d_latent, int32_t k);
int mla_max_k();  // largest k of the 64-head bf16 MFMA path
// workspace of one layer; a call over n layers needs n times this
size_t mla_workspace_bytes(int32_t total_q, int32_t n_heads, int32_t d_latent, int32_t k);
// Device address of the calling thread's current GPU's copy of the library's
// static MLA scratch array (DSA_MLA_NOALLOC_SCRATCH_BYTES), found once per device.
hipError_t mla_scratch(void **ptr);
hipError_t launch_sparse_mla(const BatchArgs &bt, const MlaLayer *layers, int n_layers,
                             int32_t q_dtype, int32_t n_heads, int32_t d_latent, int32_t d_rope,
                             const int32_t *indices, int32_t k, float scale, void *workspace,
                             size_t ws_bytes, hipStream_t stream);

// Query-blocked sparse MLA (bf16, 512 + 64; 8 heads, or 16 to 64 in groups
// of 16): the union of each block of query rows, then attention over it.
int mla_qblock_qb(int32_t n_heads);  // query rows per block
bool mla_qblock_supported(int32_t q_dtype, int32_t n_heads, int32_t d_latent, int32_t d_rope,
                          int32_t k);
size_t mla_qblock_workspace_bytes(int32_t total_q, int32_t n_heads, int32_t k);
hipError_t launch_sparse_mla_qblocked(const BatchArgs &bt, const MlaLayer &layer, int32_t n_heads,
                                      const int32_t *indices, int32_t k, float scale,
                                      void *workspace, hipStream_t stream);

hipError_t launch_page_scores(const BatchArgs &bt, const float *scores, int64_t ld,
                              int32_t page_size, float *page_scores, int64_t ld_pages,
                              hipStream_t stream);
hipError_t launch_page_topk(const BatchArgs &bt, const float *page_scores, int64_t ld_pages,
                            int32_t page_size, int32_t kp, int32_t *pages, int32_t *indices,
                            void *workspace, size_t ws_bytes, hipStream_t stream);

hipError_t launch_kv_append(const int32_t *slots, int32_t n_tokens, const void *latent,
                            const CacheArgs *kv, const void *keys, int32_t key_dtype,
                            const CacheArgs *kidx, hipStream_t stream);

}  // namespace dsa
