/*
 * dsa.h — C ABI of the MI355X (gfx950) sparse-attention decode library.
 *
 * The library computes the three device steps of DeepSeek-style sparse
 * attention over a paged latent KV cache, as GLM-5.2 uses it:
 *
 *   1. dsa_indexer_scores — lightning-indexer scores of every causal past
 *      token ("vLLM Inference Path: GLM-5.2 as an Example", section "DSA
 *      Indexer"; "Making GLM-5.2 Sparse on TPUs", section "Separate the
 *      indexer from the attention it controls"):
 *          I[t, s] = sum_j w[t, j] * ReLU(q_idx[t, j, :] . k_idx[s, :]),  s <= t
 *   2. dsa_topk — the k best token positions per query row ("GLM-5.2 on vLLM
 *      Ascend: Request-to-Backend Inference Path", section "8. The SFA
 *      backend, step by step": 2,048 positions are requested, and what is
 *      selected is individual token positions, not compressed blocks);
 *   3. dsa_sparse_mla_fwd — absorbed MLA attention over only the selected
 *      cache rows ("vLLM Inference Path: GLM-5.2 as an Example", sections
 *      "MLA Projections and KV State" and "Sparse MLA Attention"; "Making
 *      GLM-5.2 Sparse on TPUs", section "Separate the indexer from the
 *      attention it controls").
 *
 * IndexShare ("GLM-5.2 on vLLM Ascend ...", section "7. GLM-5.2
 * shared-indexer construction") is the caller passing one `indices` buffer to
 * several dsa_sparse_mla_fwd calls, one per layer.
 *
 * Conventions common to every call
 * --------------------------------
 * - Every pointer argument is a DEVICE pointer unless its comment says host.
 *   Struct arguments themselves (dsa_batch, dsa_paged_cache) live on the host
 *   and are only read during the call.
 * - The caller owns every buffer: inputs, outputs, workspace and stream. The
 *   library never allocates or frees device memory and never synchronizes.
 *   All work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *   and is complete when that stream is.
 * - Errors are status codes. All host-visible arguments are validated before
 *   anything is enqueued; on an error nothing is enqueued and no output is
 *   touched. No call aborts or throws across the ABI.
 * - An empty batch (total_q = 0) is valid: the call checks its arguments,
 *   enqueues nothing and returns DSA_OK; its per-row arrays (queries,
 *   weights, scores, indices, pages, outputs) and the batch's metadata
 *   arrays may then be NULL.
 * - Device-resident metadata (lengths, block tables, indices) is trusted to
 *   be in range, but clamped so that malformed values never make a kernel
 *   read or write outside the buffers described here: page ids are clamped
 *   to [0, num_pages), logical pages past a sequence's length are never read,
 *   rows with zero queries are empty, and indices outside [0, t] are treated
 *   as padding. Malformed metadata thus gives wrong but memory-safe results.
 * - Calls on different streams may run concurrently; apart from the scratch
 *   array of dsa_sparse_mla_fwd_noalloc (below), the library keeps no
 *   mutable state. A workspace, or the state buffer of dsa_indexer_topk,
 *   must not be shared by calls that may overlap.
 *
 * Row positions. Query rows are flattened over the batch: row r = cu_q[b] + i
 * (0 <= i < q_b = cu_q[b+1] - cu_q[b]) is the token at absolute position
 * t_r = seq_lens[b] - q_b + i, where seq_lens[b] counts this step's q_b new
 * tokens ("Making GLM-5.2 Sparse on TPUs", section "Pack requests and reuse
 * prefixes": causality uses prefix length plus local offset). Row r may use
 * positions 0..t_r of sequence b, its own position included (its key is
 * written to the cache before selection).
 *
 * Paging. Logical position s of sequence b lives in physical page
 * block_table[b * bt_stride + s / page_size], slot s % page_size. One block
 * table serves the indexer-key cache and every layer's latent cache; the
 * caches themselves are separate buffers.
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_ABI_VERSION 1

typedef enum {
  DSA_OK = 0,
  DSA_ERR_NULL = 1,        /* a required pointer is NULL */
  DSA_ERR_SHAPE = 2,       /* a size, stride or bound is out of range or inconsistent */
  DSA_ERR_DTYPE = 3,       /* an element type is not allowed for this argument */
  DSA_ERR_WORKSPACE = 4,   /* workspace missing or smaller than the size query returns */
  DSA_ERR_UNSUPPORTED = 5, /* a valid combination the library has no kernel for */
  DSA_ERR_LAUNCH = 6       /* the HIP runtime rejected a kernel launch */
} dsa_status;

typedef enum {
  DSA_F32 = 0,      /* IEEE binary32 */
  DSA_BF16 = 1,     /* bfloat16 */
  DSA_FP8_E4M3 = 2  /* OCP FP8 E4M3FN: bias 7, no infinities, S.1111.111 = NaN */
} dsa_dtype;

/* Packed batch metadata, shared by all three calls. The struct is a host
 * object; the arrays it points to are device arrays. */
typedef struct {
  const int32_t *block_table; /* device [batch, bt_stride]: physical page ids */
  const int32_t *seq_lens;    /* device [batch]: KV length L_b incl. this step's queries */
  const int32_t *cu_q;        /* device [batch + 1]: query-row offsets, cu_q[0] = 0, non-decreasing */
  int32_t batch;              /* number of sequences, >= 0 */
  int32_t bt_stride;          /* block-table row stride in entries, >= ceil(max_seq_len / page_size) */
  int32_t total_q;            /* host copy of cu_q[batch]: number of query rows T */
  int32_t max_seq_len;        /* host bound: >= every seq_lens[b] */
  int32_t max_q;              /* host bound: >= every q_b; 0 < max_q <= total_q unless total_q = 0 */
} dsa_batch;

/* One paged cache: [num_pages, page_size, row_elems] elements of `dtype`,
 * rows contiguous. For DSA_FP8_E4M3 `scale` holds one fp32 dequantisation
 * factor per token, [num_pages, page_size], and the stored key is
 * scale * e4m3(byte) ("GLM-5.2 on vLLM Ascend ...", section "7. GLM-5.2
 * shared-indexer construction": FP8 e4m3 keys carry FP32 scales). Scales
 * are finite and >= 0, as dsa_kv_append writes them (max|k| / 448); the
 * streaming indexer applies a key's scale after the ReLU, which equals the
 * definition only for non-negative scales, so a negative scale gives
 * unspecified scores. */
typedef struct {
  const void *data;   /* device */
  const float *scale; /* device [num_pages, page_size]; required for fp8, else ignored */
  int64_t num_pages;  /* > 0 */
  int32_t page_size;  /* tokens per page, > 0 */
  int32_t row_elems;  /* elements per token row (the row stride), > 0 */
  int32_t dtype;      /* dsa_dtype */
} dsa_paged_cache;

/* Stable, human-readable name of a status code (a static string). */
const char *dsa_status_str(dsa_status status);

/* DSA_ABI_VERSION of the built library. */
int32_t dsa_abi_version(void);

/*
 * Lightning-indexer scores ("vLLM Inference Path: GLM-5.2 as an Example",
 * section "DSA Indexer"; "Making GLM-5.2 Sparse on TPUs", section "Separate
 * the indexer from the attention it controls").
 *
 * For every query row r and every position s in [0, t_r]:
 *   scores[r * ld_scores + s] = sum_j w[r, j] * ReLU(sum_d q_idx[r, j, d] * k(s)[d])
 * where k(s) is the key row of position s (times its scale for fp8 keys).
 * Accumulation is fp32. Entries s > t_r of a row are not written.
 *
 *   q_idx   device [total_q, n_heads, head_dim], element type q_dtype (F32 or BF16)
 *   w       device [total_q, n_heads] fp32 per-head weights
 *   keys    paged key cache, row_elems == head_dim, dtype F32, BF16 or FP8_E4M3;
 *           F32 queries need F32 keys
 *   scores  device [total_q, ld_scores] fp32 output; ld_scores >= max_seq_len
 *
 * Errors: DSA_ERR_NULL for a NULL batch, keys, key data or fp8 scale, or
 * (with total_q > 0) a NULL q_idx, w, scores or metadata array; DSA_ERR_SHAPE for
 * non-positive heads/dims/page size, row_elems != head_dim, ld_scores <
 * max_seq_len, or inconsistent batch bounds; DSA_ERR_DTYPE for unsupported
 * element types; DSA_ERR_LAUNCH if the runtime rejects the launch.
 */
dsa_status dsa_indexer_scores(const dsa_batch *batch, const void *q_idx, int32_t q_dtype,
                              const float *w, int32_t n_heads, int32_t head_dim,
                              const dsa_paged_cache *keys, float *scores, int64_t ld_scores,
                              void *stream);

/* Bytes of workspace dsa_topk needs for these host bounds (0 if none). */
size_t dsa_topk_workspace_size(int32_t total_q, int32_t max_seq_len, int32_t k);

/*
 * Per-row top-k of the indexer scores ("GLM-5.2 on vLLM Ascend ...", section
 * "8. The SFA backend, step by step"; "vLLM Inference Path: GLM-5.2 as an
 * Example", section "DSA Indexer").
 *
 * For row r with n = t_r + 1 candidates (reads scores[r * ld_scores + s] for
 * s < n only) keeps m = min(k, n) positions: the largest scores, equal scores
 * ordered by lower position first, -0.0 equal to +0.0. Scores must not be
 * NaN (NaN ordering is unspecified). indices[r * k + 0 .. m-1] receives the
 * kept positions in ascending order and indices[r * k + m .. k-1] = -1.
 * Every entry of indices[total_q, k] is written.
 *
 *   scores    device [total_q, ld_scores] fp32, as written by dsa_indexer_scores
 *   indices   device [total_q, k] int32 output
 *   workspace device, >= dsa_topk_workspace_size(total_q, max_seq_len, k) bytes
 *             (may be NULL when that size is 0)
 *
 * Errors: DSA_ERR_NULL, DSA_ERR_SHAPE (k < 1, ld_scores < max_seq_len, bad
 * bounds), DSA_ERR_WORKSPACE, DSA_ERR_LAUNCH.
 */
dsa_status dsa_topk(const dsa_batch *batch, const float *scores, int64_t ld_scores, int32_t k,
                    int32_t *indices, void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of the per-row state dsa_indexer_topk keeps between calls. */
size_t dsa_indexer_topk_state_size(int32_t total_q);

/*
 * The indexer and the top-k in one launch ("Making GLM-5.2 Sparse on TPUs",
 * section "Stream indexer scores over live context": the selection is fed
 * from the streaming indexer; section "What the stack now delivers": token
 * top-k over few rows is the latency to cut).
 *
 * Equal to dsa_indexer_scores followed by dsa_topk with the same k: the same
 * scores in `scores` and bit-identical indices. The workgroups that score a
 * row also count their scores' top 11 key bits into the row's histogram in
 * `state`, and the row's last workgroup to finish (an atomic count; no
 * workgroup waits for another) selects the row from that histogram and the
 * scores, so the selection needs no pass of its own over the row.
 *
 * Supported for decode rows: at most one query row per sequence (max_q <= 1),
 * bf16 queries, head_dim 128, 16, 32 or 64 heads, bf16 or fp8 keys in pages
 * of a multiple of 64 rows, max_seq_len <= 16384; otherwise
 * DSA_ERR_UNSUPPORTED (the two-call route covers every case). On MI355X the
 * two calls are faster on every shape measured (1 to 32 rows of 2K to 16K
 * positions): the final selection runs on the row's one four-wave workgroup
 * instead of a 16-wave one, and each workgroup's device-scope release costs
 * more than the launch it saves. Rows that no sequence's query range holds
 * are not written.
 *
 *   scores  device [total_q, ld_scores] fp32, written as by dsa_indexer_scores
 *   indices device [total_q, k] int32, written as by dsa_topk
 *   state   device, >= dsa_indexer_topk_state_size(total_q) bytes, 256-byte
 *           aligned. It must be zero-filled before its first use (one
 *           hipMemset after allocation); every call that completes leaves
 *           the part it used zero-filled again, so one state buffer serves
 *           every later call with as many rows or fewer. Calls that overlap
 *           in time (other streams) need separate state buffers. The caller
 *           owns it.
 *
 * Errors: as for the two calls; DSA_ERR_WORKSPACE for a missing, short or
 * misaligned state; DSA_ERR_UNSUPPORTED outside the shapes above.
 */
dsa_status dsa_indexer_topk(const dsa_batch *batch, const void *q_idx, int32_t q_dtype,
                            const float *w, int32_t n_heads, int32_t head_dim,
                            const dsa_paged_cache *keys, int32_t k, float *scores,
                            int64_t ld_scores, int32_t *indices, void *state,
                            size_t state_bytes, void *stream);

/* Bytes of workspace dsa_sparse_mla_fwd needs for these host bounds. */
size_t dsa_sparse_mla_workspace_size(int32_t total_q, int32_t n_heads, int32_t d_latent,
                                     int32_t k);

/*
 * Absorbed sparse MLA attention over the selected rows ("vLLM Inference
 * Path: GLM-5.2 as an Example", sections "MLA Projections and KV State" and
 * "Sparse MLA Attention"; "Making GLM-5.2 Sparse on TPUs", section "Separate
 * the indexer from the attention it controls").
 *
 * Each cache row is [latent (d_latent) | RoPE key (d_rope)]; each query row
 * holds n_heads absorbed queries of the same width. For row r, head h and the
 * selected positions S_r = { indices[r * k + i] : 0 <= indices[r*k+i] <= t_r }:
 *   l_s      = scale * q[r, h, :] . row(s)                 (all d_latent + d_rope dims)
 *   out[r,h] = sum_{s in S_r} softmax_s(l) * row(s)[0 : d_latent]
 *   lse[r,h] = log sum_{s in S_r} exp(l_s)                  (natural log)
 * Rows with no selected position get out = 0 and lse = -inf. A position
 * listed twice counts twice. The scale is passed explicitly (the pages tie it
 * to 1/sqrt(192 + 64), not to the absorbed width). Accumulation is fp32.
 *
 * bf16 with d_latent 512, d_rope 64 and 1..64 heads runs on the matrix
 * cores, each tile of selected rows feeding 64 (query, head) columns; with
 * fewer than 64 heads the missing columns are computed on zero queries, so a
 * head-sharded share costs about what 64 heads cost (dsa_sparse_mla_fwd_qblocked
 * fills the columns with other queries instead). Other shapes run on a
 * plain kernel.
 *
 *   q        device [total_q, n_heads, d_latent + d_rope], element type q_dtype
 *   kv       paged latent cache, row_elems == d_latent + d_rope, dtype == q_dtype
 *            (F32 or BF16)
 *   indices  device [total_q, k] int32, e.g. from dsa_topk
 *   out      device [total_q, n_heads, d_latent] fp32 output (fully written)
 *   lse      device [total_q, n_heads] fp32 output, or NULL
 *   workspace device, >= dsa_sparse_mla_workspace_size(total_q, n_heads, d_latent, k)
 *
 *   scale    finite and > 0
 *
 * Errors: DSA_ERR_NULL (a NULL kv, or with total_q > 0 a NULL q, out or
 * `indices`: a layer that has neither its own nor a shared top-k buffer is
 * rejected), DSA_ERR_SHAPE (also a scale that is not finite and positive), DSA_ERR_DTYPE,
 * DSA_ERR_WORKSPACE, DSA_ERR_LAUNCH.
 */
dsa_status dsa_sparse_mla_fwd(const dsa_batch *batch, const void *q, int32_t q_dtype,
                              int32_t n_heads, int32_t d_latent, int32_t d_rope,
                              const dsa_paged_cache *kv, const int32_t *indices, int32_t k,
                              float scale, float *out, float *lse, void *workspace,
                              size_t workspace_bytes, void *stream);

/*
 * dsa_sparse_mla_fwd for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation. Identical arguments, results bit for bit and errors, except
 * that there is no workspace argument: the split partials go to a static
 * device array that the library owns, DSA_MLA_NOALLOC_SCRATCH_BYTES per GPU,
 * held from the library's load on that GPU until the process ends. The call
 * allocates and frees nothing.
 *
 * Limit: a call whose dsa_sparse_mla_workspace_size(total_q, n_heads,
 * d_latent, k) exceeds DSA_MLA_NOALLOC_SCRATCH_BYTES returns
 * DSA_ERR_WORKSPACE before anything is enqueued (at k = 2048 every batch
 * size fits: the partials peak just under the limit at 255 query rows).
 *
 * All calls on one GPU share that GPU's array: calls that may overlap on one
 * GPU (several streams, several host threads) race and give undefined
 * results; calls ordered on one stream do not. The first call on a device
 * looks up that device's copy of the array (the device current on the
 * calling thread); DSA_ERR_LAUNCH if that lookup fails.
 */
#define DSA_MLA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
dsa_status dsa_sparse_mla_fwd_noalloc(const dsa_batch *batch, const void *q, int32_t q_dtype,
                                      int32_t n_heads, int32_t d_latent, int32_t d_rope,
                                      const dsa_paged_cache *kv, const int32_t *indices, int32_t k,
                                      float scale, float *out, float *lse, void *stream);

/*
 * IndexShare over several layers in one call ("GLM-5.2 on vLLM Ascend:
 * Request-to-Backend Inference Path", section 7: one indexer's top-k is
 * reused by the attention of the layers that share it; "vLLM Inference Path:
 * GLM-5.2 as an Example", section "DSA Indexer").
 *
 * Exactly n_layers calls of dsa_sparse_mla_fwd with the same batch, indices,
 * k, scale and shapes, and with layer l's q[l], kv[l], out[l] and lse[l]; the
 * results are bit-identical to those calls. The layers run as one launch, so
 * one layer's start-up and tail overlap another's work.
 *
 *   n_layers  1 .. 8
 *   q, out    HOST arrays of n_layers DEVICE pointers, as in dsa_sparse_mla_fwd
 *   kv        HOST array of n_layers caches: one element type, row width and
 *             page size (the batch's block table addresses all of them)
 *   lse       HOST array of n_layers device pointers (entries may be NULL),
 *             or NULL for no lse in any layer
 *   workspace device, >= dsa_sparse_mla_layers_workspace_size(n_layers, ...)
 *
 * Errors: as dsa_sparse_mla_fwd, plus DSA_ERR_SHAPE for n_layers outside
 * 1..8 or caches of different page sizes, DSA_ERR_NULL for a NULL q, kv or
 * out array.
 */
size_t dsa_sparse_mla_layers_workspace_size(int32_t n_layers, int32_t total_q, int32_t n_heads,
                                            int32_t d_latent, int32_t k);
dsa_status dsa_sparse_mla_fwd_layers(const dsa_batch *batch, int32_t n_layers,
                                     const void *const *q, int32_t q_dtype, int32_t n_heads,
                                     int32_t d_latent, int32_t d_rope, const dsa_paged_cache *kv,
                                     const int32_t *indices, int32_t k, float scale,
                                     float *const *out, float *const *lse, void *workspace,
                                     size_t workspace_bytes, void *stream);

/*
 * Query-blocked sparse MLA ("Making GLM-5.2 Sparse on TPUs", section "Reuse
 * pages across queries": a block of queries loads the union of its selected
 * rows once, and a membership mask restores each query's own selection
 * before the softmax). The same operation as dsa_sparse_mla_fwd on the same
 * arguments; only the order of the fp32 sums differs, so results agree to
 * rounding, not bit for bit.
 *
 * Query rows are taken in blocks of QB consecutive rows (QB = 4 for 16 or
 * more heads, 8 for 8 heads), and each block's selections are merged into one
 * list of physical rows with a membership mask per row. Every row of the
 * list is loaded once per block and group of 64 / QB heads, and feeds 64
 * (query, head) pairs. This pays when the block's queries select overlapping
 * rows, or when a query has fewer than 64 heads (a head-sharded layer); when
 * they share nothing, it costs about QB times the logit work of the
 * per-query call. The merge needs each row's valid entries (positions in
 * [0, t_r]) first and strictly ascending, as dsa_topk and dsa_page_topk write
 * them, and the block's rows in one sequence; any other block is attended to
 * as given, each entry counted once per occurrence, like dsa_sparse_mla_fwd.
 *
 * Arguments as for dsa_sparse_mla_fwd; the workspace holds the unions.
 *   workspace  device, >= dsa_sparse_mla_qblocked_workspace_size(total_q, n_heads, k)
 *
 * Supported: bf16, d_latent 512, d_rope 64, n_heads 8 or 16, 32, 48, 64, QB * k
 * <= 2^20, max_seq_len < 2^29 and fewer than 2^32 rows in the cache;
 * otherwise DSA_ERR_UNSUPPORTED. Other errors as for dsa_sparse_mla_fwd.
 */
size_t dsa_sparse_mla_qblocked_workspace_size(int32_t total_q, int32_t n_heads, int32_t k);
dsa_status dsa_sparse_mla_fwd_qblocked(const dsa_batch *batch, const void *q, int32_t q_dtype,
                                       int32_t n_heads, int32_t d_latent, int32_t d_rope,
                                       const dsa_paged_cache *kv, const int32_t *indices, int32_t k,
                                       float scale, float *out, float *lse, void *workspace,
                                       size_t workspace_bytes, void *stream);

/*
 * Page scores for page-budget selection, the alternative to token top-k that
 * bounds the pages attention reads ("Making GLM-5.2 Sparse on TPUs", section
 * "Make the sparsity unit match the memory unit": a page is ranked by its
 * highest legal token score, and the causal and valid-length masks apply
 * before that maximum, so an invisible token never promotes its page;
 * section "Stream indexer scores over live context": the selection consumes
 * page maxima).
 *
 * Pages are logical pages of page_size positions of the row's sequence (the
 * block table plays no part). For row r and every page p <= t_r / page_size:
 *   page_scores[r * ld_pages + p] = max { scores[r * ld_scores + s] :
 *                                         p * page_size <= s < (p + 1) * page_size, s <= t_r }
 * Pages past t_r / page_size are not written; scores past t_r are never read.
 *
 *   scores       device [total_q, ld_scores] fp32 token scores (dsa_indexer_scores)
 *   page_scores  device [total_q, ld_pages] fp32 output, ld_pages >= ceil(max_seq_len / page_size)
 *
 * Errors: DSA_ERR_NULL, DSA_ERR_SHAPE (page_size < 1, short row strides, bad
 * bounds, misaligned pointers), DSA_ERR_LAUNCH.
 */
dsa_status dsa_page_scores(const dsa_batch *batch, const float *scores, int64_t ld_scores,
                           int32_t page_size, float *page_scores, int64_t ld_pages, void *stream);

/*
 * The same page scores straight from the indexer, with no token score in
 * memory ("Making GLM-5.2 Sparse on TPUs", section "Stream indexer scores over
 * live context": the streaming indexer applies the masks and pools page
 * maxima on chip, so only page scores reach HBM).
 *
 * Equal to dsa_indexer_scores followed by dsa_page_scores with the same
 * page_size, and bit-identical to that pair where it runs (same arithmetic per
 * token score). Arguments as for dsa_indexer_scores, plus page_size and the
 * page_scores output of dsa_page_scores.
 *
 * Supported where the key stream runs in 64-key blocks: bf16 queries, head_dim
 * 128, 16, 32 or 64 heads, bf16 or fp8 keys in pages of a multiple of 64 rows,
 * fewer than 16 queries per sequence, and page_size 64 (one streamed block);
 * otherwise DSA_ERR_UNSUPPORTED (the two-call route covers every case).
 * Other errors as for the two calls.
 */
dsa_status dsa_indexer_page_scores(const dsa_batch *batch, const void *q_idx, int32_t q_dtype,
                                   const float *w, int32_t n_heads, int32_t head_dim,
                                   const dsa_paged_cache *keys, int32_t page_size,
                                   float *page_scores, int64_t ld_pages, void *stream);

/* Bytes of workspace dsa_page_topk needs for these host bounds (0 if none). */
size_t dsa_page_topk_workspace_size(int32_t total_q, int32_t max_seq_len, int32_t page_size,
                                    int32_t kp);

/*
 * Page-budget selection (same sections): per row the kp pages with the
 * highest page scores among pages 0 .. t_r / page_size, equal scores ordered
 * by lower page first, listed in ascending page order and padded with -1:
 * pages[r * kp + i]. With `indices` non-NULL, also the legal token positions
 * of those pages, the index list of dsa_sparse_mla_fwd with k = kp * page_size:
 *   indices[r * kp * page_size + i * page_size + o] = pages[r * kp + i] * page_size + o
 * when that page is not -1 and the position is <= t_r, else -1 (ascending
 * among the valid entries).
 *
 *   page_scores  device [total_q, ld_pages] fp32, as written by dsa_page_scores
 *   pages        device [total_q, kp] int32 output (fully written)
 *   indices      device [total_q, kp * page_size] int32 output (fully written), or NULL
 *   workspace    device, >= dsa_page_topk_workspace_size(...) bytes (NULL when 0)
 *
 * Errors: DSA_ERR_NULL, DSA_ERR_SHAPE (page_size or kp < 1, short ld_pages,
 * kp * page_size past int32, misaligned pointers), DSA_ERR_WORKSPACE,
 * DSA_ERR_UNSUPPORTED (more pages per row than the selection handles),
 * DSA_ERR_LAUNCH.
 */
dsa_status dsa_page_topk(const dsa_batch *batch, const float *page_scores, int64_t ld_pages,
                         int32_t page_size, int32_t kp, int32_t *pages, int32_t *indices,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * Append this step's new tokens to the paged caches, the write that precedes
 * selection ("GLM-5.2 on vLLM Ascend: Request-to-Backend Inference Path",
 * section "8. The SFA backend, step by step", "Write paged cache": the slot
 * mapping scatters the new latent KV and, for layers that own an indexer, the
 * new indexer keys and scales into their physical pages; "Making GLM-5.2
 * Sparse on TPUs", section "Append new KV without moving the resident
 * cache": only the new rows are written, the resident ones stay intact).
 *
 * Token i goes to physical slot slot_mapping[i] = page * page_size + offset
 * of every cache given. A negative slot, or one at or past num_pages *
 * page_size, skips the token. No other byte of either cache is written. When
 * two tokens map to one slot, which of them lands is unspecified.
 *
 *   slot_mapping  device [n_tokens] int32
 *   latent        device [n_tokens, kv->row_elems] of kv->dtype (F32 or BF16),
 *                 copied into the latent cache; NULL together with kv = NULL
 *   kv            paged latent cache, written in place (the call writes through
 *                 its `data` pointer)
 *   idx_keys      device [n_tokens, k_idx->row_elems] of key_dtype (F32 or
 *                 BF16), finite; NULL together with k_idx = NULL
 *   k_idx         paged indexer-key cache, written in place (data, and scale
 *                 for fp8). An F32 or BF16 cache takes a copy of the row and
 *                 needs key_dtype equal to its dtype. An FP8_E4M3 cache takes
 *                 the row quantised per token: sigma = max_d |k[d]| / 448 in
 *                 fp32 (sigma = 1 for an all-zero row), byte[d] = the e4m3
 *                 value nearest to clamp(k[d] / sigma, -448, 448), ties to the
 *                 even code, and scale[slot] = sigma, so that sigma *
 *                 e4m3(byte) is the stored key.
 *
 * With n_tokens = 0 nothing is enqueued and the row and slot arrays may be
 * NULL.
 *
 * Errors: DSA_ERR_NULL (both caches NULL; with n_tokens > 0, a cache without
 * its source rows or the reverse, or a NULL slot_mapping; NULL cache data or
 * fp8 scale), DSA_ERR_SHAPE (n_tokens < 0, bad cache geometry, misaligned
 * pointers), DSA_ERR_DTYPE (an fp8 latent cache, a key type that does not fit
 * the cache), DSA_ERR_LAUNCH.
 */
dsa_status dsa_kv_append(const int32_t *slot_mapping, int32_t n_tokens, const void *latent,
                         const dsa_paged_cache *kv, const void *idx_keys, int32_t key_dtype,
                         const dsa_paged_cache *k_idx, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H_ */
