// Host-side checks of the C-ABI library, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on its host code (tests/test_sanitize.py):
//  1. the clamping arithmetic the kernels apply to device metadata (row_clamp,
//     clamp_page from dsa_device.h, shared with the kernels) keeps every
//     position and page id in bounds for malformed lengths, offsets and
//     page ids, and leaves well-formed metadata exact;
//  2. every entry point rejects bad arguments with its status code before
//     any HIP call, and takes an empty batch as a validated no-op.
// No GPU is used: every call below fails validation or has nothing to do.
#include <stdio.h>
#include <stdlib.h>

#include <random>

#include "../../sparse_attention_decode_lightning_amd/csrc/dsa_device.h"
#include "dsa.h"

static int failures = 0;
#define CHECK(cond)                                                  \
  do {                                                               \
    if (!(cond)) {                                                   \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                    \
    }                                                                \
  } while (0)

static void check_clamps() {
  std::mt19937_64 rng(12345);
  auto pick = [&](int lo, int hi) { return (int)(lo + (int64_t)(rng() % (uint64_t)((int64_t)hi - lo + 1))); };
  const int extremes[] = {-2147483647 - 1, -70000, -1, 0, 1, 63, 64, 65, 8191, 8192, 245760, 2147483647};
  for (int it = 0; it < 400000; ++it) {
    const int total_q = pick(1, 5000), max_seq_len = pick(1, 300000);
    auto wild = [&]() { return (rng() & 3) == 0 ? extremes[rng() % 12] : pick(-10, 300010); };
    const int c0 = wild(), c1 = wild(), len = wild();
    const int row = pick(0, total_q - 1);
    const dsa::RowInfo ri = dsa::row_clamp(3, c0, c1, len, total_q, max_seq_len, row);
    // whatever the metadata, the row's positions 0..t stay inside the bound
    // the host validated the buffers against
    CHECK(ri.b == 3);
    CHECK(ri.t >= -1 && ri.t < max_seq_len);
    // well-formed metadata gives the exact position
    if (0 <= c0 && c0 <= row && row < c1 && c1 <= total_q && len >= c1 - c0 && len <= max_seq_len)
      CHECK(ri.t == len - (c1 - c0) + (row - c0));
    if (row < c0 || row >= c1) CHECK(ri.t == -1);
  }
  const int64_t pages[] = {INT64_MIN, -5, -1, 0, 1, 7, 8, 9, 1 << 30, INT64_MAX};
  for (int64_t num_pages : {(int64_t)1, (int64_t)8, (int64_t)4096, (int64_t)1 << 40})
    for (int64_t p : pages) {
      const int64_t c = dsa::clamp_page(p, num_pages);
      CHECK(c >= 0 && c < num_pages);
      if (p >= 0 && p < num_pages) CHECK(c == p);
    }
}

static const uintptr_t kFake = 0x100000;  // aligned, never dereferenced
#define FAKE ((void *)kFake)

static dsa_batch batch(int32_t total_q = 2) {
  dsa_batch b;
  b.block_table = (const int32_t *)FAKE;
  b.seq_lens = (const int32_t *)FAKE;
  b.cu_q = (const int32_t *)FAKE;
  b.batch = 2;
  b.bt_stride = 4;
  b.total_q = total_q;
  b.max_seq_len = 200;
  b.max_q = total_q > 0 ? 1 : 0;
  return b;
}

static dsa_paged_cache cache(int32_t row_elems, int32_t dtype) {
  dsa_paged_cache c;
  c.data = FAKE;
  c.scale = (const float *)FAKE;
  c.num_pages = 10;
  c.page_size = 64;
  c.row_elems = row_elems;
  c.dtype = dtype;
  return c;
}

static void check_abi() {
  dsa_batch b = batch();
  dsa_paged_cache keys = cache(128, DSA_BF16), kv = cache(576, DSA_BF16);
  float *fp = (float *)FAKE;
  int32_t *ip = (int32_t *)FAKE;
  CHECK(dsa_indexer_scores(nullptr, FAKE, DSA_BF16, fp, 32, 128, &keys, fp, 256, nullptr) == DSA_ERR_NULL);
  CHECK(dsa_indexer_scores(&b, FAKE, DSA_BF16, fp, 32, 128, &keys, fp, 199, nullptr) == DSA_ERR_SHAPE);
  CHECK(dsa_indexer_scores(&b, FAKE, 7, fp, 32, 128, &keys, fp, 256, nullptr) == DSA_ERR_DTYPE);
  CHECK(dsa_indexer_scores(&b, FAKE, DSA_BF16, fp, 32, 64, &keys, fp, 256, nullptr) == DSA_ERR_SHAPE);
  CHECK(dsa_topk(&b, fp, 256, 0, ip, nullptr, 0, nullptr) == DSA_ERR_SHAPE);
  CHECK(dsa_topk(&b, nullptr, 256, 64, ip, nullptr, 0, nullptr) == DSA_ERR_NULL);
  dsa_batch long_rows = batch();
  long_rows.max_seq_len = 100000;
  long_rows.bt_stride = 2000;
  CHECK(dsa_topk(&long_rows, fp, 100000, 2048, ip, nullptr, 0, nullptr) == DSA_ERR_WORKSPACE);
  CHECK(dsa_sparse_mla_fwd(&b, FAKE, DSA_BF16, 64, 512, 32, &kv, ip, 2048, 0.0625f, fp, fp, FAKE,
                           (size_t)1 << 40, nullptr) == DSA_ERR_SHAPE);
  CHECK(dsa_sparse_mla_fwd(&b, FAKE, DSA_BF16, 64, 512, 64, &kv, ip, 2048, -1.0f, fp, fp, FAKE,
                           (size_t)1 << 40, nullptr) == DSA_ERR_SHAPE);
  CHECK(dsa_sparse_mla_fwd(&b, FAKE, DSA_BF16, 64, 512, 64, &kv, nullptr, 2048, 0.0625f, fp, fp,
                           FAKE, (size_t)1 << 40, nullptr) == DSA_ERR_NULL);
  CHECK(dsa_sparse_mla_fwd(&b, FAKE, DSA_BF16, 64, 512, 64, &kv, ip, 2048, 0.0625f, fp, fp, nullptr,
                           16, nullptr) == DSA_ERR_WORKSPACE);
  dsa_batch big = batch(32);
  big.batch = 32;
  big.max_seq_len = 70000;
  big.bt_stride = 1100;
  CHECK(dsa_sparse_mla_fwd_noalloc(&big, FAKE, DSA_BF16, 64, 512, 64, &kv, ip, 65536, 0.0625f, fp,
                                   fp, nullptr) == DSA_ERR_WORKSPACE);
  const void *qs[3] = {FAKE, FAKE, FAKE};
  float *outs[3] = {fp, fp, fp};
  dsa_paged_cache kvs[3] = {kv, kv, kv};
  kvs[1].page_size = 32;
  CHECK(dsa_sparse_mla_fwd_layers(&b, 3, qs, DSA_BF16, 64, 512, 64, kvs, ip, 2048, 0.0625f, outs,
                                  nullptr, FAKE, (size_t)1 << 40, nullptr) == DSA_ERR_SHAPE);
  CHECK(dsa_sparse_mla_fwd_layers(&b, 9, qs, DSA_BF16, 64, 512, 64, kvs, ip, 2048, 0.0625f, outs,
                                  nullptr, FAKE, (size_t)1 << 40, nullptr) == DSA_ERR_SHAPE);
  CHECK(dsa_page_scores(&b, fp, 256, 0, fp, 4, nullptr) == DSA_ERR_SHAPE);
  CHECK(dsa_page_topk(&b, fp, 4, 64, 0, ip, ip, nullptr, 0, nullptr) == DSA_ERR_SHAPE);
  CHECK(dsa_indexer_page_scores(&b, FAKE, DSA_BF16, fp, 32, 128, &keys, 16, fp, 13, nullptr) ==
        DSA_ERR_UNSUPPORTED);
  dsa_paged_cache fp8 = cache(128, DSA_FP8_E4M3);
  fp8.scale = nullptr;
  CHECK(dsa_kv_append(ip, 4, FAKE, &kv, FAKE, DSA_BF16, &fp8, nullptr) == DSA_ERR_NULL);
  CHECK(dsa_kv_append(ip, -1, FAKE, &kv, FAKE, DSA_BF16, &keys, nullptr) == DSA_ERR_SHAPE);
  // an empty batch: validated, nothing to enqueue, NULL per-row arrays allowed
  dsa_batch e;
  e.block_table = nullptr;
  e.seq_lens = nullptr;
  e.cu_q = nullptr;
  e.batch = 0;
  e.bt_stride = 0;
  e.total_q = 0;
  e.max_seq_len = 0;
  e.max_q = 0;
  CHECK(dsa_indexer_scores(&e, nullptr, DSA_BF16, nullptr, 32, 128, &keys, nullptr, 1, nullptr) == DSA_OK);
  CHECK(dsa_topk(&e, nullptr, 1, 64, nullptr, nullptr, 0, nullptr) == DSA_OK);
  CHECK(dsa_sparse_mla_fwd(&e, nullptr, DSA_BF16, 64, 512, 64, &kv, nullptr, 2048, 0.0625f, nullptr,
                           nullptr, nullptr, 0, nullptr) == DSA_OK);
  CHECK(dsa_sparse_mla_fwd_noalloc(&e, nullptr, DSA_BF16, 64, 512, 64, &kv, nullptr, 2048, 0.0625f,
                                   nullptr, nullptr, nullptr) == DSA_OK);
  CHECK(dsa_kv_append(nullptr, 0, nullptr, &kv, nullptr, DSA_BF16, nullptr, nullptr) == DSA_OK);
  for (int code = 0; code <= 7; ++code) CHECK(dsa_status_str((dsa_status)code) != nullptr);
  CHECK(dsa_abi_version() == DSA_ABI_VERSION);
  CHECK(dsa_topk_workspace_size(32, 245760, 2048) > 0);
  CHECK(dsa_sparse_mla_workspace_size(0, 64, 512, 2048) == 0);
}

int main() {
  check_clamps();
  check_abi();
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("host checks ok\n");
  return 0;
}
