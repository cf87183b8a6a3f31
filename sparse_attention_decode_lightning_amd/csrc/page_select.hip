// Page-budget selection on gfx950 ("Making GLM-5.2 Sparse on TPUs", section
// "Make the sparsity unit match the memory unit": a page is ranked by its
// highest legal token score, the causal and valid-length masks coming before
// that maximum, and attention then reads every legal token of the kp best
// pages; section "Stream indexer scores over live context": what the
// selection consumes is the page maxima).
//
// page_scores_kernel: one wave per (row, logical page) takes the maximum of
// the page's scores at positions <= t (a page wholly past t is not written).
// The page top-k is the token top-k kernel family run over page maxima (the
// candidates of a row are its pages 0..t / P, ties to the lower page).
// expand_pages_kernel turns a row's kp pages into the kp * P token positions
// they hold, in ascending order, positions past t (and empty page slots) -1.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kPageThreads = 256;
constexpr int kPageWaves = kPageThreads / kWave;

__global__ __launch_bounds__(kPageThreads) void page_scores_kernel(
    const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ cu_q, int batch,
    int total_q, int max_seq_len, const float *__restrict__ scores, int64_t ld, int page_size,
    FastDiv pdiv, float *__restrict__ page_scores, int64_t ld_pages) {
  const int row = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int page = blockIdx.x * kPageWaves + (threadIdx.x >> 6);
  const int t = row_info(cu_q, seq_lens, batch, total_q, max_seq_len, row).t;
  if (t < 0 || page > (int)fast_div((uint32_t)t, pdiv)) return;
  const int s0 = page * page_size;
  const int s1 = min(s0 + page_size, t + 1);  // legal positions of the page: [s0, s1)
  const float *src = scores + (int64_t)row * ld;
  float m = -INFINITY;
  for (int s = s0 + lane; s < s1; s += kWave) m = fmaxf(m, src[s]);
  m = wave_max(m);
  if (lane == 0) page_scores[(int64_t)row * ld_pages + page] = m;
}

__global__ __launch_bounds__(kPageThreads) void expand_pages_kernel(
    const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ cu_q, int batch,
    int total_q, int max_seq_len, const int32_t *__restrict__ pages, int kp, int page_size,
    FastDiv pdiv, int32_t *__restrict__ indices) {
  const int row = blockIdx.y;
  const int t = row_info(cu_q, seq_lens, batch, total_q, max_seq_len, row).t;
  const int64_t k = (int64_t)kp * page_size;
  const int64_t i = (int64_t)blockIdx.x * kPageThreads + threadIdx.x;
  if (i >= k) return;
  const uint32_t slot = fast_div((uint32_t)i, pdiv);
  const int o = (int)(i - (int64_t)slot * page_size);
  const int p = pages[(int64_t)row * kp + slot];
  const int64_t pos = (int64_t)p * page_size + o;
  indices[(int64_t)row * k + i] = (p >= 0 && pos <= t) ? (int32_t)pos : -1;
}

}  // namespace

hipError_t launch_page_scores(const BatchArgs &bt, const float *scores, int64_t ld,
                              int32_t page_size, float *page_scores, int64_t ld_pages,
                              hipStream_t stream) {
  if (bt.total_q == 0 || bt.max_seq_len == 0) return hipSuccess;
  const int max_pages = candidate_bound(bt.max_seq_len, page_size);
  if (bt.total_q > 65535) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)((max_pages + kPageWaves - 1) / kPageWaves), (unsigned)bt.total_q);
  hipLaunchKernelGGL(page_scores_kernel, grid, dim3(kPageThreads), 0, stream, bt.seq_lens,
                     bt.cu_q, bt.batch, bt.total_q, bt.max_seq_len, scores, ld, page_size,
                     make_fast_div((uint32_t)page_size), page_scores, ld_pages);
  return hipGetLastError();
}

hipError_t launch_page_topk(const BatchArgs &bt, const float *page_scores, int64_t ld_pages,
                            int32_t page_size, int32_t kp, int32_t *pages, int32_t *indices,
                            void *workspace, size_t ws_bytes, hipStream_t stream) {
  if (bt.total_q == 0) return hipSuccess;
  // the one-workgroup selection expands its pages itself; the longer paths
  // leave it to expand_pages_kernel
  bool expanded = false;
  hipError_t e = launch_topk(bt, page_scores, ld_pages, kp, page_size, pages, workspace, ws_bytes,
                             stream, indices, &expanded);
  if (e != hipSuccess || indices == nullptr || expanded) return e;
  if (bt.total_q > 65535) return hipErrorInvalidConfiguration;
  const int64_t k = (int64_t)kp * page_size;
  const dim3 grid((unsigned)((k + kPageThreads - 1) / kPageThreads), (unsigned)bt.total_q);
  hipLaunchKernelGGL(expand_pages_kernel, grid, dim3(kPageThreads), 0, stream, bt.seq_lens,
                     bt.cu_q, bt.batch, bt.total_q, bt.max_seq_len, pages, kp, page_size,
                     make_fast_div((uint32_t)page_size), indices);
  return hipGetLastError();
}

}  // namespace dsa
