// Per-row top-k of the indexer scores on gfx950 ("GLM-5.2 on vLLM Ascend:
// Request-to-Backend Inference Path", section "8. The SFA backend, step by
// step": the indexer returns token positions, 2,048 per query).
//
// One 1024-thread workgroup selects one row by radix select:
//  * scores map to order-preserving 32-bit keys (-0.0 first folded into +0.0,
//    so the two compare equal);
//  * four 8-bit digit passes, most significant first, each a histogram of the
//    keys that still match the chosen prefix (one private histogram per wave to
//    spread LDS atomics), find the k-th largest key tau and how many keys equal
//    to tau must be taken;
//  * one ordered pass then keeps every key > tau and the first `need` keys
//    == tau in position order; wave ballots give each kept position its rank,
//    so the output is written in ascending position order without a sort.
// Rows of up to kCacheKeys candidates are staged once in LDS as keys; longer
// rows are re-read from global memory (L2) on every pass.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / kWave;
constexpr int kCacheKeys = 32768;

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  u = (u == 0x80000000u) ? 0u : u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <bool CACHED>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(
    const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ cu_q, int batch,
    int total_q, int max_seq_len, const float *__restrict__ scores, int64_t ld, int k,
    int32_t *__restrict__ indices) {
  extern __shared__ uint32_t cache[];
  __shared__ uint32_t hist[kTopkWaves][256];
  __shared__ uint32_t suffix[256];
  __shared__ uint32_t wave_eq[kTopkWaves], wave_sel[kTopkWaves];
  __shared__ uint32_t s_digit, s_need;

  const int row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n = row_info(cu_q, seq_lens, batch, total_q, max_seq_len, row).t + 1;
  int32_t *out = indices + (int64_t)row * k;
  if (n <= k) {
    for (int i = tid; i < k; i += kTopkThreads) out[i] = i < n ? i : -1;
    return;
  }
  const float *src = scores + (int64_t)row * ld;
  if constexpr (CACHED) {
    for (int i = tid; i < n; i += kTopkThreads) cache[i] = order_key(src[i]);
  }
  auto key_at = [&](int i) -> uint32_t {
    if constexpr (CACHED) return cache[i];
    else return order_key(src[i]);
  };

  uint32_t prefix = 0, mask = 0;
  uint32_t need = (uint32_t)k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    uint32_t *hflat = &hist[0][0];
    for (int i = tid; i < kTopkWaves * 256; i += kTopkThreads) hflat[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kTopkThreads) {
      const uint32_t key = key_at(i);
      if ((key & mask) == prefix) atomicAdd(&hist[wv][(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 256) {
      uint32_t c = 0;
#pragma unroll
      for (int w = 0; w < kTopkWaves; ++w) c += hist[w][tid];
      suffix[tid] = c;
    }
    __syncthreads();
    // inclusive suffix sums: suffix[d] = number of candidates with digit >= d
    for (int off = 1; off < 256; off <<= 1) {
      uint32_t v = 0;
      if (tid < 256 && tid + off < 256) v = suffix[tid + off];
      __syncthreads();
      if (tid < 256) suffix[tid] += v;
      __syncthreads();
    }
    if (tid < 256) {
      const uint32_t above = tid == 255 ? 0u : suffix[tid + 1];
      if (suffix[tid] >= need && above < need) {
        s_digit = (uint32_t)tid;
        s_need = need - above;
      }
    }
    __syncthreads();
    prefix |= s_digit << shift;
    mask |= 255u << shift;
    need = s_need;
    __syncthreads();
  }

  // Ordered selection: keys > tau, then the first `need` keys == tau.
  const uint32_t tau = prefix;
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  uint32_t base_eq = 0, base_sel = 0;
  for (int c0 = 0; c0 < n; c0 += kTopkThreads) {
    const int i = c0 + tid;
    const uint32_t key = i < n ? key_at(i) : 0u;
    const bool gt = i < n && key > tau;
    const bool eq = i < n && key == tau;
    const uint64_t beq = __ballot(eq);
    if (lane == 0) wave_eq[wv] = (uint32_t)__popcll(beq);
    __syncthreads();
    uint32_t eq_rank = base_eq + (uint32_t)__popcll(beq & lt_mask), eq_tot = 0;
#pragma unroll
    for (int w = 0; w < kTopkWaves; ++w) {
      const uint32_t v = wave_eq[w];
      eq_rank += w < wv ? v : 0u;
      eq_tot += v;
    }
    const bool sel = gt || (eq && eq_rank < need);
    const uint64_t bsel = __ballot(sel);
    if (lane == 0) wave_sel[wv] = (uint32_t)__popcll(bsel);
    __syncthreads();
    uint32_t slot = base_sel + (uint32_t)__popcll(bsel & lt_mask), sel_tot = 0;
#pragma unroll
    for (int w = 0; w < kTopkWaves; ++w) {
      const uint32_t v = wave_sel[w];
      slot += w < wv ? v : 0u;
      sel_tot += v;
    }
    if (sel && slot < (uint32_t)k) out[slot] = i;
    base_eq += eq_tot;
    base_sel += sel_tot;
    __syncthreads();
  }
}

}  // namespace

size_t topk_workspace_bytes(int32_t, int32_t, int32_t) { return 0; }

hipError_t launch_topk(const BatchArgs &bt, const float *scores, int64_t ld, int32_t k,
                       int32_t *indices, void *, size_t, hipStream_t stream) {
  if (bt.total_q == 0) return hipSuccess;
  if (bt.max_seq_len <= kCacheKeys) {
    const size_t lds = (size_t)(bt.max_seq_len > 0 ? bt.max_seq_len : 1) * sizeof(uint32_t);
    hipError_t e = hipFuncSetAttribute((const void *)topk_kernel<true>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_kernel<true>, dim3(bt.total_q), dim3(kTopkThreads), lds, stream,
                       bt.seq_lens, bt.cu_q, bt.batch, bt.total_q, bt.max_seq_len, scores, ld, k, indices);
  } else {
    hipLaunchKernelGGL(topk_kernel<false>, dim3(bt.total_q), dim3(kTopkThreads), 0, stream,
                       bt.seq_lens, bt.cu_q, bt.batch, bt.total_q, bt.max_seq_len, scores, ld, k, indices);
  }
  return hipGetLastError();
}

}  // namespace dsa
