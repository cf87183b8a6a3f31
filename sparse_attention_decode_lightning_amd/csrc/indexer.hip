// Lightning-indexer scores on gfx950.
//
// I[t, s] = sum_j w[t, j] * ReLU(q_idx[t, j, :] . k(s)), s <= t
// ("vLLM Inference Path: GLM-5.2 as an Example", section "DSA Indexer";
// "Making GLM-5.2 Sparse on TPUs", section "Separate the indexer from the
// attention it controls").
//
// MFMA path (bf16 queries, bf16 or e4m3 keys, head_dim 128): the q . k
// contraction is a [heads x 128] x [128 x 16 keys] product per key tile on
// v_mfma_f32_16x16x32_bf16, M = 16 query heads per tile, N = 16 keys, K = 32
// dims per step. The 16x16 accumulator leaves each lane with four heads of one
// key, so ReLU, the per-head weight and the in-lane part of the head sum run
// in registers, and two cross-lane adds finish the head sum. e4m3 keys are
// widened exactly to bf16 in registers; their per-token scale multiplies each
// head's dot product before the ReLU, so k = scale * e4m3 holds for any scale.
// Keys are read straight from HBM into MFMA operand registers, every key byte
// once per query group; each lane's 16-byte loads from one key row keep all
// of a 64-byte (bf16) or 32-byte (fp8) run in one instruction.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kIdxDim = 128;
constexpr int kIdxThreads = 256;
constexpr int kIdxWaves = kIdxThreads / kWave;
constexpr int kTilesPerWave = 4;
constexpr int kKeysPerBlock = kIdxWaves * kTilesPerWave * 16;

// Dim offset supplied by lane group g at MFMA step s. Both operands use the
// same map, so the contraction covers every dim exactly once. bf16 keys take
// 32 contiguous dims per step (16 rows x 64 B per load); e4m3 keys give each
// lane group one contiguous 32-byte run of its key row.
template <bool FP8>
__device__ __forceinline__ int dim_of(int s, int g) {
  return FP8 ? (32 * g + 8 * s) : (32 * s + 8 * g);
}

template <int NMT, int QG, bool FP8>
__global__ __launch_bounds__(kIdxThreads) void indexer_mfma_kernel(
    const int32_t *__restrict__ block_table, const int32_t *__restrict__ seq_lens,
    const int32_t *__restrict__ cu_q, int batch, int total_q, int max_seq_len, int64_t bt_stride,
    const uint16_t *__restrict__ q_idx, const float *__restrict__ w,
    const uint8_t *__restrict__ kdata, const float *__restrict__ kscale, int64_t num_pages,
    int page_size, float *__restrict__ scores, int64_t ld) {
  constexpr int H = NMT * 16;
  const int chunk = blockIdx.x, qgrp = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int g = lane >> 4, j = lane & 15;
  if (b >= batch) return;
  const int L = min(max(seq_lens[b], 0), max_seq_len);
  const int q0 = min(max(cu_q[b], 0), total_q);
  const int qn = min(max(cu_q[b + 1], q0), total_q) - q0;
  const int i0 = qgrp * QG;
  if (i0 >= qn) return;
  const int nq = min(QG, qn - i0);
  const int t_first = L - qn + i0;
  const int t_last = t_first + nq - 1;
  const int key0 = chunk * kKeysPerBlock;
  if (t_last < 0 || key0 > t_last) return;

  // Query fragments: lane (g, j) holds head 16*mt + j, dims dim_of(s, g) .. +8.
  u32x4_t a[QG][NMT][4];
  float wr[QG][NMT][4];
#pragma unroll
  for (int qi = 0; qi < QG; ++qi) {
    const int64_t row = q0 + i0 + min(qi, nq - 1);
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      const uint16_t *qp = q_idx + (row * H + mt * 16 + j) * kIdxDim;
#pragma unroll
      for (int s = 0; s < 4; ++s) a[qi][mt][s] = ldg16(qp + dim_of<FP8>(s, g));
#pragma unroll
      for (int r = 0; r < 4; ++r) wr[qi][mt][r] = w[row * H + mt * 16 + 4 * g + r];
    }
  }

  // Issue every key load of this wave before any MFMA.
  u32x4_t kb[kTilesPerWave][FP8 ? 2 : 4];
  float ksc[kTilesPerWave];
#pragma unroll
  for (int i = 0; i < kTilesPerWave; ++i) {
    const int tile0 = key0 + (wv * kTilesPerWave + i) * 16;
    ksc[i] = 1.0f;
    if (tile0 > t_last) continue;
    const int pos = min(tile0 + j, t_last);
    const int64_t row = paged_row(block_table, bt_stride, b, pos, page_size, num_pages);
    if constexpr (FP8) {
      const uint8_t *kp = kdata + row * kIdxDim + 32 * g;
      kb[i][0] = ldg16(kp);
      kb[i][1] = ldg16(kp + 16);
      ksc[i] = kscale[row];
    } else {
      const uint8_t *kp = kdata + row * (2 * kIdxDim);
#pragma unroll
      for (int s = 0; s < 4; ++s) kb[i][s] = ldg16(kp + 2 * dim_of<false>(s, g));
    }
  }

#pragma unroll
  for (int i = 0; i < kTilesPerWave; ++i) {
    const int tile0 = key0 + (wv * kTilesPerWave + i) * 16;
    if (tile0 > t_last) continue;
    u32x4_t bb[4];
    if constexpr (FP8) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const u32x4_t src = kb[i][s >> 1];
        const u32x2_t lo = e4m3x4_to_bf16x4((s & 1) ? src.z : src.x);
        const u32x2_t hi = e4m3x4_to_bf16x4((s & 1) ? src.w : src.y);
        bb[s] = u32x4_t{lo.x, lo.y, hi.x, hi.y};
      }
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) bb[s] = kb[i][s];
    }
    float part[QG];
#pragma unroll
    for (int qi = 0; qi < QG; ++qi) {
      float p = 0.0f;
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = mfma_16x16x32_bf16(a[qi][mt][s], bb[s], acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) p += wr[qi][mt][r] * fmaxf(acc[r] * ksc[i], 0.0f);
      }
      p += __shfl_xor(p, 16);
      p += __shfl_xor(p, 32);
      part[qi] = p;
    }
    const int pos = tile0 + j;
#pragma unroll
    for (int qi = 0; qi < QG; ++qi) {
      if ((qi & 3) == g && qi < nq && pos <= t_first + qi)
        scores[(int64_t)(q0 + i0 + qi) * ld + pos] = part[qi];
    }
  }
}

// Any element types and sizes: one thread per (query row, key position), fp32
// fused multiply-adds over dims and heads.
template <typename QT, int KDT>
__global__ __launch_bounds__(256) void indexer_generic_kernel(
    const int32_t *__restrict__ block_table, const int32_t *__restrict__ seq_lens,
    const int32_t *__restrict__ cu_q, int batch, int total_q, int max_seq_len, int64_t bt_stride,
    const QT *__restrict__ q_idx,
    const float *__restrict__ w, int H, int D, const void *__restrict__ kdata,
    const float *__restrict__ kscale, int64_t num_pages, int page_size,
    float *__restrict__ scores, int64_t ld) {
  const int row = blockIdx.y;
  const RowInfo ri = row_info(cu_q, seq_lens, batch, total_q, max_seq_len, row);
  const int b = ri.b, t = ri.t;
  const int pos = blockIdx.x * blockDim.x + threadIdx.x;
  if (pos > t) return;
  const int64_t kr = paged_row(block_table, bt_stride, b, pos, page_size, num_pages);
  const float sc = KDT == DSA_FP8_E4M3 ? kscale[kr] : 1.0f;
  float total = 0.0f;
  for (int h = 0; h < H; ++h) {
    const QT *qp = q_idx + ((int64_t)row * H + h) * D;
    float dot = 0.0f;
    for (int d = 0; d < D; ++d) {
      float kv;
      if constexpr (KDT == DSA_F32) kv = reinterpret_cast<const float *>(kdata)[kr * D + d];
      else if constexpr (KDT == DSA_BF16)
        kv = bf16_to_f32(reinterpret_cast<const uint16_t *>(kdata)[kr * D + d]);
      else kv = e4m3_to_f32(reinterpret_cast<const uint8_t *>(kdata)[kr * D + d]);
      float qv;
      if constexpr (sizeof(QT) == 4) qv = qp[d];
      else qv = bf16_to_f32(qp[d]);
      dot = fmaf(qv, kv, dot);
    }
    total = fmaf(w[(int64_t)row * H + h], fmaxf(dot * sc, 0.0f), total);
  }
  scores[(int64_t)row * ld + pos] = total;
}

template <int NMT, int QG, bool FP8>
hipError_t launch_mfma(const BatchArgs &bt, const void *q_idx, const float *w,
                       const CacheArgs &keys, float *scores, int64_t ld, hipStream_t stream) {
  const int chunks = (bt.max_seq_len + kKeysPerBlock - 1) / kKeysPerBlock;
  const int qgroups = (bt.max_q + QG - 1) / QG;
  if (qgroups > 65535 || bt.batch > 65535) return hipErrorInvalidConfiguration;
  dim3 grid(chunks, qgroups, bt.batch);
  hipLaunchKernelGGL((indexer_mfma_kernel<NMT, QG, FP8>), grid, dim3(kIdxThreads), 0, stream,
                     bt.block_table, bt.seq_lens, bt.cu_q, bt.batch, bt.total_q, bt.max_seq_len, bt.bt_stride,
                     static_cast<const uint16_t *>(q_idx), w,
                     static_cast<const uint8_t *>(keys.data), keys.scale, keys.num_pages,
                     keys.page_size, scores, ld);
  return hipGetLastError();
}

template <bool FP8>
hipError_t dispatch_mfma(const BatchArgs &bt, const void *q_idx, const float *w, int n_heads,
                         const CacheArgs &keys, float *scores, int64_t ld, hipStream_t stream) {
  const bool multi = bt.max_q > 1;
  switch (n_heads) {
    case 16:
      return multi ? launch_mfma<1, 8, FP8>(bt, q_idx, w, keys, scores, ld, stream)
                   : launch_mfma<1, 1, FP8>(bt, q_idx, w, keys, scores, ld, stream);
    case 32:
      return multi ? launch_mfma<2, 4, FP8>(bt, q_idx, w, keys, scores, ld, stream)
                   : launch_mfma<2, 1, FP8>(bt, q_idx, w, keys, scores, ld, stream);
    default:
      return multi ? launch_mfma<4, 2, FP8>(bt, q_idx, w, keys, scores, ld, stream)
                   : launch_mfma<4, 1, FP8>(bt, q_idx, w, keys, scores, ld, stream);
  }
}

template <typename QT, int KDT>
hipError_t launch_generic(const BatchArgs &bt, const void *q_idx, const float *w, int H, int D,
                          const CacheArgs &keys, float *scores, int64_t ld, hipStream_t stream) {
  if (bt.total_q > 65535) return hipErrorInvalidConfiguration;
  dim3 grid((bt.max_seq_len + 255) / 256, bt.total_q);
  hipLaunchKernelGGL((indexer_generic_kernel<QT, KDT>), grid, dim3(256), 0, stream,
                     bt.block_table, bt.seq_lens, bt.cu_q, bt.batch, bt.total_q, bt.max_seq_len, bt.bt_stride,
                     static_cast<const QT *>(q_idx), w, H, D, keys.data, keys.scale,
                     keys.num_pages, keys.page_size, scores, ld);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_indexer_scores(const BatchArgs &bt, const void *q_idx, int32_t q_dtype,
                                 const float *w, int32_t n_heads, int32_t head_dim,
                                 const CacheArgs &keys, float *scores, int64_t ld_scores,
                                 hipStream_t stream) {
  if (bt.total_q == 0 || bt.max_seq_len == 0) return hipSuccess;
  const bool mfma_shape = head_dim == kIdxDim && (n_heads == 16 || n_heads == 32 || n_heads == 64);
  if (q_dtype == DSA_BF16 && mfma_shape) {
    if (keys.dtype == DSA_BF16)
      return dispatch_mfma<false>(bt, q_idx, w, n_heads, keys, scores, ld_scores, stream);
    if (keys.dtype == DSA_FP8_E4M3)
      return dispatch_mfma<true>(bt, q_idx, w, n_heads, keys, scores, ld_scores, stream);
  }
  if (q_dtype == DSA_F32)
    return launch_generic<float, DSA_F32>(bt, q_idx, w, n_heads, head_dim, keys, scores,
                                          ld_scores, stream);
  if (keys.dtype == DSA_BF16)
    return launch_generic<uint16_t, DSA_BF16>(bt, q_idx, w, n_heads, head_dim, keys, scores,
                                              ld_scores, stream);
  return launch_generic<uint16_t, DSA_FP8_E4M3>(bt, q_idx, w, n_heads, head_dim, keys, scores,
                                                ld_scores, stream);
}

}  // namespace dsa
