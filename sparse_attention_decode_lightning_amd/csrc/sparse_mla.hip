// Absorbed sparse MLA attention over the selected cache rows on gfx950
// ("vLLM Inference Path: GLM-5.2 as an Example", sections "MLA Projections and
// KV State" and "Sparse MLA Attention"; "Making GLM-5.2 Sparse on TPUs",
// section "Separate the indexer from the attention it controls": the cache
// row is a 512-d latent plus a 64-d RoPE key, the key projection is absorbed
// into the 576-d query and the value is the latent itself).
//
// MFMA path (bf16, 64 heads, 512 + 64): one 256-thread workgroup owns one
// query row and one contiguous slice ("split") of its k index slots.
//  * Gather: the slice is walked in tiles of 32 selected rows; each thread
//    translates nothing but copies 16-byte chunks, so a tile is fetched with
//    fully coalesced 1152-byte row reads into LDS (rows padded to 1168 bytes
//    so the MFMA operand reads below are bank-conflict free).
//  * Logits: wave w computes the 16 heads 16w..16w+15 against the 32 rows,
//    K = 576, on v_mfma_f32_16x16x32_bf16; its 16 x 576 query block stays in
//    registers for the whole slice.
//  * Online softmax (base 2, scale folded with log2 e) per head, max and sum
//    reduced across the 16 lanes holding a head's row.
//  * PV: the probabilities go to LDS as bf16 hi + lo pairs (p ~= hi + lo to
//    2^-16 relative, so rounding p costs no accuracy); wave w then owns the
//    output dims 128w..128w+127 for all 64 heads and accumulates hi.V + lo.V.
//  * Several splits of a row are merged by a small log-sum-exp combine kernel.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

constexpr int kH = 64;
constexpr int kDL = 512;
constexpr int kDR = 64;
constexpr int kD = kDL + kDR;            // 576
constexpr int kRowBytes = kD * 2;        // 1152
constexpr int kRowStride = kRowBytes + 16;  // LDS row stride (bytes)
constexpr int kTileN = 32;
constexpr int kChunksPerRow = kRowBytes / 16;  // 72
constexpr int kMlaThreads = 256;
constexpr int kGatherPerThread = kTileN * kChunksPerRow / kMlaThreads;  // 9
constexpr int kPStride = kTileN * 2 + 16;  // bytes per head row of P
constexpr int kSteps = kD / 32;            // 18 MFMA k-steps for the logits
constexpr int kMinRowsPerSplit = 128;

static_assert(kTileN * kChunksPerRow % kMlaThreads == 0, "gather must tile evenly");

__global__ __launch_bounds__(kMlaThreads) void sparse_mla_bf16_kernel(
    const int32_t *__restrict__ block_table, const int32_t *__restrict__ seq_lens,
    const int32_t *__restrict__ cu_q, int batch, int total_q, int max_seq_len, int64_t bt_stride,
    const uint16_t *__restrict__ q, const uint8_t *__restrict__ kv, int64_t num_pages,
    int page_size, const int32_t *__restrict__ indices, int k, int n_splits, int rows_per_split,
    float scale_log2, float *__restrict__ out, float *__restrict__ lse,
    float *__restrict__ ws_acc, float *__restrict__ ws_ml) {
  __shared__ __attribute__((aligned(16))) uint8_t s_rows[kTileN * kRowStride];
  __shared__ __attribute__((aligned(16))) uint8_t s_phi[kH * kPStride];
  __shared__ __attribute__((aligned(16))) uint8_t s_plo[kH * kPStride];
  __shared__ float s_alpha[kH];
  __shared__ float s_ml[kH][2];
  __shared__ int64_t s_off[kTileN];

  const int row = blockIdx.x / n_splits;
  const int split = blockIdx.x % n_splits;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 4, j = lane & 15;

  const RowInfo ri = row_info(cu_q, seq_lens, batch, total_q, max_seq_len, row);
  const int b = ri.b, t = ri.t;
  const int slot_begin = split * rows_per_split;
  const int slot_end = min(k, slot_begin + rows_per_split);
  const int32_t *idx_row = indices + (int64_t)row * k;

  // Query block of this wave's 16 heads: lane (g, i) holds head 16*wv + i,
  // dims 32*s + 8*g .. +8 for every step s.
  u32x4_t qf[kSteps];
  {
    const uint16_t *qp = q + ((int64_t)row * kH + 16 * wv + j) * kD + 8 * g;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) qf[s] = ldg16(qp + 32 * s);
  }

  f32x4_t o[4][8];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) o[mt][nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run[4], l_run[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m_run[r] = -INFINITY;
    l_run[r] = 0.0f;
  }

  for (int tile0 = slot_begin; tile0 < slot_end; tile0 += kTileN) {
    // 1. translate this tile's selected positions to byte offsets
    if (tid < kTileN) {
      const int slot = tile0 + tid;
      int64_t off = -1;
      if (slot < slot_end) {
        const int pos = idx_row[slot];
        if (pos >= 0 && pos <= t)
          off = paged_row(block_table, bt_stride, b, pos, page_size, num_pages) * kRowBytes;
      }
      s_off[tid] = off;
    }
    __syncthreads();
    // 2. gather the rows into LDS (invalid rows become zeros)
    {
      u32x4_t buf[kGatherPerThread];
#pragma unroll
      for (int m = 0; m < kGatherPerThread; ++m) {
        const int c = tid + m * kMlaThreads;
        const int rr = c / kChunksPerRow, cc = c % kChunksPerRow;
        const int64_t off = s_off[rr];
        buf[m] = off >= 0 ? ldg16(kv + off + cc * 16) : u32x4_t{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int m = 0; m < kGatherPerThread; ++m) {
        const int c = tid + m * kMlaThreads;
        const int rr = c / kChunksPerRow, cc = c % kChunksPerRow;
        *reinterpret_cast<u32x4_t *>(s_rows + rr * kRowStride + cc * 16) = buf[m];
      }
    }
    __syncthreads();

    // 3. logits for heads 16*wv.. against the 32 rows
    f32x4_t sacc[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      sacc[nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      const uint8_t *rp = s_rows + (nt * 16 + j) * kRowStride + 16 * g;
#pragma unroll
      for (int s = 0; s < kSteps; ++s)
        sacc[nt] = mfma_16x16x32_bf16(qf[s], *reinterpret_cast<const u32x4_t *>(rp + 64 * s),
                                      sacc[nt]);
    }
    // 4. online softmax; lane (g, j) holds heads 16*wv + 4*g + r of rows j, 16 + j
    bool valid[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) valid[nt] = s_off[nt * 16 + j] >= 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float x0 = valid[0] ? sacc[0][r] * scale_log2 : -INFINITY;
      float x1 = valid[1] ? sacc[1][r] * scale_log2 : -INFINITY;
      float mx = fmaxf(x0, x1);
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
      const float m_new = fmaxf(m_run[r], mx);
      const float m_use = m_new == -INFINITY ? 0.0f : m_new;
      const float alpha = exp2f(m_run[r] - m_use);
      const float p0 = exp2f(x0 - m_use);
      const float p1 = exp2f(x1 - m_use);
      float ps = p0 + p1;
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) ps += __shfl_xor(ps, off);
      l_run[r] = l_run[r] * alpha + ps;
      m_run[r] = m_new;
      const int head = 16 * wv + 4 * g + r;
      if (j == 0) s_alpha[head] = alpha;
      const uint32_t h0 = f32_to_bf16_rne(p0), h1 = f32_to_bf16_rne(p1);
      const uint32_t l0 = f32_to_bf16_rne(p0 - bf16_to_f32(h0));
      const uint32_t l1 = f32_to_bf16_rne(p1 - bf16_to_f32(h1));
      uint16_t *ph = reinterpret_cast<uint16_t *>(s_phi + head * kPStride);
      uint16_t *pl = reinterpret_cast<uint16_t *>(s_plo + head * kPStride);
      ph[j] = (uint16_t)h0;
      ph[16 + j] = (uint16_t)h1;
      pl[j] = (uint16_t)l0;
      pl[16 + j] = (uint16_t)l1;
    }
    __syncthreads();

    // 5. rescale and accumulate P.V for dims 128*wv .. +128, all heads
    {
      float al[4][4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) al[mt][r] = s_alpha[16 * mt + 4 * g + r];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
#pragma unroll
          for (int r = 0; r < 4; ++r) o[mt][nt][r] *= al[mt][r];
      u32x4_t pa_hi[4], pa_lo[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        pa_hi[mt] = *reinterpret_cast<const u32x4_t *>(s_phi + (16 * mt + j) * kPStride + 16 * g);
        pa_lo[mt] = *reinterpret_cast<const u32x4_t *>(s_plo + (16 * mt + j) * kPStride + 16 * g);
      }
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const int dim = 128 * wv + 16 * nt + j;
        const uint16_t *vp = reinterpret_cast<const uint16_t *>(s_rows + (8 * g) * kRowStride) + dim;
        uint32_t v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = vp[e * (kRowStride / 2)];
        const u32x4_t vb = {v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16),
                            v[6] | (v[7] << 16)};
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          o[mt][nt] = mfma_16x16x32_bf16(pa_hi[mt], vb, o[mt][nt]);
          o[mt][nt] = mfma_16x16x32_bf16(pa_lo[mt], vb, o[mt][nt]);
        }
      }
    }
    __syncthreads();
  }

  // 6. publish per-head (m, l) and write the output or this split's partials
  if (j == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int head = 16 * wv + 4 * g + r;
      s_ml[head][0] = m_run[r];
      s_ml[head][1] = l_run[r];
    }
  }
  __syncthreads();
  if (n_splits == 1) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int head = 16 * mt + 4 * g + r;
        const float l = s_ml[head][1];
        const float inv = l > 0.0f ? 1.0f / l : 0.0f;
        float *op = out + ((int64_t)row * kH + head) * kDL + 128 * wv + j;
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) op[16 * nt] = o[mt][nt][r] * inv;
      }
    if (lse != nullptr && tid < kH) {
      const float m = s_ml[tid][0], l = s_ml[tid][1];
      lse[(int64_t)row * kH + tid] = l > 0.0f ? m * kLn2 + logf(l) : -INFINITY;
    }
  } else {
    const int64_t part = (int64_t)row * n_splits + split;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int head = 16 * mt + 4 * g + r;
        float *op = ws_acc + (part * kH + head) * kDL + 128 * wv + j;
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) op[16 * nt] = o[mt][nt][r];
      }
    if (tid < kH) {
      ws_ml[(part * kH + tid) * 2 + 0] = s_ml[tid][0];
      ws_ml[(part * kH + tid) * 2 + 1] = s_ml[tid][1];
    }
  }
}

// Merge the splits of one (row, head): O = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s.
__global__ __launch_bounds__(128) void mla_combine_kernel(int n_splits, int H, int DL,
                                                          const float *__restrict__ ws_acc,
                                                          const float *__restrict__ ws_ml,
                                                          float *__restrict__ out,
                                                          float *__restrict__ lse) {
  const int rh = blockIdx.x;  // row * H + head
  const int row = rh / H, head = rh % H;
  float M = -INFINITY;
  for (int s = 0; s < n_splits; ++s)
    M = fmaxf(M, ws_ml[(((int64_t)row * n_splits + s) * H + head) * 2]);
  const float Mu = M == -INFINITY ? 0.0f : M;
  float Lsum = 0.0f;
  for (int s = 0; s < n_splits; ++s) {
    const float *ml = ws_ml + (((int64_t)row * n_splits + s) * H + head) * 2;
    Lsum += exp2f(ml[0] - Mu) * ml[1];
  }
  const float inv = Lsum > 0.0f ? 1.0f / Lsum : 0.0f;
  for (int d = threadIdx.x; d < DL; d += blockDim.x) {
    float acc = 0.0f;
    for (int s = 0; s < n_splits; ++s) {
      const int64_t part = (int64_t)row * n_splits + s;
      const float wgt = exp2f(ws_ml[(part * H + head) * 2] - Mu);
      acc += wgt * ws_acc[(part * H + head) * DL + d];
    }
    out[(int64_t)rh * DL + d] = acc * inv;
  }
  if (lse != nullptr && threadIdx.x == 0)
    lse[rh] = Lsum > 0.0f ? M * kLn2 + logf(Lsum) : -INFINITY;
}

// Any head count, widths and element type: one 256-thread workgroup per
// (row, head) walks the selected slots, reducing each logit across the block.
template <typename T>
__global__ __launch_bounds__(256) void sparse_mla_generic_kernel(
    const int32_t *__restrict__ block_table, const int32_t *__restrict__ seq_lens,
    const int32_t *__restrict__ cu_q, int batch, int total_q, int max_seq_len, int64_t bt_stride,
    const T *__restrict__ q,
    const T *__restrict__ kv, int64_t num_pages, int page_size, int H, int DL, int DR,
    const int32_t *__restrict__ indices, int k, float scale_log2, float *__restrict__ out,
    float *__restrict__ lse) {
  constexpr int kMaxPer = 4;  // supports d_latent <= 1024
  __shared__ float s_red[4];
  const int rh = blockIdx.x;
  const int row = rh / H, head = rh % H;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int D = DL + DR;
  const RowInfo ri = row_info(cu_q, seq_lens, batch, total_q, max_seq_len, row);
  const int b = ri.b, t = ri.t;
  auto ld = [](const T *p, int64_t i) -> float {
    if constexpr (sizeof(T) == 4) return p[i];
    else return bf16_to_f32(p[i]);
  };
  const T *qp = q + ((int64_t)row * H + head) * D;
  float acc[kMaxPer];
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) acc[i] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;
  for (int slot = 0; slot < k; ++slot) {
    const int pos = indices[(int64_t)row * k + slot];
    if (pos < 0 || pos > t) continue;
    const int64_t rr = paged_row(block_table, bt_stride, b, pos, page_size, num_pages) * D;
    float part = 0.0f;
    for (int d = tid; d < D; d += 256) part = fmaf(ld(qp, d), ld(kv, rr + d), part);
    part = wave_sum(part);
    if (lane == 0) s_red[wv] = part;
    __syncthreads();
    const float x = (s_red[0] + s_red[1] + s_red[2] + s_red[3]) * scale_log2;
    __syncthreads();
    const float m_new = fmaxf(m_run, x);
    const float alpha = exp2f(m_run - m_new);
    const float p = exp2f(x - m_new);
    l_run = l_run * alpha + p;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
      const int d = tid + 256 * i;
      if (d < DL) acc[i] = acc[i] * alpha + p * ld(kv, rr + d);
    }
  }
  const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    const int d = tid + 256 * i;
    if (d < DL) out[(int64_t)rh * DL + d] = acc[i] * inv;
  }
  if (lse != nullptr && tid == 0) lse[rh] = l_run > 0.0f ? m_run * kLn2 + logf(l_run) : -INFINITY;
}

bool mfma_shape(int32_t q_dtype, int32_t n_heads, int32_t d_latent, int32_t d_rope) {
  return q_dtype == DSA_BF16 && n_heads == kH && d_latent == kDL && d_rope == kDR;
}

}  // namespace

int mla_num_splits(int32_t total_q, int32_t n_heads, int32_t d_latent, int32_t k) {
  if (total_q <= 0 || n_heads != kH || d_latent != kDL) return 1;
  // enough workgroups for every CU, but never slices shorter than kMinRowsPerSplit
  int want = (256 + total_q - 1) / total_q;
  int cap = (k + kMinRowsPerSplit - 1) / kMinRowsPerSplit;
  int s = want < cap ? want : cap;
  return s < 1 ? 1 : s;
}

size_t mla_workspace_bytes(int32_t total_q, int32_t n_heads, int32_t d_latent, int32_t k) {
  const int s = mla_num_splits(total_q, n_heads, d_latent, k);
  if (s <= 1) return 0;
  return (size_t)total_q * s * n_heads * (d_latent + 2) * sizeof(float);
}

hipError_t launch_sparse_mla(const BatchArgs &bt, const void *q, int32_t q_dtype, int32_t n_heads,
                             int32_t d_latent, int32_t d_rope, const CacheArgs &kv,
                             const int32_t *indices, int32_t k, float scale, float *out, float *lse,
                             void *workspace, size_t, hipStream_t stream) {
  if (bt.total_q == 0) return hipSuccess;
  const float scale_log2 = scale * kLog2e;
  if (mfma_shape(q_dtype, n_heads, d_latent, d_rope)) {
    const int S = mla_num_splits(bt.total_q, n_heads, d_latent, k);
    const int per = (((k + S - 1) / S) + kTileN - 1) / kTileN * kTileN;
    float *ws_acc = static_cast<float *>(workspace);
    float *ws_ml = ws_acc == nullptr ? nullptr
                                     : ws_acc + (size_t)bt.total_q * S * n_heads * d_latent;
    hipLaunchKernelGGL(sparse_mla_bf16_kernel, dim3(bt.total_q * S), dim3(kMlaThreads), 0,
                       stream, bt.block_table, bt.seq_lens, bt.cu_q, bt.batch, bt.total_q, bt.max_seq_len,
                       bt.bt_stride,
                       static_cast<const uint16_t *>(q), static_cast<const uint8_t *>(kv.data),
                       kv.num_pages, kv.page_size, indices, k, S, per, scale_log2, out, lse,
                       ws_acc, ws_ml);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || S == 1) return e;
    hipLaunchKernelGGL(mla_combine_kernel, dim3(bt.total_q * n_heads), dim3(128), 0, stream, S,
                       n_heads, d_latent, ws_acc, ws_ml, out, lse);
    return hipGetLastError();
  }
  if (q_dtype == DSA_F32) {
    hipLaunchKernelGGL(sparse_mla_generic_kernel<float>, dim3(bt.total_q * n_heads), dim3(256), 0,
                       stream, bt.block_table, bt.seq_lens, bt.cu_q, bt.batch, bt.total_q, bt.max_seq_len,
                       bt.bt_stride,
                       static_cast<const float *>(q), static_cast<const float *>(kv.data),
                       kv.num_pages, kv.page_size, n_heads, d_latent, d_rope, indices, k,
                       scale_log2, out, lse);
  } else {
    hipLaunchKernelGGL(sparse_mla_generic_kernel<uint16_t>, dim3(bt.total_q * n_heads), dim3(256),
                       0, stream, bt.block_table, bt.seq_lens, bt.cu_q, bt.batch, bt.total_q, bt.max_seq_len,
                       bt.bt_stride,
                       static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(kv.data),
                       kv.num_pages, kv.page_size, n_heads, d_latent, d_rope, indices, k,
                       scale_log2, out, lse);
  }
  return hipGetLastError();
}

}  // namespace dsa
