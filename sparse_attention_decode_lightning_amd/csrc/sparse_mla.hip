// Absorbed sparse MLA attention over the selected cache rows on gfx950
// ("vLLM Inference Path: GLM-5.2 as an Example", sections "MLA Projections and
// KV State" and "Sparse MLA Attention"; "Making GLM-5.2 Sparse on TPUs",
// section "Separate the indexer from the attention it controls": the cache
// row is a 512-d latent plus a 64-d RoPE key, the key projection is absorbed
// into the 576-d query and the value is the latent itself).
//
// MFMA path (bf16, 64 heads, 512 + 64): one 512-thread workgroup (8 waves)
// owns one query row and one contiguous slice ("split") of its k index slots,
// walked in tiles of 32 selected rows.
//  * All selected positions of the split are translated to physical rows once,
//    up front, into an LDS table.
//  * Gather: every selected 1152-byte row is read with coalesced 16-byte loads
//    (wave w fetches rows 4w..4w+3 of a tile, 1024 contiguous bytes of one row
//    per instruction from a row base in scalar registers). Tile i+2 is loaded
//    into registers while tile i is computed, and stored into the LDS buffer
//    tile i-1 used (two buffers; rows padded to 1168 bytes so that the MFMA
//    operand reads below are bank-conflict free).
//  * Logits: waves (hg, kh) and (hg, 1-kh) compute heads 16hg..16hg+15
//    against the 32 rows over dims 288kh..288kh+287 (v_mfma_f32_16x16x32_bf16,
//    query block in registers, operand reads one k-step ahead of the MFMAs).
//    Each hands its partial logits to the other through LDS, so both hold the
//    full logits and run the online softmax (base 2, scale folded with
//    log2 e) for their 16 heads without further exchange.
//  * PV: probabilities go to LDS as bf16 hi + lo pairs (p = hi + lo to 2^-16
//    relative, so rounding p costs no accuracy); wave w owns output dims
//    64w..64w+63 for all 64 heads. The value operand needs 8 consecutive rows
//    of one dim per lane; ds_read_b64_tr_b16 delivers exactly that from the
//    row-major tile (each 16-lane group reads a 4 x 16 block and gets it
//    transposed), two reads per operand.
//  * Two barriers per tile: after the partial-logit exchange and after the
//    probabilities are written.
//  * Workgroups are numbered so that all splits of a row land on the same XCD
//    (workgroups are dispatched round-robin over the 8 XCDs), so the row's
//    query block is fetched from HBM once and then served by that XCD's L2.
//  * Splits of a row are merged by a log-sum-exp combine kernel.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

constexpr int kH = 64;
constexpr int kDL = 512;
constexpr int kDR = 64;
constexpr int kD = kDL + kDR;               // 576
constexpr int kRowBytes = kD * 2;           // 1152
constexpr int kRowStride = kRowBytes + 16;  // LDS row stride (bytes)
constexpr int kTileN = 32;
constexpr int kMlaThreads = 512;
constexpr int kPStride = kTileN * 2 + 16;  // bytes per head row of P
constexpr int kSteps = kD / 32;            // 18 MFMA k-steps for the logits
constexpr int kHalfSteps = kSteps / 2;     // each wave of a head group covers half the dims
constexpr int kMinRowsPerSplit = 128;
constexpr int kXcds = 8;
constexpr int kMaxRowsPerSplit = 2048;
constexpr int kMaxSplits = 64;
constexpr int kRowBufs = 3;  // row tiles in LDS: computed, next, landing
constexpr float kLazy = 8.0f;  // log2 headroom before the reference maximum moves

// Row <-> MFMA k-slot map of the PV contraction. Lane group g of the value
// operand reads rows 16L + 8(g&1) + (g>>1) + 2e (e < 4) in transposed load L,
// so each 32-lane half of a ds_read_b64_tr_b16 touches only even or only odd
// rows and the 1168-byte row stride keeps its banks disjoint. The
// probabilities are stored in the same k order.
__device__ __forceinline__ int pv_slot(int row) {
  const int L = row >> 4, r = row & 15;
  const int g = 2 * (r & 1) + (r >> 3);
  return 8 * g + 4 * L + ((r & 7) >> 1);
}

static_assert(kTileN == 32 && kMlaThreads == 512, "gather map below assumes 4 rows per wave");

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short __attribute__((address_space(3))) *lds_i16_ptr;

// Lane i of each 16-lane group receives column i of the 4 x 16 block of
// 16-bit values whose row e is supplied (4 values each) by lanes 4e..4e+3.
__device__ __forceinline__ uint2 lds_read_tr16(const void *p) {
  const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4_t *)((lds_i16_ptr)(const_cast<void *>(p))));
  return __builtin_bit_cast(uint2, v);
}

__global__ __launch_bounds__(kMlaThreads) void sparse_mla_bf16_kernel(
    const int32_t *__restrict__ block_table, const int32_t *__restrict__ seq_lens,
    const int32_t *__restrict__ cu_q, int batch, int total_q, int max_seq_len, int64_t bt_stride,
    const uint16_t *__restrict__ q, const uint8_t *__restrict__ kv, int64_t num_pages,
    int page_size, const int32_t *__restrict__ indices, int k, int n_splits, int rows_per_split,
    float scale_log2, float *__restrict__ out, float *__restrict__ lse,
    float *__restrict__ ws_acc, float *__restrict__ ws_ml) {
  __shared__ __attribute__((aligned(16))) uint8_t s_rows[kRowBufs][kTileN * kRowStride];
  __shared__ __attribute__((aligned(16))) uint8_t s_phi[kH * kPStride];
  __shared__ __attribute__((aligned(16))) uint8_t s_plo[kH * kPStride];
  __shared__ f32x4_t s_xchg[8][2][kWave];  // partial logits handed to the other dim half
  __shared__ float s_alpha[kH];
  __shared__ float s_ml[kH][2][2];  // per head, per dim half: (m, l)
  __shared__ int s_rescale[2];      // some head's reference max moved (tile parity)
  __shared__ __attribute__((aligned(16))) int32_t s_rowid[kMaxRowsPerSplit + kTileN];

  // XCD-aware numbering: block id = ((row / 8) * n_splits + split) * 8 + row % 8
  const int xcd = blockIdx.x % kXcds;
  const int rest = blockIdx.x / kXcds;
  const int split = rest % n_splits;
  const int row = (rest / n_splits) * kXcds + xcd;
  if (row >= total_q) return;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 4, j = lane & 15;
  const int hg = wv & 3, kh = wv >> 2;

  const RowInfo ri = row_info(cu_q, seq_lens, batch, total_q, max_seq_len, row);
  const int b = ri.b, t = ri.t;
  const int slot_begin = split * rows_per_split;
  const int slot_end = min(k, slot_begin + rows_per_split);
  const int nrows = max(0, slot_end - slot_begin);
  const int ntiles = (nrows + kTileN - 1) / kTileN;
  const int32_t *idx_row = indices + (int64_t)row * k;
  auto rowid_of = [&](int i) -> int32_t {  // physical row of slot i of the split, or -1
    if (i >= nrows) return -1;
    const int pos = idx_row[slot_begin + i];
    if (pos < 0 || pos > t) return -1;
    return (int32_t)paged_row(block_table, bt_stride, b, pos, page_size, num_pages);
  };

  // Query block of heads 16hg.. over dim half kh: lane (g, i) holds head
  // 16hg + i, dims 288kh + 32s + 8g .. +8.
  u32x4_t qf[kHalfSteps];
  {
    const uint16_t *qp = q + ((int64_t)row * kH + 16 * hg + j) * kD + 288 * kh + 8 * g;
#pragma unroll
    for (int s = 0; s < kHalfSteps; ++s) qf[s] = ldg16(qp + 32 * s);
  }

  // Gather map of a 32-row tile (72 chunks of 16 bytes per row): wave wv owns
  // rows 4wv..4wv+3; chunks 0..63 of row 4wv+m go to lane = chunk, chunks
  // 64..71 of row 4wv + lane/8 to lanes 0..31.
  u32x4_t buf[5];
  auto load_rows = [&](int r0, int r1, int r2, int r3) {
    const int rids[4] = {r0, r1, r2, r3};
#pragma unroll
    for (int m = 0; m < 4; ++m)
      buf[m] = rids[m] >= 0 ? ldg16(kv + (int64_t)rids[m] * kRowBytes + 16 * lane)
                            : u32x4_t{0u, 0u, 0u, 0u};
    const int q4 = lane >> 3;
    const int r5 = q4 == 0 ? r0 : (q4 == 1 ? r1 : (q4 == 2 ? r2 : r3));
    buf[4] = (lane < 32 && r5 >= 0) ? ldg16(kv + (int64_t)r5 * kRowBytes + 16 * (64 + (lane & 7)))
                                    : u32x4_t{0u, 0u, 0u, 0u};
  };
  auto issue_loads = [&](int tile) {
    const int4 rid4 = *reinterpret_cast<const int4 *>(&s_rowid[tile * kTileN + 4 * wv]);
    load_rows(__builtin_amdgcn_readfirstlane(rid4.x), __builtin_amdgcn_readfirstlane(rid4.y),
              __builtin_amdgcn_readfirstlane(rid4.z), __builtin_amdgcn_readfirstlane(rid4.w));
  };
  auto store_tile = [&](int tb) {
    uint8_t *base = s_rows[tb] + (4 * wv) * kRowStride;
#pragma unroll
    for (int m = 0; m < 4; ++m)
      *reinterpret_cast<u32x4_t *>(base + m * kRowStride + 16 * lane) = buf[m];
    if (lane < 32)
      *reinterpret_cast<u32x4_t *>(base + (lane >> 3) * kRowStride + 16 * (64 + (lane & 7))) =
          buf[4];
  };
  // partial logits of heads 16hg + 4g + r against rows 16nt + j of a tile,
  // dims of half kh, with operand reads one k-step ahead of the MFMAs
  auto logits = [&](int tb, f32x4_t (&acc)[2]) {
    const uint8_t *rp = s_rows[tb] + j * kRowStride + 576 * kh + 16 * g;
    u32x4_t bcur[2], bnext[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      acc[nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      bcur[nt] = *reinterpret_cast<const u32x4_t *>(rp + nt * 16 * kRowStride);
    }
#pragma unroll
    for (int s = 0; s < kHalfSteps; ++s) {
      if (s + 1 < kHalfSteps) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          bnext[nt] = *reinterpret_cast<const u32x4_t *>(rp + nt * 16 * kRowStride + 64 * (s + 1));
      }
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) acc[nt] = mfma_16x16x32_bf16(qf[s], bcur[nt], acc[nt]);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) bcur[nt] = bnext[nt];
    }
  };

  // ---- prologue: tile 0 is gathered before the full row table exists ----
  if (ntiles > 0) {
    const int mine = lane < 4 ? rowid_of(4 * wv + lane) : -1;
    load_rows(__builtin_amdgcn_readlane(mine, 0), __builtin_amdgcn_readlane(mine, 1),
              __builtin_amdgcn_readlane(mine, 2), __builtin_amdgcn_readlane(mine, 3));
  }
  // translate every selected position of the split once (padding to whole
  // tiles with -1), so the tile loop never waits on index or block-table reads
  for (int i = tid; i < ntiles * kTileN; i += kMlaThreads) s_rowid[i] = rowid_of(i);
  if (tid < 2) s_rescale[tid] = 0;

  f32x4_t o[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) o[mt][nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  // m_run is each head's reference maximum: probabilities are 2^(x - m_run),
  // and m_run only moves (with a rescale of everything accumulated so far)
  // when a logit exceeds it by more than kLazy, so p <= 2^kLazy. l_run sums
  // the probabilities of this wave's 16 rows of every tile.
  float m_run[4], l_run[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m_run[r] = -INFINITY;
    l_run[r] = 0.0f;
  }

  f32x4_t sacc[2], snext[2];
  if (ntiles > 0) {
    store_tile(0);
    __syncthreads();  // row table and tile 0 visible
    if (ntiles > 1) issue_loads(1);
    logits(0, sacc);
    if (ntiles > 1) {
      store_tile(1);
      if (ntiles > 2) issue_loads(2);
    }
    s_xchg[wv][0][lane] = sacc[0];
    s_xchg[wv][1][lane] = sacc[1];
  }
  __syncthreads();  // A(0): partials of tile 0 and tile 1's rows visible

  for (int tile = 0; tile < ntiles; ++tile) {
    // a. logits of the next tile start in the matrix pipe while this tile's
    //    softmax runs on the vector units
    if (tile + 1 < ntiles) logits((tile + 1) % kRowBufs, snext);

    // b. full logits and online softmax of this wave's 16 heads; both waves of
    //    a head group see all 32 rows (same maximum), wave kh owns rows 16kh + j
    float x[2][4];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const f32x4_t full = sacc[nt] + s_xchg[wv ^ 4][nt][lane];
      const bool valid = s_rowid[tile * kTileN + 16 * nt + j] >= 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) x[nt][r] = valid ? full[r] * scale_log2 : -INFINITY;
    }
    if (tid == 0) s_rescale[(tile + 1) & 1] = 0;  // its last reader was PV(tile - 1)
    float pmine[4];
    bool moved = false;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int head = 16 * hg + 4 * g + r;
      const float tmax = row16_max(fmaxf(x[0][r], x[1][r]));
      const bool up = tmax > m_run[r] + kLazy;  // false while the tile is all padding
      const float m_new = up ? tmax : m_run[r];
      const float m_use = m_new == -INFINITY ? 0.0f : m_new;
      const float alpha = up ? fast_exp2(m_run[r] - m_use) : 1.0f;
      const float p = fast_exp2((kh == 0 ? x[0][r] : x[1][r]) - m_use);
      l_run[r] = l_run[r] * alpha + row16_sum(p);
      m_run[r] = m_new;
      moved |= up;
      if (kh == 0 && j == 0) s_alpha[head] = alpha;
      pmine[r] = p;
    }
    if (kh == 0 && __ballot(moved) != 0 && lane == 0) s_rescale[tile & 1] = 1;
    {
      // p = hi + lo, both bf16 (round to nearest even on the conversion unit)
      const int slot = pv_slot(16 * kh + j);
#pragma unroll
      for (int r = 0; r < 4; r += 2) {
        const f32x2_t pp = {pmine[r], pmine[r + 1]};
        const bf16x2_t hi = __builtin_convertvector(pp, bf16x2_t);
        const f32x2_t hf = __builtin_convertvector(hi, f32x2_t);
        const bf16x2_t lo = __builtin_convertvector(pp - hf, bf16x2_t);
        const int head = 16 * hg + 4 * g + r;
        reinterpret_cast<__bf16 *>(s_phi + head * kPStride)[slot] = hi.x;
        reinterpret_cast<__bf16 *>(s_phi + (head + 1) * kPStride)[slot] = hi.y;
        reinterpret_cast<__bf16 *>(s_plo + head * kPStride)[slot] = lo.x;
        reinterpret_cast<__bf16 *>(s_plo + (head + 1) * kPStride)[slot] = lo.y;
      }
    }

    // c. the tile after next lands in the buffer PV(tile - 1) used
    if (tile + 2 < ntiles) {
      store_tile((tile + 2) % kRowBufs);
      if (tile + 3 < ntiles) issue_loads(tile + 3);
    }
    __syncthreads();  // B(tile): probabilities and rescale factors visible

    // d. rescale (only when a reference maximum moved) and accumulate P.V for
    //    dims 64wv .. +64, all heads, K = 32 rows
    if (s_rescale[tile & 1]) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float al = s_alpha[16 * mt + 4 * g + r];
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) o[mt][nt][r] *= al;
        }
    }
    {
      const uint8_t *rows = s_rows[tile % kRowBufs];
      // lane (g, i) of transposed load L reads row 16L + 8(g&1) + (g>>1) + 2(i>>2)
      const uint8_t *vbase = rows + (8 * (g & 1) + (g >> 1) + 2 * (j >> 2)) * kRowStride +
                             (64 * wv + 4 * (j & 3)) * 2;
      u32x4_t vb[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const uint2 v0 = lds_read_tr16(vbase + 32 * nt);
        const uint2 v1 = lds_read_tr16(vbase + 16 * kRowStride + 32 * nt);
        vb[nt] = u32x4_t{v0.x, v0.y, v1.x, v1.y};
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int poff = (16 * mt + j) * kPStride + 16 * g;
        const u32x4_t pa_hi = *reinterpret_cast<const u32x4_t *>(s_phi + poff);
        const u32x4_t pa_lo = *reinterpret_cast<const u32x4_t *>(s_plo + poff);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) o[mt][nt] = mfma_16x16x32_bf16(pa_hi, vb[nt], o[mt][nt]);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) o[mt][nt] = mfma_16x16x32_bf16(pa_lo, vb[nt], o[mt][nt]);
      }
    }

    // e. hand the next tile's partial logits over
    if (tile + 1 < ntiles) {
      s_xchg[wv][0][lane] = snext[0];
      s_xchg[wv][1][lane] = snext[1];
      sacc[0] = snext[0];
      sacc[1] = snext[1];
    }
    __syncthreads();  // A(tile + 1)
  }

  // 5. combine the two dim halves' sums per head; write the output or this
  //    split's partials
  if (j == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int head = 16 * hg + 4 * g + r;
      s_ml[head][kh][0] = m_run[r];
      s_ml[head][kh][1] = l_run[r];
    }
  }
  __syncthreads();
  if (n_splits == 1) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int head = 16 * mt + 4 * g + r;
        const float l = s_ml[head][0][1] + s_ml[head][1][1];
        const float inv = l > 0.0f ? 1.0f / l : 0.0f;
        float *op = out + ((int64_t)row * kH + head) * kDL + 64 * wv + j;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) op[16 * nt] = o[mt][nt][r] * inv;
      }
    if (lse != nullptr && tid < kH) {
      const float m = s_ml[tid][0][0], l = s_ml[tid][0][1] + s_ml[tid][1][1];
      lse[(int64_t)row * kH + tid] = l > 0.0f ? m * kLn2 + logf(l) : -INFINITY;
    }
  } else {
    const int64_t part = (int64_t)row * n_splits + split;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int head = 16 * mt + 4 * g + r;
        float *op = ws_acc + (part * kH + head) * kDL + 64 * wv + j;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) op[16 * nt] = o[mt][nt][r];
      }
    if (tid < kH) {
      ws_ml[(part * kH + tid) * 2 + 0] = s_ml[tid][0][0];
      ws_ml[(part * kH + tid) * 2 + 1] = s_ml[tid][0][1] + s_ml[tid][1][1];
    }
  }
}

// Merge the splits of one row: 256 threads = 4 heads x 64 threads x 8 dims.
// O = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s, lse = M ln 2 + ln(sum ...).
__global__ __launch_bounds__(256) void mla_combine_kernel(int n_splits,
                                                          const float *__restrict__ ws_acc,
                                                          const float *__restrict__ ws_ml,
                                                          float *__restrict__ out,
                                                          float *__restrict__ lse) {
  const int row = blockIdx.x / (kH / 4);
  const int head = (blockIdx.x % (kH / 4)) * 4 + (threadIdx.x >> 6);
  const int d0 = (threadIdx.x & 63) * 8;
  const float *ml = ws_ml + ((int64_t)row * n_splits * kH + head) * 2;  // split s at + s*kH*2
  float M = -INFINITY;
  for (int s = 0; s < n_splits; ++s) M = fmaxf(M, ml[s * kH * 2]);
  const float Mu = M == -INFINITY ? 0.0f : M;
  float Lsum = 0.0f;
  f32x4_t a0 = {0.0f, 0.0f, 0.0f, 0.0f}, a1 = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int s = 0; s < n_splits; ++s) {
    const float wgt = exp2f(ml[s * kH * 2] - Mu);
    Lsum += wgt * ml[s * kH * 2 + 1];
    const float *src = ws_acc + ((((int64_t)row * n_splits + s) * kH + head) * kDL + d0);
    a0 += wgt * *reinterpret_cast<const f32x4_t *>(src);
    a1 += wgt * *reinterpret_cast<const f32x4_t *>(src + 4);
  }
  const float inv = Lsum > 0.0f ? 1.0f / Lsum : 0.0f;
  float *dst = out + (((int64_t)row * kH + head) * kDL + d0);
  *reinterpret_cast<f32x4_t *>(dst) = a0 * inv;
  *reinterpret_cast<f32x4_t *>(dst + 4) = a1 * inv;
  if (lse != nullptr && (threadIdx.x & 63) == 0)
    lse[(int64_t)row * kH + head] = Lsum > 0.0f ? M * kLn2 + logf(Lsum) : -INFINITY;
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
  // enough workgroups for every CU, never slices shorter than kMinRowsPerSplit,
  // never more than kMaxRowsPerSplit rows (the per-split LDS row table)
  const int want = (256 + total_q - 1) / total_q;
  const int cap = (k + kMinRowsPerSplit - 1) / kMinRowsPerSplit;
  const int need = (k + kMaxRowsPerSplit - 1) / kMaxRowsPerSplit;
  int s = want < cap ? want : cap;
  s = s < need ? need : s;
  return s < 1 ? 1 : s;
}

int mla_max_k() { return kMaxSplits * kMaxRowsPerSplit; }

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
    const int64_t rows_padded = (int64_t)(bt.total_q + kXcds - 1) / kXcds * kXcds;
    hipLaunchKernelGGL(sparse_mla_bf16_kernel, dim3((unsigned)(rows_padded * S)),
                       dim3(kMlaThreads), 0, stream, bt.block_table, bt.seq_lens, bt.cu_q,
                       bt.batch, bt.total_q, bt.max_seq_len, bt.bt_stride,
                       static_cast<const uint16_t *>(q), static_cast<const uint8_t *>(kv.data),
                       kv.num_pages, kv.page_size, indices, k, S, per, scale_log2, out, lse,
                       ws_acc, ws_ml);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || S == 1) return e;
    hipLaunchKernelGGL(mla_combine_kernel, dim3(bt.total_q * (n_heads / 4)), dim3(256), 0, stream,
                       S, ws_acc, ws_ml, out, lse);
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
