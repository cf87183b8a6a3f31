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
#include <algorithm>

#include "dsa_device.h"
#include "dsa_internal.h"
#include "dsa_select.h"

namespace dsa {
namespace {

constexpr int kIdxDim = 128;

typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16_t mfma_32x32x16_bf16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
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

// Streaming decode path (bf16 queries, bf16 or e4m3 keys, head_dim 128, pages
// holding whole 64-key blocks). One 256-thread workgroup walks a run of
// blocks of 64 consecutive keys of one sequence (16 blocks per query row of
// the workgroup, fewer when the batch is small); each block is copied into an
// LDS stage by direct global-to-LDS loads (16 bytes per lane, 1 KB per wave
// instruction, the 16-byte chunks of each key XOR-permuted by the key's low
// bits through the choice of source address) three blocks ahead of the one
// being computed, with one barrier per block. Wave w multiplies the query
// fragments held in registers with keys 16w..16w+15 of the block (operands
// from LDS), so the memory system sees a few long contiguous streams per CU
// instead of every key request of the launch at once.
constexpr int kStreamBlocks = 16;  // blocks of scores buffered in LDS between write-outs
constexpr int kStreamWorkgroups = 512;
constexpr int kStreamStages = 4;
constexpr int kStreamKeys = 64;
constexpr int kFusedHistOff = 64;                       // words: the count, then padding
constexpr int kFusedRowWords = kFusedHistOff + kSelBins;  // per row, 256-byte multiple
static_assert(kSelBins == 8 * 256, "eight bins per thread of a 256-thread workgroup");

// Direct global-to-LDS copy, 16 (or 4) bytes per lane, at lds + 16 l (4 l).
// Issued as inline assembly so the compiler's automatic waits ignore it;
// completion is awaited by the explicit vmcnt waits before the barriers.
__device__ __forceinline__ void idx_lds_load16(const void *src, const __attribute__((address_space(3))) void *lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  uint32_t saved;  // m0 is reserved to the compiler: restore it
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved)
               : "v"(src), "s"(m0)
               : "memory");
}
__device__ __forceinline__ void idx_lds_load4(const void *src, const __attribute__((address_space(3))) void *lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  uint32_t saved;  // m0 is reserved to the compiler: restore it
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dword %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved)
               : "v"(src), "s"(m0)
               : "memory");
}

// s_waitcnt immediate: vmcnt n (bits 3:0, 15:14), expcnt and lgkmcnt 0.
constexpr int vm_wait(int n) { return (n & 15) | ((n >> 4) << 14); }

// Workgroup barrier ordering LDS only: waits for this wave's LDS operations
// (lgkmcnt 0) but not for memory loads in flight, which a full
// __syncthreads() (release fence) would drain.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt 63, expcnt 7, lgkmcnt 0
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Fused top-k state of one query row: the count of the row's workgroups that
// have finished, then (from word kFusedHistOff) the row's level-1 histogram.
struct FusedTopk {
  int k;
  int32_t *indices;  // [total_q, k]
  uint32_t *state;   // [total_q, kFusedRowWords], zero between calls
};

// PMAX: instead of the token scores, each row's page maxima over logical
// pages of one 64-key block (the selection's pages):
// scores[row * ld + page] = max of the page's scores at positions <= t (pages
// wholly past t are not written).
// TR > 0 (one query row per workgroup, runs of at most kStreamBlocks blocks):
// the scores are written as without it, and the row's top-k goes to
// tk.indices, selected by the row's last workgroup to finish; TR is the
// candidates per lane of that selection (rows of up to 256 TR positions).
template <int NMT, int QG, bool FP8, bool PMAX, int TR = 0>
__global__ __launch_bounds__(256) void indexer_stream_kernel(
    const int32_t *__restrict__ block_table, const int32_t *__restrict__ seq_lens,
    const int32_t *__restrict__ cu_q, int batch, int total_q, int max_seq_len, int64_t bt_stride,
    const uint16_t *__restrict__ q_idx, const float *__restrict__ w,
    const uint8_t *__restrict__ kdata, const float *__restrict__ kscale, int64_t num_pages,
    int page_size, FastDiv pdiv, float *__restrict__ scores, int64_t ld, int run_blocks,
    int page_blocks, FusedTopk tk) {
  static_assert(TR == 0 || (QG == 1 && !PMAX), "fused selection: one row per workgroup");
  constexpr int H = NMT * 16;
  constexpr int RB = FP8 ? kIdxDim : 2 * kIdxDim;    // bytes per key row
  constexpr int CPK = RB / 16;                      // 16-byte chunks per key
  constexpr int SB = kStreamKeys * RB;              // stage bytes
  constexpr int NI = SB / 1024 / 4;                 // key copies per wave per block
  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  __shared__ __attribute__((aligned(1024))) uint8_t s_st[kStreamStages][SB];
  __shared__ __attribute__((aligned(256))) float s_sc[kStreamStages][kStreamKeys];
  // scores of the workgroup's keys, written out after the loop so that the
  // only memory operations inside it are the direct copies
  __shared__ __attribute__((aligned(16))) float s_out[QG][kStreamBlocks * kStreamKeys];

  const int chunk = blockIdx.x, qgrp = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
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
  const int key0 = chunk * run_blocks * kStreamKeys;
  if (t_last < 0 || key0 > t_last) {
    if constexpr (TR > 0) {
      // a row with no position: its first workgroup writes the empty list
      if (t_last < 0 && chunk == 0)
        for (int i = tid; i < tk.k; i += 256) tk.indices[(int64_t)(q0 + i0) * tk.k + i] = -1;
    }
    return;
  }
  const int nblk = min(run_blocks, (t_last - key0) / kStreamKeys + 1);

  // Four query rows of 32 heads (draft verification) take the wide path:
  // wave wv computes query rows 2 (wv >> 1) + {0, 1} against keys
  // 32 (wv & 1) .. + 31 of a block on v_mfma_f32_32x32x16_bf16 (M = the 32
  // heads of a row, N = 32 keys, 8 K-steps), whose 32-cycle MFMAs leave room
  // for the ReLU and weight work of the other row. Lane (h, n): head or key
  // n, dims 64 h + 8 s .. + 8 at step s on both operands; accumulator
  // element 4 i + r is head 8 i + 4 h + r.
  constexpr bool kWide = QG == 4 && NMT == 2;
  const int wn = lane & 31, wh = lane >> 5;
  constexpr int kA = kWide ? 1 : QG, kM = kWide ? 1 : NMT;
  u32x4_t a[kA][kM][4];
  float wr[kA][kM][4];
  u32x4_t a2[kWide ? 2 : 1][8];
  float w2[kWide ? 2 : 1][16];
  if constexpr (kWide) {
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      const int64_t row = q0 + i0 + min(2 * (wv >> 1) + qq, nq - 1);
      const uint16_t *qp = q_idx + (row * H + wn) * kIdxDim + 64 * wh;
#pragma unroll
      for (int s_ = 0; s_ < 8; ++s_) a2[qq][s_] = ldg16(qp + 8 * s_);
#pragma unroll
      for (int e = 0; e < 16; ++e) w2[qq][e] = w[row * H + 8 * (e >> 2) + 4 * wh + (e & 3)];
    }
  } else {
    // Query fragments: lane (g, j) holds head 16 mt + j, dims dim_of(s, g).
#pragma unroll
    for (int qi = 0; qi < QG; ++qi) {
      const int64_t row = q0 + i0 + min(qi, nq - 1);
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        const uint16_t *qp = q_idx + (row * H + mt * 16 + j) * kIdxDim;
#pragma unroll
        for (int s_ = 0; s_ < 4; ++s_) a[qi][mt][s_] = ldg16(qp + dim_of<FP8>(s_, g));
#pragma unroll
        for (int r = 0; r < 4; ++r) wr[qi][mt][r] = w[row * H + mt * 16 + 4 * g + r];
      }
    }
  }
  // Copy map: wave wv's copy i of a block moves stage chunks 64 (4 i + wv) + l,
  // i.e. key c / CPK, stored chunk c % CPK, fetched from chunk swz of the key.
  auto swz = [](int c, int r) { return FP8 ? (c ^ ((r >> 1) & 7)) : (c ^ (r & 15)); };
  uint32_t goff[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int c = 64 * (4 * i + wv) + lane;
    const int r = c / CPK, lc = c % CPK;
    goff[i] = (uint32_t)(r * RB + 16 * swz(lc, r));
  }
  const int64_t bt_row = (int64_t)b * bt_stride;
  auto copy_block = [&](int blk) {
    const int kb0 = key0 + blk * kStreamKeys;
    const int pidx = (int)fast_div((uint32_t)kb0, pdiv);
    const int64_t page = dsa::clamp_page(block_table[bt_row + pidx], num_pages);
    const int64_t row0 = page * page_size + (kb0 - pidx * page_size);
    const uint8_t *base = kdata + row0 * RB;
    const lds_u8 *st = (const lds_u8 *)s_st[blk % kStreamStages];
#pragma unroll
    for (int i = 0; i < NI; ++i) idx_lds_load16(base + goff[i], st + 1024 * (4 * i + wv));
    if constexpr (FP8) {
      if (wv == 0) idx_lds_load4(kscale + row0 + lane, (const lds_u8 *)s_sc[blk % kStreamStages]);
    }
  };
  // loads of this wave per block (the scale copy is wave 0's)
  const int per_blk = NI + ((FP8 && wv == 0) ? 1 : 0);

  // every compiler-visible load has landed before the first direct copies
  __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
  for (int p = 0; p < kStreamStages - 1; ++p)
    if (p < nblk) copy_block(p);

  for (int blk = 0; blk < nblk; ++blk) {
    const int ahead = min(nblk - 1 - blk, kStreamStages - 2);
    // this wave's copies of blk have landed
    if (ahead >= 2) {
      if (per_blk == NI) __builtin_amdgcn_s_waitcnt(vm_wait(2 * NI));
      else __builtin_amdgcn_s_waitcnt(vm_wait(2 * NI + 2));
    } else if (ahead == 1) {
      if (per_blk == NI) __builtin_amdgcn_s_waitcnt(vm_wait(NI));
      else __builtin_amdgcn_s_waitcnt(vm_wait(NI + 1));
    } else {
      __builtin_amdgcn_s_waitcnt(vm_wait(0));
    }
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    if (blk + kStreamStages - 1 < nblk) copy_block(blk + kStreamStages - 1);

    if constexpr (kWide) {
    const int kr = 32 * (wv & 1) + wn;  // key of this lane within the block
    if (key0 + blk * kStreamKeys + 32 * (wv & 1) <= t_last) {
    const lds_u8 *st = (const lds_u8 *)s_st[blk % kStreamStages];
    u32x4_t bq[8];
    if constexpr (FP8) {
      // bytes 64 h .. 64 h + 63 of the key: four chunks of two K-steps each
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const u32x4_t src = *(const __attribute__((address_space(3))) u32x4_t *)(
            st + kr * RB + 16 * swz(4 * wh + t, kr));
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const u32x2_t lo = e4m3x4_to_bf16x4(e ? src.z : src.x);
          const u32x2_t hi = e4m3x4_to_bf16x4(e ? src.w : src.y);
          bq[2 * t + e] = u32x4_t{lo.x, lo.y, hi.x, hi.y};
        }
      }
    } else {
#pragma unroll
      for (int s_ = 0; s_ < 8; ++s_)
        bq[s_] = *(const __attribute__((address_space(3))) u32x4_t *)(st + kr * RB + 16 * swz(8 * wh + s_, kr));
    }
    const float ksc = FP8 ? *(const __attribute__((address_space(3))) float *)((const lds_u8 *)s_sc[blk % kStreamStages] + 4 * kr) : 1.0f;
    // row 0's MFMAs (the key conversions go in between), then row 1's, each
    // followed by the ReLU and weight work of two of row 0's accumulator
    // elements: the 32-cycle MFMAs hide that work
    f32x16_t acc0, acc1;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      acc0[e] = 0.0f;
      acc1[e] = 0.0f;
    }
#pragma unroll
    for (int s_ = 0; s_ < 8; ++s_) acc0 = mfma_32x32x16_bf16(a2[0][s_], bq[s_], acc0);
    float p0 = 0.0f, p1 = 0.0f;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s_ = 0; s_ < 8; ++s_) {
      acc1 = mfma_32x32x16_bf16(a2[1][s_], bq[s_], acc1);
      p0 = fmaf(w2[0][2 * s_], relu_bits(acc0[2 * s_]), p0);
      p0 = fmaf(w2[0][2 * s_ + 1], relu_bits(acc0[2 * s_ + 1]), p0);
      asm volatile("" : "+v"(p0));  // keeps the two steps here, not sunk to the end
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) p1 = fmaf(w2[1][e], relu_bits(acc1[e]), p1);
    // lanes n and n + 32 hold the two halves of a row's head sum
    float pt[2];
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      const float p = qq ? p1 : p0;
      auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(p), __float_as_uint(p), false, false);
      pt[qq] = (__uint_as_float(sw[0]) + __uint_as_float(sw[1])) * ksc;
    }
    // half h of the wave stores query row 2 (wv >> 1) + h
    s_out[2 * (wv >> 1) + wh][(blk % kStreamBlocks) * kStreamKeys + kr] = wh ? pt[1] : pt[0];
    }
    } else {
    const int tile0 = key0 + blk * kStreamKeys + 16 * wv;
    if (tile0 <= t_last) {
    const lds_u8 *st = (const lds_u8 *)s_st[blk % kStreamStages];
    const int kr = 16 * wv + j;  // key of this lane within the block
    u32x4_t bb[4];
    if constexpr (FP8) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x4_t src = *(const __attribute__((address_space(3))) u32x4_t *)(
            st + kr * RB + 16 * swz(2 * g + h, kr));
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const u32x2_t lo = e4m3x4_to_bf16x4(e ? src.z : src.x);
          const u32x2_t hi = e4m3x4_to_bf16x4(e ? src.w : src.y);
          bb[2 * h + e] = u32x4_t{lo.x, lo.y, hi.x, hi.y};
        }
      }
    } else {
#pragma unroll
      for (int s_ = 0; s_ < 4; ++s_)
        bb[s_] = *(const __attribute__((address_space(3))) u32x4_t *)(st + kr * RB + 16 * swz(4 * s_ + g, kr));
    }
    const float ksc = FP8 ? *(const __attribute__((address_space(3))) float *)((const lds_u8 *)s_sc[blk % kStreamStages] + 4 * kr) : 1.0f;
    // every MFMA of the block first, then the epilogues, with no branch
    // between them: the ReLU and weight work of one (query, head tile) then
    // issues under the MFMAs of the next
    f32x4_t acc[QG][NMT];
#pragma unroll
    for (int qi = 0; qi < QG; ++qi)
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        acc[qi][mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s_ = 0; s_ < 4; ++s_) acc[qi][mt] = mfma_16x16x32_bf16(a[qi][mt][s_], bb[s_], acc[qi][mt]);
      }
    float mine = 0.0f;  // lane group g keeps query g % QG
#pragma unroll
    for (int qi = 0; qi < QG; ++qi) {
      float p = 0.0f;
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) p = fmaf(wr[qi][mt][r], relu_bits(acc[qi][mt][r]), p);
      // head sum over the four lane groups; the positive per-key scale of
      // e4m3 keys factors out of the ReLU
      auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(p), __float_as_uint(p), false, false);
      p = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
      auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p), __float_as_uint(p), false, false);
      p = (__uint_as_float(s32[0]) + __uint_as_float(s32[1])) * ksc;
      mine = (g % QG == qi) ? p : mine;
    }
    // (lanes of groups that keep the same query store the same value)
    s_out[g % QG][(blk % kStreamBlocks) * kStreamKeys + 16 * wv + j] = mine;
    }
    }
    // every kStreamBlocks blocks (and at the end) write the buffered scores out
    if (blk % kStreamBlocks == kStreamBlocks - 1 || blk == nblk - 1) {
      lds_barrier();
      const int base = key0 + (blk - blk % kStreamBlocks) * kStreamKeys;  // first buffered key
      const int nbuf = (blk % kStreamBlocks + 1) * kStreamKeys;
      if constexpr (!PMAX) {
#pragma unroll
        for (int qi = 0; qi < QG; ++qi) {
          if (qi >= nq) break;
          const int lim = min(nbuf, t_first + qi + 1 - base);  // causal: pos <= t
          float *dst = scores + (int64_t)(q0 + i0 + qi) * ld + base;
          for (int i = tid; i < lim; i += 256) dst[i] = s_out[qi][i];
        }
      } else {
        // pages of one 64-key block: thread tid takes keys 4 tid .. 4 tid + 3 of
        // the buffer, 16 lanes make a page, whose maximum over positions <= t
        // a DPP reduction gives to its first lane (the buffer starts on a page)
        const int kk = 4 * tid;
#pragma unroll
        for (int qi = 0; qi < QG; ++qi) {
          if (qi >= nq) break;
          const int lim = min(nbuf, t_first + qi + 1 - base);  // causal: pos <= t
          const f32x4_t v = *reinterpret_cast<const f32x4_t *>(&s_out[qi][kk]);
          float m = -INFINITY;
#pragma unroll
          for (int e = 0; e < 4; ++e) m = kk + e < lim ? fmaxf(m, v[e]) : m;
          m = row16_max(m);
          if ((lane & 15) == 0 && kk < lim)
            scores[(int64_t)(q0 + i0 + qi) * ld + base / kStreamKeys + tid / 16] = m;
        }
      }
      lds_barrier();
    }
  }
  if constexpr (TR > 0) {
    // The run's scores are still in s_out[0]. Count their level-1 digits,
    // add the counts to the row's histogram, and count this workgroup in:
    // the row's last workgroup to arrive has every score and every count,
    // and selects the row. No workgroup waits for another.
    using Sh = SelectShared<4, TR>;
    static_assert(sizeof(Sh) <= sizeof(s_st), "the selection reuses the stage buffers");
    Sh &sh = *reinterpret_cast<Sh *>(&s_st[0][0]);
    __shared__ uint32_t s_last;
    const int64_t row = q0 + i0;
    const int nrun = min(nblk * kStreamKeys, t_last + 1 - key0);  // positions of this run
    uint32_t *st = tk.state + row * kFusedRowWords;
    uint32_t *gh = st + kFusedHistOff;
    select_clear(sh);
    __syncthreads();
    for (int i = tid; i < nrun; i += 256)
      atomicAdd(&sh.hist1[sel_bin(order_key(s_out[0][i]) >> 21)], 1u);
    __syncthreads();
    for (int bin = tid; bin < kSelBins; bin += 256) {
      const uint32_t c = sh.hist1[sel_bin(bin)];
      if (c != 0u) atomicAdd(gh + bin, c);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");  // this run's scores and counts, then the arrival
    __syncthreads();
    const int parts = t_last / (run_blocks * kStreamKeys) + 1;  // workgroups of the row
    if (tid == 0) s_last = atomicAdd(st, 1u) == (uint32_t)(parts - 1) ? 1u : 0u;
    __syncthreads();
    if (s_last == 0u) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // the other runs' scores and counts
    // the row's histogram into LDS (hist2 and hist3 cleared), and the state
    // cleared for the next call
    select_clear(sh);
    __syncthreads();
    {
      const int b8 = 8 * tid;  // bins b8 .. b8 + 7, one padded run of LDS words
      const u32x4_t lo = *reinterpret_cast<const u32x4_t *>(gh + b8);
      const u32x4_t hi = *reinterpret_cast<const u32x4_t *>(gh + b8 + 4);
      *reinterpret_cast<u32x4_t *>(&sh.hist1[sel_bin(b8)]) = lo;
      *reinterpret_cast<u32x4_t *>(&sh.hist1[sel_bin(b8) + 4]) = hi;
      *reinterpret_cast<u32x4_t *>(gh + b8) = u32x4_t{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4_t *>(gh + b8 + 4) = u32x4_t{0u, 0u, 0u, 0u};
      if (tid == 0) st[0] = 0u;
    }
    const int n = t_last + 1;
    int32_t *out = tk.indices + row * tk.k;
    if (n <= tk.k) {
      for (int i = tid; i < tk.k; i += 256) out[i] = i < n ? i : -1;
      return;
    }
    // every load below max_seq_len <= ld, issued together; candidates past
    // the row's n are masked inside the selection
    const int w0 = wv * (kWave * TR);
    const float *src = scores + row * ld + w0 + lane;
    const int lim = max_seq_len - w0;
    float v[TR];
#pragma unroll
    for (int u = 0; u < TR; ++u) v[u] = lane < lim - u * kWave ? src[u * kWave] : 0.0f;
    uint32_t key[TR];
#pragma unroll
    for (int u = 0; u < TR; ++u) key[u] = order_key(v[u]);
    select_run<true>(key, n, tk.k, sh, [&](int u, int slot) { out[slot] = sel_cand<TR>(u); });
  }
}

// Prefill path (bf16 queries and keys, head_dim 128, many queries per
// sequence). The scores of a block of consecutive query rows form a GEMM
// [rows x heads, 128] x [128, keys] followed by the per-head ReLU and weighted
// head sum, and the same keys serve every row of the block. A workgroup of 8
// waves keeps the query fragments of its rows in registers for its whole key
// range and streams the keys through LDS in blocks of 128.
//
// Each wave owns 64 (query, head) rows as two 32-row M-tiles of
// v_mfma_f32_32x32x16_bf16 (4, 2 or 1 queries for 16, 32 or 64 heads) and a
// block is four 32-key N-tiles, 8 K-steps each. The 32x32 shape leaves
// room for about five VALU ops under each 32-cycle MFMA, which the ReLU,
// weight and head sum (two ops per accumulator element) fit: each N-tile's
// MFMAs issue alongside the previous N-tile's epilogue (the first one's
// alongside the previous block's last), so the barrier between blocks never
// leaves the matrix core without work.
//
// Keys reach LDS by direct global-to-LDS copies (two buffers): a block's
// copies go out at the start of the previous block and are awaited before the
// barrier that ends it, so no key passes through registers (against staging
// through registers and LDS stores: 823-837 vs 843-858 us at the 4096-query
// prefill). LDS rows are 256 B with their 16-byte chunks XOR-swizzled by the
// key's low bits, applied through the choice of source address, so the 32 keys
// of one B fragment spread over all bank groups. A lane's
// head sum covers 16 or 32 of its query's heads; one permlane32 swap adds the
// other half and leaves lane l with the score of key l of the block, so every
// query row stores 256 contiguous bytes.
constexpr int kPfThreads = 512;
constexpr int kPfWaves = kPfThreads / kWave;
// Keys per LDS block (four 32-key N-tiles): against blocks of 64, half the
// barriers and score-store branches per key (838 vs 865 us at the 4096-query
// prefill with 32 heads, 476-479 vs 499-514 us with 16).
constexpr int kPfKeys = 128;


// CONTIG: the page size is a multiple of the key block, so each block is
// consecutive rows of one page, found with one (scalar) block-table read.
template <int H, bool CONTIG>
__global__ __launch_bounds__(kPfThreads, 1) void indexer_prefill_kernel(
    const int32_t *__restrict__ block_table, const int32_t *__restrict__ seq_lens,
    const int32_t *__restrict__ cu_q, int batch, int total_q, int max_seq_len, int64_t bt_stride,
    const uint16_t *__restrict__ q_idx, const float *__restrict__ w,
    const uint8_t *__restrict__ kdata, int64_t num_pages, int page_size,
    float *__restrict__ scores, int64_t ld, int keys_per_split, FastDiv pdiv) {
  constexpr int QW = 64 / H;           // query rows per wave
  constexpr int QB = kPfWaves * QW;    // query rows per workgroup
  constexpr int KB = kPfKeys;                            // keys per LDS block
  constexpr int kNT = KB / 32;                           // 32-key N-tiles per block
  static_assert(kNT == 4, "the block loop below is written for four N-tiles");
  constexpr int kPfChunks = KB * kIdxDim * 2 / 16;       // 16-byte chunks per block
  __shared__ u32x4_t kbuf[2][kPfChunks];

  const int qblk = blockIdx.x, split = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int lc = lane & 31, lh = lane >> 5;
  if (b >= batch) return;
  const int L = min(max(seq_lens[b], 0), max_seq_len);
  const int q0 = min(max(cu_q[b], 0), total_q);
  const int qn = min(max(cu_q[b + 1], q0), total_q) - q0;
  const int i0 = qblk * QB;
  if (i0 >= qn) return;
  const int nq = min(QB, qn - i0);
  const int t_first = L - qn + i0;
  const int t_last = t_first + nq - 1;
  const int kbeg = split * keys_per_split;
  if (t_last < 0 || kbeg > t_last) return;
  const int kend = min(kbeg + keys_per_split, t_last + 1);
  const int nblk = (kend - kbeg + KB - 1) / KB;

  // Row 32 * m + x of this wave is (query u = (32 m + x) / H, head (32 m + x) % H).
  // A fragments: lane (lh, lc) holds row 32 * m + lc, dims 16 * s + 8 * lh .. + 8.
  // Accumulator element 4 * i + r of M-tile m is row 32 * m + 8 * i + 4 * lh + r.
  u32x4_t a[2][8];
  float wr[2][16];
  int tq[QW];
  int64_t orow[QW];
#pragma unroll
  for (int u = 0; u < QW; ++u) {
    const int qi = wv * QW + u;
    orow[u] = (int64_t)(q0 + i0 + min(qi, nq - 1)) * ld;
    tq[u] = qi < nq ? t_first + qi : -1;
  }
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int xa = 32 * m + lc;
    const int64_t rowa = q0 + i0 + min(wv * QW + xa / H, nq - 1);
    const uint16_t *qp = q_idx + (rowa * H + xa % H) * kIdxDim + 8 * lh;
#pragma unroll
    for (int s = 0; s < 8; ++s) a[m][s] = ldg16(qp + 16 * s);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int x = 32 * m + 8 * (e >> 2) + 4 * lh + (e & 3);
      const int64_t roww = q0 + i0 + min(wv * QW + x / H, nq - 1);
      wr[m][e] = w[roww * H + x % H];
    }
  }

  // Staging: direct global-to-LDS copies. Copy i of wave wv fills the block's
  // LDS chunks 64 (8 i + wv) + lane: key 4 (8 i + wv) + lane / 16, slot
  // lane % 16, which holds the key's global chunk slot ^ (key & 15).
  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  constexpr int kCopies = KB / 32;  // per wave per block
  const int64_t bt_row = (int64_t)b * bt_stride;
  int btv[kCopies];
  auto ckey = [&](int i) { return 4 * (8 * i + wv) + (lane >> 4); };
  auto key_pos = [&](int blk, int i) { return min(kbeg + blk * KB + ckey(i), t_last); };
  auto clamp_page = [&](int64_t page) { return dsa::clamp_page(page, num_pages); };
  auto bt_load = [&](int blk) {
    if constexpr (CONTIG) {
      btv[0] = block_table[bt_row + (int)fast_div((uint32_t)(kbeg + blk * KB), pdiv)];
    } else {
#pragma unroll
      for (int i = 0; i < kCopies; ++i)
        btv[i] = block_table[bt_row + (int)fast_div((uint32_t)key_pos(blk, i), pdiv)];
    }
  };
  auto copy = [&](int blk, int buf) {
    const lds_u8 *dst0 = (const lds_u8 *)&kbuf[buf][0];
    if constexpr (CONTIG) {
      const int kb0 = kbeg + blk * KB;
      const int pidx = (int)fast_div((uint32_t)kb0, pdiv);
      const int64_t page = clamp_page(btv[0]);
      const uint8_t *base = kdata + (page * page_size + (kb0 - pidx * page_size)) * (2 * kIdxDim);
#pragma unroll
      for (int i = 0; i < kCopies; ++i) {
        const int key = ckey(i);
        idx_lds_load16(base + key * (2 * kIdxDim) + 16 * ((lane & 15) ^ (key & 15)),
                       dst0 + 1024 * (8 * i + wv));
      }
    } else {
#pragma unroll
      for (int i = 0; i < kCopies; ++i) {
        const int key = ckey(i);
        const int pos = key_pos(blk, i);
        const int in_page = pos - (int)fast_div((uint32_t)pos, pdiv) * page_size;
        const int64_t row = clamp_page(btv[i]) * page_size + in_page;
        idx_lds_load16(kdata + row * (2 * kIdxDim) + 16 * ((lane & 15) ^ (key & 15)),
                       dst0 + 1024 * (8 * i + wv));
      }
    }
  };

  // B fragment of N-tile n, step s: lane (lh, lc) reads key 32 n + lc, chunk 2 s + lh.
  auto mma = [&](const u32x4_t *kb, int n, f32x16_t (&acc)[2]) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[m][e] = 0.0f;
    const int key = 32 * n + lc;
    u32x4_t bq[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) bq[s] = kb[key * 16 + ((2 * s + lh) ^ (key & 15))];
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int m = 0; m < 2; ++m) acc[m] = mfma_32x32x16_bf16(a[m][s], bq[s], acc[m]);
  };
  // Issue order of one N-tile phase: B reads run two K-steps ahead of the
  // MFMAs that use them, and four VALU ops of the other tile's epilogue follow
  // each MFMA.
  auto phase_order = [&]() {
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      if ((i & 1) == 0 && i / 2 + 2 < 8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };
  auto epi = [&](const f32x16_t (&acc)[2], float (&p)[QW]) {
#pragma unroll
    for (int u = 0; u < QW; ++u) p[u] = 0.0f;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int u = (32 * m + 8 * (e >> 2)) / H;
        p[u] = fmaf(wr[m][e], relu_bits(acc[m][e]), p[u]);
      }
  };
  // Lanes l and l ^ 32 hold the two halves of a query's head sum for key
  // 32 n + (l & 31); the swap pairs tile 0's upper half with tile 1's lower.
  // half h of block blk: keys 64 h .. 64 h + 63
  auto store = [&](int blk, int half, const float (&p0)[QW], const float (&p1)[QW]) {
    const int pos = kbeg + blk * KB + 64 * half + lane;
#pragma unroll
    for (int u = 0; u < QW; ++u) {
      auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0[u]), __float_as_uint(p1[u]),
                                                 false, false);
      const float v = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      if (pos <= tq[u] && pos < kend) scores[orow[u] + pos] = v;
    }
  };

  bt_load(0);
  // every compiler-visible load (queries, weights, the first table entry)
  // lands before the first direct copies, which the compiler does not count
  __builtin_amdgcn_s_waitcnt(0);
  copy(0, 0);
  if (nblk > 1) bt_load(1);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // Block blk: N-tile 0's MFMAs with the epilogue of block blk - 1's N-tile 3
  // (zeros before the first block, never stored), then each N-tile's MFMAs
  // with the previous N-tile's epilogue; the previous block's second half is
  // stored after N-tile 0, this block's first half after N-tile 2. The issue
  // pattern interleaves one MFMA with four VALU.
  f32x16_t acc0[2], acc1[2];
  float p0[QW], p1[QW];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc1[m][e] = 0.0f;
#pragma unroll
  for (int u = 0; u < QW; ++u) p0[u] = 0.0f;
  // (the empty asm statements keep each epilogue in its N-tile's block, where
  // the issue pattern interleaves it with the MFMAs; left alone, the compiler
  // sinks it below the branches that follow, after the last MFMA)
  auto pin = [](float (&p)[QW]) {
#pragma unroll
    for (int u = 0; u < QW; ++u) asm volatile("" : "+v"(p[u]));
  };
  for (int blk = 0; blk < nblk; ++blk) {
    const u32x4_t *kb = kbuf[blk & 1];
    // the other buffer was last read in block blk - 1, before the barrier
    if (blk + 1 < nblk) copy(blk + 1, (blk & 1) ^ 1);
    mma(kb, 0, acc0);
    epi(acc1, p1);
    phase_order();
    pin(p1);
    if (blk > 0) store(blk - 1, 1, p0, p1);
    mma(kb, 1, acc1);
    epi(acc0, p0);
    phase_order();
    pin(p0);
    mma(kb, 2, acc0);
    epi(acc1, p1);
    phase_order();
    pin(p1);
    store(blk, 0, p0, p1);
    mma(kb, 3, acc1);
    epi(acc0, p0);
    phase_order();
    pin(p0);
    if (blk + 2 < nblk) bt_load(blk + 2);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt 0: this wave's copies of block blk + 1 landed
    __syncthreads();
  }
  epi(acc1, p1);
  store(nblk - 1, 1, p0, p1);
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

// Workgroups that fill the chip once: the prefill grid splits each sequence's
// key range until the query blocks times the splits reach this count.
constexpr int kFillWorkgroups = 256;
// Queries per sequence from which the prefill kernel takes over.
constexpr int kPrefillMinQ = 16;

template <int H>
hipError_t launch_prefill(const BatchArgs &bt, const void *q_idx, const float *w,
                          const CacheArgs &keys, float *scores, int64_t ld, hipStream_t stream) {
  constexpr int QB = kPfWaves * (64 / H);
  constexpr int KB = kPfKeys;
  const int qblocks = (bt.max_q + QB - 1) / QB;
  const int kblocks = (bt.max_seq_len + KB - 1) / KB;
  const int64_t units = (int64_t)qblocks * bt.batch;
  int splits = (int)std::min<int64_t>((kFillWorkgroups + units - 1) / units, kblocks);
  splits = std::max(splits, 1);
  const int keys_per_split = ((kblocks + splits - 1) / splits) * KB;
  splits = (bt.max_seq_len + keys_per_split - 1) / keys_per_split;
  if (splits > 65535 || bt.batch > 65535) return hipErrorInvalidConfiguration;
  dim3 grid(qblocks, splits, bt.batch);
  const FastDiv pdiv = make_fast_div((uint32_t)keys.page_size);
  auto kernel = keys.page_size % KB == 0 ? indexer_prefill_kernel<H, true>
                                         : indexer_prefill_kernel<H, false>;
  hipLaunchKernelGGL(kernel, grid, dim3(kPfThreads), 0, stream, bt.block_table, bt.seq_lens,
                     bt.cu_q, bt.batch, bt.total_q, bt.max_seq_len, bt.bt_stride,
                     static_cast<const uint16_t *>(q_idx), w,
                     static_cast<const uint8_t *>(keys.data), keys.num_pages, keys.page_size,
                     scores, ld, keys_per_split, pdiv);
  return hipGetLastError();
}

template <int NMT, int QG, bool FP8, bool PMAX = false, int TR = 0>
hipError_t launch_stream(const BatchArgs &bt, const void *q_idx, const float *w,
                         const CacheArgs &keys, float *scores, int64_t ld, hipStream_t stream,
                         int page_blocks = 1, FusedTopk tk = {}) {
  const int qgroups = (bt.max_q + QG - 1) / QG;
  const int64_t seq_blocks = (bt.max_seq_len + kStreamKeys - 1) / kStreamKeys;
  const int64_t units = (int64_t)qgroups * bt.batch;
  // kStreamBlocks blocks per query row of the group (the query block a
  // workgroup loads grows with the group; short runs keep ragged batches
  // balanced), shortened when the batch would give too few workgroups
  int64_t run = (int64_t)kStreamBlocks * QG;
  run = std::min<int64_t>(run, std::max<int64_t>(kStreamBlocks,
                                                 seq_blocks * units / kStreamWorkgroups));
  run = std::min<int64_t>(run, seq_blocks);
  if (TR > 0 && run > kStreamBlocks) return hipErrorInvalidConfiguration;  // one buffer per run
  const int64_t chunks = (seq_blocks + run - 1) / run;
  if (qgroups > 65535 || bt.batch > 65535 || chunks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  dim3 grid((unsigned)chunks, qgroups, bt.batch);
  hipLaunchKernelGGL((indexer_stream_kernel<NMT, QG, FP8, PMAX, TR>), grid, dim3(256), 0, stream,
                     bt.block_table, bt.seq_lens, bt.cu_q, bt.batch, bt.total_q, bt.max_seq_len,
                     bt.bt_stride, static_cast<const uint16_t *>(q_idx), w,
                     static_cast<const uint8_t *>(keys.data), keys.scale, keys.num_pages,
                     keys.page_size, make_fast_div((uint32_t)keys.page_size), scores, ld, (int)run,
                     page_blocks, tk);
  return hipGetLastError();
}

template <bool FP8>
hipError_t dispatch_mfma(const BatchArgs &bt, const void *q_idx, const float *w, int n_heads,
                         const CacheArgs &keys, float *scores, int64_t ld, hipStream_t stream) {
  // pages holding whole 64-key blocks: stream the keys through LDS
  if (keys.page_size % kStreamKeys == 0 && bt.max_q < kPrefillMinQ) {
    const bool multi = bt.max_q > 1;
    switch (n_heads) {
      case 16:
        return multi ? launch_stream<1, 4, FP8>(bt, q_idx, w, keys, scores, ld, stream)
                     : launch_stream<1, 1, FP8>(bt, q_idx, w, keys, scores, ld, stream);
      case 32:
        return multi ? launch_stream<2, 4, FP8>(bt, q_idx, w, keys, scores, ld, stream)
                     : launch_stream<2, 1, FP8>(bt, q_idx, w, keys, scores, ld, stream);
      default:
        return multi ? launch_stream<4, 2, FP8>(bt, q_idx, w, keys, scores, ld, stream)
                     : launch_stream<4, 1, FP8>(bt, q_idx, w, keys, scores, ld, stream);
    }
  }
  if (!FP8 && bt.max_q >= kPrefillMinQ) {
    switch (n_heads) {
      case 16: return launch_prefill<16>(bt, q_idx, w, keys, scores, ld, stream);
      case 32: return launch_prefill<32>(bt, q_idx, w, keys, scores, ld, stream);
      default: return launch_prefill<64>(bt, q_idx, w, keys, scores, ld, stream);
    }
  }
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

// Page maxima straight from the streaming kernel (no token scores in HBM):
// keys streamed in 64-key blocks and selection pages of one block.
template <bool FP8>
hipError_t dispatch_page_max(const BatchArgs &bt, const void *q_idx, const float *w, int n_heads,
                             const CacheArgs &keys, int32_t sel_page, float *page_scores,
                             int64_t ld_pages, hipStream_t stream) {
  const int pb = sel_page / kStreamKeys;
  const bool multi = bt.max_q > 1;
  switch (n_heads) {
    case 16:
      return multi ? launch_stream<1, 4, FP8, true>(bt, q_idx, w, keys, page_scores, ld_pages, stream, pb)
                   : launch_stream<1, 1, FP8, true>(bt, q_idx, w, keys, page_scores, ld_pages, stream, pb);
    case 32:
      return multi ? launch_stream<2, 4, FP8, true>(bt, q_idx, w, keys, page_scores, ld_pages, stream, pb)
                   : launch_stream<2, 1, FP8, true>(bt, q_idx, w, keys, page_scores, ld_pages, stream, pb);
    default:
      return multi ? launch_stream<4, 2, FP8, true>(bt, q_idx, w, keys, page_scores, ld_pages, stream, pb)
                   : launch_stream<4, 1, FP8, true>(bt, q_idx, w, keys, page_scores, ld_pages, stream, pb);
  }
}

// Scores plus the fused top-k: one query row per sequence, keys streamed in
// 64-key blocks; TR candidates per lane of the final selection.
constexpr int kFusedMaxLen = 256 * 64;  // positions per row (TR = 64)

template <bool FP8, int TR>
hipError_t dispatch_fused_topk(const BatchArgs &bt, const void *q_idx, const float *w,
                               int n_heads, const CacheArgs &keys, float *scores, int64_t ld,
                               FusedTopk tk, hipStream_t stream) {
  switch (n_heads) {
    case 16: return launch_stream<1, 1, FP8, false, TR>(bt, q_idx, w, keys, scores, ld, stream, 1, tk);
    case 32: return launch_stream<2, 1, FP8, false, TR>(bt, q_idx, w, keys, scores, ld, stream, 1, tk);
    default: return launch_stream<4, 1, FP8, false, TR>(bt, q_idx, w, keys, scores, ld, stream, 1, tk);
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

bool indexer_page_max_supported(const BatchArgs &bt, int32_t q_dtype, int32_t n_heads,
                                int32_t head_dim, const CacheArgs &keys, int32_t sel_page) {
  const bool heads_ok = n_heads == 16 || n_heads == 32 || n_heads == 64;
  const bool page_ok = sel_page == kStreamKeys;
  return q_dtype == DSA_BF16 && head_dim == kIdxDim && heads_ok && page_ok &&
         (keys.dtype == DSA_BF16 || keys.dtype == DSA_FP8_E4M3) &&
         keys.page_size % kStreamKeys == 0 && bt.max_q < kPrefillMinQ;
}

hipError_t launch_indexer_page_scores(const BatchArgs &bt, const void *q_idx, const float *w,
                                      int32_t n_heads, const CacheArgs &keys, int32_t sel_page,
                                      float *page_scores, int64_t ld_pages, hipStream_t stream) {
  if (bt.total_q == 0 || bt.max_seq_len == 0) return hipSuccess;
  if (keys.dtype == DSA_FP8_E4M3)
    return dispatch_page_max<true>(bt, q_idx, w, n_heads, keys, sel_page, page_scores, ld_pages,
                                   stream);
  return dispatch_page_max<false>(bt, q_idx, w, n_heads, keys, sel_page, page_scores, ld_pages,
                                  stream);
}

bool indexer_topk_supported(const BatchArgs &bt, int32_t q_dtype, int32_t n_heads,
                            int32_t head_dim, const CacheArgs &keys) {
  const bool heads_ok = n_heads == 16 || n_heads == 32 || n_heads == 64;
  return q_dtype == DSA_BF16 && head_dim == kIdxDim && heads_ok &&
         (keys.dtype == DSA_BF16 || keys.dtype == DSA_FP8_E4M3) &&
         keys.page_size % kStreamKeys == 0 && bt.max_q <= 1 && bt.max_seq_len <= kFusedMaxLen;
}

size_t indexer_topk_state_bytes(int32_t total_q) {
  return total_q < 1 ? 0 : (size_t)total_q * kFusedRowWords * sizeof(uint32_t);
}

hipError_t launch_indexer_topk(const BatchArgs &bt, const void *q_idx, const float *w,
                               int32_t n_heads, const CacheArgs &keys, int32_t k,
                               int32_t *indices, float *scores, int64_t ld_scores,
                               uint32_t *state, hipStream_t stream) {
  if (bt.total_q == 0) return hipSuccess;
  BatchArgs b = bt;
  b.max_seq_len = std::max(b.max_seq_len, 1);  // empty rows still get their -1 lists
  const FusedTopk tk{k, indices, state};
  const bool fp8 = keys.dtype == DSA_FP8_E4M3;
  if (b.max_seq_len <= 128 * 64)
    return fp8 ? dispatch_fused_topk<true, 32>(b, q_idx, w, n_heads, keys, scores, ld_scores, tk, stream)
               : dispatch_fused_topk<false, 32>(b, q_idx, w, n_heads, keys, scores, ld_scores, tk, stream);
  return fp8 ? dispatch_fused_topk<true, 64>(b, q_idx, w, n_heads, keys, scores, ld_scores, tk, stream)
             : dispatch_fused_topk<false, 64>(b, q_idx, w, n_heads, keys, scores, ld_scores, tk, stream);
}

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
