// Exact block-wide top-k selection over scores held in registers ("GLM-5.2 on
// vLLM Ascend: Request-to-Backend Inference Path", section "8. The SFA
// backend, step by step": the indexer returns the 2,048 best token
// positions).
//
// Order: larger score first; equal scores by lower position first; -0.0 is
// folded into +0.0 so the two compare equal. Scores map to order-preserving
// 32-bit keys, so the order is (key descending, position ascending).
//
// A block of NW waves holds candidates wave-major: wave w, slice u < R, lane
// l holds candidate 64 R w + 64 u + l (sel_cand), so a slice is 64
// consecutive candidates (one coalesced 256-byte load) and a wave's
// candidates are one contiguous range.
//  * Three radix levels (11, 11 and 10 bits) use three LDS histograms that are
//    cleared before the first level. With eight or more waves one wave scans
//    a level's histogram and hands the digit to the others through LDS (a
//    second barrier, but one scan of the histogram instead of one per wave:
//    the scans' LDS reads were the level's cost); with fewer waves each wave
//    scans it itself, and a level costs one barrier.
//    Bin b sits at word b + 4 (b / 32): lane l of a scanning wave owns bins
//    [32 l, 32 l + 32) and reads them with 16-byte loads that no other lane of
//    its group of eight shares a bank with.
//  * The selection stops at the first level whose chosen bin is kept whole
//    (its count equals what is still needed): the keys above the bin and all
//    keys in it are then the top k. Continuous scores usually stop after two
//    levels.
//  * Ordered emit: each wave counts its keys above the bin and in it, one
//    scan of the NW wave totals gives every wave its offsets, and inside the
//    wave the slices are walked in order with running counts plus a popcount
//    of the slice's ballot below the lane: every kept candidate gets its slot
//    in ascending candidate order, with no sort.
#pragma once

#include "dsa_device.h"

namespace dsa {

constexpr int kSelBins = 2048;                    // 11-bit digits
constexpr int kSelBinsWords = kSelBins / 32 * 36;  // padded histogram
// Levels 1 and 2 may count into C1 and C2 copies of their histograms, lane
// l into copy l % copies, so lanes whose keys share a bin hit different
// words; copies sit kSelCopyWords apart, 8 words past a multiple of the 32
// banks, so the same bin of two copies is in different banks. This pays
// where the keys crowd into few bins (the survivors of earlier selections);
// on whole rows of scores the extra histogram reads cost more than the
// spared conflicts.
constexpr int kSelCopyWords = kSelBinsWords + 8;

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  u = (u == 0x80000000u) ? 0u : u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int sel_bin(uint32_t b) { return (int)(b + 4 * (b >> 5)); }

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}

// Scans over the 64 lanes of a wave without LDS: DPP row shifts scan each row
// of 16 lanes (lanes shifted in from outside the row read 0), then the totals
// of the other rows, read as scalars from lanes 0, 16, 32 and 48 (suffix) or
// 15, 31, 47 (prefix), are added per row.
// Suffix sum: lane l gets the total of lanes >= l (row_shl n: lane l reads l + n).
__device__ __forceinline__ uint32_t wave_suffix_sum(uint32_t v) {
  v += dpp_u32<0x101>(v);
  v += dpp_u32<0x102>(v);
  v += dpp_u32<0x104>(v);
  v += dpp_u32<0x108>(v);
  const uint32_t r1 = __builtin_amdgcn_readlane(v, 16), r2 = __builtin_amdgcn_readlane(v, 32),
                 r3 = __builtin_amdgcn_readlane(v, 48);
  const int row = (threadIdx.x & 63) >> 4;
  return v + (row == 0 ? r1 + r2 + r3 : row == 1 ? r2 + r3 : row == 2 ? r3 : 0u);
}

// Inclusive prefix sum: lane l gets the total of lanes <= l (row_shr n: lane l reads l - n).
__device__ __forceinline__ uint32_t wave_prefix_sum(uint32_t v) {
  v += dpp_u32<0x111>(v);
  v += dpp_u32<0x112>(v);
  v += dpp_u32<0x114>(v);
  v += dpp_u32<0x118>(v);
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31),
                 r2 = __builtin_amdgcn_readlane(v, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return v + (row == 3 ? r0 + r1 + r2 : row == 2 ? r0 + r1 : row == 1 ? r0 : 0u);
}

// Every lane of the calling wave: the digit of the need-th largest candidate
// in a histogram of NB bins (sel_bin layout), how many candidates with that
// digit are still needed, and how many there are. Two stages, neither with a
// serial search: lane totals of 32 (16) bins and their suffix sums find the
// lane L whose bins hold the crossing; then lane i < 32 (16) reads bin
// 32 L + i, and a second suffix sum and ballot find the bin.
template <int NB, int C = 1>
__device__ __forceinline__ void wave_pick(const uint32_t *hist, uint32_t need, uint32_t &digit,
                                          uint32_t &rest, uint32_t &count) {
  constexpr int per = NB / 64;
  const int lane = threadIdx.x & 63;
  uint32_t mine = 0;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const u32x4_t *src = reinterpret_cast<const u32x4_t *>(hist + c * kSelCopyWords + sel_bin(per * lane));
#pragma unroll
    for (int i = 0; i < per / 4; ++i) {
      const u32x4_t q = src[i];
      mine += (q.x + q.y) + (q.z + q.w);
    }
  }
  const uint32_t suf = wave_suffix_sum(mine);
  const uint32_t above = suf - mine;
  const uint64_t who = __ballot(above < need && suf >= need);
  const int L = who != 0ull ? __ffsll((unsigned long long)who) - 1 : 0;
  const uint32_t above_l = __builtin_amdgcn_readlane(above, L);
  uint32_t hb = 0;
  if (lane < per) {
#pragma unroll
    for (int c = 0; c < C; ++c) hb += hist[c * kSelCopyWords + sel_bin(per * L + lane)];
  }
  const uint32_t s2 = wave_suffix_sum(hb);  // lanes >= per add 0
  const uint64_t hit = __ballot(lane < per && above_l + s2 >= need);
  const int i = hit != 0ull ? 63 - __clzll(hit) : 0;
  const uint32_t s_i = __builtin_amdgcn_readlane(s2, i), h_i = __builtin_amdgcn_readlane(hb, i);
  digit = (uint32_t)(per * L + i);
  count = h_i;
  rest = need - (above_l + s_i - h_i);
}

// The digit pick of one level: with many waves one wave scans the histogram
// and hands the result to the others through LDS (one barrier instead of
// every wave reading the whole histogram); with few waves each picks itself.
template <int NB, int C, int NW>
__device__ __forceinline__ void block_pick(const uint32_t *hist, uint32_t need_in, uint32_t *slot,
                                           uint32_t &digit, uint32_t &rest, uint32_t &count) {
  if constexpr (NW >= 8) {
    if ((threadIdx.x >> 6) == 0) {
      wave_pick<NB, C>(hist, need_in, digit, rest, count);
      if ((threadIdx.x & 63) == 0) {
        slot[0] = digit;
        slot[1] = rest;
        slot[2] = count;
      }
    }
    __syncthreads();
    digit = slot[0];
    rest = slot[1];
    count = slot[2];
  } else {
    wave_pick<NB, C>(hist, need_in, digit, rest, count);
  }
}

// LDS of one selection: the three histograms and the packed per-wave counts.
template <int NW, int R, int C1 = 1, int C2 = 1>
struct alignas(16) SelectShared {
  static constexpr int kCopies1 = C1, kCopies2 = C2;
  uint32_t hist1[C1 * kSelCopyWords];
  uint32_t hist2[C2 * kSelCopyWords];
  uint32_t hist3[kSelBinsWords];
  uint32_t cnt[NW];
  uint32_t pick[3];  // digit, still needed, count: one wave's pick for the block
};

// Candidate index held by slice u of the calling lane (wave-major layout).
template <int R>
__device__ __forceinline__ int sel_cand(int u) {
  return (threadIdx.x >> 6) * (kWave * R) + u * kWave + (threadIdx.x & 63);
}

// Zero the histograms (no barrier: select_run starts with one).
template <class Sh>
__device__ __forceinline__ void select_clear(Sh &sh) {
  constexpr int NW = sizeof(sh.cnt) / sizeof(uint32_t);
  constexpr int kWords = (Sh::kCopies1 + Sh::kCopies2) * kSelCopyWords + kSelBinsWords;
  static_assert(kWords % 4 == 0, "16-byte clears");
  u32x4_t *h = reinterpret_cast<u32x4_t *>(&sh.hist1[0]);
  for (int i = threadIdx.x; i < kWords / 4; i += NW * kWave) h[i] = u32x4_t{0u, 0u, 0u, 0u};
}

// The k best of the n candidates sel_cand(u) < n (n > k): emit(u, slot) is
// called once for every kept candidate, with its slot in [0, k) of the
// ascending-candidate list. Every thread of the block must call it.
// kH1Given: the caller has already filled hist1 (one copy) with the level-1
// counts of exactly these n keys, e.g. summed over the workgroups that
// produced them, and the level-1 pass is skipped.
template <bool kH1Given = false, int NW, int R, int C1, int C2, typename Emit>
__device__ __forceinline__ void select_run(const uint32_t (&key)[R], int n, int k,
                                           SelectShared<NW, R, C1, C2> &sh, Emit emit) {
  static_assert(!kH1Given || C1 == 1, "a given level-1 histogram has one copy");
  static_assert(NW * R * kWave < 65536, "16-bit packed counts");
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // candidates of this wave: slice u, lane l exists when l < n_w - 64 u
  const int n_w = __builtin_amdgcn_readfirstlane(n) - wv * (kWave * R);
  // (with 32 slices the bound passes through an empty asm, so that each use
  // compares afresh instead of keeping R lane masks live in scalar registers)
  auto valid = [&](int u) {
    int b = n_w - u * kWave;
    if constexpr (R >= 32) asm volatile("" : "+s"(b));
    return lane < b;
  };
  __syncthreads();  // histograms cleared
  uint32_t *h1 = sh.hist1 + (lane % C1) * kSelCopyWords;
  uint32_t *h2 = sh.hist2 + (lane % C2) * kSelCopyWords;

  // level 1: bits 31..21
  if constexpr (!kH1Given) {
#pragma unroll
    for (int u = 0; u < R; ++u)
      if (valid(u)) atomicAdd(&h1[sel_bin(key[u] >> 21)], 1u);
    __syncthreads();
  }
  uint32_t d, need, count;
  block_pick<kSelBins, C1, NW>(sh.hist1, (uint32_t)k, sh.pick, d, need, count);
  uint32_t prefix = d << 21;
  int shift = 21;
  if (need != count) {
    // level 2: bits 20..10 of the keys in the chosen bin
#pragma unroll
    for (int u = 0; u < R; ++u)
      if (valid(u) && (key[u] >> 21) == d)
        atomicAdd(&h2[sel_bin((key[u] >> 10) & 2047u)], 1u);
    __syncthreads();
    block_pick<kSelBins, C2, NW>(sh.hist2, need, sh.pick, d, need, count);
    prefix |= d << 10;
    shift = 10;
    if (need != count) {
      // level 3: bits 9..0
#pragma unroll
      for (int u = 0; u < R; ++u)
        if (valid(u) && (key[u] >> 10) == (prefix >> 10))
          atomicAdd(&sh.hist3[sel_bin(key[u] & 1023u)], 1u);
      __syncthreads();
      block_pick<kSelBins / 2, 1, NW>(sh.hist3, need, sh.pick, d, need, count);
      prefix |= d;
      shift = 0;
    }
  }
  const uint32_t tp = prefix >> shift;

  // ordered emit: "above" = keys above the chosen bin, "in" = keys in it, of
  // which the first `need` (in candidate order) are kept. Wave totals,
  // packed (above << 16 | in), then the exclusive sum over earlier waves.
  uint32_t ngt = 0, neq = 0;
#pragma unroll
  for (int u = 0; u < R; ++u) {
    const uint32_t hd = key[u] >> shift;
    const bool vu = valid(u);
    ngt += (vu && hd > tp) ? 1u : 0u;
    neq += (vu && hd == tp) ? 1u : 0u;
  }
  const uint32_t wsum = wave_prefix_sum((ngt << 16) | neq);
  if (lane == kWave - 1) sh.cnt[wv] = wsum;
  __syncthreads();
  const uint32_t before = wave_prefix_sum(lane < wv ? sh.cnt[lane] : 0u);
  uint32_t off = __builtin_amdgcn_readlane(before, kWave - 1);
  uint32_t gt_run = off >> 16, eq_run = off & 0xFFFFu;
#pragma unroll
  for (int u = 0; u < R; ++u) {
    const uint32_t hd = key[u] >> shift;
    const bool vu = valid(u);
    const bool gt = vu && hd > tp;
    const bool eq = vu && hd == tp;
    const uint64_t mg = __ballot(gt);
    const uint64_t me = __ballot(eq);
    const uint32_t gt_before =
        gt_run + __builtin_amdgcn_mbcnt_hi((uint32_t)(mg >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mg, 0u));
    const uint32_t eq_before =
        eq_run + __builtin_amdgcn_mbcnt_hi((uint32_t)(me >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)me, 0u));
    const uint32_t slot = gt ? gt_before + min(eq_before, need)
                             : (eq && eq_before < need) ? gt_before + eq_before : (uint32_t)k;
    if (slot < (uint32_t)k) emit(u, (int)slot);
    gt_run += (uint32_t)__popcll(mg);
    eq_run += (uint32_t)__popcll(me);
  }
}

}  // namespace dsa
