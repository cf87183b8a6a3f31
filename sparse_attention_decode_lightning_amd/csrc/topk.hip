// Per-row top-k of the indexer scores on gfx950 ("GLM-5.2 on vLLM Ascend:
// Request-to-Backend Inference Path", section "8. The SFA backend, step by
// step": the indexer returns token positions, 2,048 per query).
//
// Order: larger score first; equal scores by lower position first; -0.0 is
// folded into +0.0 so the two compare equal. Scores map to order-preserving
// 32-bit keys, so the order is (key descending, position ascending).
//
// One 1024-thread workgroup selects among at most kChunk candidates held in
// LDS as keys:
//  * three radix passes (11, 11 and 10 bits, most significant first) over the
//    candidates that still match the chosen prefix find the k-th largest key
//    tau and how many keys equal to tau must be kept ("need"); each pass is a
//    shared LDS histogram that one wave then scans from the top, so a pass
//    costs two barriers;
//  * one ordered pass: each thread owns a contiguous run of candidates, counts
//    its keys > tau and == tau, and a block-wide exclusive scan of those counts
//    gives every kept candidate its output slot, so positions come out in
//    ascending order with no sort.
// Rows longer than kChunk run in two phases: phase 1 selects the top-k of each
// kChunk-position chunk (one workgroup per row and chunk), phase 2 selects the
// top-k among the chunks' survivors (one workgroup per row). This is exact: a
// position in the row's top-k is also in its chunk's top-k under the same
// order, and the survivors stay in ascending position order when the chunks'
// lists are concatenated.
#include "dsa_device.h"
#include "dsa_internal.h"
#include "dsa_select.h"

namespace dsa {
namespace {

// Candidates of a row: its positions 0..t (unit 1), or the groups of `unit`
// consecutive positions (pages) that hold them, 0..t / unit; none when the
// row has no position.
__device__ __forceinline__ int row_cands(const int32_t *cu_q, const int32_t *seq_lens, int batch,
                                         int total_q, int max_seq_len, int row, FastDiv unit) {
  const int t = row_info(cu_q, seq_lens, batch, total_q, max_seq_len, row).t;
  return t < 0 ? 0 : (int)fast_div((uint32_t)t, unit) + 1;
}

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / kWave;
constexpr int kChunk = 32768;  // candidates per workgroup (keys cached in LDS)
constexpr int kBinsA = 2048;   // 11-bit digits: key bits 31..21, 20..10, then 9..0

// Histogram bins are padded by one word per 64, so that a lane reading 64
// consecutive bins hits a different bank than its neighbours.
__device__ __forceinline__ int padded(int bin) { return bin + (bin >> 6); }

struct TopkShared {
  uint32_t hist_a[kBinsA + kBinsA / 64];
  uint32_t hist_b[kBinsA + kBinsA / 64];
  uint32_t wave_tot[kTopkWaves];
  uint32_t digit, need;
};

// Inclusive prefix sum over the 1024 threads of the block (v per thread).
__device__ __forceinline__ uint32_t block_inclusive_scan(uint32_t v, TopkShared &sh) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t u = __shfl_up(v, off);
    if (lane >= off) v += u;
  }
  if (lane == 63) sh.wave_tot[wv] = v;
  __syncthreads();
  uint32_t before = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) before += w < wv ? sh.wave_tot[w] : 0u;
  __syncthreads();
  return v + before;
}

// One wave finds, in a padded histogram of NB bins, the digit d holding the
// need-th largest candidate: count(digit > d) < need <= count(digit >= d).
// Lane l owns bins [NB/64 * l, NB/64 * (l+1)).
template <int NB>
__device__ __forceinline__ void wave_pick_digit(const uint32_t *hist, uint32_t need,
                                                TopkShared &sh) {
  constexpr int per = NB / 64;
  const int lane = threadIdx.x & 63;
  uint32_t h[per];  // the lane's bins, read once (independent loads, no bank conflicts)
#pragma unroll
  for (int i = 0; i < per; ++i) h[i] = hist[padded(per * lane + i)];
  uint32_t mine = 0;
#pragma unroll
  for (int i = 0; i < per; ++i) mine += h[i];
  // suffix sum over lanes: total of lanes >= l
  uint32_t suf = mine;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t u = __shfl_down(suf, off);
    if (lane + off < 64) suf += u;
  }
  const uint32_t above = suf - mine;  // candidates in lanes > l
  if (above < need && suf >= need) {
    uint32_t acc = above, digit = 0, rest = 0;
    bool found = false;
#pragma unroll
    for (int i = per - 1; i >= 0; --i) {
      const bool here = !found && acc + h[i] >= need;
      digit = here ? (uint32_t)(per * lane + i) : digit;
      rest = here ? need - acc : rest;
      found |= here;
      acc += h[i];
    }
    sh.digit = digit;
    sh.need = rest;
  }
}

// Finds tau (the k-th largest key among keys[0..n)) and how many keys equal to
// tau belong to the top-k. Requires n > k. Both histograms must be zero on
// entry. Passes alternate between the two histograms so that one is cleared
// while the other is counted.
__device__ void radix_select(const uint32_t *keys, int n, uint32_t k, TopkShared &sh,
                             uint32_t &tau, uint32_t &need_out) {
  const int tid = threadIdx.x, wv = tid >> 6;
  // pass 1: bits 31..21 into hist_a
  for (int i = tid; i < n; i += kTopkThreads) atomicAdd(&sh.hist_a[padded(keys[i] >> 21)], 1u);
  __syncthreads();
  if (wv == 0) wave_pick_digit<kBinsA>(sh.hist_a, k, sh);
  __syncthreads();
  uint32_t prefix = sh.digit << 21, need = sh.need;
  // pass 2: bits 20..10 into hist_b (zero on entry) while hist_a is cleared
  for (int i = tid; i < kBinsA + kBinsA / 64; i += kTopkThreads) sh.hist_a[i] = 0;
  for (int i = tid; i < n; i += kTopkThreads) {
    const uint32_t key = keys[i];
    if ((key >> 21) == (prefix >> 21)) atomicAdd(&sh.hist_b[padded((key >> 10) & 2047u)], 1u);
  }
  __syncthreads();
  if (wv == 0) wave_pick_digit<kBinsA>(sh.hist_b, need, sh);
  __syncthreads();
  prefix |= sh.digit << 10;
  need = sh.need;
  // pass 3: bits 9..0 into hist_a
  for (int i = tid; i < n; i += kTopkThreads) {
    const uint32_t key = keys[i];
    if ((key >> 10) == (prefix >> 10)) atomicAdd(&sh.hist_a[padded(key & 1023u)], 1u);
  }
  __syncthreads();
  if (wv == 0) wave_pick_digit<kBinsA / 2>(sh.hist_a, need, sh);
  __syncthreads();
  tau = prefix | sh.digit;
  need_out = sh.need;
}

// Loads n scores into LDS as order keys, with every load of a thread in
// flight before any is converted.
__device__ __forceinline__ void load_keys(const float *src, int n, uint32_t *keys) {
  constexpr int kU = 8;
  for (int base = 0; base < n; base += kU * kTopkThreads) {
    float v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = base + u * kTopkThreads + (int)threadIdx.x;
      v[u] = i < n ? src[i] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = base + u * kTopkThreads + (int)threadIdx.x;
      if (i < n) keys[i] = order_key(v[u]);
    }
  }
}

__device__ __forceinline__ void clear_hists(TopkShared &sh) {
  for (int i = threadIdx.x; i < kBinsA + kBinsA / 64; i += kTopkThreads) sh.hist_a[i] = 0;
  for (int i = threadIdx.x; i < kBinsA + kBinsA / 64; i += kTopkThreads) sh.hist_b[i] = 0;
}

// Writes the kept candidates' positions in candidate order: every key > tau
// and the first `need` keys == tau. pos_of(i) gives candidate i's position;
// out_key (optional) also receives the kept keys.
template <typename PosFn>
__device__ void ordered_emit(const uint32_t *keys, int n, uint32_t tau, uint32_t need,
                             TopkShared &sh, PosFn pos_of, int32_t *out_pos,
                             uint32_t *out_key) {
  const int tid = threadIdx.x;
  const int per = (n + kTopkThreads - 1) / kTopkThreads;
  const int b0 = min(n, tid * per), b1 = min(n, b0 + per);
  uint32_t gt = 0, eq = 0;
  for (int i = b0; i < b1; ++i) {
    const uint32_t key = keys[i];
    gt += key > tau;
    eq += key == tau;
  }
  // counts fit in 16 bits (n <= kChunk), so one scan carries both
  const uint32_t packed = block_inclusive_scan((gt << 16) | eq, sh) - ((gt << 16) | eq);
  uint32_t gt_before = packed >> 16, eq_before = packed & 0xFFFFu;
  for (int i = b0; i < b1; ++i) {
    const uint32_t key = keys[i];
    if (key > tau) {
      const uint32_t slot = gt_before + min(eq_before, need);
      out_pos[slot] = pos_of(i);
      if (out_key) out_key[slot] = key;
      ++gt_before;
    } else if (key == tau) {
      if (eq_before < need) {
        const uint32_t slot = gt_before + eq_before;
        out_pos[slot] = pos_of(i);
        if (out_key) out_key[slot] = key;
      }
      ++eq_before;
    }
  }
}

// Single-phase row top-k (rows of at most kChunk candidates), or phase 1 of
// the two-phase path (one chunk of a long row; survivors to the workspace).
template <bool PHASE1>
__global__ __launch_bounds__(kTopkThreads) void topk_rows_kernel(
    const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ cu_q, int batch,
    int total_q, int max_seq_len, int n_max, FastDiv unit, const float *__restrict__ scores,
    int64_t ld, int k,
    int32_t *__restrict__ indices, int n_chunks, uint32_t *__restrict__ ws_key,
    int32_t *__restrict__ ws_pos) {
  extern __shared__ uint32_t s_keys[];
  __shared__ TopkShared sh;
  const int row = PHASE1 ? blockIdx.x / n_chunks : blockIdx.x;
  const int chunk = PHASE1 ? blockIdx.x % n_chunks : 0;
  const int tid = threadIdx.x;
  const int n_row = row_cands(cu_q, seq_lens, batch, total_q, max_seq_len, row, unit);
  if (!PHASE1 && n_row <= k) {
    int32_t *out = indices + (int64_t)row * k;
    for (int i = tid; i < k; i += kTopkThreads) out[i] = i < n_row ? i : -1;
    return;
  }
  const int c0 = chunk * kChunk;
  const int n = min(kChunk, n_row - c0);
  if (n <= 0) return;
  const float *src = scores + (int64_t)row * ld + c0;
  clear_hists(sh);
  load_keys(src, n, s_keys);
  __syncthreads();
  int32_t *out_pos;
  uint32_t *out_key = nullptr;
  if constexpr (PHASE1) {
    const int64_t base = ((int64_t)row * n_chunks + chunk) * k;
    out_pos = ws_pos + base;
    out_key = ws_key + base;
    if (n <= k) {  // the whole chunk survives
      for (int i = tid; i < n; i += kTopkThreads) {
        out_pos[i] = c0 + i;
        out_key[i] = s_keys[i];
      }
      return;
    }
  } else {
    out_pos = indices + (int64_t)row * k;
  }
  uint32_t tau, need;
  radix_select(s_keys, n, (uint32_t)k, sh, tau, need);
  ordered_emit(s_keys, n, tau, need, sh, [&](int i) { return c0 + i; }, out_pos, out_key);
}

// Phase 2: top-k among the concatenated chunk survivors of one row.
__global__ __launch_bounds__(kTopkThreads) void topk_merge_kernel(
    const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ cu_q, int batch,
    int total_q, int max_seq_len, int n_max, FastDiv unit, int k, int n_chunks,
    const uint32_t *__restrict__ ws_key,
    const int32_t *__restrict__ ws_pos, int32_t *__restrict__ indices) {
  extern __shared__ uint32_t s_keys[];
  __shared__ TopkShared sh;
  __shared__ int s_start[64];
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int n_row = row_cands(cu_q, seq_lens, batch, total_q, max_seq_len, row, unit);
  int32_t *out = indices + (int64_t)row * k;
  if (n_row <= k) {
    for (int i = tid; i < k; i += kTopkThreads) out[i] = i < n_row ? i : -1;
    return;
  }
  // survivors of chunk c: min(k, its length), stored at [c * k, ...)
  if (tid == 0) {
    int acc = 0;
    for (int c = 0; c < n_chunks; ++c) {
      s_start[c] = acc;
      const int len = max(0, min(kChunk, n_row - c * kChunk));
      acc += min(k, len);
    }
    s_start[n_chunks] = acc;
  }
  __syncthreads();
  const int n = s_start[n_chunks];
  const int64_t base = (int64_t)row * n_chunks * k;
  clear_hists(sh);
  auto chunk_of = [&](int i) {
    int c = 0;
    while (c + 1 < n_chunks && s_start[c + 1] <= i) ++c;
    return c;
  };
  constexpr int kU = 8;
  for (int b0 = 0; b0 < n; b0 += kU * kTopkThreads) {
    uint32_t v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = b0 + u * kTopkThreads + tid;
      const int c = chunk_of(i);
      v[u] = i < n ? ws_key[base + (int64_t)c * k + (i - s_start[c])] : 0u;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = b0 + u * kTopkThreads + tid;
      if (i < n) s_keys[i] = v[u];
    }
  }
  __syncthreads();
  auto pos_of = [&](int i) -> int32_t {
    const int c = chunk_of(i);
    return ws_pos[base + (int64_t)c * k + (i - s_start[c])];
  };
  if (n <= k) {  // a single chunk already reduced to exactly k survivors
    for (int i = tid; i < n; i += kTopkThreads) out[i] = pos_of(i);
    return;
  }
  uint32_t tau, need;
  radix_select(s_keys, n, (uint32_t)k, sh, tau, need);
  ordered_emit(s_keys, n, tau, need, sh, pos_of, out, nullptr);
}

constexpr int kRegThreads = 1024;

// Rows of at most R * NT candidates (every row of up to 32K tokens):
// NT threads holding the candidates as keys in registers (slice u of lane l
// of wave w: candidate sel_cand(u) = 64 R w + 64 u + l), selected by select_run (three pre-cleared LDS histograms, one
// barrier per radix level, per-wave digit picks, an early stop once the chosen
// bin is kept whole, a ballot-based ordered emit). The row's scores are
// requested before its length is known (every load stays below
// max_seq_len <= ld) and masked afterwards.
// With `expand` set (a page budget: candidates are pages of `unit`
// positions), the workgroup then also writes the token positions its kept
// pages hold: expand[row][i * unit + o] = page_i * unit + o when that is <= t,
// else -1.
template <int NT, int R>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(8))) void topk_reg_kernel(
    const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ cu_q, int batch,
    int total_q, int max_seq_len, int n_max, FastDiv unit, const float *__restrict__ scores,
    int64_t ld, int k, int32_t *__restrict__ indices, int32_t *__restrict__ expand,
    int unit_size) {
  constexpr int kRegThreads = NT;
  __shared__ SelectShared<NT / kWave, R> sh;
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w0 = __builtin_amdgcn_readfirstlane(tid >> 6) * (kWave * R);  // the wave's first candidate
  const float *src = scores + (int64_t)row * ld + w0 + lane;
  const int lim = n_max - w0;  // slice u of this lane is below n_max when lane < lim - 64 u
  float v[R];
#pragma unroll
  for (int u = 0; u < R; ++u) v[u] = lane < lim - u * kWave ? src[u * kWave] : 0.0f;
  select_clear(sh);
  const int n = row_cands(cu_q, seq_lens, batch, total_q, max_seq_len, row, unit);
  int32_t *out = indices + (int64_t)row * k;
  if (n <= k) {
    for (int i = tid; i < k; i += kRegThreads) out[i] = i < n ? i : -1;
  } else {
    uint32_t key[R];
#pragma unroll
    for (int u = 0; u < R; ++u) key[u] = order_key(v[u]);
    select_run(key, n, k, sh, [&](int u, int slot) { out[slot] = sel_cand<R>(u); });
  }
  if (expand == nullptr) return;
  __syncthreads();  // the row's kept pages, written above by the workgroup, are visible
  const int t = row_info(cu_q, seq_lens, batch, total_q, max_seq_len, row).t;
  const int P = unit_size;
  int32_t *dst = expand + (int64_t)row * k * P;
  for (int j = tid; j < k * P; j += kRegThreads) {
    const int i = (int)fast_div((uint32_t)j, unit);
    const int pg = out[i];
    const int pos = pg * P + (j - i * P);
    dst[j] = (pg >= 0 && pos <= t) ? pos : -1;
  }
}

// Rows longer than one register block (32K): two phases on the same selection.
// Phase 1 selects the top-k of every chunk of a row (16K positions; 32K
// past 128K, where fewer survivors make the merge cheaper) (one
// 1024-thread workgroup per row and chunk) and writes the chunk's survivors,
// keys and positions, in ascending position order to slots [c k, c k + m_c)
// of the row's workspace, m_c = min(k, candidates of the chunk). Phase 2 (one
// workgroup per row) selects among the nc * k slots, slots past a chunk's m_c
// taking key 0 (below every score's key), so they are never kept. This is
// exact: a position in the row's top-k is also in its chunk's top-k under the
// same order, and slot order is position order among the survivors, so ties
// still go to the lower position.
constexpr int kSplitCands = 32 * kRegThreads;    // phase-2 slots: 1024 threads x 32 keys

// phase-1 chunk: 1024 threads x 16 (or 32) keys
int split_chunk(int32_t max_seq_len) {
  return max_seq_len > 128 * kRegThreads ? 32 * kRegThreads : 16 * kRegThreads;
}
int split_chunks(int32_t max_seq_len) {
  const int c = split_chunk(max_seq_len);
  return (max_seq_len + c - 1) / c;
}

bool split_path(int32_t max_seq_len, int32_t k) {
  return max_seq_len > 32 * kRegThreads && (int64_t)split_chunks(max_seq_len) * k <= kSplitCands;
}

template <int R>
__global__ __launch_bounds__(kRegThreads) __attribute__((amdgpu_waves_per_eu(8))) void topk_chunk_kernel(
    const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ cu_q, int batch,
    int total_q, int max_seq_len, int n_max, FastDiv unit, const float *__restrict__ scores,
    int64_t ld, int k, int nc,
    uint32_t *__restrict__ ws_key, int32_t *__restrict__ ws_pos) {
  constexpr int kSplitChunk = R * kRegThreads;
  __shared__ SelectShared<kRegThreads / kWave, R, 4, 2> sh;
  const int c = blockIdx.x, row = blockIdx.y;
  const int tid = threadIdx.x;
  const int base = c * kSplitChunk;
  const int lane = tid & 63;
  const int w0 = __builtin_amdgcn_readfirstlane(tid >> 6) * (kWave * R);
  const float *src = scores + (int64_t)row * ld + base + w0 + lane;
  const int lim = n_max - base - w0;
  float v[R];
#pragma unroll
  for (int u = 0; u < R; ++u) v[u] = lane < lim - u * kWave ? src[u * kWave] : 0.0f;
  select_clear(sh);
  const int n = row_cands(cu_q, seq_lens, batch, total_q, max_seq_len, row, unit);
  const int m = min(max(n - base, 0), kSplitChunk);  // candidates of this chunk
  uint32_t *okey = ws_key + ((int64_t)row * nc + c) * k;
  int32_t *opos = ws_pos + ((int64_t)row * nc + c) * k;
  uint32_t key[R];
#pragma unroll
  for (int u = 0; u < R; ++u) key[u] = order_key(v[u]);
  if (m <= k) {
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int i = sel_cand<R>(u);
      if (i < m) {
        okey[i] = key[u];
        opos[i] = base + i;
      }
    }
    return;
  }
  select_run(key, m, k, sh, [&](int u, int slot) {
    okey[slot] = key[u];
    opos[slot] = base + sel_cand<R>(u);
  });
}

template <int R>
__global__ __launch_bounds__(kRegThreads) void topk_split_merge_kernel(
    const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ cu_q, int batch,
    int total_q, int max_seq_len, int n_max, FastDiv unit, int k, FastDiv kdiv, int nc, int chunk,
    const uint32_t *__restrict__ ws_key,
    const int32_t *__restrict__ ws_pos, int32_t *__restrict__ indices) {
  __shared__ SelectShared<kRegThreads / kWave, R, 4, 2> sh;
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  select_clear(sh);
  const int n = row_cands(cu_q, seq_lens, batch, total_q, max_seq_len, row, unit);
  int32_t *out = indices + (int64_t)row * k;
  if (n <= k) {
    for (int i = tid; i < k; i += kRegThreads) out[i] = i < n ? i : -1;
    return;
  }
  const uint32_t *ikey = ws_key + (int64_t)row * nc * k;
  const int32_t *ipos = ws_pos + (int64_t)row * nc * k;
  uint32_t key[R];
  int32_t pos[R];
#pragma unroll
  for (int u = 0; u < R; ++u) {
    const int j = sel_cand<R>(u);
    const int c = (int)fast_div((uint32_t)j, kdiv);
    const int s = j - c * k;
    const int m = min(min(max(n - c * chunk, 0), chunk), k);  // survivors of chunk c
    const bool ok = j < nc * k && s < m;
    key[u] = ok ? ikey[j] : 0u;
    pos[u] = ok ? ipos[j] : -1;
  }
  select_run(key, nc * k, k, sh, [&](int u, int slot) { out[slot] = pos[u]; });
}

int chunks_of(int32_t max_seq_len) { return (max_seq_len + kChunk - 1) / kChunk; }

bool two_phase(int32_t max_seq_len) { return max_seq_len > kChunk; }

hipError_t set_lds(const void *fn, size_t bytes) {
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

}  // namespace

int candidate_bound(int32_t max_seq_len, int32_t unit) {
  return unit <= 1 ? max_seq_len : (int)(((int64_t)max_seq_len + unit - 1) / unit);
}

size_t topk_workspace_bytes(int32_t total_q, int32_t max_seq_len, int32_t k) {
  if (total_q < 1 || k < 1) return 0;
  const size_t per = (size_t)total_q * k * (sizeof(uint32_t) + sizeof(int32_t));
  if (split_path(max_seq_len, k)) return per * split_chunks(max_seq_len);
  if (!two_phase(max_seq_len)) return 0;
  return per * chunks_of(max_seq_len);
}

bool topk_supported(int32_t max_seq_len, int32_t k) {
  if (!two_phase(max_seq_len) || split_path(max_seq_len, k)) return true;
  const int nc = chunks_of(max_seq_len);
  return nc < 64 && (int64_t)nc * (k < kChunk ? k : kChunk) <= kChunk;
}

hipError_t launch_topk(const BatchArgs &bt, const float *scores, int64_t ld, int32_t k,
                       int32_t unit, int32_t *indices, void *workspace, size_t,
                       hipStream_t stream, int32_t *expand, bool *expanded) {
  if (expanded != nullptr) *expanded = false;
  if (bt.total_q == 0) return hipSuccess;
  // candidates of a row: positions (unit 1) or groups of `unit` positions
  const int n_max = candidate_bound(bt.max_seq_len, unit);
  const FastDiv fu = make_fast_div((uint32_t)unit);
  if (n_max <= 32 * kRegThreads) {
    // short rows (a page budget's candidates, small k) on 256 threads: a
    // smaller workgroup reaches the same selection with less barrier latency
    auto kernel = n_max <= 256                 ? topk_reg_kernel<256, 1>
                  : n_max <= 1024              ? topk_reg_kernel<256, 4>
                  : n_max <= 4 * kRegThreads   ? topk_reg_kernel<kRegThreads, 4>
                  : n_max <= 8 * kRegThreads   ? topk_reg_kernel<kRegThreads, 8>
                  : n_max <= 16 * kRegThreads  ? topk_reg_kernel<kRegThreads, 16>
                                               : topk_reg_kernel<kRegThreads, 32>;
    const int nt = n_max <= 1024 ? 256 : kRegThreads;
    hipLaunchKernelGGL(kernel, dim3(bt.total_q), dim3(nt), 0, stream, bt.seq_lens,
                       bt.cu_q, bt.batch, bt.total_q, bt.max_seq_len, n_max, fu, scores, ld, k,
                       indices, expand, unit);
    if (expanded != nullptr) *expanded = expand != nullptr;
    return hipGetLastError();
  }
  hipError_t e;
  if (split_path(n_max, k)) {
    const int nc = split_chunks(n_max);
    if (bt.total_q > 65535) return hipErrorInvalidConfiguration;
    uint32_t *ws_key = static_cast<uint32_t *>(workspace);
    int32_t *ws_pos = reinterpret_cast<int32_t *>(ws_key + (size_t)bt.total_q * nc * k);
    const int chunk = split_chunk(n_max);
    auto ck = chunk == 32 * kRegThreads ? topk_chunk_kernel<32> : topk_chunk_kernel<16>;
    hipLaunchKernelGGL(ck, dim3(nc, bt.total_q), dim3(kRegThreads), 0, stream,
                       bt.seq_lens, bt.cu_q, bt.batch, bt.total_q, bt.max_seq_len, n_max, fu,
                       scores, ld, k, nc, ws_key, ws_pos);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t cands = (int64_t)nc * k;
    auto merge = cands <= 8 * kRegThreads    ? topk_split_merge_kernel<8>
                 : cands <= 16 * kRegThreads ? topk_split_merge_kernel<16>
                                             : topk_split_merge_kernel<32>;
    hipLaunchKernelGGL(merge, dim3(bt.total_q), dim3(kRegThreads), 0, stream, bt.seq_lens,
                       bt.cu_q, bt.batch, bt.total_q, bt.max_seq_len, n_max, fu, k,
                       make_fast_div((uint32_t)k), nc, chunk, ws_key, ws_pos, indices);
    return hipGetLastError();
  }
  const size_t lds = (size_t)kChunk * sizeof(uint32_t);
  if (!two_phase(n_max)) {
    if ((e = set_lds((const void *)topk_rows_kernel<false>, lds)) != hipSuccess) return e;
    hipLaunchKernelGGL(topk_rows_kernel<false>, dim3(bt.total_q), dim3(kTopkThreads), lds, stream,
                       bt.seq_lens, bt.cu_q, bt.batch, bt.total_q, bt.max_seq_len, n_max, fu,
                       scores, ld, k, indices, 1, nullptr, nullptr);
    return hipGetLastError();
  }
  const int nc = chunks_of(n_max);
  uint32_t *ws_key = static_cast<uint32_t *>(workspace);
  int32_t *ws_pos = reinterpret_cast<int32_t *>(ws_key + (size_t)bt.total_q * nc * k);
  if ((e = set_lds((const void *)topk_rows_kernel<true>, lds)) != hipSuccess) return e;
  if ((e = set_lds((const void *)topk_merge_kernel, lds)) != hipSuccess) return e;
  hipLaunchKernelGGL(topk_rows_kernel<true>, dim3(bt.total_q * nc), dim3(kTopkThreads), lds,
                     stream, bt.seq_lens, bt.cu_q, bt.batch, bt.total_q, bt.max_seq_len, n_max,
                     fu, scores, ld, k, indices, nc, ws_key, ws_pos);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(topk_merge_kernel, dim3(bt.total_q), dim3(kTopkThreads), lds, stream,
                     bt.seq_lens, bt.cu_q, bt.batch, bt.total_q, bt.max_seq_len, n_max, fu, k, nc,
                     ws_key, ws_pos, indices);
  return hipGetLastError();
}

}  // namespace dsa
