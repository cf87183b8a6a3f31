// Absorbed sparse MLA attention over the selected cache rows on gfx950
// ("vLLM Inference Path: GLM-5.2 as an Example", sections "MLA Projections and
// KV State" and "Sparse MLA Attention"; "Making GLM-5.2 Sparse on TPUs",
// section "Separate the indexer from the attention it controls": the cache
// row is a 512-d latent plus a 64-d RoPE key, the key projection is absorbed
// into the 576-d query and the value is the latent itself).
//
// MFMA path (bf16, 64 heads, 512 + 64): one 256-thread workgroup (4 waves,
// one per SIMD) owns one query row and one contiguous slice ("split") of its
// k index slots, walked in tiles of 32 selected rows. Wave w owns heads
// 16w..16w+15 for the whole slice: their logits, online softmax and the full
// 16 x 512 output, so the waves share nothing but the row tiles.
//  * All selected positions of the split are translated to physical rows once,
//    up front, into an LDS table (invalid slots point at a valid row of the
//    sequence and are masked), with a validity bitmask per tile.
//  * Gather: each tile is copied by direct global-to-LDS loads, three tiles
//    ahead of the one being computed (four LDS stages, one barrier per tile).
//    Wave w moves rows 8w..8w+7: 8 x 1152 bytes are exactly nine 64-lane
//    16-byte instructions. Rows are stored unpadded, their 16-byte chunks
//    XOR-permuted by the row's low bits so that both operand read patterns
//    below hit distinct banks.
//  * Logits, transposed: S^T = C Q^T on v_mfma_f32_16x16x32_bf16 with tile rows
//    on M (A operand from LDS) and the wave's 16 heads on N (the query block
//    stays in registers for the whole slice). Each lane then holds one head's
//    logits for 8 rows: the softmax maximum and sum are in-lane, plus two
//    permlane swaps for the tile maximum across the four lane groups.
//  * The probabilities of a lane are already the A operand of the PV product
//    (head on M, the 8 rows as its k-slots), split as p = hi + lo in bf16 (two
//    MFMAs per value operand) so that rounding p costs no accuracy; the value
//    operand needs 8 rows of one dim per lane, which ds_read_b64_tr_b16
//    delivers from the row-major tile, two reads per operand.
//  * Softmax in base 2 with the scale folded into one multiply-add, against a
//    reference maximum per head fixed by its first valid tile. Later logits
//    may exceed it by up to kHeadroom (p <= 2^kHeadroom keeps every sum
//    finite); a tile beyond that restarts the split with a higher reference.
//    The accumulated output is thus only ever written by MFMAs in the loop.
//  * Workgroups are numbered so that all splits of a row land on the same XCD
//    (workgroups are dispatched round-robin over the 8 XCDs), so the row's
//    query block is fetched from HBM once and then served by that XCD's L2.
//  * Splits of a row are merged by a log-sum-exp combine kernel.
#include <mutex>
#include <type_traits>

#include "dsa_device.h"
#include "dsa_internal.h"
#include "dsa_select.h"

// Library-owned workspace of dsa_sparse_mla_fwd_noalloc, for callers that
// cannot allocate: the split partials of one call, at most
// DSA_MLA_NOALLOC_SCRATCH_BYTES. Every GPU that loads this code holds its own
// copy (zero-filled at load) until the process ends. In host code `scratch`
// names a host-side stand-in, never a device address: the device address of
// each GPU's copy comes from hipGetSymbolAddress (dsa::mla_scratch below).
static __device__ __align__(256) uint8_t scratch[DSA_MLA_NOALLOC_SCRATCH_BYTES];

namespace dsa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

constexpr int kH = 64;
constexpr int kDL = 512;
constexpr int kDR = 64;
constexpr int kD = kDL + kDR;               // 576
constexpr int kRowBytes = kD * 2;           // 1152
constexpr int kTileN = 32;
constexpr int kTileBytes = kTileN * kRowBytes;
constexpr int kMlaThreads = 256;
constexpr int kMlaWaves = kMlaThreads / kWave;
constexpr int kStages = 4;                  // LDS row tiles: one computed, three landing
constexpr int kSteps = kD / 32;             // 18 MFMA k-steps for the logits
constexpr int kGatherInsts = kTileBytes / kMlaWaves / (kWave * 16);  // 9 per wave per tile
constexpr int kMinRowsPerSplit = 128;
constexpr int kXcds = 8;
constexpr int kMaxRowsPerSplit = 2048;
constexpr int kMaxSplits = 64;
constexpr float kHeadroom = 64.0f;  // log2 headroom of p above 1 before a restart
constexpr uint32_t kInvalid = 0x80000000u;  // row-table flag: slot masked

static_assert(kGatherInsts * kWave * 16 * kMlaWaves == kTileBytes, "gather covers a tile");

// Tile row held by lane x of M-tile m of the logits product: the even rows of
// the 16-row half, then the odd ones. Each 32-lane half of a transposed value
// read then touches rows of one parity, whose chunks fill all 64 banks.
__device__ __forceinline__ int tile_row(int m, int x) { return 16 * m + 2 * (x & 7) + (x >> 3); }

// Chunk c (16 bytes) of tile row r is stored at chunk chunk_swz(c, r) of the
// row; the map is its own inverse. Latent chunks are XOR-ed with the row's low
// 4 bits, the 8 RoPE chunks with bits 1..3 (within 64..71).
__device__ __forceinline__ int chunk_swz(int c, int r) {
  return c < 64 ? (c ^ (r & 15)) : (64 + ((c - 64) ^ ((r >> 1) & 7)));
}

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short __attribute__((address_space(3))) *lds_i16_ptr;

// Lane i of each 16-lane group receives column i of the 4 x 16 block of
// 16-bit values whose row e is supplied (4 values each) by lanes 4e..4e+3.
__device__ __forceinline__ uint2 lds_read_tr16(const __attribute__((address_space(3))) void *p) {
  const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4_t *)(const_cast<__attribute__((address_space(3))) void *>(p)));
  return __builtin_bit_cast(uint2, v);
}

// Direct global-to-LDS copy of one wave's eight rows of a tile: nine 16-byte
// loads per lane, instruction n landing at lds + 1024 n + 16 lane (lds
// wave-uniform). The loads go out in groups of four sharing one m0 value
// (lds, lds + 4096, lds + 8192); the rest of the 1024 n step comes from the
// instruction offset, which moves the LDS and the global address alike, so
// the caller's address for instruction n is 1024 (n % 4) below its source.
// Issued as inline assembly so the compiler's automatic waits ignore the
// copies: their completion is awaited only by the explicit vmcnt waits before
// the tile barriers (the compiler's per-buffer tracking of such copies does
// not survive the tile loop's back edge, and would stall every tile on the
// copies three tiles ahead). m0 is reserved to the compiler and restored; one
// wait state separates each m0 write from the copies that read it.
// Addresses as 32-bit offsets from a scalar base (pools below 4 GiB) ...
__device__ __forceinline__ void lds_copy9(const uint8_t *base, const uint32_t (&v)[9], uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %10\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %11\n\t"
      "global_load_lds_dwordx4 %2, %11 offset:1024\n\t"
      "global_load_lds_dwordx4 %3, %11 offset:2048\n\t"
      "global_load_lds_dwordx4 %4, %11 offset:3072\n\t"
      "s_add_u32 m0, %10, 0x1000\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %5, %11\n\t"
      "global_load_lds_dwordx4 %6, %11 offset:1024\n\t"
      "global_load_lds_dwordx4 %7, %11 offset:2048\n\t"
      "global_load_lds_dwordx4 %8, %11 offset:3072\n\t"
      "s_add_u32 m0, %10, 0x2000\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %9, %11\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]),
        "v"(v[8]), "s"(lds), "s"(base)
      : "memory", "scc");
}

// ... or as full 64-bit addresses (any pool size).
__device__ __forceinline__ void lds_copy9(const uint64_t (&v)[9], uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %10\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "global_load_lds_dwordx4 %2, off offset:1024\n\t"
      "global_load_lds_dwordx4 %3, off offset:2048\n\t"
      "global_load_lds_dwordx4 %4, off offset:3072\n\t"
      "s_add_u32 m0, %10, 0x1000\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %5, off\n\t"
      "global_load_lds_dwordx4 %6, off offset:1024\n\t"
      "global_load_lds_dwordx4 %7, off offset:2048\n\t"
      "global_load_lds_dwordx4 %8, off offset:3072\n\t"
      "s_add_u32 m0, %10, 0x2000\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %9, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]),
        "v"(v[8]), "s"(lds)
      : "memory", "scc");
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// Maximum over the four 16-lane groups (lanes with equal lane % 16).
__device__ __forceinline__ float group4_max(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

__device__ __forceinline__ float group4_sum(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// Per-layer pointers of one launch (kernel argument, indexed by the block's
// layer). Layers share the batch, the block table and the index list.
struct MlaLayerArgs {
  const uint16_t *q[kMlaMaxLayers];
  const uint8_t *kv[kMlaMaxLayers];
  int64_t num_pages[kMlaMaxLayers];
  float *out[kMlaMaxLayers];
  float *lse[kMlaMaxLayers];
};

// Direct copies of a wave's eight rows of a row tile into an LDS stage.
// Instruction n of wave wv moves chunks 64n..64n+63 of the 576 chunks of rows
// 8wv..8wv+7; lane l's chunk is row 8wv + (64n+l)/72, stored chunk
// (64n+l)%72, fetched from that row's chunk chunk_swz(., row). The row is one
// of two known to the instruction: 64n/72, or the next from lane
// 72(64n/72 + 1) - 64n on. goff[n] holds the chunk's byte offset in its row,
// less the 1024 (n % 4) that the copy's instruction offset adds back (plus
// 3072 on the 32-bit path, whose base sits 3072 bytes below the cache so that
// every offset stays non-negative). Row ids carry kInvalid as a flag, which
// the copy strips (a flagged slot's row is a valid stand-in).
template <bool kOff32>
struct TileGather {
  static constexpr uint32_t kBias = kOff32 ? 3072u : 0u;
  uint32_t goff[kGatherInsts];
  const uint8_t *kv;
  uint32_t lds_wave;  // this wave's part of stage 0
  int lane;

  __device__ __forceinline__ TileGather(const uint8_t *kv_, uint32_t lds_tiles, int wv, int lane_)
      : kv(kv_), lds_wave(lds_tiles + 8 * wv * kRowBytes), lane(lane_) {
#pragma unroll
    for (int n = 0; n < kGatherInsts; ++n) {
      const int qc = 64 * n + lane;
      const int rl = qc / 72, lc = qc % 72;
      goff[n] = (uint32_t)(16 * chunk_swz(lc, 8 * wv + rl)) + kBias - 1024u * (n % 4);
    }
  }

  __device__ __forceinline__ void copy(int stage, const u32x4_t ra, const u32x4_t rb) const {
    const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_wave + (uint32_t)stage * kTileBytes);
    const uint32_t rid[8] = {ra.x & ~kInvalid, ra.y & ~kInvalid, ra.z & ~kInvalid, ra.w & ~kInvalid,
                             rb.x & ~kInvalid, rb.y & ~kInvalid, rb.z & ~kInvalid, rb.w & ~kInvalid};
    if constexpr (kOff32) {
      uint32_t v[kGatherInsts];
#pragma unroll
      for (int n = 0; n < kGatherInsts; ++n) {
        const int q0 = (64 * n) / 72;
        const int split_lane = 72 * (q0 + 1) - 64 * n;
        const uint32_t r = (q0 == 7 || lane < split_lane) ? rid[q0] : rid[q0 + 1];
        v[n] = __umul24(r, (uint32_t)kRowBytes) + goff[n];
      }
      lds_copy9(kv - kBias, v, lds);
    } else {
      uint64_t v[kGatherInsts];
#pragma unroll
      for (int n = 0; n < kGatherInsts; ++n) {
        const int q0 = (64 * n) / 72;
        const int split_lane = 72 * (q0 + 1) - 64 * n;
        const uint32_t r = (q0 == 7 || lane < split_lane) ? rid[q0] : rid[q0 + 1];
        v[n] = (uint64_t)((int64_t)(uintptr_t)kv + (int64_t)r * kRowBytes + (int32_t)goff[n]);
      }
      lds_copy9(v, lds);
    }
  }
};

// Per-lane operand offsets inside a row tile (loop-invariant), for lane
// (g, j) of a wave: logits A operand: lane (g, i) reads tile row
// tile_row(0, i), chunk 4s + g (M-tile 1 is 16 rows further with the same
// permutation); latent steps s use a_lat[s & 3] plus 256 (s >> 2), the two
// RoPE steps a_rope[s - 16]. Value operand: transposed read L covers rows
// tile_row(L, 4g + j / 4), dims 4(j & 3) .. +4 of the 16-dim tile nt, which
// uses v_off[nt & 7] plus 256 (nt >> 3); read L = 1 is 16 rows further.
// lrow[m][r]: the tile row of this lane's logit (m, r), tile_row(m, 4g + r).
struct TileLane {
  uint32_t a_lat[4], a_rope[2];
  uint32_t v_off[8];
  int lrow[2][4];
};

__device__ __forceinline__ TileLane tile_lane(int g, int j) {
  TileLane tl;
  const int ar = tile_row(0, j);
#pragma unroll
  for (int s = 0; s < 4; ++s) tl.a_lat[s] = ar * kRowBytes + 16 * chunk_swz(4 * s + g, ar);
#pragma unroll
  for (int s = 0; s < 2; ++s) tl.a_rope[s] = ar * kRowBytes + 16 * chunk_swz(64 + 4 * s + g, ar);
  const int vr = tile_row(0, 4 * g + (j >> 2));
#pragma unroll
  for (int c = 0; c < 8; ++c)
    tl.v_off[c] = vr * kRowBytes + 16 * ((2 * c + ((j & 3) >> 1)) ^ (vr & 15)) + 8 * (j & 1);
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int r = 0; r < 4; ++r) tl.lrow[m][r] = tile_row(m, 4 * g + r);
  return tl;
}

// One 32-row tile of the attention for the calling wave's 16 columns (a
// column is one (query, head) pair; its query block is the B operand qf):
// logits, softmax against the running reference, and PV into o. Bit r of
// vmask (per lane: the tile's valid rows for this lane's column) masks tile
// row r. The wave's restart flag is written to *over_flag.
__device__ __forceinline__ void mla_tile(const lds_u8 *tb, uint32_t vmask, const TileLane &tl,
                                         const u32x4_t (&qf)[kSteps], f32x4_t (&o)[32],
                                         float &m_run, float &l_run, bool &overflow,
                                         float scale_log2, int *over_flag) {
  // logits (transposed): acc[m][r] = S[column j][row lrow[m][r]], A
  // operands read one k-step ahead of the MFMAs
  f32x4_t acc[2] = {f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}};
  auto a_off = [&](int s_) -> uint32_t {
    return s_ < 16 ? tl.a_lat[s_ & 3] + 256 * (s_ >> 2) : tl.a_rope[s_ - 16];
  };
  // A operands run kAhead k-steps ahead of their MFMAs
  constexpr int kAhead = 4;
  u32x4_t abuf[kSteps][2];
#pragma unroll
  for (int s_ = 0; s_ < kAhead; ++s_)
#pragma unroll
    for (int m = 0; m < 2; ++m)
      abuf[s_][m] = *(const __attribute__((address_space(3))) u32x4_t *)(tb + a_off(s_) + m * 16 * kRowBytes);
#pragma unroll
  for (int s_ = 0; s_ < kSteps; ++s_) {
    if (s_ + kAhead < kSteps) {
#pragma unroll
      for (int m = 0; m < 2; ++m)
        abuf[s_ + kAhead][m] = *(const __attribute__((address_space(3))) u32x4_t *)(
            tb + a_off(s_ + kAhead) + m * 16 * kRowBytes);
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) acc[m] = mfma_16x16x32_bf16(abuf[s_][m], qf[s_], acc[m]);
  }
  // issue order: 2 * kAhead operand reads, then one read per MFMA
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * kAhead, 0);
#pragma unroll
  for (int i = 0; i < 2 * (kSteps - kAhead); ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 2 * kAhead, 0);

  // Value operands (transposed reads, two per 16-dim tile nt) run kVAhead
  // tiles ahead of their MFMAs; the first kVAhead go out before the softmax
  // so their latency hides under it.
  auto vread = [&](int nt) -> u32x4_t {
    const lds_u8 *vp = tb + tl.v_off[nt & 7] + 256 * (nt >> 3);
    const uint2 v0 = lds_read_tr16(vp);
    const uint2 v1 = lds_read_tr16(vp + 16 * kRowBytes);
    return u32x4_t{v0.x, v0.y, v1.x, v1.y};
  };
  constexpr int kVAhead = 6;
  u32x4_t vbuf[32];
#pragma unroll
  for (int nt = 0; nt < kVAhead; ++nt) vbuf[nt] = vread(nt);
  __builtin_amdgcn_sched_barrier(0);
  if (vmask != 0xFFFFFFFFu) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (!((vmask >> tl.lrow[m][r]) & 1u)) acc[m][r] = -INFINITY;
  }
  // softmax of column j in base 2 against a reference maximum m_run
  // fixed by the head's first valid tile: p = 2^(x - m_run). A later tile
  // may exceed it by up to kHeadroom (p <= 2^kHeadroom keeps every sum
  // finite); beyond that the whole split restarts with a higher reference,
  // so the accumulated output is never rescaled in the loop.
  float mx = fmaxf(fmaxf(fmaxf(acc[0][0], acc[0][1]), fmaxf(acc[0][2], acc[0][3])),
                   fmaxf(fmaxf(acc[1][0], acc[1][1]), fmaxf(acc[1][2], acc[1][3])));
  mx = group4_max(mx) * scale_log2;
  m_run = m_run == -INFINITY ? mx : m_run;
  const bool over = mx > m_run + kHeadroom;
  m_run = over ? mx : m_run;  // per lane: a restarted pass starts from here
  overflow |= over;
  // every lane writes the same word, so no branch splits the tile's code;
  // the flag is read by all waves after the next barrier (a restarted
  // split discards whatever this tile accumulates)
  *over_flag = __ballot(overflow) != 0ull ? 1 : 0;
  // until the head's first valid row every logit is -inf: subtract 0, not -inf
  const float m_sub = m_run == -INFINITY ? 0.0f : m_run;
  float p[2][4];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[m][r] = fast_exp2(fmaf(acc[m][r], scale_log2, -m_sub));
      l_run += p[m][r];
    }
  // P as the A operand of PV: head j, k-slots 8g + 4m + r <-> rows lrow[m][r].
  // p = hi + lo in bf16 to 2^-16 relative: bf16 rounding of p alone (2^-9)
  // is too coarse for rows that attend to only a few positions.
  u32x4_t pa, pl;
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t hi = pack_bf16x2(p[m][2 * h], p[m][2 * h + 1]);
      const float r0 = p[m][2 * h] - __uint_as_float(hi << 16);
      const float r1 = p[m][2 * h + 1] - __uint_as_float(hi & 0xFFFF0000u);
      pa[2 * m + h] = hi;
      pl[2 * m + h] = pack_bf16x2(r0, r1);
    }
  // PV in a fixed order: each pair of MFMAs is preceded by the reads of
  // the tile kVAhead further on. (Left to itself the scheduler sinks every
  // read to just before its MFMAs, which exposes the whole LDS latency once
  // per pair.)
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int nt = 0; nt < 32; ++nt) {
    if (nt + kVAhead < 32) vbuf[nt + kVAhead] = vread(nt + kVAhead);
    o[nt] = mfma_16x16x32_bf16(pa, vbuf[nt], o[nt]);
    o[nt] = mfma_16x16x32_bf16(pl, vbuf[nt], o[nt]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// kFull: the query has all 64 heads (no zero columns, constant row stride).
template <bool kOff32, bool kFull>
__global__ __launch_bounds__(kMlaThreads, 1) void sparse_mla_bf16_kernel(
    const int32_t *__restrict__ block_table, const int32_t *__restrict__ seq_lens,
    const int32_t *__restrict__ cu_q, int batch, int total_q, int max_seq_len, int64_t bt_stride,
    const MlaLayerArgs layers, int blocks_per_layer, int page_size, FastDiv pdiv,
    const int32_t *__restrict__ indices, int k, int n_splits, int rows_per_split,
    float scale_log2, float *__restrict__ ws_acc, float *__restrict__ ws_ml, int n_heads) {
  // ring of row tiles: tile i lives in stage i % kStages
  __shared__ __attribute__((aligned(1024))) uint8_t s_tiles[kStages * kTileBytes];
  __shared__ __attribute__((aligned(16))) uint32_t s_rowid[kMaxRowsPerSplit + kTileN];
  __shared__ uint32_t s_vmask[kMaxRowsPerSplit / kTileN + 1];
  __shared__ float s_ml[kH][2];
  __shared__ int s_over[kMlaWaves];

  // Layers take consecutive ranges of blocks, so one layer's tail overlaps
  // the next one's start. Within a layer, XCD-aware numbering: block id =
  // ((row / 8) * n_splits + split) * 8 + row % 8 (blocks_per_layer is a
  // multiple of 8, so the XCD of a block is its row % 8 in every layer).
  const int layer = (int)(blockIdx.x / (unsigned)blocks_per_layer);
  const int bid = (int)blockIdx.x - layer * blocks_per_layer;
  const int xcd = bid % kXcds;
  const int rest = bid / kXcds;
  const int split = rest % n_splits;
  const int row = (rest / n_splits) * kXcds + xcd;
  if (row >= total_q) return;
  const uint16_t *__restrict__ q = layers.q[layer];
  const uint8_t *__restrict__ kv = layers.kv[layer];
  const int64_t num_pages = layers.num_pages[layer];
  float *__restrict__ out = layers.out[layer];
  float *__restrict__ lse = layers.lse[layer];
  if (n_splits > 1) {
    ws_acc += (int64_t)layer * total_q * n_splits * kH * kDL;
    ws_ml += (int64_t)layer * total_q * n_splits * kH * 2;
  }

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 4, j = lane & 15;

  const int slot_begin = split * rows_per_split;
  const int slot_end = min(k, slot_begin + rows_per_split);
  const int nrows = max(0, slot_end - slot_begin);
  const int ntiles = (nrows + kTileN - 1) / kTileN;
  const int32_t *idx_row = indices + (int64_t)row * k + slot_begin;

  // The query block of heads 16wv..16wv+15, the B operand of the logits:
  // lane (g, j) holds head 16wv + j, dims 32s + 8g .. +8. The first split of
  // a row loads it at once, beside the row table's round trips; the other
  // splits (same XCD) load it once their table is built, from the L2 that
  // the first one filled, so the row's HBM reads of it are not repeated.
  // With fewer than 64 heads the missing heads' queries are zero (nothing is
  // loaded for them) and their outputs are not written.
  u32x4_t qf[kSteps];
  const int nh = kFull ? kH : n_heads;
  const bool q_head = kFull || 16 * wv + j < nh;
  const uint16_t *qp = q + ((int64_t)row * nh + (q_head ? 16 * wv + j : 0)) * kD + 8 * g;
  const bool q_first = split == 0;
  if (q_first) {
#pragma unroll
    for (int s = 0; s < kSteps; ++s) qf[s] = q_head ? ldg16(qp + 32 * s) : u32x4_t{0u, 0u, 0u, 0u};
  }

  // Row table, first round trip: the selected positions of this thread's
  // entries (entry e covers slot kMlaThreads e + tid of the split), and in
  // parallel the row's sequence and causal position. Every lane loads from
  // an address inside the split (slots past it read its last entry; the
  // table below drops them), so the loads need no branch: a load under a
  // lane mask ends in a wait for all loads before the next one, which would
  // serialize them. Nothing uses the values before the row's metadata
  // arrives, so both land in one round trip.
  constexpr int kEntries = kMaxRowsPerSplit / kMlaThreads;
  int pos[kEntries];
#pragma unroll
  for (int e = 0; e < kEntries; ++e) pos[e] = -1;
  if (nrows > 0) {
#pragma unroll
    for (int e = 0; e < kEntries; ++e) {
      const int i = e * kMlaThreads + tid;
      pos[e] = idx_row[min(i, nrows - 1)];
    }
  }
  const RowInfo ri = row_info(cu_q, seq_lens, batch, total_q, max_seq_len, row);
  const int b = ri.b, t = ri.t;

  // Second round trip: the page of every entry (positions clamped into
  // [0, t] so the reads stay inside the row's table whatever a slot holds;
  // slots outside it are masked below) and the page of position 0 (the
  // stand-in row of masked slots); again without a branch per load.
  int page[kEntries];
  int page0 = 0;
  if (t >= 0) {
    const int32_t *bt_row = block_table + (int64_t)b * bt_stride;
#pragma unroll
    for (int e = 0; e < kEntries; ++e) {
      const int p = min(max(pos[e], 0), t);
      page[e] = bt_row[fast_div((uint32_t)p, pdiv)];
    }
    page0 = bt_row[0];
  }
  auto clamp_page = [&](int64_t pg) -> uint32_t { return (uint32_t)dsa::clamp_page(pg, num_pages); };
  const uint32_t safe_row = clamp_page(page0) * (uint32_t)page_size;
#pragma unroll
  for (int e = 0; e < kEntries; ++e) {
    const int i = e * kMlaThreads + tid;
    if (e * kMlaThreads >= ntiles * kTileN) break;
    const int p = pos[e];
    const bool valid = i < nrows && p >= 0 && p <= t;
    const uint32_t pq = fast_div((uint32_t)max(p, 0), pdiv);
    const uint32_t rid =
        valid ? clamp_page(page[e]) * (uint32_t)page_size + ((uint32_t)p - pq * (uint32_t)page_size)
              : safe_row;
    if (i < ntiles * kTileN) s_rowid[i] = valid ? rid : (rid | kInvalid);
    const uint64_t vb = __ballot(valid && i < ntiles * kTileN);
    if (lane == 0 && i < ntiles * kTileN) {
      s_vmask[i / kTileN] = (uint32_t)vb;
      if (i + kTileN < ntiles * kTileN) s_vmask[i / kTileN + 1] = (uint32_t)(vb >> 32);
    }
  }

  const lds_u8 *tiles = (const lds_u8 *)s_tiles;
  const uint32_t lds_tiles = (uint32_t)(uintptr_t)tiles;
  const TileGather<kOff32> tg(kv, lds_tiles, wv, lane);
  // row ids of this wave's eight rows of a tile (read one tile ahead of the
  // copy that needs them, so the copy never waits on this LDS read)
  auto rowids = [&](int tile, u32x4_t &ra, u32x4_t &rb) {
    ra = *reinterpret_cast<const u32x4_t *>(s_rowid + tile * kTileN + 8 * wv);
    rb = *reinterpret_cast<const u32x4_t *>(s_rowid + tile * kTileN + 8 * wv + 4);
  };
  auto gather = [&](int tile, const u32x4_t ra, const u32x4_t rb) {
    tg.copy(tile & (kStages - 1), ra, rb);
  };

  const TileLane tl = tile_lane(g, j);
  f32x4_t o[32];
#pragma unroll
  for (int nt = 0; nt < 32; ++nt) o[nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -INFINITY, l_run = 0.0f;  // head 16wv + j; l_run covers this lane's rows
  bool overflow = false;

  if (!q_first) {
#pragma unroll
    for (int s = 0; s < kSteps; ++s) qf[s] = q_head ? ldg16(qp + 32 * s) : u32x4_t{0u, 0u, 0u, 0u};
  }
  if (tid < kMlaWaves) s_over[tid] = 0;
  // every compiler-visible load (query block, row table) has landed before the
  // first direct copies, which the compiler does not count (a load of its own
  // still in flight would make it wait for all of them inside the tile loop)
  __builtin_amdgcn_s_waitcnt(0x0070);
  __syncthreads();  // row table visible

  u32x4_t ra_n, rb_n;  // row ids of the next tile to copy
  auto step = [&](int tile) {
    // this wave's loads of `tile` have landed (later tiles may be in flight)
    const int ahead = min(ntiles - 1 - tile, kStages - 2);
    // (s_waitcnt fields: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8;
    // lgkmcnt 0 also completes this wave's LDS stores, e.g. the restart flag)
    if (ahead >= 2) __builtin_amdgcn_s_waitcnt(0x0070 | ((2 * kGatherInsts) & 15) | (((2 * kGatherInsts) >> 4) << 14));
    else if (ahead == 1) __builtin_amdgcn_s_waitcnt(0x0070 | (kGatherInsts & 15) | ((kGatherInsts >> 4) << 14));
    else __builtin_amdgcn_s_waitcnt(0x0070);
    // Barrier with no release fence: the wait above already covers this
    // wave's part of `tile`, and a release fence would also wait for the
    // later tiles' loads. Every wave's part of `tile` is visible after it, and
    // every wave is done with the stage of tile - 1.
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    if (tile + kStages - 1 < ntiles) gather(tile + kStages - 1, ra_n, rb_n);
    rowids(min(tile + kStages, ntiles - 1), ra_n, rb_n);

    // (a fully masked tile is computed like any other: its logits are all
    // -inf and add nothing)
    mla_tile(tiles + (tile & (kStages - 1)) * kTileBytes, s_vmask[tile], tl, qf, o, m_run, l_run,
             overflow, scale_log2, s_over + wv);
  };

  // Passes over the split: normally one. A pass in which some tile
  // overflowed runs to its end (its sums stay finite: the reference is raised
  // before the overflowing tile's probabilities are taken, and every earlier
  // one is at most 2^kHeadroom), then the split is walked again from the
  // raised references. Not leaving the tile loop early keeps the
  // accumulators in the registers the MFMAs write.
  auto first_gathers = [&]() {
    for (int tile = 0; tile < min(ntiles, kStages - 1); ++tile) {
      rowids(tile, ra_n, rb_n);
      gather(tile, ra_n, rb_n);
    }
    rowids(max(min(kStages - 1, ntiles - 1), 0), ra_n, rb_n);
  };
  first_gathers();
  for (;;) {
    for (int tile = 0; tile < ntiles; ++tile) step(tile);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // no direct load of this pass in flight
    __syncthreads();
    if ((s_over[0] | s_over[1] | s_over[2] | s_over[3]) == 0) break;
    __syncthreads();  // every wave has read the flags
    if (tid < kMlaWaves) s_over[tid] = 0;
#pragma unroll
    for (int nt = 0; nt < 32; ++nt) o[nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    l_run = 0.0f;
    overflow = false;
    __syncthreads();
    first_gathers();
  }

  // (m, l) of head 16wv + j: every lane group holds the same m; l is summed
  // over the groups' rows. O rows of lane (g, j) are heads 16wv + 4g + r.
  const float l_tot = group4_sum(l_run);
  if (g == 0) {
    s_ml[16 * wv + j][0] = m_run;
    s_ml[16 * wv + j][1] = l_tot;
  }
  __syncthreads();
  if (n_splits == 1) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int head = 16 * wv + 4 * g + r;
      if (!kFull && head >= nh) continue;
      const float l = s_ml[head][1];
      const float inv = l > 0.0f ? 1.0f / l : 0.0f;
      float *op = out + ((int64_t)row * nh + head) * kDL + j;
#pragma unroll
      for (int nt = 0; nt < 32; ++nt) op[16 * nt] = o[nt][r] * inv;
    }
    if (lse != nullptr && tid < nh) {
      const float m = s_ml[tid][0], l = s_ml[tid][1];
      lse[(int64_t)row * nh + tid] = l > 0.0f ? m * kLn2 + logf(l) : -INFINITY;
    }
  } else {
    // the split's accumulators in register order: value (nt, r) of lane l
    // of wave wv at float4 (wv * 32 + nt) * 64 + l, so that every store
    // instruction writes 1 KB of whole cache lines
    const int64_t part = (int64_t)row * n_splits + split;
    f32x4_t *op = reinterpret_cast<f32x4_t *>(ws_acc + part * kH * kDL) + wv * 32 * kWave + lane;
#pragma unroll
    for (int nt = 0; nt < 32; ++nt) op[nt * kWave] = o[nt];
    if (tid < kH) {
      ws_ml[(part * kH + tid) * 2 + 0] = s_ml[tid][0];
      ws_ml[(part * kH + tid) * 2 + 1] = s_ml[tid][1];
    }
  }
}

// Merge the splits of one row. The accumulators of a split are stored in the
// main kernel's register order: float4 f = (wv * 32 + nt) * 64 + 16 g + j
// holds heads 16 wv + 4 g + (0..3) at dim 16 nt + j. Thread (row, f) with
// nt < 16 reads float4 f and f + 1024 (dim tile nt + 16, same heads) of every
// split, whole lines, with the (m, l) pairs of its four heads, and merges:
// O = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s, lse = M ln 2 +
// ln(sum ...). Splits are taken eight at a time with every load of the eight
// issued before any is used; the running sums move to each chunk's maximum.
constexpr int kCombineThreads = 256;
constexpr int kCombineBlocksPerRow = kH * kDL / 8 / kCombineThreads;  // 16

template <bool kFull>
__global__ __launch_bounds__(kCombineThreads) void mla_combine_kernel(
    int total_q, int n_splits, const float *__restrict__ ws_acc, const float *__restrict__ ws_ml,
    const MlaLayerArgs layers, int n_heads) {
  constexpr int kU = 8;
  const int per_layer = total_q * kCombineBlocksPerRow;
  const int layer = (int)(blockIdx.x / (unsigned)per_layer);
  const int lb = (int)blockIdx.x - layer * per_layer;
  const int row = lb / kCombineBlocksPerRow;
  const int i = (lb % kCombineBlocksPerRow) * kCombineThreads + threadIdx.x;  // < 4096
  float *__restrict__ out = layers.out[layer];
  float *__restrict__ lse = layers.lse[layer];
  ws_acc += (int64_t)layer * total_q * n_splits * kH * kDL;
  ws_ml += (int64_t)layer * total_q * n_splits * kH * 2;
  const int wv = i >> 10, nt = (i >> 6) & 15, l = i & 63;
  const int head0 = 16 * wv + 4 * (l >> 4), dim = 16 * nt + (l & 15);
  const int64_t split_f4 = kH * kDL / 4;
  const f32x4_t *acc = reinterpret_cast<const f32x4_t *>(ws_acc) +
                       (int64_t)row * n_splits * split_f4 + (wv * 32 + nt) * kWave + l;
  const f32x4_t *ml = reinterpret_cast<const f32x4_t *>(ws_ml) +
                      ((int64_t)row * n_splits * kH + head0) / 2;  // + s * kH / 2
  float M[4], Lsum[4];
  f32x4_t a0 = {0.0f, 0.0f, 0.0f, 0.0f}, a1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    M[r] = -INFINITY;
    Lsum[r] = 0.0f;
  }
  for (int s0 = 0; s0 < n_splits; s0 += kU) {
    f32x4_t x0[kU], x1[kU], p0[kU], p1[kU];  // p0 = (m, l) of heads 0, 1; p1 of heads 2, 3
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const bool in = s0 + u < n_splits;
      const int64_t so = (int64_t)(s0 + u);
      x0[u] = in ? acc[so * split_f4] : f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      x1[u] = in ? acc[so * split_f4 + 16 * kWave] : f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      p0[u] = in ? ml[so * (kH / 2)] : f32x4_t{-INFINITY, 0.0f, -INFINITY, 0.0f};
      p1[u] = in ? ml[so * (kH / 2) + 1] : f32x4_t{-INFINITY, 0.0f, -INFINITY, 0.0f};
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      auto m_of = [&](int u) { return r < 2 ? p0[u][2 * r] : p1[u][2 * r - 4]; };
      auto l_of = [&](int u) { return r < 2 ? p0[u][2 * r + 1] : p1[u][2 * r - 3]; };
      float Mc = M[r];
#pragma unroll
      for (int u = 0; u < kU; ++u) Mc = fmaxf(Mc, m_of(u));
      if (Mc == -INFINITY) continue;  // nothing valid yet
      const float rescale = exp2f(M[r] - Mc);  // 0 while M is -inf
      float ls = Lsum[r] * rescale, s0v = a0[r] * rescale, s1v = a1[r] * rescale;
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const float wgt = exp2f(m_of(u) - Mc);
        ls += wgt * l_of(u);
        s0v += wgt * x0[u][r];
        s1v += wgt * x1[u][r];
      }
      M[r] = Mc;
      Lsum[r] = ls;
      a0[r] = s0v;
      a1[r] = s1v;
    }
  }
  // (heads past n_heads are the zero-query columns of a smaller head count)
  const int nh = kFull ? kH : n_heads;
  float *dst = out + ((int64_t)row * nh + head0) * kDL + dim;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (!kFull && head0 + r >= nh) continue;
    const float inv = Lsum[r] > 0.0f ? 1.0f / Lsum[r] : 0.0f;
    dst[r * kDL] = a0[r] * inv;
    dst[r * kDL + 256] = a1[r] * inv;
    if (lse != nullptr && nt == 0 && (l & 15) == 0)
      lse[(int64_t)row * nh + head0 + r] =
          Lsum[r] > 0.0f ? M[r] * kLn2 + logf(Lsum[r]) : -INFINITY;
  }
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


// ---------------------------------------------------------------------------
// Query-blocked sparse MLA ("Making GLM-5.2 Sparse on TPUs", section "Reuse
// pages across queries": a block of queries loads the union of its selected
// rows once and restores each query's own support with a membership mask
// before the softmax; the union is sorted and compacted, and membership is
// indexed by compact union slot).
//
// A workgroup serves 64 columns (query, head) of one block of QB consecutive
// query rows: QB = 4 queries x 16 heads when a query has 16 or more heads
// (one workgroup per group of 16 heads), QB = 8 queries x 8 heads for
// 8-head shards. Every row tile of the union feeds all 64 columns, as a tile
// of one query's rows feeds its 64 heads in the unblocked kernel; so the
// blocked form pays where a query alone has fewer than 64 heads to offer a
// tile, and saves row loads wherever the block's selections overlap.
// ---------------------------------------------------------------------------

constexpr int kQbMaxSlots = 1 << 20;  // QB * k of one block (32-bit slot arithmetic)
constexpr int kUnionThreads = 256;
constexpr int kUnionWindow = 32768;  // positions per membership map (one byte each, 32 KB of LDS)
constexpr int kUnionPages = 2048;    // block-table entries staged per window
constexpr int kUnionBatch = 8;       // index entries a thread requests at once
constexpr int kChunkRows = kMaxRowsPerSplit;  // union slots per row table of the attention kernel

// Physical row of position pos of sequence b (the page id clamped into the pool).
__device__ __forceinline__ uint32_t phys_row(const int32_t *block_table, int64_t bt_stride, int b,
                                             uint32_t pos, int page_size, FastDiv pdiv,
                                             int64_t num_pages) {
  const uint32_t pidx = fast_div(pos, pdiv);
  const int64_t page = clamp_page(block_table[(int64_t)b * bt_stride + pidx], num_pages);
  return (uint32_t)(page * page_size + (pos - pidx * (uint32_t)page_size));
}

// Bytes of x that are not zero, as their top bits (no carry crosses a byte:
// (b & 0x7F) + 0x7F <= 0xFE).
__device__ __forceinline__ uint32_t nonzero_bytes(uint32_t x) {
  return (((x & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | x) & 0x80808080u;
}

// One workgroup per block m (rows QB m .. QB m + QB - 1): the union of the
// rows' selected positions as physical rows, ascending by position, with a
// QB-bit membership mask per slot (bit q: row QB m + q selected it); slots
// beyond u_count[m] are unused. Entries outside [0, t] are dropped. The
// positions are taken in windows of W = min(kUnionWindow, kUnionPages x page
// size): each window is a byte map in LDS (byte p: the rows that selected
// position window + p, set with LDS atomics) beside the window's slice of the
// block table, and two scans of the map in position order give every
// non-zero byte its slot (each wave walks its quarter of the map 64 words at
// a time, so the reads are conflict-free, and a prefix over the waves orders
// the quarters). This needs the rows in one sequence and every row's valid
// entries first and strictly ascending (what dsa_topk and dsa_page_topk
// write), so that a slot stands for one position of one sequence; any other
// block takes its rows' entries as they are, one slot and one membership bit
// each (a position listed twice then counts twice, as in the unblocked
// kernel).
template <int QB>
__global__ __launch_bounds__(kUnionThreads) void mla_union_kernel(
    const int32_t *__restrict__ block_table, const int32_t *__restrict__ seq_lens,
    const int32_t *__restrict__ cu_q, int batch, int total_q, int max_seq_len, int64_t bt_stride,
    int page_size, FastDiv pdiv, int64_t num_pages, const int32_t *__restrict__ indices, int k,
    FastDiv kdiv, uint32_t *__restrict__ u_rows, uint8_t *__restrict__ u_mask,
    int32_t *__restrict__ u_count) {
  constexpr int kW = kUnionThreads / kWave;
  constexpr int kWords = kUnionWindow / 4;
  constexpr int kWaveWords = kWords / kW;
  __shared__ __attribute__((aligned(16))) uint32_t s_map[kWords];
  __shared__ uint32_t s_pg[kUnionPages + 2];
  __shared__ int s_bq[QB], s_tq[QB], s_nq[QB];
  __shared__ int s_bad;
  __shared__ uint32_t s_wsum[kW];
  const int m = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int cap = QB * k;
  const int64_t ubase = (int64_t)m * cap;
  if (tid < QB) s_nq[tid] = 0;
  if (tid == 0) s_bad = 0;
  // the rows' sequences and positions (a wave per row)
  for (int q = wv; q < QB; q += kW) {
    const int r = m * QB + q;
    RowInfo ri{0, -1};
    if (r < total_q) ri = row_info(cu_q, seq_lens, batch, total_q, max_seq_len, r);
    if (lane == 0) {
      s_bq[q] = ri.b;
      s_tq[q] = ri.t;
    }
  }
  // the first window's map is cleared before the count pass, which fills it
  const int W = (int)min((int64_t)kUnionWindow, (int64_t)kUnionPages * page_size);
  u32x4_t *m4 = reinterpret_cast<u32x4_t *>(s_map);
  for (int i = tid; i < kWords / 4; i += kUnionThreads) m4[i] = u32x4_t{0u, 0u, 0u, 0u};
  __syncthreads();
  // entry e of the block: row q = e / k, slot e - q k of its list (-1 past the batch)
  auto entry = [&](int e, int &q) -> int {
    q = (int)fast_div((uint32_t)e, kdiv);
    const int r = m * QB + q;
    return r < total_q ? indices[(int64_t)r * k + (e - q * k)] : -1;
  };
  // window [w0, w0 + W) of the map: every valid entry in it sets its row's bit
  auto insert = [&](int x, int q, int w0) {
    if (x >= w0 && x - w0 < W && x <= s_tq[q]) {
      const int p = x - w0;
      atomicOr(&s_map[p >> 2], (1u << q) << (8 * (p & 3)));
    }
  };
  // count pass: valid entries per row, whether every row's list is canonical
  // (valid entries first, strictly ascending), and the first window's map;
  // each thread requests kUnionBatch entries (and their successors) at once
  uint32_t nq[QB];
#pragma unroll
  for (int q = 0; q < QB; ++q) nq[q] = 0;
  bool bad = false;
  for (int e0 = tid; e0 < cap; e0 += kUnionBatch * kUnionThreads) {
    int xs[kUnionBatch], ys[kUnionBatch], qs[kUnionBatch];
#pragma unroll
    for (int j = 0; j < kUnionBatch; ++j) {
      const int e = e0 + j * kUnionThreads;
      int q1;
      xs[j] = e < cap ? entry(e, qs[j]) : -1;
      qs[j] = e < cap ? qs[j] : 0;
      ys[j] = (e < cap && e + 1 < (qs[j] + 1) * k) ? entry(e + 1, q1) : -1;
    }
#pragma unroll
    for (int j = 0; j < kUnionBatch; ++j) {
      const int q = qs[j], x = xs[j], y = ys[j];
      const bool vx = x >= 0 && x <= s_tq[q];
      const bool vy = y >= 0 && y <= s_tq[q];
#pragma unroll
      for (int qq = 0; qq < QB; ++qq) nq[qq] += (vx && q == qq) ? 1u : 0u;
      bad |= vy && (!vx || x >= y);
      insert(x, q, 0);
    }
  }
#pragma unroll
  for (int q = 0; q < QB; ++q) {
    const uint32_t t = __builtin_amdgcn_readlane(wave_prefix_sum(nq[q]), kWave - 1);
    if (lane == 0 && t != 0u) atomicAdd(&s_nq[q], (int)t);
  }
  if (__ballot(bad) != 0ull && lane == 0) s_bad = 1;
  bool one_seq = true;
  int tmax = -1;
#pragma unroll
  for (int q = 0; q < QB; ++q) {
    if (q > 0 && m * QB + q < total_q && s_bq[q] != s_bq[0]) one_seq = false;
    tmax = max(tmax, s_tq[q]);
  }
  __syncthreads();
  if (s_bad != 0 || !one_seq) {
    // unused slots read a stand-in row that holds written data: position 0
    // of the first row's sequence that has a valid entry (no such row: an
    // empty union)
    int qs = -1;
#pragma unroll
    for (int q = QB - 1; q >= 0; --q)
      if (s_nq[q] > 0) qs = q;
    if (qs < 0) {
      if (tid == 0) u_count[m] = 0;
      return;
    }
    const uint32_t safe = phys_row(block_table, bt_stride, s_bq[qs], 0u, page_size, pdiv, num_pages);
    for (int e0 = tid; e0 < cap; e0 += kUnionBatch * kUnionThreads) {
      int xs[kUnionBatch], qv[kUnionBatch];
#pragma unroll
      for (int j = 0; j < kUnionBatch; ++j) {
        const int e = e0 + j * kUnionThreads;
        xs[j] = e < cap ? entry(e, qv[j]) : -1;
        qv[j] = e < cap ? qv[j] : 0;
      }
#pragma unroll
      for (int j = 0; j < kUnionBatch; ++j) {
        const int e = e0 + j * kUnionThreads;
        if (e >= cap) continue;
        const int q = qv[j], x = xs[j];
        const bool valid = x >= 0 && x <= s_tq[q];
        u_rows[ubase + e] = valid ? phys_row(block_table, bt_stride, s_bq[q], (uint32_t)x,
                                             page_size, pdiv, num_pages)
                                  : safe;
        u_mask[ubase + e] = valid ? (uint8_t)(1u << q) : (uint8_t)0;
      }
    }
    if (tid == 0) u_count[m] = cap;
    return;
  }
  const int32_t *bt_row = block_table + (int64_t)s_bq[0] * bt_stride;
  uint32_t done = 0;  // slots written by earlier windows
  for (int w0 = 0; w0 <= tmax; w0 += W) {
    if (w0 > 0) {
      // (the first window's map was filled by the count pass)
      for (int i = tid; i < kWords / 4; i += kUnionThreads) m4[i] = u32x4_t{0u, 0u, 0u, 0u};
      __syncthreads();
      for (int e0 = tid; e0 < cap; e0 += kUnionBatch * kUnionThreads) {
        int xs[kUnionBatch], qv[kUnionBatch];
#pragma unroll
        for (int j = 0; j < kUnionBatch; ++j) {
          const int e = e0 + j * kUnionThreads;
          xs[j] = e < cap ? entry(e, qv[j]) : -1;
          qv[j] = e < cap ? qv[j] : 0;
        }
#pragma unroll
        for (int j = 0; j < kUnionBatch; ++j) insert(xs[j], qv[j], w0);
      }
    }
    // the window's pages [p0, p0 + np) of the sequence (np <= W / page size + 1)
    const int wtop = min(w0 + W, tmax + 1) - 1;
    const int p0 = (int)fast_div((uint32_t)w0, pdiv);
    const int np = (int)fast_div((uint32_t)wtop, pdiv) - p0 + 1;
    for (int i = tid; i < np; i += kUnionThreads)
      s_pg[i] = (uint32_t)clamp_page(bt_row[p0 + i], num_pages);
    __syncthreads();
    // wave wv's quarter of the map, words [wv kWaveWords, (wv + 1) kWaveWords),
    // read 64 consecutive words at a time; only words up to the last position
    const int wlast = (wtop - w0) >> 2;
    const int wbeg = wv * kWaveWords;
    const int wend = min(wbeg + kWaveWords, wlast + 1);
    uint32_t cnt = 0;
    for (int c = wbeg; c < wend; c += kWave) {
      const int wi = c + lane;
      cnt += wi < wend ? (uint32_t)__popc(nonzero_bytes(s_map[wi])) : 0u;
    }
    const uint32_t wtot = wave_prefix_sum(cnt);
    if (lane == kWave - 1) s_wsum[wv] = wtot;
    __syncthreads();
    uint32_t run = done, total = 0;
#pragma unroll
    for (int w = 0; w < kW; ++w) {
      run += w < wv ? s_wsum[w] : 0u;
      total += s_wsum[w];
    }
    for (int c = wbeg; c < wend; c += kWave) {
      const int wi = c + lane;
      const uint32_t x = wi < wend ? s_map[wi] : 0u;
      const uint32_t n = (uint32_t)__popc(nonzero_bytes(x));
      const uint32_t incl = wave_prefix_sum(n);
      uint32_t slot = run + incl - n;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t mk = (x >> (8 * j)) & 0xFFu;
        if (mk != 0u) {
          const uint32_t pos = (uint32_t)(w0 + 4 * wi + j);
          const uint32_t pidx = fast_div(pos, pdiv);
          u_rows[ubase + slot] = s_pg[pidx - p0] * (uint32_t)page_size + (pos - pidx * (uint32_t)page_size);
          u_mask[ubase + slot] = (uint8_t)mk;
          ++slot;
        }
      }
      run += __builtin_amdgcn_readlane(incl, kWave - 1);
    }
    done += total;
    __syncthreads();  // the map, page slice and wave totals are free for the next window
  }
  if (tid == 0) u_count[m] = (int32_t)done;
}

// Attention over a block's union: one workgroup per (block, group of 64 / QB
// heads), the four waves over the 64 columns (wave w: columns 16w..16w+15,
// column c = query c / (64 / QB) of the block, head c % (64 / QB) of the
// group). The union is walked in chunks of kChunkRows slots (row table and
// per-query tile masks in LDS), each chunk's tiles through the same four-stage
// ring and tile compute as the unblocked kernel, with each lane's row mask that
// of its column's query. The whole union stays in one workgroup, so there are
// no split partials.
template <bool kOff32, int QB>
__global__ __launch_bounds__(kMlaThreads, 1) void sparse_mla_qblock_kernel(
    int total_q, int n_heads, int n_hg, const uint16_t *__restrict__ q,
    const uint8_t *__restrict__ kv, const uint32_t *__restrict__ u_rows,
    const uint8_t *__restrict__ u_mask, const int32_t *__restrict__ u_count, int cap,
    float scale_log2, float *__restrict__ out, float *__restrict__ lse) {
  constexpr int kHg = kH / QB;  // heads of a query in this workgroup
  __shared__ __attribute__((aligned(1024))) uint8_t s_tiles[kStages * kTileBytes];
  __shared__ __attribute__((aligned(16))) uint32_t s_rowid[kChunkRows + kTileN];
  __shared__ uint32_t s_vm[kChunkRows / kTileN + 1][QB];
  __shared__ float s_ml[kH][2];
  __shared__ int s_over[kMlaWaves];

  // the n_hg workgroups of a block are numbered onto one XCD (block ids are
  // dealt to the 8 XCDs in turn), so they read the union's rows from its L2
  const int bid = (int)blockIdx.x;
  const int xcd = bid % kXcds, rest = bid / kXcds;
  const int hgi = rest % n_hg;
  const int m = (rest / n_hg) * kXcds + xcd;
  const int n_blocks = (total_q + QB - 1) / QB;
  if (m >= n_blocks) return;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 4, j = lane & 15;
  const int64_t ubase = (int64_t)m * cap;
  const int count = min(max(u_count[m], 0), cap);

  // this lane's column: query qi of the block (row m QB + qi), head `head`
  const int col = 16 * wv + j;
  const int qi = col / kHg;
  const int head = hgi * kHg + col % kHg;
  const int qrow = min(m * QB + qi, total_q - 1);
  u32x4_t qf[kSteps];
  const uint16_t *qp = q + ((int64_t)qrow * n_heads + head) * kD + 8 * g;
#pragma unroll
  for (int s = 0; s < kSteps; ++s) qf[s] = ldg16(qp + 32 * s);

  const lds_u8 *tiles = (const lds_u8 *)s_tiles;
  const TileGather<kOff32> tg(kv, (uint32_t)(uintptr_t)tiles, wv, lane);
  const TileLane tl = tile_lane(g, j);
  f32x4_t o[32];
#pragma unroll
  for (int nt = 0; nt < 32; ++nt) o[nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -INFINITY, l_run = 0.0f;
  bool overflow = false;
  if (tid < kMlaWaves) s_over[tid] = 0;

  u32x4_t ra_n, rb_n;
  auto rowids = [&](int tile, u32x4_t &ra, u32x4_t &rb) {
    ra = *reinterpret_cast<const u32x4_t *>(s_rowid + tile * kTileN + 8 * wv);
    rb = *reinterpret_cast<const u32x4_t *>(s_rowid + tile * kTileN + 8 * wv + 4);
  };
  // one chunk of the union: row table, then its tiles through the ring
  auto chunk = [&](int c0) {
    const int n = min(kChunkRows, count - c0);
    const int ntiles = (n + kTileN - 1) / kTileN;
    // slots past the union repeat slot c0's row (a valid stand-in) with no
    // membership; every lane loads (indices inside the chunk), no branch
    for (int e0 = 0; e0 < ntiles * kTileN; e0 += kMlaThreads) {
      const int e = e0 + tid;
      const bool in = e < n;
      const int64_t src = ubase + c0 + (in ? e : 0);
      const uint32_t rid = u_rows[src];
      const uint32_t mk = in ? u_mask[src] : 0u;
      if (e < ntiles * kTileN) s_rowid[e] = rid;
#pragma unroll
      for (int qq = 0; qq < QB; ++qq) {
        const uint64_t bits = __ballot(((mk >> qq) & 1u) != 0u && e < ntiles * kTileN);
        if (lane == 0 && e < ntiles * kTileN) {
          s_vm[e / kTileN][qq] = (uint32_t)bits;
          if (e + kTileN < ntiles * kTileN) s_vm[e / kTileN + 1][qq] = (uint32_t)(bits >> 32);
        }
      }
    }
    // (the compiler's loads have landed before the first direct copies)
    __builtin_amdgcn_s_waitcnt(0x0070);
    __syncthreads();
    for (int tile = 0; tile < min(ntiles, kStages - 1); ++tile) {
      rowids(tile, ra_n, rb_n);
      tg.copy(tile & (kStages - 1), ra_n, rb_n);
    }
    rowids(max(min(kStages - 1, ntiles - 1), 0), ra_n, rb_n);
    for (int tile = 0; tile < ntiles; ++tile) {
      const int ahead = min(ntiles - 1 - tile, kStages - 2);
      if (ahead >= 2) __builtin_amdgcn_s_waitcnt(0x0070 | ((2 * kGatherInsts) & 15) | (((2 * kGatherInsts) >> 4) << 14));
      else if (ahead == 1) __builtin_amdgcn_s_waitcnt(0x0070 | (kGatherInsts & 15) | ((kGatherInsts >> 4) << 14));
      else __builtin_amdgcn_s_waitcnt(0x0070);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      if (tile + kStages - 1 < ntiles) tg.copy((tile + kStages - 1) & (kStages - 1), ra_n, rb_n);
      rowids(min(tile + kStages, ntiles - 1), ra_n, rb_n);
      mla_tile(tiles + (tile & (kStages - 1)) * kTileBytes, s_vm[tile][qi], tl, qf, o, m_run, l_run,
               overflow, scale_log2, s_over + wv);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // no direct load of this chunk in flight
    __syncthreads();                     // stages and row table free for the next chunk
  };
  // passes over the union (a pass that overflowed the headroom is walked again
  // from the raised references, as in the unblocked kernel)
  for (;;) {
    for (int c0 = 0; c0 < count; c0 += kChunkRows) chunk(c0);
    __syncthreads();
    if ((s_over[0] | s_over[1] | s_over[2] | s_over[3]) == 0) break;
    __syncthreads();
    if (tid < kMlaWaves) s_over[tid] = 0;
#pragma unroll
    for (int nt = 0; nt < 32; ++nt) o[nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    l_run = 0.0f;
    overflow = false;
    __syncthreads();
  }

  const float l_tot = group4_sum(l_run);
  if (g == 0) {
    s_ml[col][0] = m_run;
    s_ml[col][1] = l_tot;
  }
  __syncthreads();
  // o[nt][r] of lane (g, j): column 16 wv + 4 g + r, dim 16 nt + j
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int c = 16 * wv + 4 * g + r;
    const int row_c = m * QB + c / kHg;
    if (row_c >= total_q) continue;
    const float l = s_ml[c][1];
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    float *op = out + ((int64_t)row_c * n_heads + hgi * kHg + c % kHg) * kDL + j;
#pragma unroll
    for (int nt = 0; nt < 32; ++nt) op[16 * nt] = o[nt][r] * inv;
  }
  if (lse != nullptr && tid < kH) {
    const int row_c = m * QB + tid / kHg;
    if (row_c < total_q) {
      const float mm = s_ml[tid][0], l = s_ml[tid][1];
      lse[(int64_t)row_c * n_heads + hgi * kHg + tid % kHg] =
          l > 0.0f ? mm * kLn2 + logf(l) : -INFINITY;
    }
  }
}

// The MFMA kernel serves 1..64 heads: a workgroup's 64 columns are the
// query's heads, any missing ones computed on zero queries and dropped.
bool mfma_shape(int32_t q_dtype, int32_t n_heads, int32_t d_latent, int32_t d_rope) {
  return q_dtype == DSA_BF16 && n_heads >= 1 && n_heads <= kH && d_latent == kDL && d_rope == kDR;
}

}  // namespace

int mla_num_splits(int32_t total_q, int32_t n_heads, int32_t d_latent, int32_t k) {
  if (total_q <= 0 || n_heads < 1 || n_heads > kH || d_latent != kDL) return 1;
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

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, once found
}  // namespace

hipError_t mla_scratch(void **ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    // with `dev` current: this GPU's copy of the array
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

size_t mla_workspace_bytes(int32_t total_q, int32_t n_heads, int32_t d_latent, int32_t k) {
  const int s = mla_num_splits(total_q, n_heads, d_latent, k);
  if (s <= 1) return 0;
  // split partials are kept for all 64 columns of the MFMA kernel
  return (size_t)total_q * s * kH * (d_latent + 2) * sizeof(float);
}

hipError_t launch_sparse_mla(const BatchArgs &bt, const MlaLayer *ly, int n_layers,
                             int32_t q_dtype, int32_t n_heads, int32_t d_latent, int32_t d_rope,
                             const int32_t *indices, int32_t k, float scale, void *workspace,
                             size_t, hipStream_t stream) {
  if (bt.total_q == 0 || n_layers < 1) return hipSuccess;
  if (n_layers > kMlaMaxLayers) return hipErrorInvalidValue;
  const float scale_log2 = scale * kLog2e;
  if (mfma_shape(q_dtype, n_heads, d_latent, d_rope)) {
    const int S = mla_num_splits(bt.total_q, n_heads, d_latent, k);
    const int per = (((k + S - 1) / S) + kTileN - 1) / kTileN * kTileN;
    float *ws_acc = static_cast<float *>(workspace);
    float *ws_ml = ws_acc == nullptr
                       ? nullptr
                       : ws_acc + (size_t)n_layers * bt.total_q * S * kH * kDL;
    const int64_t rows_padded = (int64_t)(bt.total_q + kXcds - 1) / kXcds * kXcds;
    const int64_t bpl = rows_padded * S;
    if (bpl * n_layers > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    MlaLayerArgs la{};
    // 32-bit row offsets (from a base 3072 bytes below each cache) when every
    // layer's pool lies within 4 GiB of that base
    bool off32 = true;
    for (int l = 0; l < n_layers; ++l) {
      la.q[l] = static_cast<const uint16_t *>(ly[l].q);
      la.kv[l] = static_cast<const uint8_t *>(ly[l].kv.data);
      la.num_pages[l] = ly[l].kv.num_pages;
      la.out[l] = ly[l].out;
      la.lse[l] = ly[l].lse;
      const uint64_t pool_bytes = (uint64_t)ly[l].kv.num_pages * (uint64_t)ly[l].kv.page_size * kRowBytes;
      off32 = off32 && pool_bytes + 4096 <= (1ull << 32);
    }
    const bool full = n_heads == kH;
    auto kern = off32 ? (full ? sparse_mla_bf16_kernel<true, true> : sparse_mla_bf16_kernel<true, false>)
                      : (full ? sparse_mla_bf16_kernel<false, true> : sparse_mla_bf16_kernel<false, false>);
    const int page_size = ly[0].kv.page_size;
    hipLaunchKernelGGL(kern, dim3((unsigned)(bpl * n_layers)), dim3(kMlaThreads), 0, stream,
                       bt.block_table, bt.seq_lens, bt.cu_q, bt.batch, bt.total_q,
                       bt.max_seq_len, bt.bt_stride, la, (int)bpl, page_size,
                       make_fast_div((uint32_t)page_size), indices, k, S, per, scale_log2,
                       ws_acc, ws_ml, n_heads);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || S == 1) return e;
    auto ck = full ? mla_combine_kernel<true> : mla_combine_kernel<false>;
    hipLaunchKernelGGL(ck,
                       dim3((unsigned)((int64_t)bt.total_q * kCombineBlocksPerRow * n_layers)),
                       dim3(kCombineThreads), 0, stream, bt.total_q, S, ws_acc, ws_ml, la, n_heads);
    return hipGetLastError();
  }
  for (int l = 0; l < n_layers; ++l) {
    const CacheArgs &kv = ly[l].kv;
    if (q_dtype == DSA_F32) {
      hipLaunchKernelGGL(sparse_mla_generic_kernel<float>, dim3(bt.total_q * n_heads), dim3(256), 0,
                         stream, bt.block_table, bt.seq_lens, bt.cu_q, bt.batch, bt.total_q,
                         bt.max_seq_len, bt.bt_stride, static_cast<const float *>(ly[l].q),
                         static_cast<const float *>(kv.data), kv.num_pages, kv.page_size, n_heads,
                         d_latent, d_rope, indices, k, scale_log2, ly[l].out, ly[l].lse);
    } else {
      hipLaunchKernelGGL(sparse_mla_generic_kernel<uint16_t>, dim3(bt.total_q * n_heads), dim3(256),
                         0, stream, bt.block_table, bt.seq_lens, bt.cu_q, bt.batch, bt.total_q,
                         bt.max_seq_len, bt.bt_stride, static_cast<const uint16_t *>(ly[l].q),
                         static_cast<const uint16_t *>(kv.data), kv.num_pages, kv.page_size,
                         n_heads, d_latent, d_rope, indices, k, scale_log2, ly[l].out, ly[l].lse);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// query-blocked launcher
// ---------------------------------------------------------------------------

int mla_qblock_qb(int32_t n_heads) { return n_heads >= 16 ? 4 : 8; }

bool mla_qblock_supported(int32_t q_dtype, int32_t n_heads, int32_t d_latent, int32_t d_rope,
                          int32_t k) {
  if (q_dtype != DSA_BF16 || d_latent != kDL || d_rope != kDR) return false;
  if (!(n_heads == 8 || (n_heads >= 16 && n_heads <= kH && n_heads % 16 == 0))) return false;
  return (int64_t)mla_qblock_qb(n_heads) * k <= kQbMaxSlots;
}

namespace {
struct QbLayout {
  int64_t n_blocks, cap;
  size_t rows_off, mask_off, count_off, bytes;
};
QbLayout qb_layout(int32_t total_q, int32_t n_heads, int32_t k) {
  QbLayout L{};
  const int QB = mla_qblock_qb(n_heads);
  L.n_blocks = (total_q + QB - 1) / QB;
  L.cap = (int64_t)QB * k;
  auto up16 = [](size_t x) { return (x + 15) & ~(size_t)15; };
  L.rows_off = 0;
  L.mask_off = up16((size_t)L.n_blocks * L.cap * sizeof(uint32_t));
  L.count_off = L.mask_off + up16((size_t)L.n_blocks * L.cap);
  L.bytes = L.count_off + up16((size_t)L.n_blocks * sizeof(int32_t));
  return L;
}
}  // namespace

size_t mla_qblock_workspace_bytes(int32_t total_q, int32_t n_heads, int32_t k) {
  if (total_q < 1 || n_heads < 1 || k < 1) return 0;
  return qb_layout(total_q, n_heads, k).bytes;
}

hipError_t launch_sparse_mla_qblocked(const BatchArgs &bt, const MlaLayer &ly, int32_t n_heads,
                                      const int32_t *indices, int32_t k, float scale,
                                      void *workspace, hipStream_t stream) {
  if (bt.total_q == 0) return hipSuccess;
  const int QB = mla_qblock_qb(n_heads);
  const QbLayout L = qb_layout(bt.total_q, n_heads, k);
  if (L.n_blocks > 0x7FFFFFFF / kXcds) return hipErrorInvalidConfiguration;
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  uint32_t *u_rows = reinterpret_cast<uint32_t *>(ws + L.rows_off);
  uint8_t *u_mask = ws + L.mask_off;
  int32_t *u_count = reinterpret_cast<int32_t *>(ws + L.count_off);
  const CacheArgs &kv = ly.kv;
  const FastDiv pdiv = make_fast_div((uint32_t)kv.page_size);
  const FastDiv kdiv = make_fast_div((uint32_t)k);
  auto uk = QB == 4 ? mla_union_kernel<4> : mla_union_kernel<8>;
  hipLaunchKernelGGL(uk, dim3((unsigned)L.n_blocks), dim3(kUnionThreads), 0, stream, bt.block_table,
                     bt.seq_lens, bt.cu_q, bt.batch, bt.total_q, bt.max_seq_len, bt.bt_stride,
                     kv.page_size, pdiv, kv.num_pages, indices, k, kdiv, u_rows, u_mask, u_count);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n_hg = n_heads / (kH / QB);
  const int64_t blocks = (L.n_blocks + kXcds - 1) / kXcds * kXcds * n_hg;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const uint64_t pool_bytes = (uint64_t)kv.num_pages * (uint64_t)kv.page_size * kRowBytes;
  const bool off32 = pool_bytes + 4096 <= (1ull << 32);
  auto ak = QB == 4 ? (off32 ? sparse_mla_qblock_kernel<true, 4> : sparse_mla_qblock_kernel<false, 4>)
                    : (off32 ? sparse_mla_qblock_kernel<true, 8> : sparse_mla_qblock_kernel<false, 8>);
  hipLaunchKernelGGL(ak, dim3((unsigned)blocks), dim3(kMlaThreads), 0, stream, bt.total_q, n_heads,
                     n_hg, static_cast<const uint16_t *>(ly.q),
                     static_cast<const uint8_t *>(kv.data), u_rows, u_mask, u_count, (int)L.cap,
                     scale * kLog2e, ly.out, ly.lse);
  return hipGetLastError();
}

}  // namespace dsa
