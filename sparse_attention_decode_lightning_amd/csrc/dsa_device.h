// Device-side helpers shared by the gfx950 kernels: element conversions,
// MFMA fragment types, wave reductions and paged-cache addressing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits (inputs here are finite probabilities).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// OCP E4M3FN -> bf16 on the gfx950 conversion unit (scale 1.0, so exact:
// every e4m3fn value is a bf16 value). Four bytes of a dword -> two dwords of
// bf16 pairs, lowest byte first.
__device__ __forceinline__ u32x2_t e4m3x4_to_bf16x4(uint32_t w) {
  u32x2_t r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
  return r;
}

// One OCP E4M3FN byte -> fp32 (exact).
__device__ __forceinline__ float e4m3_to_f32(uint32_t byte) {
  return __builtin_amdgcn_cvt_f32_fp8((int)byte, 0);
}

__device__ __forceinline__ f32x4_t mfma_16x16x32_bf16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x4_t ldg16(const void *p) {
  return *reinterpret_cast<const u32x4_t *>(p);
}

// Reductions over each row of 16 lanes with DPP lane permutes (no LDS): swap
// neighbours, swap pairs, mirror within 8 lanes, mirror within 16 lanes. Every
// lane of the row ends with the row's result.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141; // row_half_mirror
constexpr int kDppMirror = 0x140;     // row_mirror

__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp<kDppXor1>(v));
  v = fmaxf(v, dpp<kDppXor2>(v));
  v = fmaxf(v, dpp<kDppHalfMirror>(v));
  return fmaxf(v, dpp<kDppMirror>(v));
}

__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  v += dpp<kDppHalfMirror>(v);
  return v + dpp<kDppMirror>(v);
}

// 2^x on the hardware exp unit (inputs here are <= 0; -inf gives 0).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Division by a runtime divisor d >= 1 as a multiply-high and a shift
// (Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994, round-up variant): with l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1, n / d = (mulhi(n, m) + n) >> l for every
// 0 <= n < 2^31. The host fills the pair; kernels divide with two VALU ops.
struct FastDiv {
  uint32_t mul;
  uint32_t shift;
};

inline FastDiv make_fast_div(uint32_t d) {
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  const uint64_t m = (((1ull << 32) * ((1ull << l) - d)) / d) + 1;
  return FastDiv{(uint32_t)m, l};
}

__device__ __forceinline__ uint32_t fast_div(uint32_t n, FastDiv f) {
  return (__umulhi(n, f.mul) + n) >> f.shift;
}

// max(x, 0) as an integer max on the bits: negative floats (and -0) have the
// sign bit set and compare below 0 as int32, non-negative floats keep their bits.
__device__ __forceinline__ float relu_bits(float x) {
  return __builtin_bit_cast(float, max(__builtin_bit_cast(int, x), 0));
}

struct RowInfo {
  int b;  // sequence of the row
  int t;  // absolute position of the row; -1 if the metadata leaves it none
};

// The clamping half of row_info, shared with host-side checks: sequence b
// (already found) with query offsets c0 = cu_q[b], c1 = cu_q[b + 1] and
// length len, as read from memory. Offsets are clamped into [0, total_q],
// the length into [0, max_seq_len], and the position to at most L - 1, so
// that whatever the metadata holds, t is -1 or in [0, max_seq_len).
__host__ __device__ inline int clamp_int(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

__host__ __device__ inline RowInfo row_clamp(int b, int c0, int c1, int len, int total_q,
                                             int max_seq_len, int row) {
  RowInfo ri;
  ri.b = b;
  const int q0 = clamp_int(c0, 0, total_q);
  const int q1 = clamp_int(c1, q0, total_q);
  const int L = clamp_int(len, 0, max_seq_len);
  const int t = L - (q1 - q0) + (row - q0);
  ri.t = (row < q0 || row >= q1) ? -1 : (t < L - 1 ? t : L - 1);
  ri.t = ri.t < -1 ? -1 : ri.t;
  return ri;
}

// A physical page id from a block table, clamped into the pool [0, num_pages).
__host__ __device__ inline int64_t clamp_page(int64_t page, int64_t num_pages) {
  return page < 0 ? 0 : (page >= num_pages ? num_pages - 1 : page);
}

// Sequence and causal position of a flattened query row: b is the largest
// b < batch with cu_q[b] <= row (0 if none). Wave-cooperative: every lane of
// the wave must be active and pass the same row. With non-decreasing offsets
// the lanes whose offset is <= row form a prefix, so one load per lane and a
// ballot replace a chain of dependent loads. Every value is
// clamped so malformed metadata can never index past the caller's buffers:
// q offsets into [0, total_q], lengths into [0, max_seq_len], t <= L - 1.
// One round trip: with the offset each lane also loads the next offset and
// the length of its sequence, and the row's three values are read from the
// lane of the sequence found (lane 0 of the first chunk when none is).
__device__ __forceinline__ RowInfo row_info(const int32_t *cu_q, const int32_t *seq_lens,
                                            int batch, int total_q, int max_seq_len, int row) {
  const int lane = threadIdx.x & 63;
  int b = 0, c0 = 0, c1 = 0, len = 0;
  for (int base = 0; base < batch; base += 64) {
    const int i = base + lane;
    const bool in = i < batch;
    const int a0 = in ? cu_q[i] : 0;
    const int a1 = in ? cu_q[i + 1] : 0;
    const int al = in ? seq_lens[i] : 0;
    const uint64_t hit = __ballot(in && a0 <= row);
    if (base == 0 || hit != 0ull) {
      const int src = hit != 0ull ? 63 - __clzll(hit) : 0;
      b = base + src;
      c0 = __builtin_amdgcn_readlane(a0, src);
      c1 = __builtin_amdgcn_readlane(a1, src);
      len = __builtin_amdgcn_readlane(al, src);
    }
    if (hit != ~0ull) break;
  }
  return row_clamp(b, c0, c1, len, total_q, max_seq_len, row);
}

// Element offset of token `pos` of sequence `b` in a paged cache, with the
// physical page id clamped into the pool so malformed tables stay in bounds.
__device__ __forceinline__ int64_t paged_row(const int32_t *block_table, int64_t bt_stride, int b,
                                             int pos, int page_size, int64_t num_pages) {
  const int64_t page = clamp_page(block_table[(int64_t)b * bt_stride + pos / page_size], num_pages);
  return page * page_size + pos % page_size;
}

}  // namespace dsa
