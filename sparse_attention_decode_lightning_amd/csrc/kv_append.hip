// Appending this step's tokens to the paged caches on gfx950 ("GLM-5.2 on
// vLLM Ascend: Request-to-Backend Inference Path", section "8. The SFA
// backend, step by step", "Write paged cache": a slot mapping scatters the new
// latent rows and, for layers that own an indexer, the new indexer keys and
// scales into their physical pages; "Making GLM-5.2 Sparse on TPUs", section
// "Append new KV without moving the resident cache": the work scales with the
// new rows, and the resident rows are left untouched).
//
// One wave per (token, cache). A copied row moves in 16-byte pieces when the
// row length allows it (2-byte or 4-byte elements otherwise). A key row bound
// for an e4m3 cache is quantised per token: sigma = max|k| / 448 (1 when the
// row is all zeros), each element k / sigma clamped to [-448, 448] and
// rounded to the nearest e4m3 value, ties to the even code; sigma goes to the
// scale array so that sigma * e4m3(byte) is the stored key.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kAppendThreads = 256;
constexpr int kAppendWaves = kAppendThreads / kWave;

// fp32 (finite, |x| <= 448) -> OCP e4m3fn byte, round to nearest, ties to
// even, worked on the binary32 fields: keep 3 mantissa bits below the
// leading one for normal results (exponent >= -6), or the multiple of 2^-9
// for subnormal ones, rounding the dropped bits.
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t mag = u & 0x7FFFFFFFu;
  if (mag == 0u) return sign;
  const int e = (int)(mag >> 23) - 127;            // unbiased exponent (input is normal or subnormal fp32)
  uint32_t m = (mag & 0x7FFFFFu) | (e > -127 ? 0x800000u : 0u);  // 24-bit significand
  const int e_eff = e > -127 ? e : -126;
  // value = m * 2^(e_eff - 23); the code counts units of 2^(max(e_eff, -6) - 3)
  const int unit_exp = (e_eff >= -6 ? e_eff : -6) - 3;
  const int shift = unit_exp - (e_eff - 23);  // >= 20
  uint32_t q;
  if (shift >= 32) {
    q = 0u;
  } else {
    q = m >> shift;
    const uint32_t rem = m & ((1u << shift) - 1u);
    const uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (q & 1u))) ++q;
  }
  if (e_eff >= -6) {
    // q in [8, 16]: leading one at bit 3; 16 carries into the next binade
    int be = e_eff + 7;
    if (q >= 16u) {
      q >>= 1;
      ++be;
    }
    return sign | ((uint32_t)be << 3) | (q & 7u);
  }
  // subnormal range: q in [0, 8]; 8 is the smallest normal, code 0x08
  return sign | q;
}

template <typename T>
__device__ __forceinline__ float load_f32(const T *p, int i) {
  if constexpr (sizeof(T) == 4) return reinterpret_cast<const float *>(p)[i];
  else return bf16_to_f32(reinterpret_cast<const uint16_t *>(p)[i]);
}

// Copy `bytes` bytes (a multiple of `esize`) from src to dst with one wave.
__device__ __forceinline__ void wave_copy(uint8_t *dst, const uint8_t *src, int64_t bytes,
                                          int esize, int lane) {
  if ((bytes & 15) == 0 && ((uintptr_t)dst & 15) == 0 && ((uintptr_t)src & 15) == 0) {
    for (int64_t c = lane; c < bytes / 16; c += kWave)
      reinterpret_cast<u32x4_t *>(dst)[c] = reinterpret_cast<const u32x4_t *>(src)[c];
  } else if (esize == 4) {
    for (int64_t c = lane; c < bytes / 4; c += kWave)
      reinterpret_cast<uint32_t *>(dst)[c] = reinterpret_cast<const uint32_t *>(src)[c];
  } else {
    for (int64_t c = lane; c < bytes / 2; c += kWave)
      reinterpret_cast<uint16_t *>(dst)[c] = reinterpret_cast<const uint16_t *>(src)[c];
  }
}

template <typename TK>
__global__ __launch_bounds__(kAppendThreads) void kv_append_kernel(
    const int32_t *__restrict__ slots, int n_tokens, const uint8_t *__restrict__ latent,
    uint8_t *__restrict__ kv, int64_t kv_slots, int64_t kv_row_bytes, int kv_esize,
    const TK *__restrict__ keys, uint8_t *__restrict__ kc, float *__restrict__ kscale,
    int64_t k_slots, int k_dim, int k_esize_out, bool k_fp8) {
  const int lane = threadIdx.x & 63;
  const int64_t job = (int64_t)blockIdx.x * kAppendWaves + (threadIdx.x >> 6);
  const int n_lat = latent != nullptr ? n_tokens : 0;
  const int n_key = keys != nullptr ? n_tokens : 0;
  if (job < n_lat) {
    const int64_t s = slots[job];
    if (s >= 0 && s < kv_slots)
      wave_copy(kv + s * kv_row_bytes, latent + job * kv_row_bytes, kv_row_bytes, kv_esize, lane);
    return;
  }
  const int64_t i = job - n_lat;
  if (i >= n_key) return;
  const int64_t s = slots[i];
  if (s < 0 || s >= k_slots) return;
  const TK *src = keys + i * k_dim;
  if (!k_fp8) {
    wave_copy(kc + s * (int64_t)k_dim * k_esize_out, reinterpret_cast<const uint8_t *>(src),
              (int64_t)k_dim * k_esize_out, k_esize_out, lane);
    return;
  }
  float amax = 0.0f;
  for (int d = lane; d < k_dim; d += kWave) amax = fmaxf(amax, fabsf(load_f32(src, d)));
  amax = wave_max(amax);
  const float sigma = amax > 0.0f ? amax / 448.0f : 1.0f;
  uint8_t *dst = kc + s * (int64_t)k_dim;
  for (int d = lane; d < k_dim; d += kWave) {
    const float q = fminf(fmaxf(load_f32(src, d) / sigma, -448.0f), 448.0f);
    dst[d] = (uint8_t)e4m3_encode(q);
  }
  if (lane == 0) kscale[s] = sigma;
}

}  // namespace

hipError_t launch_kv_append(const int32_t *slots, int32_t n_tokens, const void *latent,
                            const CacheArgs *kv, const void *keys, int32_t key_dtype,
                            const CacheArgs *kidx, hipStream_t stream) {
  if (n_tokens == 0) return hipSuccess;
  const int jobs = (latent != nullptr ? n_tokens : 0) + (keys != nullptr ? n_tokens : 0);
  const dim3 grid((unsigned)((jobs + kAppendWaves - 1) / kAppendWaves));
  const int kv_esize = kv != nullptr ? (kv->dtype == DSA_F32 ? 4 : 2) : 2;
  uint8_t *kv_data = kv != nullptr ? static_cast<uint8_t *>(const_cast<void *>(kv->data)) : nullptr;
  const int64_t kv_slots = kv != nullptr ? kv->num_pages * kv->page_size : 0;
  const int64_t kv_row = kv != nullptr ? (int64_t)kv->row_elems * kv_esize : 0;
  uint8_t *kc = kidx != nullptr ? static_cast<uint8_t *>(const_cast<void *>(kidx->data)) : nullptr;
  float *ks = kidx != nullptr ? const_cast<float *>(kidx->scale) : nullptr;
  const int64_t k_slots = kidx != nullptr ? kidx->num_pages * kidx->page_size : 0;
  const int k_dim = kidx != nullptr ? kidx->row_elems : 0;
  const bool fp8 = kidx != nullptr && kidx->dtype == DSA_FP8_E4M3;
  const int k_esize_out = kidx == nullptr ? 2 : (kidx->dtype == DSA_F32 ? 4 : (fp8 ? 1 : 2));
  const uint8_t *lat = static_cast<const uint8_t *>(latent);
  if (keys == nullptr || key_dtype == DSA_BF16) {
    hipLaunchKernelGGL(kv_append_kernel<uint16_t>, grid, dim3(kAppendThreads), 0, stream, slots,
                       n_tokens, lat, kv_data, kv_slots, kv_row, kv_esize,
                       static_cast<const uint16_t *>(keys), kc, ks, k_slots, k_dim, k_esize_out,
                       fp8);
  } else {
    hipLaunchKernelGGL(kv_append_kernel<float>, grid, dim3(kAppendThreads), 0, stream, slots,
                       n_tokens, lat, kv_data, kv_slots, kv_row, kv_esize,
                       static_cast<const float *>(keys), kc, ks, k_slots, k_dim, k_esize_out, fp8);
  }
  return hipGetLastError();
}

}  // namespace dsa
