// Read-stream probe for the benchmark's second roofline denominator: the HBM
// read rate a plain streaming kernel reaches on this device. Not part of the
// decode path; built into its own library (libdsa_bench.so).
//
// Each thread reads 16-byte words with a grid stride, eight loads in flight
// per thread, and folds them with XOR into one word per workgroup written to
// `sink` (so no load can be dropped). Every address read lies inside
// [buf, buf + bytes): the 16-byte body is walked in full groups of eight
// words, then one word at a time, and the last bytes % 16 are read as bytes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsa_bench.h"

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void read_stream_kernel(const u32x4 *__restrict__ buf,
                                                               uint64_t n_words,
                                                               const uint8_t *__restrict__ tail,
                                                               uint32_t n_tail,
                                                               uint32_t *__restrict__ sink) {
  __shared__ uint32_t s_red[kThreads / 64];
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  // groups of kUnroll words, each word stride apart: every load of a group is
  // issued before any is used
  for (; i + (kUnroll - 1) * stride < n_words; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
  }
  for (; i < n_words; i += stride) acc ^= buf[i];
  uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  const uint32_t g = blockIdx.x * kThreads + threadIdx.x;
  if (g < n_tail) x ^= tail[g];
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o);
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = s_red[0] ^ s_red[1] ^ s_red[2] ^ s_red[3];
}

}  // namespace

extern "C" {

uint32_t dsa_bench_read_blocks(void) { return 256u * 16u; }

int dsa_bench_read(const void *buf, size_t bytes, uint32_t *sink, void *stream) {
  if (buf == nullptr || sink == nullptr || bytes == 0) return 1;
  if ((reinterpret_cast<uintptr_t>(buf) & 15u) != 0) return 2;
  const uint64_t n_words = bytes / 16;
  const uint32_t n_tail = (uint32_t)(bytes % 16);
  const uint32_t blocks = dsa_bench_read_blocks();
  hipLaunchKernelGGL(read_stream_kernel, dim3(blocks), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4 *>(buf), n_words,
                     static_cast<const uint8_t *>(buf) + n_words * 16, n_tail, sink);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

}  // extern "C"
