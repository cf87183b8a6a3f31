/*
 * dsa_bench.h — a measurement helper shipped beside the decode library, in
 * its own shared library (libdsa_bench.so). It is not a step of the decode
 * path: the benchmark uses it to measure the HBM read rate that a plain
 * streaming kernel reaches on the device, the second denominator of its
 * roofline fractions (the first is the vendor's 8 TB/s).
 */
#ifndef DSA_BENCH_H_
#define DSA_BENCH_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Number of workgroups dsa_bench_read launches: `sink` needs that many
 * uint32 entries. */
uint32_t dsa_bench_read_blocks(void);

/*
 * Read every byte of `buf` once (16-byte non-temporal loads, grid-stride) and
 * write one XOR-fold per workgroup to sink[0 .. dsa_bench_read_blocks() - 1].
 * Enqueued on `stream` (a hipStream_t); the caller times it with events.
 *
 *   buf    device, 16-byte aligned, `bytes` readable bytes (bytes > 0)
 *   sink   device uint32[dsa_bench_read_blocks()]
 *
 * Returns 0 on success, 1 for a NULL pointer or zero size, 2 for a
 * misaligned buffer, 6 if the runtime rejects the launch. Owns nothing,
 * allocates nothing.
 */
int dsa_bench_read(const void *buf, size_t bytes, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_BENCH_H_ */
