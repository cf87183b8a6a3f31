/* A plain C client of libdsa.so: device buffers from the HIP runtime, the
 * three calls of one decode step through the C ABI, no other runtime.
 *
 * Input file (little-endian, from the test): int32 B, L, P, T, H_I, D_I, K,
 * H, DL, DR, n_pages; then int32 block_table[B * (L / P)], seq_lens[B],
 * cu_q[B + 1]; float q_idx[T * H_I * D_I], w[T * H_I], keys[n_pages * P *
 * D_I], q[T * H * (DL + DR)], kv[n_pages * P * (DL + DR)], scale.
 * Output file: int32 indices[T * K], float out[T * H * DL], lse[T * H]. */
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "dsa.h"

static void *upload(const void *host, size_t bytes) {
  void *d = NULL;
  if (hipMalloc(&d, bytes ? bytes : 4) != hipSuccess) exit(3);
  if (host != NULL && bytes && hipMemcpy(d, host, bytes, hipMemcpyHostToDevice) != hipSuccess)
    exit(3);
  return d;
}

static void *readn(FILE *f, size_t bytes) {
  void *p = malloc(bytes ? bytes : 4);
  if (p == NULL || fread(p, 1, bytes, f) != bytes) exit(2);
  return p;
}

int main(int argc, char **argv) {
  if (argc != 3) return 1;
  FILE *f = fopen(argv[1], "rb");
  if (f == NULL) return 2;
  int32_t hdr[11];
  if (fread(hdr, 4, 11, f) != 11) return 2;
  const int B = hdr[0], L = hdr[1], P = hdr[2], T = hdr[3], HI = hdr[4], DI = hdr[5], K = hdr[6];
  const int H = hdr[7], DL = hdr[8], DR = hdr[9], NP = hdr[10];
  const int bts = L / P;
  int32_t *bt = readn(f, 4u * B * bts), *lens = readn(f, 4u * B), *cu = readn(f, 4u * (B + 1));
  float *qi = readn(f, 4u * T * HI * DI), *w = readn(f, 4u * T * HI);
  float *keys = readn(f, 4u * NP * P * DI), *q = readn(f, 4u * T * H * (DL + DR));
  float *kv = readn(f, 4u * NP * P * (DL + DR)), scale;
  if (fread(&scale, 4, 1, f) != 1) return 2;
  fclose(f);

  dsa_batch b = {upload(bt, 4u * B * bts), upload(lens, 4u * B), upload(cu, 4u * (B + 1)),
                 B, bts, T, L, 1};
  dsa_paged_cache kc = {upload(keys, 4u * NP * P * DI), NULL, NP, P, DI, DSA_F32};
  dsa_paged_cache vc = {upload(kv, 4u * NP * P * (DL + DR)), NULL, NP, P, DL + DR, DSA_F32};
  float *scores = upload(NULL, 4u * T * L);
  int32_t *idx = upload(NULL, 4u * T * K);
  float *out = upload(NULL, 4u * T * H * DL), *lse = upload(NULL, 4u * T * H);
  size_t tws = dsa_topk_workspace_size(T, L, K), mws = dsa_sparse_mla_workspace_size(T, H, DL, K);
  void *tw = tws ? upload(NULL, tws) : NULL, *mw = mws ? upload(NULL, mws) : NULL;

  dsa_status st = dsa_indexer_scores(&b, upload(qi, 4u * T * HI * DI), DSA_F32,
                                     upload(w, 4u * T * HI), HI, DI, &kc, scores, L, NULL);
  if (st == DSA_OK) st = dsa_topk(&b, scores, L, K, idx, tw, tws, NULL);
  if (st == DSA_OK)
    st = dsa_sparse_mla_fwd(&b, upload(q, 4u * T * H * (DL + DR)), DSA_F32, H, DL, DR, &vc, idx,
                            K, scale, out, lse, mw, mws, NULL);
  if (st != DSA_OK) {
    fprintf(stderr, "%s\n", dsa_status_str(st));
    return 4;
  }
  if (hipDeviceSynchronize() != hipSuccess) return 3;
  int32_t *hidx = malloc(4u * T * K);
  float *hout = malloc(4u * T * H * DL), *hlse = malloc(4u * T * H);
  hipMemcpy(hidx, idx, 4u * T * K, hipMemcpyDeviceToHost);
  hipMemcpy(hout, out, 4u * T * H * DL, hipMemcpyDeviceToHost);
  hipMemcpy(hlse, lse, 4u * T * H, hipMemcpyDeviceToHost);
  FILE *o = fopen(argv[2], "wb");
  if (o == NULL) return 2;
  fwrite(hidx, 4, (size_t)T * K, o);
  fwrite(hout, 4, (size_t)T * H * DL, o);
  fwrite(hlse, 4, (size_t)T * H, o);
  fclose(o);
  printf("ok\n");
  return 0;
}
