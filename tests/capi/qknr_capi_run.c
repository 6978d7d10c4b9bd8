/*
 * Drives libqknr.so through its C ABI alone (include/qknr.h + the HIP runtime;
 * no Python, no torch): reads a case file written by the test, copies the
 * inputs to the device, runs qknr_inplace on a stream of its own, copies q and
 * k back and writes them out for the test to compare with the fp64 oracle.
 * It then runs the same case again from the same inputs through qknr_inplace_ex
 * with the element-granular kernel requested (qknr_launch_cfg.generic) and prints
 * the launch report. It also exercises qknr_can_use, qknr_status_string and one
 * rejection.
 *
 * Case file (little endian): int64 T, Hq, Hkv, head_dim, rope_dim, is_neox,
 * dtype, pos_dtype, cache_rows; float eps; then q (T*Hq*D u16), k (T*Hkv*D u16),
 * wq (D u16), wk (D u16), cache (cache_rows*R f32), positions (T i32 or i64).
 * Output file: q then k from qknr_inplace, then q and k from qknr_inplace_ex,
 * as u16.
 * Exit status 0 on success; a message on stderr otherwise.
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "qknr.h"

#define CHECK_HIP(x)                                                      \
  do {                                                                    \
    hipError_t e_ = (x);                                                  \
    if (e_ != hipSuccess) {                                               \
      fprintf(stderr, "HIP error %d at %s:%d\n", (int)e_, __FILE__, __LINE__); \
      return 2;                                                           \
    }                                                                     \
  } while (0)

static int read_all(FILE* f, void* dst, size_t n) { return fread(dst, 1, n, f) == n ? 0 : -1; }

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s case.bin out.bin\n", argv[0]);
    return 1;
  }
  FILE* f = fopen(argv[1], "rb");
  if (!f) { perror("case"); return 1; }
  int64_t hdr[9];
  float eps;
  if (read_all(f, hdr, sizeof hdr) || read_all(f, &eps, sizeof eps)) { fprintf(stderr, "short header\n"); return 1; }
  const int64_t T = hdr[0], Hq = hdr[1], Hkv = hdr[2], D = hdr[3], R = hdr[4], neox = hdr[5];
  const int64_t dtype = hdr[6], pos_dtype = hdr[7], rows = hdr[8];
  const size_t nq = (size_t)(T * Hq * D), nk = (size_t)(T * Hkv * D);
  const size_t psz = pos_dtype == QKNR_I64 ? 8 : 4;
  const size_t bytes_q = nq * 2, bytes_k = nk * 2, bytes_w = (size_t)D * 2;
  const size_t bytes_c = (size_t)(rows * R) * 4, bytes_p = (size_t)T * psz;
  char* host = (char*)malloc(bytes_q + bytes_k + 2 * bytes_w + bytes_c + bytes_p);
  if (!host) return 1;
  char* hq = host;
  char* hk = hq + bytes_q;
  char* hwq = hk + bytes_k;
  char* hwk = hwq + bytes_w;
  char* hc = hwk + bytes_w;
  char* hp = hc + bytes_c;
  if (read_all(f, host, bytes_q + bytes_k + 2 * bytes_w + bytes_c + bytes_p)) { fprintf(stderr, "short body\n"); return 1; }
  fclose(f);

  if (!qknr_can_use((int32_t)D, (int32_t)R, (int32_t)neox, (int32_t)dtype, (int32_t)pos_dtype)) {
    fprintf(stderr, "qknr_can_use says no\n");
    return 3;
  }
  /* a rejection must come back before any work: eps < 0 */
  int32_t rc = qknr_inplace(NULL, NULL, NULL, NULL, NULL, NULL, T, (int32_t)Hq, (int32_t)Hkv,
                            (int32_t)D, (int32_t)R, (int32_t)neox, -1.0f, 0, 0, 0, 0,
                            (int32_t)dtype, (int32_t)pos_dtype, NULL);
  if (rc != QKNR_E_ARG || strstr(qknr_status_string(rc), "eps") == NULL) {
    fprintf(stderr, "expected QKNR_E_ARG, got %d (%s)\n", rc, qknr_status_string(rc));
    return 4;
  }

  void *dq, *dk, *dwq, *dwk, *dc, *dp;
  CHECK_HIP(hipMalloc(&dq, bytes_q ? bytes_q : 16));
  CHECK_HIP(hipMalloc(&dk, bytes_k ? bytes_k : 16));
  CHECK_HIP(hipMalloc(&dwq, bytes_w));
  CHECK_HIP(hipMalloc(&dwk, bytes_w));
  CHECK_HIP(hipMalloc(&dc, bytes_c));
  CHECK_HIP(hipMalloc(&dp, bytes_p ? bytes_p : 16));
  CHECK_HIP(hipMemcpy(dq, hq, bytes_q, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dk, hk, bytes_k, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dwq, hwq, bytes_w, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dwk, hwk, bytes_w, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dc, hc, bytes_c, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dp, hp, bytes_p, hipMemcpyHostToDevice));
  hipStream_t s;
  CHECK_HIP(hipStreamCreate(&s));
  rc = qknr_inplace(dq, dk, dwq, dwk, (const float*)dc, dp, T, (int32_t)Hq, (int32_t)Hkv,
                    (int32_t)D, (int32_t)R, (int32_t)neox, eps, Hq * D * 2, D * 2, Hkv * D * 2,
                    D * 2, (int32_t)dtype, (int32_t)pos_dtype, s);
  if (rc != QKNR_OK) {
    fprintf(stderr, "qknr_inplace: %s\n", qknr_status_string(rc));
    return 5;
  }
  CHECK_HIP(hipStreamSynchronize(s));
  char* out = (char*)malloc(2 * (bytes_q + bytes_k) + 2);
  if (!out) return 1;
  CHECK_HIP(hipMemcpy(out, dq, bytes_q, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(out + bytes_q, dk, bytes_k, hipMemcpyDeviceToHost));

  /* the same case from the same inputs, element-granular kernel requested */
  CHECK_HIP(hipMemcpy(dq, hq, bytes_q, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dk, hk, bytes_k, hipMemcpyHostToDevice));
  qknr_launch_cfg cfg;
  memset(&cfg, 0, sizeof cfg);
  cfg.generic = 1;
  qknr_launch_info info;
  memset(&info, 0, sizeof info);
  rc = qknr_inplace_ex(dq, dk, dwq, dwk, (const float*)dc, dp, T, (int32_t)Hq, (int32_t)Hkv,
                       (int32_t)D, (int32_t)R, (int32_t)neox, eps, Hq * D * 2, D * 2,
                       Hkv * D * 2, D * 2, (int32_t)dtype, (int32_t)pos_dtype, s, &cfg, &info);
  if (rc != QKNR_OK) {
    fprintf(stderr, "qknr_inplace_ex: %s\n", qknr_status_string(rc));
    return 6;
  }
  CHECK_HIP(hipStreamSynchronize(s));
  CHECK_HIP(hipMemcpy(out + bytes_q + bytes_k, dq, bytes_q, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(out + 2 * bytes_q + bytes_k, dk, bytes_k, hipMemcpyDeviceToHost));
  printf("launch: generic=%d lanes_per_head=%d elems_per_lane=%d groups_per_item=%d "
         "block_threads=%d grid_blocks=%d items=%lld\n", info.generic, info.lanes_per_head,
         info.elems_per_lane, info.groups_per_item, info.block_threads, info.grid_blocks,
         (long long)info.items);
  CHECK_HIP(hipStreamDestroy(s));
  hipFree(dq); hipFree(dk); hipFree(dwq); hipFree(dwk); hipFree(dc); hipFree(dp);

  FILE* o = fopen(argv[2], "wb");
  const size_t n_out = 2 * (bytes_q + bytes_k);
  if (!o || fwrite(out, 1, n_out, o) != n_out) {
    fprintf(stderr, "cannot write output\n");
    return 1;
  }
  fclose(o);
  free(out);
  free(host);
  printf("qknr C ABI run ok: T=%lld Hq=%lld Hkv=%lld D=%lld R=%lld neox=%lld\n", (long long)T,
         (long long)Hq, (long long)Hkv, (long long)D, (long long)R, (long long)neox);
  return 0;
}
