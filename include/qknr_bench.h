/*
 * qknr_bench.h -- measurement aids shipped in libqknr.so beside the op.
 *
 * They are not part of the QK RMSNorm + RoPE operation. The benchmark uses
 * them to put its numbers in context on the same GPU:
 *   - qknr_copy streams `bytes` from src to dst; its hardware counters
 *     (bytes fetched from and written to memory) calibrate the counter runs
 *     of the op, since it moves a known number of bytes;
 *   - qknr_rmw reads, XORs with `key` and writes back `bytes` in place: the
 *     same read-then-overwrite pattern as the op with no arithmetic, i.e. the
 *     practical bandwidth ceiling of an in-place stream. key == 0 leaves the
 *     buffer's contents unchanged.
 * Both use 16-byte accesses with the op's cache policies (nontemporal loads;
 * nontemporal, agent-scope stores): pointers must be 16-byte aligned and bytes a
 * multiple of 16 (else QKNR_E_ALIGN); bytes < 0 gives QKNR_E_SHAPE, bytes == 0
 * is a no-op. Asynchronous on `stream`; the caller owns all memory.
 */
#ifndef QKNR_BENCH_H
#define QKNR_BENCH_H

#include "qknr.h"

#ifdef __cplusplus
extern "C" {
#endif

QKNR_API int32_t qknr_copy(void* dst, const void* src, int64_t bytes, hipStream_t stream);
QKNR_API int32_t qknr_rmw(void* buf, int64_t bytes, uint32_t key, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QKNR_BENCH_H */
