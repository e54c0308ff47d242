/*
 * Measurement aid for the benchmark, in its own library (libqsa_probe.so); not part
 * of the QSA computation and not exported by libqsa.so.
 *
 * The gather ceiling of the memory system for the access pattern of the sparse
 * attention's kept-token gather: n_waves waves each read `steps` x 4 blocks of
 * 4 KiB from buf, block j of wave w step s at buf + 4096 * block_ids[(w*steps+s)*4+j];
 * the data is folded into a value written to sink[0..1023] only in a never-taken
 * case.
 *   buf        device buffer of buf_bytes bytes (16-byte aligned)
 *   block_ids  device int32 [n_waves * steps * 4]; every id must be < buf_bytes / 4096
 *              (the caller checks this: the kernel does not)
 *   sink       device uint32 [1024]
 *   stream     hipStream_t the launch is enqueued on
 * Bytes read per call: n_waves * steps * 16384. Returns 0 on success, 1 for a bad
 * argument (null or misaligned pointer, negative size), 4 when the launch fails.
 *
 * The write-stream ceiling for the score GEMM's output: qsa_probe_write fills the
 * first `bytes` bytes of buf with 16-byte float values, each wave instruction writing
 * 1 KiB of consecutive bytes, with the non-temporal hint when nontemporal != 0.
 *   buf     device buffer, 16-byte aligned; bytes a multiple of 16
 *   stream  hipStream_t the launch is enqueued on
 * Returns 0 on success, 1 for a bad argument, 4 when the launch fails.
 */
#ifndef QSA_PROBE_H
#define QSA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int qsa_probe_gather(const void* buf, size_t buf_bytes, const int32_t* block_ids,
                     int64_t n_waves, int steps, uint32_t* sink, void* stream);

int qsa_probe_write(void* buf, size_t bytes, int nontemporal, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QSA_PROBE_H */
