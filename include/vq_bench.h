/*
 * vq_bench.h — a measurement kernel that is not part of the verify pass: the
 * streaming-read ceiling of the GPU's HBM, against which the pass's kernels are
 * compared. Decode, and so the verify pass, is bound by how fast the weights
 * and the KV cache stream from memory (page "The fastest way to run local LLMs
 * on a Mac", section "Decode is a memory-bandwidth problem"); this call reads a
 * buffer and does nothing else, so its rate is what a kernel of the pass could
 * reach at best.
 *
 * Same conventions as vq.h: caller-owned device pointers, asynchronous on
 * `stream`, host-side validation (VQ_ERR_INVALID_ARG), no allocation.
 */
#ifndef VQ_BENCH_H_
#define VQ_BENCH_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` bytes from the device buffer `src` (16-byte aligned, bytes a
 * positive multiple of 16) with coalesced 16-byte loads, ordinary
 * (nontemporal = 0) or with the non-temporal hint (nontemporal = 1), spread
 * over `workgroups` workgroups of 256 threads (1 .. 2^20; workgroup w reads the
 * 16 KiB blocks w, w + workgroups, ...). Each workgroup folds what it read into
 * 4 words written to sink[4w .. 4w + 3] (sink: caller-owned device buffer of at
 * least 4 * workgroups uint32), so that no load can be dropped; their values
 * carry no meaning. */
int vq_stream_read(const void* src, size_t bytes, int nontemporal, int workgroups, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VQ_BENCH_H_ */
