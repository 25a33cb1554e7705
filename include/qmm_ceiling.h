/*
 * qmm_ceiling.h -- measurement kernels (libqmm_ceiling.so), separate from
 * libqmm: they set the floor a single launch of the decode GEMV's size can
 * reach on the GPU, and are used by the benchmark only.
 *
 * All pointers are device pointers owned by the caller; work is queued on
 * `stream` (a hipStream_t as void*, NULL = default stream). Return 0 on
 * success, 1 for a rejected argument (nothing launched), 2 for a launch
 * error.
 */
#ifndef QMM_CEILING_H
#define QMM_CEILING_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` (a positive multiple of 16) from `src` (16-byte aligned) in
 * one launch of `blocks` workgroups of `threads` threads (a multiple of 64,
 * at most 1024), 16-byte nontemporal loads; writes one uint32 per workgroup
 * to `sink` ([blocks]). */
int qmm_ceiling_read(const void* src, int64_t bytes, void* sink, int blocks, int threads,
                     void* stream);

/* Launch `blocks` workgroups of `threads` threads of an empty kernel. */
int qmm_ceiling_empty(int blocks, int threads, void* stream);

#ifdef __cplusplus
}
#endif

#endif
