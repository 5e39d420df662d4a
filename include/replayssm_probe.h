/*
 * replayssm_probe.h: streaming kernels that calibrate the HBM bandwidth the
 * ReplaySSM kernels are measured against.  They move the same 32 KiB per
 * workgroup with the same 16-byte loads as one checkpoint tile.
 *
 * Not part of the method; used by the benchmark to report the fraction of the
 * measured streaming ceiling next to the fraction of the published peak.
 * All pointers are device pointers; work goes on `stream`; the return value is
 * 0 or RSSM_ERR_* from replayssm.h.
 */
#ifndef REPLAYSSM_PROBE_H
#define REPLAYSSM_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Number of floats `sink` must hold for rssm_probe_read of `bytes` bytes. */
size_t rssm_probe_sink_elems(size_t bytes);

/* Read `bytes` (a multiple of 32768) from src.  sink (one float per 32 KiB
 * block) is only written if a block's words xor to a fixed pattern, which
 * keeps the loads alive without adding traffic. */
int rssm_probe_read(const void *src, size_t bytes, float *sink, void *stream);

/* Copy `bytes` (a multiple of 32768) from src to dst (non-overlapping). */
int rssm_probe_copy(void *dst, const void *src, size_t bytes, void *stream);

/* The flush's stochastic rounding of an FP16 checkpoint (RSSM_F16), applied to
 * src[0 .. n) fp32 -> dst[0 .. n) fp16 bits: value i is rounded with random
 * word i % 4 of Philox4x32-10 (Salmon et al., "Parallel random numbers: as
 * easy as 1, 2, 3", SC 2011) at counter (v low 32 bits, v high 32 bits, 0, 0),
 * v = vec0 + i / 4, under the key (seed low, seed high): exactly the words the
 * flush uses for checkpoint elements 4 v .. 4 v + 3 (row-major over the whole
 * checkpoint) with rssm_params.sr_seed = seed.  n a multiple of 4; src 16-byte
 * and dst 8-byte aligned, else RSSM_ERR_SHAPE.  Used by tests to pin the
 * rounding against a host implementation. */
int rssm_probe_sr_f16(const float *src, uint16_t *dst, size_t n, uint64_t vec0, uint64_t seed, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* REPLAYSSM_PROBE_H */
