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

#ifdef __cplusplus
}
#endif

#endif /* REPLAYSSM_PROBE_H */
