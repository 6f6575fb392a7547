/*
 * dah_probe.h -- memory-system probes used by the benchmark, not part of the
 * attention path.  They give two reference points for the decode kernel's
 * roofline on the same device:
 *
 *   dah_probe_copy  a plain copy of `bytes` bytes with 16-byte vector loads
 *                   and stores: a kernel of exactly known traffic (bytes read,
 *                   bytes written), used to calibrate hardware byte counters;
 *   dah_probe_read  a streaming read of `bytes` bytes with the same 16-byte
 *                   non-temporal loads the decode kernel issues: the highest
 *                   read bandwidth a plain kernel reaches, i.e. the practical
 *                   ceiling under the 8 TB/s HBM peak.
 *
 * Pointers are device pointers, 16-byte aligned; `bytes` must be a positive
 * multiple of 16.  `sink` receives one word per workgroup (at least
 * `sink_words` words; dah_probe_read uses min(sink_words, 65536) workgroups).
 * Calls are asynchronous on `stream` (a hipStream_t) and return a dah_status
 * value (include/dah.h): DAH_ERR_NULL, DAH_ERR_SHAPE, DAH_ERR_ALIGN or
 * DAH_ERR_HIP on failure.
 */
#ifndef DAH_PROBE_H
#define DAH_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int dah_probe_copy(const void* src, void* dst, size_t bytes, void* stream);
int dah_probe_read(const void* src, size_t bytes, uint32_t* sink, int sink_words, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DAH_PROBE_H */
