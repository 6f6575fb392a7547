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
 *                   ceiling under the 8 TB/s HBM peak;
 *   dah_probe_paged_read  the cached pages of a batch read through the block
 *                   table in the decode kernel's arrangement and nothing else
 *                   (one workgroup of 8 waves per sequence, wave g reading KV
 *                   head g's K and V tiles of each of the sequence's
 *                   ceil(seq_lens[b] / 16) pages, two pages in flight): the
 *                   ceiling of that access pattern.  Pools, block table and
 *                   lengths as for paged_decode_gqa (include/dah.h); page ids
 *                   outside the pool read page 0, lengths outside
 *                   1 .. max_seq_len read nothing; `sink` receives B * 8 words.
 *
 * Pointers are device pointers, 16-byte aligned (block tables, lengths and
 * sinks 4-byte aligned); `bytes` must be a positive multiple of 16.
 * dah_probe_read's `sink` receives one word per workgroup (at least
 * `sink_words` words; it uses min(sink_words, 65536) workgroups).
 * Calls are asynchronous on `stream` (a hipStream_t) and return a dah_status
 * value (include/dah.h): DAH_ERR_NULL, DAH_ERR_SHAPE, DAH_ERR_DTYPE, DAH_ERR_ALIGN
 * or DAH_ERR_HIP on failure.
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
int dah_probe_paged_read(const void* k_cache, const void* v_cache, int cache_dtype,
                         int64_t num_pages, const int32_t* block_table, int max_pages_per_seq,
                         const int32_t* seq_lens, int B, int max_seq_len, uint32_t* sink,
                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DAH_PROBE_H */
