/* s4kv_probe.h -- measurement aid of libs4kv.so (not part of the cache path).
 *
 * The decode kernels stream every cache byte exactly once, chunk by chunk,
 * from pages scattered by the page table (the paged layout of the
 * PagedAttention explainers: gyaansetu.com "KV-Cache und PagedAttention",
 * section "Wie PagedAttention das loest"; polaris7.io signal page). This probe
 * reads chunks the same way with nothing else attached, so a benchmark can set
 * a decode kernel's rate against what the load path itself sustains on the
 * device at hand.
 */
#ifndef S4KV_PROBE_H_
#define S4KV_PROBE_H_

#include <stddef.h>
#include <stdint.h>

#include "s4kv.h"

#ifdef __cplusplus
extern "C" {
#endif

#define S4KV_PROBE_CHUNK_BYTES 4096 /* bytes read per chunk id */

/* Read chunks of a device buffer with the decode kernels' load path.
 *
 * waves one-wave work-groups; wave w reads the 4096-byte chunks
 * chunk_ids[w * chunks_per_wave .. (w + 1) * chunks_per_wave - 1] of pool,
 * each with four 16-byte-per-lane DMA loads into LDS (content discarded),
 * waiting for each chunk before the next is issued, as a one-stage ring.
 *
 * Args:
 *   pool             device buffer, pool_bytes long (read only).
 *   chunk_ids        device int32 [waves * chunks_per_wave]; an id whose chunk
 *                    would end past pool_bytes (or is negative) is skipped.
 *   non_temporal     host int: nonzero sets the non-temporal load policy, as
 *                    the decode kernels do.
 *   stream           hipStream_t (NULL: default stream); the call is
 *                    asynchronous.
 * Returns S4KV_OK; S4KV_ERR_INVALID_ARG for null pointers or non-positive
 * sizes; S4KV_ERR_HIP if the launch fails. */
s4kv_status s4kv_probe_read(const void* pool, size_t pool_bytes, const int32_t* chunk_ids,
                            int32_t chunks_per_wave, int32_t waves, int32_t non_temporal,
                            void* stream);

#ifdef __cplusplus
}
#endif

#endif /* S4KV_PROBE_H_ */
