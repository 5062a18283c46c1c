/*
 * ep_probe.h: a measurement aid beside the dispatch / combine library.
 *
 * It is not part of the dispatch / combine path.  It serves callers that
 * report how close the path's kernels come to what this GPU's memory system
 * actually sustains: a plain streaming read, write or copy of a large
 * buffer, with the same 16-byte accesses the kernels use, either with
 * non-temporal (streaming) cache policy or with plain accesses.
 */
#ifndef EP_PROBE_H
#define EP_PROBE_H

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ep.h"

#ifdef __cplusplus
extern "C" {
#endif

enum {
  EP_PROBE_READ = 0,  /* read `bytes` of src (nothing is written) */
  EP_PROBE_WRITE = 1, /* write `bytes` of dst (src unused, may be NULL) */
  EP_PROBE_COPY = 2   /* copy `bytes` from src to dst */
};

/*
 * Enqueues one pass of the chosen kind on `stream` and returns without
 * waiting.  src and dst are caller-owned device pointers, 16-byte aligned;
 * bytes is a positive multiple of 16.  nontemporal != 0 uses streaming
 * loads and stores.  workgroups (1 .. 2^20) of 256 threads walk the buffer
 * with a grid-wide stride, four 16-byte accesses per thread in flight.  The
 * caller times the pass (events on the same stream) and counts bytes (read),
 * bytes (write) or 2 * bytes (copy) as moved.
 * Returns EP_ERR_INVALID_ARG (nothing enqueued) for a bad kind, workgroup
 * count, size, alignment or NULL pointer, EP_ERR_HIP if the launch fails,
 * else EP_OK.
 */
ep_status_t ep_hbm_probe(int32_t kind, int32_t nontemporal, int32_t workgroups, const void *src,
                         void *dst, size_t bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* EP_PROBE_H */
