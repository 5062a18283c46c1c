/*
 * ep_probe.h: a measurement aid beside the dispatch / combine library.
 *
 * It is not part of the dispatch / combine path.  It serves callers that
 * report how close the path's kernels come to what this GPU's memory system
 * actually sustains: a plain streaming read, write or copy of a large
 * buffer, with the same 16-byte accesses the kernels use, either with
 * non-temporal (streaming) cache policy or with plain accesses; and the
 * duration of one kernel of the path, timed by the kernel's own events.
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

/*
 * Kernel timing: the calling thread's next call of ep_get_dispatch_layout,
 * ep_dispatch, ep_layout_dispatch, ep_dispatch_fp8_input or ep_combine that
 * launches kernels records `start` when its first kernel begins executing
 * and `stop` when its last kernel ends (hipExtLaunchKernelGGL's events), so
 * that hipEventElapsedTime(start, stop) is the call's own GPU time, without
 * the gaps that event markers enqueued around a call add.  Both events are
 * caller-created timing events (either may be NULL).  The request is
 * consumed by that call; NULL, NULL cancels it.  Never fails (EP_OK).
 */
ep_status_t ep_time_next_kernel(hipEvent_t start, hipEvent_t stop);

#ifdef __cplusplus
}
#endif

#endif /* EP_PROBE_H */
