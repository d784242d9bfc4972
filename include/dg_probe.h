/* dg_probe.h — measurement aid for the canvas sampler (libdgprobe.so).
 *
 * The statistics pass is bound by HBM reads: it streams every logit once. Its
 * roofline is stated against the chip's published HBM peak, and beside it
 * against the rate a plain streaming read reaches on the same buffer. This
 * library holds only that plain read, a kernel that loads every 16-byte word of
 * a buffer and folds it into one XOR, so that the time is the read alone. It is
 * not part of the sampling method and the sampler library does not use it.
 */
#ifndef DG_PROBE_H
#define DG_PROBE_H
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

/* dg_probe_stream_read — enqueue one streaming read of `bytes` bytes at `buf`.
 *
 *   buf    device pointer, 16-byte aligned; read only.
 *   bytes  > 0 and a multiple of 16.
 *   grid   workgroups, 1..65536.  block: threads per workgroup, a multiple of
 *          64 in 64..1024. Each thread reads four 16-byte words per round,
 *          grid-stride over the buffer (rounds that would pass the end fall back
 *          to one word at a time).
 *   sink   device pointer to one uint32; written only when the XOR of the
 *          buffer equals 0x9E3779B9 (keeps the loads live; callers ignore it).
 *   stream hipStream_t, borrowed; the call is asynchronous on it.
 *
 * Returns 0 when the kernel was enqueued, 1 for an argument outside the ranges
 * above (nothing is enqueued), 4 when the launch failed.
 */
int dg_probe_stream_read(const void* buf, int64_t bytes, int32_t grid, int32_t block,
                         uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif
