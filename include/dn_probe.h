/*
 * dn_probe.h -- measurement only (libdn_probe): the device's read-stream and read-modify-write
 * ceilings.
 *
 * The decode step is bound by HBM bandwidth; its achieved rate is reported against the vendor
 * peak and against what a plain streaming read (and, for the batched step's state, an in-place
 * read-modify-write stream) reaches on the same device. This library holds those streams. It is not
 * part of the decode path.
 */
#ifndef DN_PROBE_H
#define DN_PROBE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DN_PROBE_MAX_BLOCKS 65536

/* Enqueue one streaming read of `bytes` bytes of device memory at buf (16-byte aligned, bytes a
 * multiple of 16) with `blocks` workgroups of 256 threads, each thread keeping `in_flight` (4, 8 or
 * 16) nontemporal 16-byte loads in flight; each workgroup writes one word of a fold of what it read
 * to sink[block] (device memory of at least `blocks` words). hip_stream: a hipStream_t (NULL = the
 * default stream). Returns 0, -1 (bad arguments) or -3 (launch error). */
int dn_probe_read_stream(const void *buf, size_t bytes, unsigned *sink, int blocks, int in_flight, void *hip_stream);

/* Enqueue one in-place read-modify-write stream over `bytes` bytes of device memory at buf (16-byte
 * aligned, bytes a multiple of 16): every 16-byte piece read with a nontemporal load and written back
 * unchanged (times 1.0f as four floats) with a nontemporal store, `blocks` workgroups of 256 threads,
 * `in_flight` (4, 8 or 16) pieces per thread between a thread's loads and its stores. The state
 * stream of a batched step (each state tile read, updated and written back) is this access pattern.
 * Same arguments and return codes as dn_probe_read_stream otherwise; the buffer's contents are kept
 * (fp32 NaN payloads aside). */
int dn_probe_rmw_stream(void *buf, size_t bytes, int blocks, int in_flight, void *hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* DN_PROBE_H */
