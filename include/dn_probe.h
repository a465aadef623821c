/*
 * dn_probe.h -- measurement only (libdn_probe): the device's read-stream and read-modify-write
 * ceilings.
 *
 * The decode step is bound by HBM bandwidth; its achieved rate is reported against the vendor
 * peak and against what a plain streaming read (and, for the batched step's state, an in-place
 * read-modify-write stream) reaches on the same device. This library holds those streams, and a
 * probe of the latency of a hand-off between workgroups, which bounds the whole-stack decode kernel
 * (three hand-offs per layer). It is not part of the decode path.
 */
#ifndef DN_PROBE_H
#define DN_PROBE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DN_PROBE_MAX_BLOCKS 65536
#define DN_PROBE_XCHG_MAX_WG 1024

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

/* Enqueue one hand-off latency measurement on `nwg` workgroups of 768 threads, which must all be
 * resident at once (one per compute unit on an otherwise idle device; every wait is bounded, so a
 * grid that cannot be resident ends with *err counted instead of hanging). Words are stored with
 * relaxed device-scope atomics and polled with device-coherent loads, as the whole-stack kernel's
 * hand-offs are. Times are in ticks of the 100 MHz device clock.
 *   mode 0 (ping): workgroups 0 and `arg` (0 < arg < nwg) pass a round number back and forth
 *     `rounds` times; ticks[0] receives workgroup 0's time for all of them (a one-way hand-off is
 *     ticks[0] / (2 rounds)). words: at least 1024 bytes.
 *   mode 1 (all-gather): every workgroup contributes arg / nwg words, stored as 16-byte stores into
 *     eight replicas (one per XCD), and polls all `arg` words of its own XCD's replica, `rounds`
 *     times (rounds alternate between two sets of replicas); ticks[w] receives workgroup w's time.
 *     arg: 1024, 2048, 4096 or 8192, a multiple of 4 nwg, with 2 arg / nwg <= 64. words: at least
 *     2 * 8 * arg * 4 bytes. ticks: nwg entries.
 * words must be zero and 16-byte aligned on entry (the caller clears it before every call).
 * stream_in_flight: 0, or 1..4 to have eight waves of every workgroup stream nontemporal 16-byte
 * reads over stream_buf (16-byte aligned, at least nwg * 8 KiB) with that many loads in flight per
 * lane while the measurement runs, as the whole-stack kernel's weight prefetch does. err: one device
 * word, incremented for every wave whose bounded wait ran out. sink: nwg * 8 device words. Returns
 * 0, -1 (bad arguments) or -3 (launch error). */
int dn_probe_exchange(int mode, int arg, int rounds, int stream_in_flight, unsigned *words, size_t words_bytes,
                      const void *stream_buf, size_t stream_bytes, unsigned long long *ticks, unsigned *err,
                      unsigned *sink, int nwg, void *hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* DN_PROBE_H */
