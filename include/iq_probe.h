/*
 * iq_probe.h -- measurement helper shipped beside libiq.so, in its own library
 * (libiq_probe.so): a read-only streaming kernel, the bandwidth ceiling that the
 * decode's achieved HBM rate is compared with on the same device.  Not part of
 * the decode path.
 */
#ifndef IQ_PROBE_H
#define IQ_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * iq_probe_stream_read -- reads every byte of buf once (16-byte loads in a
 * grid-stride loop over n_blocks work-groups of 256 threads) and discards the
 * data; sink (4 device bytes) is written when a thread's XOR checksum happens to
 * equal a fixed value, which keeps the loads from being removed (the contents of
 * sink mean nothing).  Asynchronous on stream (NULL: default).
 *   buf       device pointer, 16-byte aligned
 *   bytes     a multiple of 16, > 0
 *   n_blocks  1 .. 65535
 * Returns 0, -1 for invalid arguments, -4 if the launch fails.
 */
int iq_probe_stream_read(const void* buf, int64_t bytes, int32_t n_blocks, void* sink, void* stream);

/*
 * iq_probe_stream_read_nt -- iq_probe_stream_read with non-temporal loads (the
 * cache-policy hint that the decode's loads of the packed cache carry).
 * Arguments and returns as iq_probe_stream_read.
 */
int iq_probe_stream_read_nt(const void* buf, int64_t bytes, int32_t n_blocks, void* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif
