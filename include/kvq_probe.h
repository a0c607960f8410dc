/*
 * kvq_probe.h — a measurement aid of libkvq, no part of the method: a plain
 * streaming read of a device buffer on AMD Instinct MI355X (gfx950), whose
 * time gives the HBM read rate this GPU reaches with simple wide loads.  The
 * benchmark reports it beside the decode kernel's rate as the practical
 * ceiling for a read-only stream (the published peak is the other reference).
 * Conventions (status codes, streams, alignment) are those of kvq.h.
 */
#ifndef KVQ_PROBE_H_
#define KVQ_PROBE_H_

#include "kvq.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Reads bytes bytes of buf (device memory, 16-byte aligned; bytes a positive
 * multiple of 16) with 16-byte loads from a grid of resident waves, and
 * writes one word per wave into sink (device, at least
 * kvq_probe_sink_words() uint32 entries) so that no load can be dropped.
 * Enqueues one kernel on stream. */
int kvq_probe_stream_read(const void *buf, size_t bytes, uint32_t *sink, void *stream);
/* Entries sink must hold. */
int kvq_probe_sink_words(int32_t *words);

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* KVQ_PROBE_H_ */
