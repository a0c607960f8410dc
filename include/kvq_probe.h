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

/* The same read in a chosen launch shape, for sweeping the read rate against
 * the bytes a wave keeps in flight: waves_per_simd x 4 x (compute units)
 * single-wave workgroups (1 <= waves_per_simd <= 8), each reading one
 * contiguous share in batches of loads_per_lane (1, 2, 4, 8 or 16) 16-byte
 * loads per lane, with the next batch requested before the current one is
 * used.  nontemporal selects the load: 0 plain, 1 nontemporal, 2 nontemporal
 * direct loads into LDS (global_load_lds_dwordx4, each batch read back from
 * LDS), 3 plain direct loads into LDS (KVQ_ERR_RANGE otherwise; for 2 and 3
 * bytes must be a multiple of 1024).  Waves beyond what
 * the GPU keeps resident run after the first ones finish.  Status codes and
 * sink as kvq_probe_stream_read. */
int kvq_probe_stream_read_sweep(const void *buf, size_t bytes, uint32_t *sink,
                                int32_t waves_per_simd, int32_t loads_per_lane,
                                int32_t nontemporal, void *stream);

/* The decode partial kernel's load stream without its arithmetic, for
 * telling a kernel bound by its loads from one bound by its instructions:
 * n_chunks chunks of four pieces, piece i of chunk c being bytes_i bytes at
 * buf_i + c * bytes_i (buf_i device memory of n_chunks * bytes_i bytes,
 * 16-byte aligned, owned by the caller and only read; each bytes_i a
 * multiple of 512, the four summing to at most 4096), each chunk brought into
 * a per-wave ring of two LDS slots with nontemporal direct loads
 * (global_load_lds_dwordx4, 1 KB per instruction, a 512-byte rest with half
 * the lanes), the next chunk requested before the current one is read back,
 * then spin dependent fp32 multiply-adds (0 <= spin <= 4096) standing in for
 * the per-chunk arithmetic.  2 x 4 x (compute units) single-wave workgroups,
 * each a contiguous share of the chunks.  Returns KVQ_ERR_RANGE for sizes
 * outside these bounds; status codes and sink as kvq_probe_stream_read. */
int kvq_probe_chunk_stream(const void *buf_a, const void *buf_b, const void *buf_c,
                           const void *buf_d, int64_t n_chunks, int32_t bytes_a,
                           int32_t bytes_b, int32_t bytes_c, int32_t bytes_d, int32_t spin,
                           uint32_t *sink, void *stream);

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* KVQ_PROBE_H_ */
