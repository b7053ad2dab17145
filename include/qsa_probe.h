/*
 * qsa_probe.h -- memory-traffic probes of libqsa: kernels that only load
 * bytes, for setting a kernel of the step against what its access pattern
 * alone costs on the device.  They compute nothing of the method.
 *
 * Conventions are those of qsa.h (device pointers owned by the caller,
 * validation before any enqueue, QSA_* return codes, no allocation, no
 * synchronisation).  Each probe XOR-folds every 32-bit word it loads into
 * sink_dev[wavefront % n_sink] (each wavefront into its own word when n_sink
 * is at least the number of wavefronts -- at most 8192 for the stream read,
 * ceil(n_q/8)*8*n_head_kv*4 for the gather -- atomically otherwise), so the
 * XOR of the n_sink words after the call is the XOR of all words loaded
 * (XOR'ed into what the sink held).  Calls that share a sink must not
 * overlap.
 */
#ifndef QSA_PROBE_H
#define QSA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "qsa.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Read n_bytes of src_dev once, 16 bytes per load.  nontemporal != 0 marks
 * the loads as streaming (they do not displace cached data).
 *   src_dev   16-byte aligned; n_bytes a multiple of 16 (0: nothing enqueued)
 *   sink_dev  n_sink >= 1 uint32, 4-byte aligned
 * QSA_EINVAL on a NULL or misaligned pointer, n_bytes not a multiple of 16,
 * or n_sink < 1.
 */
int qsa_probe_stream_read(const void *src_dev, size_t n_bytes, int32_t nontemporal,
                          uint32_t *sink_dev, int32_t n_sink, void *stream);

/*
 * The K/V row gather of qsa_sparse_attn_prefill over a q8_0 cache without
 * its arithmetic: the same grid, work split and loads (each query's listed
 * cells, both KV rows of every slot of its 32-cell chunks; padding slots of a
 * last chunk and cells not present read the sequence's cell 0).  Arguments
 * as qsa_sparse_attn_prefill, without the queries, output and workspace,
 * and with the same validation.  QSA_ENOTSUP unless dims->kv_type is
 * QSA_KV_Q8_0 and the sequences have no cell table.
 */
int qsa_probe_gather_prefill(const qsa_dims *dims, const qsa_seqs *seqs,
                             const int32_t *q_seq_dev, int32_t n_q, const void *k_cache_dev,
                             const void *v_cache_dev, const int32_t *sel_cells_dev,
                             const int32_t *n_sel_dev, uint32_t *sink_dev, int32_t n_sink,
                             void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QSA_PROBE_H */
