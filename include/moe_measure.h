/*
 * moe_measure.h -- measurement helpers of the MoE layer library.  Not part
 * of the layer: they exist so that a benchmark can put the layer's HBM rate
 * next to what a plain read stream reaches on the same GPU.
 */
#ifndef MOE_MEASURE_H_
#define MOE_MEASURE_H_

#include <stddef.h>
#include <stdint.h>

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Enqueues on `stream` one read of `bytes` of device memory at `src` (16-byte
 * aligned, bytes a multiple of 16), spread over `blocks` workgroups of 256
 * threads (1 .. 65536) whose waves each read whole 4 KB runs (four 1 KB loads
 * in flight), the runs dealt to the waves round-robin, and XOR-fold what they
 * read into *sink (one
 * device word, caller-owned, which the call XORs into and does not clear).
 * The fold keeps the loads from being optimised away and lets a test check
 * that every byte was read: starting from 0, *sink ends as the XOR of all
 * 32-bit words of the buffer.  Nothing else is written.  Argument errors
 * return MOE_ERR_INVALID_ARG before anything is enqueued. */
moe_status moe_hbm_read_probe(const void *src, size_t bytes, uint32_t *sink, int32_t blocks, moe_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MEASURE_H_ */
