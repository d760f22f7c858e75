/*
 * swin_offload.h - moving the forward pass's saved state to pinned host memory and back,
 * on copy streams of its own (same library as swin_attn.h).
 *
 * [TERRA] section V-C (budget-constrained offloading) and its implementation paragraph: the
 * tensors saved at a checkpoint boundary go to pinned host buffers through asynchronous
 * device-to-host copies when they are saved, and come back through host-to-device copies
 * before the backward needs them. Here the unit is a byte range of device memory, typically
 * the `saved` buffer of swin_attn_fwd or swin_block_fwd, so a caller can drop a module's saved
 * state from HBM between its forward and backward passes while other modules compute.
 *
 * An offload engine owns two streams created at the default priority (one per copy
 * direction, so a store and a load can run at the same time) and a ring of HIP events.
 * Every copy is ordered after all work already enqueued on the caller's stream at the time of
 * the call, and returns a ticket; swin_offload_wait makes a stream wait for a ticket's copy.
 * No call blocks the host except swin_offload_sync, and the ring's reuse of an event (see
 * swin_offload_store). Device memory, host memory and streams belong to the caller; host
 * buffers must be pinned (swin_pinned_alloc, or any hipHostMalloc allocation), so that the
 * copies are asynchronous DMA transfers.
 *
 * An engine belongs to the device that was current when it was created, and calls on it must
 * come from one host thread at a time with that device current.
 *
 * The caller keeps the usual rules of asynchronous copies: do not overwrite or free the
 * device source of a store, or read the device destination of a load, before waiting for its
 * ticket on the stream that does so; do not touch the host buffer until the ticket's copy is
 * complete (swin_offload_query or swin_offload_sync).
 */
#ifndef SWIN_OFFLOAD_H_
#define SWIN_OFFLOAD_H_

#include "swin_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct swin_offload swin_offload;

/* Tickets are positive and increase by one per copy; 0 is never a ticket. */
typedef uint64_t swin_ticket;

/* Creates an engine on the current HIP device: two non-blocking streams at the default
 * priority and `ring` events (0 means 64; at most 4096). Errors: SWIN_ERR_ARG (NULL out, ring
 * out of range), SWIN_ERR_HIP. */
swin_status swin_offload_create(int32_t ring, swin_offload** out);

/* Waits for every copy of the engine, then releases its streams and events. NULL is a no-op. */
void swin_offload_destroy(swin_offload* engine);

/* Pinned (page-locked) host memory for the copies: hipHostMalloc / hipHostFree. bytes > 0.
 * Errors: SWIN_ERR_ARG, SWIN_ERR_HIP (allocation failed). */
swin_status swin_pinned_alloc(size_t bytes, void** host);
swin_status swin_pinned_free(void* host);

/* Device -> host copy of `bytes` bytes from `dev` to `host`, after all work enqueued on
 * `after` (a hipStream_t; NULL = the null stream) so far. *ticket receives the copy's ticket.
 * When the event ring is full, the call first waits on the host for the copy that used the
 * slot `ring` tickets ago (its ticket then counts as complete). `dev` must be device memory of
 * the engine's device and `host` pinned host memory. Errors: SWIN_ERR_ARG (NULL engine,
 * pointer or ticket, bytes == 0, a pointer of the wrong kind, another current device),
 * SWIN_ERR_HIP. */
swin_status swin_offload_store(swin_offload* engine, const void* dev, void* host, size_t bytes, void* after,
                               swin_ticket* ticket);

/* Host -> device copy, otherwise as swin_offload_store. */
swin_status swin_offload_load(swin_offload* engine, const void* host, void* dev, size_t bytes, void* after,
                              swin_ticket* ticket);

/* Makes `stream` (NULL = the null stream) wait for the copy of `ticket` without blocking the
 * host; a ticket whose event slot has been reused is already complete and needs no wait.
 * Errors: SWIN_ERR_ARG (NULL engine, ticket 0 or not issued yet), SWIN_ERR_HIP. */
swin_status swin_offload_wait(swin_offload* engine, swin_ticket ticket, void* stream);

/* *done = 1 if the copy of `ticket` has completed, else 0 (non-blocking). Errors as for
 * swin_offload_wait. */
swin_status swin_offload_query(swin_offload* engine, swin_ticket ticket, int32_t* done);

/* Blocks the host until every copy issued so far has completed. */
swin_status swin_offload_sync(swin_offload* engine);

/* Bytes moved by the engine so far in each direction (for throughput reports). */
swin_status swin_offload_bytes(const swin_offload* engine, uint64_t* stored, uint64_t* loaded);

#ifdef __cplusplus
}
#endif

#endif /* SWIN_OFFLOAD_H_ */
