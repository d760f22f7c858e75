/*
 * swin_route.h - TERRA's token routes between rank layouts, as the single-GPU pieces a
 * multi-rank run is built from: per-destination packing, the exchange of the packed
 * segments (here a loopback on one device), and the restore at the destinations.
 * Same library and conventions as swin_attn.h.
 *
 * [TERRA] section IV-D: a token's global grid coordinate fixes where it lives in each layout.
 * Under the DMP stripe layout that is a source rank and an offset in the rank's spatial
 * stripe; under a window assignment it is the rank that owns the token's window and the
 * token's offset in that rank's window-major tensor. Tokens bound for one destination are
 * gathered into a contiguous send buffer, the buffers are exchanged peer to peer, and every
 * destination puts each received token at its offset. The shift route is the same mechanism
 * between the unshifted and the shifted window partitions, and the backward of a route is the
 * route with source and destination swapped.
 * [TERRA] section V-A, Eq. 4: with M windows in row-major order (batch, level, lat, lon),
 * window rank r of R owns the contiguous range [floor(r M / R), floor((r + 1) M / R)).
 *
 * Layouts (a route goes from one to another; any pair is allowed):
 *   SWIN_LAYOUT_STRIPES  rank p of P holds latitude rows [floor(p H / P), floor((p + 1) H / P))
 *                        of every batch element and level, as a grid-order [B, D, H_p, W, C]
 *                        tensor (the same split as Eq. 4, applied to rows).
 *   SWIN_LAYOUT_WINDOWS  the window partition of the descriptor's grid and window under the
 *                        layout's shift (ragged edge windows included), rank r holding the
 *                        windows of Eq. 4 window-major, rows in window order, row-major inside
 *                        a window: the rank's slice of the window-major tensor of swin_attn.
 * Buffers: the send buffer of source p holds its tokens for destination 0, then 1, ...,
 * each segment in destination-offset order; the receive buffer of destination r is the
 * concatenation of the segments (p -> r) over p = 0, 1, ... All rows are C elements of the
 * descriptor's dtype.
 */
#ifndef SWIN_ROUTE_H_
#define SWIN_ROUTE_H_

#include "swin_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

enum { SWIN_LAYOUT_STRIPES = 0, SWIN_LAYOUT_WINDOWS = 1 };

typedef struct swin_rank_layout {
  int32_t kind;      /* SWIN_LAYOUT_STRIPES or SWIN_LAYOUT_WINDOWS */
  int32_t ranks;     /* >= 1; SWIN_LAYOUT_STRIPES also needs ranks <= H */
  int32_t shift[3];  /* SWIN_LAYOUT_WINDOWS: shift of the partition, 0 <= shift < window; else 0 */
} swin_rank_layout;

typedef struct swin_route_plan swin_route_plan;

/* Plans the route from layout src to layout dst over the token grid of `grid`: its ndim,
 * dtype, batch, grid, channels, window and periodic fields are used (shift, heads and scale
 * are ignored; the window layouts carry their own shifts). Uploads the index tables (4 bytes
 * per token per side). Errors: SWIN_ERR_ARG (an invalid descriptor or layout),
 * SWIN_ERR_UNSUPPORTED (more than 2^31 - 1 tokens), SWIN_ERR_HIP. */
swin_status swin_route_plan_create(const swin_attn_desc* grid, const swin_rank_layout* src,
                                   const swin_rank_layout* dst, swin_route_plan** out);
void swin_route_plan_destroy(swin_route_plan* plan);

/* Route sizes: counts[p * R + r] = tokens sent from source p to destination r, src_sizes[p]
 * and dst_sizes[r] = tokens each rank holds. Any output may be NULL. */
swin_status swin_route_counts(const swin_route_plan* plan, int64_t* counts, int64_t* src_sizes, int64_t* dst_sizes);

/* Host-only tables of the same route (no device needed): counts as above, send_src (the
 * local source offset of every send-buffer row, sources in rank order, n_tokens entries) and
 * recv_dst (the local destination offset of every receive-buffer row, destinations in rank
 * order). Any output may be NULL. */
swin_status swin_route_host_tables(const swin_attn_desc* grid, const swin_rank_layout* src,
                                   const swin_rank_layout* dst, int64_t* counts, int32_t* send_src,
                                   int32_t* recv_dst);

/* Pack for source rank p: send[i] = local[send_src_p[i]] (rows), every destination's segment
 * in order. local holds src_sizes[p] rows, send the same number; no aliasing. Errors:
 * SWIN_ERR_ARG (NULL plan or pointer, p out of range, aliasing), SWIN_ERR_HIP. */
swin_status swin_route_pack(const swin_route_plan* plan, int32_t p, const void* local, void* send, void* stream);

/* Restore for destination rank r: local[recv_dst_r[i]] = recv[i]. recv and local hold
 * dst_sizes[r] rows; no aliasing. Errors as for swin_route_pack. */
swin_status swin_route_unpack(const swin_route_plan* plan, int32_t r, const void* recv, void* local, void* stream);

/* The exchange on one device (loopback in place of the peer-to-peer transfers): for every
 * (p, r) with tokens, copies segment (p -> r) of send[p] to its place in recv[r]. send is an
 * array of P device pointers, recv of R; a rank with no tokens may pass NULL. Errors:
 * SWIN_ERR_ARG (NULL arrays, a NULL buffer that has tokens), SWIN_ERR_HIP. */
swin_status swin_route_loopback(const swin_route_plan* plan, const void* const* send, void* const* recv, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SWIN_ROUTE_H_ */
