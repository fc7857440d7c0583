/*
 * sparse_decode_timeline.h - extra export of the measurement build of
 * libsparse_decode.so (libsparse_decode_timeline.so, compiled with
 * SD_TIMELINE).  The product library does not export it.
 *
 * In that build the one-launch step (sparse_decode_step) records, per
 * workgroup, wall_clock64() timestamps (a 100 MHz counter common to the
 * device) at the phase boundaries of its role, indexed by the flat workgroup
 * number x + X (y + Y z) of the (KV head, sequence, role) grid, role z < tiles
 * being a score tile, tiles <= z < tiles + P an attention part and
 * z = tiles + P the unit's MAW worker:
 *   score tile:     0 first instruction, 1 keys written, 2 tile list published,
 *                   3 arrived, 4 top-k done (last arriver only), 6 the fast
 *                   top-k gave up (the full top-k runs), 7 the band's exact
 *                   re-score started
 *   attention part: 0 first instruction, 1 dense pages done (wave 0), 2 selection count
 *                   seen, 3 selected pages done (wave 0), 4 partial written
 *                   and arrived, 5 fusion done (last part only), 6 the
 *                   first dense page ids read (wave 0)
 *   MAW worker:     0 first instruction, 6 the parts' and the top-k's
 *                   arrivals seen, 7 the unit's MAW updated
 * Slots not reached stay 0.
 */
#ifndef SPARSE_DECODE_TIMELINE_H
#define SPARSE_DECODE_TIMELINE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Synchronise the device, copy the first `bytes` bytes of the timestamp table
 * ([max_wg][slots] uint64) to host_dst, then zero the whole table.  *slots and
 * *max_wg (if not NULL) receive its shape.  SD_EINVAL (-1) if host_dst is
 * NULL or bytes exceeds the table; SD_EHIP (-3) if a copy fails. */
int32_t sd_timeline_read(void *host_dst, size_t bytes, int32_t *slots, int32_t *max_wg);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_DECODE_TIMELINE_H */
