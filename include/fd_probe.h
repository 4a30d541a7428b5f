/*
 * fd_probe.h -- a measurement aid in the same library as fd_attn.h (AMD
 * MI355X, gfx950); not part of the method the other headers implement.
 *
 * fd_probe_read measures how fast this GPU can move the bytes of a decode
 * call's units with a decode kernel's own load pattern, and nothing else.
 * For each unit it streams the unit's bytes of two buffers (the K and the V
 * cache) into LDS and computes nothing: one workgroup per unit; the unit's
 * groups of K and V bytes are dealt to the workgroup's wavefronts in turn,
 * and each wavefront moves its groups through a ring of LDS stages with 1 KiB
 * non-temporal DMA instructions (buffer-to-LDS on a contiguous cache,
 * global-to-LDS through the page list on a paged one) -- the instructions and
 * cache policy of the decode kernels.  Timed over the units of a decode call
 * (in that kernel's unit order), it gives the rate that call's loads can
 * reach on the device, beside which the decode kernel's own rate (which also
 * computes, stores partials and merges) is read.
 *
 *   k, v        device buffers holding every unit's bytes, 16-byte aligned
 *   units       device array of num_units {offset, bytes}.  Contiguous
 *               (pages NULL): the unit reads [offset, offset + bytes) of k
 *               and of v, offset a multiple of 16; bytes past its end are
 *               never read (the DMA's buffer range ends there).  Paged: the
 *               unit's pages are pages[offset .. offset + n), n =
 *               ceil(bytes / page_bytes), at most 64 (pages past the 64th
 *               are not read), and its pages are read whole
 *   num_units   >= 0; 0 enqueues nothing; at most 2^31 - 1
 *   pages       NULL, or a device array of byte offsets into k and v, each
 *               the start of a page of page_bytes bytes, 16-byte aligned
 *   page_bytes  paged only: a multiple of 1024, at most 2^20
 *   shape       the ring: 0 = 4 wavefronts x 2 stages of 8 KiB (the grouped
 *               bf16 kernel's shape 0, 64 KiB of LDS, two workgroups per
 *               compute unit), 1 = 4 x 3 stages of 8 KiB (its shape 1, 96 KiB,
 *               one), 2 = 2 x 3 stages of 4 KiB (the bytes in flight of the
 *               cooperative kernel's shared ring of 3 x 8 KiB, 24 KiB, six)
 *   sink        device uint32_t that the kernel may write (so the compiler
 *               keeps the loads); its value means nothing
 *   stream      hipStream_t, or NULL for the null stream
 *
 * Ownership: every pointer is the caller's; nothing is allocated.  The
 * caller guarantees that every unit (and, paged, every page offset) lies
 * inside both buffers: they sit in device memory and are not checked.
 * Returns FD_OK, FD_ERR_NULL (k, v, sink, or units with num_units > 0),
 * FD_ERR_SHAPE (num_units < 0, shape not 0..2, or with pages a page_bytes
 * that is not a multiple of 1024 in [1024, 2^20]), FD_ERR_ALIGN (k or v not
 * 16-byte aligned) or FD_ERR_LAUNCH; asynchronous on `stream`.
 */
#ifndef FD_PROBE_H
#define FD_PROBE_H

#include <stdint.h>

#include "fd_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    uint64_t offset;   /* contiguous: bytes from the start of k (and v); paged: first entry in pages */
    uint32_t bytes;    /* bytes of the unit in each buffer */
    uint32_t reserved; /* 0 */
} fd_probe_unit_t;

int fd_probe_read(const void *k, const void *v, const fd_probe_unit_t *units, int32_t num_units,
                  const uint64_t *pages, int32_t page_bytes, int32_t shape, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif
