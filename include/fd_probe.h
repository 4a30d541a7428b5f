/*
 * fd_probe.h -- a measurement aid in the same library as fd_attn.h (AMD
 * MI355X, gfx950); not part of the method the other headers implement.
 *
 * fd_probe_read measures how fast this GPU can move the bytes of a decode
 * call's units with the decode kernels' own load pattern, and nothing else.
 * For each unit it streams `bytes` bytes at `offset` of two buffers (the K
 * and the V cache) into LDS and computes nothing: one workgroup of four
 * wavefronts per unit; the unit's 4 KiB groups of K and V are dealt to the
 * wavefronts in turn, and each wavefront moves its groups through a ring of
 * `stages` LDS stages of 8 KiB (the K group and the V group) with 1 KiB
 * non-temporal buffer-to-LDS DMA instructions -- the instruction, cache
 * policy, stage size and ring depth of the grouped-query bf16 chunk kernel.
 * Timed over the units of a decode call (in that kernel's unit order), it
 * gives the rate that call's loads can reach on the device, beside which the
 * decode kernel's own rate (which also computes, stores partials and merges)
 * is read.
 *
 *   k, v       device buffers holding every unit's bytes, 16-byte aligned
 *   units      device array of num_units {offset, bytes}: the unit reads
 *              [offset, offset + bytes) of k and of v; offset a multiple of
 *              16; bytes past a unit's end are never read (the DMA's buffer
 *              range ends there and returns zeros)
 *   num_units  >= 0; 0 enqueues nothing; at most 2^31 - 1
 *   stages     2 (64 KiB of LDS per workgroup, two per compute unit) or 3
 *              (96 KiB, one per compute unit)
 *   sink       device uint32_t that the kernel may write (so the compiler
 *              keeps the loads); its value means nothing
 *   stream     hipStream_t, or NULL for the null stream
 *
 * Ownership: every pointer is the caller's; nothing is allocated.  The
 * caller guarantees that every unit lies inside both buffers (the offsets sit
 * in device memory and are not checked).  Returns FD_OK, FD_ERR_NULL (k, v,
 * sink, or units with num_units > 0), FD_ERR_SHAPE (num_units < 0 or stages
 * not 2 or 3), FD_ERR_ALIGN (k or v not 16-byte aligned) or FD_ERR_LAUNCH;
 * asynchronous on `stream`.
 */
#ifndef FD_PROBE_H
#define FD_PROBE_H

#include <stdint.h>

#include "fd_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    uint64_t offset;   /* bytes from the start of k (and of v) */
    uint32_t bytes;    /* bytes of the unit in each buffer */
    uint32_t reserved; /* 0 */
} fd_probe_unit_t;

int fd_probe_read(const void *k, const void *v, const fd_probe_unit_t *units, int32_t num_units,
                  int32_t stages, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif
