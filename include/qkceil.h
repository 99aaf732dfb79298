/*
 * qkceil.h -- C ABI of libqkceil: measurement kernels that bound what any
 * kernel moving the same bytes can reach on this GPU. They perform no part
 * of the normalisation; the benchmark times them beside the QK-Norm kernels,
 * under the same launch gating, so that a QK-Norm time can be read against
 * the fastest plain stream of its bytes.
 *
 * The QK-Norm pass reads every row once and writes it once (SwiftQK
 * technical review, Algorithm 1: only the normalised shard is written out),
 * so its practical ceiling is a copy of the same bytes; the read-only and
 * write-only streams split that copy into its two directions, and the empty
 * launch is the fixed cost every launch pays before and after its work.
 *
 * Conventions
 *  - Memory: device pointers owned by the caller; nothing is allocated.
 *  - `bytes` is a multiple of 16 and at most 2^35; pointers are 16-byte
 *    aligned. bytes == 0 returns QKCEIL_OK without a launch.
 *  - `vectors_per_lane` (1, 2, 4 or 8) sets the work per workgroup of 256
 *    lanes: each lane moves that many 16-byte vectors, all loads issued
 *    before any store, with non-temporal (streaming) cache policy, as the
 *    QK-Norm kernels move rows.
 *  - `stream` is a hipStream_t (NULL = the null stream) on the current
 *    device. Calls only enqueue work.
 *  - Errors: QKCEIL_OK (0) or a negative code; arguments are checked on the
 *    host before any HIP call.
 */
#ifndef QKCEIL_H
#define QKCEIL_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QKCEIL_OK = 0,
    QKCEIL_ERR_NULL = -1,    /* a required pointer is NULL                       */
    QKCEIL_ERR_SIZE = -2,    /* bytes not a multiple of 16, or above 2^35        */
    QKCEIL_ERR_ALIGN = -3,   /* a pointer is not 16-byte aligned                 */
    QKCEIL_ERR_CONFIG = -4,  /* vectors_per_lane is not 1, 2, 4 or 8; or
                                workgroups is 0                                  */
    QKCEIL_ERR_DEVICE = -5   /* the launch failed                                */
} qkceil_status;

/* dst[0, bytes) = src[0, bytes). src and dst must not overlap.
 * Status: QKCEIL_ERR_NULL, _SIZE, _ALIGN, _CONFIG, _DEVICE, in that order. */
int qkceil_copy(const void *src, void *dst, uint64_t bytes, int vectors_per_lane, void *stream);

/* Reads src[0, bytes) and discards it. `sink` (16-byte aligned, 1 KiB) is
 * written only if the bytes read combine to a fixed 32-bit pattern, which
 * keeps the loads from being optimised away.
 * Status: as for qkceil_copy. */
int qkceil_read(const void *src, uint64_t bytes, int vectors_per_lane, void *sink, void *stream);

/* Fills dst[0, bytes) with a pattern derived from the position.
 * Status: as for qkceil_copy. */
int qkceil_write(void *dst, uint64_t bytes, int vectors_per_lane, void *stream);

/* A kernel that does nothing, over `workgroups` workgroups of 256 lanes:
 * the fixed cost of a launch. Status: QKCEIL_ERR_CONFIG, QKCEIL_ERR_DEVICE. */
int qkceil_empty(unsigned workgroups, void *stream);

/* Samples the shader clock of the compute unit that runs it (one
 * wavefront): out[0] = cycles of that clock, out[1] = ticks of the fixed
 * 100 MHz real-time clock, over about 2 us; the clock ran at 100 * out[0] /
 * out[1] MHz. Queued between other launches, it shows the clock those
 * launches met. `out` is two 8-byte-aligned uint64 values in device memory.
 * Status: QKCEIL_ERR_NULL, QKCEIL_ERR_ALIGN (out not 8-byte aligned),
 * QKCEIL_ERR_DEVICE. */
int qkceil_clock(uint64_t *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QKCEIL_H */
