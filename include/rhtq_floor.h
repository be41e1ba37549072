/* rhtq_floor.h -- streaming floor of a launch shape: a measurement aid that ships beside the
 * method in librhtq.so, not part of it.
 *
 * A kernel's time is bounded below by what a kernel of the same launch shape needs just to
 * move the same bytes.  rhtq_stream_floor moves exactly the bytes of a per-row 4-bit forward
 * call (rhtq_forward with a per-token or per-group scale) for the two row widths that carry the
 * headline measurements -- it reads tokens x n bf16 values and writes tokens x n/2 code bytes
 * plus tokens x scale_bytes_per_row scale bytes -- using the forward kernel's grid, its
 * workgroup shape (two 64-lane waves per row, each taking half the row) and its 16-byte
 * non-temporal loads in lane order, with no arithmetic beyond an XOR fold of the loaded words
 * into the stored ones.  The forward call's time over this one is what the rotation and the
 * quantisation cost beyond the memory traffic of that shape.
 *
 *  - n = 4096: one workgroup per row (the grid of the paired 4096 kernel, which serves up to
 *    4096 rows; beyond that the forward call uses another kernel and the floor keeps this grid);
 *  - n = 12288: the persistent grid of the 12288 kernel (its resident-workgroup count from an
 *    occupancy query, capped at the row count), rows taken in grid-stride order with the next
 *    row's loads issued before the current row's stores.
 *
 * The output bytes are not codes: they only depend on the input, so that no load or store can
 * be dropped by the compiler.  packed_out[r][k] and scales_out hold the XOR folds described at
 * the kernel (tests check them), and nothing else should read them.
 *
 * Arguments: x [tokens][n] bf16, 16-byte aligned; packed_out [tokens][n/2] bytes, 4-byte
 * aligned; scales_out [tokens][scale_bytes_per_row] bytes, 4-byte aligned; every pointer a
 * device pointer owned by the caller; stream a hipStream_t (NULL = default stream).
 * scale_bytes_per_row: a multiple of 4 in [4, 512] (4 = one f32 per row; 192 = 96 f16 group
 * scales of a 12288-wide row in groups of 128).
 * Returns RHTQ_OK (enqueued; tokens == 0 enqueues nothing), RHTQ_EINVAL (negative tokens, null
 * pointer, misalignment, bad scale_bytes_per_row), RHTQ_EUNSUPPORTED (n other than 4096 or
 * 12288) or RHTQ_EHIP, with the same conventions as the calls of rhtq.h.
 */
#ifndef RHTQ_FLOOR_H
#define RHTQ_FLOOR_H

#include <stdint.h>

#include "rhtq.h"

#ifdef __cplusplus
extern "C" {
#endif

int rhtq_stream_floor(const void* x, int64_t tokens, int32_t n, void* packed_out, void* scales_out,
                      int32_t scale_bytes_per_row, rhtq_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* RHTQ_FLOOR_H */
