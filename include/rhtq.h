/*
 * rhtq.h -- randomized Hadamard rotation fused with 4-bit quantisation (gfx950).
 *
 * C ABI of librhtq.so.  What the calls compute comes from these pages:
 *
 *  - "QuaRot: Outlier-Free 4-Bit Inference in Rotated LLMs" (reviews page):
 *      review 1, Summary ..... Hadamard rotations that cannot be folded into the
 *                              weights are applied online with the Walsh-Hadamard
 *                              fast algorithm; combined with grouped quantisation.
 *      review 2, Summary ..... the random Hadamard transform is invertible up to
 *                              machine precision; activations are quantised to INT4.
 *      review 2, Questions ... widths with a large non-power-of-two part, 172 for
 *                              Llama 2 7B (11008 = 172 x 64), are costly.
 *      review 3, Strengths ... the online Hadamard is applied to activations and to
 *                              the KV cache.
 *      review 3, Questions ... the Hadamard block computes Y = X H^T.
 *      reviewer 2 follow-up .. activations use nearest rounding; per-batch RHT is
 *                              data parallelism.
 *  - "incoh_rotate=true degrades W4 PPL on Qwen3-8B" (KronQ issue #2), Model
 *    Details table: 12288 = 12 x 1024 is Hadamard-compatible.
 *  - "Methodology checks for NVFP4 W4A4 on Qwen3-8B", the NVFP4 results and the
 *    block-Hadamard comment: E2M1 codes with E4M3 block scales, INT4-g128, and MXFP4
 *    compared with both.  MXFP4 itself is defined by the OCP Microscaling Formats (MX)
 *    v1.0 specification (32-element blocks, E8M0 shared scale, E2M1 elements).
 *
 * Per row x of width n (rows contiguous, row-major [tokens][n]):
 *
 *     y = H_n * diag(s) * x / sqrt(n)          (row form Y = X D H^T / sqrt(n))
 *
 * H_n is the Sylvester Hadamard matrix (H[i][j] = (-1)^popcount(i&j)) for
 * n = 2^k, and H12 (x) H_m with index j = j1*m + j2 for n = 12*m, where H12 is
 * the Williamson array [[A,B,B,B],[-B,A,-B,B],[-B,B,A,-B],[-B,-B,B,A]] with
 * A = J3 (all ones) and B = J3 - 2*I3.  For n = 172*m it is H172 (x) H_m, H172
 * the array [[A,B,C,D],[-B,A,-D,C],[-C,D,A,-B],[-D,-C,B,A]] of the symmetric
 * order-43 circulants whose first rows are +1 at 0 and, at k != 0, -1 exactly when
 * k lies in the listed cosets of the subgroup {1,6,7,36,37,42} of the units mod 43
 * (coset c = 3^c * subgroup): A {4,5,6}, B {0,3,4,6}, C {0,2,6}, D {0,1,4}.
 * s is a +-1 vector shared by all rows.
 *
 * Conventions shared by every call:
 *  - Every data pointer is a DEVICE pointer owned by the caller; the library
 *    allocates nothing and keeps no state between calls.  Calls are thread-safe.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream) and
 *    the call returns once it is enqueued.  A fault inside a kernel surfaces at
 *    the caller's next synchronisation, as usual for HIP.
 *  - The calls enqueue kernels only (no memset, copy or host synchronisation; the
 *    dynamic NVFP4 path clears its tensor-scale word with a kernel), so they can be
 *    captured into a HIP graph on a capturing stream, the first call of a kernel
 *    variant included (its one-time occupancy query is a host call that stream
 *    capture permits).
 *  - Arguments are checked on the host before any HIP call; on error nothing is
 *    enqueued and the status says why.  tokens == 0 is a valid no-op.
 *  - Inputs must be finite; results for NaN/Inf inputs are unspecified.  Denormal bf16 or
 *    fp32 input values (below 1.2e-38 in magnitude) may be read as zero by the matrix-core
 *    kernels, so a row made only of them does not get fp32 accuracy; for fp32 input at the
 *    172 x 2^k widths the same holds for rows whose values all lie below about 1e-33 (2^-110).
 *    fp16 input is read exactly, its subnormals (below 6.1e-5) included.
 *  - Alignment: x, y_out, packed_out, x_out and signs must be 16-byte aligned;
 *    scale buffers aligned to their element size.
 *  - Supported widths: n = 2^k with 16 <= n <= 16384, n = 12 * 2^k with
 *    256 <= 2^k <= 2048 (3072, 6144, 12288, 24576), and n = 172 * 2^k with
 *    16 <= 2^k <= 128 (2752, 5504, 11008, 22016).
 *  - signs: device int8 [n] with values +1 / -1, or NULL for all +1 (plain
 *    Hadamard).  Other values are undefined behaviour.
 */
#ifndef RHTQ_H
#define RHTQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RHTQ_ABI_VERSION 4   /* 2: MXFP4 format and E8M0 scales; 3: block-diagonal calls; 4: fp16 input */

/* Status codes. */
#define RHTQ_OK           0   /* enqueued (or nothing to do)                       */
#define RHTQ_EINVAL       1   /* bad argument: null pointer, negative size, alignment */
#define RHTQ_EUNSUPPORTED 2   /* valid but unsupported width / format / group combo */
#define RHTQ_EHIP         3   /* a HIP runtime call failed while enqueueing         */
/* The environment variable RHTQ_TEST_FAIL_LAUNCH=1 (read once per process) makes every entry point
   return RHTQ_EHIP where it would first call HIP, after all argument checks, having enqueued
   nothing: a test hook for the launch-error path. */

/* Input element types. */
#define RHTQ_IN_BF16 0
#define RHTQ_IN_F32  1
#define RHTQ_IN_F16  2   /* IEEE binary16: the FP16 baseline models of the QuaRot reviews page, review 4 Weaknesses */

/* 4-bit formats. */
#define RHTQ_FMT_INT4  0      /* symmetric absmax INT4, two's complement nibbles     */
#define RHTQ_FMT_NVFP4 1      /* E2M1 codes, E4M3 block-16 scales, fp32 tensor scale */
#define RHTQ_FMT_MXFP4 2      /* E2M1 codes, E8M0 (power-of-two) block-32 scales     */

/* Scale storage types. */
#define RHTQ_SCALE_F32  0
#define RHTQ_SCALE_F16  1
#define RHTQ_SCALE_E4M3 2
#define RHTQ_SCALE_E8M0 3     /* byte = exponent + 127 */

/* NVFP4 tensor-scale handling. */
#define RHTQ_TENSOR_SCALE_DYNAMIC 0   /* g = fl32(max|y| / (6*448)) computed and written */
#define RHTQ_TENSOR_SCALE_GIVEN   1   /* g is read from *tensor_scale                   */

typedef void* rhtq_stream_t;  /* a hipStream_t */

/* Returns RHTQ_ABI_VERSION of the loaded library. */
int rhtq_abi_version(void);

/* Static text for a status code ("ok", "invalid argument", ...). */
const char* rhtq_status_str(int status);

/* 1 if (n, fmt, group) is supported, else 0.  INT4: group 0 (one group per row) or
 * a power of two >= 16 dividing n.  NVFP4: group 16.  MXFP4: group 32. */
int rhtq_supported(int32_t n, int fmt, int32_t group);

/*
 * Rotation only:  y_out[t][i] = (H_n diag(s) x[t])[i] / sqrt(n), fp32.
 *   x       [tokens][n] bf16 (RHTQ_IN_BF16), fp16 (RHTQ_IN_F16) or fp32 (RHTQ_IN_F32)
 *   signs   [n] int8 or NULL
 *   y_out   [tokens][n] fp32
 * Cite: QuaRot reviews, review 1 Summary (Walsh-Hadamard algorithm) and review 2
 * Summary (randomised, invertible); review 3 Questions (Y = X H^T).
 */
int rhtq_rotate(const void* x, int in_dtype, int64_t tokens, int32_t n,
                const int8_t* signs, float* y_out, rhtq_stream_t stream);

/*
 * Rotation fused with 4-bit quantisation and nibble packing.
 *   packed_out  [tokens][n/2] bytes: element 2k in the low nibble, 2k+1 in the high.
 *
 * INT4 (fmt RHTQ_FMT_INT4; QuaRot reviews, review 2 Summary and reviewer 2
 * follow-up: INT4, nearest rounding; review 1 Summary: grouped quantisation):
 *   group       0 (one group per row) or a power of two >= 16 dividing n
 *   scale_dtype RHTQ_SCALE_F32 or RHTQ_SCALE_F16
 *   scales_out  [tokens][n/group] (group 0: [tokens][1]); s = max|y|/7 over the group,
 *               rounded to the storage type (nearest even; fp16 saturates at 65504)
 *   codes       q = clamp(round_half_even(y / s_stored), -8, 7); a zero group stores
 *               s = 0 and codes 0.  While the stored scale is a normal number of its
 *               type, |y| <= 7 s and codes stay in [-7, 7].  When an fp16 scale
 *               saturates at 65504 (amax / 7 above it) or is subnormal, y / s can
 *               exceed 7 in magnitude and the clamp applies: codes may then be -8.
 *   tensor_scale, tensor_scale_mode: ignored (may be NULL / 0)
 *
 * NVFP4-style (fmt RHTQ_FMT_NVFP4; NVFP4 methodology thread):
 *   group 16, scale_dtype RHTQ_SCALE_E4M3
 *   tensor_scale  device float: DYNAMIC -> written with g = fl32(max|y| / 2688) over the
 *                 whole call (two passes over x); GIVEN -> g is read (one pass)
 *   scales_out    [tokens][n/16] E4M3FN codes of max|y_block| / (6 g), nearest even,
 *                 saturating at 448, never NaN
 *   codes         bit 3 = sign of y, bits 0-2 = E2M1 magnitude of |y| / (dec(s_b) g)
 *                 ({0,.5,1,1.5,2,3,4,6}, nearest even, saturating at 6); a block whose
 *                 scale decodes to 0 stores code 0.
 *
 * MXFP4 (fmt RHTQ_FMT_MXFP4; OCP MX v1.0, named in the NVFP4 methodology thread):
 *   group 32, scale_dtype RHTQ_SCALE_E8M0; tensor_scale, tensor_scale_mode ignored
 *   scales_out    [tokens][n/32] bytes e + 127 with e = floor(log2(max|y_block|)) - 2
 *                 clamped to [-127, 127] (-127 for an all-zero block); X = 2^e
 *   codes         bit 3 = sign of y, bits 0-2 = E2M1 magnitude of |y| / X (nearest even,
 *                 saturating at 6); an all-zero block stores code 0.
 */
int rhtq_forward(const void* x, int in_dtype, int64_t tokens, int32_t n,
                 const int8_t* signs, int fmt, int32_t group, int scale_dtype,
                 uint8_t* packed_out, void* scales_out, float* tensor_scale,
                 int tensor_scale_mode, rhtq_stream_t stream);

/*
 * Inverse of rhtq_forward: unpack, dequantise with the stored scales (INT4 q*s;
 * NVFP4 e2m1(c) * dec(s_b) * g; MXFP4 e2m1(c) * 2^(byte - 127)) and undo the rotation, x_out = diag(s) H_n^T y / sqrt(n)
 * (fp32 [tokens][n]).  Arguments mirror rhtq_forward; tensor_scale is read for NVFP4.
 * Cite: QuaRot reviews, review 2 Summary (the RHT is invertible).
 */
int rhtq_inverse(const uint8_t* packed, const void* scales, const float* tensor_scale,
                 int64_t tokens, int32_t n, const int8_t* signs, int fmt, int32_t group,
                 int scale_dtype, float* x_out, rhtq_stream_t stream);

/*
 * Block-diagonal variants (NVFP4 methodology thread, the block-Hadamard-128 comment: a Hadamard
 * per 128-element block instead of one over the whole row).  Per row x of width n, with the sign
 * vector s of length n applied first and H_b on every contiguous block of b elements:
 *
 *     y = (I_{n/b} (x) H_b) diag(s) x / sqrt(b)
 *
 *   block   a power of two, 16 <= block < n, dividing n; the row width n itself may then be any
 *           multiple of block up to 2^20 (for example 11008 = 86 x 128, the Llama 2 7B
 *           intermediate width, rotated per 128-block instead of by H172 (x) H64).
 *           block == n is the plain call (n a supported width).
 *   group   quantisation groups lie inside a block: INT4 a power of two >= 16 dividing block
 *           (group 0, one group per row, only when block == n); NVFP4 16; MXFP4 32
 * Every other argument, layout and status is as in the plain call of the same name.
 */
int rhtq_rotate_blocked(const void* x, int in_dtype, int64_t tokens, int32_t n, int32_t block,
                        const int8_t* signs, float* y_out, rhtq_stream_t stream);

int rhtq_forward_blocked(const void* x, int in_dtype, int64_t tokens, int32_t n, int32_t block,
                         const int8_t* signs, int fmt, int32_t group, int scale_dtype,
                         uint8_t* packed_out, void* scales_out, float* tensor_scale,
                         int tensor_scale_mode, rhtq_stream_t stream);

/* x_out = diag(s) (I (x) H_b^T) y_hat / sqrt(b) with y_hat dequantised as in rhtq_inverse. */
int rhtq_inverse_blocked(const uint8_t* packed, const void* scales, const float* tensor_scale,
                         int64_t tokens, int32_t n, int32_t block, const int8_t* signs, int fmt,
                         int32_t group, int scale_dtype, float* x_out, rhtq_stream_t stream);

/*
 * Host helper: a random sign vector from a seed with splitmix64 (Steele, Lea and
 * Flood, OOPSLA 2014): output i = mix(seed + (i+1) * 0x9E3779B97F4A7C15); the sign is
 * -1 when its top bit is set.  host_out is HOST memory [n].  The pages draw the
 * rotation at random and leave the generator open (NVFP4 methodology thread:
 * results vary with the transform seed).
 */
int rhtq_signs_from_seed(uint64_t seed, int32_t n, int8_t* host_out);

#ifdef __cplusplus
}
#endif

#endif /* RHTQ_H */
