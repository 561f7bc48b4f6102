/*
 * adasum.h - C ABI of the MI355X (gfx950) Adasum gradient combiner.
 *
 * On one GPU, combines K per-worker gradient buffers that already live in
 * device memory into one gradient with the pairwise Adasum operator
 *
 *     Adasum(a, b) = (1 - a.b / (2 |a|^2)) a + (1 - a.b / (2 |b|^2)) b
 *
 * applied in a fixed binary tree: level 1 pairs (g0,g1), (g2,g3), ...; each
 * later level pairs the previous level's results the same way; when a level
 * has an odd count its last vector is carried up unchanged.  An operand with
 * zero norm gets coefficient 1 (the pair is then the plain sum).  Every
 * segment (layer) of the buffers is combined on its own.
 *
 * Source: "Scaling Distributed Training with Adaptive Summation"
 * (arXiv 2006.02924): the operator is the average of the two emulated
 * sequential SGD orders (derivation after Eq. 2); it sums orthogonal and
 * averages parallel gradients (the discussion before Figure 1); it is applied
 * per layer (the paragraph after Figure 1); more than two gradients are
 * combined by recursive application, and the dot product and norms of a pair
 * must be known before it can be combined, so the operation is not
 * elementwise and cannot be streamed (Sec. 4).
 *
 * Conventions shared by all entry points
 *   - Return 0 (ADASUM_OK) on success or a negative ADASUM_E* code.  The text
 *     of the last failure on the calling thread is adasum_last_error().
 *   - Arguments are validated on the host before any HIP call, so invalid
 *     arguments never reach the GPU and never leave work enqueued.
 *   - Pointers named "device" must be device memory of the current HIP device
 *     (hipSetDevice); pointers named "host" are ordinary host memory read
 *     during the call only.
 *   - stream is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls are asynchronous: they enqueue kernels on stream and return.
 *     Kernel faults surface at the next synchronisation of that stream.
 *   - The caller owns every buffer.  Inputs are read-only and must stay
 *     alive and unchanged until the stream has passed the call.
 *   - Results are bitwise deterministic: the same inputs, K, offsets and
 *     dtype give the same bits on every call and on every stream.
 *   - Device base pointers (inputs, out, workspace) must be 16-byte aligned;
 *     segment boundaries inside the buffers may fall anywhere.
 */
#ifndef ADASUM_H
#define ADASUM_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define ADASUM_API __attribute__((visibility("default")))
#else
#define ADASUM_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of the inputs and of the result.  Intermediate tree levels
 * are always held in fp32; statistics and coefficients in fp64. */
typedef enum {
  ADASUM_F32 = 0,
  ADASUM_F16 = 1,
  ADASUM_BF16 = 2
} adasum_dtype_t;

#define ADASUM_OK 0
#define ADASUM_EINVAL (-1) /* bad argument: see adasum_last_error()          */
#define ADASUM_ENOMEM (-2) /* a device or host allocation failed             */
#define ADASUM_EHIP (-3)   /* a HIP API call or kernel launch failed         */

/*
 * adasum_combine - tree Adasum of K gradients, per segment.
 *
 *   grads        host array of K device pointers; grads[k] holds N elements
 *                of dtype, N = seg_offsets[nseg].  Pointers may repeat.
 *   K            number of workers, >= 1.  K = 1 copies grads[0] to out.
 *   seg_offsets  host int64 array of nseg + 1 CSR offsets: seg_offsets[0]
 *                = 0, non-decreasing; segment s is elements
 *                [seg_offsets[s], seg_offsets[s+1]).  Empty segments are
 *                allowed (their output is empty).
 *   nseg         number of segments, >= 0.
 *   dtype        adasum_dtype_t of the inputs and of out.
 *   out          device pointer to N elements of dtype; must not overlap any
 *                input.  Rounded once, to nearest even, from the fp64 combine.
 *
 * Uses a workspace that the library allocates and caches per (device,
 * stream); the first call for a given shape may therefore allocate.
 * Errors: ADASUM_EINVAL (null pointers with N > 0, K < 1, nseg < 0, bad
 * offsets, unknown dtype, misaligned pointer, out overlapping an input),
 * ADASUM_ENOMEM, ADASUM_EHIP.
 */
ADASUM_API int adasum_combine(const void* const* grads, int K, const int64_t* seg_offsets, int nseg,
                   int dtype, void* out, void* stream);

/*
 * adasum_workspace_bytes - device workspace adasum_combine_ex needs for this
 * shape, in bytes (0 when none is needed).  Returns a negative ADASUM_E*
 * code for invalid arguments (same checks as adasum_combine on K, offsets,
 * nseg and dtype).
 */
ADASUM_API int64_t adasum_workspace_bytes(int K, const int64_t* seg_offsets, int nseg, int dtype);

/*
 * adasum_combine_ex - adasum_combine with caller-provided memory and the
 * per-node statistics exposed.
 *
 *   workspace, workspace_bytes
 *                device buffer of at least adasum_workspace_bytes(...)
 *                bytes, 16-byte aligned, not overlapping any other argument;
 *                may be NULL when that size is 0.  Its contents on entry do
 *                not matter; calls sharing one workspace must be ordered on
 *                one stream.
 *   coeffs       device fp64 array [K-1][nseg][2] receiving (ca, cb) of every
 *                tree node, nodes in level-major order (level 1 left to
 *                right, then level 2, ...), or NULL.
 *   stats        device fp64 array [K-1][nseg][3] receiving (a.b, |a|^2,
 *                |b|^2) of every tree node in the same order, or NULL.
 *                Within each block of up to 16 operands (four tree levels)
 *                the statistics are evaluated in fp64 from the Gram matrix of
 *                the block's operands; above a block, from the fp32 values
 *                its result was stored in.
 *   Other arguments as for adasum_combine.
 */
ADASUM_API int adasum_combine_ex(const void* const* grads, int K, const int64_t* seg_offsets, int nseg,
                      int dtype, void* out, void* workspace, size_t workspace_bytes,
                      double* coeffs, double* stats, void* stream);

/*
 * Kernel timing, for benchmarks.  Between adasum_profile_begin() and
 * adasum_profile_end(), every kernel launch that any combine call of this
 * process enqueues is bracketed by a pair of HIP events recorded on that
 * call's stream.  adasum_profile_end() waits for those events, disables the
 * recording, and writes one row per kernel kind: the launch count, the summed
 * launch durations and the summed algorithmic bytes (every operand read
 * once, every result written once).  Returns the number of rows written (at
 * most max_rows; rows may be NULL when max_rows is 0) or a negative code.
 */
typedef struct {
  char kernel[32];     /* "gram", "tree", "wsum", "widen", "copy" */
  int launches;
  double milliseconds;
  double bytes;
} adasum_kernel_time_t;

ADASUM_API int adasum_profile_begin(void);
ADASUM_API int adasum_profile_end(adasum_kernel_time_t* rows, int max_rows);

/* Static text for an ADASUM_* code. */
ADASUM_API const char* adasum_strerror(int code);

/* Text of the last failure on the calling thread ("" if none). */
ADASUM_API const char* adasum_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
ADASUM_API int adasum_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ADASUM_H */
