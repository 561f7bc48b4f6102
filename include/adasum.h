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
 *   - Arguments are validated before any work is enqueued, so invalid
 *     arguments never reach the GPU: first on the host alone (shapes,
 *     NULLs, alignment, overlaps), then with the HIP runtime's pointer
 *     queries (ADASUM_EINVAL for host memory, memory of another device, or
 *     a buffer shorter than the call needs where the runtime knows its
 *     allocation's extent).
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
 *   - Graph capture: the first call for a shape (K, offsets, dtype,
 *     schedule) on a device uploads that shape's tables; adasum_combine's
 *     first call on a stream, or for a larger shape, also allocates its
 *     workspace.  A later call of that shape enqueues kernels only (no
 *     allocation, copy, memset or synchronisation), so it may be captured
 *     into a HIP graph, as long as the library still caches the shape (the
 *     64 most recently used shapes; making room for a new shape waits for
 *     the device).  Profiling (adasum_profile_begin) must be off while
 *     capturing.
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

/* Element type of the inputs and of the result.  Inside a block of up to 16
 * operands (all of them for at most 64 16-bit inputs in the tree) nothing
 * intermediate is stored: statistics are quadratic
 * forms in the block's fp64 Gram matrix and the block's result is one
 * weighted sum; a block result that feeds a later stage (K above 16, or
 * above 64 for 16-bit inputs in the tree) is kept in fp64.
 * Statistics and coefficients are fp64. */
typedef enum {
  ADASUM_F32 = 0,
  ADASUM_F16 = 1,
  ADASUM_BF16 = 2
} adasum_dtype_t;

/* Order in which the pairwise operator is applied to the K gradients. */
typedef enum {
  ADASUM_TREE = 0, /* level by level: (g0,g1), (g2,g3), ...; the odd last vector is carried */
  ADASUM_CHAIN = 1 /* left to right: acc = Adasum(acc, g_{i+1}), the linear recursion */
} adasum_schedule_t;

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
 * stream); the first call for a given shape may therefore allocate.  The
 * cache is keyed by the stream handle and kept until the process ends:
 * calls on one stream share one buffer in stream order, so a stream with
 * calls still pending must be synchronized before it is destroyed if a new
 * stream could be given the same handle.
 * Errors: ADASUM_EINVAL (null pointers with N > 0, K < 1, nseg < 0, bad
 * offsets, unknown dtype, misaligned pointer, out overlapping an input,
 * N > 2^40, K * nseg > 2^31 - 1), ADASUM_ENOMEM, ADASUM_EHIP.
 */
ADASUM_API int adasum_combine(const void* const* grads, int K, const int64_t* seg_offsets, int nseg,
                   int dtype, void* out, void* stream);

/*
 * adasum_workspace_bytes - device workspace adasum_combine_ex needs for this
 * shape and schedule, in bytes.  Returns a negative ADASUM_E* code for
 * invalid arguments (same checks as adasum_combine_ex on K, offsets, nseg,
 * dtype and schedule).
 */
ADASUM_API int64_t adasum_workspace_bytes(int K, const int64_t* seg_offsets, int nseg, int dtype,
                                          int schedule);

/*
 * adasum_combine_ex - adasum_combine with a choice of schedule, caller-
 * provided memory and the per-node statistics exposed.
 *
 *   schedule     ADASUM_TREE (the combine above) or ADASUM_CHAIN (the linear
 *                recursion the text introduces first: the running result
 *                meets g_1, g_2, ... in turn).
 *   workspace, workspace_bytes
 *                device buffer of at least adasum_workspace_bytes(...)
 *                bytes, 16-byte aligned, not overlapping any other argument.
 *                Its contents on entry do not matter; calls sharing one
 *                workspace must be ordered on one stream.
 *   coeffs       device fp64 array [K-1][nseg][2] receiving (ca, cb) of every
 *                node, or NULL.  Tree nodes are in level-major order (level 1
 *                left to right, then level 2, ...); chain nodes in step order.
 *   stats        device fp64 array [K-1][nseg][3] receiving (a.b, |a|^2,
 *                |b|^2) of every node in the same order, or NULL.
 *                Within each block of up to 16 operands (four tree levels;
 *                32 or 64 operands, five or six levels, when at most 64
 *                16-bit inputs make the whole tree one block; a chain
 *                takes blocks of up to 16 whatever the dtype) the statistics are evaluated
 *                from the Gram matrix of the block's operands, accumulated
 *                in fp64 (double-double where a merge cancels deeply enough
 *                for the fp64 rounding to matter); above a block, from its
 *                result kept in fp64.  coeffs, stats and ortho must be 8-byte aligned
 *                and overlap no other argument.
 *   ortho        device fp64 array [nseg] receiving, per segment, the
 *                orthogonality ratio |result|^2 / sum_k |g_k|^2 of Figure 1
 *                (1 for mutually orthogonal gradients, 1/K for K equal ones;
 *                NaN when every gradient of the segment is zero or the
 *                segment is empty), or NULL.
 *   Other arguments as for adasum_combine.
 */
ADASUM_API int adasum_combine_ex(const void* const* grads, int K, const int64_t* seg_offsets, int nseg,
                                 int dtype, int schedule, void* out, void* workspace,
                                 size_t workspace_bytes, double* coeffs, double* stats, double* ortho,
                                 void* stream);

/*
 * adasum_combine_noalloc - adasum_combine_ex for callers that cannot allocate
 * device memory (tight serving loops, harnesses that forbid hipMalloc).  It
 * allocates nothing: the call's workspace and plan tables live in a fixed
 * array of device memory that the library holds on every GPU it runs on,
 * 64 MiB each, kept until the process ends.  The tables are copied into it
 * on `stream` from host memory with hipMemcpyAsync, so a call cannot be
 * captured into a HIP graph (refused with ADASUM_EINVAL; capture
 * adasum_combine_ex with a workspace allocated before the capture instead).
 *
 *   Arguments as for adasum_combine_ex, without the workspace.
 *   Errors: as adasum_combine_ex, and ADASUM_EINVAL when the shape's
 *   workspace and tables need more than the array holds (the message gives
 *   the bytes needed; adasum_combine_ex then serves the shape).
 *   Every call on one GPU shares that GPU's array and leaves its contents
 *   behind: calls that overlap on one GPU (on different streams, or from
 *   different threads without ordering) race and give wrong results.
 *   Calls ordered on one stream are safe.
 */
ADASUM_API int adasum_combine_noalloc(const void* const* grads, int K, const int64_t* seg_offsets, int nseg,
                                      int dtype, int schedule, void* out, double* coeffs, double* stats,
                                      double* ortho, void* stream);

/*
 * adasum_sum - the synchronous-SGD combination the text compares against:
 * out = g_0 + g_1 + ... + g_{K-1}, element by element, accumulated in fp64 in
 * worker order and rounded once to dtype (Sec. 2 of the text: the allreduce
 * that sums the local gradients).  Segments play no role.
 *
 *   grads, K, dtype, out, stream   as for adasum_combine; N elements each.
 *   workspace    device buffer of adasum_sum_workspace_bytes(K, N, dtype)
 *                bytes (0 for K <= 64, then NULL is allowed), 16-byte
 *                aligned.
 */
ADASUM_API int adasum_sum(const void* const* grads, int K, int64_t N, int dtype, void* out, void* workspace,
                          size_t workspace_bytes, void* stream);
ADASUM_API int64_t adasum_sum_workspace_bytes(int K, int64_t N, int dtype);

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
  char kernel[32];     /* "gram", "tree", "exact", "wsum" (a small combine's
                          fused walk and weighted sum counts here), "sum" */
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
