/*
 * gptq2d.h -- C ABI of the GPTQ-2D two-sided adaptive rounding library (gfx950).
 *
 * Operation (sources cited by page title and section):
 *   "GPTQ-2D: Cubic-Time Two-Sided Adaptive Rounding" (arxivlens page), Abstract,
 *   Results, Methodology, Technical contributions; mind-verse.de article "Neue
 *   Ansaetze zur Effizienzsteigerung von Large Language Models durch GPTQ-2D",
 *   sections "GPTQ-2D: Eine Weiterentwicklung der adaptiven Rundung" and "Die
 *   algorithmische Neuerung und ihre Auswirkungen".
 *
 *   Given a real m x n matrix W, SPD matrices A (m x m, acting on rows) and
 *   B (n x n, acting on columns) and per-row scales s, produce integer codes
 *   Z in [lo, hi] = [-2^(bits-1), 2^(bits-1)-1] and Q = diag(s) Z by adaptive
 *   rounding under tr(A (W-Q) B (W-Q)^T): the exact trajectory of one-dimensional
 *   GPTQ on the row-major vectorisation of W with Gram A (x) B, computed in cubic
 *   work by rounding anti-diagonals of W in parallel with separable rank-one
 *   feedback.  The triangular feedback factors are U' = diag(U)^-1 U with
 *   A^-1 = U^T U (U upper), i.e. GPTQ's inverse-Hessian Cholesky factor scaled to
 *   a unit diagonal; rint is round-half-to-even of t/s followed by the clamp.
 *
 * Conventions for every entry point
 *   - Matrices are dense, row-major and contiguous, in DEVICE memory.
 *   - dtype selects the element type of all floating-point arguments of a call:
 *     GPTQ2D_F32 (float) or GPTQ2D_F64 (double).  Factorisations always run in
 *     float64 internally; in F32 mode the sweep runs in float32.
 *   - All work is enqueued on `stream` (a hipStream_t passed as void*; NULL is the
 *     null stream) and the call returns without synchronising.  The caller owns
 *     every buffer; the library keeps no pointer after a call returns.
 *   - Inputs are never modified.
 *   - Return value: 0 on success; -i when argument i (1-based) is invalid, checked
 *     on the host before any HIP call; a positive GPTQ2D_ERR_* code when a HIP
 *     runtime call fails.  Numerical failures are reported through `info`, a
 *     DEVICE int[2] that the call first clears (may be NULL): info[0] = 1 if A is
 *     not positive definite, 2 if B is not, 3 if a scale is <= 0 or not finite,
 *     4 if a dependency wait inside one of the persistent kernels (the sweep, or the
 *     factor stage's Cholesky and inverse) exceeded its bound (the kernel then stops early
 *     instead of hanging); info[1] = 1-based index of the failing pivot or row.  When
 *     info[0] != 0 the outputs are undefined.
 *   - Limit of every call that factors or sweeps: its persistent kernels launch one grid of
 *     (compute units x resident workgroups per CU) and need all of it resident at once,
 *     spread over the device's XCDs by the hardware's round-robin dispatch (the sweep
 *     deals bands to XCDs and needs band workers on each of them).  Another kernel that
 *     occupies compute units during the call, or a device partition whose dispatch does not
 *     spread workgroups over its XCDs, can leave a dependency unserved: the call then ends
 *     with info[0] = 4 after the wait bound (of the order of seconds), not with a hang.
 *   - workspace: DEVICE scratch of at least the size returned by the matching
 *     *_workspace_bytes function, 256-byte aligned.  Passing NULL and 0 makes the
 *     library allocate (and free) it stream-ordered on `stream`.
 *   - Calls that overlap in time must not share a workspace.
 */
#ifndef GPTQ2D_H
#define GPTQ2D_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GPTQ2D_F32 0
#define GPTQ2D_F64 1

#define GPTQ2D_ERR_HIP 1          /* a HIP runtime call failed */
#define GPTQ2D_ERR_ALLOC 2        /* device allocation failed */
#define GPTQ2D_ERR_SCRATCH 3      /* problem too large for gptq2d_quantize_noalloc's buffer */

/* Size of the static per-device scratch buffer of gptq2d_quantize_noalloc (64 MiB). */
#define GPTQ2D_NOALLOC_SCRATCH_BYTES (64ull << 20)

/*
 * Factor stage: the unit upper triangular feedback factor of one SPD matrix.
 * (mind-verse article, "GPTQ-2D: Eine Weiterentwicklung der adaptiven Rundung":
 * errors propagate through a triangular feedback matrix; arxivlens page,
 * Limitations: fixed bases, factorisations computed once.)
 *   p        order of A (>= 1)                                         [arg 1]
 *   dtype    GPTQ2D_F32 or GPTQ2D_F64                                   [arg 2]
 *   A        p x p SPD, symmetric; only the lower triangle is read      [arg 3]
 *   U_unit   p x p output: U' (unit diagonal, upper; lower part zero)   [arg 4]
 *   workspace, workspace_bytes  see conventions                      [args 5, 6]
 *   info     device int[2] or NULL; info[0] = 1 if A is not SPD        [arg 7]
 *   stream   hipStream_t                                                [arg 8]
 */
int gptq2d_factor(int64_t p, int dtype, const void* A, void* U_unit,
                  void* workspace, size_t workspace_bytes, int* info, void* stream);
size_t gptq2d_factor_workspace_bytes(int64_t p, int dtype);

/*
 * Sweep stage: two-sided adaptive rounding given both unit factors.
 * (arxivlens page, Results/Methodology: anti-diagonal rounds in parallel with an
 * accumulated-feedback buffer and rank-one separable updates.)
 *   m, n     shape of W (>= 1 each)                                  [args 1, 2]
 *   bits     grid width, 2..8                                           [arg 3]
 *   dtype    GPTQ2D_F32 or GPTQ2D_F64                                   [arg 4]
 *   W        m x n weights                                              [arg 5]
 *   Ua_unit  m x m unit upper factor of A (as from gptq2d_factor)       [arg 6]
 *   Ub_unit  n x n unit upper factor of B                               [arg 7]
 *   scales   m per-row scales, > 0 and finite                           [arg 8]
 *   codes    m x n int8 output, values in [lo, hi]                      [arg 9]
 *   Q        m x n output, Q[k,l] = scales[k] * codes[k,l]             [arg 10]
 *   workspace, workspace_bytes                                     [args 11, 12]
 *   info     device int[2] or NULL; info[0] = 3 for a bad scale        [arg 13]
 *   stream                                                             [arg 14]
 */
int gptq2d_quantize_factored(int64_t m, int64_t n, int bits, int dtype, const void* W,
                             const void* Ua_unit, const void* Ub_unit, const void* scales,
                             int8_t* codes, void* Q, void* workspace, size_t workspace_bytes,
                             int* info, void* stream);
size_t gptq2d_sweep_workspace_bytes(int64_t m, int64_t n, int dtype);

/*
 * Whole call: factor A and B, then sweep (the problem statement of both pages).
 *   m, n, bits, dtype, W                                             [args 1-5]
 *   A        m x m SPD (lower triangle read)                            [arg 6]
 *   B        n x n SPD (lower triangle read)                            [arg 7]
 *   scales, codes, Q, workspace, workspace_bytes, info, stream     [args 8-14]
 */
int gptq2d_quantize(int64_t m, int64_t n, int bits, int dtype, const void* W, const void* A,
                    const void* B, const void* scales, int8_t* codes, void* Q,
                    void* workspace, size_t workspace_bytes, int* info, void* stream);
size_t gptq2d_workspace_bytes(int64_t m, int64_t n, int dtype);

/*
 * gptq2d_quantize for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  Same arguments,
 * semantics and results as gptq2d_quantize, minus the workspace: the library uses a static
 * scratch buffer of GPTQ2D_NOALLOC_SCRATCH_BYTES in each device's memory (reserved when
 * the library's code is first loaded on a device and held until the process ends) and
 * calls no allocating routine (hipMalloc, hipMallocAsync, hipFree, torch).
 *   Limit: problems with gptq2d_workspace_bytes(m, n, dtype) > GPTQ2D_NOALLOC_SCRATCH_BYTES
 *   return GPTQ2D_ERR_SCRATCH before any HIP call (m = n = 896 in F64 and m = n = 1024 in
 *   F32 fit).
 *   All calls on one device share that device's buffer: calls that overlap in time on one
 *   device (two streams, two threads) race on it and their outputs are undefined.  The
 *   buffer keeps the last call's contents; the kernels clear or overwrite everything they
 *   read before reading it.
 *   args: m, n, bits, dtype, W, A, B, scales, codes, Q, info, stream (as gptq2d_quantize)
 */
int gptq2d_quantize_noalloc(int64_t m, int64_t n, int bits, int dtype, const void* W,
                            const void* A, const void* B, const void* scales, int8_t* codes,
                            void* Q, int* info, void* stream);

/*
 * Three Kronecker factors ("GPTQ-2D: Cubic-Time Two-Sided Adaptive Rounding", arxivlens
 * page, Abstract: the algorithm extends to Hessians with any number of Kronecker
 * factors).  W is an m1 x m2 x m3 tensor (row-major: the last index is fastest) and the
 * Gram of its vectorisation is A1 (x) A2 (x) A3; the result is the trajectory of
 * one-dimensional GPTQ on that vectorisation, in that order.  When U1' (x) U2' takes at
 * most 4 GiB (m1 m2 <= 23170 in F64, <= 32768 in F32) the tensor is rounded as one
 * (m1 m2) x m3 two-factor problem under (A1 (x) A2, A3), whose unit factor is
 * U1' (x) U2'; above that, slab by slab: slab k (the m2 x m3 matrix W[k]) receives the
 * feedback of the earlier slabs through U1', then is rounded as a two-factor problem
 * under (A2, A3).  Both routes give the same trajectory; gptq2d_workspace3_bytes sizes
 * the route the call takes.
 *   m1, m2, m3  tensor extents, each in [1, 262140]                   [args 1-3]
 *   bits, dtype                                                        [args 4-5]
 *   W        m1 x m2 x m3                                               [arg 6]
 *   A1, A2, A3  m1 x m1, m2 x m2, m3 x m3 SPD (lower triangles read)  [args 7-9]
 *   scales   m1 x m2: one grid step per fibre W[k][i][:]               [arg 10]
 *   codes    m1 x m2 x m3 int8 out; Q m1 x m2 x m3 out (dtype)       [args 11-12]
 *   workspace, workspace_bytes (gptq2d_workspace3_bytes), info, stream [args 13-16]
 * info[0] = 5, 6 or 7 if A1, A2 or A3 is not positive definite; 3 for a bad scale, with
 * info[1] the 1-based index k m2 + i + 1 of a fibre W[k][i][:] whose scale is bad; 4 as
 * above.
 */
int gptq2d_quantize3(int64_t m1, int64_t m2, int64_t m3, int bits, int dtype, const void* W,
                     const void* A1, const void* A2, const void* A3, const void* scales,
                     int8_t* codes, void* Q, void* workspace, size_t workspace_bytes, int* info,
                     void* stream);
size_t gptq2d_workspace3_bytes(int64_t m1, int64_t m2, int64_t m3, int dtype);

/*
 * Packed codes: the step after the quantizer, whose output is an integer matrix
 * ("GPTQ-2D: Cubic-Time Two-Sided Adaptive Rounding", arxivlens page, Abstract).  The pages
 * define no storage format; this one is dense: a code z in [lo, hi] is the field
 * u = z - lo (bits wide); row r is one little-endian bit string in which code c occupies
 * bits c*bits .. c*bits+bits-1, held in gptq2d_packed_row_words(n, bits) = ceil(n*bits/32)
 * uint32 words (row-major, rows back to back); padding bits are zero.  rows, n >= 1 and
 * <= 2^40; bits in [2, 8].  Device pointers; enqueued on `stream`.
 *
 * gptq2d_pack: codes (rows x n int8, values in [lo, hi]; others are stored modulo 2^bits)
 *   -> packed (rows x words uint32).                        args: rows, n, bits, codes, packed
 * gptq2d_unpack: Q = s[r] * z (rows x n, dtype) from packed and scales (rows, dtype).
 *   args: rows, n, bits, dtype, packed, scales, Q
 * gptq2d_packed_gemv: Y[b][r] = s[r] * sum_c z[r][c] * X[b][c] for b < batch (1..8);
 *   X batch x n, Y batch x rows, dtype.  args: rows, n, bits, dtype, packed, scales, batch,
 *   X, Y.  The sum runs in dtype in an order of the kernel's choosing.
 * A row must hold fewer than 2^31 - 32 bits (n * bits); longer rows return GPTQ2D_ERR_HIP.
 * Return 0, -i for invalid argument i, or GPTQ2D_ERR_HIP.  No info flag.
 */
size_t gptq2d_packed_row_words(int64_t n, int bits);
int gptq2d_pack(int64_t rows, int64_t n, int bits, const int8_t* codes, uint32_t* packed,
                void* stream);
int gptq2d_unpack(int64_t rows, int64_t n, int bits, int dtype, const uint32_t* packed,
                  const void* scales, void* Q, void* stream);
int gptq2d_packed_gemv(int64_t rows, int64_t n, int bits, int dtype, const uint32_t* packed,
                       const void* scales, int batch, const void* X, void* Y, void* stream);

/*
 * Kronecker factor accumulation, the step before the quantizer: the pages take the
 * factors of a Kronecker-factored Hessian as given ("GPTQ-2D: Cubic-Time Two-Sided
 * Adaptive Rounding", arxivlens page, Abstract) and do not say how they are estimated;
 * this is the plain second-moment (Gram) accumulation over a block of samples:
 *   A <- A + alpha * X^T X,   X: N x p (N samples of dimension p, row-major), A: p x p.
 * A must be symmetric on entry: its lower triangle (diagonal included) is read and updated,
 * then copied onto the upper triangle, so A leaves symmetric.  Both in `dtype`; the sums
 * run in dtype on the matrix cores in an order of the kernel's choosing.  p in [1, 262140]
 * with p*p*sizeof(dtype) < 2^31 (else GPTQ2D_ERR_HIP); N >= 1; alpha finite.
 *   args: p, N, dtype, X, alpha, A, stream
 * gptq2d_gram_accumulate_batched: the same for `count` layers in one call (host arrays of
 * length count: p, N, X, alpha, A), enqueued in order on `stream`; an invalid entry of an
 * array returns the index of that array argument.
 *   args: count, p, N, dtype, X, alpha, A, stream
 */
int gptq2d_gram_accumulate(int64_t p, int64_t N, int dtype, const void* X, double alpha,
                           void* A, void* stream);
int gptq2d_gram_accumulate_batched(int count, const int64_t* p, const int64_t* N, int dtype,
                                   const void* const* X, const double* alpha, void* const* A,
                                   void* stream);

/*
 * Measurement hook (not part of the method): when enabled, every kernel launch of
 * the library is bracketed by a pair of HIP events on its stream and accounted to a
 * kernel class (0 sweep, 2 factor: the persistent Cholesky and inverse, 3 other, 4 the
 * mode-1 feedback between slabs of gptq2d_quantize3, 5 packed: gptq2d_pack, gptq2d_unpack
 * and gptq2d_packed_gemv, 6 gram: gptq2d_gram_accumulate) with the
 * algorithmic flops and HBM bytes of that launch.  Class 1 (band_gemm) is counted
 * inside the persistent sweep kernel: its milliseconds are the summed busy time of the
 * workgroups that ran band-update tasks (CU-milliseconds), its launches the tasks and
 * its flops their dense GEMM flops.  Process-wide, off by default; it adds event
 * records to the stream and three atomics per band-update task while on.
 * gptq2d_profile_read waits for the recorded events, writes per-class totals since
 * the previous read (milliseconds, launches, flops, bytes; host arrays, any pointer
 * may be NULL) for the first min(n_classes, 7) classes and resets the totals.
 * Returns 0, -1 if n_classes < 0, or GPTQ2D_ERR_HIP if an event query failed.
 */
int gptq2d_profile_enable(int on);
/*
 * The band-update tasks of the window that the last gptq2d_profile_read closed, split by
 * task class (0 near: 64 deep from the last few bands or column blocks; 1 next: 256 deep,
 * the first targets of a finished outer band or block; 2 far: 256 deep, the rest): summed
 * busy time of the workgroups that ran them in CU-milliseconds, task count and dense GEMM
 * flops, for the first min(n_classes, 3) classes (host arrays, any may be NULL).  Returns 0
 * or -1 if n_classes < 0.
 */
int gptq2d_profile_task_classes(int n_classes, double* cu_ms, int64_t* tasks, double* flops);
int gptq2d_profile_read(int n_classes, double* ms, int64_t* launches, double* flops,
                        double* bytes);
const char* gptq2d_profile_class_name(int cls);

/* Static description of a return code (never NULL). */
const char* gptq2d_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* GPTQ2D_H */
