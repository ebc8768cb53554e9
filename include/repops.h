/*
 * repops.h -- C ABI of the reproducible fixed-order FP32 matrix multiply for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (Verde and RepOps article, section 3.2 "RepOps design
 * principles", item 2, the matrix-multiplication example) is
 *
 *     C(i, j) = sum over k = 0, 1, ..., K-1 of op(A)(i, k) * op(B)(k, j)
 *
 * evaluated, for every (i, j), as: s = +0.0f; for k ascending:
 * s = RN(s + RN(a * b)); C(i, j) = s.  RN is binary32 round-to-nearest-even
 * with gradual underflow; the multiply and the add are rounded separately
 * (no fused multiply-add: the Zoo chain-soundness spec, "Detailed proof:
 * deterministic ordering", turns it off in deterministic mode).  (i, j) is
 * the only parallel dimension and k is never split, so every finite output
 * has one correct bit pattern, whatever the tiling, launch shape, variant,
 * transposes or strides (the article, section 3.1, lists operation order and
 * tensor strides as the sources of nondeterminism this removes).  Infinities
 * follow IEEE 754; a NaN result is some NaN (its payload and sign are not
 * specified).  Because s starts at +0, no output is ever -0.
 *
 * Layout.  Strides are in elements (not bytes) and describe the matrix as
 * stored.  op(A)(i, k) = A[i*a_rs + k*a_cs] when trans_a == 0 and
 * A[k*a_rs + i*a_cs] when trans_a == 1; op(B)(k, j) = B[k*b_rs + j*b_cs]
 * when trans_b == 0 and B[j*b_rs + k*b_cs] when trans_b == 1.  C is M x N,
 * C(i, j) = C[i*c_rs + j*c_cs].  A row-major M x K matrix has a_rs = K,
 * a_cs = 1.  Strides must be >= 0; zero strides are allowed on A and B
 * (broadcast) but C's strides must map distinct (i, j) to distinct
 * elements.
 *
 * Ownership.  A, B and C are device pointers owned by the caller; they are
 * borrowed until the work queued on `stream` has completed.  C is
 * overwritten and never read.  The library allocates no device memory, keeps
 * no mutable global state and is safe to call from several host threads.
 *
 * Errors.  Every entry point returns a repops_status and never throws.  All
 * argument errors are detected on the host before anything is queued, and
 * then nothing is written.  Launch failures are reported as REPOPS_ERR_HIP;
 * faults during execution surface at the caller's next synchronisation.
 * No entry point synchronises the stream.
 */
#ifndef REPOPS_H
#define REPOPS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum repops_status {
    REPOPS_OK = 0,
    REPOPS_ERR_NULL = 1,    /* A, B or C is NULL while the call has work to do */
    REPOPS_ERR_DIM = 2,     /* M, N or K negative, trans_a/trans_b not 0 or 1,
                               or an element offset overflows int64 */
    REPOPS_ERR_STRIDE = 3,  /* a negative stride, or C's strides map two
                               outputs to one element */
    REPOPS_ERR_ALIAS = 4,   /* the bytes C spans overlap those of A or B */
    REPOPS_ERR_VARIANT = 5, /* unknown variant index */
    REPOPS_ERR_HIP = 6      /* the HIP runtime reported an error at launch */
} repops_status;

/*
 * C = op(A) op(B) by the fixed-order definition above, queued on `stream`
 * (a hipStream_t passed as void*; NULL is the null stream).  The library
 * picks the kernel variant from the sizes and layouts.
 *
 * M == 0 or N == 0: returns REPOPS_OK without queueing anything (pointers
 * may then be NULL).  K == 0: C is filled with +0.0f (A and B are not read
 * and may be NULL).
 */
repops_status repops_matmul_f32(const float* A, int64_t a_rs, int64_t a_cs,
                                const float* B, int64_t b_rs, int64_t b_cs,
                                float* C, int64_t c_rs, int64_t c_cs,
                                int64_t M, int64_t N, int64_t K,
                                int trans_a, int trans_b, void* stream);

/*
 * The same operation with the kernel variant forced: `variant` is an index
 * in [0, repops_variant_count()), or -1 for the automatic choice.  Every
 * variant produces identical bits; the choice only changes speed.  For tests
 * and benchmarks.
 */
repops_status repops_matmul_f32_ex(const float* A, int64_t a_rs, int64_t a_cs,
                                   const float* B, int64_t b_rs, int64_t b_cs,
                                   float* C, int64_t c_rs, int64_t c_cs,
                                   int64_t M, int64_t N, int64_t K,
                                   int trans_a, int trans_b, void* stream,
                                   int variant);

/*
 * Validates the arguments exactly as repops_matmul_f32_ex does and returns
 * the status that call would return before queueing anything.  Queues
 * nothing and touches no device: A, B and C are compared as addresses and
 * never dereferenced.
 */
repops_status repops_check_args_f32(const float* A, int64_t a_rs, int64_t a_cs,
                                    const float* B, int64_t b_rs, int64_t b_cs,
                                    const float* C, int64_t c_rs, int64_t c_cs,
                                    int64_t M, int64_t N, int64_t K,
                                    int trans_a, int trans_b, int variant);

/*
 * The variant repops_matmul_f32 would run for these sizes and layouts
 * (an index into the variant table), or -1 for an invalid argument set.
 * Touches no device.
 */
int repops_pick_variant_f32(const float* A, int64_t a_rs, int64_t a_cs,
                            const float* B, int64_t b_rs, int64_t b_cs,
                            int64_t M, int64_t N, int64_t K, int trans_a, int trans_b);

/* Number of kernel variants, and a static name for each ("?" if out of range). */
int repops_variant_count(void);
const char* repops_variant_name(int variant);

/* Static text for a status code. */
const char* repops_strerror(repops_status status);

/*
 * Static text describing the build: compiler version, offload target,
 * floating-point flags, the variant table.  Lets a record of results name
 * exactly which kernels produced them.
 */
const char* repops_build_manifest(void);

#ifdef __cplusplus
}
#endif

#endif /* REPOPS_H */
