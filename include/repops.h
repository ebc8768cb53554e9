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
 * No entry point synchronises the stream.  The calls that need device scratch
 * (the tensor hash) take it from the caller as a workspace argument; one
 * variant, repops_merkle_root_noalloc, uses a fixed static device buffer
 * instead (the only global state, see there).
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
    REPOPS_ERR_HIP = 6,     /* the HIP runtime reported an error at launch */
    REPOPS_ERR_DUPLICATE = 7, /* two contributors share one identity */
    REPOPS_ERR_ALIGN = 8,   /* a pointer is not aligned as the call requires */
    REPOPS_ERR_WORKSPACE = 9, /* the workspace is NULL or smaller than required */
    REPOPS_ERR_SCRATCH = 10   /* the call needs more than the static scratch
                                 (REPOPS_NOALLOC_SCRATCH_BYTES) holds */
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
 * Batched form with an optional bias epilogue.  For each b in [0, batch),
 * with X_b = X + b * x_bs for each of A, B and C (strides in elements):
 *
 *     C_b(i, j) = RN(S_b(i, j) + bias[b*bias_bs + j*bias_s])   (bias != NULL)
 *     C_b(i, j) = S_b(i, j)                                     (bias == NULL)
 *
 * where S_b is the fixed-order sum of op(A_b) op(B_b) defined above.  Batch
 * is one more free dimension (the Verde and RepOps article, section 3.2
 * item 1: dimensions that do not touch the order are parallelised freely);
 * the bias is one more separately rounded add after the whole sum (a bias of
 * -0 on an exact-zero sum gives +0).  K == 0 gives RN(+0 + bias).
 * `variant` as in repops_matmul_f32_ex (-1: automatic).  Batch strides must
 * be >= 0; C's (b, i, j) must map to distinct elements; C may not overlap A,
 * B or the bias.  batch == 0 is a successful no-op.  Errors as above.
 */
repops_status repops_matmul_batched_f32(const float* A, int64_t a_bs, int64_t a_rs, int64_t a_cs,
                                        const float* B, int64_t b_bs, int64_t b_rs, int64_t b_cs,
                                        float* C, int64_t c_bs, int64_t c_rs, int64_t c_cs,
                                        int64_t M, int64_t N, int64_t K, int64_t batch,
                                        int trans_a, int trans_b,
                                        const float* bias, int64_t bias_bs, int64_t bias_s,
                                        void* stream, int variant);

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

/* ------------------------------------------------------------------------
 * Fixed-order gradient average and SGD step (Zoo Per-LLM Chain Soundness,
 * section "Detailed proof: deterministic ordering", paragraphs "Ordering
 * subroutine", "Determinism of left-fold" and "Update step"; the aggregation
 * rule and the order lemma of section "Deterministic gradient ordering").
 * ---------------------------------------------------------------------- */

/* Contributors one pass of the fold kernel reads; longer folds run in several
 * passes that carry the running sum through `gbar`. */
#define REPOPS_FOLD_MAX_PER_PASS 64

/*
 * Canonical contributor order: the k contributors sorted lexicographically by
 * the bytes of their identities (unsigned byte comparison; a proper prefix
 * sorts first).  dids[c] points at did_lens[c] bytes (may be NULL when the
 * length is 0).  On success order_out[r] is the index c of the contributor
 * at rank r.  Host only; touches no device.
 * Errors: REPOPS_ERR_NULL (NULL array with k > 0, or NULL bytes with a
 * nonzero length), REPOPS_ERR_DIM (k < 0 or a negative length),
 * REPOPS_ERR_DUPLICATE (two identical identities: the batch is keyed by
 * contributor).  order_out is unspecified after an error.
 */
repops_status repops_canonical_order(const uint8_t* const* dids, const int64_t* did_lens,
                                     int64_t k, int64_t* order_out);

/*
 * For every parameter e in [0, d), with contributors in the order given:
 *     S        = (((g_0[e] + g_1[e]) + g_2[e]) + ...) + g_{k-1}[e]
 *     gbar[e]  = RN(RN(1/k) * S)
 *     theta[e] = RN(theta[e] - RN(eta * gbar[e]))
 * each operation a separately rounded binary32 operation (round to nearest
 * even, gradual underflow, no fused multiply-add).  The fold starts from
 * g_0 itself; "(1/k) *" is the binary32 quotient 1/k rounded once, then a
 * multiply.  Bits never depend on launch shape or pointer alignment.
 *
 * grads: host array of k device pointers, already in canonical order (see
 * repops_canonical_order), each to d contiguous floats.  theta: device, d
 * floats, updated in place.  gbar: device, d floats, receives gbar; may be
 * NULL when k <= REPOPS_FOLD_MAX_PER_PASS, required above that (it holds the
 * running sum between passes).  Queued on `stream` (a hipStream_t as void*).
 * The grads array itself is read before the call returns; the gradients are
 * borrowed until the queued work completes.
 * Errors: REPOPS_ERR_NULL, REPOPS_ERR_DIM (k < 1, k > 2^24, d < 0, or an
 * offset overflow), REPOPS_ERR_ALIAS (theta or gbar overlaps a gradient, or
 * gbar overlaps theta), REPOPS_ERR_HIP.  d == 0 is a successful no-op.
 */
repops_status repops_fold_mean_sgd_f32(const float* const* grads, int64_t k, int64_t d,
                                       float eta, float* theta, float* gbar, void* stream);

/* ---- Tensor hash and the referee's single-operator re-execution ----------
 *
 * Verde and RepOps article, section 2.3.1 (every node of the training
 * graph carries hash lists of its input and output tensors), section 2.3.2
 * (checkpoint hashes are Merkle trees) and section 2.4, case 3 (when two
 * trainers agree on a node's inputs but not on its output hash, the referee
 * runs that one operator and sees which output hash it reproduces).  The
 * article names no hash function.  These calls use SHA-256 (FIPS 180-4) in
 * the Merkle tree of RFC 6962, section 2.1:
 *     leaf hash  SHA-256(0x00 || leaf bytes)
 *     node hash  SHA-256(0x01 || left digest || right digest)
 *     the left subtree of n > 1 leaves holds the largest power of two < n
 *     the empty input hashes to SHA-256 of the empty string.
 * The data is cut into leaves of leaf_bytes from its first byte, the last
 * leaf shorter when nbytes is not a multiple.  A float32 tensor is hashed as
 * its elements in logical row-major order, each in little-endian binary32
 * encoding: the bytes of a contiguous row-major tensor on this device.
 * The root is written to device memory as the 32 digest bytes.
 */

/* The leaf size the Python binding uses when none is given. */
#define REPOPS_MERKLE_DEFAULT_LEAF_BYTES 1024

/*
 * Bytes of device workspace repops_merkle_root needs for nbytes of data in
 * leaves of leaf_bytes (0 when the tree fits one workgroup, i.e. at most 256
 * leaves), or -1 when the sizes are invalid (see repops_merkle_root).  It
 * holds intermediate digests: 32 bytes per leaf for leaves of 1 KiB or more,
 * at most nbytes / 8 for shorter ones, plus under 1 %.  Host only; touches
 * no device.
 */
int64_t repops_merkle_workspace_bytes(int64_t nbytes, int64_t leaf_bytes);

/*
 * root = the Merkle tree hash above of the nbytes bytes at data, queued on
 * `stream`.  data: device, 4-byte aligned (16-byte aligned with leaf_bytes a
 * multiple of 16 takes the wide-load path; the hash is the same).  nbytes:
 * a multiple of 4 in [0, 2^50].  leaf_bytes: a multiple of 4 in [4, 2^24].
 * workspace: device, 16-byte aligned, at least
 * repops_merkle_workspace_bytes(nbytes, leaf_bytes) bytes (may be NULL when
 * that is 0); its contents are scratch, overwritten.  root: device, 32
 * bytes, 4-byte aligned.  All are borrowed until the queued work completes;
 * calls that share a workspace must be ordered on one stream.
 * Errors: REPOPS_ERR_DIM (sizes out of range or not multiples of 4),
 * REPOPS_ERR_NULL (root NULL, or data NULL with nbytes > 0),
 * REPOPS_ERR_ALIGN, REPOPS_ERR_WORKSPACE, REPOPS_ERR_ALIAS (root, workspace
 * and data overlap), REPOPS_ERR_HIP.
 */
repops_status repops_merkle_root(const void* data, int64_t nbytes, int64_t leaf_bytes,
                                 void* workspace, int64_t workspace_bytes, void* root,
                                 void* stream);

/*
 * Bytes of the static device scratch behind repops_merkle_root_noalloc.
 */
#define REPOPS_NOALLOC_SCRATCH_BYTES (16 * 1024 * 1024)

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * repops_merkle_root without a workspace argument.  The intermediate digests
 * go to a static device array of REPOPS_NOALLOC_SCRATCH_BYTES (16 MiB) that
 * the library holds on each GPU it runs on until the process ends; this call
 * allocates nothing.  The result is the same root as repops_merkle_root's.
 * data, nbytes, leaf_bytes, root, stream: as in repops_merkle_root.
 * Limit: repops_merkle_workspace_bytes(nbytes, leaf_bytes) must be at most
 * REPOPS_NOALLOC_SCRATCH_BYTES (in 1 KiB leaves, up to about 512 MiB of data),
 * else REPOPS_ERR_SCRATCH and nothing is queued.  The device is the current
 * one, which must be the stream's; its first call looks up that device's
 * array address (REPOPS_ERR_HIP if that fails).  Every call on one GPU shares
 * that GPU's array: calls whose queued work may overlap in time on one GPU
 * (other streams, other host threads, other graphs) race and must be ordered
 * by the caller, e.g. all on one stream.  Errors: those of repops_merkle_root,
 * with REPOPS_ERR_SCRATCH in place of REPOPS_ERR_WORKSPACE.
 */
repops_status repops_merkle_root_noalloc(const void* data, int64_t nbytes, int64_t leaf_bytes,
                                         void* root, void* stream);

/*
 * The referee's decision on an output-hash dispute over a matmul: queue
 * C = op(A) op(B) (repops_matmul_f32 with C contiguous row-major, c_rs = N,
 * c_cs = 1), root = the tensor hash of C with leaves of leaf_bytes, and
 * match[c] = 1 if claim c (32 bytes at claims + 32*c) equals root, else 0,
 * for c < nclaims.  A trainer's claim that is not reproduced is wrong; when
 * none is, both trainers are.  Everything is device memory and queued on
 * `stream`; nothing is synchronised.  A, B, C, M, N, K, trans_a, trans_b as
 * in repops_matmul_f32; workspace as in repops_merkle_root for nbytes =
 * 4*M*N.  claims: device, 4-byte aligned (may be NULL when nclaims == 0).
 * root: device, 32 bytes.  match: device, nclaims int32 values.
 * Errors: those of repops_matmul_f32 and repops_merkle_root, plus
 * REPOPS_ERR_DIM (nclaims < 0 or above 2^40), REPOPS_ERR_NULL (claims or
 * match NULL with nclaims > 0), REPOPS_ERR_ALIGN and REPOPS_ERR_ALIAS (match,
 * claims, root, C and the workspace overlap).
 */
repops_status repops_referee_matmul_f32(const float* A, int64_t a_rs, int64_t a_cs, const float* B,
                                        int64_t b_rs, int64_t b_cs, float* C, int64_t M, int64_t N,
                                        int64_t K, int trans_a, int trans_b, int64_t leaf_bytes,
                                        void* workspace, int64_t workspace_bytes,
                                        const void* claims, int64_t nclaims, void* root,
                                        int32_t* match, void* stream);

/* ---- Other RepOps operators: ERF, GeLU, LayerNorm ------------------------
 *
 * The Verde and RepOps article (section 4.3) names LayerNorm, GeLU and ERF as
 * RepOps operators without giving formulas.  Each call below evaluates one
 * fixed sequence of binary32 operations, every +, -, *, / and square root
 * rounded to nearest even on its own (gradual underflow, no fused
 * multiply-add; division and square root are the correctly rounded IEEE
 * operations), so every output has one bit pattern on any IEEE machine.
 */

/*
 * y[i] = erf(x[i]) for i < n, evaluated in two pieces split at |x| = 1:
 *   |x| < 1:  s = Horner's rule in w = x*x over c10 .. c0, c_n the binary32
 *             value of (2/sqrt pi) (-1)^n / (n! (2n+1)) (the Maclaurin series);
 *             erf = s * x.
 *   |x| >= 1 and NaN: Abramowitz and Stegun, Handbook of Mathematical
 *             Functions, 7.1.28: y = |x|; p = Horner's rule over a6 .. a1, 1
 *             in y; q = p^16 by four squarings; erf = sign(x) * (1 - 1/q).
 * Error against the true erf: at most 3 units in the last place below 1,
 * 4.7e-7 absolute above.  erf(+-0) = +-0, erf(+-inf) = +-1.
 * x, y: device, n floats (y may equal x; other overlaps are rejected).
 * Errors: REPOPS_ERR_DIM (n < 0 or above 2^46), REPOPS_ERR_NULL,
 * REPOPS_ERR_ALIAS, REPOPS_ERR_HIP.  n == 0 is a successful no-op.
 */
repops_status repops_erf_f32(const float* x, float* y, int64_t n, void* stream);

/*
 * y[i] = GeLU(x[i]) = (x * 0.5) * (1 + erf(x * c)) with c = 1/sqrt(2) rounded
 * to binary32 and erf as in repops_erf_f32, left to right.  Error against
 * x * Phi(x): at most 3.5e-7 * max(1, |x|).  GeLU(-inf) is NaN (-inf * 0).
 * Arguments and errors as in repops_erf_f32.
 */
repops_status repops_gelu_f32(const float* x, float* y, int64_t n, void* stream);

/*
 * LayerNorm of each of `rows` rows of H floats (Ba, Kiros and Hinton,
 * "Layer Normalization", 2016), per row:
 *     S  = +0; for i ascending: S = S + x_i;            mu = S / H
 *     S2 = +0; for i ascending: d = x_i - mu; S2 = S2 + d * d
 *     var = S2 / H;  rstd = 1 / sqrt(var + eps)
 *     y_i = ((x_i - mu) * rstd) * gamma_i + beta_i
 * Row r of x starts at x + r * x_rs, of y at y + r * y_rs (strides in
 * elements).  gamma, beta: H floats each, or NULL to leave out the multiply
 * or the add.  mean, rstd: `rows` floats each receiving mu and rstd, or NULL.
 * All device memory, borrowed until the queued work completes.  y may equal x
 * with y_rs == x_rs (in place); no other overlaps between x, y, gamma, beta,
 * mean and rstd are allowed.
 * Errors: REPOPS_ERR_DIM (rows < 0, H < 1 or above 2^24, offsets above 2^46
 * elements), REPOPS_ERR_STRIDE (x_rs < 0, y_rs < 0, or y_rs < H with more
 * than one row), REPOPS_ERR_NULL (x or y NULL with rows > 0),
 * REPOPS_ERR_ALIAS, REPOPS_ERR_HIP.  rows == 0 is a successful no-op.
 */
repops_status repops_layernorm_f32(const float* x, int64_t x_rs, const float* gamma,
                                   const float* beta, float* y, int64_t y_rs, int64_t rows,
                                   int64_t H, float eps, float* mean, float* rstd, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* REPOPS_H */
