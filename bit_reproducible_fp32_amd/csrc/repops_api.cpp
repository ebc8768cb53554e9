// C-ABI front end of the reproducible fixed-order FP32 matmul: argument
// validation, layout classification, variant table and dispatch.  Pure host
// C++; every device action goes through the launchers in repops_kernels.hip.
#include <stdint.h>
#include <string.h>

#include <algorithm>

#include "../../include/repops.h"
#include "repops_internal.h"

#ifndef REPOPS_BUILD_FLAGS
#define REPOPS_BUILD_FLAGS "unknown"
#endif
#ifndef REPOPS_OFFLOAD_ARCH
#define REPOPS_OFFLOAD_ARCH "unknown"
#endif

using namespace repops;

namespace {

enum Kind { KIND_NAIVE = 0, KIND_TILED = 1, KIND_MPROD = 2, KIND_SROW = 3 };

struct Variant {
    const char* name;
    int kind;
    int cfg;    // TileCfg for KIND_TILED
    int order;  // TileOrder for KIND_TILED
};

// Every entry computes identical bits; they differ in tile shape, lane block
// and workgroup traversal order only.
const Variant kVariants[] = {
    {"naive_lane_per_output", KIND_NAIVE, 0, 0},
    {"valu_t128x128x16_r8x8_row", KIND_TILED, CFG_128x128, ORDER_ROW},
    {"valu_t128x128x16_r8x8_col", KIND_TILED, CFG_128x128, ORDER_COL},
    {"valu_t128x128x16_r8x8_xcd", KIND_TILED, CFG_128x128, ORDER_XCD_GROUP},
    {"valu_t64x64x16_r4x4_row", KIND_TILED, CFG_64x64, ORDER_ROW},
    {"valu_t64x64x16_r4x4_xcd", KIND_TILED, CFG_64x64, ORDER_XCD_GROUP},
    {"valu_t128x64x16_r8x4_xcd", KIND_TILED, CFG_128x64, ORDER_XCD_GROUP},
    {"valu_t64x128x16_r4x8_col", KIND_TILED, CFG_64x128, ORDER_COL},
    {"mprod_t128x128x16_w4_xcd", KIND_MPROD, MCFG_128x128_W4, ORDER_XCD_GROUP},
    {"mprod_t128x128x16_w8_xcd", KIND_MPROD, MCFG_128x128_W8, ORDER_XCD_GROUP},
    {"mprod_t256x128x16_w8_xcd", KIND_MPROD, MCFG_256x128_W8, ORDER_XCD_GROUP},
    {"mprod_t64x64x16_w2_row", KIND_MPROD, MCFG_64x64_W2, ORDER_ROW},
    {"mprod_t128x128x16_w4_col", KIND_MPROD, MCFG_128x128_W4, ORDER_COL},
    {"mprod1_t128x128x16_w8_xcd", KIND_MPROD, MCFG_128x128_W8_P1, ORDER_XCD_GROUP},
    {"mprod1_t128x128x16_w4_xcd", KIND_MPROD, MCFG_128x128_W4_P1, ORDER_XCD_GROUP},
    {"mprod1_t256x128x16_w8_xcd", KIND_MPROD, MCFG_256x128_W8_P1, ORDER_XCD_GROUP},
    {"mprod16_t128x128x32_w16_xcd", KIND_MPROD, M16CFG_128x128_W16, ORDER_XCD_GROUP},
    {"mprod16_t128x64x32_w8_xcd", KIND_MPROD, M16CFG_128x64_W8, ORDER_XCD_GROUP},
    {"mprod16_t128x128x16_w8_xcd", KIND_MPROD, M16CFG_128x128_W8, ORDER_XCD_GROUP},
    {"srow_t4x64x32_r1c1_w4_row", KIND_SROW, SCFG_R1C1_W4, ORDER_ROW},
    {"srow_t16x64x32_r4c1_w4_row", KIND_SROW, SCFG_R4C1_W4, ORDER_ROW},
    {"srow_t16x64x32_r4c1_w4_xcd", KIND_SROW, SCFG_R4C1_W4, ORDER_XCD_GROUP},
    {"srow_t8x128x32_r2c2_w4_row", KIND_SROW, SCFG_R2C2_W4, ORDER_ROW},
    {"srow_t32x64x32_r8c1_w4_col", KIND_SROW, SCFG_R8C1_W4, ORDER_COL},
    {"srow_t32x128x32_r4c2_w8_xcd", KIND_SROW, SCFG_R4C2_W8, ORDER_XCD_GROUP},
    {"srow_t64x128x32_r8c2_w8_xcd", KIND_SROW, SCFG_R8C2_W8, ORDER_XCD_GROUP},
    {"mprod1_t128x128x32_w8_xcd", KIND_MPROD, MCFG_128x128_W8_P1_K32, ORDER_XCD_GROUP},
};
constexpr int kNumVariants = static_cast<int>(sizeof(kVariants) / sizeof(kVariants[0]));

// Index of a variant by name (-1 if absent).
int variant_index(const char* name) {
    for (int v = 0; v < kNumVariants; ++v)
        if (strcmp(kVariants[v].name, name) == 0) return v;
    return -1;
}

// Work-items in one dispatch must fit the 32-bit grid size.
constexpr int64_t kMaxBlocks = (int64_t(1) << 32) / 256 - 1;

struct Problem {
    OperandView a, b;
    OutView c;
    int64_t M, N, K, batch;
};

// Largest element offset reached by a (d0 x d1 x d2) block with strides
// (s0, s1, s2), or -1 on int64 overflow.  Requires d >= 1, s >= 0.
int64_t max_offset3(int64_t d0, int64_t d1, int64_t d2, int64_t s0, int64_t s1, int64_t s2) {
    int64_t a, b, c, t, u;
    if (__builtin_mul_overflow(d0 - 1, s0, &a)) return -1;
    if (__builtin_mul_overflow(d1 - 1, s1, &b)) return -1;
    if (__builtin_mul_overflow(d2 - 1, s2, &c)) return -1;
    if (__builtin_add_overflow(a, b, &t)) return -1;
    if (__builtin_add_overflow(t, c, &u)) return -1;
    if (u > INT64_MAX / 4 - 4) return -1;  // byte offsets must fit too
    return u;
}

bool overlaps(const void* p, int64_t p_elems, const void* q, int64_t q_elems) {
    const uintptr_t p0 = reinterpret_cast<uintptr_t>(p), q0 = reinterpret_cast<uintptr_t>(q);
    const uintptr_t p1 = p0 + static_cast<uintptr_t>(p_elems) * 4;
    const uintptr_t q1 = q0 + static_cast<uintptr_t>(q_elems) * 4;
    return p0 < q1 && q0 < p1;
}

// The map (b, i, j) -> b*s0 + i*s1 + j*s2 is injective on the index box.
// Sufficient test (strides >= 0): ordering the axes with extent > 1 by
// stride, each stride exceeds the largest offset the smaller ones reach.
bool injective3(int64_t d0, int64_t d1, int64_t d2, int64_t s0, int64_t s1, int64_t s2) {
    struct Axis {
        int64_t s, d;
    } ax[3] = {{s0, d0}, {s1, d1}, {s2, d2}};
    std::sort(ax, ax + 3, [](const Axis& x, const Axis& y) { return x.s < y.s; });
    int64_t reach = 0;  // largest offset reached by the axes so far
    for (const Axis& a : ax) {
        if (a.d <= 1) continue;
        if (a.s <= reach) return false;
        int64_t span;
        if (__builtin_mul_overflow(a.s, a.d - 1, &span)) return false;
        if (__builtin_add_overflow(reach, span, &reach)) return false;
    }
    return true;
}

// Sizes, flags and variant index.
repops_status check_dims(int64_t M, int64_t N, int64_t K, int64_t batch, int trans_a,
                         int trans_b, int variant) {
    if (M < 0 || N < 0 || K < 0 || batch < 0) return REPOPS_ERR_DIM;
    if ((trans_a != 0 && trans_a != 1) || (trans_b != 0 && trans_b != 1)) return REPOPS_ERR_DIM;
    if (variant < -1 || variant >= kNumVariants) return REPOPS_ERR_VARIANT;
    // Grid limits: the largest grid any variant launches for these sizes.
    const int64_t bm = (M + 15) / 16, bn = (N + 15) / 16;
    if (bm > kMaxBlocks || bn > kMaxBlocks || (bn > 0 && bm > kMaxBlocks / bn))
        return REPOPS_ERR_DIM;
    return REPOPS_OK;
}

// A and B (only when K > 0): pointers, strides, offset overflow; fills the
// X x K operand views and their element extents.
repops_status check_operands(const float* A, int64_t a_bs, int64_t a_rs, int64_t a_cs,
                             const float* B, int64_t b_bs, int64_t b_rs, int64_t b_cs, int64_t M,
                             int64_t N, int64_t K, int64_t batch, int trans_a, int trans_b,
                             Problem* p, int64_t* a_extent, int64_t* b_extent) {
    if (A == nullptr || B == nullptr) return REPOPS_ERR_NULL;
    if (a_bs < 0 || a_rs < 0 || a_cs < 0 || b_bs < 0 || b_rs < 0 || b_cs < 0)
        return REPOPS_ERR_STRIDE;
    // Stored shapes: A is M x K (K x M when transposed), B is K x N (N x K).
    const int64_t a_rows = trans_a ? K : M, a_cols = trans_a ? M : K;
    const int64_t b_rows = trans_b ? N : K, b_cols = trans_b ? K : N;
    const int64_t a_max = max_offset3(batch, a_rows, a_cols, a_bs, a_rs, a_cs);
    const int64_t b_max = max_offset3(batch, b_rows, b_cols, b_bs, b_rs, b_cs);
    if (a_max < 0 || b_max < 0) return REPOPS_ERR_DIM;
    // op(A)(i, k) and op(B)(k, j) as X x K views.
    p->a = OperandView{A, trans_a ? a_cs : a_rs, trans_a ? a_rs : a_cs, M, a_bs};
    p->b = OperandView{B, trans_b ? b_rs : b_cs, trans_b ? b_cs : b_rs, N, b_bs};
    *a_extent = a_max + 1;
    *b_extent = b_max + 1;
    return REPOPS_OK;
}

repops_status validate(const float* A, int64_t a_bs, int64_t a_rs, int64_t a_cs, const float* B,
                       int64_t b_bs, int64_t b_rs, int64_t b_cs, const float* C, int64_t c_bs,
                       int64_t c_rs, int64_t c_cs, int64_t M, int64_t N, int64_t K,
                       int64_t batch, int trans_a, int trans_b, const float* bias,
                       int64_t bias_bs, int64_t bias_s, int variant, Problem* out) {
    repops_status st = check_dims(M, N, K, batch, trans_a, trans_b, variant);
    if (st != REPOPS_OK) return st;
    if (M == 0 || N == 0 || batch == 0) return REPOPS_OK;  // nothing to do
    if (C == nullptr) return REPOPS_ERR_NULL;
    Problem p{};
    p.M = M; p.N = N; p.K = K; p.batch = batch;
    int64_t a_extent = 0, b_extent = 0;
    if (K > 0) {
        st = check_operands(A, a_bs, a_rs, a_cs, B, b_bs, b_rs, b_cs, M, N, K, batch, trans_a,
                            trans_b, &p, &a_extent, &b_extent);
        if (st != REPOPS_OK) return st;
    }
    if (c_bs < 0 || c_rs < 0 || c_cs < 0) return REPOPS_ERR_STRIDE;
    const int64_t c_max = max_offset3(batch, M, N, c_bs, c_rs, c_cs);
    if (c_max < 0) return REPOPS_ERR_DIM;
    if (!injective3(batch, M, N, c_bs, c_rs, c_cs)) return REPOPS_ERR_STRIDE;
    if (K > 0 && (overlaps(C, c_max + 1, A, a_extent) || overlaps(C, c_max + 1, B, b_extent)))
        return REPOPS_ERR_ALIAS;
    p.c = OutView{const_cast<float*>(C), c_rs, c_cs, c_bs, nullptr, 0, 0};
    if (bias != nullptr) {
        if (bias_bs < 0 || bias_s < 0) return REPOPS_ERR_STRIDE;
        const int64_t bias_max = max_offset3(batch, 1, N, bias_bs, 0, bias_s);
        if (bias_max < 0) return REPOPS_ERR_DIM;
        if (overlaps(C, c_max + 1, bias, bias_max + 1)) return REPOPS_ERR_ALIAS;
        p.c.bias = bias;
        p.c.bias_s = bias_s;
        p.c.bias_sb = bias_bs;
    }
    if (out) *out = p;
    return REPOPS_OK;
}

bool aligned16(const float* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Fast loaders need unit stride along one axis, 16-byte aligned base and a
// multiple-of-4 stride along the other axis (so every float4 is aligned);
// loads along x also need 4 | X so a clamped vector stays inside the operand.
int classify(const OperandView& v, int64_t K, int64_t batch) {
    if (!aligned16(v.p)) return LAY_GEN;
    if (batch > 1 && v.s_b % 4 != 0) return LAY_GEN;  // every batch's base must stay aligned
    if (v.s_k == 1 && (v.s_x % 4 == 0 || v.X == 1)) return LAY_KC;
    if (v.s_x == 1 && (v.s_k % 4 == 0 || K == 1) && v.X % 4 == 0) return LAY_XC;
    return LAY_GEN;
}

// The automatic choice.  Below 2^17 outputs the one-row scalar-row kernel.
// Above, the candidate with the least estimated time, where the estimate is
// the busiest CU's share of the work: with T tiles of BM x BN outputs over
// 256 CUs, L = ceil(T / 256) tiles per CU, each at the family's measured
// efficiency with L tiles queued on a CU (from a sweep of square and
// rectangular products from 640 to 8192: a CU with one tile runs below its
// steady rate, and tile counts just above a multiple of 256 leave CUs idle).
// The 128 x 128 product kernel is kept unless another is estimated at least
// 2 % faster: it is the measured best on every transformer-shaped product.
// (The efficiencies are those of the kernel forms each launch runs: with
// more tiles than CUs, the raised-priority forms.)
// The choice never changes a bit.
struct PickFamily {
    const char* name;
    int64_t bm, bn;
    double eff[5];  // efficiency with 1, 2, 3, 4 and 5 or more tiles per CU
};

double pick_estimate(const PickFamily& f, const Problem& p) {
    const int64_t tiles = ((p.M + f.bm - 1) / f.bm) * ((p.N + f.bn - 1) / f.bn) * p.batch;
    const int64_t per_cu = (tiles + 255) / 256;
    const double e = f.eff[per_cu < 5 ? per_cu - 1 : 4];
    return static_cast<double>(per_cu) * static_cast<double>(f.bm * f.bn) / e;
}

int pick(const Problem& p) {
    static const PickFamily kLarge = {"mprod1_t128x128x32_w8_xcd", 128, 128,
                                      {0.75, 0.84, 0.86, 0.87, 0.87}};
    static const PickFamily kOthers[] = {
        {"mprod16_t128x64x32_w8_xcd", 128, 64, {0.65, 0.77, 0.79, 0.83, 0.83}},
        {"srow_t32x128x32_r4c2_w8_xcd", 32, 128, {0.49, 0.55, 0.60, 0.63, 0.63}},
        {"srow_t16x64x32_r4c1_w4_xcd", 16, 64, {0.30, 0.38, 0.45, 0.48, 0.52}},
    };
    static const int tiny = variant_index("srow_t4x64x32_r1c1_w4_row");
    static const int large_index = variant_index(kLarge.name);
    static const int other_index[3] = {variant_index(kOthers[0].name),
                                       variant_index(kOthers[1].name),
                                       variant_index(kOthers[2].name)};
    if (p.M * p.N * p.batch < (int64_t(1) << 17)) return tiny;
    int best = 0;
    double best_t = pick_estimate(kOthers[0], p);
    for (int f = 1; f < 3; ++f) {
        const double t = pick_estimate(kOthers[f], p);
        if (t < best_t) best = f, best_t = t;
    }
    return best_t < 0.98 * pick_estimate(kLarge, p) ? other_index[best] : large_index;
}

// The scalar-row kernels count k, and A's byte offsets along k, in 32 bits;
// beyond that the register-blocked VALU kernel runs instead (every variant
// gives the same bits).
constexpr int64_t kSrowMaxK = (int64_t(1) << 30) - 1;

int runnable(int v, const Problem& p) {
    if (kVariants[v].kind == KIND_SROW && p.K > kSrowMaxK) {
        static const int fallback = variant_index("valu_t64x64x16_r4x4_row");
        return fallback;
    }
    return v;
}

repops_status run(const Problem& p, int variant, void* stream) {
    if (p.M == 0 || p.N == 0 || p.batch == 0) return REPOPS_OK;
    const int v = p.K == 0 ? -1 : runnable(variant < 0 ? pick(p) : variant, p);
    const int la = p.K == 0 ? 0 : classify(p.a, p.K, p.batch);
    const int lb = p.K == 0 ? 0 : classify(p.b, p.K, p.batch);
    // The grid's batch dimension is limited; longer batches run in chunks.
    for (int64_t b0 = 0; b0 < p.batch; b0 += kMaxBatchPerLaunch) {
        const int64_t nb = p.batch - b0 < kMaxBatchPerLaunch ? p.batch - b0 : kMaxBatchPerLaunch;
        OperandView a = p.a, b = p.b;
        OutView c = p.c;
        a.p += b0 * a.s_b;
        b.p += b0 * b.s_b;
        c.p += b0 * c.s_b;
        if (c.bias) c.bias += b0 * c.bias_sb;
        int err;
        if (p.K == 0) {
            err = launch_fill_zero(c, p.M, p.N, nb, stream);
        } else if (kVariants[v].kind == KIND_NAIVE) {
            err = launch_naive(a, b, c, p.M, p.N, p.K, nb, stream);
        } else if (kVariants[v].kind == KIND_SROW) {
            err = launch_srow(kVariants[v].cfg, la, lb, a, b, c, p.M, p.N, p.K, nb,
                              kVariants[v].order, stream);
        } else if (kVariants[v].kind == KIND_MPROD) {
            err = launch_mprod(kVariants[v].cfg, la, lb, a, b, c, p.M, p.N, p.K, nb,
                               kVariants[v].order, stream);
        } else {
            err = launch_tiled(kVariants[v].cfg, la, lb, a, b, c, p.M, p.N, p.K, nb,
                               kVariants[v].order, stream);
        }
        if (err != 0) return REPOPS_ERR_HIP;
    }
    return REPOPS_OK;
}

}  // namespace

extern "C" {

repops_status repops_matmul_batched_f32(const float* A, int64_t a_bs, int64_t a_rs, int64_t a_cs,
                                        const float* B, int64_t b_bs, int64_t b_rs, int64_t b_cs,
                                        float* C, int64_t c_bs, int64_t c_rs, int64_t c_cs,
                                        int64_t M, int64_t N, int64_t K, int64_t batch,
                                        int trans_a, int trans_b, const float* bias,
                                        int64_t bias_bs, int64_t bias_s, void* stream,
                                        int variant) {
    Problem p{};
    const repops_status st = validate(A, a_bs, a_rs, a_cs, B, b_bs, b_rs, b_cs, C, c_bs, c_rs,
                                      c_cs, M, N, K, batch, trans_a, trans_b, bias, bias_bs,
                                      bias_s, variant, &p);
    if (st != REPOPS_OK) return st;
    return run(p, variant, stream);
}

repops_status repops_matmul_f32_ex(const float* A, int64_t a_rs, int64_t a_cs, const float* B,
                                   int64_t b_rs, int64_t b_cs, float* C, int64_t c_rs,
                                   int64_t c_cs, int64_t M, int64_t N, int64_t K, int trans_a,
                                   int trans_b, void* stream, int variant) {
    return repops_matmul_batched_f32(A, 0, a_rs, a_cs, B, 0, b_rs, b_cs, C, 0, c_rs, c_cs, M, N,
                                     K, 1, trans_a, trans_b, nullptr, 0, 0, stream, variant);
}

repops_status repops_matmul_f32(const float* A, int64_t a_rs, int64_t a_cs, const float* B,
                                int64_t b_rs, int64_t b_cs, float* C, int64_t c_rs, int64_t c_cs,
                                int64_t M, int64_t N, int64_t K, int trans_a, int trans_b,
                                void* stream) {
    return repops_matmul_f32_ex(A, a_rs, a_cs, B, b_rs, b_cs, C, c_rs, c_cs, M, N, K, trans_a,
                                trans_b, stream, -1);
}

repops_status repops_check_args_f32(const float* A, int64_t a_rs, int64_t a_cs, const float* B,
                                    int64_t b_rs, int64_t b_cs, const float* C, int64_t c_rs,
                                    int64_t c_cs, int64_t M, int64_t N, int64_t K, int trans_a,
                                    int trans_b, int variant) {
    return validate(A, 0, a_rs, a_cs, B, 0, b_rs, b_cs, C, 0, c_rs, c_cs, M, N, K, 1, trans_a,
                    trans_b, nullptr, 0, 0, variant, nullptr);
}

int repops_pick_variant_f32(const float* A, int64_t a_rs, int64_t a_cs, const float* B,
                            int64_t b_rs, int64_t b_cs, int64_t M, int64_t N, int64_t K,
                            int trans_a, int trans_b) {
    if (M <= 0 || N <= 0 || K <= 0) return -1;
    if (check_dims(M, N, K, 1, trans_a, trans_b, -1) != REPOPS_OK) return -1;
    Problem p{};
    p.M = M; p.N = N; p.K = K; p.batch = 1;
    int64_t ae, be;
    if (check_operands(A, 0, a_rs, a_cs, B, 0, b_rs, b_cs, M, N, K, 1, trans_a, trans_b, &p, &ae,
                       &be) != REPOPS_OK)
        return -1;
    return runnable(pick(p), p);
}

int repops_variant_count(void) { return kNumVariants; }

const char* repops_variant_name(int variant) {
    if (variant < 0 || variant >= kNumVariants) return "?";
    return kVariants[variant].name;
}

const char* repops_strerror(repops_status status) {
    switch (status) {
        case REPOPS_OK: return "success";
        case REPOPS_ERR_NULL: return "a required pointer is NULL";
        case REPOPS_ERR_DIM: return "invalid size, transpose flag or offset overflow";
        case REPOPS_ERR_STRIDE: return "negative stride or overlapping output strides";
        case REPOPS_ERR_ALIAS: return "output overlaps an input";
        case REPOPS_ERR_VARIANT: return "unknown kernel variant";
        case REPOPS_ERR_HIP: return "HIP launch error";
        case REPOPS_ERR_DUPLICATE: return "two contributors share one identity";
        case REPOPS_ERR_ALIGN: return "a pointer is not aligned as the call requires";
        case REPOPS_ERR_WORKSPACE: return "the workspace is missing or too small";
        case REPOPS_ERR_SCRATCH:
            return "the call needs more scratch than the library's static buffer holds";
    }
    return "unknown status";
}

const char* repops_build_manifest(void) {
    // Built once; function-local static initialisation is thread-safe.
    static const struct Text {
        char buf[4096];
        Text() {
            size_t n = 0;
            buf[0] = 0;
            auto put = [&](const char* s) {
                const size_t l = strlen(s);
                if (n + l + 1 < sizeof(buf)) { memcpy(buf + n, s, l); n += l; buf[n] = 0; }
            };
            put("{\"library\": \"repops\", \"compiler\": \"");
            put(__VERSION__);
            put("\", \"offload_arch\": \"" REPOPS_OFFLOAD_ARCH "\", \"flags\": \""
                REPOPS_BUILD_FLAGS "\", \"variants\": [");
            for (int v = 0; v < kNumVariants; ++v) {
                put(v ? ", \"" : "\"");
                put(kVariants[v].name);
                put("\"");
            }
            put("]}");
        }
    } text;
    return text.buf;
}

}  // extern "C"
