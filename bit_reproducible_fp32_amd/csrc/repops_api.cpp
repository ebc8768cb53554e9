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

enum Kind { KIND_NAIVE = 0, KIND_TILED = 1, KIND_MPROD = 2 };

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
    int64_t M, N, K;
};

// Largest element offset reached by (rows x cols) with strides (rs, cs), or
// -1 on int64 overflow.  Requires rows, cols >= 1 and rs, cs >= 0.
int64_t max_offset(int64_t rows, int64_t cols, int64_t rs, int64_t cs) {
    int64_t a, b, s;
    if (__builtin_mul_overflow(rows - 1, rs, &a)) return -1;
    if (__builtin_mul_overflow(cols - 1, cs, &b)) return -1;
    if (__builtin_add_overflow(a, b, &s)) return -1;
    if (s > INT64_MAX / 4 - 4) return -1;  // byte offsets must fit too
    return s;
}

bool overlaps(const void* p, int64_t p_elems, const void* q, int64_t q_elems) {
    const uintptr_t p0 = reinterpret_cast<uintptr_t>(p), q0 = reinterpret_cast<uintptr_t>(q);
    const uintptr_t p1 = p0 + static_cast<uintptr_t>(p_elems) * 4;
    const uintptr_t q1 = q0 + static_cast<uintptr_t>(q_elems) * 4;
    return p0 < q1 && q0 < p1;
}

// C's strides map distinct (i, j) to distinct elements.  Sufficient test
// (strides >= 0): the smaller stride is nonzero when its extent is > 1 and
// the larger stride steps over a whole run of the smaller one.
bool injective(int64_t M, int64_t N, int64_t s_i, int64_t s_j) {
    if (M > 1 && s_i == 0) return false;
    if (N > 1 && s_j == 0) return false;
    if (M <= 1 || N <= 1) return true;
    int64_t s_small = s_i, d_small = M, s_big = s_j;
    if (s_j < s_i || (s_j == s_i && N < M)) {
        s_small = s_j; d_small = N; s_big = s_i;
    }
    int64_t need;
    if (__builtin_mul_overflow(s_small, d_small, &need)) return false;
    return s_big >= need;
}

// Sizes, flags and variant index.
repops_status check_dims(int64_t M, int64_t N, int64_t K, int trans_a, int trans_b,
                         int variant) {
    if (M < 0 || N < 0 || K < 0) return REPOPS_ERR_DIM;
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
repops_status check_operands(const float* A, int64_t a_rs, int64_t a_cs, const float* B,
                             int64_t b_rs, int64_t b_cs, int64_t M, int64_t N, int64_t K,
                             int trans_a, int trans_b, Problem* p, int64_t* a_extent,
                             int64_t* b_extent) {
    if (A == nullptr || B == nullptr) return REPOPS_ERR_NULL;
    if (a_rs < 0 || a_cs < 0 || b_rs < 0 || b_cs < 0) return REPOPS_ERR_STRIDE;
    // Stored shapes: A is M x K (K x M when transposed), B is K x N (N x K).
    const int64_t a_rows = trans_a ? K : M, a_cols = trans_a ? M : K;
    const int64_t b_rows = trans_b ? N : K, b_cols = trans_b ? K : N;
    const int64_t a_max = max_offset(a_rows, a_cols, a_rs, a_cs);
    const int64_t b_max = max_offset(b_rows, b_cols, b_rs, b_cs);
    if (a_max < 0 || b_max < 0) return REPOPS_ERR_DIM;
    // op(A)(i, k) and op(B)(k, j) as X x K views.
    p->a = OperandView{A, trans_a ? a_cs : a_rs, trans_a ? a_rs : a_cs, M};
    p->b = OperandView{B, trans_b ? b_rs : b_cs, trans_b ? b_cs : b_rs, N};
    *a_extent = a_max + 1;
    *b_extent = b_max + 1;
    return REPOPS_OK;
}

repops_status validate(const float* A, int64_t a_rs, int64_t a_cs, const float* B, int64_t b_rs,
                       int64_t b_cs, const float* C, int64_t c_rs, int64_t c_cs, int64_t M,
                       int64_t N, int64_t K, int trans_a, int trans_b, int variant,
                       Problem* out) {
    repops_status st = check_dims(M, N, K, trans_a, trans_b, variant);
    if (st != REPOPS_OK) return st;
    if (M == 0 || N == 0) return REPOPS_OK;  // nothing to do
    if (C == nullptr) return REPOPS_ERR_NULL;
    Problem p{};
    p.M = M; p.N = N; p.K = K;
    int64_t a_extent = 0, b_extent = 0;
    if (K > 0) {
        st = check_operands(A, a_rs, a_cs, B, b_rs, b_cs, M, N, K, trans_a, trans_b, &p,
                            &a_extent, &b_extent);
        if (st != REPOPS_OK) return st;
    }
    if (c_rs < 0 || c_cs < 0) return REPOPS_ERR_STRIDE;
    const int64_t c_max = max_offset(M, N, c_rs, c_cs);
    if (c_max < 0) return REPOPS_ERR_DIM;
    if (!injective(M, N, c_rs, c_cs)) return REPOPS_ERR_STRIDE;
    if (K > 0 && (overlaps(C, c_max + 1, A, a_extent) || overlaps(C, c_max + 1, B, b_extent)))
        return REPOPS_ERR_ALIAS;
    p.c = OutView{const_cast<float*>(C), c_rs, c_cs};
    if (out) *out = p;
    return REPOPS_OK;
}

bool aligned16(const float* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Fast loaders need unit stride along one axis, 16-byte aligned base and a
// multiple-of-4 stride along the other axis (so every float4 is aligned);
// loads along x also need 4 | X so a clamped vector stays inside the operand.
int classify(const OperandView& v, int64_t K) {
    if (!aligned16(v.p)) return LAY_GEN;
    if (v.s_k == 1 && (v.s_x % 4 == 0 || v.X == 1)) return LAY_KC;
    if (v.s_x == 1 && (v.s_k % 4 == 0 || K == 1) && v.X % 4 == 0) return LAY_XC;
    return LAY_GEN;
}

int pick(const Problem& p) {
    static const int large = variant_index("mprod1_t128x128x16_w8_xcd");
    static const int small = variant_index("valu_t64x64x16_r4x4_row");
    const int64_t tiles = ((p.M + 127) / 128) * ((p.N + 127) / 128);
    // 256 CUs: 128x128 product tiles when there are at least two per CU;
    // below that the problem cannot fill the chip and the 64x64 VALU tiles
    // (more workgroups, measured faster at 256^3 and 1024^3) win.
    return tiles >= 512 ? large : small;
}

repops_status run(const Problem& p, int variant, void* stream) {
    if (p.M == 0 || p.N == 0) return REPOPS_OK;
    int err;
    if (p.K == 0) {
        err = launch_fill_zero(p.c, p.M, p.N, stream);
    } else {
        const int v = variant < 0 ? pick(p) : variant;
        const Variant& var = kVariants[v];
        if (var.kind == KIND_NAIVE) {
            err = launch_naive(p.a, p.b, p.c, p.M, p.N, p.K, stream);
        } else if (var.kind == KIND_MPROD) {
            err = launch_mprod(var.cfg, classify(p.a, p.K), classify(p.b, p.K), p.a, p.b, p.c,
                               p.M, p.N, p.K, var.order, stream);
        } else {
            err = launch_tiled(var.cfg, classify(p.a, p.K), classify(p.b, p.K), p.a, p.b, p.c,
                               p.M, p.N, p.K, var.order, stream);
        }
    }
    return err == 0 ? REPOPS_OK : REPOPS_ERR_HIP;
}

}  // namespace

extern "C" {

repops_status repops_matmul_f32_ex(const float* A, int64_t a_rs, int64_t a_cs, const float* B,
                                   int64_t b_rs, int64_t b_cs, float* C, int64_t c_rs,
                                   int64_t c_cs, int64_t M, int64_t N, int64_t K, int trans_a,
                                   int trans_b, void* stream, int variant) {
    Problem p{};
    const repops_status st = validate(A, a_rs, a_cs, B, b_rs, b_cs, C, c_rs, c_cs, M, N, K,
                                      trans_a, trans_b, variant, &p);
    if (st != REPOPS_OK) return st;
    return run(p, variant, stream);
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
    return validate(A, a_rs, a_cs, B, b_rs, b_cs, C, c_rs, c_cs, M, N, K, trans_a, trans_b,
                    variant, nullptr);
}

int repops_pick_variant_f32(const float* A, int64_t a_rs, int64_t a_cs, const float* B,
                            int64_t b_rs, int64_t b_cs, int64_t M, int64_t N, int64_t K,
                            int trans_a, int trans_b) {
    if (M <= 0 || N <= 0 || K <= 0) return -1;
    if (check_dims(M, N, K, trans_a, trans_b, -1) != REPOPS_OK) return -1;
    Problem p{};
    p.M = M; p.N = N; p.K = K;
    int64_t ae, be;
    if (check_operands(A, a_rs, a_cs, B, b_rs, b_cs, M, N, K, trans_a, trans_b, &p, &ae, &be) !=
        REPOPS_OK)
        return -1;
    return pick(p);
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
