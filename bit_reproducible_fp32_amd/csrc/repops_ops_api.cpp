// C-ABI front end of ERF, GeLU and LayerNorm (Verde and RepOps article,
// section 4.3).  Host C++; the kernels are in repops_ops.hip.
#include <stdint.h>

#include "../../include/repops.h"
#include "repops_internal.h"

using namespace repops;

namespace {

constexpr int64_t kMaxElems = int64_t(1) << 46;
constexpr int64_t kMaxRows = int64_t(0x7fffffff) * 64;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Byte spans [p, p + 4*n) overlap (empty spans never do).
bool overlap(const void* p, int64_t n, const void* q, int64_t m) {
    if (p == nullptr || q == nullptr || n <= 0 || m <= 0) return false;
    const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
    return a < b + static_cast<uintptr_t>(m) * 4 && b < a + static_cast<uintptr_t>(n) * 4;
}

repops_status unary(int op, const float* x, float* y, int64_t n, void* stream) {
    if (n < 0 || n > kMaxElems) return REPOPS_ERR_DIM;
    if (n == 0) return REPOPS_OK;
    if (x == nullptr || y == nullptr) return REPOPS_ERR_NULL;
    if (x != y && overlap(x, n, y, n)) return REPOPS_ERR_ALIAS;
    const bool vec = aligned16(x) && aligned16(y);
    return launch_unary(op, x, y, n, vec, stream) == 0 ? REPOPS_OK : REPOPS_ERR_HIP;
}

}  // namespace

extern "C" {

repops_status repops_erf_f32(const float* x, float* y, int64_t n, void* stream) {
    return unary(0, x, y, n, stream);
}

repops_status repops_gelu_f32(const float* x, float* y, int64_t n, void* stream) {
    return unary(1, x, y, n, stream);
}

repops_status repops_layernorm_f32(const float* x, int64_t x_rs, const float* gamma,
                                   const float* beta, float* y, int64_t y_rs, int64_t rows,
                                   int64_t H, float eps, float* mean, float* rstd, void* stream) {
    if (rows < 0 || rows > kMaxRows) return REPOPS_ERR_DIM;
    if (rows == 0) return REPOPS_OK;
    if (H < 1 || H > (int64_t(1) << 24)) return REPOPS_ERR_DIM;
    if (x_rs < 0 || (rows > 1 && y_rs < H) || y_rs < 0) return REPOPS_ERR_STRIDE;
    const int64_t widest = x_rs > y_rs ? x_rs : y_rs;
    if (rows - 1 > (kMaxElems - H) / (widest > 0 ? widest : 1)) return REPOPS_ERR_DIM;
    if (x == nullptr || y == nullptr) return REPOPS_ERR_NULL;
    const int64_t xs = (rows - 1) * x_rs + H, ys = (rows - 1) * y_rs + H;
    const bool in_place = x == y && x_rs == y_rs;
    if (!in_place && overlap(x, xs, y, ys)) return REPOPS_ERR_ALIAS;
    if (overlap(gamma, H, y, ys) || overlap(beta, H, y, ys)) return REPOPS_ERR_ALIAS;
    const void* outs[2] = {mean, rstd};
    for (const void* o : outs) {
        if (overlap(o, rows, x, xs) || overlap(o, rows, y, ys) || overlap(o, rows, gamma, H) ||
            overlap(o, rows, beta, H))
            return REPOPS_ERR_ALIAS;
    }
    if (overlap(mean, rows, rstd, rows)) return REPOPS_ERR_ALIAS;
    const bool vec = aligned16(x) && aligned16(y) && (gamma == nullptr || aligned16(gamma)) &&
                     (beta == nullptr || aligned16(beta)) && (x_rs & 3) == 0 &&
                     (y_rs & 3) == 0 && (H & 3) == 0;
    return launch_layernorm(x, x_rs, gamma, beta, y, y_rs, rows, H, eps, mean, rstd, vec,
                            stream) == 0
               ? REPOPS_OK
               : REPOPS_ERR_HIP;
}

}  // extern "C"
