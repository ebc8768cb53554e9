// C-ABI front end of the fixed-order gradient average / SGD step and the
// canonical contributor order.  Host C++; the kernel is in repops_fold.hip.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "../../include/repops.h"
#include "repops_internal.h"

#pragma clang fp contract(off)

using namespace repops;

namespace {

bool overlap(const float* p, const float* q, int64_t d) {
    const uintptr_t p0 = reinterpret_cast<uintptr_t>(p), q0 = reinterpret_cast<uintptr_t>(q);
    const uintptr_t n = static_cast<uintptr_t>(d) * 4;
    return p0 < q0 + n && q0 < p0 + n;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Byte-lexicographic comparison: first differing byte (unsigned) decides, else
// the shorter identity first.
int compare_ids(const uint8_t* a, int64_t la, const uint8_t* b, int64_t lb) {
    const int64_t n = la < lb ? la : lb;
    if (n > 0) {
        const int r = memcmp(a, b, static_cast<size_t>(n));
        if (r != 0) return r;
    }
    return la < lb ? -1 : (la > lb ? 1 : 0);
}

}  // namespace

extern "C" {

repops_status repops_canonical_order(const uint8_t* const* dids, const int64_t* did_lens,
                                     int64_t k, int64_t* order_out) {
    if (k < 0) return REPOPS_ERR_DIM;
    if (k == 0) return REPOPS_OK;
    if (dids == nullptr || did_lens == nullptr || order_out == nullptr) return REPOPS_ERR_NULL;
    for (int64_t c = 0; c < k; ++c) {
        if (did_lens[c] < 0) return REPOPS_ERR_DIM;
        if (did_lens[c] > 0 && dids[c] == nullptr) return REPOPS_ERR_NULL;
    }
    std::vector<int64_t> idx(static_cast<size_t>(k));
    for (int64_t c = 0; c < k; ++c) idx[static_cast<size_t>(c)] = c;
    std::sort(idx.begin(), idx.end(), [&](int64_t x, int64_t y) {
        return compare_ids(dids[x], did_lens[x], dids[y], did_lens[y]) < 0;
    });
    for (int64_t r = 1; r < k; ++r) {
        const int64_t x = idx[static_cast<size_t>(r - 1)], y = idx[static_cast<size_t>(r)];
        if (compare_ids(dids[x], did_lens[x], dids[y], did_lens[y]) == 0)
            return REPOPS_ERR_DUPLICATE;
    }
    for (int64_t r = 0; r < k; ++r) order_out[r] = idx[static_cast<size_t>(r)];
    return REPOPS_OK;
}

repops_status repops_fold_mean_sgd_f32(const float* const* grads, int64_t k, int64_t d,
                                       float eta, float* theta, float* gbar, void* stream) {
    if (k < 1 || k > (int64_t(1) << 24) || d < 0) return REPOPS_ERR_DIM;
    if (d > INT64_MAX / 16) return REPOPS_ERR_DIM;
    if (d == 0) return REPOPS_OK;
    if (grads == nullptr || theta == nullptr) return REPOPS_ERR_NULL;
    if (gbar == nullptr && k > kFoldMax) return REPOPS_ERR_NULL;
    bool vec = aligned16(theta) && (gbar == nullptr || aligned16(gbar));
    for (int64_t c = 0; c < k; ++c) {
        if (grads[c] == nullptr) return REPOPS_ERR_NULL;
        if (overlap(grads[c], theta, d)) return REPOPS_ERR_ALIAS;
        if (gbar && overlap(grads[c], gbar, d)) return REPOPS_ERR_ALIAS;
        vec = vec && aligned16(grads[c]);
    }
    if (gbar && overlap(gbar, theta, d)) return REPOPS_ERR_ALIAS;

    // 1/k as a binary32 quotient, rounded once (k <= 2^24 converts exactly).
    const float inv_k = 1.0f / static_cast<float>(k);
    for (int64_t c0 = 0; c0 < k; c0 += kFoldMax) {
        const int n = static_cast<int>(k - c0 < kFoldMax ? k - c0 : kFoldMax);
        FoldArgs G{};
        for (int c = 0; c < n; ++c) G.g[c] = grads[c0 + c];
        const bool first = c0 == 0, last = c0 + n == k;
        const int err = launch_fold(G, n, first, last, gbar, theta, gbar, inv_k, eta, d, vec,
                                    stream);
        if (err != 0) return REPOPS_ERR_HIP;
    }
    return REPOPS_OK;
}

}  // extern "C"
