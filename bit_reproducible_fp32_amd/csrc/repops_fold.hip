// gfx950 kernel for the fixed-order gradient average and SGD step (Zoo
// Per-LLM Chain Soundness, "Detailed proof: deterministic ordering":
// "Ordering subroutine", "Determinism of left-fold", "Update step").
//
// Element e of the d parameters, for contributors in the canonical order:
//     S = (((g_0[e] + g_1[e]) + g_2[e]) + ...) + g_{k-1}[e]
//     gbar[e] = RN(RN(1/k) * S)
//     theta[e] = RN(theta[e] - RN(eta * gbar[e]))
// Parameters are a free dimension (any lane, any order); the contributors
// are the fixed-order dimension and every lane walks them in order.  Each
// operation is a separately rounded binary32 operation (-ffp-contract=off and
// the pragma below; the build's instruction scan rejects fused forms).
//
// One pass reads at most kFoldMax contributors.  A longer fold runs several
// passes on one stream: the first starts from g_0, later passes start from
// the running sum left in `sum` by the previous pass, and only the last pass
// scales and updates.  The operation sequence per element is unchanged.
#include <hip/hip_runtime.h>

#include "repops_internal.h"

#pragma clang fp contract(off)

namespace repops {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Streaming loads (each gradient is read once).  V is float or f32x4; vector
// arithmetic below is elementwise: each lane is its own separately rounded
// binary32 operation.
template <typename V>
__device__ __forceinline__ V ld(const float* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const V*>(p));
}

template <typename V>
__device__ __forceinline__ void st(float* p, V v) {
    *reinterpret_cast<V*>(p) = v;
}

// One element (V = float) or four (V = f32x4) of one pass.  Contributors are
// taken in chunks of 8: the chunk's loads are issued together, then added to
// the running sum one by one in order.
template <typename V>
__device__ __forceinline__ void fold_at(const FoldArgs& G, int n, bool first, bool last,
                                        float* sum, float* theta, float* gbar, float inv_k,
                                        float eta, int64_t e) {
    V s = first ? ld<V>(G.g[0] + e) : ld<V>(sum + e);
    V th;
    if (last) th = ld<V>(theta + e);  // issued with the gradients' loads
    for (int c = first ? 1 : 0; c < n; c += 8) {
        V x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (c + u < n) x[u] = ld<V>(G.g[c + u] + e);
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (c + u < n) s = s + x[u];
    }
    if (!last) {
        st<V>(sum + e, s);
        return;
    }
    const V gb = inv_k * s;
    if (gbar) st<V>(gbar + e, gb);
    const V step = eta * gb;
    st<V>(theta + e, th - step);
}

// VEC: every pointer is 16-byte aligned; float4 over the first 4*(d/4)
// elements, scalars for the rest.
template <bool VEC>
__global__ __launch_bounds__(256) void repops_fold_kernel(FoldArgs G, int n, int first, int last,
                                                          float* sum, float* theta, float* gbar,
                                                          float inv_k, float eta, int64_t d) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    int64_t scalar_from = 0;
    if constexpr (VEC) {
        const int64_t nv = d >> 2;
        for (int64_t v = t0; v < nv; v += stride)
            fold_at<f32x4>(G, n, first, last, sum, theta, gbar, inv_k, eta, v << 2);
        scalar_from = nv << 2;
    }
    for (int64_t e = scalar_from + t0; e < d; e += stride)
        fold_at<float>(G, n, first, last, sum, theta, gbar, inv_k, eta, e);
}

}  // namespace

int launch_fold(const FoldArgs& G, int n, bool first, bool last, float* sum, float* theta,
                float* gbar, float inv_k, float eta, int64_t d, bool vec, void* stream) {
    // One item (a float4, or one float) per lane: measured faster than fewer
    // workgroups looping (6.4 vs 5.6-5.9 TB/s at k=8); grid-stride only past
    // 2^20 workgroups.
    const int64_t items = vec ? (d >> 2) + 3 : d;
    int64_t blocks = (items + 255) / 256;
    if (blocks > (int64_t(1) << 20)) blocks = int64_t(1) << 20;
    if (blocks < 1) blocks = 1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (vec)
        hipLaunchKernelGGL(repops_fold_kernel<true>, dim3(static_cast<unsigned>(blocks)), dim3(256),
                           0, s, G, n, first ? 1 : 0, last ? 1 : 0, sum, theta, gbar, inv_k, eta, d);
    else
        hipLaunchKernelGGL(repops_fold_kernel<false>, dim3(static_cast<unsigned>(blocks)),
                           dim3(256), 0, s, G, n, first ? 1 : 0, last ? 1 : 0, sum, theta, gbar,
                           inv_k, eta, d);
    return static_cast<int>(hipGetLastError());
}

}  // namespace repops
