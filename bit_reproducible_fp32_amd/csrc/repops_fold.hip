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

__device__ __forceinline__ float add_rn(float a, float b) { return a + b; }
__device__ __forceinline__ float mul_rn(float a, float b) { return a * b; }
__device__ __forceinline__ float sub_rn(float a, float b) { return a - b; }

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Streaming 16-byte load (each gradient is read once).
__device__ __forceinline__ float4 ld4(const float* p) {
    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}

// One element (or one float4 of elements) of one pass.
template <typename T>
struct Lanes;

template <>
struct Lanes<float> {
    __device__ static float load(const float* p) { return __builtin_nontemporal_load(p); }
    __device__ static float add(float a, float b) { return add_rn(a, b); }
    __device__ static float scale(float a, float s) { return mul_rn(s, a); }
    __device__ static float update(float th, float eta, float gb) {
        return sub_rn(th, mul_rn(eta, gb));
    }
    __device__ static void store(float* p, float v) { *p = v; }
};

template <>
struct Lanes<float4> {
    __device__ static float4 load(const float* p) { return ld4(p); }
    __device__ static float4 add(float4 a, float4 b) {
        return make_float4(add_rn(a.x, b.x), add_rn(a.y, b.y), add_rn(a.z, b.z), add_rn(a.w, b.w));
    }
    __device__ static float4 scale(float4 a, float s) {
        return make_float4(mul_rn(s, a.x), mul_rn(s, a.y), mul_rn(s, a.z), mul_rn(s, a.w));
    }
    __device__ static float4 update(float4 th, float eta, float4 gb) {
        return make_float4(sub_rn(th.x, mul_rn(eta, gb.x)), sub_rn(th.y, mul_rn(eta, gb.y)),
                           sub_rn(th.z, mul_rn(eta, gb.z)), sub_rn(th.w, mul_rn(eta, gb.w)));
    }
    __device__ static void store(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
};

template <typename T>
__device__ __forceinline__ void fold_at(const FoldArgs& G, int n, bool first, bool last,
                                        float* sum, float* theta, float* gbar, float inv_k,
                                        float eta, int64_t e) {
    using L = Lanes<T>;
    T s = first ? L::load(G.g[0] + e) : L::load(sum + e);
    // Contributors in order; loads may be issued ahead, the adds stay in order.
#pragma unroll 8
    for (int c = first ? 1 : 0; c < n; ++c) s = L::add(s, L::load(G.g[c] + e));
    if (!last) {
        L::store(sum + e, s);
        return;
    }
    const T gb = L::scale(s, inv_k);
    if (gbar) L::store(gbar + e, gb);
    L::store(theta + e, L::update(L::load(theta + e), eta, gb));
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
            fold_at<float4>(G, n, first, last, sum, theta, gbar, inv_k, eta, v << 2);
        scalar_from = nv << 2;
    }
    for (int64_t e = scalar_from + t0; e < d; e += stride)
        fold_at<float>(G, n, first, last, sum, theta, gbar, inv_k, eta, e);
}

}  // namespace

int launch_fold(const FoldArgs& G, int n, bool first, bool last, float* sum, float* theta,
                float* gbar, float inv_k, float eta, int64_t d, bool vec, void* stream) {
    // Enough workgroups to keep every CU streaming; grid-stride beyond that.
    const int64_t items = vec ? (d >> 2) + 3 : d;
    int64_t blocks = (items + 255) / 256;
    if (blocks > 256 * 16) blocks = 256 * 16;
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
