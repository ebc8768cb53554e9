// gfx950 kernels for the other RepOps operators the Verde and RepOps article
// names (section 4.3: LayerNorm, GeLU, ERF).  Each evaluates one fixed
// sequence of binary32 operations, every +, -, *, / and square root rounded to
// nearest even on its own with gradual underflow (no contraction: the pragma
// below and -ffp-contract=off; division and square root are the correctly
// rounded IEEE operations), so the bits do not depend on the launch shape.
//
// erf x, in two pieces split at |x| = 1:
//   |x| < 1:  the Maclaurin series (2/sqrt pi) sum_n (-1)^n x^(2n+1) / (n! (2n+1)),
//             n = 0..10, coefficients rounded to binary32; w = x*x, Horner's
//             rule in w from c10 down, then times x.
//   |x| >= 1 (and NaN): Abramowitz and Stegun, Handbook of Mathematical
//             Functions (1964), 7.1.28: erf y = 1 - 1/(1 + a1 y + ... + a6 y^6)^16,
//             y = |x|; Horner's rule from a6 down, the 16th power by four
//             squarings, r = 1/q, e = 1 - r, the sign of x.
// GeLU x = (x * 0.5) * (1 + erf(x * c)), c = 1/sqrt 2 rounded to binary32.
// LayerNorm of a row of H (Ba, Kiros and Hinton 2016): ascending sums from +0,
//   mu = S/H, var = (sum of (x_i - mu)^2)/H, rstd = 1/sqrt(var + eps),
//   y_i = ((x_i - mu) * rstd) * gamma_i + beta_i.
#include <hip/hip_runtime.h>

#include "repops_internal.h"

#pragma clang fp contract(off)

namespace repops {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// (2/sqrt pi) (-1)^n / (n! (2n+1)), n = 0..10, to 22 significant digits.
constexpr float kErfSeries[11] = {
    1.128379167095512573896e+0f, -3.761263890318375246321e-1f, 1.128379167095512573896e-1f,
    -2.686617064513125175943e-2f, 5.223977625442187842112e-3f, -8.548327023450852832547e-4f,
    1.205533298178966425103e-4f, -1.492565035840625097746e-5f, 1.646211436588924740161e-6f,
    -1.636584469123492431739e-7f, 1.480719281587921723955e-8f};
// Abramowitz and Stegun 7.1.28: a1 .. a6.
constexpr float kErfAS[6] = {0.0705230784f, 0.0422820123f, 0.0092705272f,
                             0.0001520143f, 0.0002765672f, 0.0000430638f};
constexpr float kInvSqrt2 = 0.70710678118654752440f;

__device__ __forceinline__ float erf_fixed(float x) {
    const float y = __builtin_fabsf(x);
    if (y < 1.0f) {
        const float w = x * x;
        float s = kErfSeries[10];
#pragma unroll
        for (int n = 9; n >= 0; --n) {
            s = s * w;
            s = s + kErfSeries[n];
        }
        return s * x;
    }
    float p = kErfAS[5];
#pragma unroll
    for (int i = 4; i >= 0; --i) {
        p = p * y;
        p = p + kErfAS[i];
    }
    p = p * y;
    p = p + 1.0f;
    float q = p * p;
    q = q * q;
    q = q * q;
    q = q * q;
    const float r = 1.0f / q;
    const float e = 1.0f - r;
    return __builtin_copysignf(e, x);
}

__device__ __forceinline__ float gelu_fixed(float x) {
    const float u = x * kInvSqrt2;
    const float e = erf_fixed(u);
    const float h = x * 0.5f;
    const float t = 1.0f + e;
    return h * t;
}

template <int OP>
__device__ __forceinline__ float unary(float x) {
    return OP == 0 ? erf_fixed(x) : gelu_fixed(x);
}

// OP 0: erf, 1: GeLU.  VEC: x and y 16-byte aligned; lanes take one float4
// each over the first 4*(n/4) elements, then single elements.
// y may be x itself (each element is read and then written by one lane).
template <int OP, bool VEC>
__global__ __launch_bounds__(256) void repops_unary_kernel(const float* x, float* y, int64_t n) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    int64_t from = 0;
    if constexpr (VEC) {
        const int64_t nv = n >> 2;
        for (int64_t v = t0; v < nv; v += stride) {
            const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(x) + v);
            f32x4 b;
            b.x = unary<OP>(a.x);
            b.y = unary<OP>(a.y);
            b.z = unary<OP>(a.z);
            b.w = unary<OP>(a.w);
            __builtin_nontemporal_store(b, reinterpret_cast<f32x4*>(y) + v);
        }
        from = nv << 2;
    }
    for (int64_t e = from + t0; e < n; e += stride) y[e] = unary<OP>(x[e]);
}

// Four consecutive floats of a row (VEC: one 16-byte load).
template <bool VEC>
__device__ __forceinline__ f32x4 load4(const float* p) {
    if constexpr (VEC) {
        return *reinterpret_cast<const f32x4*>(p);
    } else {
        f32x4 v;
        v.x = p[0];
        v.y = p[1];
        v.z = p[2];
        v.w = p[3];
        return v;
    }
}

template <bool VEC>
__device__ __forceinline__ void store4(float* p, f32x4 v) {
    if constexpr (VEC) {
        *reinterpret_cast<f32x4*>(p) = v;
    } else {
        p[0] = v.x;
        p[1] = v.y;
        p[2] = v.z;
        p[3] = v.w;
    }
}

// Rows are walked in blocks of 16 floats in ascending order.  One lane owns
// a row and there are only as many lanes as rows, so the latency of each
// lane's loads is hidden by keeping several blocks of its row in flight: a
// ring of blocks in registers, each refilled as soon as it has been used.
constexpr int kRing = 8;      // blocks in flight in the two summing passes
constexpr int kRingOut = 4;   // blocks (of x, gamma and beta) in the output pass

template <bool VEC>
__device__ __forceinline__ void load_block(const float* p, f32x4 (&b)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) b[q] = load4<VEC>(p + 4 * q);
}

// f(v) for every float4 v of the first 16*nblk floats of row xr, in order.
template <bool VEC, typename F>
__device__ __forceinline__ void walk_row(const float* xr, int64_t nblk, F&& f) {
    f32x4 ring[kRing][4];
#pragma unroll
    for (int j = 0; j < kRing; ++j)
        if (j < nblk) load_block<VEC>(xr + 16 * j, ring[j]);
    for (int64_t base = 0; base < nblk; base += kRing) {
#pragma unroll
        for (int j = 0; j < kRing; ++j) {
            const int64_t blk = base + j;
            if (blk < nblk) {
                f32x4 cur[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) cur[q] = ring[j][q];
                if (blk + kRing < nblk) load_block<VEC>(xr + 16 * (blk + kRing), ring[j]);
#pragma unroll
                for (int q = 0; q < 4; ++q) f(cur[q]);
            }
        }
    }
}

// One lane per row (the sums over a row are the fixed-order dimension; rows
// are free).  VEC: x, y, gamma, beta 16-byte aligned and x_rs, y_rs, H
// multiples of 4.  y may be x itself with y_rs == x_rs: a lane rewrites only
// its own row, after its last read of each element.
template <bool VEC>
__global__ __launch_bounds__(64) void repops_layernorm_kernel(
    const float* x, int64_t x_rs, const float* __restrict__ gamma,
    const float* __restrict__ beta, float* y, int64_t y_rs, int64_t rows, int64_t H, float eps,
    float* __restrict__ mean_out, float* __restrict__ rstd_out) {
    const int64_t r = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (r >= rows) return;
    const float* xr = x + r * x_rs;
    float* yr = y + r * y_rs;
    const int64_t nblk = H >> 4;
    const int64_t tail = nblk << 4;
    const float fh = static_cast<float>(H);

    // pass 1: S = ((+0 + x_0) + x_1) + ...
    float s = 0.0f;
    walk_row<VEC>(xr, nblk, [&](f32x4 v) {
        s = s + v.x;
        s = s + v.y;
        s = s + v.z;
        s = s + v.w;
    });
    for (int64_t i = tail; i < H; ++i) s = s + xr[i];
    const float mu = s / fh;

    // pass 2: S2 = sum of (x_i - mu)^2 in the same order
    float s2 = 0.0f;
    walk_row<VEC>(xr, nblk, [&](f32x4 v) {
        const f32x4 d = v - mu;
        const f32x4 sq = d * d;
        s2 = s2 + sq.x;
        s2 = s2 + sq.y;
        s2 = s2 + sq.z;
        s2 = s2 + sq.w;
    });
    for (int64_t i = tail; i < H; ++i) {
        const float d = xr[i] - mu;
        const float sq = d * d;
        s2 = s2 + sq;
    }
    const float var = s2 / fh;
    const float ve = var + eps;
    const float sd = __builtin_sqrtf(ve);
    const float rs = 1.0f / sd;

    // pass 3: y_i = ((x_i - mu) * rstd) * gamma_i + beta_i, with blocks of x,
    // gamma and beta in flight.
    {
        f32x4 rx[kRingOut][4], rg[kRingOut][4], rb[kRingOut][4];
        auto fill = [&](int j, int64_t blk) {
            load_block<VEC>(xr + 16 * blk, rx[j]);
            if (gamma) load_block<VEC>(gamma + 16 * blk, rg[j]);
            if (beta) load_block<VEC>(beta + 16 * blk, rb[j]);
        };
#pragma unroll
        for (int j = 0; j < kRingOut; ++j)
            if (j < nblk) fill(j, j);
        for (int64_t base = 0; base < nblk; base += kRingOut) {
#pragma unroll
            for (int j = 0; j < kRingOut; ++j) {
                const int64_t blk = base + j;
                if (blk < nblk) {
                    f32x4 t[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const f32x4 d = rx[j][q] - mu;
                        t[q] = d * rs;
                        if (gamma) t[q] = t[q] * rg[j][q];
                        if (beta) t[q] = t[q] + rb[j][q];
                    }
                    if (blk + kRingOut < nblk) fill(j, blk + kRingOut);
#pragma unroll
                    for (int q = 0; q < 4; ++q) store4<VEC>(yr + 16 * blk + 4 * q, t[q]);
                }
            }
        }
    }
    for (int64_t i = tail; i < H; ++i) {
        const float d = xr[i] - mu;
        float t = d * rs;
        if (gamma) t = t * gamma[i];
        if (beta) t = t + beta[i];
        yr[i] = t;
    }
    if (mean_out) mean_out[r] = mu;
    if (rstd_out) rstd_out[r] = rs;
}

}  // namespace

int launch_unary(int op, const float* x, float* y, int64_t n, bool vec, void* stream) {
    const int64_t items = vec ? (n >> 2) + 3 : n;
    int64_t blocks = (items + 255) / 256;
    if (blocks > (int64_t(1) << 20)) blocks = int64_t(1) << 20;
    if (blocks < 1) blocks = 1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    using Fn = void (*)(const float*, float*, int64_t);
    Fn fn = op == 0 ? (vec ? repops_unary_kernel<0, true> : repops_unary_kernel<0, false>)
                    : (vec ? repops_unary_kernel<1, true> : repops_unary_kernel<1, false>);
    hipLaunchKernelGGL(fn, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, x, y, n);
    return static_cast<int>(hipGetLastError());
}

int launch_layernorm(const float* x, int64_t x_rs, const float* gamma, const float* beta, float* y,
                     int64_t y_rs, int64_t rows, int64_t H, float eps, float* mean, float* rstd,
                     bool vec, void* stream) {
    const int64_t blocks = (rows + 63) / 64;
    hipStream_t s = static_cast<hipStream_t>(stream);
    using Fn = void (*)(const float*, int64_t, const float*, const float*, float*, int64_t,
                        int64_t, int64_t, float, float*, float*);
    Fn fn = vec ? repops_layernorm_kernel<true> : repops_layernorm_kernel<false>;
    hipLaunchKernelGGL(fn, dim3(static_cast<unsigned>(blocks)), dim3(64), 0, s, x, x_rs, gamma,
                       beta, y, y_rs, rows, H, eps, mean, rstd);
    return static_cast<int>(hipGetLastError());
}

}  // namespace repops
