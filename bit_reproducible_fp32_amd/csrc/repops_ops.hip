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

// OP 0: erf, 1: GeLU.  VEC: x and y 16-byte aligned; lanes take float4s
// (grid-stride) over the first 4*(n/4) elements, then single elements.
// y may be x itself (each element is read and then written by one lane).
template <int OP, bool VEC>
__global__ __launch_bounds__(256) void repops_unary_kernel(const float* x, float* y, int64_t n) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    int64_t from = 0;
    if constexpr (VEC) {
        const int64_t nv = n >> 2;
        const f32x4* xv = reinterpret_cast<const f32x4*>(x);
        f32x4* yv = reinterpret_cast<f32x4*>(y);
        // Two float4 per lane in flight: both loads are issued before either
        // value is used.
        int64_t v = t0;
        for (; v + stride < nv; v += 2 * stride) {
            const f32x4 a = __builtin_nontemporal_load(xv + v);
            const f32x4 a2 = __builtin_nontemporal_load(xv + v + stride);
            f32x4 b, b2;
            b.x = unary<OP>(a.x);
            b.y = unary<OP>(a.y);
            b.z = unary<OP>(a.z);
            b.w = unary<OP>(a.w);
            b2.x = unary<OP>(a2.x);
            b2.y = unary<OP>(a2.y);
            b2.z = unary<OP>(a2.z);
            b2.w = unary<OP>(a2.w);
            __builtin_nontemporal_store(b, yv + v);
            __builtin_nontemporal_store(b2, yv + v + stride);
        }
        for (; v < nv; v += stride) {
            const f32x4 a = __builtin_nontemporal_load(xv + v);
            f32x4 b;
            b.x = unary<OP>(a.x);
            b.y = unary<OP>(a.y);
            b.z = unary<OP>(a.z);
            b.w = unary<OP>(a.w);
            __builtin_nontemporal_store(b, yv + v);
        }
        from = nv << 2;
    }
    for (int64_t e = from + t0; e < n; e += stride) y[e] = unary<OP>(x[e]);
}

// LayerNorm.  The two sums over a row are the fixed-order dimension, so one
// lane owns a row and walks it in ascending order; rows are the free
// dimension.  To keep the loads coalesced, a workgroup of kLnThreads lanes owns
// kLnRows consecutive rows and streams them through LDS in tiles of kLnRows x
// kLnCols: every lane helps load a tile (consecutive lanes read consecutive
// floats of a row), then lane r consumes row r of the tile.  Tiles are loaded
// kLnDepth ahead into registers and double-buffered in LDS.  The output pass
// has no order to keep, so all lanes stream it directly.
constexpr int kLnRows = 16;
constexpr int kLnCols = 64;
constexpr int kLnThreads = 64;
constexpr int kLnPitch = kLnCols + 4;            // 16-byte rows, staggered banks
constexpr int kLnPerThread = kLnRows * kLnCols / kLnThreads;
constexpr int kLnDepth = 4;                      // tiles in flight per workgroup

struct LnTile {
    alignas(16) float x[2][kLnRows][kLnPitch];
    float mu[kLnRows];
    float rs[kLnRows];
};

// Loads of one tile (columns c0 .. c0+kLnCols-1 of the block's rows) into
// registers; out-of-range elements are left as 0 and never consumed.  VEC
// (x 16-byte aligned, x_rs and H multiples of 4): lane t loads float4 number
// t + 64k of the tile, so 16 consecutive lanes cover one row's 256 bytes;
// otherwise element t + 64k.
struct LnLoad {
    float v[kLnPerThread];
};

template <bool VEC>
__device__ __forceinline__ void ln_load(LnLoad& L, const float* x, int64_t x_rs, int64_t row0,
                                        int64_t rows, int64_t H, int64_t c0, int tid) {
    if constexpr (VEC) {
#pragma unroll
        for (int k = 0; k < kLnPerThread / 4; ++k) {
            const int q = tid + k * kLnThreads;
            const int r = q / (kLnCols / 4), c = 4 * (q % (kLnCols / 4));
            f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
            if (row0 + r < rows && c0 + c < H)
                v = *reinterpret_cast<const f32x4*>(x + (row0 + r) * x_rs + c0 + c);
            L.v[4 * k] = v.x;
            L.v[4 * k + 1] = v.y;
            L.v[4 * k + 2] = v.z;
            L.v[4 * k + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int k = 0; k < kLnPerThread; ++k) {
            const int e = tid + k * kLnThreads;
            const int r = e / kLnCols, c = e % kLnCols;
            L.v[k] = (row0 + r < rows && c0 + c < H) ? x[(row0 + r) * x_rs + c0 + c] : 0.0f;
        }
    }
}

// Moves a tile from registers into LDS buffer buf (the inverse of ln_load's
// mapping).  PASS 0 stores x; PASS 1 stores (x - mu_r)^2, each element as
// d = x - mu_r and then d * d (every lane computes the same two rounded
// operations the definition names, so which lane does it does not matter);
// the owner lanes then only add.
template <int PASS, bool VEC>
__device__ __forceinline__ void ln_store(const LnLoad& L, LnTile& T, int buf, int tid) {
#pragma unroll
    for (int k = 0; k < kLnPerThread; ++k) {
        int r, c;
        if constexpr (VEC) {
            const int q = tid + (k / 4) * kLnThreads;
            r = q / (kLnCols / 4);
            c = 4 * (q % (kLnCols / 4)) + k % 4;
        } else {
            const int e = tid + k * kLnThreads;
            r = e / kLnCols;
            c = e % kLnCols;
        }
        float v = L.v[k];
        if constexpr (PASS == 1) {
            const float d = v - T.mu[r];
            v = d * d;
        }
        T.x[buf][r][c] = v;
    }
}

// PASS 0: s = s + x; PASS 1: d = x - mu, s = s + d*d; PASS 2: y.
// One pass over the block's rows.  Tiles are loaded kLnDepth ahead into a
// ring of registers; tile t+1 moves from the ring into the LDS buffer the
// consumers are not reading while they consume tile t.
// PASS 0 returns S = sum of x_i, PASS 1 S2 = sum of (x_i - mu)^2, both from
// +0 in ascending i (in the owner lane of each row; T.mu holds the means for
// PASS 1).
template <int PASS, bool VEC>
__device__ __forceinline__ float ln_pass(LnTile& T, const float* x, int64_t x_rs, int64_t row0,
                                         int64_t rows, int64_t H, int tid) {
    const int64_t ntiles = (H + kLnCols - 1) / kLnCols;
    const bool owner = tid < kLnRows && row0 + tid < rows;
    float s = 0.0f;
    LnLoad ring[kLnDepth];
#pragma unroll
    for (int j = 0; j < kLnDepth; ++j)
        if (j < ntiles) ln_load<VEC>(ring[j], x, x_rs, row0, rows, H, j * kLnCols, tid);
    ln_store<PASS, VEC>(ring[0], T, 0, tid);
    __syncthreads();
    for (int64_t base = 0; base < ntiles; base += kLnDepth) {
#pragma unroll
        for (int j = 0; j < kLnDepth; ++j) {
            const int64_t t = base + j;
            if (t >= ntiles) break;
            const int buf = static_cast<int>(t & 1);
            const int64_t c0 = t * kLnCols;
            // ring[j] held tile t, already in LDS: refill it with tile t + depth
            if (t + kLnDepth < ntiles)
                ln_load<VEC>(ring[j], x, x_rs, row0, rows, H, c0 + kLnDepth * kLnCols, tid);
            const int64_t left = H - c0;
            const int cols = left < kLnCols ? static_cast<int>(left) : kLnCols;
            if (owner) {
                if (cols == kLnCols) {
                    // A full tile: all 64 values (and gamma, beta) into
                    // registers first, then the chain in column order.
                    f32x4 v[kLnCols / 4];
#pragma unroll
                    for (int q = 0; q < kLnCols / 4; ++q)
                        v[q] = *reinterpret_cast<const f32x4*>(&T.x[buf][tid][4 * q]);
#pragma unroll
                    for (int q = 0; q < kLnCols / 4; ++q) {
                        s = s + v[q].x;
                        s = s + v[q].y;
                        s = s + v[q].z;
                        s = s + v[q].w;
                    }
                } else {
                    for (int c = 0; c < cols; ++c) s = s + T.x[buf][tid][c];
                }
            }
            if (t + 1 < ntiles) ln_store<PASS, VEC>(ring[(j + 1) % kLnDepth], T, buf ^ 1, tid);
            __syncthreads();
        }
    }
    return s;
}

// y = ((x - mu) * rstd) * gamma + beta for W consecutive elements (W = 4:
// 16-byte accesses).
template <int W>
struct LnVec {
    float v[W];
};

template <int W>
__device__ __forceinline__ LnVec<W> ln_get(const float* p) {
    LnVec<W> o;
    if constexpr (W == 4) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(p);
        o.v[0] = a.x;
        o.v[1] = a.y;
        o.v[2] = a.z;
        o.v[3] = a.w;
    } else {
        o.v[0] = p[0];
    }
    return o;
}

template <int W>
__device__ __forceinline__ void ln_put(float* p, const LnVec<W>& o) {
    if constexpr (W == 4) {
        f32x4 a;
        a.x = o.v[0];
        a.y = o.v[1];
        a.z = o.v[2];
        a.w = o.v[3];
        *reinterpret_cast<f32x4*>(p) = a;
    } else {
        p[0] = o.v[0];
    }
}

// Pass 3 has no order to keep: every lane computes outputs, consecutive lanes
// on consecutive W-element groups of a row, four rows and four groups per
// lane at a time so that sixteen loads are in flight.  y may be x itself with
// y_rs == x_rs: each element is read and then written by one lane, after both
// summing passes, and other workgroups own other rows.
template <int W>
__device__ __forceinline__ void ln_output(const LnTile& T, const float* x, int64_t x_rs,
                                          const float* gamma, const float* beta, float* y,
                                          int64_t y_rs, int64_t row0, int nr, int64_t H,
                                          int tid) {
    constexpr int RU = 4, CU = 4;
    const int64_t groups = H / W;
    for (int r0 = 0; r0 < nr; r0 += RU) {
        for (int64_t gb = 0; gb < groups; gb += CU * kLnThreads) {
            LnVec<W> v[RU][CU], g[CU], b[CU];
#pragma unroll
            for (int u = 0; u < CU; ++u) {
                const int64_t gi = gb + tid + u * kLnThreads;
                if (gi < groups) {
                    if (gamma) g[u] = ln_get<W>(gamma + gi * W);
                    if (beta) b[u] = ln_get<W>(beta + gi * W);
#pragma unroll
                    for (int rr = 0; rr < RU; ++rr)
                        if (r0 + rr < nr) v[rr][u] = ln_get<W>(x + (row0 + r0 + rr) * x_rs + gi * W);
                }
            }
#pragma unroll
            for (int rr = 0; rr < RU; ++rr) {
                if (r0 + rr >= nr) break;
                const float m = T.mu[r0 + rr], q = T.rs[r0 + rr];
#pragma unroll
                for (int u = 0; u < CU; ++u) {
                    const int64_t gi = gb + tid + u * kLnThreads;
                    if (gi < groups) {
                        LnVec<W> o;
#pragma unroll
                        for (int w = 0; w < W; ++w) {
                            const float d = v[rr][u].v[w] - m;
                            float t = d * q;
                            if (gamma) t = t * g[u].v[w];
                            if (beta) t = t + b[u].v[w];
                            o.v[w] = t;
                        }
                        ln_put<W>(y + (row0 + r0 + rr) * y_rs + gi * W, o);
                    }
                }
            }
        }
    }
}

// VEC: x, y, gamma, beta 16-byte aligned; x_rs, y_rs and H multiples of 4.
template <bool VEC>
__global__ __launch_bounds__(kLnThreads) void repops_layernorm_kernel(
    const float* x, int64_t x_rs, const float* __restrict__ gamma,
    const float* __restrict__ beta, float* y, int64_t y_rs, int64_t rows, int64_t H, float eps,
    float* __restrict__ mean_out, float* __restrict__ rstd_out) {
    __shared__ LnTile T;
    const int tid = static_cast<int>(threadIdx.x);
    const int64_t row0 = static_cast<int64_t>(blockIdx.x) * kLnRows;
    const float fh = static_cast<float>(H);

    // pass 1: S = ((+0 + x_0) + x_1) + ...;  mu = S / H (owner lanes)
    const float s = ln_pass<0, VEC>(T, x, x_rs, row0, rows, H, tid);
    const float mu = s / fh;
    if (tid < kLnRows) T.mu[tid] = mu;
    __syncthreads();

    // pass 2: S2 = sum of (x_i - mu)^2 in the same order; rstd = 1/sqrt(S2/H + eps)
    const float s2 = ln_pass<1, VEC>(T, x, x_rs, row0, rows, H, tid);
    const float var = s2 / fh;
    const float ve = var + eps;
    const float sd = __builtin_sqrtf(ve);
    const float rs = 1.0f / sd;
    if (tid < kLnRows) {
        T.rs[tid] = rs;
        if (row0 + tid < rows) {
            if (mean_out) mean_out[row0 + tid] = mu;
            if (rstd_out) rstd_out[row0 + tid] = rs;
        }
    }
    __syncthreads();

    // pass 3: y_i = ((x_i - mu) * rstd) * gamma_i + beta_i, all lanes
    const int nr = rows - row0 < kLnRows ? static_cast<int>(rows - row0) : kLnRows;
    ln_output<VEC ? 4 : 1>(T, x, x_rs, gamma, beta, y, y_rs, row0, nr, H, tid);
}

// The resident form, for rows short enough that kLnResRows of them fit in
// LDS: the block is read from memory once; lane r sums row r from LDS; then
// every lane replaces x_i by d_i = x_i - mu (the operation the definition
// names, rounded once), lane r sums d_i * d_i, and every lane writes
// y_i = (d_i * rstd) * gamma_i + beta_i.  A small block lets many workgroups
// share a CU, so one block's loads overlap another's sums.  ld_h: the row
// pitch in LDS (H rounded up to 4, plus 4).
constexpr int kLnResRows = 4;

template <bool VEC>
__global__ __launch_bounds__(kLnThreads) void repops_layernorm_resident_kernel(
    const float* x, int64_t x_rs, const float* __restrict__ gamma,
    const float* __restrict__ beta, float* y, int64_t y_rs, int64_t rows, int64_t H, int ld_h,
    float eps, float* __restrict__ mean_out, float* __restrict__ rstd_out) {
    extern __shared__ float4 ln_dyn[];
    float* blk = reinterpret_cast<float*>(ln_dyn);
    __shared__ float mu_s[kLnResRows], rs_s[kLnResRows];
    const int tid = static_cast<int>(threadIdx.x);
    const int64_t row0 = static_cast<int64_t>(blockIdx.x) * kLnResRows;
    const int nr = rows - row0 < kLnResRows ? static_cast<int>(rows - row0) : kLnResRows;
    constexpr int W = VEC ? 4 : 1;
    const int groups = static_cast<int>(H / W);  // W-element groups per row
    const int total = nr * groups;
    const float fh = static_cast<float>(H);

    // the block into LDS, sixteen loads in flight per lane
    for (int base = 0; base < total; base += 16 * kLnThreads) {
        LnVec<W> v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int e = base + u * kLnThreads + tid;
            if (e < total) {
                const int r = e / groups, gi = e - r * groups;
                v[u] = ln_get<W>(x + (row0 + r) * x_rs + static_cast<int64_t>(gi) * W);
            }
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int e = base + u * kLnThreads + tid;
            if (e < total) {
                const int r = e / groups, gi = e - r * groups;
                ln_put<W>(blk + r * ld_h + gi * W, v[u]);
            }
        }
    }
    __syncthreads();

    // S = ((+0 + x_0) + x_1) + ...;  mu = S / H
    const int64_t H64 = H & ~int64_t(63);
    if (tid < nr) {
        const float* row = blk + tid * ld_h;
        float s = 0.0f;
        for (int64_t c = 0; c < H64; c += 64) {
            f32x4 v[16];
#pragma unroll
            for (int q = 0; q < 16; ++q) v[q] = *reinterpret_cast<const f32x4*>(row + c + 4 * q);
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                s = s + v[q].x;
                s = s + v[q].y;
                s = s + v[q].z;
                s = s + v[q].w;
            }
        }
        for (int64_t c = H64; c < H; ++c) s = s + row[c];
        mu_s[tid] = s / fh;
    }
    __syncthreads();

    // d_i = x_i - mu, in place, every lane
    for (int e = tid; e < total; e += kLnThreads) {
        const int r = e / groups, gi = e - r * groups;
        float* p = blk + r * ld_h + gi * W;
        LnVec<W> v = ln_get<W>(p);
        const float m = mu_s[r];
#pragma unroll
        for (int w = 0; w < W; ++w) v.v[w] = v.v[w] - m;
        ln_put<W>(p, v);
    }
    __syncthreads();

    // S2 = sum of d_i * d_i in the same order; rstd = 1 / sqrt(S2 / H + eps)
    if (tid < nr) {
        const float* row = blk + tid * ld_h;
        float s2 = 0.0f;
        for (int64_t c = 0; c < H64; c += 64) {
            f32x4 v[16];
#pragma unroll
            for (int q = 0; q < 16; ++q) v[q] = *reinterpret_cast<const f32x4*>(row + c + 4 * q);
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const f32x4 sq = v[q] * v[q];
                s2 = s2 + sq.x;
                s2 = s2 + sq.y;
                s2 = s2 + sq.z;
                s2 = s2 + sq.w;
            }
        }
        for (int64_t c = H64; c < H; ++c) {
            const float sq = row[c] * row[c];
            s2 = s2 + sq;
        }
        const float var = s2 / fh;
        const float ve = var + eps;
        const float sd = __builtin_sqrtf(ve);
        const float rs = 1.0f / sd;
        rs_s[tid] = rs;
        if (mean_out) mean_out[row0 + tid] = mu_s[tid];
        if (rstd_out) rstd_out[row0 + tid] = rs;
    }
    __syncthreads();

    // y_i = (d_i * rstd) * gamma_i + beta_i, every lane
    for (int e = tid; e < total; e += kLnThreads) {
        const int r = e / groups, gi = e - r * groups;
        const LnVec<W> v = ln_get<W>(blk + r * ld_h + gi * W);
        LnVec<W> g, b, o;
        if (gamma) g = ln_get<W>(gamma + static_cast<int64_t>(gi) * W);
        if (beta) b = ln_get<W>(beta + static_cast<int64_t>(gi) * W);
        const float q = rs_s[r];
#pragma unroll
        for (int w = 0; w < W; ++w) {
            float t = v.v[w] * q;
            if (gamma) t = t * g.v[w];
            if (beta) t = t + b.v[w];
            o.v[w] = t;
        }
        ln_put<W>(y + (row0 + r) * y_rs + static_cast<int64_t>(gi) * W, o);
    }
}

// Lane 4q + g of the result holds lane 4q + (g + 3) % 4 of s: one step of a
// ring around each quad (DPP quad permutation [3, 0, 1, 2]).
__device__ __forceinline__ float quad_ring_step(float s) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s), 0x93, 0xF, 0xF, false));
}

// Every lane of a quad receives lane 3's s (quad permutation [3, 3, 3, 3]).
__device__ __forceinline__ float quad_from_last(float s) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s), 0xFF, 0xF, 0xF, false));
}

// The register-resident form, for rows of at most 4 * S elements.  A row
// belongs to one quad of lanes (16 rows per wave) and is dealt out in pieces
// of 8 elements: piece j of lane g is elements [32 j + 8 g, 32 j + 8 g + 8),
// so that the quad reads and writes 128 contiguous bytes per piece.  Every
// row is on chip at once and x is read once.
//
// A fixed-order sum walks the pieces in row order, which visits the lanes of
// the quad in turn: before each piece the running sums take one step around
// the quad, so lane g receives the sum that lane g - 1 has just carried
// through its piece, and adds its own 8 elements in ascending order.  All
// four lanes run every step (three of them on values that the next steps
// overwrite), so the adds that reach the result are exactly x_0, x_1, ...
// in ascending order from +0.  The padding past H holds +0, which leaves a
// running sum unchanged: it starts at +0 and so is never -0, and s + (+0) == s
// for every other s (a NaN stays a NaN).
//
// FULL (16 live rows of exactly 4 * S elements) drops every bounds test, so
// that the loads are unconditional and issued in piece order, and the sum
// can start on the first piece while the later ones are still in flight.
template <int S, bool VEC, bool FULL>
__device__ __forceinline__ void ln_regs_group(const float* xs, float* ys, int hl, bool live,
                                              int64_t row, int seg, float fh, float eps,
                                              const float* gs, const float* bs,
                                              float* __restrict__ mean_out,
                                              float* __restrict__ rstd_out) {
    constexpr int kPieces = S / 8;
    float v[S];
    if constexpr (VEC) {
#pragma unroll
        for (int q = 0; q < S / 4; ++q) {
            const int o = 32 * (q >> 1) + 4 * (q & 1);
            f32x4 a = {0.0f, 0.0f, 0.0f, 0.0f};
            if (FULL || o < hl) a = *reinterpret_cast<const f32x4*>(xs + o);
            v[4 * q] = a.x;
            v[4 * q + 1] = a.y;
            v[4 * q + 2] = a.z;
            v[4 * q + 3] = a.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < S; ++i) {
            const int o = 32 * (i >> 3) + (i & 7);
            v[i] = (FULL || o < hl) ? xs[o] : 0.0f;
        }
    }

    // S = ((+0 + x_0) + x_1) + ...
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < kPieces; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            s = quad_ring_step(s);
#pragma unroll
            for (int k = 0; k < 8; ++k) s = s + v[8 * j + k];
        }
    }
    s = quad_from_last(s);
    const float mu = s / fh;

    // d_i = x_i - mu in place (+0 in the padding); S2 = sum of d_i * d_i
#pragma unroll
    for (int i = 0; i < S; ++i) {
        const int o = 32 * (i >> 3) + (i & 7);
        v[i] = (FULL || o < hl) ? v[i] - mu : 0.0f;
    }
    float s2 = 0.0f;
#pragma unroll
    for (int j = 0; j < kPieces; ++j) {
        float sq[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) sq[k] = v[8 * j + k] * v[8 * j + k];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            s2 = quad_ring_step(s2);
#pragma unroll
            for (int k = 0; k < 8; ++k) s2 = s2 + sq[k];
        }
    }
    s2 = quad_from_last(s2);
    const float var = s2 / fh;
    const float ve = var + eps;
    const float sd = __builtin_sqrtf(ve);
    const float rs = 1.0f / sd;
    if (live && seg == 0) {
        if (mean_out) mean_out[row] = mu;
        if (rstd_out) rstd_out[row] = rs;
    }

    // y_i = (d_i * rstd) * gamma_i + beta_i
    if constexpr (VEC) {
#pragma unroll
        for (int q = 0; q < S / 4; ++q) {
            const int o = 32 * (q >> 1) + 4 * (q & 1);
            if (FULL || o < hl) {
                f32x4 t;
                t.x = v[4 * q] * rs;
                t.y = v[4 * q + 1] * rs;
                t.z = v[4 * q + 2] * rs;
                t.w = v[4 * q + 3] * rs;
                t = t * *reinterpret_cast<const f32x4*>(gs + o);
                t = t + *reinterpret_cast<const f32x4*>(bs + o);
                *reinterpret_cast<f32x4*>(ys + o) = t;
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < S; ++i) {
            const int o = 32 * (i >> 3) + (i & 7);
            if (FULL || o < hl) {
                float t = v[i] * rs;
                t = t * gs[o];
                t = t + bs[o];
                ys[o] = t;
            }
        }
    }
}

template <int S, bool VEC>
__global__ __launch_bounds__(64) void repops_layernorm_regs_kernel(
    const float* x, int64_t x_rs, const float* __restrict__ gamma,
    const float* __restrict__ beta, float* y, int64_t y_rs, int64_t rows, int64_t H, float eps,
    float* __restrict__ mean_out, float* __restrict__ rstd_out) {
    // gamma and beta, staged once per workgroup.  A missing gamma is staged
    // as 1 and a missing beta as -0: t * 1 == t and t + (-0) == t for every
    // binary32 t (signed zeros, infinities and NaN included), so the output
    // step needs no branch and matches skipping the operation.
    __shared__ __align__(16) float ln_g[4 * S];
    __shared__ __align__(16) float ln_b[4 * S];
    const int lane = static_cast<int>(threadIdx.x);
    const int seg = lane & 3;
    const int64_t groups = (rows + 15) / 16;
    const float fh = static_cast<float>(H);
    const int hi = static_cast<int>(H);
    if constexpr (VEC) {
        for (int c = 4 * lane; c < 4 * S; c += 256) {
            f32x4 gv = {1.0f, 1.0f, 1.0f, 1.0f}, bv = {-0.0f, -0.0f, -0.0f, -0.0f};
            if (gamma && c < hi) gv = *reinterpret_cast<const f32x4*>(gamma + c);
            if (beta && c < hi) bv = *reinterpret_cast<const f32x4*>(beta + c);
            *reinterpret_cast<f32x4*>(ln_g + c) = gv;
            *reinterpret_cast<f32x4*>(ln_b + c) = bv;
        }
    } else {
        for (int c = lane; c < 4 * S; c += 64) {
            ln_g[c] = gamma && c < hi ? gamma[c] : 1.0f;
            ln_b[c] = beta && c < hi ? beta[c] : -0.0f;
        }
    }
    __syncthreads();
    for (int64_t rg = blockIdx.x; rg < groups; rg += gridDim.x) {
        const int64_t row = rg * 16 + (lane >> 2);
        const bool live = row < rows;
        // element 32 j + 8 seg + k of the row is at offset o = 32 j + k from
        // xs, and exists when o < hl
        const int hl = live ? hi - 8 * seg : 0;
        const float* xs = x + (live ? row : 0) * x_rs + 8 * seg;
        float* ys = y + (live ? row : 0) * y_rs + 8 * seg;
        const bool full = (rg + 1) * 16 <= rows && hi == 4 * S;
        if (full)
            ln_regs_group<S, VEC, true>(xs, ys, hl, live, row, seg, fh, eps, ln_g + 8 * seg,
                                        ln_b + 8 * seg, mean_out, rstd_out);
        else
            ln_regs_group<S, VEC, false>(xs, ys, hl, live, row, seg, fh, eps, ln_g + 8 * seg,
                                         ln_b + 8 * seg, mean_out, rstd_out);
    }
}

}  // namespace

int launch_unary(int op, const float* x, float* y, int64_t n, bool vec, void* stream) {
    const int64_t items = vec ? (n >> 2) + 3 : n;
    int64_t blocks = (items + 255) / 256;
    // At most 16384 workgroups of 256 lanes (64 waves per SIMD): measured
    // best for long inputs, with two float4 per lane per step.
    if (blocks > 16384) blocks = 16384;
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
    hipStream_t s = static_cast<hipStream_t>(stream);
    // Register-resident form for rows of at most 768 elements (the row and
    // its squared deviations are both held: 2 * 192 registers per lane).
    if (H <= 768) {
        using Gn = void (*)(const float*, int64_t, const float*, const float*, float*, int64_t,
                            int64_t, int64_t, float, float*, float*);
        Gn gn;
        if (H <= 256)
            gn = vec ? repops_layernorm_regs_kernel<64, true> : repops_layernorm_regs_kernel<64, false>;
        else if (H <= 512)
            gn = vec ? repops_layernorm_regs_kernel<128, true> : repops_layernorm_regs_kernel<128, false>;
        else
            gn = vec ? repops_layernorm_regs_kernel<192, true> : repops_layernorm_regs_kernel<192, false>;
        const int64_t groups = (rows + 15) / 16;
        const int64_t gblocks = groups < (int64_t(1) << 20) ? groups : (int64_t(1) << 20);
        hipLaunchKernelGGL(gn, dim3(static_cast<unsigned>(gblocks)), dim3(64), 0, s, x, x_rs,
                           gamma, beta, y, y_rs, rows, H, eps, mean, rstd);
        return static_cast<int>(hipGetLastError());
    }
    // Resident form when a block of kLnResRows rows fits in 32 KB of LDS.
    const int64_t ld_h = ((H + 3) & ~int64_t(3)) + 4;
    const int64_t lds = kLnResRows * ld_h * 4;
    if (lds <= 32768) {
        using Rn = void (*)(const float*, int64_t, const float*, const float*, float*, int64_t,
                            int64_t, int64_t, int, float, float*, float*);
        Rn rn = vec ? repops_layernorm_resident_kernel<true>
                    : repops_layernorm_resident_kernel<false>;
        const int64_t rblocks = (rows + kLnResRows - 1) / kLnResRows;
        hipLaunchKernelGGL(rn, dim3(static_cast<unsigned>(rblocks)), dim3(kLnThreads),
                           static_cast<unsigned>(lds), s, x, x_rs, gamma, beta, y, y_rs, rows, H,
                           static_cast<int>(ld_h), eps, mean, rstd);
        return static_cast<int>(hipGetLastError());
    }
    const int64_t blocks = (rows + kLnRows - 1) / kLnRows;
    using Fn = void (*)(const float*, int64_t, const float*, const float*, float*, int64_t,
                        int64_t, int64_t, float, float*, float*);
    Fn fn = vec ? repops_layernorm_kernel<true> : repops_layernorm_kernel<false>;
    hipLaunchKernelGGL(fn, dim3(static_cast<unsigned>(blocks)), dim3(kLnThreads), 0, s, x, x_rs,
                       gamma, beta, y, y_rs, rows, H, eps, mean, rstd);
    return static_cast<int>(hipGetLastError());
}

}  // namespace repops
