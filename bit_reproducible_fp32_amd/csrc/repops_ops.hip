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

// One step of a ring around each group of L lanes (L = 4 or 16): lane
// g of a group receives lane (g - 1) mod L's s.  DPP quad permutation
// [3, 0, 1, 2] for L = 4, row rotation by one for L = 16.
template <int L>
__device__ __forceinline__ float ring_step(float s) {
    static_assert(L == 4 || L == 16, "ring of 4 or 16 lanes");
    constexpr int kCtrl = L == 4 ? 0x93 : 0x121;
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s), kCtrl, 0xF, 0xF, false));
}

// Every lane of a group of L receives the group's last lane's s.
template <int L>
__device__ __forceinline__ float from_last(float s) {
    if constexpr (L == 4)  // quad permutation [3, 3, 3, 3]
        return __builtin_bit_cast(
            float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s), 0xFF, 0xF, 0xF, false));
    else
        return __shfl(s, L - 1, L);
}

// The register-resident form, for rows of at most L * S elements.  A row
// belongs to a group of L consecutive lanes (64 / L rows per wave) and is
// dealt out in pieces of P elements: piece j of lane g is elements
// [j L P + g P, j L P + g P + P), so that the group reads and writes L P
// contiguous floats per piece.  A wave keeps its rows in registers from load
// to output, so x is read once.
//
// A fixed-order sum walks the pieces in row order, which visits the lanes of
// the group in turn: before each piece the running sums take one step around
// the ring, so lane g receives the sum that lane g - 1 has just carried
// through its piece, and adds its own P elements in ascending order.  All
// lanes run every step (all but one on values that later steps overwrite),
// so the adds that reach the result are exactly x_0, x_1, ... in ascending
// order from +0.  The padding past H holds +0, which leaves a running sum
// unchanged: it starts at +0 and so is never -0, and s + (+0) == s for every
// other s (a NaN stays a NaN).
//
// FULL (every row of the wave live and exactly L * S long) drops every
// bounds test, so that the loads are unconditional and issued in piece order,
// and the sum can start on the first piece while later ones are in flight.
template <int L, int S, bool VEC, bool FULL, class AfterLoads>
__device__ __forceinline__ void ln_regs_group(const float* xs, float* ys, int hl, bool live,
                                              int64_t row, int seg, float fh, float eps,
                                              const float* gs, const float* bs,
                                              float* __restrict__ mean_out,
                                              float* __restrict__ rstd_out,
                                              AfterLoads after_loads) {
    constexpr int P = L == 4 ? 8 : 4;  // elements per piece
    constexpr int kPieces = S / P;
    constexpr int kStride = L * P;     // row offset from one piece of a lane to its next
    float v[S];
    if constexpr (VEC) {
#pragma unroll
        for (int q = 0; q < S / 4; ++q) {
            const int o = kStride * (q / (P / 4)) + 4 * (q % (P / 4));
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
            const int o = kStride * (i / P) + i % P;
            v[i] = (FULL || o < hl) ? xs[o] : 0.0f;
        }
    }
    after_loads();

    // S = ((+0 + x_0) + x_1) + ...
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < kPieces; ++j) {
#pragma unroll
        for (int g = 0; g < L; ++g) {
            s = ring_step<L>(s);
#pragma unroll
            for (int k = 0; k < P; ++k) s = s + v[P * j + k];
        }
    }
    s = from_last<L>(s);
    const float mu = s / fh;

    // d_i = x_i - mu in place (+0 in the padding); S2 = sum of d_i * d_i
#pragma unroll
    for (int i = 0; i < S; ++i) {
        const int o = kStride * (i / P) + i % P;
        v[i] = (FULL || o < hl) ? v[i] - mu : 0.0f;
    }
    float s2 = 0.0f;
#pragma unroll
    for (int j = 0; j < kPieces; ++j) {
        float sq[P];
#pragma unroll
        for (int k = 0; k < P; ++k) sq[k] = v[P * j + k] * v[P * j + k];
#pragma unroll
        for (int g = 0; g < L; ++g) {
            s2 = ring_step<L>(s2);
#pragma unroll
            for (int k = 0; k < P; ++k) s2 = s2 + sq[k];
        }
    }
    s2 = from_last<L>(s2);
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
            const int o = kStride * (q / (P / 4)) + 4 * (q % (P / 4));
            if (FULL || o < hl) {
                f32x4 t;
                t.x = v[4 * q] * rs;
                t.y = v[4 * q + 1] * rs;
                t.z = v[4 * q + 2] * rs;
                t.w = v[4 * q + 3] * rs;
                t = t * *reinterpret_cast<const f32x4*>(gs + o);
                t = t + *reinterpret_cast<const f32x4*>(bs + o);
                // 16 lanes write whole 256-byte runs of a row, which
                // nontemporal stores pass on without keeping them; a quad's
                // stores write half lines, which only plain stores let the
                // cache merge
                if constexpr (L == 16)
                    __builtin_nontemporal_store(t, reinterpret_cast<f32x4*>(ys + o));
                else
                    *reinterpret_cast<f32x4*>(ys + o) = t;
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < S; ++i) {
            const int o = kStride * (i / P) + i % P;
            if (FULL || o < hl) {
                float t = v[i] * rs;
                t = t * gs[o];
                t = t + bs[o];
                ys[o] = t;
            }
        }
    }
}

template <int L, int S, bool VEC>
__global__ __launch_bounds__(64) void repops_layernorm_regs_kernel(
    const float* x, int64_t x_rs, const float* __restrict__ gamma,
    const float* __restrict__ beta, float* y, int64_t y_rs, int64_t rows, int64_t H, float eps,
    float* __restrict__ mean_out, float* __restrict__ rstd_out) {
    constexpr int P = L == 4 ? 8 : 4;
    constexpr int R = 64 / L;  // rows per wave
    // gamma and beta, staged once per workgroup.  A missing gamma is staged
    // as 1 and a missing beta as -0: t * 1 == t and t + (-0) == t for every
    // binary32 t (signed zeros, infinities and NaN included), so the output
    // step needs no branch and matches skipping the operation.
    __shared__ __align__(16) float ln_g[L * S];
    __shared__ __align__(16) float ln_b[L * S];
    const int lane = static_cast<int>(threadIdx.x);
    const int seg = lane % L;
    const int64_t groups = (rows + R - 1) / R;
    const float fh = static_cast<float>(H);
    const int hi = static_cast<int>(H);
    // The staging loads are issued at once.  In the vector quad forms they
    // are written to LDS only after the first row group's loads are in
    // flight, so that their latency overlaps those loads instead of
    // preceding them; the other forms write them at once (holding them
    // across their loads would spill or cost occupancy).
    constexpr bool kEarly = VEC && L == 4;
    constexpr int kW = VEC ? 4 : 1;                        // floats per staging load
    constexpr int kN = (L * S + 64 * kW - 1) / (64 * kW);  // staging loads per lane
    f32x4 gv[kN], bv[kN];
#pragma unroll
    for (int q = 0; q < kN; ++q) {
        const int c = kW * lane + 64 * kW * q;
        gv[q] = f32x4{1.0f, 1.0f, 1.0f, 1.0f};
        bv[q] = f32x4{-0.0f, -0.0f, -0.0f, -0.0f};
        if constexpr (VEC) {
            if (c < L * S && gamma && c < hi) gv[q] = *reinterpret_cast<const f32x4*>(gamma + c);
            if (c < L * S && beta && c < hi) bv[q] = *reinterpret_cast<const f32x4*>(beta + c);
        } else {
            if (c < L * S && gamma && c < hi) gv[q].x = gamma[c];
            if (c < L * S && beta && c < hi) bv[q].x = beta[c];
        }
    }
    bool staged = false;
    auto stage = [&]() {
        if (staged) return;
#pragma unroll
        for (int q = 0; q < kN; ++q) {
            const int c = kW * lane + 64 * kW * q;
            if (c < L * S) {
                if constexpr (VEC) {
                    *reinterpret_cast<f32x4*>(ln_g + c) = gv[q];
                    *reinterpret_cast<f32x4*>(ln_b + c) = bv[q];
                } else {
                    ln_g[c] = gv[q].x;
                    ln_b[c] = bv[q].x;
                }
            }
        }
        __syncthreads();
        staged = true;
    };
    if constexpr (!kEarly) stage();
    for (int64_t rg = blockIdx.x; rg < groups; rg += gridDim.x) {
        const int64_t row = rg * R + lane / L;
        const bool live = row < rows;
        // element j L P + seg P + k of the row is at offset o = j L P + k from
        // xs, and exists when o < hl
        const int hl = live ? hi - P * seg : 0;
        const float* xs = x + (live ? row : 0) * x_rs + P * seg;
        float* ys = y + (live ? row : 0) * y_rs + P * seg;
        const bool full = (rg + 1) * R <= rows && hi == L * S;
        if (full)
            ln_regs_group<L, S, VEC, true>(xs, ys, hl, live, row, seg, fh, eps, ln_g + P * seg,
                                           ln_b + P * seg, mean_out, rstd_out, stage);
        else
            ln_regs_group<L, S, VEC, false>(xs, ys, hl, live, row, seg, fh, eps, ln_g + P * seg,
                                            ln_b + P * seg, mean_out, rstd_out, stage);
    }
}

// The ring-streaming form, for rows longer than 2048.  As in the
// 16-lane register form, a row belongs to 16 consecutive lanes (4 rows per
// one-wave workgroup) and round j deals elements [64 j, 64 j + 64) out in
// pieces of 4 (lane g: 64 j + 4 g ...); the fixed-order sums walk the rounds
// with the same ring step before every piece.  The row is read in chunks of
// C rounds.  Its first NL chunks are kept in LDS and the next NR in
// registers from the first pass on; the rest streams through two register
// buffers three times (sum, sum of squared deviations, output), the next
// chunk loaded while the current one is summed.  Every load is issued
// unconditionally: a position past H reads the row's last piece and is then
// replaced by +0, which leaves a running sum unchanged.  The output pass
// takes the streamed chunks last to first (the ones the second pass read
// last come first) and then the kept ones; y is written with nontemporal
// stores, which keep the caches for x's second and third reads.

// This lane's pieces of rounds j0 .. j0 + R - 1 of the row at xr (hi = H):
// element k of round j0 + q is a[4 q + k], +0 past H.  IN: the rounds lie
// inside the row, so no position needs the test.
template <bool VEC, int R, bool IN = false>
__device__ __forceinline__ void rs_load(const float* xr, int hi, int j0, int seg,
                                        float (&a)[4 * R]) {
#pragma unroll
    for (int q = 0; q < R; ++q) {
        const int o = 64 * (j0 + q) + 4 * seg;
        if constexpr (IN && VEC) {
            const f32x4 t = *reinterpret_cast<const f32x4*>(xr + o);
            a[4 * q] = t.x;
            a[4 * q + 1] = t.y;
            a[4 * q + 2] = t.z;
            a[4 * q + 3] = t.w;
        } else if constexpr (IN) {
#pragma unroll
            for (int k = 0; k < 4; ++k) a[4 * q + k] = xr[o + k];
        } else if constexpr (VEC) {
            const bool in = o < hi;
            const f32x4 t = *reinterpret_cast<const f32x4*>(xr + (in ? o : hi - 4));
            a[4 * q] = in ? t.x : 0.0f;
            a[4 * q + 1] = in ? t.y : 0.0f;
            a[4 * q + 2] = in ? t.z : 0.0f;
            a[4 * q + 3] = in ? t.w : 0.0f;
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const bool in = o + k < hi;
                const float t = xr[in ? o + k : hi - 1];
                a[4 * q + k] = in ? t : 0.0f;
            }
        }
    }
}

// s runs on through R rounds: before each piece a ring step, then the
// piece's 4 adds.
template <int R>
__device__ __forceinline__ void rs_sum(float& s, const float (&a)[4 * R]) {
#pragma unroll
    for (int q = 0; q < R; ++q) {
#pragma unroll
        for (int g = 0; g < 16; ++g) {
            s = ring_step<16>(s);
#pragma unroll
            for (int k = 0; k < 4; ++k) s = s + a[4 * q + k];
        }
    }
}

// The same over the squared deviations d = x - mu of R rounds (+0 past H).
template <int R, bool IN = false>
__device__ __forceinline__ void rs_sum_sq(float& s, const float (&a)[4 * R], float mu, int hi,
                                          int j0, int seg) {
#pragma unroll
    for (int q = 0; q < R; ++q) {
        float sq[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int e = 64 * (j0 + q) + 4 * seg + k;
            const float d = (IN || e < hi) ? a[4 * q + k] - mu : 0.0f;
            sq[k] = d * d;
        }
#pragma unroll
        for (int g = 0; g < 16; ++g) {
            s = ring_step<16>(s);
#pragma unroll
            for (int k = 0; k < 4; ++k) s = s + sq[k];
        }
    }
}

// y_i = ((x_i - mu) * rstd) * gamma_i + beta_i for R rounds from j0, with
// gamma and beta loaded SPLIT parts at a time (a scheduling barrier before
// each part keeps the compiler from loading them all at once).  A missing
// gamma acts as 1 and a missing beta as -0 (t * 1 == t, t + (-0) == t).
// Positions past H load the row's last piece and are never stored.
template <bool VEC, int R, int SPLIT, bool IN = false>
__device__ __forceinline__ void rs_out(const float (&c)[4 * R], int j0, int hi, int seg, bool live,
                                       const float* xr, float* yr, const float* gamma,
                                       const float* beta, float mu, float rs) {
    const bool has_g = gamma != nullptr, has_b = beta != nullptr;
    const float* gs = has_g ? gamma : xr;
    const float* bs = has_b ? beta : xr;
    constexpr int Q = R / SPLIT;
#pragma unroll
    for (int h = 0; h < SPLIT; ++h) {
        if constexpr (SPLIT > 1) __builtin_amdgcn_sched_barrier(0);
        float gv[4 * Q], bv[4 * Q];
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int o = 64 * (j0 + h * Q + q) + 4 * seg;
            if constexpr (VEC) {
                const int oc = (IN || o < hi) ? o : hi - 4;
                const f32x4 tg = *reinterpret_cast<const f32x4*>(gs + oc);
                const f32x4 tb = *reinterpret_cast<const f32x4*>(bs + oc);
                gv[4 * q] = tg.x;
                gv[4 * q + 1] = tg.y;
                gv[4 * q + 2] = tg.z;
                gv[4 * q + 3] = tg.w;
                bv[4 * q] = tb.x;
                bv[4 * q + 1] = tb.y;
                bv[4 * q + 2] = tb.z;
                bv[4 * q + 3] = tb.w;
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int ok = (IN || o + k < hi) ? o + k : hi - 1;
                    gv[4 * q + k] = gs[ok];
                    bv[4 * q + k] = bs[ok];
                }
            }
        }
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            float t4[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                float t = c[4 * (h * Q + q) + k] - mu;
                t = t * rs;
                t = t * (has_g ? gv[4 * q + k] : 1.0f);
                t = t + (has_b ? bv[4 * q + k] : -0.0f);
                t4[k] = t;
            }
            const int e0 = 64 * (j0 + h * Q + q) + 4 * seg;
            if constexpr (VEC) {
                // H is a multiple of 4 here, so e0 < H covers the whole float4
                if (live && (IN || e0 < hi)) {
                    const f32x4 w = {t4[0], t4[1], t4[2], t4[3]};
                    __builtin_nontemporal_store(w, reinterpret_cast<f32x4*>(yr + e0));
                }
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    if (live && (IN || e0 + k < hi)) yr[e0 + k] = t4[k];
            }
        }
    }
}

// Rows up to this length take the form with more of the row kept on chip.
constexpr int64_t kStreamKeepH = 4096;

template <bool VEC, int C, int NL, int NR>
__global__ __launch_bounds__(64) void repops_layernorm_stream_kernel(
    const float* x, int64_t x_rs, const float* __restrict__ gamma,
    const float* __restrict__ beta, float* y, int64_t y_rs, int64_t rows, int64_t H, float eps,
    float* __restrict__ mean_out, float* __restrict__ rstd_out) {
    static_assert(NL >= 1 && NR >= 0 && C % 2 == 0, "kept chunks: at least one in LDS");
    constexpr int K = NL + NR;  // kept chunks
    // launched for rows longer than 2048 only, so the first KIN chunks lie
    // inside every row and take no bounds tests
    constexpr int KIN = 2048 / (64 * C);
    // gamma and beta in half chunks for the short chunks, whole for long ones
    constexpr int kOutSplit = C <= 4 ? 2 : 1;
    __shared__ f32x4 kept[NL][C][64];
    const int lane = static_cast<int>(threadIdx.x);
    const int seg = lane & 15;
    const int hi = static_cast<int>(H);
    const float fh = static_cast<float>(H);
    const int rounds = (hi + 63) / 64;
    const int64_t groups = (rows + 3) / 4;
    auto put = [&](int slot, const float (&c)[4 * C]) {
#pragma unroll
        for (int q = 0; q < C; ++q)
            kept[slot][q][lane] = f32x4{c[4 * q], c[4 * q + 1], c[4 * q + 2], c[4 * q + 3]};
    };
    auto get = [&](int slot, float (&c)[4 * C]) {
#pragma unroll
        for (int q = 0; q < C; ++q) {
            const f32x4 t = kept[slot][q][lane];
            c[4 * q] = t.x;
            c[4 * q + 1] = t.y;
            c[4 * q + 2] = t.z;
            c[4 * q + 3] = t.w;
        }
    };
    for (int64_t rg = blockIdx.x; rg < groups; rg += gridDim.x) {
        const int64_t row = rg * 4 + (lane >> 4);
        const bool live = row < rows;
        const float* xr = x + (live ? row : 0) * x_rs;
        float sb[2][4 * C];                 // LDS staging, then the streamed chunks
        float kr[NR > 0 ? NR : 1][4 * C];   // chunks NL .. K - 1
        // where chunk c is loaded in the first pass (c is a constant in the
        // unrolled loops below, so this resolves to one array)
        auto home = [&](int c) -> float (&)[4 * C] {
            return c < NL ? sb[c & 1] : (c < K ? kr[c - NL] : sb[0]);
        };

        // S = ((+0 + x_0) + x_1) + ...
        float s = 0.0f;
        rs_load<VEC, C, true>(xr, hi, 0, seg, home(0));
#pragma unroll
        for (int c = 0; c < K; ++c) {
            if (c + 1 < KIN)
                rs_load<VEC, C, true>(xr, hi, (c + 1) * C, seg, home(c + 1));
            else
                rs_load<VEC, C>(xr, hi, (c + 1) * C, seg, home(c + 1));
            if (c < NL) put(c, home(c));
            rs_sum<C>(s, home(c));
        }
        for (int j = K * C; j < rounds; j += 2 * C) {
            rs_load<VEC, C>(xr, hi, j + C, seg, sb[1]);
            rs_sum<C>(s, sb[0]);
            if (j + C >= rounds) break;
            rs_load<VEC, C>(xr, hi, j + 2 * C, seg, sb[0]);
            rs_sum<C>(s, sb[1]);
        }
        // the chunks kept in LDS are read back from there, not carried in
        // registers across the passes
        asm volatile("" ::: "memory");
        s = __shfl(s, 15, 16);
        const float mu = s / fh;

        // S2 = sum of (x_i - mu) * (x_i - mu), the same way
        float s2 = 0.0f;
        rs_load<VEC, C>(xr, hi, K * C, seg, sb[0]);
#pragma unroll
        for (int c = 0; c < NL; ++c) {
            get(c, sb[1]);
            if (c < KIN)
                rs_sum_sq<C, true>(s2, sb[1], mu, hi, c * C, seg);
            else
                rs_sum_sq<C>(s2, sb[1], mu, hi, c * C, seg);
        }
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            if (NL + r < KIN)
                rs_sum_sq<C, true>(s2, kr[r], mu, hi, (NL + r) * C, seg);
            else
                rs_sum_sq<C>(s2, kr[r], mu, hi, (NL + r) * C, seg);
        }
        for (int j = K * C; j < rounds; j += 2 * C) {
            rs_load<VEC, C>(xr, hi, j + C, seg, sb[1]);
            rs_sum_sq<C>(s2, sb[0], mu, hi, j, seg);
            if (j + C >= rounds) break;
            rs_load<VEC, C>(xr, hi, j + 2 * C, seg, sb[0]);
            rs_sum_sq<C>(s2, sb[1], mu, hi, j + C, seg);
        }
        asm volatile("" ::: "memory");
        s2 = __shfl(s2, 15, 16);
        const float var = s2 / fh;
        const float ve = var + eps;
        const float sd = __builtin_sqrtf(ve);
        const float rs = 1.0f / sd;
        if (live && seg == 0) {
            if (mean_out) mean_out[row] = mu;
            if (rstd_out) rstd_out[row] = rs;
        }

        // the streamed chunks last to first, then the kept ones
        float* yr = y + (live ? row : 0) * y_rs;
        const int nch = (rounds + C - 1) / C;
        if (nch > K) {
            rs_load<VEC, C>(xr, hi, (nch - 1) * C, seg, sb[0]);
            for (int c = nch - 1; c >= K; c -= 2) {
                if (c - 1 >= K) rs_load<VEC, C>(xr, hi, (c - 1) * C, seg, sb[1]);
                rs_out<VEC, C, kOutSplit>(sb[0], c * C, hi, seg, live, xr, yr, gamma, beta, mu, rs);
                if (c - 1 < K) break;
                if (c - 2 >= K) rs_load<VEC, C>(xr, hi, (c - 2) * C, seg, sb[0]);
                rs_out<VEC, C, kOutSplit>(sb[1], (c - 1) * C, hi, seg, live, xr, yr, gamma, beta, mu, rs);
            }
        }
#pragma unroll
        for (int r = NR - 1; r >= 0; --r) {
            __builtin_amdgcn_sched_barrier(0);
            if (NL + r < KIN)
                rs_out<VEC, C, kOutSplit, true>(kr[r], (NL + r) * C, hi, seg, live, xr, yr,
                                                gamma, beta, mu, rs);
            else
                rs_out<VEC, C, kOutSplit>(kr[r], (NL + r) * C, hi, seg, live, xr, yr, gamma,
                                          beta, mu, rs);
        }
#pragma unroll
        for (int c = NL - 1; c >= 0; --c) {
            __builtin_amdgcn_sched_barrier(0);
            get(c, sb[0]);
            if (c < KIN)
                rs_out<VEC, C, kOutSplit, true>(sb[0], c * C, hi, seg, live, xr, yr, gamma, beta,
                                                mu, rs);
            else
                rs_out<VEC, C, kOutSplit>(sb[0], c * C, hi, seg, live, xr, yr, gamma, beta, mu,
                                          rs);
        }
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
    // Register-resident forms for rows of at most 2048 elements: a quad of
    // lanes per row up to 768 (16 rows per wave), 16 lanes per row above
    // (4 rows per wave).  S (elements per lane) is the smallest that holds
    // the row, since every sum walks all L * S slots.  (Forms for 3072 and
    // 4096 would need 269 and 462 VGPRs, one wave per SIMD; the streaming
    // form below matches them there and is faster in between.)
    if (H <= 2048) {
        using Gn = void (*)(const float*, int64_t, const float*, const float*, float*, int64_t,
                            int64_t, int64_t, float, float*, float*);
        Gn gn;
        int rows_per_wave = 4;
        if (H <= 256) {
            gn = vec ? repops_layernorm_regs_kernel<4, 64, true>
                     : repops_layernorm_regs_kernel<4, 64, false>;
            rows_per_wave = 16;
        } else if (H <= 512) {
            gn = vec ? repops_layernorm_regs_kernel<4, 128, true>
                     : repops_layernorm_regs_kernel<4, 128, false>;
            rows_per_wave = 16;
        } else if (H <= 768) {
            gn = vec ? repops_layernorm_regs_kernel<4, 192, true>
                     : repops_layernorm_regs_kernel<4, 192, false>;
            rows_per_wave = 16;
        } else if (H <= 1024) {
            gn = vec ? repops_layernorm_regs_kernel<16, 64, true>
                     : repops_layernorm_regs_kernel<16, 64, false>;
        } else if (H <= 1536) {
            gn = vec ? repops_layernorm_regs_kernel<16, 96, true>
                     : repops_layernorm_regs_kernel<16, 96, false>;
        } else {
            gn = vec ? repops_layernorm_regs_kernel<16, 128, true>
                     : repops_layernorm_regs_kernel<16, 128, false>;
        }
        const int64_t groups = (rows + rows_per_wave - 1) / rows_per_wave;
        const int64_t gblocks = groups < (int64_t(1) << 20) ? groups : (int64_t(1) << 20);
        hipLaunchKernelGGL(gn, dim3(static_cast<unsigned>(gblocks)), dim3(64), 0, s, x, x_rs,
                           gamma, beta, y, y_rs, rows, H, eps, mean, rstd);
        return static_cast<int>(hipGetLastError());
    }
    // Longer rows stream, 16 lanes per row.  Chunks of 4 rounds, 5 kept in
    // LDS and 3 in registers (2048 elements of each row) up to 4096; above,
    // chunks of 8 rounds with 2 kept in LDS; the unaligned (scalar-load) form
    // uses the latter everywhere, as the former would spill there.
    const int64_t groups = (rows + 3) / 4;
    const int64_t blocks = groups < (int64_t(1) << 20) ? groups : (int64_t(1) << 20);
    using Fn = void (*)(const float*, int64_t, const float*, const float*, float*, int64_t,
                        int64_t, int64_t, float, float*, float*);
    Fn fn = !vec ? repops_layernorm_stream_kernel<false, 8, 2, 0>
            : H <= kStreamKeepH ? repops_layernorm_stream_kernel<true, 4, 5, 5>
                                : repops_layernorm_stream_kernel<true, 8, 2, 1>;
    hipLaunchKernelGGL(fn, dim3(static_cast<unsigned>(blocks)), dim3(64), 0, s, x, x_rs, gamma,
                       beta, y, y_rs, rows, H, eps, mean, rstd);
    return static_cast<int>(hipGetLastError());
}

}  // namespace repops
