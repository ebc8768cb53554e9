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

// LayerNorm, streaming form (rows longer than the register-resident forms
// below hold).  The two sums over a row are the fixed-order dimension, so one
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
template <int L, int S, bool VEC, bool FULL>
__device__ __forceinline__ void ln_regs_group(const float* xs, float* ys, int hl, bool live,
                                              int64_t row, int seg, float fh, float eps,
                                              const float* gs, const float* bs,
                                              float* __restrict__ mean_out,
                                              float* __restrict__ rstd_out) {
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
    if constexpr (VEC) {
        for (int c = 4 * lane; c < L * S; c += 256) {
            f32x4 gv = {1.0f, 1.0f, 1.0f, 1.0f}, bv = {-0.0f, -0.0f, -0.0f, -0.0f};
            if (gamma && c < hi) gv = *reinterpret_cast<const f32x4*>(gamma + c);
            if (beta && c < hi) bv = *reinterpret_cast<const f32x4*>(beta + c);
            *reinterpret_cast<f32x4*>(ln_g + c) = gv;
            *reinterpret_cast<f32x4*>(ln_b + c) = bv;
        }
    } else {
        for (int c = lane; c < L * S; c += 64) {
            ln_g[c] = gamma && c < hi ? gamma[c] : 1.0f;
            ln_b[c] = beta && c < hi ? beta[c] : -0.0f;
        }
    }
    __syncthreads();
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
                                           ln_b + P * seg, mean_out, rstd_out);
        else
            ln_regs_group<L, S, VEC, false>(xs, ys, hl, live, row, seg, fh, eps, ln_g + P * seg,
                                            ln_b + P * seg, mean_out, rstd_out);
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
    // Register-resident forms for rows of at most 4096 elements: a quad of
    // lanes per row up to 768 (16 rows per wave), 16 lanes per row above
    // (4 rows per wave).  S (elements per lane) is the smallest that holds
    // the row, since every sum walks all L * S slots.
    if (H <= 4096) {
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
        } else if (H <= 2048) {
            gn = vec ? repops_layernorm_regs_kernel<16, 128, true>
                     : repops_layernorm_regs_kernel<16, 128, false>;
        } else if (H <= 3072) {
            gn = vec ? repops_layernorm_regs_kernel<16, 192, true>
                     : repops_layernorm_regs_kernel<16, 192, false>;
        } else {
            gn = vec ? repops_layernorm_regs_kernel<16, 256, true>
                     : repops_layernorm_regs_kernel<16, 256, false>;
        }
        const int64_t groups = (rows + rows_per_wave - 1) / rows_per_wave;
        const int64_t gblocks = groups < (int64_t(1) << 20) ? groups : (int64_t(1) << 20);
        hipLaunchKernelGGL(gn, dim3(static_cast<unsigned>(gblocks)), dim3(64), 0, s, x, x_rs,
                           gamma, beta, y, y_rs, rows, H, eps, mean, rstd);
        return static_cast<int>(hipGetLastError());
    }
    // Longer rows stream through LDS.
    const int64_t blocks = (rows + kLnRows - 1) / kLnRows;
    using Fn = void (*)(const float*, int64_t, const float*, const float*, float*, int64_t,
                        int64_t, int64_t, float, float*, float*);
    Fn fn = vec ? repops_layernorm_kernel<true> : repops_layernorm_kernel<false>;
    hipLaunchKernelGGL(fn, dim3(static_cast<unsigned>(blocks)), dim3(kLnThreads), 0, s, x, x_rs,
                       gamma, beta, y, y_rs, rows, H, eps, mean, rstd);
    return static_cast<int>(hipGetLastError());
}

}  // namespace repops
