// gfx950 kernels for the reproducible fixed-order FP32 matmul.
//
// Every output element is computed by exactly one lane as
//     s = +0.0f;  for k = 0 .. K-1:  s = RN(s + RN(a_k * b_k));  C(i,j) = s
// (Verde and RepOps article, section 3.2 "RepOps design principles", item 2:
// (i, j) may run in any order, k runs in a fixed order).  The multiply and
// the add are two separately rounded binary32 operations: this file is
// compiled with -ffp-contract=off and the pragma below, so no fused
// multiply-add can be formed, and the build's instruction scan rejects any
// v_fma/v_fmac/v_mad/v_mac/v_dot/packed-FP32 instruction in the result.
// There is no split-K and no cross-lane reduction: the only thing the tiling
// changes is which lane computes which (i, j) and when its operands arrive.
//
// K tails are padded with +0 on both operands.  A padded step computes
// s + RN(0 * 0) = s + (+0), which equals s because s is never -0 (it starts
// at +0, and under round-to-nearest an addition returns -0 only when both
// addends are -0).  So padding does not change a bit.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "repops_internal.h"

#pragma clang fp contract(off)

namespace repops {
namespace {

constexpr int kThreads = 256;
constexpr int kPad = 4;  // LDS row padding (floats); keeps rows 16-byte aligned

// Binary32 multiply and add, each rounded on its own (contraction is off).
__device__ __forceinline__ float mul_rn(float a, float b) { return a * b; }
__device__ __forceinline__ float add_rn(float a, float b) { return a + b; }

// Moves the views to batch blockIdx.y (batch is a free dimension).
__device__ __forceinline__ void select_batch(OperandView& A, OperandView& B, OutView& C) {
    const int64_t b = blockIdx.y;
    A.p += b * A.s_b;
    B.p += b * B.s_b;
    C.p += b * C.s_b;
    if (C.bias) C.bias += b * C.bias_sb;
}

// The stored value of output column j: the fixed-order sum, then (with a
// bias) one more separately rounded add.
__device__ __forceinline__ float epilogue_value(const OutView& C, int64_t j, float sum) {
    return C.bias ? add_rn(sum, C.bias[j * C.bias_s]) : sum;
}

// ---------------------------------------------------------------------------
// Global -> register -> LDS staging of one X x BK operand tile.
// LDS holds the tile k-major: lds[k * (BX + kPad) + x].  Each lane owns kNV
// loads at fixed tile coordinates; their addresses are formed once and
// advanced by BK * s_k per k-tile.
//
// Rows beyond the operand (x >= X) are clamped to a valid row: they only feed
// outputs that are never stored, so their values do not matter and the
// steady-state loads need no masks.  Only the last, partial k-tile (when BK
// does not divide K) is masked, and there both operands read +0 for k >= K.
template <int BX, int BK, int LAY, int NT = kThreads>
struct TileStage {
    static constexpr int kElems = BX * BK / NT;        // floats per lane
    static constexpr int kVec = (LAY == LAY_GEN) ? 1 : 4;
    static constexpr int kNV = kElems / kVec;          // loads per lane
    static constexpr int kLd = BX + kPad;
    static_assert(kElems * NT == BX * BK, "tile must split evenly over lanes");
    static_assert(kNV * kVec == kElems, "vector loads must split evenly");

    float r[kElems];
    const float* src[kNV];  // address of load v in the next k-tile to load
    int kofs[kNV];          // k offset of load v inside its tile
    int64_t step;           // BK * s_k

    // Coordinates (x, k) inside the tile of the first element of load v.
    __device__ static void coords(int tid, int v, int& x, int& k) {
        const int f = tid + NT * v;
        if constexpr (LAY == LAY_KC) {         // 4 consecutive k of one row
            // 16 consecutive lanes take 16 consecutive rows and the next 16
            // the next group of 4 k: a wave's loads still cover 16 whole
            // 64-byte row pieces, and each of its four k-major LDS stores
            // (row pitch BX + 4 = 4 mod 32 words) hits 64 distinct banks.
            static_assert(BX % 16 == 0, "rows come in groups of 16");
            constexpr int KQ = BK / 4;         // groups of 4 k per row
            x = (f & 15) + 16 * (f / (16 * KQ));
            k = ((f >> 4) % KQ) * 4;
        } else if constexpr (LAY == LAY_XC) {  // 4 consecutive x of one k
            x = (f % (BX / 4)) * 4;
            k = f / (BX / 4);
        } else {                               // consecutive lanes, consecutive x
            x = f % BX;
            k = f / BX;
        }
    }

    __device__ void init(const OperandView& op, int64_t x0, int tid) {
        step = static_cast<int64_t>(BK) * op.s_k;
#pragma unroll
        for (int v = 0; v < kNV; ++v) {
            int x, k;
            coords(tid, v, x, k);
            int64_t gx = x0 + x;
            // LAY_XC is only chosen when 4 divides X, so a clamped vector
            // start X-4 keeps all four elements inside the operand.
            const int64_t last = (LAY == LAY_XC) ? op.X - 4 : op.X - 1;
            gx = gx < last ? gx : last;
            kofs[v] = k;
            src[v] = op.p + gx * op.s_x + static_cast<int64_t>(k) * op.s_k;
        }
    }

    // A k-tile that lies entirely inside [0, K).
    __device__ void load_full() {
#pragma unroll
        for (int v = 0; v < kNV; ++v) {
            const float* p = src[v];
            src[v] = p + step;
            if constexpr (LAY == LAY_GEN) {
                r[v] = *p;
            } else {
                const float4 q = *reinterpret_cast<const float4*>(p);
                r[4 * v + 0] = q.x; r[4 * v + 1] = q.y; r[4 * v + 2] = q.z; r[4 * v + 3] = q.w;
            }
        }
    }

    // The k-tile starting at k0 that crosses K: elements with k >= K read +0.
    __device__ void load_tail(int64_t k0, int64_t K, int64_t s_k) {
#pragma unroll
        for (int v = 0; v < kNV; ++v) {
            const float* p = src[v];
            src[v] = p + step;
            const int64_t gk = k0 + kofs[v];
            if constexpr (LAY == LAY_GEN) {
                r[v] = gk < K ? *p : 0.0f;
            } else if constexpr (LAY == LAY_KC) {  // s_k == 1: 4 consecutive k
#pragma unroll
                for (int e = 0; e < 4; ++e) r[4 * v + e] = gk + e < K ? p[e] : 0.0f;
            } else {                               // one k, 4 consecutive x
#pragma unroll
                for (int e = 0; e < 4; ++e) r[4 * v + e] = gk < K ? p[e] : 0.0f;
            }
        }
        (void)s_k;
    }

    __device__ void store(float* lds, int tid) const {
#pragma unroll
        for (int v = 0; v < kNV; ++v) {
            int x, k;
            coords(tid, v, x, k);
            if constexpr (LAY == LAY_GEN) {
                lds[k * kLd + x] = r[v];
            } else if constexpr (LAY == LAY_KC) {
#pragma unroll
                for (int e = 0; e < 4; ++e) lds[(k + e) * kLd + x] = r[4 * v + e];
            } else {
                *reinterpret_cast<float4*>(&lds[k * kLd + x]) =
                    make_float4(r[4 * v + 0], r[4 * v + 1], r[4 * v + 2], r[4 * v + 3]);
            }
        }
    }
};

// ---------------------------------------------------------------------------
// Workgroup -> (tile row, tile column).  Any bijection is correct; these
// orders only change cache reuse.  Divisions by runtime sizes use the
// host-computed multiply-shift constants of TileGrid (integer only).
__device__ __forceinline__ uint32_t fdiv(uint32_t n, FastDiv f) {
    return static_cast<uint32_t>((static_cast<uint64_t>(n) * f.m) >> f.s);
}

__device__ __forceinline__ void tile_of_block(const TileGrid& g, int& tm, int& tn) {
    const uint32_t w = blockIdx.x;
    if (g.order == ORDER_ROW) {
        const uint32_t q = fdiv(w, g.div_n);
        tm = static_cast<int>(q);
        tn = static_cast<int>(w - q * g.div_n.d);
        return;
    }
    if (g.order == ORDER_COL) {
        const uint32_t q = fdiv(w, g.div_m);
        tn = static_cast<int>(q);
        tm = static_cast<int>(w - q * g.div_m.d);
        return;
    }
    // Workgroups are dealt round-robin to the 8 XCDs, each with its own L2.
    // Give XCD x the contiguous tile range [x*per, (x+1)*per) so tiles that
    // share operand panels meet in one L2; the remainder keeps its identity.
    const uint32_t total = static_cast<uint32_t>(g.tiles_m) * static_cast<uint32_t>(g.tiles_n);
    const uint32_t per = total >> 3;
    uint32_t t = w;
    if (w < (per << 3)) t = (w & 7) * per + (w >> 3);
    // Then walk groups of 8 tile rows, tile rows fastest inside a group; the
    // last group may have fewer rows.
    const uint32_t group = fdiv(t, g.div_span);  // span = 8 * tiles_n
    const uint32_t first_m = group << 3;
    const uint32_t local = t - group * g.div_span.d;
    uint32_t q;
    if (first_m + 8 <= static_cast<uint32_t>(g.tiles_m)) {
        q = local >> 3;
        tm = static_cast<int>(first_m + (local & 7));
    } else {  // rows = tiles_m - first_m = tiles_m % 8
        q = fdiv(local, g.div_last);
        tm = static_cast<int>(first_m + (local - q * g.div_last.d));
    }
    tn = static_cast<int>(q);
}

// The TM row operands and TN column operands of one k step, as float4 reads
// of the k-major LDS tiles (as/bs already offset by the lane's ty*4 / tx*4).
template <int RG, int CG, int RSPAN, int CSPAN>
__device__ __forceinline__ void read_lane_operands(const float* as, const float* bs, float* a,
                                                   float* b) {
#pragma unroll
    for (int g = 0; g < RG; ++g) {
        const float4 q = *reinterpret_cast<const float4*>(as + g * RSPAN);
        a[4 * g + 0] = q.x; a[4 * g + 1] = q.y; a[4 * g + 2] = q.z; a[4 * g + 3] = q.w;
    }
#pragma unroll
    for (int h = 0; h < CG; ++h) {
        const float4 q = *reinterpret_cast<const float4*>(bs + h * CSPAN);
        b[4 * h + 0] = q.x; b[4 * h + 1] = q.y; b[4 * h + 2] = q.z; b[4 * h + 3] = q.w;
    }
}

// BK ascending k steps of one lane's TM x TN block: acc += a*b, the multiply
// and the add separately rounded.  Operands of step k+1 are read into the
// other register set while step k computes, so only two steps of operands
// are ever live.
template <int BK, int TM, int TN, int RSPAN, int CSPAN, int LDA, int LDB>
__device__ __forceinline__ void lane_tile_steps(const float* as, const float* bs,
                                                float (&acc)[TM][TN]) {
    constexpr int RG = TM / 4, CG = TN / 4;
    float a[2][TM], b[2][TN];
    read_lane_operands<RG, CG, RSPAN, CSPAN>(as, bs, a[0], b[0]);
#pragma unroll
    for (int k = 0; k < BK; ++k) {
        const int c = k & 1;
        if (k + 1 < BK)
            read_lane_operands<RG, CG, RSPAN, CSPAN>(as + (k + 1) * LDA, bs + (k + 1) * LDB,
                                                     a[c ^ 1], b[c ^ 1]);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = add_rn(acc[i][j], mul_rn(a[c][i], b[c][j]));
        // Pin step k's adds here: an empty volatile asm that reads and writes
        // each accumulator is ordered with the LDS reads, so the instruction
        // selector cannot sink the arithmetic below later reads.
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) asm volatile("" : "+v"(acc[i][j]));
        __builtin_amdgcn_sched_barrier(0);
    }
}

// ---------------------------------------------------------------------------
// Register-blocked VALU kernel.  256 lanes own a BM x BN output tile; lane
// (ty, tx) owns TM x TN outputs in groups of 4 consecutive rows/columns:
// rows g*(BM/(TM/4)) + ty*4 + e, columns h*(BN/(TN/4)) + tx*4 + f.  Operand
// tiles are double-buffered in LDS with one barrier per BK step.
template <int BM, int BN, int BK, int TM, int TN, int LA, int LB>
__global__ __launch_bounds__(kThreads) void repops_tiled_kernel(OperandView A, OperandView B,
                                                                OutView C, int64_t M, int64_t N,
                                                                int64_t K, TileGrid grid) {
    static_assert((BM / TM) * (BN / TN) == kThreads, "one lane per TM x TN block");
    static_assert(TM % 4 == 0 && TN % 4 == 0, "lane blocks are groups of 4");
    constexpr int RG = TM / 4, CG = TN / 4;
    constexpr int RSPAN = BM / RG, CSPAN = BN / CG;
    constexpr int LDA = BM + kPad, LDB = BN + kPad;

    __shared__ __attribute__((aligned(16))) float As[2][BK * LDA];
    __shared__ __attribute__((aligned(16))) float Bs[2][BK * LDB];

    const int tid = static_cast<int>(threadIdx.x);
    const int tx = tid % (BN / TN);
    const int ty = tid / (BN / TN);
    int tm, tn;
    tile_of_block(grid, tm, tn);
    select_batch(A, B, C);
    const int64_t m0 = static_cast<int64_t>(tm) * BM;
    const int64_t n0 = static_cast<int64_t>(tn) * BN;

    float acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = 0.0f;  // s = +0

    TileStage<BM, BK, LA> sa;
    TileStage<BN, BK, LB> sb;
    sa.init(A, m0, tid);
    sb.init(B, n0, tid);
    const int64_t nfull = K / BK;              // k-tiles entirely inside [0, K)
    const bool tail = (K % BK) != 0;           // one more, partial k-tile
    const float* as0 = &As[0][ty * 4];
    const float* bs0 = &Bs[0][tx * 4];
    const float* as1 = &As[1][ty * 4];
    const float* bs1 = &Bs[1][tx * 4];

    if (nfull > 0) {
        sa.load_full();
        sb.load_full();
    } else {
        sa.load_tail(0, K, A.s_k);
        sb.load_tail(0, K, B.s_k);
    }
    sa.store(As[0], tid);
    sb.store(Bs[0], tid);
    __syncthreads();

    // k-tile kt sits in LDS buffer kt&1 while tile kt+1 is fetched into
    // registers.  One copy of the compute: the next-tile loads sit behind
    // uniform branches, fenced off by empty asm memory barriers so the
    // compiler cannot move the compute's LDS reads across them.
    const int64_t ktiles = nfull + (tail ? 1 : 0);
    for (int64_t kt = 0; kt < ktiles; ++kt) {
        const bool more = kt + 1 < ktiles;
        if (kt + 1 < nfull) {
            sa.load_full();
            sb.load_full();
        } else if (more) {
            sa.load_tail(nfull * BK, K, A.s_k);
            sb.load_tail(nfull * BK, K, B.s_k);
        }
        asm volatile("" ::: "memory");
        const bool odd = (kt & 1) != 0;
        lane_tile_steps<BK, TM, TN, RSPAN, CSPAN, LDA, LDB>(odd ? as1 : as0, odd ? bs1 : bs0, acc);
        asm volatile("" ::: "memory");
        if (more) {
            sa.store(odd ? As[0] : As[1], tid);
            sb.store(odd ? Bs[0] : Bs[1], tid);
        }
        __syncthreads();
    }

    // Epilogue: plain stores of s; C is never read.
    const bool vec_store = (C.s_j == 1) && ((C.s_i & 3) == 0) &&
                           ((reinterpret_cast<uintptr_t>(C.p) & 15) == 0);
#pragma unroll
    for (int g = 0; g < RG; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t i = m0 + g * RSPAN + ty * 4 + e;
            if (i >= M) continue;
#pragma unroll
            for (int h = 0; h < CG; ++h) {
                const int64_t j0 = n0 + h * CSPAN + tx * 4;
                const float* v = &acc[4 * g + e][4 * h];
                if (vec_store && j0 + 3 < N) {
                    *reinterpret_cast<float4*>(C.p + i * C.s_i + j0) =
                        make_float4(epilogue_value(C, j0, v[0]), epilogue_value(C, j0 + 1, v[1]),
                                    epilogue_value(C, j0 + 2, v[2]), epilogue_value(C, j0 + 3, v[3]));
                } else {
#pragma unroll
                    for (int f = 0; f < 4; ++f)
                        if (j0 + f < N)
                            C.p[i * C.s_i + (j0 + f) * C.s_j] = epilogue_value(C, j0 + f, v[f]);
                }
            }
        }
}

// ---------------------------------------------------------------------------
// Scalar-row kernel.  Each wave owns R whole rows of a BM x BN output tile
// (BM = R * W for W waves, BN = 64 * CN), so for every k the R values
// op(A)(i, k) the wave needs are the same in all 64 lanes.  They come in
// through scalar loads into SGPRs, AK consecutive k at a time, one chunk
// ahead of use, and every v_mul_f32 takes one of them as its scalar operand.
// Lane l owns the CN columns n0 + l + 64c; its B values come from the
// k-major LDS tile (double-buffered, staged as in the other kernels), read
// one chunk ahead.  A lane reads 1/R LDS words per multiply-accumulate and
// needs only R x CN outputs: a problem too small to fill the chip with the
// register-blocked tiles still gets several waves per SIMD.
//
// Rows beyond M are clamped to row M-1 (their sums are never stored); k >= K
// reads +0 for A (a clamped, in-bounds address, then a uniform select) and for
// B (the tile loader), so a padded step adds +0 to s and changes no bit.
//
// A is read through the constant address space: it is not written while the
// kernel runs (the host refuses a C that overlaps it), and a wave-uniform load
// from that space is always a scalar load.
typedef const __attribute__((address_space(4))) float* ConstF32Ptr;

// A wave-uniform pointer held in SGPRs (64-bit compares and multiplies may be
// formed on the VALU, so a value derived from them is moved back explicitly).
__device__ __forceinline__ ConstF32Ptr uniform_ptr(ConstF32Ptr p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(v)));
    const uint32_t hi =
        static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(v >> 32)));
    return reinterpret_cast<ConstF32Ptr>((static_cast<uint64_t>(hi) << 32) | lo);
}

template <int R, int CN, int W, int BK, int LA, int LB, bool PRIO>
__global__ __launch_bounds__(64 * W) void repops_srow_kernel(OperandView A, OperandView B,
                                                             OutView C, int64_t M, int64_t N,
                                                             int64_t K, TileGrid grid) {
    constexpr int NT = 64 * W;
    constexpr int BM = R * W, BN = 64 * CN;
    constexpr int LDB = BN + kPad;
    // k values per row in one scalar chunk: two chunks (the one in use and the
    // next) of R x AK SGPRs stay within 32 registers, next to the kernel
    // arguments and addresses that also live in SGPRs.
    constexpr int AK = (R >= 8) ? 2 : (R >= 4 ? 4 : (R >= 2 ? 8 : 16));
    constexpr int CHUNKS = BK / AK;  // chunks per k-tile
    static_assert(BK % AK == 0, "a k-tile holds whole scalar chunks");

    __shared__ __attribute__((aligned(16))) float Bs[2][BK * LDB];

    const int tid = static_cast<int>(threadIdx.x);
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int tm, tn;
    tile_of_block(grid, tm, tn);
    select_batch(A, B, C);
    const int64_t m0 = static_cast<int64_t>(tm) * BM;
    const int64_t n0 = static_cast<int64_t>(tn) * BN;

    // This wave's rows of op(A), clamped into the operand.
    const ConstF32Ptr a0 = (ConstF32Ptr)(A.p);
    const int64_t sk = (LA == LAY_KC) ? 1 : A.s_k;
    const int64_t sx = (LA == LAY_XC) ? 1 : A.s_x;
    ConstF32Ptr pa[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t i = m0 + wave * R + r;
        pa[r] = uniform_ptr(a0 + (i < M ? i : M - 1) * sx);
    }
    // Loads the next scalar chunk.  Rows stored along k (LAY_KC) keep fixed
    // row pointers and one 32-bit byte offset, which the scalar load takes as
    // its offset register (one scalar add per chunk; the host launches these
    // kernels only for K < 2^30).  Other layouts walk each row pointer along
    // k.  The offset or pointers pass through an empty asm first, so the
    // compiler cannot hoist or merge the loads of later chunks: only two
    // chunks are ever live in SGPRs.
    uint32_t koff = 0;
    auto load_chunk = [&](float (&dst)[R][AK]) {
        if constexpr (LA == LAY_KC) {
            asm volatile("" : "+s"(koff));
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const ConstF32Ptr p =
                    (ConstF32Ptr)((const __attribute__((address_space(4))) char*)(pa[r]) + koff);
#pragma unroll
                for (int kk = 0; kk < AK; ++kk) dst[r][kk] = p[kk];
            }
            koff += AK * 4;
        } else {
#pragma unroll
            for (int r = 0; r < R; ++r) asm volatile("" : "+s"(pa[r]));
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int kk = 0; kk < AK; ++kk) dst[r][kk] = pa[r][kk * sk];
#pragma unroll
            for (int r = 0; r < R; ++r) pa[r] = uniform_ptr(pa[r] + AK * sk);
        }
    };

    float acc[R][CN];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < CN; ++c) acc[r][c] = 0.0f;  // s = +0

    // k bookkeeping is 32-bit, so each test on it is a scalar compare and the
    // values it selects stay in SGPRs.
    TileStage<BN, BK, LB, NT> sb;
    sb.init(B, n0, tid);
    const int Kr = static_cast<int>(K);
    const int nfull = Kr / BK;                 // k-tiles entirely inside [0, K)
    const bool tail = (Kr % BK) != 0;

    float ac[R][AK];
    if (nfull > 0) {
        load_chunk(ac);
        sb.load_full();
    } else {
        sb.load_tail(0, K, B.s_k);
    }
    sb.store(Bs[0], tid);
    __syncthreads();

    auto read_b = [&](float (&dst)[AK][CN], const float* bk) {
#pragma unroll
        for (int kk = 0; kk < AK; ++kk)
#pragma unroll
            for (int c = 0; c < CN; ++c) dst[kk][c] = bk[kk * LDB + 64 * c];
    };
    // One whole k-tile.  Every scalar chunk of it lies inside [0, K); the
    // next chunk's scalar loads go out before the current chunk's steps,
    // except after the last chunk of the last whole tile (LAST), where there
    // is no next whole chunk.  B values are read one chunk ahead inside the
    // tile.
    auto whole_tile = [&](int kt, auto last) {
        constexpr bool LAST = decltype(last)::value;
        const bool more = !LAST || tail;
        if (!LAST) sb.load_full();
        else if (tail) sb.load_tail(static_cast<int64_t>(nfull) * BK, K, B.s_k);
        asm volatile("" ::: "memory");
        const float* bs = &Bs[kt & 1][lane];
        float bc[AK][CN];
        read_b(bc, bs);
#pragma unroll
        for (int h = 0; h < CHUNKS; ++h) {
            // Scalar loads and LDS reads share one completion counter and
            // scalar loads may return out of order, so everything issued
            // before is waited for here (the empty asm uses this chunk's B
            // values): this chunk's B values and A chunk, both issued one
            // chunk earlier.  Then the next chunk's LDS reads and scalar loads
            // go out, and overlap this chunk's arithmetic.
#pragma unroll
            for (int kk = 0; kk < AK; ++kk)
#pragma unroll
                for (int c = 0; c < CN; ++c) asm volatile("" ::"v"(bc[kk][c]));
            float bn[AK][CN];
            if (h + 1 < CHUNKS) read_b(bn, bs + (h + 1) * AK * LDB);
            // (a constant once the loop over h is unrolled)
            const bool next = !LAST || h + 1 < CHUNKS;
            float an[R][AK];
            if (next) load_chunk(an);
            // Nothing moves across: the loads stay ahead of the arithmetic.
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int kk = 0; kk < AK; ++kk)
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int c = 0; c < CN; ++c)
                        acc[r][c] = add_rn(acc[r][c], mul_rn(ac[r][kk], bc[kk][c]));
            // Pin this chunk's adds here, ahead of the next chunk's waits.
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int c = 0; c < CN; ++c) asm volatile("" : "+v"(acc[r][c]));
            if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
            if (next) {
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int kk = 0; kk < AK; ++kk) ac[r][kk] = an[r][kk];
            }
            if (h + 1 < CHUNKS) {
#pragma unroll
                for (int kk = 0; kk < AK; ++kk)
#pragma unroll
                    for (int c = 0; c < CN; ++c) bc[kk][c] = bn[kk][c];
            }
        }
        asm volatile("" ::: "memory");
        if (more) sb.store(Bs[(kt + 1) & 1], tid);
        __syncthreads();
    };
    for (int kt = 0; kt + 1 < nfull; ++kt) whole_tile(kt, std::false_type{});
    if (nfull > 0) whole_tile(nfull - 1, std::true_type{});

    // The partial last k-tile: k >= K reads +0 on both sides (for A, a
    // clamped in-bounds load, then a uniform select kept scalar).
    if (tail) {
        const float* bs = &Bs[nfull & 1][lane];
        const int rem = Kr - nfull * BK;
        ConstF32Ptr pt[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t i = m0 + wave * R + r;
            pt[r] = uniform_ptr(a0 + (i < M ? i : M - 1) * sx +
                                static_cast<int64_t>(nfull) * BK * sk);
        }
#pragma unroll 1
        for (int kk = 0; kk < BK; ++kk) {
            float b[CN];
#pragma unroll
            for (int c = 0; c < CN; ++c) b[c] = bs[kk * LDB + 64 * c];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float v = pt[r][(kk < rem ? kk : rem - 1) * sk];
                const float a = __int_as_float(
                    __builtin_amdgcn_readfirstlane(__float_as_int(kk < rem ? v : 0.0f)));
#pragma unroll
                for (int c = 0; c < CN; ++c) acc[r][c] = add_rn(acc[r][c], mul_rn(a, b[c]));
            }
        }
    }

    // Epilogue: each row's CN sums, 64 consecutive columns per store.
    float bias[CN];
#pragma unroll
    for (int c = 0; c < CN; ++c) {
        const int64_t j = n0 + lane + 64 * c;
        bias[c] = (C.bias != nullptr && j < N) ? C.bias[j * C.bias_s] : 0.0f;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t i = m0 + wave * R + r;
        if (i >= M) continue;
#pragma unroll
        for (int c = 0; c < CN; ++c) {
            const int64_t j = n0 + lane + 64 * c;
            if (j < N)
                C.p[i * C.s_i + j * C.s_j] = C.bias ? add_rn(acc[r][c], bias[c]) : acc[r][c];
        }
    }
}

// ---------------------------------------------------------------------------
// Matrix-core products, VALU sums.
//
// v_mfma_f32_32x32x1_2b_f32 has an inner dimension of 1: with the addend C
// set to +0 it returns, for each of its 2 x 32 x 32 outputs, the single
// product a_i * b_j + 0 rounded once to binary32 -- the same bits as a
// separately rounded binary32 multiply (gradual underflow, round to nearest
// even), except that an exact -0 product comes back as +0.  That exception
// cannot change a result: the running sum s starts at +0 and never becomes
// -0, and s + (+0) == s + (-0) for every such s.  The matrix core therefore
// forms the products of one k step while the VALU adds the previous step's
// products into the accumulators, one v_add_f32 per multiply-accumulate, in
// ascending k.  No sum is ever formed inside the matrix core.
//
// Wave layout: lane l feeds row l of a 64-row strip (block l/32 of the
// instruction) and column l%32 of a 32-column block (the same column in both
// halves of the wave).  Register v of lane l then holds output row
// 32*(v/16) + 8*((v%16)/4) + 4*(l/32) + v%4 and column l%32.
typedef float f32x32 __attribute__((ext_vector_type(32)));

__device__ __forceinline__ int mprod_row(int v, int lane) {
    return 32 * (v >> 4) + 8 * ((v & 15) >> 2) + 4 * (lane >> 5) + (v & 3);
}

// BK ascending k steps for one wave: TN column blocks of 32.  as/bs point at
// this lane's row / column in the k-major LDS tiles.  Operands are read one
// step ahead.  PIPE == 2 also forms products one step ahead (the matrix
// instruction for k+1 is issued before the adds of step k, two product
// buffers); PIPE == 1 keeps one product buffer and relies on the other waves
// of the SIMD to fill the wait, which halves the product registers and
// raises occupancy.  The empty asm pins each step's adds before the next
// step's LDS reads.
template <int BK, int TN, int LDA, int LDB, int PIPE, bool PRIO>
__device__ __forceinline__ void mprod_tile_steps(const float* as, const float* bs,
                                                 float (&acc)[TN][32]) {
    const f32x32 zero = {};
    if constexpr (PIPE == 2) {
        f32x32 p[2][TN];
        float a[2], b[2][TN];
        a[0] = as[0];
#pragma unroll
        for (int t = 0; t < TN; ++t) b[0][t] = bs[t * 32];
        if (BK > 1) {
            a[1] = as[LDA];
#pragma unroll
            for (int t = 0; t < TN; ++t) b[1][t] = bs[LDB + t * 32];
        }
#pragma unroll
        for (int t = 0; t < TN; ++t)
            p[0][t] = __builtin_amdgcn_mfma_f32_32x32x1f32(a[0], b[0][t], zero, 0, 0, 0);
#pragma unroll
        for (int k = 0; k < BK; ++k) {
            const int c = k & 1;
            if (k + 1 < BK) {
#pragma unroll
                for (int t = 0; t < TN; ++t)
                    p[c ^ 1][t] = __builtin_amdgcn_mfma_f32_32x32x1f32(a[c ^ 1], b[c ^ 1][t],
                                                                       zero, 0, 0, 0);
            }
            if (k + 2 < BK) {
                a[c] = as[(k + 2) * LDA];
#pragma unroll
                for (int t = 0; t < TN; ++t) b[c][t] = bs[(k + 2) * LDB + t * 32];
            }
            if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int t = 0; t < TN; ++t)
#pragma unroll
                for (int v = 0; v < 32; ++v) acc[t][v] = add_rn(acc[t][v], p[c][t][v]);
#pragma unroll
            for (int t = 0; t < TN; ++t)
#pragma unroll
                for (int v = 0; v < 32; ++v) asm volatile("" : "+v"(acc[t][v]));
            if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
            // Inside the step: matrix instructions, LDS reads, then the adds
            // (which read products issued one step earlier).
            __builtin_amdgcn_sched_group_barrier(0x008, TN, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1 + TN, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 32 * TN, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    } else {
        float a[2], b[2][TN];
        a[0] = as[0];
#pragma unroll
        for (int t = 0; t < TN; ++t) b[0][t] = bs[t * 32];
#pragma unroll
        for (int k = 0; k < BK; ++k) {
            const int c = k & 1;
            f32x32 p[TN];
#pragma unroll
            for (int t = 0; t < TN; ++t)
                p[t] = __builtin_amdgcn_mfma_f32_32x32x1f32(a[c], b[c][t], zero, 0, 0, 0);
            if (k + 1 < BK) {
                a[c ^ 1] = as[(k + 1) * LDA];
#pragma unroll
                for (int t = 0; t < TN; ++t) b[c ^ 1][t] = bs[(k + 1) * LDB + t * 32];
            }
            if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int t = 0; t < TN; ++t)
#pragma unroll
                for (int v = 0; v < 32; ++v) acc[t][v] = add_rn(acc[t][v], p[t][v]);
#pragma unroll
            for (int t = 0; t < TN; ++t)
#pragma unroll
                for (int v = 0; v < 32; ++v) asm volatile("" : "+v"(acc[t][v]));
            if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
            __builtin_amdgcn_sched_group_barrier(0x008, TN, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1 + TN, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 32 * TN, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// The same scheme with v_mfma_f32_16x16x1_4b_f32: four 16x16 blocks of
// single products.  Lane l feeds row l of a 64-row strip (block l/16) and
// column l%16 of a 16-column block (the same column in all four blocks);
// register v of lane l then holds row 16*(v/4) + 4*((l%64)/16) + v%4 and
// column l%16.  Half the registers of the 32x32 shape per wave, so more
// waves fit on a SIMD.
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int mprod16_row(int v, int lane) {
    return 16 * (v >> 2) + 4 * (lane >> 4) + (v & 3);
}

template <int BK, int TN, int LDA, int LDB, bool PRIO>
__device__ __forceinline__ void mprod16_tile_steps(const float* as, const float* bs,
                                                   float (&acc)[TN][16]) {
    const f32x16 zero = {};
    float a[2], b[2][TN];
    a[0] = as[0];
#pragma unroll
    for (int t = 0; t < TN; ++t) b[0][t] = bs[t * 16];
#pragma unroll
    for (int k = 0; k < BK; ++k) {
        const int c = k & 1;
        f32x16 p[TN];
#pragma unroll
        for (int t = 0; t < TN; ++t)
            p[t] = __builtin_amdgcn_mfma_f32_16x16x1f32(a[c], b[c][t], zero, 0, 0, 0);
        if (k + 1 < BK) {
            a[c ^ 1] = as[(k + 1) * LDA];
#pragma unroll
            for (int t = 0; t < TN; ++t) b[c ^ 1][t] = bs[(k + 1) * LDB + t * 16];
        }
        if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int t = 0; t < TN; ++t)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[t][v] = add_rn(acc[t][v], p[t][v]);
#pragma unroll
        for (int t = 0; t < TN; ++t)
#pragma unroll
            for (int v = 0; v < 16; ++v) asm volatile("" : "+v"(acc[t][v]));
        if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_group_barrier(0x008, TN, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1 + TN, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 16 * TN, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int WAVES_M, int WAVES_N, int TN, int BK, int LA, int LB, bool PRIO>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void repops_mprod16_kernel(
    OperandView A, OperandView B, OutView C, int64_t M, int64_t N, int64_t K, TileGrid grid) {
    constexpr int NT = 64 * WAVES_M * WAVES_N;
    constexpr int BM = 64 * WAVES_M, BN = 16 * TN * WAVES_N;
    constexpr int LDA = BM + kPad, LDB = BN + kPad;

    __shared__ __attribute__((aligned(16))) float As[2][BK * LDA];
    __shared__ __attribute__((aligned(16))) float Bs[2][BK * LDB];

    const int tid = static_cast<int>(threadIdx.x);
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave % WAVES_M, wn = wave / WAVES_M;
    int tm, tn;
    tile_of_block(grid, tm, tn);
    select_batch(A, B, C);
    const int64_t m0 = static_cast<int64_t>(tm) * BM;
    const int64_t n0 = static_cast<int64_t>(tn) * BN;

    float acc[TN][16];
#pragma unroll
    for (int t = 0; t < TN; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[t][v] = 0.0f;  // s = +0

    TileStage<BM, BK, LA, NT> sa;
    TileStage<BN, BK, LB, NT> sb;
    sa.init(A, m0, tid);
    sb.init(B, n0, tid);
    const int64_t nfull = K / BK;
    const bool tail = (K % BK) != 0;
    const int arow = wm * 64 + lane;
    const int bcol = wn * 16 * TN + (lane & 15);
    const float* as0 = &As[0][arow];
    const float* bs0 = &Bs[0][bcol];
    const float* as1 = &As[1][arow];
    const float* bs1 = &Bs[1][bcol];

    if (nfull > 0) {
        sa.load_full();
        sb.load_full();
    } else {
        sa.load_tail(0, K, A.s_k);
        sb.load_tail(0, K, B.s_k);
    }
    sa.store(As[0], tid);
    sb.store(Bs[0], tid);
    __syncthreads();

    const int64_t ktiles = nfull + (tail ? 1 : 0);
    for (int64_t kt = 0; kt < ktiles; ++kt) {
        const bool more = kt + 1 < ktiles;
        if (kt + 1 < nfull) {
            sa.load_full();
            sb.load_full();
        } else if (more) {
            sa.load_tail(nfull * BK, K, A.s_k);
            sb.load_tail(nfull * BK, K, B.s_k);
        }
        asm volatile("" ::: "memory");
        const bool odd = (kt & 1) != 0;
        mprod16_tile_steps<BK, TN, LDA, LDB, PRIO>(odd ? as1 : as0, odd ? bs1 : bs0, acc);
        asm volatile("" ::: "memory");
        if (more) {
            sa.store(odd ? As[0] : As[1], tid);
            sb.store(odd ? Bs[0] : Bs[1], tid);
        }
        __syncthreads();
    }

#pragma unroll
    for (int t = 0; t < TN; ++t) {
        const int64_t j = n0 + wn * 16 * TN + t * 16 + (lane & 15);
        if (j >= N) continue;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int64_t i = m0 + wm * 64 + mprod16_row(v, lane);
            if (i < M) C.p[i * C.s_i + j * C.s_j] = epilogue_value(C, j, acc[t][v]);
        }
    }
}

template <int WAVES_M, int WAVES_N, int TN, int BK, int PIPE, int LA, int LB, bool PRIO>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void repops_mprod_kernel(
    OperandView A, OperandView B, OutView C, int64_t M, int64_t N, int64_t K, TileGrid grid) {
    constexpr int NT = 64 * WAVES_M * WAVES_N;
    constexpr int BM = 64 * WAVES_M, BN = 32 * TN * WAVES_N;
    constexpr int LDA = BM + kPad, LDB = BN + kPad;

    __shared__ __attribute__((aligned(16))) float As[2][BK * LDA];
    __shared__ __attribute__((aligned(16))) float Bs[2][BK * LDB];

    const int tid = static_cast<int>(threadIdx.x);
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave % WAVES_M, wn = wave / WAVES_M;
    int tm, tn;
    tile_of_block(grid, tm, tn);
    select_batch(A, B, C);
    const int64_t m0 = static_cast<int64_t>(tm) * BM;
    const int64_t n0 = static_cast<int64_t>(tn) * BN;

    float acc[TN][32];
#pragma unroll
    for (int t = 0; t < TN; ++t)
#pragma unroll
        for (int v = 0; v < 32; ++v) acc[t][v] = 0.0f;  // s = +0

    TileStage<BM, BK, LA, NT> sa;
    TileStage<BN, BK, LB, NT> sb;
    sa.init(A, m0, tid);
    sb.init(B, n0, tid);
    const int64_t nfull = K / BK;
    const bool tail = (K % BK) != 0;
    const int arow = wm * 64 + lane;
    const int bcol = wn * 32 * TN + (lane & 31);
    const float* as0 = &As[0][arow];
    const float* bs0 = &Bs[0][bcol];
    const float* as1 = &As[1][arow];
    const float* bs1 = &Bs[1][bcol];

    if (nfull > 0) {
        sa.load_full();
        sb.load_full();
    } else {
        sa.load_tail(0, K, A.s_k);
        sb.load_tail(0, K, B.s_k);
    }
    sa.store(As[0], tid);
    sb.store(Bs[0], tid);
    __syncthreads();

    const int64_t ktiles = nfull + (tail ? 1 : 0);
    for (int64_t kt = 0; kt < ktiles; ++kt) {
        const bool more = kt + 1 < ktiles;
        if (kt + 1 < nfull) {
            sa.load_full();
            sb.load_full();
        } else if (more) {
            sa.load_tail(nfull * BK, K, A.s_k);
            sb.load_tail(nfull * BK, K, B.s_k);
        }
        asm volatile("" ::: "memory");
        const bool odd = (kt & 1) != 0;
        mprod_tile_steps<BK, TN, LDA, LDB, PIPE, PRIO>(odd ? as1 : as0, odd ? bs1 : bs0, acc);
        asm volatile("" ::: "memory");
        if (more) {
            sa.store(odd ? As[0] : As[1], tid);
            sb.store(odd ? Bs[0] : Bs[1], tid);
        }
        __syncthreads();
    }

    // Epilogue: for each register v, lanes 0-31 and 32-63 each write 32
    // consecutive columns of one row, row i0 + r(v) with r(v) = mprod_row(v, 0)
    // (i0 holds the lane's 4-row shift).  With a bias, the sums become
    // RN(sum + bias[j]) in place first, so the one load is waited for before
    // any store (on gfx9 one counter tracks loads and stores: a wait placed
    // between stores would also wait for every store issued before it).  A
    // tile wholly inside M stores without row tests.
    const int64_t i0 = m0 + wm * 64 + 4 * (lane >> 5);
    const int64_t rows_left = M - i0;  // rows i0 + r exist for r < rows_left
    const bool full_m = m0 + BM <= M;
#pragma unroll
    for (int t = 0; t < TN; ++t) {
        const int64_t j = n0 + wn * 32 * TN + t * 32 + (lane & 31);
        if (j >= N) continue;
        if (C.bias) {
            const float b = C.bias[j * C.bias_s];
#pragma unroll
            for (int v = 0; v < 32; ++v) acc[t][v] = add_rn(acc[t][v], b);
        }
        float* const cp = C.p + i0 * C.s_i + j * C.s_j;
        if (full_m) {
#pragma unroll
            for (int v = 0; v < 32; ++v) cp[mprod_row(v, 0) * C.s_i] = acc[t][v];
        } else {
#pragma unroll
            for (int v = 0; v < 32; ++v) {
                const int r = mprod_row(v, 0);
                if (r < rows_left) cp[r * C.s_i] = acc[t][v];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// One lane per output, operands straight from global memory.  The plainest
// GPU form of the definition; every other variant must match it bit for bit.
__global__ __launch_bounds__(256) void repops_naive_kernel(OperandView A, OperandView B,
                                                          OutView C, int64_t M, int64_t N,
                                                          int64_t K, FastDiv blocks_n) {
    const uint32_t by = fdiv(blockIdx.x, blocks_n);
    const uint32_t bx = blockIdx.x - by * blocks_n.d;
    const int64_t i = static_cast<int64_t>(by) * 16 + threadIdx.x / 16;
    const int64_t j = static_cast<int64_t>(bx) * 16 + threadIdx.x % 16;
    if (i >= M || j >= N) return;
    select_batch(A, B, C);
    const float* a = A.p + i * A.s_x;
    const float* b = B.p + j * B.s_x;
    float s = 0.0f;
    for (int64_t k = 0; k < K; ++k) s = add_rn(s, mul_rn(a[k * A.s_k], b[k * B.s_k]));
    C.p[i * C.s_i + j * C.s_j] = epilogue_value(C, j, s);
}

// K == 0: every sum is empty, +0 (then the bias, if any, is added to it).
// Grid-stride over rows and columns (no integer division).
__global__ __launch_bounds__(256) void repops_fill_zero_kernel(OutView C, int64_t M, int64_t N) {
    const int64_t b = blockIdx.y;
    C.p += b * C.s_b;
    if (C.bias) C.bias += b * C.bias_sb;
    for (int64_t i = blockIdx.x; i < M; i += gridDim.x)
        for (int64_t j = threadIdx.x; j < N; j += 256)
            C.p[i * C.s_i + j * C.s_j] = epilogue_value(C, j, 0.0f);
}

// ---------------------------------------------------------------------------
using TiledFn = void (*)(OperandView, OperandView, OutView, int64_t, int64_t, int64_t, TileGrid);

template <int BM, int BN, int BK, int TM, int TN>
struct CfgTable {
    using Fn = TiledFn;
    template <int LA, int LB>
    static constexpr Fn fn() { return &repops_tiled_kernel<BM, BN, BK, TM, TN, LA, LB>; }
    static Fn get(int la, int lb) {
        static const Fn t[LAY_COUNT][LAY_COUNT] = {
            {fn<0, 0>(), fn<0, 1>(), fn<0, 2>()},
            {fn<1, 0>(), fn<1, 1>(), fn<1, 2>()},
            {fn<2, 0>(), fn<2, 1>(), fn<2, 2>()},
        };
        return t[la][lb];
    }
};

template <int WM, int WN, int TN, int BK, int PIPE, bool PRIO = false>
struct MprodTable {
    template <int LA, int LB>
    static constexpr TiledFn fn() { return &repops_mprod_kernel<WM, WN, TN, BK, PIPE, LA, LB, PRIO>; }
    static TiledFn get(int la, int lb) {
        static const TiledFn t[LAY_COUNT][LAY_COUNT] = {
            {fn<0, 0>(), fn<0, 1>(), fn<0, 2>()},
            {fn<1, 0>(), fn<1, 1>(), fn<1, 2>()},
            {fn<2, 0>(), fn<2, 1>(), fn<2, 2>()},
        };
        return t[la][lb];
    }
};

template <int WM, int WN, int TN, int BK, bool PRIO = false>
struct Mprod16Table {
    template <int LA, int LB>
    static constexpr TiledFn fn() { return &repops_mprod16_kernel<WM, WN, TN, BK, LA, LB, PRIO>; }
    static TiledFn get(int la, int lb) {
        static const TiledFn t[LAY_COUNT][LAY_COUNT] = {
            {fn<0, 0>(), fn<0, 1>(), fn<0, 2>()},
            {fn<1, 0>(), fn<1, 1>(), fn<1, 2>()},
            {fn<2, 0>(), fn<2, 1>(), fn<2, 2>()},
        };
        return t[la][lb];
    }
};

template <int R, int CN, int W, int BK, bool PRIO = false>
struct SrowTable {
    template <int LA, int LB>
    static constexpr TiledFn fn() { return &repops_srow_kernel<R, CN, W, BK, LA, LB, PRIO>; }
    static TiledFn get(int la, int lb) {
        static const TiledFn t[LAY_COUNT][LAY_COUNT] = {
            {fn<0, 0>(), fn<0, 1>(), fn<0, 2>()},
            {fn<1, 0>(), fn<1, 1>(), fn<1, 2>()},
            {fn<2, 0>(), fn<2, 1>(), fn<2, 2>()},
        };
        return t[la][lb];
    }
};

}  // namespace

FastDiv make_fastdiv(uint32_t d) {
    // floor(n / d) == (n * m) >> s for 0 <= n < 2^31 when s = 31 + ceil(log2 d)
    // and m = ceil(2^s / d): the error n*(m*d - 2^s)/(d*2^s) is below 1/d.
    uint32_t l = 0;
    while ((uint64_t(1) << l) < d) ++l;
    const uint32_t s = 31 + l;
    const uint64_t m = ((uint64_t(1) << s) + d - 1) / d;
    return FastDiv{d, static_cast<uint32_t>(m), s};
}

TileGrid make_tile_grid(int tiles_m, int tiles_n, int order) {
    TileGrid g{};
    g.tiles_m = tiles_m;
    g.tiles_n = tiles_n;
    g.order = order;
    g.div_n = make_fastdiv(static_cast<uint32_t>(tiles_n));
    g.div_m = make_fastdiv(static_cast<uint32_t>(tiles_m));
    g.div_span = make_fastdiv(8u * static_cast<uint32_t>(tiles_n));
    const uint32_t last = static_cast<uint32_t>(tiles_m) & 7u;
    g.div_last = make_fastdiv(last ? last : 8u);
    return g;
}

void tile_shape(int cfg, int* bm, int* bn) {
    switch (cfg) {
        case CFG_128x128: *bm = 128; *bn = 128; break;
        case CFG_64x64: *bm = 64; *bn = 64; break;
        case CFG_128x64: *bm = 128; *bn = 64; break;
        case CFG_64x128: *bm = 64; *bn = 128; break;
        case MCFG_128x128_W4: *bm = 128; *bn = 128; break;
        case MCFG_128x128_W8: *bm = 128; *bn = 128; break;
        case MCFG_256x128_W8: *bm = 256; *bn = 128; break;
        case MCFG_128x128_W8_P1: *bm = 128; *bn = 128; break;
        case MCFG_128x128_W8_P1_K32: *bm = 128; *bn = 128; break;
        case MCFG_128x128_W4_P1: *bm = 128; *bn = 128; break;
        case MCFG_256x128_W8_P1: *bm = 256; *bn = 128; break;
        case M16CFG_128x128_W16: *bm = 128; *bn = 128; break;
        case M16CFG_128x64_W8: *bm = 128; *bn = 64; break;
        case M16CFG_128x128_W8: *bm = 128; *bn = 128; break;
        case SCFG_R1C1_W4: *bm = 4; *bn = 64; break;
        case SCFG_R4C1_W4: *bm = 16; *bn = 64; break;
        case SCFG_R2C2_W4: *bm = 8; *bn = 128; break;
        case SCFG_R8C1_W4: *bm = 32; *bn = 64; break;
        case SCFG_R4C2_W8: *bm = 32; *bn = 128; break;
        case SCFG_R8C2_W8: *bm = 64; *bn = 128; break;
        default: *bm = 64; *bn = 64; break;  // MCFG_64x64_W2
    }
}

// Tiles beyond which a launch uses the raised-priority kernel forms: one per CU.
constexpr int64_t kPrioTiles = 256;

int launch_mprod(int cfg, int lay_a, int lay_b, OperandView A, OperandView B, OutView C,
                 int64_t M, int64_t N, int64_t K, int64_t batch, int order, void* stream) {
    int bm, bn;
    tile_shape(cfg, &bm, &bn);
    const int tiles_m = static_cast<int>((M + bm - 1) / bm);
    const int tiles_n = static_cast<int>((N + bn - 1) / bn);
    const dim3 grid(static_cast<unsigned>(tiles_m) * static_cast<unsigned>(tiles_n),
                    static_cast<unsigned>(batch));
    hipStream_t s = static_cast<hipStream_t>(stream);
    // With more tiles than CUs (several workgroups per CU), the kernels the
    // automatic choice uses raise their waves' priority while they issue a
    // step's adds (s_setprio 1), so that a wave that has its products goes
    // on to its next matrix instruction or scalar loads sooner.  With one
    // tile per CU or fewer the same hurt (measured), so it is off there.
    const bool prio = static_cast<int64_t>(tiles_m) * tiles_n * batch > kPrioTiles;
    TiledFn fn;
    int threads;
    switch (cfg) {
        case MCFG_128x128_W4: fn = MprodTable<2, 2, 2, 16, 2>::get(lay_a, lay_b); threads = 256; break;
        case MCFG_128x128_W8: fn = MprodTable<2, 4, 1, 16, 2>::get(lay_a, lay_b); threads = 512; break;
        case MCFG_256x128_W8: fn = MprodTable<4, 2, 2, 16, 2>::get(lay_a, lay_b); threads = 512; break;
        case MCFG_128x128_W8_P1: fn = MprodTable<2, 4, 1, 16, 1>::get(lay_a, lay_b); threads = 512; break;
        case MCFG_128x128_W8_P1_K32:
            fn = prio ? MprodTable<2, 4, 1, 32, 1, true>::get(lay_a, lay_b)
                      : MprodTable<2, 4, 1, 32, 1>::get(lay_a, lay_b);
            threads = 512;
            break;
        case MCFG_128x128_W4_P1: fn = MprodTable<2, 2, 2, 16, 1>::get(lay_a, lay_b); threads = 256; break;
        case MCFG_256x128_W8_P1: fn = MprodTable<4, 2, 2, 16, 1>::get(lay_a, lay_b); threads = 512; break;
        case M16CFG_128x128_W16: fn = Mprod16Table<2, 8, 1, 32>::get(lay_a, lay_b); threads = 1024; break;
        case M16CFG_128x64_W8:
            fn = prio ? Mprod16Table<2, 4, 1, 32, true>::get(lay_a, lay_b)
                      : Mprod16Table<2, 4, 1, 32>::get(lay_a, lay_b);
            threads = 512;
            break;
        case M16CFG_128x128_W8: fn = Mprod16Table<2, 4, 2, 16>::get(lay_a, lay_b); threads = 512; break;
        default: fn = MprodTable<1, 2, 1, 16, 2>::get(lay_a, lay_b); threads = 128; break;
    }
    hipLaunchKernelGGL(fn, grid, dim3(threads), 0, s, A, B, C, M, N, K,
                       make_tile_grid(tiles_m, tiles_n, order));
    return static_cast<int>(hipGetLastError());
}

int launch_srow(int cfg, int lay_a, int lay_b, OperandView A, OperandView B, OutView C,
                int64_t M, int64_t N, int64_t K, int64_t batch, int order, void* stream) {
    int bm, bn;
    tile_shape(cfg, &bm, &bn);
    const int tiles_m = static_cast<int>((M + bm - 1) / bm);
    const int tiles_n = static_cast<int>((N + bn - 1) / bn);
    const dim3 grid(static_cast<unsigned>(tiles_m) * static_cast<unsigned>(tiles_n),
                    static_cast<unsigned>(batch));
    hipStream_t s = static_cast<hipStream_t>(stream);
    // Wave priority around the arithmetic, as in launch_mprod.
    const bool prio = static_cast<int64_t>(tiles_m) * tiles_n * batch > kPrioTiles;
    TiledFn fn;
    int threads;
    switch (cfg) {
        case SCFG_R1C1_W4: fn = SrowTable<1, 1, 4, 32>::get(lay_a, lay_b); threads = 256; break;
        case SCFG_R2C2_W4: fn = SrowTable<2, 2, 4, 32>::get(lay_a, lay_b); threads = 256; break;
        case SCFG_R8C1_W4: fn = SrowTable<8, 1, 4, 32>::get(lay_a, lay_b); threads = 256; break;
        case SCFG_R4C2_W8:
            fn = prio ? SrowTable<4, 2, 8, 32, true>::get(lay_a, lay_b)
                      : SrowTable<4, 2, 8, 32>::get(lay_a, lay_b);
            threads = 512;
            break;
        case SCFG_R8C2_W8: fn = SrowTable<8, 2, 8, 32>::get(lay_a, lay_b); threads = 512; break;
        default:  // SCFG_R4C1_W4
            fn = prio ? SrowTable<4, 1, 4, 32, true>::get(lay_a, lay_b)
                      : SrowTable<4, 1, 4, 32>::get(lay_a, lay_b);
            threads = 256;
            break;
    }
    hipLaunchKernelGGL(fn, grid, dim3(threads), 0, s, A, B, C, M, N, K,
                       make_tile_grid(tiles_m, tiles_n, order));
    return static_cast<int>(hipGetLastError());
}

int launch_tiled(int cfg, int lay_a, int lay_b, OperandView A, OperandView B, OutView C,
                 int64_t M, int64_t N, int64_t K, int64_t batch, int order, void* stream) {
    int bm, bn;
    tile_shape(cfg, &bm, &bn);
    const int tiles_m = static_cast<int>((M + bm - 1) / bm);
    const int tiles_n = static_cast<int>((N + bn - 1) / bn);
    const dim3 grid(static_cast<unsigned>(tiles_m) * static_cast<unsigned>(tiles_n),
                    static_cast<unsigned>(batch));
    const dim3 block(kThreads);
    hipStream_t s = static_cast<hipStream_t>(stream);
    TiledFn fn;
    switch (cfg) {
        case CFG_128x128: fn = CfgTable<128, 128, 16, 8, 8>::get(lay_a, lay_b); break;
        case CFG_64x64: fn = CfgTable<64, 64, 16, 4, 4>::get(lay_a, lay_b); break;
        case CFG_128x64: fn = CfgTable<128, 64, 16, 8, 4>::get(lay_a, lay_b); break;
        default: fn = CfgTable<64, 128, 16, 4, 8>::get(lay_a, lay_b); break;
    }
    hipLaunchKernelGGL(fn, grid, block, 0, s, A, B, C, M, N, K,
                       make_tile_grid(tiles_m, tiles_n, order));
    return static_cast<int>(hipGetLastError());
}

int launch_naive(OperandView A, OperandView B, OutView C, int64_t M, int64_t N, int64_t K,
                 int64_t batch, void* stream) {
    const int blocks_n = static_cast<int>((N + 15) / 16);
    const int blocks_m = static_cast<int>((M + 15) / 16);
    hipLaunchKernelGGL(repops_naive_kernel,
                       dim3(static_cast<unsigned>(blocks_m) * static_cast<unsigned>(blocks_n),
                            static_cast<unsigned>(batch)),
                       dim3(256), 0, static_cast<hipStream_t>(stream), A, B, C, M, N, K,
                       make_fastdiv(static_cast<uint32_t>(blocks_n)));
    return static_cast<int>(hipGetLastError());
}

int launch_fill_zero(OutView C, int64_t M, int64_t N, int64_t batch, void* stream) {
    const unsigned blocks = static_cast<unsigned>(M < 65536 ? M : 65536);
    hipLaunchKernelGGL(repops_fill_zero_kernel, dim3(blocks, static_cast<unsigned>(batch)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), C, M, N);
    return static_cast<int>(hipGetLastError());
}

}  // namespace repops
