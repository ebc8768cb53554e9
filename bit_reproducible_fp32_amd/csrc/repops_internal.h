// Internal interface between the C-ABI front end (repops_api.cpp) and the
// gfx950 kernels (repops_kernels.hip).  Not installed, not part of the ABI.
#pragma once

#include <stdint.h>

namespace repops {

// One operand seen as an X x K matrix: element (x, k) of batch b is
// p[b*s_b + x*s_x + k*s_k].  For A, x is the output row i; for B, x is the
// output column j.  Both operands therefore share one loader and one LDS
// layout.
struct OperandView {
    const float* p;
    int64_t s_x;
    int64_t s_k;
    int64_t X;
    int64_t s_b;
};

// Output: element (i, j) of batch b is p[b*s_b + i*s_i + j*s_j].  With a
// bias, the stored value is RN(sum + bias[b*bias_sb + j*bias_s]).
struct OutView {
    float* p;
    int64_t s_i;
    int64_t s_j;
    int64_t s_b;
    const float* bias;  // nullptr: no bias
    int64_t bias_s;
    int64_t bias_sb;
};

// How an operand tile is fetched from global memory.
enum Layout : int {
    LAY_KC = 0,   // s_k == 1, 16-byte aligned rows: float4 loads along k
    LAY_XC = 1,   // s_x == 1, 16-byte aligned columns: float4 loads along x
    LAY_GEN = 2,  // anything else: one element per load
    LAY_COUNT = 3
};

// Tile shapes of the register-blocked VALU kernel.
enum TileCfg : int {
    CFG_128x128 = 0,  // BM=128 BN=128 BK=16, 8x8 outputs per lane
    CFG_64x64 = 1,    // BM=64  BN=64  BK=16, 4x4 outputs per lane
    CFG_128x64 = 2,   // BM=128 BN=64  BK=16, 8x4 outputs per lane
    CFG_64x128 = 3,   // BM=64  BN=128 BK=16, 4x8 outputs per lane
    // Matrix-core-product kernels (products on the matrix core, sums on the
    // VALU): tile, waves per workgroup.
    MCFG_128x128_W4 = 4,  // 2x2 waves, each 64 rows x 2 blocks of 32 columns
    MCFG_128x128_W8 = 5,  // 2x4 waves, each 64 rows x 32 columns
    MCFG_256x128_W8 = 6,  // 4x2 waves, each 64 rows x 2 blocks of 32 columns
    MCFG_64x64_W2 = 7,    // 1x2 waves, each 64 rows x 32 columns
    // The same with one product buffer per wave (fewer registers, more waves).
    MCFG_128x128_W8_P1 = 8,
    MCFG_128x128_W4_P1 = 9,
    MCFG_256x128_W8_P1 = 10,
    // 16x16x1 four-block shape: waves of 64 rows x 16*TN columns.
    M16CFG_128x128_W16 = 11,  // 2x8 waves, TN=1 (1024 lanes), BK=32
    M16CFG_128x64_W8 = 12,    // 2x4 waves, TN=1, BK=32
    M16CFG_128x128_W8 = 13,   // 2x4 waves, TN=2
    // Scalar-row kernels (each wave's A values wave-uniform in SGPRs, products
    // and sums on the VALU): rows per wave R, 64-column groups per lane C,
    // waves W; 32-deep k-tiles.
    SCFG_R1C1_W4 = 14,  // 4 x 64 tile
    SCFG_R4C1_W4 = 15,  // 16 x 64
    SCFG_R2C2_W4 = 16,  // 8 x 128
    SCFG_R8C1_W4 = 17,  // 32 x 64
    SCFG_R4C2_W8 = 18,  // 32 x 128
    SCFG_R8C2_W8 = 19,  // 64 x 128
    // MCFG_128x128_W8_P1 with 32-deep k-tiles: a row stored along k gives
    // whole 128-byte lines per k-tile (67.6 KB of LDS, two workgroups per CU).
    MCFG_128x128_W8_P1_K32 = 20,
};

// Workgroup -> output-tile traversal orders (never change a bit).
enum TileOrder : int {
    ORDER_ROW = 0,       // tile rows outer, tile columns inner
    ORDER_COL = 1,       // tile columns outer, tile rows inner
    ORDER_XCD_GROUP = 2  // contiguous tile ranges per XCD, grouped by 8 tile rows
};

// Integer division by a runtime divisor as a multiply and shift:
// floor(n / d) == (n * m) >> s for 0 <= n < 2^31 (see make_fastdiv).
struct FastDiv {
    uint32_t d, m, s;
};

// Tile grid of one launch: tile counts, traversal order and the divisors the
// workgroup -> tile mapping needs.
struct TileGrid {
    int tiles_m, tiles_n, order;
    FastDiv div_n, div_m, div_span, div_last;
};

FastDiv make_fastdiv(uint32_t d);
TileGrid make_tile_grid(int tiles_m, int tiles_n, int order);
void tile_shape(int cfg, int* bm, int* bn);

// Each returns a hipError_t value (0 on success) from the launch.  `batch`
// (1..kMaxBatchPerLaunch) is the grid's second dimension; each batch index
// offsets A, B, C and the bias by their batch strides.
constexpr int64_t kMaxBatchPerLaunch = 65535;
int launch_tiled(int cfg, int lay_a, int lay_b, OperandView A, OperandView B, OutView C,
                 int64_t M, int64_t N, int64_t K, int64_t batch, int order, void* stream);
int launch_mprod(int cfg, int lay_a, int lay_b, OperandView A, OperandView B, OutView C,
                 int64_t M, int64_t N, int64_t K, int64_t batch, int order, void* stream);
int launch_srow(int cfg, int lay_a, int lay_b, OperandView A, OperandView B, OutView C,
                int64_t M, int64_t N, int64_t K, int64_t batch, int order, void* stream);
int launch_naive(OperandView A, OperandView B, OutView C, int64_t M, int64_t N, int64_t K,
                 int64_t batch, void* stream);
int launch_fill_zero(OutView C, int64_t M, int64_t N, int64_t batch, void* stream);

// Fixed-order gradient fold: the contributors one pass reads, in fold order.
constexpr int kFoldMax = 64;
struct FoldArgs {
    const float* g[kFoldMax];
};

// One pass of the fold over n <= kFoldMax contributors (see repops_fold.hip).
int launch_fold(const FoldArgs& G, int n, bool first, bool last, float* sum, float* theta,
                float* gbar, float inv_k, float eta, int64_t d, bool vec, void* stream);

// Tensor hash (repops_merkle.hip): SHA-256 Merkle root of total_words 32-bit
// words cut into leaves of leaf_words.  The root is written as the digest's
// 32 bytes; `ws` holds merkle_workspace_bytes(n_leaves, leaf_words) bytes.
// vec: data is 16-byte aligned and leaf_words is a multiple of 4.
int64_t merkle_workspace_bytes(int64_t n_leaves, int64_t leaf_words);
int launch_merkle_root(const uint32_t* data, int64_t total_words, int64_t leaf_words, void* ws,
                       uint32_t* root, bool vec, void* stream);
// Size of the static device scratch behind repops_merkle_root_noalloc, and
// the current device's address of it (nullptr, with the HIP error in
// *hip_error, when the lookup fails).
constexpr int64_t kStaticScratchBytes = int64_t(16) << 20;
void* static_scratch_device_ptr(int* hip_error);
// match[c] = (claims[8c .. 8c+7] == root[0 .. 7]) for c < nclaims.
int launch_merkle_match(const uint32_t* root, const uint32_t* claims, int64_t nclaims,
                        int32_t* match, void* stream);

// ERF (op 0) and GeLU (op 1) over n floats; LayerNorm over rows of H
// (repops_ops.hip).  vec: every pointer 16-byte aligned (and, for LayerNorm,
// the row strides and H multiples of 4).
int launch_unary(int op, const float* x, float* y, int64_t n, bool vec, void* stream);
int launch_layernorm(const float* x, int64_t x_rs, const float* gamma, const float* beta, float* y,
                     int64_t y_rs, int64_t rows, int64_t H, float eps, float* mean, float* rstd,
                     bool vec, void* stream);

}  // namespace repops
