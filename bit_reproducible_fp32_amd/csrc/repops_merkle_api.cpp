// C-ABI front end of the tensor hash and the referee's re-execution of a
// disputed matmul (Verde and RepOps article, sections 2.3 and 2.4, case 3).
// Host C++; the kernels are in repops_merkle.hip.
#include <stdint.h>

#include "../../include/repops.h"
#include "repops_internal.h"

using namespace repops;

namespace {

constexpr int64_t kMaxLeafBytes = int64_t(1) << 24;
constexpr int64_t kMaxBytes = int64_t(1) << 50;
constexpr int64_t kGroupLeaves = 256;
constexpr int64_t kMaxBlocks = 0x7fffffff;

bool sizes_ok(int64_t nbytes, int64_t leaf_bytes) {
    if (nbytes < 0 || nbytes > kMaxBytes || (nbytes & 3) != 0) return false;
    if (leaf_bytes < 4 || leaf_bytes > kMaxLeafBytes || (leaf_bytes & 3) != 0) return false;
    const int64_t n_leaves = (nbytes + leaf_bytes - 1) / leaf_bytes;
    return (n_leaves + kGroupLeaves - 1) / kGroupLeaves <= kMaxBlocks;
}

int64_t workspace_for(int64_t nbytes, int64_t leaf_bytes) {
    if (nbytes == 0) return 0;
    return merkle_workspace_bytes((nbytes + leaf_bytes - 1) / leaf_bytes, leaf_bytes / 4);
}

bool span_overlap(const void* p, int64_t np, const void* q, int64_t nq) {
    if (p == nullptr || q == nullptr || np <= 0 || nq <= 0) return false;
    const uintptr_t p0 = reinterpret_cast<uintptr_t>(p), q0 = reinterpret_cast<uintptr_t>(q);
    return p0 < q0 + static_cast<uintptr_t>(nq) && q0 < p0 + static_cast<uintptr_t>(np);
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Everything repops_merkle_root checks, shared with the referee call.
repops_status check_merkle(const void* data, int64_t nbytes, int64_t leaf_bytes,
                           const void* workspace, int64_t workspace_bytes, const void* root) {
    if (!sizes_ok(nbytes, leaf_bytes)) return REPOPS_ERR_DIM;
    if (root == nullptr || (nbytes > 0 && data == nullptr)) return REPOPS_ERR_NULL;
    if (!aligned(root, 4) || (nbytes > 0 && !aligned(data, 4))) return REPOPS_ERR_ALIGN;
    const int64_t need = workspace_for(nbytes, leaf_bytes);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return REPOPS_ERR_WORKSPACE;
    if (need > 0 && !aligned(workspace, 16)) return REPOPS_ERR_ALIGN;
    if (span_overlap(root, 32, data, nbytes) || span_overlap(workspace, need, data, nbytes) ||
        span_overlap(root, 32, workspace, need))
        return REPOPS_ERR_ALIAS;
    return REPOPS_OK;
}

repops_status launch_root(const void* data, int64_t nbytes, int64_t leaf_bytes, void* workspace,
                          void* root, void* stream) {
    const bool vec = aligned(data, 16) && (leaf_bytes & 15) == 0;
    const int err = launch_merkle_root(static_cast<const uint32_t*>(data), nbytes / 4,
                                       leaf_bytes / 4, workspace, static_cast<uint32_t*>(root), vec,
                                       stream);
    return err == 0 ? REPOPS_OK : REPOPS_ERR_HIP;
}

}  // namespace

extern "C" {

int64_t repops_merkle_workspace_bytes(int64_t nbytes, int64_t leaf_bytes) {
    if (!sizes_ok(nbytes, leaf_bytes)) return -1;
    return workspace_for(nbytes, leaf_bytes);
}

repops_status repops_merkle_root(const void* data, int64_t nbytes, int64_t leaf_bytes,
                                 void* workspace, int64_t workspace_bytes, void* root,
                                 void* stream) {
    const repops_status st = check_merkle(data, nbytes, leaf_bytes, workspace, workspace_bytes, root);
    if (st != REPOPS_OK) return st;
    return launch_root(data, nbytes, leaf_bytes, workspace, root, stream);
}

repops_status repops_merkle_root_noalloc(const void* data, int64_t nbytes, int64_t leaf_bytes,
                                         void* root, void* stream) {
    static_assert(REPOPS_NOALLOC_SCRATCH_BYTES == kStaticScratchBytes, "one scratch size");
    if (!sizes_ok(nbytes, leaf_bytes)) return REPOPS_ERR_DIM;
    const int64_t need = workspace_for(nbytes, leaf_bytes);
    if (need > kStaticScratchBytes) return REPOPS_ERR_SCRATCH;
    void* ws = nullptr;
    if (need > 0) {
        int err = 0;
        ws = static_scratch_device_ptr(&err);
        if (ws == nullptr) return REPOPS_ERR_HIP;
    }
    const repops_status st = check_merkle(data, nbytes, leaf_bytes, ws, need, root);
    if (st != REPOPS_OK) return st;
    return launch_root(data, nbytes, leaf_bytes, ws, root, stream);
}

repops_status repops_referee_matmul_f32(const float* A, int64_t a_rs, int64_t a_cs, const float* B,
                                        int64_t b_rs, int64_t b_cs, float* C, int64_t M, int64_t N,
                                        int64_t K, int trans_a, int trans_b, int64_t leaf_bytes,
                                        void* workspace, int64_t workspace_bytes,
                                        const void* claims, int64_t nclaims, void* root,
                                        int32_t* match, void* stream) {
    repops_status st = repops_check_args_f32(A, a_rs, a_cs, B, b_rs, b_cs, C, N, 1, M, N, K,
                                             trans_a, trans_b, -1);
    if (st != REPOPS_OK) return st;
    if (M > 0 && N > kMaxBytes / 4 / M) return REPOPS_ERR_DIM;
    const int64_t nbytes = M * N * 4;
    st = check_merkle(C, nbytes, leaf_bytes, workspace, workspace_bytes, root);
    if (st != REPOPS_OK) return st;
    if (nclaims < 0 || nclaims > (int64_t(1) << 40)) return REPOPS_ERR_DIM;
    if (nclaims > 0) {
        if (claims == nullptr || match == nullptr) return REPOPS_ERR_NULL;
        if (!aligned(claims, 4) || !aligned(match, 4)) return REPOPS_ERR_ALIGN;
        const int64_t need = workspace_for(nbytes, leaf_bytes);
        const int64_t cb = nclaims * 32, mb = nclaims * 4;
        if (span_overlap(match, mb, C, nbytes) || span_overlap(match, mb, workspace, need) ||
            span_overlap(match, mb, root, 32) || span_overlap(match, mb, claims, cb) ||
            span_overlap(root, 32, claims, cb) || span_overlap(claims, cb, C, nbytes) ||
            span_overlap(claims, cb, workspace, need))
            return REPOPS_ERR_ALIAS;
    }
    st = repops_matmul_f32(A, a_rs, a_cs, B, b_rs, b_cs, C, N, 1, M, N, K, trans_a, trans_b,
                           stream);
    if (st != REPOPS_OK) return st;
    st = launch_root(C, nbytes, leaf_bytes, workspace, root, stream);
    if (st != REPOPS_OK) return st;
    const int err = launch_merkle_match(static_cast<const uint32_t*>(root),
                                        static_cast<const uint32_t*>(claims), nclaims, match, stream);
    return err == 0 ? REPOPS_OK : REPOPS_ERR_HIP;
}

}  // extern "C"
