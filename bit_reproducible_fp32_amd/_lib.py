"""ctypes binding of librepops.so: argument marshalling only.

Every entry point of ``include/repops.h`` is exposed under the same name;
all computation happens in the library's gfx950 kernels.  If the library has
not been built, loading raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librepops.so")

REPOPS_OK = 0
REPOPS_ERR_NULL = 1
REPOPS_ERR_DIM = 2
REPOPS_ERR_STRIDE = 3
REPOPS_ERR_ALIAS = 4
REPOPS_ERR_VARIANT = 5
REPOPS_ERR_HIP = 6
REPOPS_ERR_DUPLICATE = 7
REPOPS_ERR_ALIGN = 8
REPOPS_ERR_WORKSPACE = 9
REPOPS_ERR_SCRATCH = 10
REPOPS_NOALLOC_SCRATCH_BYTES = 16 * 1024 * 1024
REPOPS_FOLD_MAX_PER_PASS = 64
REPOPS_MERKLE_DEFAULT_LEAF_BYTES = 1024

EXPORTS = (
    "repops_matmul_f32",
    "repops_matmul_f32_ex",
    "repops_matmul_batched_f32",
    "repops_check_args_f32",
    "repops_pick_variant_f32",
    "repops_variant_count",
    "repops_variant_name",
    "repops_strerror",
    "repops_build_manifest",
    "repops_canonical_order",
    "repops_fold_mean_sgd_f32",
    "repops_merkle_workspace_bytes",
    "repops_merkle_root",
    "repops_merkle_root_noalloc",
    "repops_referee_matmul_f32",
    "repops_erf_f32",
    "repops_gelu_f32",
    "repops_layernorm_f32",
)

_lib = None


class RepopsError(RuntimeError):
    def __init__(self, status: int, where: str = ""):
        self.status = status
        msg = "%s: %s (status %d)" % (where or "repops", strerror(status), status)
        super().__init__(msg)


def load():
    """The loaded library (raises OSError if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise OSError("librepops.so is not built (expected at %s); run "
                      "bit_reproducible_fp32_amd.build.build()" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    i64, vp, ci, cp = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_char_p
    mm = [vp, i64, i64, vp, i64, i64, vp, i64, i64, i64, i64, i64, ci, ci]
    lib.repops_matmul_f32.argtypes = mm + [vp]
    lib.repops_matmul_f32.restype = ci
    lib.repops_matmul_f32_ex.argtypes = mm + [vp, ci]
    lib.repops_matmul_f32_ex.restype = ci
    lib.repops_matmul_batched_f32.argtypes = [vp, i64, i64, i64, vp, i64, i64, i64, vp, i64, i64,
                                              i64, i64, i64, i64, i64, ci, ci, vp, i64, i64,
                                              vp, ci]
    lib.repops_matmul_batched_f32.restype = ci
    lib.repops_check_args_f32.argtypes = mm + [ci]
    lib.repops_check_args_f32.restype = ci
    lib.repops_pick_variant_f32.argtypes = [vp, i64, i64, vp, i64, i64, i64, i64, i64, ci, ci]
    lib.repops_pick_variant_f32.restype = ci
    lib.repops_variant_count.argtypes = []
    lib.repops_variant_count.restype = ci
    lib.repops_variant_name.argtypes = [ci]
    lib.repops_variant_name.restype = cp
    lib.repops_strerror.argtypes = [ci]
    lib.repops_strerror.restype = cp
    lib.repops_build_manifest.argtypes = []
    lib.repops_build_manifest.restype = cp
    lib.repops_canonical_order.argtypes = [vp, vp, i64, vp]
    lib.repops_canonical_order.restype = ci
    lib.repops_fold_mean_sgd_f32.argtypes = [vp, i64, i64, ctypes.c_float, vp, vp, vp]
    lib.repops_fold_mean_sgd_f32.restype = ci
    lib.repops_merkle_workspace_bytes.argtypes = [i64, i64]
    lib.repops_merkle_workspace_bytes.restype = i64
    lib.repops_merkle_root.argtypes = [vp, i64, i64, vp, i64, vp, vp]
    lib.repops_merkle_root.restype = ci
    lib.repops_merkle_root_noalloc.argtypes = [vp, i64, i64, vp, vp]
    lib.repops_merkle_root_noalloc.restype = ci
    lib.repops_referee_matmul_f32.argtypes = [vp, i64, i64, vp, i64, i64, vp, i64, i64, i64, ci,
                                              ci, i64, vp, i64, vp, i64, vp, vp, vp]
    lib.repops_referee_matmul_f32.restype = ci
    for name in ("repops_erf_f32", "repops_gelu_f32"):
        getattr(lib, name).argtypes = [vp, vp, i64, vp]
        getattr(lib, name).restype = ci
    lib.repops_layernorm_f32.argtypes = [vp, i64, vp, vp, vp, i64, i64, i64, ctypes.c_float, vp,
                                         vp, vp]
    lib.repops_layernorm_f32.restype = ci
    _lib = lib
    return lib


# ---- the C ABI, name for name (pointers and streams are Python ints) -------
def repops_matmul_f32(A, a_rs, a_cs, B, b_rs, b_cs, C, c_rs, c_cs, M, N, K, trans_a, trans_b,
                      stream) -> int:
    return load().repops_matmul_f32(A, a_rs, a_cs, B, b_rs, b_cs, C, c_rs, c_cs, M, N, K,
                                    int(trans_a), int(trans_b), stream)


def repops_matmul_f32_ex(A, a_rs, a_cs, B, b_rs, b_cs, C, c_rs, c_cs, M, N, K, trans_a, trans_b,
                         stream, variant) -> int:
    return load().repops_matmul_f32_ex(A, a_rs, a_cs, B, b_rs, b_cs, C, c_rs, c_cs, M, N, K,
                                       int(trans_a), int(trans_b), stream, int(variant))


def repops_matmul_batched_f32(A, a_bs, a_rs, a_cs, B, b_bs, b_rs, b_cs, C, c_bs, c_rs, c_cs, M,
                              N, K, batch, trans_a, trans_b, bias, bias_bs, bias_s, stream,
                              variant=-1) -> int:
    return load().repops_matmul_batched_f32(A, a_bs, a_rs, a_cs, B, b_bs, b_rs, b_cs, C, c_bs,
                                            c_rs, c_cs, M, N, K, batch, int(trans_a),
                                            int(trans_b), bias, bias_bs, bias_s, stream,
                                            int(variant))


def repops_check_args_f32(A, a_rs, a_cs, B, b_rs, b_cs, C, c_rs, c_cs, M, N, K, trans_a, trans_b,
                          variant=-1) -> int:
    return load().repops_check_args_f32(A, a_rs, a_cs, B, b_rs, b_cs, C, c_rs, c_cs, M, N, K,
                                        int(trans_a), int(trans_b), int(variant))


def repops_pick_variant_f32(A, a_rs, a_cs, B, b_rs, b_cs, M, N, K, trans_a, trans_b) -> int:
    return load().repops_pick_variant_f32(A, a_rs, a_cs, B, b_rs, b_cs, M, N, K, int(trans_a),
                                          int(trans_b))


def repops_variant_count() -> int:
    return load().repops_variant_count()


def repops_variant_name(variant: int) -> str:
    return load().repops_variant_name(int(variant)).decode()


def repops_strerror(status: int) -> str:
    return load().repops_strerror(int(status)).decode()


def repops_build_manifest() -> str:
    return load().repops_build_manifest().decode()


def repops_canonical_order(dids):
    """(status, order): order[r] is the index of the contributor at rank r
    in byte-lexicographic order of the identities (bytes objects)."""
    k = len(dids)
    bufs = [bytes(x) for x in dids]
    ptrs = (ctypes.c_char_p * max(k, 1))(*bufs)
    lens = (ctypes.c_int64 * max(k, 1))(*[len(b) for b in bufs])
    out = (ctypes.c_int64 * max(k, 1))()
    st = load().repops_canonical_order(ctypes.cast(ptrs, ctypes.c_void_p),
                                       ctypes.cast(lens, ctypes.c_void_p), k,
                                       ctypes.cast(out, ctypes.c_void_p))
    return st, [int(out[r]) for r in range(k)]


def repops_fold_mean_sgd_f32(grads, k, d, eta, theta, gbar, stream) -> int:
    """grads: sequence of k device addresses (ints), in fold order."""
    arr = (ctypes.c_void_p * max(int(k), 1))(*[int(g) for g in grads])
    return load().repops_fold_mean_sgd_f32(ctypes.cast(arr, ctypes.c_void_p), int(k), int(d),
                                           float(eta), theta, gbar, stream)


def repops_merkle_workspace_bytes(nbytes, leaf_bytes) -> int:
    return load().repops_merkle_workspace_bytes(int(nbytes), int(leaf_bytes))


def repops_merkle_root(data, nbytes, leaf_bytes, workspace, workspace_bytes, root, stream) -> int:
    return load().repops_merkle_root(data, int(nbytes), int(leaf_bytes), workspace,
                                     int(workspace_bytes), root, stream)


def repops_merkle_root_noalloc(data, nbytes, leaf_bytes, root, stream) -> int:
    return load().repops_merkle_root_noalloc(data, int(nbytes), int(leaf_bytes), root, stream)


def repops_referee_matmul_f32(A, a_rs, a_cs, B, b_rs, b_cs, C, M, N, K, trans_a, trans_b,
                              leaf_bytes, workspace, workspace_bytes, claims, nclaims, root, match,
                              stream) -> int:
    return load().repops_referee_matmul_f32(A, a_rs, a_cs, B, b_rs, b_cs, C, M, N, K,
                                            int(trans_a), int(trans_b), int(leaf_bytes),
                                            workspace, int(workspace_bytes), claims, int(nclaims),
                                            root, match, stream)


def repops_erf_f32(x, y, n, stream) -> int:
    return load().repops_erf_f32(x, y, int(n), stream)


def repops_gelu_f32(x, y, n, stream) -> int:
    return load().repops_gelu_f32(x, y, int(n), stream)


def repops_layernorm_f32(x, x_rs, gamma, beta, y, y_rs, rows, H, eps, mean, rstd, stream) -> int:
    return load().repops_layernorm_f32(x, int(x_rs), gamma, beta, y, int(y_rs), int(rows), int(H),
                                       float(eps), mean, rstd, stream)


strerror = repops_strerror


def variant_names():
    return [repops_variant_name(v) for v in range(repops_variant_count())]
