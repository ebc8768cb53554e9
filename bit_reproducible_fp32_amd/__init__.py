"""Reproducible fixed-order FP32 matrix multiply for AMD MI355X (gfx950).

``matmul(a, b)`` computes C = op(a) op(b) where every output element is
s = +0; for k ascending: s = RN(s + RN(a_ik * b_kj)) -- the matrix
multiplication of the RepOps operator library (Verde and RepOps article,
section 3.2, item 2), with the multiply and the add rounded separately.  The
bits of C do not depend on the kernel variant, launch shape, transposes or
strides.

The arithmetic runs in the HIP kernels of ``librepops.so`` behind the C ABI
declared in ``include/repops.h``; this package only marshals arguments (torch
supplies device memory and the stream).  Without the built library every
call raises -- there is no CPU path.
"""
from __future__ import annotations

from ._lib import (  # noqa: F401
    EXPORTS,
    REPOPS_ERR_ALIAS,
    REPOPS_ERR_ALIGN,
    REPOPS_ERR_DIM,
    REPOPS_ERR_DUPLICATE,
    REPOPS_FOLD_MAX_PER_PASS,
    REPOPS_ERR_HIP,
    REPOPS_ERR_NULL,
    REPOPS_ERR_STRIDE,
    REPOPS_ERR_VARIANT,
    REPOPS_ERR_SCRATCH,
    REPOPS_ERR_WORKSPACE,
    REPOPS_MERKLE_DEFAULT_LEAF_BYTES,
    REPOPS_NOALLOC_SCRATCH_BYTES,
    REPOPS_OK,
    RepopsError,
    load,
    repops_build_manifest,
    repops_canonical_order,
    repops_check_args_f32,
    repops_erf_f32,
    repops_fold_mean_sgd_f32,
    repops_gelu_f32,
    repops_layernorm_f32,
    repops_matmul_batched_f32,
    repops_matmul_f32,
    repops_matmul_f32_ex,
    repops_merkle_root,
    repops_merkle_root_noalloc,
    repops_merkle_workspace_bytes,
    repops_pick_variant_f32,
    repops_referee_matmul_f32,
    repops_strerror,
    repops_variant_count,
    repops_variant_name,
    variant_names,
)


def _logical(a, b, trans_a, trans_b):
    M, K = (a.shape[1], a.shape[0]) if trans_a else (a.shape[0], a.shape[1])
    K2, N = (b.shape[1], b.shape[0]) if trans_b else (b.shape[0], b.shape[1])
    if K != K2:
        raise ValueError("inner dimensions differ: op(a) is %dx%d, op(b) is %dx%d" % (M, K, K2, N))
    return M, N, K


def matmul(a, b, *, trans_a: bool = False, trans_b: bool = False, out=None, variant=None,
           stream=None):
    """C = op(a) @ op(b) on the GPU, bit-reproducible.

    ``a`` and ``b`` are the stored 2-D float32 CUDA tensors (any strides);
    ``trans_a``/``trans_b`` select op(x) = x^T.  ``out`` (M x N float32 on the
    same device, any non-overlapping strides) is overwritten; ``variant``
    forces a kernel variant (index or name); ``stream`` is a torch stream
    (default: the current stream).  Returns ``out``.
    """
    import torch

    for name, t in (("a", a), ("b", b)):
        if not isinstance(t, torch.Tensor) or t.dim() != 2:
            raise TypeError("%s must be a 2-D torch tensor" % name)
        if t.dtype != torch.float32:
            raise TypeError("%s must be float32" % name)
        if not t.is_cuda:
            raise ValueError("%s must be on a GPU; this library has no CPU path" % name)
    if a.device != b.device:
        raise ValueError("a and b are on different devices")
    M, N, K = _logical(a, b, trans_a, trans_b)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=a.device)
    elif out.shape != (M, N) or out.dtype != torch.float32 or out.device != a.device:
        raise ValueError("out must be float32 of shape (%d, %d) on %s" % (M, N, a.device))
    if variant is None:
        v = -1
    elif isinstance(variant, str):
        names = variant_names()
        if variant not in names:
            raise ValueError("unknown variant %r; known: %s" % (variant, ", ".join(names)))
        v = names.index(variant)
    else:
        v = int(variant)
    if stream is None:
        stream = torch.cuda.current_stream(a.device)
    with torch.cuda.device(a.device):
        st = repops_matmul_f32_ex(a.data_ptr(), a.stride(0), a.stride(1),
                                  b.data_ptr(), b.stride(0), b.stride(1),
                                  out.data_ptr(), out.stride(0), out.stride(1),
                                  M, N, K, trans_a, trans_b, stream.cuda_stream, v)
    if st != REPOPS_OK:
        raise RepopsError(st, "repops_matmul_f32")
    return out


def _variant_index(variant):
    if variant is None:
        return -1
    if isinstance(variant, str):
        names = variant_names()
        if variant not in names:
            raise ValueError("unknown variant %r; known: %s" % (variant, ", ".join(names)))
        return names.index(variant)
    return int(variant)


def matmul_batched(a, b, *, trans_a: bool = False, trans_b: bool = False, bias=None, out=None,
                   variant=None, stream=None):
    """C[n] = op(a[n]) @ op(b[n]) (+ bias) on the GPU, bit-reproducible.

    ``a``/``b``: stored 3-D float32 CUDA tensors (batch, rows, cols), any
    strides; ``bias``: (N,) shared by all batches or (batch, N), added once
    after each fixed-order sum.  ``out``: (batch, M, N).  Returns ``out``.
    """
    import torch

    for name, t in (("a", a), ("b", b)):
        if not isinstance(t, torch.Tensor) or t.dim() != 3 or t.dtype != torch.float32:
            raise TypeError("%s must be a 3-D float32 tensor" % name)
        if not t.is_cuda:
            raise ValueError("%s must be on a GPU; this library has no CPU path" % name)
    if a.shape[0] != b.shape[0]:
        raise ValueError("batch sizes differ")
    batch = a.shape[0]
    M, N, K = _logical(a[0] if batch else a.new_empty(a.shape[1:]),
                       b[0] if batch else b.new_empty(b.shape[1:]), trans_a, trans_b)
    if out is None:
        out = torch.empty((batch, M, N), dtype=torch.float32, device=a.device)
    elif tuple(out.shape) != (batch, M, N) or out.dtype != torch.float32:
        raise ValueError("out must be float32 of shape (%d, %d, %d)" % (batch, M, N))
    bptr, bbs, bs = None, 0, 0
    if bias is not None:
        if bias.dtype != torch.float32 or not bias.is_cuda:
            raise TypeError("bias must be a float32 CUDA tensor")
        if bias.dim() == 1 and bias.shape[0] == N:
            bptr, bbs, bs = bias.data_ptr(), 0, bias.stride(0)
        elif bias.dim() == 2 and tuple(bias.shape) == (batch, N):
            bptr, bbs, bs = bias.data_ptr(), bias.stride(0), bias.stride(1)
        else:
            raise ValueError("bias must be (N,) or (batch, N)")
    if stream is None:
        stream = torch.cuda.current_stream(a.device)
    with torch.cuda.device(a.device):
        st = repops_matmul_batched_f32(a.data_ptr(), a.stride(0), a.stride(1), a.stride(2),
                                       b.data_ptr(), b.stride(0), b.stride(1), b.stride(2),
                                       out.data_ptr(), out.stride(0), out.stride(1),
                                       out.stride(2), M, N, K, batch, trans_a, trans_b, bptr,
                                       bbs, bs, stream.cuda_stream, _variant_index(variant))
    if st != REPOPS_OK:
        raise RepopsError(st, "repops_matmul_batched_f32")
    return out


def canonical_order(dids):
    """Contributor indices in byte-lexicographic order of their identities
    (bytes or str), computed by the library; raises on duplicates."""
    st, order = repops_canonical_order([d.encode() if isinstance(d, str) else bytes(d)
                                        for d in dids])
    if st != REPOPS_OK:
        raise RepopsError(st, "repops_canonical_order")
    return order


def fold_mean_sgd(grads, theta, eta, *, dids=None, gbar=None, stream=None):
    """Fixed-order gradient average and SGD step on the GPU, bit-reproducible.

    ``grads``: list of k contiguous 1-D float32 CUDA tensors of length d (one
    per contributor); when ``dids`` (their identities) is given they are
    folded in canonical DID order, else in list order.  ``theta`` (d float32,
    contiguous) is updated in place: theta -= eta * gbar with
    gbar = RN(1/k) * (((g_1 + g_2) + ...) + g_k).  ``gbar``: optional output
    tensor (required when k > REPOPS_FOLD_MAX_PER_PASS).  Returns gbar.
    """
    import numpy as np
    import torch

    k = len(grads)
    if k < 1:
        raise ValueError("need at least one gradient")
    if dids is not None:
        if len(dids) != k:
            raise ValueError("one identity per gradient")
        grads = [grads[c] for c in canonical_order(dids)]
    d = theta.numel()
    for t in list(grads) + [theta] + ([gbar] if gbar is not None else []):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float32:
            raise TypeError("gradients, theta and gbar must be float32 tensors")
        if not t.is_cuda:
            raise ValueError("tensors must be on a GPU; this library has no CPU path")
        if not t.is_contiguous() or t.numel() != d:
            raise ValueError("every tensor must be contiguous with d = %d elements" % d)
    if gbar is None and k > REPOPS_FOLD_MAX_PER_PASS:
        gbar = torch.empty_like(theta)
    if stream is None:
        stream = torch.cuda.current_stream(theta.device)
    with torch.cuda.device(theta.device):
        st = repops_fold_mean_sgd_f32([g.data_ptr() for g in grads], k, d,
                                      float(np.float32(eta)), theta.data_ptr(),
                                      gbar.data_ptr() if gbar is not None else None,
                                      stream.cuda_stream)
    if st != REPOPS_OK:
        raise RepopsError(st, "repops_fold_mean_sgd_f32")
    return gbar


def _workspace(nbytes, leaf_bytes, device, workspace):
    import torch

    need = repops_merkle_workspace_bytes(nbytes, leaf_bytes)
    if need < 0:
        raise ValueError("invalid sizes: %d bytes in leaves of %d (both multiples of 4, "
                         "leaf_bytes in [4, 2^24])" % (nbytes, leaf_bytes))
    if need == 0:
        return None, 0
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < need or not workspace.is_contiguous():
            raise ValueError("workspace must be contiguous with at least %d bytes" % need)
        return workspace, workspace.numel() * workspace.element_size()
    return torch.empty(need, dtype=torch.uint8, device=device), need


def merkle_root(t, *, leaf_bytes: int = REPOPS_MERKLE_DEFAULT_LEAF_BYTES, out=None,
                workspace=None, stream=None):
    """SHA-256 Merkle tree hash (RFC 6962 shape) of a contiguous CUDA tensor's
    bytes, computed on the GPU.  For a float32 tensor this is the tensor hash
    of its elements in row-major order.  With ``out`` (a 32-byte uint8 CUDA
    tensor) the root is written there and nothing is synchronised; otherwise
    the 32 root bytes are returned as ``bytes``."""
    import torch

    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError("t must be a CUDA tensor; this library has no CPU path")
    if not t.is_contiguous():
        raise ValueError("t must be contiguous (the hash covers its row-major bytes)")
    nbytes = t.numel() * t.element_size()
    ws, ws_bytes = _workspace(nbytes, leaf_bytes, t.device, workspace)
    root = out if out is not None else torch.empty(32, dtype=torch.uint8, device=t.device)
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    with torch.cuda.device(t.device):
        st = repops_merkle_root(t.data_ptr() if nbytes else None, nbytes, leaf_bytes,
                                ws.data_ptr() if ws is not None else None, ws_bytes,
                                root.data_ptr(), stream.cuda_stream)
    if st != REPOPS_OK:
        raise RepopsError(st, "repops_merkle_root")
    if out is not None:
        return out
    stream.synchronize()
    return bytes(root.cpu().numpy().tobytes())


def referee_matmul(a, b, claims, *, trans_a: bool = False, trans_b: bool = False,
                   leaf_bytes: int = REPOPS_MERKLE_DEFAULT_LEAF_BYTES, out=None, workspace=None,
                   stream=None):
    """The referee's decision on a disputed matmul output: recompute
    C = op(a) op(b) on the GPU, hash it, and compare with each trainer's
    claimed 32-byte output hash.  Returns (root bytes, [bool per claim], C)."""
    import numpy as np
    import torch

    for name, t in (("a", a), ("b", b)):
        if not isinstance(t, torch.Tensor) or t.dim() != 2 or t.dtype != torch.float32:
            raise TypeError("%s must be a 2-D float32 tensor" % name)
        if not t.is_cuda:
            raise ValueError("%s must be on a GPU; this library has no CPU path" % name)
    M, N, K = _logical(a, b, trans_a, trans_b)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=a.device)
    elif tuple(out.shape) != (M, N) or out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 (%d, %d) tensor" % (M, N))
    claims = [bytes(c) for c in claims]
    if any(len(c) != 32 for c in claims):
        raise ValueError("each claim is a 32-byte digest")
    dev = a.device
    ws, ws_bytes = _workspace(M * N * 4, leaf_bytes, dev, workspace)
    cl = (torch.from_numpy(np.frombuffer(b"".join(claims), dtype=np.uint8).copy()).to(dev)
          if claims else None)
    root = torch.empty(32, dtype=torch.uint8, device=dev)
    match = torch.empty(max(len(claims), 1), dtype=torch.int32, device=dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        st = repops_referee_matmul_f32(a.data_ptr(), a.stride(0), a.stride(1), b.data_ptr(),
                                       b.stride(0), b.stride(1), out.data_ptr(), M, N, K,
                                       trans_a, trans_b, leaf_bytes,
                                       ws.data_ptr() if ws is not None else None, ws_bytes,
                                       cl.data_ptr() if cl is not None else None, len(claims),
                                       root.data_ptr(), match.data_ptr(), stream.cuda_stream)
    if st != REPOPS_OK:
        raise RepopsError(st, "repops_referee_matmul_f32")
    stream.synchronize()
    return (bytes(root.cpu().numpy().tobytes()),
            [bool(v) for v in match.cpu().numpy()[:len(claims)]], out)


def _unary(name, fn, x, out, stream):
    import torch

    if not isinstance(x, torch.Tensor) or x.dtype != torch.float32:
        raise TypeError("x must be a float32 tensor")
    if not x.is_cuda:
        raise ValueError("x must be on a GPU; this library has no CPU path")
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    if out is None:
        out = torch.empty_like(x)
    elif out.shape != x.shape or out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 tensor shaped like x")
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    with torch.cuda.device(x.device):
        st = fn(x.data_ptr(), out.data_ptr(), x.numel(), stream.cuda_stream)
    if st != REPOPS_OK:
        raise RepopsError(st, name)
    return out


def erf(x, *, out=None, stream=None):
    """erf of every element of a contiguous float32 CUDA tensor, by the fixed
    binary32 evaluation of repops_erf_f32 (``out`` may be ``x``)."""
    return _unary("repops_erf_f32", repops_erf_f32, x, out, stream)


def gelu(x, *, out=None, stream=None):
    """GeLU (erf form) of every element, fixed binary32 evaluation."""
    return _unary("repops_gelu_f32", repops_gelu_f32, x, out, stream)


def layernorm(x, gamma=None, beta=None, eps: float = 1e-5, *, out=None, return_stats=False,
              stream=None):
    """LayerNorm over the last dimension of a float32 CUDA tensor whose rows
    are contiguous (any leading shape), fixed-order sums.  Returns y, or
    (y, mean, rstd) with ``return_stats``."""
    import numpy as np
    import torch

    if not isinstance(x, torch.Tensor) or x.dtype != torch.float32 or x.dim() < 1:
        raise TypeError("x must be a float32 tensor")
    if not x.is_cuda:
        raise ValueError("x must be on a GPU; this library has no CPU path")
    H = x.shape[-1]
    x2 = x.reshape(-1, H) if x.dim() != 2 else x
    if x2.numel() and x2.stride(1) != 1:
        raise ValueError("the rows of x must be contiguous")
    rows = x2.shape[0]
    if out is None:
        out = torch.empty(x.shape, dtype=torch.float32, device=x.device)
    y2 = out.view(-1, H) if out.dim() != 2 else out  # a view: never a copy
    if tuple(out.shape) != tuple(x.shape) or (y2.numel() and y2.stride(1) != 1):
        raise ValueError("out must be shaped like x with contiguous rows")
    for name, t in (("gamma", gamma), ("beta", beta)):
        if t is not None and (t.dtype != torch.float32 or not t.is_cuda or t.numel() != H
                              or not t.is_contiguous()):
            raise ValueError("%s must be a contiguous float32 CUDA tensor of %d elements"
                             % (name, H))
    mean = torch.empty(rows, dtype=torch.float32, device=x.device) if return_stats else None
    rstd = torch.empty(rows, dtype=torch.float32, device=x.device) if return_stats else None
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    with torch.cuda.device(x.device):
        st = repops_layernorm_f32(x2.data_ptr(), x2.stride(0) if rows > 1 else H,
                                  gamma.data_ptr() if gamma is not None else None,
                                  beta.data_ptr() if beta is not None else None,
                                  y2.data_ptr(), y2.stride(0) if rows > 1 else H, rows, H,
                                  float(np.float32(eps)),
                                  mean.data_ptr() if mean is not None else None,
                                  rstd.data_ptr() if rstd is not None else None,
                                  stream.cuda_stream)
    if st != REPOPS_OK:
        raise RepopsError(st, "repops_layernorm_f32")
    return (out, mean, rstd) if return_stats else out
