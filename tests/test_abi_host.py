"""Host-side checks of the C ABI that need no GPU.

* librepops.so loads and exports every function include/repops.h declares;
* argument validation (run through repops_check_args_f32 and through
  repops_matmul_f32 itself: invalid calls return before any device work);
* variant table, status strings and the build manifest;
* the instruction scan of the gfx950 assembly built from the same sources:
  no fused or packed FP32, no dot or matrix instructions in the VALU
  kernels, IEEE denormals and round-to-nearest-even in every kernel
  descriptor, no register spills in the tiled kernels.
"""
from __future__ import annotations

import ctypes
import json
import os
import re

import pytest

import bit_reproducible_fp32_amd as rp
from bit_reproducible_fp32_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "repops.h")
ASM = os.path.join(ROOT, "bit_reproducible_fp32_amd", "librepops_gfx950.s")

# Fake, never-dereferenced addresses: validation compares them only.
PA, PB, PC = 0x10000000, 0x20000000, 0x30000000


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(repops_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = _lib.load()
    declared = header_functions()
    assert declared, "no declarations parsed"
    for name in declared:
        assert hasattr(lib, name), "missing export %s" % name
    assert sorted(_lib.EXPORTS) == declared


def test_binding_has_the_same_names():
    for name in header_functions():
        assert callable(getattr(rp, name)), name


def ok(**kw):
    args = dict(A=PA, a_rs=64, a_cs=1, B=PB, b_rs=32, b_cs=1, C=PC, c_rs=32, c_cs=1,
                M=16, N=32, K=64, trans_a=0, trans_b=0, variant=-1)
    args.update(kw)
    return rp.repops_check_args_f32(**args)


def test_valid_arguments_pass():
    assert ok() == rp.REPOPS_OK
    assert ok(trans_a=1, a_rs=16, a_cs=1) == rp.REPOPS_OK
    assert ok(trans_b=1, b_rs=64, b_cs=1) == rp.REPOPS_OK
    assert ok(a_rs=0, a_cs=0) == rp.REPOPS_OK  # broadcast operand
    assert ok(c_rs=1, c_cs=16) == rp.REPOPS_OK  # column-major output
    for v in range(rp.repops_variant_count()):
        assert ok(variant=v) == rp.REPOPS_OK


def test_dimension_errors():
    assert ok(M=-1) == rp.REPOPS_ERR_DIM
    assert ok(N=-5) == rp.REPOPS_ERR_DIM
    assert ok(K=-1) == rp.REPOPS_ERR_DIM
    assert ok(trans_a=2) == rp.REPOPS_ERR_DIM
    assert ok(trans_b=-1) == rp.REPOPS_ERR_DIM
    assert ok(a_rs=2 ** 62) == rp.REPOPS_ERR_DIM  # offset overflow
    assert ok(M=2 ** 40, N=2 ** 40, c_rs=2 ** 40) == rp.REPOPS_ERR_DIM  # grid too large


def test_null_errors_and_empty_problems():
    assert ok(A=0) == rp.REPOPS_ERR_NULL
    assert ok(B=0) == rp.REPOPS_ERR_NULL
    assert ok(C=0) == rp.REPOPS_ERR_NULL
    assert ok(A=0, B=0, K=0) == rp.REPOPS_OK     # K = 0: operands unused
    assert ok(A=0, B=0, C=0, M=0) == rp.REPOPS_OK  # nothing to do
    assert ok(A=0, B=0, C=0, N=0) == rp.REPOPS_OK


def test_stride_errors():
    assert ok(a_rs=-64) == rp.REPOPS_ERR_STRIDE
    assert ok(b_cs=-1) == rp.REPOPS_ERR_STRIDE
    assert ok(c_rs=0) == rp.REPOPS_ERR_STRIDE    # two rows on one address
    assert ok(c_cs=0) == rp.REPOPS_ERR_STRIDE
    assert ok(c_rs=16) == rp.REPOPS_ERR_STRIDE   # rows overlap (N = 32)
    assert ok(M=1, c_rs=0) == rp.REPOPS_OK       # one row: its stride is unused


def test_alias_errors():
    # C starts inside A's span: A spans 16*64 floats from PA.
    assert ok(C=PA + 4 * 100) == rp.REPOPS_ERR_ALIAS
    assert ok(C=PB) == rp.REPOPS_ERR_ALIAS
    # C ends exactly where A starts: no overlap.
    assert ok(C=PA - 4 * 16 * 32) == rp.REPOPS_OK
    assert ok(C=PA - 4 * 16 * 32 + 4) == rp.REPOPS_ERR_ALIAS
    # K = 0 reads neither operand, so no alias is possible.
    assert ok(C=PA, K=0) == rp.REPOPS_OK


def test_variant_errors_and_table():
    n = rp.repops_variant_count()
    assert n >= 5
    assert ok(variant=n) == rp.REPOPS_ERR_VARIANT
    assert ok(variant=-2) == rp.REPOPS_ERR_VARIANT
    names = rp.variant_names()
    assert len(set(names)) == n and all(names)
    assert rp.repops_variant_name(n) == "?"
    assert names[0].startswith("naive")


def test_matmul_entry_rejects_before_any_device_work():
    """Invalid calls return their status from the real entry point (no GPU here)."""
    st = rp.repops_matmul_f32(PA, 64, 1, PB, 32, 1, PA, 32, 1, 16, 32, 64, 0, 0, 0)
    assert st == rp.REPOPS_ERR_ALIAS
    st = rp.repops_matmul_f32_ex(PA, 64, 1, PB, 32, 1, PC, 32, 1, 16, 32, 64, 0, 0, 0, 999)
    assert st == rp.REPOPS_ERR_VARIANT
    assert rp.repops_matmul_f32(0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 5, 5, 0, 0, 0) == rp.REPOPS_OK


def test_pick_variant():
    big = rp.repops_pick_variant_f32(PA, 4096, 1, PB, 14336, 1, 4096, 14336, 4096, 0, 0)
    small = rp.repops_pick_variant_f32(PA, 256, 1, PB, 256, 1, 256, 256, 256, 0, 0)
    assert 0 <= big < rp.repops_variant_count() and 0 <= small < rp.repops_variant_count()
    assert rp.repops_pick_variant_f32(PA, 1, 1, PB, 1, 1, 0, 1, 1, 0, 0) == -1


def test_strerror_and_manifest():
    for st in range(8):
        assert rp.repops_strerror(st) != "unknown status"
    assert rp.repops_strerror(99) == "unknown status"
    man = json.loads(rp.repops_build_manifest())
    assert man["offload_arch"] == "gfx950"
    assert "-ffp-contract=off" in man["flags"]
    assert man["variants"] == rp.variant_names()


def test_python_wrapper_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    a = torch.zeros(4, 4)
    with pytest.raises(ValueError):
        rp.matmul(a, a)


# ---------------------------------------------------------------- instruction scan
FORBIDDEN_FP = re.compile(
    r"^\s+(v_fma\w*|v_fmac\w*|v_mad_(f16|f32|legacy\w*|mix\w*)|v_mac_\w*|v_pk_fma_f32|"
    r"v_pk_mul_f32|v_pk_add_f32|v_dot\w*|v_fma_mix\w*)\b", re.M)
MATRIX = re.compile(r"^\s+v_(s)?mfma\w*", re.M)


def kernels():
    text = open(ASM).read()
    out = {}
    for m in re.finditer(r"^(_Z\w+):[ \t]*(;.*)?$", text, re.M):
        name = m.group(1)
        end = text.find(".Lfunc_end", m.end())
        out[name] = text[m.end():end]
    descs = dict(re.findall(r"\.amdhsa_kernel (\S+)\n(.*?)\.end_amdhsa_kernel", text, re.S))
    return out, descs


def test_isa_has_no_fused_or_packed_fp32():
    bodies, _ = kernels()
    assert bodies
    for name, body in bodies.items():
        bad = FORBIDDEN_FP.findall(body)
        if DIV_FIXUP.search(body) or SQRT.search(body):
            continue  # checked by the next test
        assert not bad, "%s uses %s" % (name, bad[:3])


DIV_FIXUP = re.compile(r"^\s+v_div_fixup_f32\b", re.M)
SQRT = re.compile(r"^\s+v_sqrt_f32\w*", re.M)
FMA_F32 = re.compile(r"^\s+(v_fma_f32|v_fmac_f32\w*)\b", re.M)


def test_isa_fused_ops_only_inside_division_and_square_root():
    """Kernels that divide or take square roots (the correctly rounded IEEE
    operations, which the compiler expands with fused multiply-adds: five per
    division, two per square root on gfx950) may hold exactly that many
    fused operations and no other forbidden form."""
    bodies, _ = kernels()
    seen = 0
    for name, body in bodies.items():
        ndiv, nsqrt = len(DIV_FIXUP.findall(body)), len(SQRT.findall(body))
        if not (ndiv or nsqrt):
            continue
        seen += 1
        fma = len(FMA_F32.findall(body))
        assert fma == 5 * ndiv + 2 * nsqrt, (name, fma, ndiv, nsqrt)
        other = [m[0] for m in FORBIDDEN_FP.findall(body)
                 if not re.match(r"v_fmac?_f32", m[0])]
        assert not other, (name, other[:3])
    assert seen >= 4


def test_isa_valu_kernels_use_no_matrix_instructions():
    bodies, _ = kernels()
    for name, body in bodies.items():
        if "tiled_kernel" in name or "naive_kernel" in name:
            assert not MATRIX.search(body), name


# FP32 matrix shapes with inner dimension 1: every output is one product.
K1_FP32_SHAPES = {"v_mfma_f32_32x32x1_2b_f32", "v_mfma_f32_16x16x1_4b_f32",
                  "v_mfma_f32_4x4x1_16b_f32"}
MFMA_LINE = re.compile(r"^\s+(v_mfma\w*)\s+([^\n]*)$", re.M)


def test_isa_matrix_product_kernels_only_form_single_products():
    """The product kernels may use only FP32 matrix shapes with inner
    dimension 1 (no sum inside the matrix core), with the addend operand the
    literal 0, no VALU multiply, and VALU adds (the fixed-order sum)."""
    bodies, _ = kernels()
    mprod = {n: b for n, b in bodies.items() if re.search(r"mprod(16)?_kernel", n)}
    assert len(mprod) >= 2
    for name, body in mprod.items():
        found = MFMA_LINE.findall(body)
        assert found, name
        for mnem, ops in found:
            assert mnem in K1_FP32_SHAPES, (name, mnem)
            assert ops.split(",")[-1].strip() == "0", (name, ops)
        assert "v_add_f32" in body and "v_mul_f32" not in body, name


def _longest_store_run_without_wait(body):
    best = cur = 0
    for line in body.splitlines():
        t = line.strip()
        if t.startswith("global_store"):
            cur += 1
            best = max(best, cur)
        elif t.startswith("s_waitcnt") and "vmcnt" in t:
            cur = 0
    return best


def test_isa_matrix_product_epilogue_stores_do_not_wait():
    """The 32-wide matrix-core product kernel stores a lane's 32 sums of a
    column block with no memory-counter wait between the stores. On gfx9 one
    counter tracks loads and stores, so a wait placed between two stores
    (for example for a bias load) would make each store wait for the one
    before it. In every instantiation, at least 32 consecutive stores have no
    vmcnt wait between them."""
    bodies, _ = kernels()
    mprod = {n: b for n, b in bodies.items() if "mprod_kernel" in n and "mprod16" not in n}
    assert len(mprod) >= 9
    for name, body in mprod.items():
        assert _longest_store_run_without_wait(body) >= 32, name


def test_isa_mul_and_add_present_in_tiled_kernels():
    bodies, _ = kernels()
    tiled = [b for n, b in bodies.items() if "tiled_kernel" in n]
    assert tiled
    for b in tiled:
        assert "v_mul_f32" in b and "v_add_f32" in b


def test_kernel_descriptors_ieee_denormals_and_rne():
    _, descs = kernels()
    assert descs
    for name, d in descs.items():
        assert re.search(r"\.amdhsa_float_denorm_mode_32 3\b", d), name
        assert re.search(r"\.amdhsa_float_round_mode_32 0\b", d), name


def test_no_kernel_spills_or_uses_scratch():
    """Every kernel keeps its state in registers and LDS: no spills and no
    per-lane scratch memory."""
    text = open(ASM).read()
    seen = 0
    for block in text.split("  - .agpr_count:")[1:]:
        name = re.search(r"\.name:\s+(\S+)", block).group(1)
        if "repops" not in name:
            continue
        seen += 1
        spill = int(re.search(r"\.vgpr_spill_count:\s+(\d+)", block).group(1))
        priv = int(re.search(r"\.private_segment_fixed_size:\s+(\d+)", block).group(1))
        assert spill == 0 and priv == 0, name
    assert seen >= 30


def test_assembly_matches_the_library_build():
    """The scanned assembly is at least as new as every kernel source."""
    from bit_reproducible_fp32_amd import build
    for src in build.KERNEL_SOURCES:
        assert os.path.getmtime(ASM) >= os.path.getmtime(src) - 1, src


def bok(**kw):
    """repops_matmul_batched_f32 through calls that all fail validation, so
    nothing is ever launched."""
    args = dict(A=PA, a_bs=16 * 64, a_rs=64, a_cs=1, B=PB, b_bs=64 * 32, b_rs=32, b_cs=1,
                C=PC, c_bs=16 * 32, c_rs=32, c_cs=1, M=16, N=32, K=64, batch=3,
                trans_a=0, trans_b=0, bias=None, bias_bs=0, bias_s=1, stream=0, variant=-1)
    args.update(kw)
    return rp.repops_matmul_batched_f32(**args)


def test_batched_validation_errors():
    assert bok(batch=-1) == rp.REPOPS_ERR_DIM
    assert bok(a_bs=-1) == rp.REPOPS_ERR_STRIDE
    assert bok(c_bs=-32) == rp.REPOPS_ERR_STRIDE
    assert bok(c_bs=16) == rp.REPOPS_ERR_STRIDE          # batches overlap in C
    assert bok(c_bs=0) == rp.REPOPS_ERR_STRIDE           # all batches on one C
    assert bok(C=PA + 4 * 100) == rp.REPOPS_ERR_ALIAS    # C inside A's batches
    assert bok(bias=PC + 8) == rp.REPOPS_ERR_ALIAS       # bias inside C
    assert bok(bias=PB, bias_s=-1) == rp.REPOPS_ERR_STRIDE
    assert bok(variant=999) == rp.REPOPS_ERR_VARIANT
    assert bok(batch=0, A=0, B=0, C=0) == rp.REPOPS_OK   # nothing to do


def test_batched_injectivity_rule():
    # interleaved heads: C viewed as (batch=4, M=8, N=16) inside an (8, 4*16)
    # row-major buffer: c_bs=16, c_rs=64, c_cs=1 is injective
    assert rp.repops_check_args_f32(PA, 64, 1, PB, 16, 1, PC, 64, 1, 8, 16, 64, 0, 0, -1) == 0
    # (C placed inside A, so each call stops with an error before any launch;
    # the alias check comes after the stride check)
    st = rp.repops_matmul_batched_f32(PA, 0, 64, 1, PB, 0, 16, 1, PA, 16, 64, 1, 8, 16, 64, 4,
                                      0, 0, None, 0, 0, 0, -1)
    assert st == rp.REPOPS_ERR_ALIAS    # strides accepted, stopped by the alias check
    st = rp.repops_matmul_batched_f32(PA, 0, 64, 1, PB, 0, 16, 1, PA, 15, 64, 1, 8, 16, 64, 4,
                                      0, 0, None, 0, 0, 0, -1)
    assert st == rp.REPOPS_ERR_STRIDE   # batch stride 15 < 16 columns: overlap


def test_pick_uses_each_kernel_family_by_size():
    """The automatic choice: the one-row scalar-row kernel below 2^17
    outputs; above, the family with the least estimated time for the busiest
    CU (tiles per CU over the family's measured efficiency at that load), the
    128x128 product kernel unless another is estimated 2 % faster; and the
    register-blocked VALU kernel instead of a scalar-row one when K reaches
    2^30 (their k offsets are 32-bit)."""
    names = rp.variant_names()

    def pick(M, N, K):
        return names[rp.repops_pick_variant_f32(PA, K, 1, PB, N, 1, M, N, K, 0, 0)]

    mp1, mp16 = "mprod1_t128x128x32_w8_xcd", "mprod16_t128x64x32_w8_xcd"
    r4c2, r4c1 = "srow_t32x128x32_r4c2_w8_xcd", "srow_t16x64x32_r4c1_w4_xcd"
    assert pick(4096, 14336, 4096) == mp1     # 3584 tiles of 128x128: 14 per CU
    assert pick(4096, 2048, 8192) == mp1      # 512: two per CU
    assert pick(2688, 2688, 2688) == mp1      # 441: two per CU
    assert pick(2048, 2048, 64) == mp16       # 512 of 128x64 (two per CU) against 256
    assert pick(1792, 1792, 1792) == mp16     # 392 of 128x64 against 196
    assert pick(2176, 2176, 2176) == mp16     # 289 of 128x128 would leave 223 CUs with one
    assert pick(1408, 1408, 1408) == mp16     # 242 of 128x64, one per CU
    assert pick(2048, 1024, 1024) == mp16     # 256 of 128x64
    assert pick(1024, 1024, 1024) == r4c2     # 256 of 32x128
    assert pick(1664, 1664, 1664) == r4c2     # 676 of 32x128: three per CU
    assert pick(1152, 1152, 1152) == r4c1     # 324 of 32x128 would leave 188 CUs with one
    assert pick(768, 768, 768) == r4c1        # 144 of 32x128
    assert pick(512, 256, 1024) == r4c1       # 2^17 outputs
    assert pick(256, 256, 256) == "srow_t4x64x32_r1c1_w4_row"
    assert pick(4, 4, (1 << 30) - 1) == "srow_t4x64x32_r1c1_w4_row"
    assert pick(4, 4, 1 << 30) == "valu_t64x64x16_r4x4_row"
