"""Host-side checks of the C ABI: the library loads without a GPU, exports every
function include/shampoo.h declares, and rejects bad arguments synchronously
before touching the GPU (no compute call is made here)."""
import ctypes
import os
import re

import pytest

from inverse_root_preconditioning_amd import capi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "shampoo.h")

FAKE = 0x10000  # a non-null address that is never dereferenced on these paths


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(shampoo_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return capi.load()


def test_header_declares_the_five_entry_points():
    fns = declared_functions()
    for name in ("shampoo_accumulate", "shampoo_scale_power", "shampoo_invroot_newton",
                 "shampoo_invroot_cheby", "shampoo_precondition"):
        assert name in fns


def test_library_exports_every_declared_symbol(lib):
    fns = declared_functions()
    assert len(fns) >= 8
    for name in fns:
        assert hasattr(lib, name), name
        assert name in capi.EXPORTED, f"binding lacks {name}"


def test_struct_layouts_match_header():
    assert ctypes.sizeof(capi.shampoo_block) == 24
    assert capi.shampoo_block.rows.offset == 16 and capi.shampoo_block.cols.offset == 20
    assert ctypes.sizeof(capi.shampoo_scale) == 16


def test_abi_version_and_strerror(lib):
    assert capi.shampoo_abi_version() == capi.ABI_VERSION
    for code in (capi.OK, capi.EINVAL, capi.EUNSUPPORTED, capi.EWORKSPACE, capi.EHIP, -99):
        assert len(capi.shampoo_strerror(code)) > 0


def test_workspace_sizes():
    ws = capi.shampoo_workspace_bytes
    B, nf = 256, 32
    stack = nf * B * B * 4
    assert ws(capi.OP_NEWTON, nf, B, capi.NDB, capi.F32) >= 5 * stack
    assert ws(capi.OP_NEWTON, nf, B, capi.CN, capi.F32) >= 7 * stack
    assert ws(capi.OP_NEWTON, nf, B, capi.CN_F16, capi.F32) >= stack + 7 * stack // 2
    assert ws(capi.OP_CHEBY, nf, B, 16, capi.F32) >= 4 * stack
    assert ws(capi.OP_CHEBY, nf, B, 16, capi.BF16_IN) > ws(capi.OP_CHEBY, nf, B, 16, capi.F32)
    assert ws(capi.OP_SCALE, nf, B, 0, capi.F32) >= 2 * nf * B * 32 * 4
    assert ws(capi.OP_PRECONDITION, nf // 2, B, 0, capi.F32) >= stack // 2
    assert ws(capi.OP_ACCUMULATE, nf // 2, B, 0, capi.F32) == 0
    assert ws(capi.OP_ACCUMULATE, nf // 2, B, 0, capi.BF16_IN) > 0
    # invalid arguments give 0
    assert ws(capi.OP_NEWTON, nf, 100, capi.NDB, capi.F32) == 0
    assert ws(capi.OP_NEWTON, -1, B, capi.NDB, capi.F32) == 0
    assert ws(99, nf, B, 0, capi.F32) == 0
    assert ws(capi.OP_NEWTON, nf, B, 7, capi.F32) == 0
    # modifier bits do not change the workspace
    for v in (capi.NDB, capi.NDB_Z, capi.CN, capi.CN_F16):
        base = ws(capi.OP_NEWTON, nf, B, v, capi.F32)
        assert ws(capi.OP_NEWTON, nf, B, v | capi.SYM_COUPLING, capi.F32) == base
        assert ws(capi.OP_NEWTON, nf, B, v | capi.FULL_PRODUCTS, capi.F32) == base


def test_validation_codes_without_gpu():
    f = capi
    # unsupported B
    assert f.shampoo_invroot_newton(FAKE, FAKE, 4, 100, 4, f.NDB, 10, FAKE, 0, FAKE, FAKE, 1 << 40, 0) == f.EUNSUPPORTED
    assert f.shampoo_invroot_newton(FAKE, FAKE, 4, 32, 4, f.NDB, 10, FAKE, 0, FAKE, FAKE, 1 << 40, 0) == f.EUNSUPPORTED
    # negative count, bad iteration count, bad p / variant
    assert f.shampoo_invroot_newton(FAKE, FAKE, -1, 64, 4, f.NDB, 10, FAKE, 0, FAKE, FAKE, 1 << 40, 0) == f.EINVAL
    assert f.shampoo_invroot_newton(FAKE, FAKE, 4, 64, 4, f.NDB, 0, FAKE, 0, FAKE, FAKE, 1 << 40, 0) == f.EINVAL
    assert f.shampoo_invroot_newton(FAKE, FAKE, 4, 64, 3, f.NDB, 5, FAKE, 0, FAKE, FAKE, 1 << 40, 0) == f.EUNSUPPORTED
    assert f.shampoo_invroot_newton(FAKE, FAKE, 4, 64, 3, f.CN, 5, FAKE, 0, FAKE, FAKE, 1 << 40, 0) == f.EUNSUPPORTED
    assert f.shampoo_invroot_newton(FAKE, FAKE, 4, 64, 4, 9, 5, FAKE, 0, FAKE, FAKE, 1 << 40, 0) == f.EINVAL
    assert f.shampoo_invroot_newton(FAKE, FAKE, 4, 192, 4, f.CN_F16, 5, FAKE, 0, FAKE, FAKE, 1 << 40, 0) == f.EUNSUPPORTED
    assert f.shampoo_invroot_newton(FAKE, FAKE, 4, 256, 3, f.CN_F16, 5, FAKE, 0, FAKE, FAKE, 1 << 40, 0) == f.EUNSUPPORTED
    assert f.shampoo_invroot_newton(FAKE, FAKE, 4, 100, 4, f.NDB_Z | f.SYM_COUPLING, 5, FAKE, 0, FAKE, FAKE, 1 << 40,
                                    0) == f.EUNSUPPORTED
    assert f.shampoo_invroot_newton(FAKE, FAKE, 4, 64, 4, 9 | f.SYM_COUPLING, 5, FAKE, 0, FAKE, FAKE, 1 << 40,
                                    0) == f.EINVAL
    # null pointers and workspace
    assert f.shampoo_invroot_newton(0, FAKE, 4, 64, 4, f.NDB, 5, FAKE, 0, FAKE, FAKE, 1 << 40, 0) == f.EINVAL
    assert f.shampoo_invroot_newton(FAKE, FAKE, 4, 64, 4, f.NDB, 5, FAKE, 0, FAKE, FAKE, 16, 0) == f.EWORKSPACE
    assert f.shampoo_invroot_newton(FAKE, FAKE, 4, 64, 4, f.NDB, 5, FAKE, 0, FAKE, 0, 1 << 40, 0) == f.EWORKSPACE
    # empty input is a no-op
    assert f.shampoo_invroot_newton(0, 0, 0, 64, 4, f.NDB, 5, 0, 0, 0, 0, 0, 0) == f.OK
    assert f.shampoo_accumulate(0, 0, 64, 0, 0.9, 0.1, f.F32, 0, 0, 0) == f.OK
    assert f.shampoo_precondition(0, 0, 0, 64, 0, f.F32, 0, 0, 0) == f.OK
    assert f.shampoo_scale_power(0, 0, 64, 0.0, f.SCALE_POWER, 0, 32, 20, 2.0, 0, 0, 0, 0, 0) == f.OK
    assert f.shampoo_invroot_cheby(0, 0, 0, 64, 4, 8, 0.0, f.F32, 0, 0, 0, 0, 0) == f.OK
    # scale: r out of range, bad safety, missing v0
    args = (FAKE, 4, 64, 0.0, f.SCALE_POWER, FAKE, 33, 20, 2.0, FAKE, FAKE, FAKE, 1 << 40, 0)
    assert f.shampoo_scale_power(*args) == f.EINVAL
    args = (FAKE, 4, 64, 0.0, f.SCALE_POWER, FAKE, 8, 20, -1.0, FAKE, FAKE, FAKE, 1 << 40, 0)
    assert f.shampoo_scale_power(*args) == f.EINVAL
    args = (FAKE, 4, 64, 0.0, f.SCALE_POWER, 0, 8, 20, 2.0, FAKE, FAKE, FAKE, 1 << 40, 0)
    assert f.shampoo_scale_power(*args) == f.EINVAL
    args = (FAKE, 4, 64, -1.0, f.SCALE_FROBENIUS, 0, 0, 0, 0.0, FAKE, FAKE, FAKE, 1 << 40, 0)
    assert f.shampoo_scale_power(*args) == f.EINVAL
    # chebyshev degree bounds, bf16 needs B % 128 == 0
    assert f.shampoo_invroot_cheby(FAKE, FAKE, 4, 64, 4, 0, 0.0, f.F32, FAKE, FAKE, FAKE, 1 << 40, 0) == f.EINVAL
    assert f.shampoo_invroot_cheby(FAKE, FAKE, 4, 64, 4, 257, 0.0, f.F32, FAKE, FAKE, FAKE, 1 << 40, 0) == f.EINVAL
    assert f.shampoo_invroot_cheby(FAKE, FAKE, 4, 192, 4, 8, 0.0, f.BF16_IN, FAKE, FAKE, FAKE, 1 << 40, 0) == f.EUNSUPPORTED
    assert f.shampoo_invroot_cheby(FAKE, FAKE, 4, 64, 4, 8, -1.0, f.F32, FAKE, FAKE, FAKE, 1 << 40, 0) == f.EINVAL
    # accumulate / precondition
    assert f.shampoo_accumulate(FAKE, 2, 64, 0, 0.9, 0.1, f.F32, 0, 0, 0) == f.EINVAL
    assert f.shampoo_accumulate(FAKE, 2, 64, FAKE, float("nan"), 0.1, f.F32, 0, 0, 0) == f.EINVAL
    assert f.shampoo_accumulate(FAKE, 2, 128, FAKE, 0.9, 0.1, f.BF16_IN, 0, 0, 0) == f.EWORKSPACE
    assert f.shampoo_accumulate(FAKE, 2, 128, FAKE, 0.9, 0.1, 5, 0, 0, 0) == f.EUNSUPPORTED
    assert f.shampoo_precondition(FAKE, FAKE, 2, 64, FAKE, f.F32, FAKE, 16, 0) == f.EWORKSPACE
    assert f.shampoo_precondition(FAKE, 0, 2, 64, FAKE, f.F32, FAKE, 1 << 40, 0) == f.EINVAL


def test_graft_validation_without_gpu():
    f = capi
    ok = (FAKE, FAKE, FAKE, FAKE, FAKE, 3, 128)
    assert f.shampoo_graft_update(*ok, 1e-3, 0.9, 0.999, 1e-8, 0, 0, FAKE, 1 << 40, 0) == f.EINVAL   # step 0
    assert f.shampoo_graft_update(*ok, 1e-3, 1.0, 0.999, 1e-8, 1, 0, FAKE, 1 << 40, 0) == f.EINVAL   # beta1 = 1
    assert f.shampoo_graft_update(*ok, float("inf"), 0.9, 0.999, 1e-8, 1, 0, FAKE, 1 << 40, 0) == f.EINVAL
    assert f.shampoo_graft_update(*ok, 1e-3, 0.9, 0.999, 1e-8, 1, 0, FAKE, 0, 0) == f.EWORKSPACE
    assert f.shampoo_graft_update(0, FAKE, FAKE, FAKE, FAKE, 3, 128, 1e-3, 0.9, 0.999, 1e-8, 1, 0, FAKE,
                                  1 << 40, 0) == f.EINVAL
    assert f.shampoo_graft_update(0, 0, 0, 0, 0, 0, 128, 1e-3, 0.9, 0.999, 1e-8, 1, 0, 0, 0, 0) == f.OK
    assert f.shampoo_workspace_bytes(f.OP_GRAFT, 10, 1024, 0, f.F32) >= 10 * 16 * 2 * 4


def test_binding_raises_when_library_missing(tmp_path):
    with pytest.raises(RuntimeError, match="not built"):
        capi.load(str(tmp_path / "missing.so"))


def test_pipeline_rejects_missing_or_host_tensors():
    import torch
    from inverse_root_preconditioning_amd import pipeline
    with pytest.raises(ValueError, match="v0 is required"):
        pipeline._check_f32_cuda(None, "v0")
    with pytest.raises(ValueError, match="CUDA tensor"):
        pipeline._check_f32_cuda(torch.zeros(2, 4, 4), "factors")


def test_residual_columns_follow_the_passes():
    from inverse_root_preconditioning_amd import pipeline
    assert pipeline.residual_columns(4, capi.NDB, 10) == 20
    assert pipeline.residual_columns(4, capi.NDB_Z | capi.SYM_COUPLING, 7) == 14
    assert pipeline.residual_columns(2, capi.NDB, 10) == 10
    assert pipeline.residual_columns(4, capi.CN | capi.FULL_PRODUCTS, 12) == 12
    assert pipeline.residual_columns(8, capi.CN_F16, 5) == 5


def test_noalloc_graft_rejects_oversized_problems_without_gpu():
    """The allocation-free grafting call refuses, before any HIP call, a problem
    whose partial norms exceed its static scratch (1 MiB: 8192 blocks at
    B = 1024, whose 16 row chunks take 128 bytes per block)."""
    f = capi
    args = (FAKE, FAKE, FAKE, FAKE, FAKE)
    limit = f.NOALLOC_SCRATCH_BYTES // 128
    assert f.shampoo_graft_update_noalloc(*args, limit + 1, 1024, 1e-3, 0.9, 0.95, 1e-8, 1, 0, 0) == f.ESCRATCH
    assert "static scratch" in f.shampoo_strerror(f.ESCRATCH)
    assert f.shampoo_graft_update_noalloc(*args, 3, 1024, 1e-3, 0.9, 0.95, 1e-8, 0, 0, 0) == f.EINVAL  # step 0
    assert f.shampoo_graft_update_noalloc(0, 0, 0, 0, 0, 0, 1024, 1e-3, 0.9, 0.95, 1e-8, 1, 0, 0) == f.OK
