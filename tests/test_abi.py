"""Host-side checks of the C ABI (CPU only: no kernel is launched).

The library must load, export every function include/nvfp4_moe.h declares,
answer the size queries, and reject bad arguments with the documented status
codes before touching the GPU.
"""
import ctypes
import os
import re

import pytest

from nvfp4_block_scaled_03_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "nvfp4_moe.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("library not built (run __graft_entry__.build())")
    return _lib.load()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"^[a-z_ ]+[ *]+([a-z0-9_]+)\s*\(", text, flags=re.M))


def test_header_symbols_exported(lib):
    names = _declared()
    assert len(names) >= 16
    assert names == set(_lib.SIGNATURES), names ^ set(_lib.SIGNATURES)
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version(lib):
    assert lib.nvfp4_abi_version() == _lib.ABI_VERSION


def _d(T=64, topk=8, E=128, H=2048, I=768, shared=0):
    return _lib.Dims(T, topk, E, H, I, shared)


def test_size_queries(lib):
    d = _d()
    P = 64 * 8
    assert lib.grouped_gemm_workspace_size(ctypes.byref(d)) == P * 2048 * 4
    # The streaming layout is a permutation of the canonical bytes.
    assert lib.nvfp4_prep_weights_size(ctypes.byref(d), 13) == 128 * 1536 * (1024 + 128)
    assert lib.nvfp4_prep_weights_size(ctypes.byref(d), 2) == 128 * 2048 * (384 + 48)
    assert lib.nvfp4_prep_weights_size(ctypes.byref(d), 5) == 0
    # per-chunk expert counts, then 1024 partial maxima of the fused global
    # scale
    assert lib.moe_align_workspace_size(ctypes.byref(d)) == 1 * 128 * 4 + 1024 * 4
    d4k = _d(T=4096)
    assert lib.moe_align_workspace_size(ctypes.byref(d4k)) == 32 * 128 * 4 + 1024 * 4
    plan = lib.moe_align_plan_size(ctypes.byref(d))
    # six tile lists (heights 16, 32, 64, 128; then 16 and 128 for the experts
    # with at most / more than 32 rows), each with room for one partial tile
    # per expert that can appear in it
    lens = [(P + bm - 1) // bm + 128 for bm in (16, 32, 64, 128, 16)] + [(P + 127) // 128 + min(128, P // 33)]
    assert plan == 4 * (12 + sum(2 * n for n in lens))
    assert lib.nvfp4_global_scale_workspace_size(1, 64 * 2048) == 8
    assert lib.nvfp4_global_scale_workspace_size(4, 1 << 22) == 4 * 8
    ds = _d(T=256, topk=10, E=512, H=4096, I=1024, shared=1)
    assert lib.grouped_gemm_workspace_size(ctypes.byref(ds)) == (2560 + 256) * 4096 * 4


@pytest.mark.parametrize("dims,code,frag", [
    (dict(H=2000), _lib.NVFP4_ESHAPE, "multiples of 128"),
    (dict(I=700), _lib.NVFP4_ESHAPE, "multiples of 128"),
    (dict(topk=0), _lib.NVFP4_ESHAPE, "topk=0"),
    (dict(topk=200), _lib.NVFP4_ESHAPE, "num_experts=128"),
    (dict(E=1024, shared=1), _lib.NVFP4_ESHAPE, "exceeds 1024"),
    (dict(shared=2), _lib.NVFP4_ESHAPE, "shared=2"),
    (dict(T=-1), _lib.NVFP4_ESHAPE, "T=-1"),
    (dict(T=1 << 22), _lib.NVFP4_ESHAPE, "exceeds 2^24"),
])
def test_dims_rejected(lib, dims, code, frag):
    d = _d(**dims)
    rc = lib.moe_align(ctypes.byref(d), None, None, None, None, None, None, 0, None)
    assert rc == code
    assert frag in _lib.last_error() and _lib.last_error().startswith("moe_align:")
    rc = lib.grouped_gemm1_swiglu(ctypes.byref(d), *([None] * 13), None)
    assert rc == code


def test_null_and_enum_errors(lib):
    assert lib.nvfp4_quantize(None, 7, 1, 16, 16, None, 1, None, None, None, None) == _lib.NVFP4_EINVAL
    assert "dtype=7" in _lib.last_error()
    assert lib.nvfp4_quantize(None, 0, 4, 24, 24, None, 1, None, None, None, None) == _lib.NVFP4_ESHAPE
    assert lib.nvfp4_quantize(None, 0, 4, 32, 36, None, 1, None, None, None, None) == _lib.NVFP4_ESHAPE
    assert lib.nvfp4_quantize(None, 0, 4, 32, 32, None, 1, None, None, None, None) == _lib.NVFP4_EINVAL
    assert lib.nvfp4_global_scale(None, 0, 1, 12, None, None, 0, None) == _lib.NVFP4_ESHAPE
    assert lib.moe_route_topk(None, 4, 8, 9, None, None, None) == _lib.NVFP4_ESHAPE
    assert lib.moe_route_topk(None, 4, 2048, 4, None, None, None) == _lib.NVFP4_ESHAPE
    d = _d()
    assert lib.nvfp4_prep_weights(ctypes.byref(d), 7, None, None, None, None) == _lib.NVFP4_EINVAL


def test_gemm2_errors_name_the_problem(lib):
    d = _d()
    rc = lib.grouped_gemm2_combine(ctypes.byref(d), *([None] * 10), None, 0, None, 0, None)
    assert rc == _lib.NVFP4_EWORKSPACE
    msg = _lib.last_error()
    for f in ("num_experts=128", "M=512", "N=2048", "K=768", "workspace_size=0"):
        assert f in msg, msg
    rc = lib.grouped_gemm2_combine(ctypes.byref(d), *([None] * 10), None, 5, None, 0, None)
    assert rc == _lib.NVFP4_EINVAL and "out_dtype=5" in _lib.last_error()


@pytest.mark.parametrize("shared", [0, 1])
def test_zero_tokens_is_a_noop(lib, shared):
    """T == 0: every layer call checks dims and returns OK without launching
    (no stream is touched, so NULL pointers are fine) -- also the fused
    activation + permutation calls."""
    d = _d(T=0, shared=shared)
    r = ctypes.byref(d)
    assert lib.grouped_gemm1_swiglu(r, *([None] * 13), None) == _lib.NVFP4_OK
    assert lib.grouped_gemm1_swiglu_w4a16(r, *([None] * 7), None) == _lib.NVFP4_OK
    assert lib.grouped_gemm2_combine(r, *([None] * 10), None, 0, None, 0, None) == _lib.NVFP4_OK
    assert lib.grouped_gemm2_combine_w4a16(r, *([None] * 7), None, 0, None, 0, None) == _lib.NVFP4_OK
    assert lib.moe_align(r, *([None] * 6), 0, None) == _lib.NVFP4_OK
    assert lib.moe_scale_and_align(r, *([None] * 3), 0, *([None] * 6), 0, None) == _lib.NVFP4_OK
    assert lib.moe_route_and_align(r, *([None] * 8), 0, None) == _lib.NVFP4_OK
    assert lib.moe_quantize_and_align(r, None, None, None, 0, *([None] * 9), 0, None) == _lib.NVFP4_OK
    assert lib.moe_mxfp4_quantize_and_align(r, *([None] * 8), None, 0, None) == _lib.NVFP4_OK
    assert lib.nvfp4_quantize(None, 0, 0, 32, 32, None, 1, None, None, None, None) == _lib.NVFP4_OK
    assert lib.moe_route_topk(None, 0, 8, 2, None, None, None) == _lib.NVFP4_OK
    assert lib.grouped_gemm1_swiglu_mxfp4(r, *([None] * 8), None) == _lib.NVFP4_OK
    assert lib.grouped_gemm2_combine_mxfp4(r, *([None] * 7), None, 0, None, 0, None) == _lib.NVFP4_OK
    assert _lib.last_error() == ""
    # bad dims are still rejected at T == 0
    bad = _d(T=0, H=100)
    assert lib.moe_quantize_and_align(ctypes.byref(bad), None, None, None, 0, *([None] * 9), 0,
                                      None) == _lib.NVFP4_ESHAPE


def test_route_and_align_errors(lib):
    d = _d()
    args = [None] * 8 + [0, None]
    rc = lib.moe_route_and_align(ctypes.byref(d), *args)
    assert rc == _lib.NVFP4_EINVAL and _lib.last_error().startswith("moe_route_and_align:")
    d = _d(topk=40)
    rc = lib.moe_route_and_align(ctypes.byref(d), *args)
    assert rc == _lib.NVFP4_ESHAPE and "topk=40" in _lib.last_error()


def test_linear_size_and_errors(lib):
    assert lib.nvfp4_linear_workspace_size(64, 2048, 768, 1) > 64 * 768 // 2
    assert lib.nvfp4_linear_workspace_size(64, 2048, 768, 0) > 0
    assert lib.nvfp4_linear_workspace_size(64, 2000, 768, 1) == 0
    rc = lib.nvfp4_linear(None, 64, 2000, 768, None, None, None, 0, None, 0, None)
    assert rc == _lib.NVFP4_ESHAPE and "N=2000" in _lib.last_error()
    rc = lib.nvfp4_linear_w4a16(None, 64, 2048, 768, None, None, None, 0, None, 0, None)
    assert rc == _lib.NVFP4_EWORKSPACE and "M=64" in _lib.last_error()
    rc = lib.nvfp4_linear(None, 64, 2048, 768, None, None, None, 7, None, 0, None)
    assert rc == _lib.NVFP4_EINVAL and "out_dtype=7" in _lib.last_error()


def test_quantize_and_align_errors(lib):
    d = _d()
    # null outputs are rejected before anything is launched
    args = [None, None, None, 0] + [None] * 9 + [0, None]
    rc = lib.moe_quantize_and_align(ctypes.byref(d), *args)
    assert rc == _lib.NVFP4_EINVAL and _lib.last_error().startswith("moe_quantize_and_align:")
    d = _d(H=2000)
    rc = lib.moe_quantize_and_align(ctypes.byref(d), *args)
    assert rc == _lib.NVFP4_ESHAPE and "multiples of 128" in _lib.last_error()


def test_mx_quantize_and_align_errors(lib):
    """Validation before any launch: null operands, misaligned x or codes,
    a workspace below moe_align_workspace_size, bad dims, T*H >= 2^31."""
    d = _d()
    r = ctypes.byref(d)
    assert lib.moe_mxfp4_quantize_and_align(r, *([None] * 8), None, 0, None) == _lib.NVFP4_EINVAL
    assert _lib.last_error().startswith("moe_mxfp4_quantize_and_align:")
    ok = [ctypes.c_void_p(256)] * 8
    ws = lib.moe_align_workspace_size(r)
    bad_x = list(ok)
    bad_x[0] = ctypes.c_void_p(256 + 8)
    assert lib.moe_mxfp4_quantize_and_align(r, *bad_x, ctypes.c_void_p(256), ws, None) == _lib.NVFP4_EINVAL
    assert "misaligned" in _lib.last_error()
    bad_q = list(ok)
    bad_q[1] = ctypes.c_void_p(256 + 2)
    assert lib.moe_mxfp4_quantize_and_align(r, *bad_q, ctypes.c_void_p(256), ws, None) == _lib.NVFP4_EINVAL
    rc = lib.moe_mxfp4_quantize_and_align(r, *ok, ctypes.c_void_p(256), ws - 4, None)
    assert rc == _lib.NVFP4_EWORKSPACE and "workspace_size" in _lib.last_error()
    dh = _d(H=2000)
    rc = lib.moe_mxfp4_quantize_and_align(ctypes.byref(dh), *ok, ctypes.c_void_p(256), ws, None)
    assert rc == _lib.NVFP4_ESHAPE and "multiples of 128" in _lib.last_error()
    big = _d(T=1 << 16, H=1 << 15)
    rc = lib.moe_mxfp4_quantize_and_align(ctypes.byref(big), *ok, ctypes.c_void_p(256), 1 << 30, None)
    assert rc == _lib.NVFP4_ESHAPE and "too large" in _lib.last_error()


def test_mxfp4_sizes_and_errors(lib):
    assert lib.mxfp4_prep_weights_size(256, 512) == 256 * 256 + 256 * 16
    assert lib.mxfp4_prep_weights_size(200, 512) == 0
    assert lib.mxfp4_linear_workspace_size(3, 256, 512) == 64 * 256 + 64 * 16   # rows padded to 64
    assert lib.mxfp4_linear_workspace_size(100, 256, 512) == 128 * 256 + 128 * 16   # to one 128-row tile
    assert lib.mxfp4_linear_workspace_size(130, 256, 512) == 256 * 256 + 256 * 16   # to whole 256-row tiles
    assert lib.mxfp4_quantize(None, 2, 4, 32, 32, None, None, None) == _lib.NVFP4_EINVAL
    assert lib.mxfp4_quantize(None, 0, 4, 48, 48, None, None, None) == _lib.NVFP4_ESHAPE
    assert lib.mxfp4_quantize(None, 0, 4, 32, 36, None, None, None) == _lib.NVFP4_ESHAPE
    assert lib.mxfp4_quantize(None, 0, 0, 32, 32, None, None, None) == _lib.NVFP4_OK
    assert lib.mxfp4_quantize(None, 0, 4, 32, 32, None, None, None) == _lib.NVFP4_EINVAL
    assert lib.mxfp4_prep_weights(256, 100, None, None, None, None) == _lib.NVFP4_ESHAPE
    rc = lib.mxfp4_linear(None, 8, 256, 512, None, None, 0, None, 0, None)
    assert rc == _lib.NVFP4_EWORKSPACE and "M=8" in _lib.last_error()
    rc = lib.mxfp4_linear(None, 8, 256, 512, None, None, 3, None, 0, None)
    assert rc == _lib.NVFP4_EINVAL and "out_dtype=3" in _lib.last_error()
    assert lib.mxfp4_linear(None, 0, 256, 512, None, None, 0, None, 0, None) == _lib.NVFP4_OK
    rc = lib.mxfp4_linear(None, 8, 1 << 20, 1 << 14, None, None, 0, None, 0, None)
    assert rc == _lib.NVFP4_ESHAPE and "4 GiB" in _lib.last_error()


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(_lib.LibraryNotBuilt):
        old = _lib._lib
        _lib._lib = None
        try:
            _lib.load(str(tmp_path / "nope.so"))
        finally:
            _lib._lib = old


def test_mx_layer_errors(lib):
    """The MXFP4 layer calls validate before launching: missing or misaligned
    operands are rejected with the GEMM's shape in the message, prep needs
    MX-sized blocks, and the 2^31 operand-offset limit is checked."""
    d = _d()
    r = ctypes.byref(d)
    assert lib.mxfp4_prep_expert_weights_size(r, 13) > 0
    assert lib.mxfp4_prep_expert_weights_size(r, 7) == 0
    assert lib.grouped_gemm1_swiglu_mxfp4(r, *([None] * 8), None) == _lib.NVFP4_EINVAL
    assert "grouped_gemm1_swiglu_mxfp4" in _lib.last_error()
    # every pointer present but a2 codes misaligned
    p = [ctypes.c_void_p(256)] * 8
    p[6] = ctypes.c_void_p(256 + 4)
    assert lib.grouped_gemm1_swiglu_mxfp4(r, *p, None) == _lib.NVFP4_EINVAL
    # GEMM2: the workspace size is checked first, then the operands
    assert lib.grouped_gemm2_combine_mxfp4(r, *([None] * 7), None, 0, None, 0, None) == _lib.NVFP4_EWORKSPACE
    ws = lib.grouped_gemm_workspace_size(r)
    assert lib.grouped_gemm2_combine_mxfp4(r, *([None] * 7), None, 0, ctypes.c_void_p(256), ws,
                                           None) == _lib.NVFP4_EINVAL
    big = _d(T=1 << 17, H=1 << 15)
    assert lib.grouped_gemm1_swiglu_mxfp4(ctypes.byref(big), *([None] * 8), None) == _lib.NVFP4_ESHAPE


def test_parts_query_and_errors(lib):
    """grouped_gemm_runs_in_parts says which dims split their GEMMs (short
    tiles on average with an expert that can exceed 64 rows); a part outside
    0..2 (GEMM1) or 0..3 (GEMM2) is rejected before anything else, naming
    the *_part call; a valid part reaches the named call's own checks."""
    assert lib.grouped_gemm_runs_in_parts(ctypes.byref(_d())) == 0            # decode: 4 rows per expert
    large_e = _d(T=256, topk=10, E=512, H=4096, I=1024, shared=1)
    assert lib.grouped_gemm_runs_in_parts(ctypes.byref(large_e)) == 1
    assert lib.grouped_gemm_runs_in_parts(ctypes.byref(_d(T=4096))) == 0      # tall tiles on average
    assert lib.grouped_gemm_runs_in_parts(ctypes.byref(_d(E=0))) == 0         # invalid dims
    r = ctypes.byref(_d())
    for part in (-1, 3):
        assert lib.grouped_gemm1_swiglu_part(r, *([None] * 13), part, None) == _lib.NVFP4_EINVAL
        assert f"grouped_gemm1_swiglu_part: EINVAL part={part}" in _lib.last_error()
        assert lib.grouped_gemm1_swiglu_w4a16_part(r, *([None] * 7), part, None) == _lib.NVFP4_EINVAL
        assert lib.grouped_gemm1_swiglu_mxfp4_part(r, *([None] * 8), part, None) == _lib.NVFP4_EINVAL
    for part in (-1, 4):
        assert lib.grouped_gemm2_combine_part(r, *([None] * 10), None, 0, None, 0, part, None) == _lib.NVFP4_EINVAL
        assert f"grouped_gemm2_combine_part: EINVAL part={part}" in _lib.last_error()
        assert lib.grouped_gemm2_combine_w4a16_part(r, *([None] * 7), None, 0, None, 0, part,
                                                    None) == _lib.NVFP4_EINVAL
        assert lib.grouped_gemm2_combine_mxfp4_part(r, *([None] * 7), None, 0, None, 0, part,
                                                    None) == _lib.NVFP4_EINVAL
    # valid parts: the named call's checks (missing workspace, missing operands)
    assert lib.grouped_gemm2_combine_part(r, *([None] * 10), None, 0, None, 0, 3, None) == _lib.NVFP4_EWORKSPACE
    assert "grouped_gemm2_combine_part: EWORKSPACE" in _lib.last_error()
    assert lib.grouped_gemm1_swiglu_part(r, *([None] * 13), 2, None) == _lib.NVFP4_EINVAL
    assert "grouped_gemm1_swiglu_part: EINVAL null" in _lib.last_error()
