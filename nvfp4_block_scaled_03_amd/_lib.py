"""ctypes loader for libnvfp4moe.so (the C ABI in include/nvfp4_moe.h).

The library is loaded on first use.  If it is missing the call raises
``LibraryNotBuilt``: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_char_p, c_int, c_int32, c_int64, c_size_t, c_void_p

# NVFP4_MOE_LIB may point at another build of the same library (e.g. a
# variant with different tile settings); the default is the in-tree build.
LIB_PATH = os.environ.get("NVFP4_MOE_LIB") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libnvfp4moe.so")
ABI_VERSION = 9

NVFP4_OK = 0
NVFP4_EINVAL = -1
NVFP4_ESHAPE = -2
NVFP4_EWORKSPACE = -3
NVFP4_ELAUNCH = -4
NVFP4_BF16 = 0
NVFP4_F32 = 1


class Dims(ctypes.Structure):
    _fields_ = [("T", c_int32), ("topk", c_int32), ("E", c_int32), ("H", c_int32),
                ("I", c_int32), ("shared", c_int32)]

    def __repr__(self):
        return "Dims(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


_P = ctypes.POINTER(Dims)

# name -> (restype, argtypes); every symbol include/nvfp4_moe.h declares.
SIGNATURES = {
    "nvfp4_abi_version": (c_int, []),
    "nvfp4_last_error": (c_char_p, []),
    "nvfp4_global_scale_workspace_size": (c_size_t, [c_int64, c_int64]),
    "nvfp4_global_scale": (c_int, [c_void_p, c_int, c_int64, c_int64, c_void_p, c_void_p,
                                   c_size_t, c_void_p]),
    "nvfp4_quantize": (c_int, [c_void_p, c_int, c_int64, c_int64, c_int64, c_void_p, c_int64,
                               c_void_p, c_void_p, c_void_p, c_void_p]),
    "moe_route_topk": (c_int, [c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p]),
    "moe_align_workspace_size": (c_size_t, [_P]),
    "moe_align_plan_size": (c_size_t, [_P]),
    "moe_align": (c_int, [_P, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                          c_void_p]),
    "moe_scale_and_align": (c_int, [_P, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p, c_void_p,
                                    c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "moe_route_and_align": (c_int, [_P, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                    c_void_p, c_void_p, c_size_t, c_void_p]),
    "moe_quantize_and_align": (c_int, [_P, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p, c_void_p,
                                       c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                       c_void_p, c_size_t, c_void_p]),
    "nvfp4_linear_workspace_size": (c_size_t, [c_int64, c_int64, c_int64, c_int]),
    "nvfp4_linear": (c_int, [c_void_p, c_int64, c_int64, c_int64, c_void_p, c_void_p, c_void_p, c_int,
                             c_void_p, c_size_t, c_void_p]),
    "nvfp4_linear_w4a16": (c_int, [c_void_p, c_int64, c_int64, c_int64, c_void_p, c_void_p, c_void_p,
                                   c_int, c_void_p, c_size_t, c_void_p]),
    "mxfp4_quantize": (c_int, [c_void_p, c_int, c_int64, c_int64, c_int64, c_void_p, c_void_p, c_void_p]),
    "mxfp4_prep_weights_size": (c_size_t, [c_int64, c_int64]),
    "mxfp4_prep_weights": (c_int, [c_int64, c_int64, c_void_p, c_void_p, c_void_p, c_void_p]),
    "mxfp4_linear_workspace_size": (c_size_t, [c_int64, c_int64, c_int64]),
    "mxfp4_linear": (c_int, [c_void_p, c_int64, c_int64, c_int64, c_void_p, c_void_p, c_int, c_void_p,
                             c_size_t, c_void_p]),
    "nvfp4_prep_weights_size": (c_size_t, [_P, c_int]),
    "nvfp4_prep_weights": (c_int, [_P, c_int, c_void_p, c_void_p, c_void_p, c_void_p]),
    "grouped_gemm_prefers_decoded": (c_int, [_P]),
    "grouped_gemm_workspace_size": (c_size_t, [_P]),
    "grouped_gemm1_swiglu": (c_int, [_P, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                     c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                     c_void_p, c_void_p, c_void_p]),
    "grouped_gemm2_combine": (c_int, [_P, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                      c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                      c_int, c_void_p, c_size_t, c_void_p]),
    "grouped_gemm1_swiglu_w4a16": (c_int, [_P, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                           c_void_p, c_void_p, c_void_p]),
    "grouped_gemm2_combine_w4a16": (c_int, [_P, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                            c_void_p, c_void_p, c_void_p, c_int, c_void_p,
                                            c_size_t, c_void_p]),
    "mxfp4_prep_expert_weights_size": (c_size_t, [_P, c_int]),
    "mxfp4_prep_expert_weights": (c_int, [_P, c_int, c_void_p, c_void_p, c_void_p, c_void_p]),
    "grouped_gemm1_swiglu_mxfp4": (c_int, [_P, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                           c_void_p, c_void_p, c_void_p]),
    "grouped_gemm2_combine_mxfp4": (c_int, [_P, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                            c_void_p, c_void_p, c_int, c_void_p, c_size_t, c_void_p]),
    "moe_mxfp4_quantize_and_align": (c_int, [_P, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                             c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "grouped_gemm2_combine_noalloc_max_bytes": (c_size_t, []),
    "grouped_gemm2_combine_noalloc": (c_int, [_P, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                              c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                              c_void_p, c_int, c_void_p]),
    "grouped_gemm_runs_in_parts": (c_int, [_P]),
}
# The *_part calls: the named call's arguments with int part before the stream.
for _name in ("grouped_gemm1_swiglu", "grouped_gemm2_combine", "grouped_gemm1_swiglu_w4a16",
              "grouped_gemm2_combine_w4a16", "grouped_gemm1_swiglu_mxfp4", "grouped_gemm2_combine_mxfp4"):
    _res, _args = SIGNATURES[_name]
    SIGNATURES[_name + "_part"] = (_res, _args[:-1] + [c_int, c_void_p])


class LibraryNotBuilt(RuntimeError):
    pass


class Nvfp4Error(RuntimeError):
    def __init__(self, name: str, code: int, message: str):
        super().__init__(f"{name} returned {code}: {message}")
        self.code = code
        self.message = message


_lib = None


def load(path: str = LIB_PATH):
    """Load the library (once) and attach signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise LibraryNotBuilt(
            f"{path} is missing: build it with `python -m nvfp4_block_scaled_03_amd.build` "
            "(or __graft_entry__.build()); there is no non-HIP fallback")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    v = lib.nvfp4_abi_version()
    if v != ABI_VERSION:
        raise LibraryNotBuilt(f"{path}: ABI version {v}, expected {ABI_VERSION}; rebuild")
    _lib = lib
    return lib


def last_error() -> str:
    return load().nvfp4_last_error().decode()


def call(name: str, *args) -> int:
    """Call a status-returning entry point; raise Nvfp4Error on failure."""
    lib = load()
    rc = getattr(lib, name)(*args)
    if rc != NVFP4_OK:
        raise Nvfp4Error(name, rc, last_error())
    return rc
