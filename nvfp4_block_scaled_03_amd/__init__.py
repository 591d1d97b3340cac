"""NVFP4 mixture-of-experts expert path for AMD Instinct MI355X (gfx950).

The compute lives in ``libnvfp4moe.so`` (HIP kernels behind the C ABI in
``include/nvfp4_moe.h``); ``ops`` marshals torch tensors into it.  Build the
library with ``python -m nvfp4_block_scaled_03_amd.build``.
"""
from ._lib import LIB_PATH, LibraryNotBuilt, Nvfp4Error  # noqa: F401

__all__ = ["LIB_PATH", "LibraryNotBuilt", "Nvfp4Error"]
