"""PATCH hybrid dense / 2:4 tile GEMM for MI355X (gfx950).

The compute path is the C-ABI library ``libpatch.so`` (HIP kernels); this
package is a thin ctypes binding over it.  Importing the package does not load
the library; the first call does, and fails loudly if it is missing.
"""
__all__ = ["pack", "gemm_grouped", "import_packed", "sample_mask", "mask_unpack", "PackedWeight", "PatchError", "lib_path",
           "checkpoint"]


def __getattr__(name):
    import importlib
    if name == "checkpoint":
        return importlib.import_module(".checkpoint", __name__)
    if name in __all__:
        return getattr(importlib.import_module(".api", __name__), name)
    raise AttributeError(name)
