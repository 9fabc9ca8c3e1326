"""MI355X-native (gfx950) forward kernels for the DeepSeek-V4-Flash compressed
attention layer (CSA / HCA / sliding window), behind a C-ABI library.

`workloads` holds the shapes and the seeded input generator; `binding` loads the HIP
library (libcsa.so) and marshals arguments into its C entry points.  Submodules are
imported on use, so the generator works without the built library.
"""
import importlib

__all__ = ["workloads", "binding"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
