"""MI355X (gfx950) DSpark sequential head: HIP kernels behind a C ABI.

`binding` mirrors include/dspark.h one to one; `ops` wraps it for torch
tensors that already live on the GPU.  Build the library with `build.build()`.
"""
from . import binding  # noqa: F401
