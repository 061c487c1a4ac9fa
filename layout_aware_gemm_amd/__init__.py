"""layout_aware_gemm_amd -- MI355X (gfx950) layout-aware bf16 GEMM library.

The computation lives in the HIP C-ABI library ``_lib/libtgemm.so`` (sources
in ``csrc/``, interface in ``include/tgemm.h``); ``tgemm`` is its ctypes
binding.  Importing this package does not load the library; the first call
does, and raises if it has not been built.
"""

from . import tgemm  # noqa: F401
from .tgemm import (  # noqa: F401
    TgemmError,
    cross_entropy,
    layout_of,
    matmul,
    outer_f32,
    rope_cos_sin,
    run,
    set_tile_config,
    validate,
)
