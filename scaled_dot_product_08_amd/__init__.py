"""MI355X (gfx950) fused multi-head attention forward.

The compute path is the HIP library ``lib/libsdpa08.so`` (C ABI in
include/attn.h); this package only binds it (``binding``), builds it
(``build``) and defines the benchmark's work accounting (``accounting``).
"""
from .binding import (  # noqa: F401
    ATTN_DTYPE_BF16,
    ATTN_DTYPE_FP16,
    AttnError,
    attn_fwd,
    attn_strerror,
    attn_version,
    fwd,
    load_library,
)
