"""DFlash draft step (fusion + KV injection, block-diffusion draft, verify) on MI355X.

The compute lives in libdflash.so (HIP for gfx950, C ABI in include/dflash.h); the
Python side is a ctypes binding that marshals torch device tensors.
"""
from . import binding  # noqa: F401
from .binding import (Drafter, DflashError, PagedCache, load_library,  # noqa: F401
                      make_config)
