"""MI355X (gfx950) mixed chunked-prefill + decode paged attention.

The library is libca.so (C ABI in include/ca.h); `binding` marshals arguments to it with ctypes.
`workload` draws seeded synthetic inputs and `accounting` counts algorithmic bytes and flops.
"""
from .binding import (PROFILE_ALL, PROFILE_APPEND, PROFILE_ATTENTION, PROFILE_MERGE,  # noqa: F401
                      PROFILE_UPLOAD, CaError, Context, Plan, RequestBatch, create, destroy,
                      header_symbols, lib, make_desc, plan_batch)
