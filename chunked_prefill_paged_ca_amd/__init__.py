"""MI355X (gfx950) mixed chunked-prefill + decode paged attention.

The library is libca.so (C ABI in include/ca.h); `binding` marshals arguments to it with ctypes.
`workload` draws seeded synthetic inputs and `accounting` counts algorithmic bytes and flops.
"""
from .binding import (CaError, Context, Plan, RequestBatch, create, destroy, header_symbols, lib,  # noqa: F401
                      make_desc, plan_batch)
