"""MI355X (gfx950) mixed chunked-prefill + decode paged attention.

The library is libca.so (C ABI in include/ca.h); `binding` marshals arguments to it with ctypes.
`workload` draws seeded synthetic inputs and `accounting` counts algorithmic bytes and flops.
"""
from .binding import (CA_REQ_FINISHED, CA_REQ_RUNNING, CA_REQ_WAITING,  # noqa: F401
                      PROFILE_ALL, PROFILE_APPEND, PROFILE_ATTENTION, PROFILE_MERGE, PROFILE_PROJECTION,
                      PROFILE_UPLOAD, CaError, Context, Plan, RequestBatch, Scheduler, create,
                      destroy, header_symbols, lib, make_desc, plan_batch)
