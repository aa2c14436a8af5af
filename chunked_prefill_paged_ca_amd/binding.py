"""ctypes binding over the C ABI of include/ca.h (argument marshalling only).

Every step of the path runs in libca.so: the plan on the host, the append and attention in HIP
kernels.  PyTorch tensors are accepted as device buffers (their data_ptr) and torch's current
stream is used by default; nothing here computes.  If libca.so is missing this module raises:
there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import List, Optional, Sequence

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libca.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "ca.h")

(CA_OK, CA_ERR_INVALID_ARG, CA_ERR_NO_PAGES, CA_ERR_CAPACITY, CA_ERR_UNSUPPORTED, CA_ERR_DEVICE,
 CA_ERR_INTERNAL) = range(7)
CA_REQ_WAITING, CA_REQ_RUNNING, CA_REQ_FINISHED = 0, 1, 2
CA_BF16, CA_FP32 = 0, 1

_i32p = ctypes.POINTER(ctypes.c_int32)


class CaRequest(ctypes.Structure):
    _fields_ = [("num_computed", ctypes.c_int32), ("num_prompt_left", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("block_table", _i32p)]


class CaPlanParams(ctypes.Structure):
    _fields_ = [("token_budget", ctypes.c_int32), ("max_chunk", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("chunk_align", ctypes.c_int32),
                ("num_pool_pages", ctypes.c_int64)]


class CaPlan(ctypes.Structure):
    _fields_ = [("cap_seqs", ctypes.c_int32), ("cap_pages", ctypes.c_int32),
                ("req_ids", _i32p), ("qo_indptr", _i32p), ("kv_page_indptr", _i32p),
                ("kv_page_indices", _i32p), ("kv_last_page_len", _i32p),
                ("num_seqs", ctypes.c_int32), ("num_decodes", ctypes.c_int32),
                ("num_tokens", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("num_deferred_decodes", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("generation", ctypes.c_uint64)]


class CaAttnDesc(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("sm_scale", ctypes.c_float),
                ("rope_theta", ctypes.c_float)]


class CaSchedRequest(ctypes.Structure):
    _fields_ = [("state", ctypes.c_int32), ("num_computed", ctypes.c_int32),
                ("num_prompt_left", ctypes.c_int32), ("num_generated", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("num_preemptions", ctypes.c_int32),
                ("block_table", _i32p)]


class CaProfileRecord(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_char_p), ("ms", ctypes.c_float)]


PROFILE_ALL, PROFILE_UPLOAD, PROFILE_APPEND, PROFILE_ATTENTION, PROFILE_MERGE = 1, 2, 4, 8, 16
PROFILE_PROJECTION = 32
VALIDATE_WRITE_TARGETS = 1


class CaError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status} ({status_string(status)}): {detail}")
        self.status = status


_LIB = None


def lib() -> ctypes.CDLL:
    """Load libca.so (built in-tree by chunked_prefill_paged_ca_amd.build)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run chunked_prefill_paged_ca_amd/build.py "
                              "(there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        vp = ctypes.c_void_p
        L.ca_create.argtypes = [ctypes.c_int, ctypes.POINTER(vp)]
        L.ca_destroy.argtypes = [vp]
        L.ca_plan_batch.argtypes = [ctypes.POINTER(CaRequest), ctypes.c_int32,
                                    ctypes.POINTER(CaPlanParams), ctypes.POINTER(CaPlan)]
        L.ca_append_kv_rope.argtypes = [vp, ctypes.POINTER(CaAttnDesc), ctypes.POINTER(CaPlan),
                                        vp, vp, vp, vp, vp, vp, ctypes.c_int64, vp]
        L.ca_mixed_attention.argtypes = [vp, ctypes.POINTER(CaAttnDesc), ctypes.POINTER(CaPlan),
                                         vp, vp, vp, ctypes.c_int64, vp, vp, vp]
        L.ca_mixed_attention_noalloc.argtypes = [vp, ctypes.POINTER(CaAttnDesc), ctypes.POINTER(CaPlan),
                                                 vp, vp, vp, ctypes.c_int64, vp, vp, vp]
        L.ca_append_kv_rope_packed.argtypes = [vp, ctypes.POINTER(CaAttnDesc), ctypes.POINTER(CaPlan),
                                               vp, vp, vp, vp, ctypes.c_int64, vp]
        L.ca_qkv_projection.argtypes = [vp, ctypes.POINTER(CaAttnDesc), ctypes.c_int32, ctypes.c_int32,
                                        vp, vp, vp, vp]
        L.ca_plan_validate.argtypes = [ctypes.POINTER(CaPlan), ctypes.c_int64, ctypes.c_int32]
        L.ca_profile_enable.argtypes = [vp, ctypes.c_int]
        L.ca_profile_read.argtypes = [vp, ctypes.POINTER(CaProfileRecord), ctypes.c_int32,
                                      ctypes.POINTER(ctypes.c_int32)]
        L.ca_sched_create.argtypes = [ctypes.POINTER(CaPlanParams), ctypes.POINTER(vp)]
        L.ca_sched_destroy.argtypes = [vp]
        L.ca_sched_add.argtypes = [vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _i32p,
                                   ctypes.POINTER(ctypes.c_int32)]
        L.ca_sched_step.argtypes = [vp, ctypes.POINTER(CaPlan)]
        L.ca_sched_commit.argtypes = [vp]
        L.ca_sched_get.argtypes = [vp, ctypes.c_int32, ctypes.POINTER(CaSchedRequest)]
        L.ca_sched_free_pages.argtypes = [vp]
        L.ca_sched_free_pages.restype = ctypes.c_int64
        for fn in ("ca_create", "ca_destroy", "ca_plan_batch", "ca_append_kv_rope",
                   "ca_mixed_attention", "ca_mixed_attention_noalloc", "ca_append_kv_rope_packed", "ca_qkv_projection",
                   "ca_plan_validate", "ca_profile_enable", "ca_profile_read", "ca_sched_create",
                   "ca_sched_destroy", "ca_sched_add", "ca_sched_step", "ca_sched_commit",
                   "ca_sched_get"):
            getattr(L, fn).restype = ctypes.c_int
        L.ca_status_string.argtypes = [ctypes.c_int]
        L.ca_status_string.restype = ctypes.c_char_p
        L.ca_last_error.argtypes = []
        L.ca_last_error.restype = ctypes.c_char_p
        _LIB = L
    return _LIB


def header_symbols() -> List[str]:
    """Every function the public header declares."""
    with open(HEADER, encoding="utf-8") as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ca_[a-z_]+)\s*\(", text)))


def status_string(status: int) -> str:
    return lib().ca_status_string(int(status)).decode()


def last_error() -> str:
    return lib().ca_last_error().decode()


def _check(status: int, where: str):
    if status != CA_OK:
        raise CaError(status, where, last_error())


# ---------------------------------------------------------------------------------------------
# Plan
# ---------------------------------------------------------------------------------------------

class Plan:
    """Owns the host arrays of one ca_plan and the ctypes struct pointing at them."""

    def __init__(self, cap_seqs: int, cap_pages: int):
        self.req_ids = np.zeros(max(cap_seqs, 1), dtype=np.int32)
        self.qo_indptr = np.zeros(cap_seqs + 1, dtype=np.int32)
        self.kv_page_indptr = np.zeros(cap_seqs + 1, dtype=np.int32)
        self.kv_page_indices = np.zeros(max(cap_pages, 1), dtype=np.int32)
        self.kv_last_page_len = np.zeros(max(cap_seqs, 1), dtype=np.int32)
        p = CaPlan()
        p.cap_seqs, p.cap_pages = cap_seqs, cap_pages
        for name in ("req_ids", "qo_indptr", "kv_page_indptr", "kv_page_indices",
                     "kv_last_page_len"):
            setattr(p, name, getattr(self, name).ctypes.data_as(_i32p))
        self.c = p
        self.status = None

    def __getattr__(self, name):
        if name in ("num_seqs", "num_decodes", "num_tokens", "num_pages",
                    "num_deferred_decodes", "page_size", "generation"):
            return getattr(self.c, name)
        raise AttributeError(name)

    def validate(self, num_pool_pages: int, write_targets: bool = False):
        """ca_plan_validate: raises CaError when the plan is inconsistent with the pool (or, with
        write_targets, when two scheduled tokens would append to the same page slot)."""
        _check(lib().ca_plan_validate(ctypes.byref(self.c), int(num_pool_pages),
                                      VALIDATE_WRITE_TARGETS if write_targets else 0),
               "ca_plan_validate")

    def arrays(self) -> dict:
        ns, npg = self.c.num_seqs, self.c.num_pages
        return {"req_ids": self.req_ids[:ns].copy(), "qo_indptr": self.qo_indptr[:ns + 1].copy(),
                "kv_page_indptr": self.kv_page_indptr[:ns + 1].copy(),
                "kv_page_indices": self.kv_page_indices[:npg].copy(),
                "kv_last_page_len": self.kv_last_page_len[:ns].copy()}


class Scheduler:
    """ca_sched: requests, the page pool's free list and one planned round at a time."""

    def __init__(self, token_budget: int, max_chunk: int, page_size: int, num_pool_pages: int,
                 chunk_align: int = 0):
        self.prm = CaPlanParams(int(token_budget), int(max_chunk), int(page_size), int(chunk_align),
                                int(num_pool_pages))
        h = ctypes.c_void_p()
        _check(lib().ca_sched_create(ctypes.byref(self.prm), ctypes.byref(h)), "ca_sched_create")
        self.h = h
        self.num_pool_pages = int(num_pool_pages)
        self.n = 0
        self._plan = None

    def close(self):
        if self.h:
            lib().ca_sched_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def add(self, prompt_len: int, max_new_tokens: int, num_cached: int = 0,
            cached_pages: Optional[np.ndarray] = None) -> int:
        rid = ctypes.c_int32()
        pages = None if cached_pages is None else np.ascontiguousarray(cached_pages, dtype=np.int32)
        ptr = pages.ctypes.data_as(_i32p) if pages is not None and pages.size else None
        if pages is not None and ptr is None:
            ptr = (ctypes.c_int32 * 1)()  # an empty prefix list, not "allocate for me"
        _check(lib().ca_sched_add(self.h, int(prompt_len), int(max_new_tokens), int(num_cached),
                                  ptr, ctypes.byref(rid)), "ca_sched_add")
        self.n += 1
        return int(rid.value)

    def step(self) -> Plan:
        """Plan the next round.  The returned Plan's arrays are reused by the next step()."""
        if self._plan is None or self._plan.c.cap_seqs < self.n:
            self._plan = Plan(max(2 * self.n, 16), self.num_pool_pages)
        plan = self._plan
        st = lib().ca_sched_step(self.h, ctypes.byref(plan.c))
        plan.status = st
        _check(st, "ca_sched_step")
        return plan

    def commit(self):
        _check(lib().ca_sched_commit(self.h), "ca_sched_commit")

    def get(self, rid: int) -> dict:
        r = CaSchedRequest()
        _check(lib().ca_sched_get(self.h, int(rid), ctypes.byref(r)), "ca_sched_get")
        table = (np.ctypeslib.as_array(r.block_table, shape=(r.num_pages,)).copy()
                 if r.num_pages > 0 else np.zeros(0, dtype=np.int32))
        return {"state": r.state, "num_computed": r.num_computed, "num_prompt_left": r.num_prompt_left,
                "num_generated": r.num_generated, "num_preemptions": r.num_preemptions,
                "block_table": table}

    def free_pages(self) -> int:
        return int(lib().ca_sched_free_pages(self.h))


class RequestBatch:
    """A ca_request array built once; plan() re-plans it with one library call.

    update(num_computed, num_prompt_left) refreshes the progress fields in place (block tables
    are fixed at construction).
    """

    def __init__(self, num_computed, num_prompt_left, block_tables, token_budget: int,
                 max_chunk: int, page_size: int, num_pool_pages: int, chunk_align: int = 0):
        n = len(num_computed)
        self.n = n
        self.tables = [np.ascontiguousarray(b, dtype=np.int32) for b in block_tables]
        self.reqs = (CaRequest * max(n, 1))()
        for i in range(n):
            self.reqs[i].num_pages = int(self.tables[i].shape[0])
            self.reqs[i].block_table = self.tables[i].ctypes.data_as(_i32p) if self.tables[i].size else None
        self.update(num_computed, num_prompt_left)
        self.prm = CaPlanParams(int(token_budget), int(max_chunk), int(page_size), int(chunk_align),
                                int(num_pool_pages))
        self.out = Plan(n, int(sum(t.shape[0] for t in self.tables)))

    def update(self, num_computed, num_prompt_left):
        for i in range(self.n):
            self.reqs[i].num_computed = int(num_computed[i])
            self.reqs[i].num_prompt_left = int(num_prompt_left[i])

    def plan(self) -> "Plan":
        st = lib().ca_plan_batch(self.reqs, self.n, ctypes.byref(self.prm), ctypes.byref(self.out.c))
        self.out.status = st
        _check(st, "ca_plan_batch")
        return self.out


def plan_batch(num_computed: Sequence[int], num_prompt_left: Sequence[int],
               block_tables: Sequence[np.ndarray], token_budget: int, max_chunk: int,
               page_size: int, num_pool_pages: int, cap_seqs: Optional[int] = None,
               cap_pages: Optional[int] = None, raise_on_error: bool = True,
               chunk_align: int = 0) -> Plan:
    """ca_plan_batch over the given requests; the Plan's arrays are filled by the library."""
    n = len(num_computed)
    tables = [np.ascontiguousarray(b, dtype=np.int32) for b in block_tables]
    reqs = (CaRequest * max(n, 1))()
    for i in range(n):
        reqs[i].num_computed = int(num_computed[i])
        reqs[i].num_prompt_left = int(num_prompt_left[i])
        reqs[i].num_pages = int(tables[i].shape[0])
        reqs[i].block_table = tables[i].ctypes.data_as(_i32p) if tables[i].size else None
    prm = CaPlanParams(int(token_budget), int(max_chunk), int(page_size), int(chunk_align),
                       int(num_pool_pages))
    if cap_seqs is None:
        cap_seqs = n
    if cap_pages is None:
        cap_pages = int(sum(t.shape[0] for t in tables))
    plan = Plan(cap_seqs, cap_pages)
    st = lib().ca_plan_batch(reqs, n, ctypes.byref(prm), ctypes.byref(plan.c))
    plan.status = st
    if raise_on_error:
        _check(st, "ca_plan_batch")
    return plan


# ---------------------------------------------------------------------------------------------
# Device calls
# ---------------------------------------------------------------------------------------------

def make_desc(num_q_heads: int, num_kv_heads: int, head_dim: int, page_size: int, dtype: str,
              sm_scale: float = 0.0, rope_theta: float = 0.0) -> CaAttnDesc:
    return CaAttnDesc(num_q_heads, num_kv_heads, head_dim, page_size,
                      CA_BF16 if dtype == "bf16" else CA_FP32, sm_scale, rope_theta)


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


_RAW_STREAM = None


def _current_stream() -> Optional[int]:
    """The calling thread's current stream on the current device, as a raw handle.  torch's
    internal getter returns the handle directly (~0.3 us); torch.cuda.current_stream() builds a
    Stream object first (~3 us per call, once per library call)."""
    global _RAW_STREAM
    import torch
    if _RAW_STREAM is None:
        get = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        dev = getattr(torch._C, "_cuda_getDevice", None)
        _RAW_STREAM = (lambda: get(dev())) if get and dev else (lambda: torch.cuda.current_stream().cuda_stream)
    return int(_RAW_STREAM()) or None


def _stream(stream) -> Optional[int]:
    if stream is None:
        return _current_stream()
    if isinstance(stream, int):
        return stream or None
    return int(stream.cuda_stream) or None


def _check_tensor(name, t, numel_min, elem_bytes):
    """Guard the raw pointers the C ABI cannot check: device, contiguity, size, element type."""
    if t is None or isinstance(t, int):
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.element_size() != elem_bytes:
        raise ValueError(f"{name} has element size {t.element_size()}, expected {elem_bytes}")
    if t.numel() < numel_min:
        raise ValueError(f"{name} has {t.numel()} elements, needs at least {numel_min}")


class Context:
    """A ca_ctx on one device (its workspace lives until close())."""

    def __init__(self, device: int = 0):
        h = ctypes.c_void_p()
        _check(lib().ca_create(int(device), ctypes.byref(h)), "ca_create")
        self.h = h
        self.device = device

    def close(self):
        if self.h:
            lib().ca_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def profile_enable(self, enable=True):
        """True / False, or an OR of the PROFILE_* flags (time only those launches)."""
        flags = PROFILE_ALL if enable is True else (0 if enable is False else int(enable))
        _check(lib().ca_profile_enable(self.h, flags), "ca_profile_enable")

    def profile_read(self, cap: int = 65536):
        """[(kernel name, ms)] of the launches since the last read (waits for their events)."""
        recs = (CaProfileRecord * max(cap, 1))()
        n = ctypes.c_int32(0)
        _check(lib().ca_profile_read(self.h, recs, cap, ctypes.byref(n)), "ca_profile_read")
        return [(recs[i].kernel.decode(), float(recs[i].ms)) for i in range(n.value)]

    def append_kv_rope(self, desc: CaAttnDesc, plan: Plan, q_in, q_out, k_new, v_new, k_cache,
                       v_cache, num_pool_pages: int, stream=None):
        eb = 2 if desc.dtype == CA_BF16 else 4
        T, hq, hkv, d, P = plan.num_tokens, desc.num_q_heads, desc.num_kv_heads, desc.head_dim, desc.page_size
        for name, t, n in (("q_in", q_in, T * hq * d), ("q_out", q_out, T * hq * d),
                           ("k_new", k_new, T * hkv * d), ("v_new", v_new, T * hkv * d),
                           ("k_cache", k_cache, num_pool_pages * hkv * P * d),
                           ("v_cache", v_cache, num_pool_pages * hkv * P * d)):
            _check_tensor(name, t, n, eb)
        st = lib().ca_append_kv_rope(self.h, ctypes.byref(desc), ctypes.byref(plan.c), _ptr(q_in),
                                     _ptr(q_out), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                                     _ptr(v_cache), int(num_pool_pages), _stream(stream))
        _check(st, "ca_append_kv_rope")

    def append_kv_rope_packed(self, desc: CaAttnDesc, plan: Plan, qkv, q_out, k_cache, v_cache,
                              num_pool_pages: int, stream=None):
        eb = 2 if desc.dtype == CA_BF16 else 4
        T, hq, hkv, d, P = plan.num_tokens, desc.num_q_heads, desc.num_kv_heads, desc.head_dim, desc.page_size
        for name, t, n in (("qkv", qkv, T * (hq + 2 * hkv) * d), ("q_out", q_out, T * hq * d),
                           ("k_cache", k_cache, num_pool_pages * hkv * P * d),
                           ("v_cache", v_cache, num_pool_pages * hkv * P * d)):
            _check_tensor(name, t, n, eb)
        st = lib().ca_append_kv_rope_packed(self.h, ctypes.byref(desc), ctypes.byref(plan.c), _ptr(qkv),
                                            _ptr(q_out), _ptr(k_cache), _ptr(v_cache),
                                            int(num_pool_pages), _stream(stream))
        _check(st, "ca_append_kv_rope_packed")

    def qkv_projection(self, desc: CaAttnDesc, num_tokens: int, hidden: int, x, w, qkv, stream=None):
        """qkv[T][Hq + 2 Hkv][d] = x[T][hidden] . w^T (w: [(Hq + 2 Hkv) d][hidden]), bf16."""
        N = (desc.num_q_heads + 2 * desc.num_kv_heads) * desc.head_dim
        for name, t, n in (("x", x, num_tokens * hidden), ("w", w, N * hidden), ("qkv", qkv, num_tokens * N)):
            _check_tensor(name, t, n, 2)
        st = lib().ca_qkv_projection(self.h, ctypes.byref(desc), int(num_tokens), int(hidden), _ptr(x),
                                     _ptr(w), _ptr(qkv), _stream(stream))
        _check(st, "ca_qkv_projection")

    def mixed_attention(self, desc: CaAttnDesc, plan: Plan, q, k_cache, v_cache,
                        num_pool_pages: int, o, lse=None, stream=None, no_alloc=False):
        """ca_mixed_attention, or with no_alloc ca_mixed_attention_noalloc (workspace in the
        library's static scratch array; nothing allocated)."""
        eb = 2 if desc.dtype == CA_BF16 else 4
        T, hq, hkv, d, P = plan.num_tokens, desc.num_q_heads, desc.num_kv_heads, desc.head_dim, desc.page_size
        for name, t, n, b in (("q", q, T * hq * d, eb), ("o", o, T * hq * d, eb),
                              ("k_cache", k_cache, num_pool_pages * hkv * P * d, eb),
                              ("v_cache", v_cache, num_pool_pages * hkv * P * d, eb),
                              ("lse", lse, T * hq, 4)):
            _check_tensor(name, t, n, b)
        fn = lib().ca_mixed_attention_noalloc if no_alloc else lib().ca_mixed_attention
        st = fn(self.h, ctypes.byref(desc), ctypes.byref(plan.c), _ptr(q), _ptr(k_cache),
                _ptr(v_cache), int(num_pool_pages), _ptr(o), _ptr(lse), _stream(stream))
        _check(st, "ca_mixed_attention_noalloc" if no_alloc else "ca_mixed_attention")


def create(device: int = 0) -> Context:
    return Context(device)


def destroy(ctx: Context):
    ctx.close()
