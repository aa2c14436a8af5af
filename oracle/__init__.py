"""CPU oracle for the mixed chunked-prefill + decode step (TEST INFRASTRUCTURE ONLY).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import this package.
The product path never does.  The arithmetic lives in oracle.c (fp64, plain loops); this file
only marshals numpy arrays and keeps the oracle's own dense, per-request view of the cache.

Parity pins for every function here are in tests/test_oracle_pins.py (values fixed by the pages'
worked example, closed forms, brute force and library routines).
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Iterable, List, Optional

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

OK, INVALID_ARG, NO_PAGES, CAPACITY = 0, 1, 2, 3

_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_f64p = ctypes.POINTER(ctypes.c_double)


def lib():
    global _LIB
    if _LIB is None:
        path = _build.LIB
        src = os.path.join(_HERE, "oracle.c")
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(src):
            _build.build()
        L = ctypes.CDLL(path)
        L.oracle_plan.restype = ctypes.c_int
        L.oracle_plan.argtypes = [ctypes.c_int32, _i32p, _i32p, _i32p, _i64p, _i32p,
                                  ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                  ctypes.c_int64,
                                  ctypes.c_int32, ctypes.c_int32,
                                  _i32p, _i32p, _i32p, _i32p, _i32p, _i32p]
        L.oracle_rope.restype = None
        L.oracle_rope.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _i32p,
                                  ctypes.c_double, _f64p, _f64p]
        L.oracle_attention.restype = ctypes.c_int
        L.oracle_attention.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_int32, _f64p, _i32p, _f64p, _f64p,
                                       ctypes.c_double, _f64p, _f64p, ctypes.c_int32]
        L.oracle_bf16_value.restype = ctypes.c_double
        L.oracle_bf16_value.argtypes = [ctypes.c_double]
        L.oracle_round.restype = None
        L.oracle_round.argtypes = [ctypes.c_int64, ctypes.c_int32, _f64p, _f64p]
        _LIB = L
    return _LIB


def _p(a: np.ndarray, t):
    return a.ctypes.data_as(t)


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)))


# ---------------------------------------------------------------------------------------------
# Plan
# ---------------------------------------------------------------------------------------------

def plan(num_computed, num_prompt_left, block_tables: List[np.ndarray], token_budget: int,
         max_chunk: int, page_size: int, num_pool_pages: int,
         cap_seqs: Optional[int] = None, cap_pages: Optional[int] = None,
         chunk_align: int = 0) -> Dict:
    """Decode-first budget plan.  Returns {"status", and on OK the metadata arrays + counts}."""
    nc = np.ascontiguousarray(num_computed, dtype=np.int32)
    nl = np.ascontiguousarray(num_prompt_left, dtype=np.int32)
    n = int(nc.shape[0])
    npg = np.asarray([len(b) for b in block_tables], dtype=np.int32)
    off = np.zeros(n + 1, dtype=np.int64)
    off[1:] = np.cumsum(npg)
    bt = (np.concatenate([np.asarray(b, dtype=np.int32) for b in block_tables])
          if n and off[-1] > 0 else np.zeros(1, dtype=np.int32))
    if cap_seqs is None:
        cap_seqs = n
    if cap_pages is None:
        cap_pages = int(off[-1])
    req_ids = np.zeros(max(cap_seqs, 1), dtype=np.int32)
    qo = np.zeros(cap_seqs + 1, dtype=np.int32)
    kvp = np.zeros(cap_seqs + 1, dtype=np.int32)
    idx = np.zeros(max(cap_pages, 1), dtype=np.int32)
    last = np.zeros(max(cap_seqs, 1), dtype=np.int32)
    counts = np.zeros(5, dtype=np.int32)
    st = lib().oracle_plan(n, _p(nc, _i32p), _p(nl, _i32p), _p(npg, _i32p), _p(off, _i64p),
                           _p(bt, _i32p), token_budget, max_chunk, chunk_align, page_size,
                           num_pool_pages,
                           cap_seqs, cap_pages, _p(req_ids, _i32p), _p(qo, _i32p),
                           _p(kvp, _i32p), _p(idx, _i32p), _p(last, _i32p), _p(counts, _i32p))
    out = {"status": int(st)}
    if st in (OK, CAPACITY):
        ns, nd, nt, npages, ndef = (int(c) for c in counts)
        out.update(num_seqs=ns, num_decodes=nd, num_tokens=nt, num_pages=npages,
                   num_deferred_decodes=ndef)
    if st == OK:
        out.update(req_ids=req_ids[:ns].copy(), qo_indptr=qo[:ns + 1].copy(),
                   kv_page_indptr=kvp[:ns + 1].copy(), kv_page_indices=idx[:npages].copy(),
                   kv_last_page_len=last[:ns].copy())
    return out


# ---------------------------------------------------------------------------------------------
# Rotary embedding, rounding, attention
# ---------------------------------------------------------------------------------------------

def rope(x: np.ndarray, pos: np.ndarray, theta: float = 10000.0) -> np.ndarray:
    """x: [ntok, nheads, d]; pos: [ntok] absolute positions.  fp64 result, not rounded."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    ntok, nh, d = x.shape
    out = np.empty_like(x)
    lib().oracle_rope(ntok, nh, d, _p(pos, _i32p), float(theta), _p(x, _f64p), _p(out, _f64p))
    return out


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """One rounding of fp64 values to bf16 or fp32, returned as fp64 values."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty_like(x)
    lib().oracle_round(x.size, 1 if dtype == "bf16" else 0, _p(x, _f64p), _p(out, _f64p))
    return out


def bf16_value(x: float) -> float:
    return float(lib().oracle_bf16_value(float(x)))


def attention(q: np.ndarray, pos: np.ndarray, k: np.ndarray, v: np.ndarray,
              scale: Optional[float] = None, nthreads: Optional[int] = None):
    """One request: q [nrows, Hq, d], k/v [kv_len, Hkv, d].  Returns (out [nrows,Hq,d], lse)."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    nrows, hq, d = q.shape
    kv_len, hkv, _ = k.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.empty((nrows, hq, d), dtype=np.float64)
    lse = np.empty((nrows, hq), dtype=np.float64)
    st = lib().oracle_attention(nrows, hq, hkv, d, kv_len, _p(q, _f64p), _p(pos, _i32p),
                                _p(k, _f64p), _p(v, _f64p), float(scale), _p(out, _f64p),
                                _p(lse, _f64p), nthreads or default_threads())
    if st != OK:
        raise ValueError(f"oracle_attention: invalid arguments (status {st})")
    return out, lse


# ---------------------------------------------------------------------------------------------
# A session: the oracle's own dense cache, advanced step by step
# ---------------------------------------------------------------------------------------------

class Session:
    """Dense fp64 K/V per tracked request, plus the request progress the plan needs.

    requests -- the request indices whose cache is kept (default: all).  Untracked requests are
                still planned (the plan only needs their sizes) but get no attention output.
    history  -- optional callable r -> (k, v) returning the same arrays as wl.history(r) (e.g.
                drawn once ahead of time); default wl.history.
    """

    def __init__(self, wl, requests: Optional[Iterable[int]] = None, history=None):
        self.wl = wl
        self.num_computed = wl.num_computed.astype(np.int32).copy()
        self.num_prompt_left = wl.num_prompt_left.astype(np.int32).copy()
        tracked = range(wl.n) if requests is None else requests
        self.k: Dict[int, np.ndarray] = {}
        self.v: Dict[int, np.ndarray] = {}
        draw = wl.history if history is None else history
        for r in tracked:
            hk, hv = draw(r)
            self.k[r] = hk.astype(np.float64)
            self.v[r] = hv.astype(np.float64)

    def fork(self) -> "Session":
        """An independent copy of the session's progress and cache (arrays are never mutated in
        place by step(), so the per-request arrays can be shared)."""
        other = Session.__new__(Session)
        other.wl = self.wl
        other.num_computed = self.num_computed.copy()
        other.num_prompt_left = self.num_prompt_left.copy()
        other.k = dict(self.k)
        other.v = dict(self.v)
        return other

    def plan(self) -> Dict:
        wl = self.wl
        return plan(self.num_computed, self.num_prompt_left, wl.block_tables, wl.token_budget,
                    wl.max_chunk, wl.page_size, wl.num_pool_pages,
                    chunk_align=getattr(wl, "chunk_align", 0))

    def step(self, p: Dict, q_raw: np.ndarray, k_raw: np.ndarray, v_raw: np.ndarray,
             rows: Optional[np.ndarray] = None, nthreads: Optional[int] = None) -> Dict:
        """Run one step from the oracle's own plan `p` on the raw new-token rows (plan order).

        Appends the rotated, rounded keys and the values of every scheduled token of tracked
        requests, then attends the chosen rows (default: every row of tracked requests).
        Returns q_rot [T,Hq,d], k_rot [T,Hkv,d], o [T,Hq,d], lse [T,Hq], pos [T] (fp64; rows not
        attended hold NaN) and, per tracked request, nothing else: the cache is self.k / self.v.
        """
        wl = self.wl
        T = int(p["num_tokens"])
        qo = p["qo_indptr"]
        pos = np.empty(T, dtype=np.int32)
        for s, r in enumerate(p["req_ids"]):
            b, e = int(qo[s]), int(qo[s + 1])
            pos[b:e] = self.num_computed[r] + np.arange(e - b, dtype=np.int32)
        q_rot = round_to(rope(q_raw, pos, wl.rope_theta), wl.dtype)
        k_rot = round_to(rope(k_raw, pos, wl.rope_theta), wl.dtype)
        v_new = np.asarray(v_raw, dtype=np.float64)
        o = np.full((T, wl.num_q_heads, wl.head_dim), np.nan)
        lse = np.full((T, wl.num_q_heads), np.nan)
        want = np.ones(T, dtype=bool) if rows is None else np.isin(np.arange(T), rows)
        for s, r in enumerate(p["req_ids"]):
            r = int(r)
            b, e = int(qo[s]), int(qo[s + 1])
            if r in self.k:
                self.k[r] = np.concatenate([self.k[r], k_rot[b:e]], axis=0)
                self.v[r] = np.concatenate([self.v[r], v_new[b:e]], axis=0)
                sel = np.nonzero(want[b:e])[0] + b
                if sel.size:
                    oo, ll = attention(q_rot[sel], pos[sel], self.k[r], self.v[r],
                                       wl.sm_scale, nthreads)
                    o[sel] = oo
                    lse[sel] = ll
            self.num_computed[r] += e - b
            if self.num_prompt_left[r] > 0:
                self.num_prompt_left[r] -= e - b
        return {"q_rot": q_rot, "k_rot": k_rot, "o": o, "lse": lse, "pos": pos}


# ---------------------------------------------------------------------------------------------
# QKV projection
# ---------------------------------------------------------------------------------------------

def linear(x: np.ndarray, w: np.ndarray, dtype: str) -> np.ndarray:
    """out[T][N] = x[T][K] . w[N][K]^T in fp64, rounded once to the storage type.

    bowenzhou.top "Sarathi：让解码搭上 prefill 的顺风车", section "Decode-maximal batching：顺车的账本":
    the linear layers of a mixed batch are one matrix product over all its tokens (decode rows
    and chunk rows alike); this is that product for the q, k, v projection.
    """
    return round_to(np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T, dtype)


# ---------------------------------------------------------------------------------------------
# Multi-step serving loop
# ---------------------------------------------------------------------------------------------

class SchedModel:
    """Plain model of the serving loop around the plan, round by round.

    magicnetworld.com "分块预填充与 Stall-free 调度", section "六·补二、调度器每一轮在做什么": in each
    round every running decode takes one token, and one that needs KV space when none is left is
    preempted (its cache is dropped and it is recomputed from its first token later); the budget
    left goes to prefill chunks, and an unfinished prompt is continued next round.
    pinghaoyang.com.cn "Sarathi-Serve 完全拆解", section "一个 512-token 预算的例子", step 4: a prompt
    that finishes is a decode from the next round on.  The packing of a round is `plan` above.

    Readings where the pages are silent (the same ones the library takes): the page pool is a
    first-in first-out free list starting as 0 .. N-1; a preempted request is not scheduled again
    in the round that preempted it; a chunk is also cut to the slots its pages and the free list
    can hold; a request decodes max_new steps after its prompt, then its pages go back to the
    free list (in block-table order).
    """

    WAITING, RUNNING, FINISHED = 0, 1, 2

    def __init__(self, token_budget: int, max_chunk: int, page_size: int, num_pool_pages: int,
                 chunk_align: int = 0):
        from collections import deque
        self.tau, self.mc, self.P, self.A = token_budget, max_chunk, page_size, chunk_align
        self.N = num_pool_pages
        self.free = deque(range(num_pool_pages))
        self.reqs: List[Dict] = []
        self.pending = None

    def add(self, prompt_len: int, max_new: int, num_cached: int = 0) -> int:
        """A request whose first num_cached tokens are already cached, in pages taken from the
        free list (the caller fills them)."""
        assert 1 <= prompt_len and 0 <= num_cached < prompt_len and max_new >= 0
        n_pages = -(-num_cached // self.P)
        assert len(self.free) >= n_pages
        pages = [self.free.popleft() for _ in range(n_pages)]
        self.reqs.append({"state": self.WAITING, "nc": num_cached, "left": prompt_len - num_cached,
                          "generated": 0, "max_new": max_new, "pages": pages, "preemptions": 0})
        return len(self.reqs) - 1

    def _cut(self, q: int, left: int) -> int:
        return q - q % self.A if self.A > 1 and q < left else q

    def step(self) -> Dict:
        assert self.pending is None, "commit the previous round first"
        budget = self.tau
        held_back = set()
        # decodes: one token each, in admission order, while the budget lasts
        for i, r in enumerate(self.reqs):
            if r["state"] != self.RUNNING or budget == 0:
                continue
            if r["nc"] + 1 > len(r["pages"]) * self.P:
                if not self.free:
                    self.free.extend(r["pages"])
                    r["pages"] = []
                    r["left"], r["nc"] = r["nc"], 0
                    r["state"] = self.WAITING
                    r["preemptions"] += 1
                    held_back.add(i)
                    continue
                r["pages"].append(self.free.popleft())
            budget -= 1
        # prefill chunks from what is left, in admission order
        for i, r in enumerate(self.reqs):
            if budget <= 0:
                break
            if r["state"] != self.WAITING or i in held_back:
                continue
            q = min(r["left"], budget)
            if self.mc:
                q = min(q, self.mc)
            q = self._cut(q, r["left"])
            fits = (len(r["pages"]) + len(self.free)) * self.P - r["nc"]
            if q > fits:
                q = self._cut(fits, r["left"])
            if q <= 0:
                continue
            while len(r["pages"]) * self.P < r["nc"] + q:
                r["pages"].append(self.free.popleft())
            budget -= q
        # the round's plan over the requests still in play
        ids = [i for i, r in enumerate(self.reqs) if r["state"] != self.FINISHED and i not in held_back]
        rs = [self.reqs[i] for i in ids]
        p = plan([r["nc"] for r in rs], [r["left"] if r["state"] == self.WAITING else 0 for r in rs],
                 [np.asarray(r["pages"], dtype=np.int32) for r in rs], self.tau, self.mc, self.P,
                 self.N, chunk_align=self.A)
        assert p["status"] == OK, p["status"]
        p["req_ids"] = np.asarray([ids[k] for k in p["req_ids"]], dtype=np.int32)
        self.pending = list(zip(p["req_ids"].tolist(), np.diff(p["qo_indptr"]).tolist()))
        return p

    def commit(self):
        assert self.pending is not None, "no planned round"
        for i, q in self.pending:
            r = self.reqs[i]
            r["nc"] += q
            if r["state"] == self.WAITING:
                r["left"] -= q
                if r["left"] == 0:
                    r["state"] = self.FINISHED if r["generated"] >= r["max_new"] else self.RUNNING
            else:
                r["generated"] += 1
                if r["generated"] >= r["max_new"]:
                    r["state"] = self.FINISHED
            if r["state"] == self.FINISHED:
                self.free.extend(r["pages"])
                r["pages"] = []
        self.pending = None


class ServeSession:
    """The serving loop (SchedModel) with the oracle's dense per-request cache.

    sc is a ServeScenario: request r is admitted with its cached prefix (sc.history) and later
    rounds append its tokens at their absolute positions.  A request the loop preempted starts
    again from an empty cache (its recompute appends every token again).
    """

    def __init__(self, sc):
        self.sc = sc
        self.model = SchedModel(sc.token_budget, sc.max_chunk, sc.page_size, sc.num_pool_pages,
                                sc.chunk_align)
        self.k: Dict[int, np.ndarray] = {}
        self.v: Dict[int, np.ndarray] = {}

    def free_pages(self) -> int:
        return len(self.model.free)

    def add(self, r: int) -> int:
        sc = self.sc
        i = self.model.add(int(sc.prompt_len[r]), int(sc.max_new[r]), int(sc.num_cached[r]))
        hk, hv = sc.history(r)
        self.k[i] = hk.astype(np.float64)
        self.v[i] = hv.astype(np.float64)
        return i

    def plan(self) -> Dict:
        p = self.model.step()
        for i, r in enumerate(self.model.reqs):
            if r["nc"] == 0:
                shape = (0, self.sc.num_kv_heads, self.sc.head_dim)
                self.k[i] = np.zeros(shape)
                self.v[i] = np.zeros(shape)
        return p

    def starts(self, p: Dict) -> np.ndarray:
        """First absolute position of each scheduled sequence of the planned round."""
        return np.asarray([self.model.reqs[int(i)]["nc"] for i in p["req_ids"]], dtype=np.int32)

    def step(self, p: Dict, q_raw: np.ndarray, k_raw: np.ndarray, v_raw: np.ndarray,
             nthreads: Optional[int] = None) -> Dict:
        """Append the round's tokens, attend every row, then commit the round."""
        sc = self.sc
        T = int(p["num_tokens"])
        qo = p["qo_indptr"]
        pos = np.empty(T, dtype=np.int32)
        for s, st in enumerate(self.starts(p)):
            b, e = int(qo[s]), int(qo[s + 1])
            pos[b:e] = st + np.arange(e - b, dtype=np.int32)
        q_rot = round_to(rope(q_raw, pos, sc.rope_theta), sc.dtype)
        k_rot = round_to(rope(k_raw, pos, sc.rope_theta), sc.dtype)
        v_new = np.asarray(v_raw, dtype=np.float64)
        o = np.full((T, sc.num_q_heads, sc.head_dim), np.nan)
        lse = np.full((T, sc.num_q_heads), np.nan)
        for s, i in enumerate(p["req_ids"]):
            i = int(i)
            b, e = int(qo[s]), int(qo[s + 1])
            self.k[i] = np.concatenate([self.k[i], k_rot[b:e]], axis=0)
            self.v[i] = np.concatenate([self.v[i], v_new[b:e]], axis=0)
            o[b:e], lse[b:e] = attention(q_rot[b:e], pos[b:e], self.k[i], self.v[i], sc.sm_scale,
                                         nthreads)
        self.model.commit()
        return {"q_rot": q_rot, "o": o, "lse": lse, "pos": pos}
