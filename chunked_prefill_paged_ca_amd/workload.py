"""Seeded synthetic workloads for one mixed chunked-prefill + decode step.

This module only draws inputs: request progress, block tables from a shuffled page pool, and
N(0, 1) token features rounded to the storage type.  It holds none of the method's arithmetic
(no plan, no rotary embedding, no attention), so both the HIP path and the CPU oracle can take
their inputs from it.

The shapes follow the mixed batches the pages describe:
  * the 512-token budget example of pinghaoyang.com.cn "Sarathi-Serve 完全拆解",
    section "一个 512-token 预算的例子" (80 decodes, prefill P with 300 left, Q with 900 left);
  * the models of the same page's section "实验口径比最高倍数更重要" (Mistral-7B, Yi-34B,
    LLaMA2-70B) at one GPU's share of heads, and LLaMA-13B of bowenzhou.top
    "Sarathi：让解码搭上 prefill 的顺风车" (Table 2) for the chunk-size sweep.
No dataset is read: the pages' public traces are replaced by seeded length distributions.

A decode "context c" means the key count after its new token is appended: c - 1 tokens of
history are already in the cache and one token is new.  History keys are drawn as
already-rotated values.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

__all__ = ["Workload", "make_config", "CONFIG_NAMES", "round_to_storage"]

CONFIG_NAMES = {
    1: "tiny fp32 mixed batch: Hq2/Hkv2/d64, L=64 prompt in chunks of 16 + 3 decodes",
    2: "Mistral-7B layer: Hq32/Hkv8/d128 bf16, tau=512, 80 decodes + P300@1200 + Q132@2048",
    3: "Llama-13B chunk sweep: Hq40/Hkv40/d128 bf16, one 8192-token prompt in chunks of c",
    4: "Yi-34B one-GPU share: Hq28/Hkv4/d128 bf16, tau=2048, 128 decodes + chunk 1920@14336",
    5: "LLaMA2-70B one-GPU share: Hq64/Hkv8/d128 bf16, tau=1536, 256 decodes + 640@0, 512@6000, 128@30000",
}


def round_to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float values to the storage type and return them as float32 (input drawing only).

    bf16: round to nearest, ties to even, on the float32 bit pattern (add 0x7fff plus the lowest
    kept bit, clear the low 16 bits) -- the same values torch's float32 -> bfloat16 conversion
    gives for finite inputs, at numpy speed; arrays holding a non-finite value go through torch."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "fp32":
        return x
    if dtype != "bf16":
        raise ValueError(dtype)
    if not np.isfinite(x).all():
        import torch  # CPU conversion; round-to-nearest-even, NaN kept

        return torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    u = x.view(np.uint32)
    r = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


@dataclass
class Workload:
    name: str
    config: int
    seed: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    dtype: str
    token_budget: int
    max_chunk: int
    num_pool_pages: int
    num_computed: np.ndarray          # int32 [n]  tokens already cached, per request
    num_prompt_left: np.ndarray       # int32 [n]  0 marks a decode
    block_tables: List[np.ndarray]    # int32 page ids, per request (sized for the scenario)
    stream_len: np.ndarray            # int32 [n]  new tokens the request may take in the scenario
    steps: int = 1
    rope_theta: float = 10000.0
    uids: Optional[np.ndarray] = None  # stable request ids keying the random draws
    q_scale: float = 1.0              # > 1 makes scores peaky (stresses the running max)
    kv_value: Optional[float] = None  # if set, every V entry is this constant (property tests)
    chunk_align: int = 0              # planner tile multiple for chunks that leave prompt behind
    notes: dict = field(default_factory=dict)

    @property
    def n(self) -> int:
        return int(self.num_computed.shape[0])

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def is_decode(self, r: int) -> bool:
        return int(self.num_prompt_left[r]) == 0

    def _rng(self, kind: int, r: int) -> np.random.Generator:
        uid = r if self.uids is None else int(self.uids[r])
        return np.random.default_rng([self.seed, kind, uid])

    def history(self, r: int) -> Tuple[np.ndarray, np.ndarray]:
        """Cached (already rotated) K and V of request r before the first step: [nc, Hkv, d]."""
        nc = int(self.num_computed[r])
        rng = self._rng(1, r)
        shape = (nc, self.num_kv_heads, self.head_dim)
        k = rng.standard_normal(shape, dtype=np.float32)
        v = rng.standard_normal(shape, dtype=np.float32)
        if self.kv_value is not None:
            v[...] = self.kv_value
        return round_to_storage(k, self.dtype), round_to_storage(v, self.dtype)

    def stream(self, r: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
        """Raw (not yet rotated) q, k, v of the new tokens request r will process, in order."""
        m = int(self.stream_len[r])
        rng = self._rng(2, r)
        q = rng.standard_normal((m, self.num_q_heads, self.head_dim), dtype=np.float32)
        k = rng.standard_normal((m, self.num_kv_heads, self.head_dim), dtype=np.float32)
        v = rng.standard_normal((m, self.num_kv_heads, self.head_dim), dtype=np.float32)
        if self.q_scale != 1.0:
            q *= np.float32(self.q_scale)
        if self.kv_value is not None:
            v[...] = self.kv_value
        return (round_to_storage(q, self.dtype), round_to_storage(k, self.dtype),
                round_to_storage(v, self.dtype))

    def final_kv_len(self, r: int) -> int:
        return int(self.num_computed[r]) + int(self.stream_len[r])


class _PagePool:
    """Free list over a pool of physical pages, shuffled by the seed."""

    def __init__(self, num_pages: int, rng: np.random.Generator, churn: bool = False):
        self.free = list(rng.permutation(num_pages).astype(np.int32))
        if churn:
            # Allocate and release blocks of random size in random order, so the free list ends
            # up interleaving many short runs (fragmentation by allocation/free order).
            held = []
            for _ in range(256):
                k = int(rng.integers(1, 257))
                held.append([self.free.pop() for _ in range(min(k, len(self.free)))])
            for i in rng.permutation(len(held)):
                self.free.extend(held[i])

    def take(self, count: int) -> np.ndarray:
        if count > len(self.free):
            raise RuntimeError("page pool exhausted")
        out = [self.free.pop() for _ in range(count)]
        return np.asarray(out, dtype=np.int32)


def _log_uniform_int(rng, lo: int, hi: int, size: int) -> np.ndarray:
    x = np.exp(rng.uniform(math.log(lo), math.log(hi), size=size))
    return np.clip(np.rint(x), lo, hi).astype(np.int64)


def make_config(config: int, seed: Optional[int] = None, *, chunk: int = 512,
                one_shot: bool = False, peaky: bool = False, kv_value: Optional[float] = None,
                dtype: Optional[str] = None) -> Workload:
    """Build one of the five workloads with a fixed seed (default: its number):
      1  tiny fp32 batch: 2/2/64, a 64-token prompt in chunks of 16 beside 3 decodes;
      2  Mistral-7B layer: 32/8/128 bf16, budget 512, 80 decodes + prefills P (300 on 1200) and
         Q (132 of 900 on 2048);
      3  Llama-13B prompt of 8192 tokens, MHA 40/40/128 bf16, in chunks of c;
      4  Yi-34B one-GPU share: 28/4/128 bf16, budget 2048, 128 decodes + a 1920-token chunk on
         14336 cached;
      5  LLaMA2-70B one-GPU share: 64/8/128 bf16, budget 1536, 256 decodes + chunks 640@0,
         512@6000, 128@30000 on a fragmented pool.

    chunk     -- the Llama-13B prompt only: the chunk size c (token budget = c, K = ceil(8192 / c)
                 steps).
    one_shot  -- the tiny batch only: the whole 64-token prompt in one step, no decodes.
    peaky     -- multiply q by 4 (seed + 100 unless a seed is given).
    kv_value  -- make every V entry this constant.
    dtype     -- override the storage type (e.g. run the tiny batch in bf16).
    """
    if seed is None:
        seed = config + (100 if peaky else 0)
    rng = np.random.default_rng([seed, 0])
    P = 16
    nc: List[int] = []
    left: List[int] = []
    stream: List[int] = []
    steps = 1
    max_chunk = 0
    churn = False
    uids: Optional[List[int]] = None

    if config == 1:
        Hq, Hkv, d, dt, pool_pages = 2, 2, 64, "fp32", 64
        # the prompt keeps request id 3 in both modes, so both draw the same prompt tokens
        if one_shot:
            tau, steps = 64, 1
            nc, left, stream, uids = [0], [64], [64], [3]
        else:
            tau, max_chunk, steps = 32, 16, 4
            for c in (40, 57, 100):
                nc.append(c - 1); left.append(0); stream.append(steps)
            nc.append(0); left.append(64); stream.append(64)
    elif config == 2:
        Hq, Hkv, d, dt, pool_pages, tau = 32, 8, 128, "bf16", 65536, 512
        ctx = rng.integers(512, 4097, size=80)
        for c in ctx:
            nc.append(int(c) - 1); left.append(0); stream.append(1)
        nc += [1200, 2048]; left += [300, 900]; stream += [300, 900]
    elif config == 3:
        Hq, Hkv, d, dt, pool_pages = 40, 40, 128, "bf16", 4096
        L = 8192
        tau = L if one_shot else int(chunk)
        steps = -(-L // tau)
        nc, left, stream = [0], [L], [L]
    elif config == 4:
        Hq, Hkv, d, dt, pool_pages, tau = 28, 4, 128, "bf16", 65536, 2048
        ctx = _log_uniform_int(rng, 256, 16384, 128)
        for c in ctx:
            nc.append(int(c) - 1); left.append(0); stream.append(1)
        nc.append(14336); left.append(1920); stream.append(1920)
    elif config == 5:
        Hq, Hkv, d, dt, pool_pages, tau = 64, 8, 128, "bf16", 131072, 1536
        churn = True
        raw = _log_uniform_int(rng, 128, 32768, 256)
        npg = np.maximum(1, np.rint(raw / P).astype(np.int64))
        last = rng.integers(1, P + 1, size=256)
        ctx = P * (npg - 1) + last
        for c in ctx:
            nc.append(int(c) - 1); left.append(0); stream.append(1)
        for h0, q in ((0, 640), (6000, 512), (30000, 128)):
            nc.append(h0); left.append(q); stream.append(q)
    else:
        raise ValueError(f"unknown config {config}")

    if dtype is not None:
        dt = dtype
    pool = _PagePool(pool_pages, np.random.default_rng([seed, 3]), churn=churn)
    tables = []
    for r in range(len(nc)):
        final = nc[r] + stream[r]
        tables.append(pool.take(-(-final // P)))

    return Workload(
        name=CONFIG_NAMES[config], config=config, seed=seed, num_q_heads=Hq, num_kv_heads=Hkv,
        head_dim=d, page_size=P, dtype=dt, token_budget=tau, max_chunk=max_chunk,
        num_pool_pages=pool_pages, num_computed=np.asarray(nc, dtype=np.int32),
        num_prompt_left=np.asarray(left, dtype=np.int32), block_tables=tables,
        stream_len=np.asarray(stream, dtype=np.int32), steps=steps,
        uids=None if uids is None else np.asarray(uids, dtype=np.int64),
        q_scale=4.0 if peaky else 1.0, kv_value=kv_value,
        notes={"chunk": chunk if config == 3 else None, "one_shot": one_shot})


class StreamCursor:
    """Hands out each request's raw new-token rows in order, as a plan schedules them.

    Pure input routing: given which requests a plan scheduled and how many tokens each got, it
    returns the next rows of their streams, concatenated in plan order.
    """

    def __init__(self, wl: Workload):
        self.wl = wl
        self.consumed = np.zeros(wl.n, dtype=np.int64)
        self._cache = {}

    def _stream(self, r: int):
        if r not in self._cache:
            self._cache[r] = self.wl.stream(r)
        return self._cache[r]

    def take(self, req_ids, q_lens):
        wl = self.wl
        T = int(np.sum(q_lens)) if len(q_lens) else 0
        q = np.empty((T, wl.num_q_heads, wl.head_dim), dtype=np.float32)
        k = np.empty((T, wl.num_kv_heads, wl.head_dim), dtype=np.float32)
        v = np.empty((T, wl.num_kv_heads, wl.head_dim), dtype=np.float32)
        row = 0
        for r, m in zip(req_ids, q_lens):
            r, m = int(r), int(m)
            sq, sk, sv = self._stream(r)
            c = int(self.consumed[r])
            if c + m > sq.shape[0]:
                raise RuntimeError(f"request {r}: stream exhausted")
            q[row:row + m] = sq[c:c + m]
            k[row:row + m] = sk[c:c + m]
            v[row:row + m] = sv[c:c + m]
            self.consumed[r] += m
            row += m
        return q, k, v


@dataclass
class ServeScenario:
    """A seeded serving scenario for the multi-step loop: requests arriving over rounds.

    Request r arrives before round arrival[r] with a prompt of prompt_len[r] tokens, of which
    the first num_cached[r] are already in the cache (a prefix hit: their K/V are drawn here,
    already rotated, like a config's history), and decodes max_new[r] steps after its prompt.
    Its token at absolute position p has raw q, k, v that depend only on (seed, request, p), so a
    request that is preempted and recomputed gets the very same inputs again.
    """
    name: str
    seed: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    dtype: str
    token_budget: int
    max_chunk: int
    chunk_align: int
    num_pool_pages: int
    arrival: np.ndarray
    prompt_len: np.ndarray
    num_cached: np.ndarray
    max_new: np.ndarray
    rounds: int
    rope_theta: float = 10000.0
    _streams: dict = field(default_factory=dict)

    @property
    def n(self) -> int:
        return int(self.arrival.shape[0])

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def history(self, r: int) -> Tuple[np.ndarray, np.ndarray]:
        """Cached K (already rotated) and V of the prefix of request r: [num_cached, Hkv, d]."""
        nc = int(self.num_cached[r])
        rng = np.random.default_rng([self.seed, 1, r])
        shape = (nc, self.num_kv_heads, self.head_dim)
        k = rng.standard_normal(shape, dtype=np.float32)
        v = rng.standard_normal(shape, dtype=np.float32)
        return round_to_storage(k, self.dtype), round_to_storage(v, self.dtype)

    def _stream(self, r: int):
        if r not in self._streams:
            m = int(self.prompt_len[r]) + int(self.max_new[r])
            rng = np.random.default_rng([self.seed, 2, r])
            q = rng.standard_normal((m, self.num_q_heads, self.head_dim), dtype=np.float32)
            k = rng.standard_normal((m, self.num_kv_heads, self.head_dim), dtype=np.float32)
            v = rng.standard_normal((m, self.num_kv_heads, self.head_dim), dtype=np.float32)
            self._streams[r] = tuple(round_to_storage(x, self.dtype) for x in (q, k, v))
        return self._streams[r]

    def take(self, req_ids, starts, q_lens):
        """Raw q, k, v rows of positions [starts[s], starts[s] + q_lens[s]) of request
        req_ids[s], concatenated in plan order."""
        T = int(np.sum(q_lens)) if len(q_lens) else 0
        q = np.empty((T, self.num_q_heads, self.head_dim), dtype=np.float32)
        k = np.empty((T, self.num_kv_heads, self.head_dim), dtype=np.float32)
        v = np.empty((T, self.num_kv_heads, self.head_dim), dtype=np.float32)
        row = 0
        for r, s0, m in zip(req_ids, starts, q_lens):
            sq, sk, sv = self._stream(int(r))
            s0, m = int(s0), int(m)
            q[row:row + m] = sq[s0:s0 + m]
            k[row:row + m] = sk[s0:s0 + m]
            v[row:row + m] = sv[s0:s0 + m]
            row += m
        return q, k, v


def make_serve_scenario(seed: int = 3, *, n: int = 14, rounds: int = 60, pool_pages: int = 48,
                        token_budget: int = 96, max_chunk: int = 0, chunk_align: int = 0,
                        dtype: str = "bf16", heads=(16, 4, 128)) -> ServeScenario:
    """Requests arriving over the first half of the rounds: prompts of 8..300 tokens (a third
    with a cached prefix of up to half the prompt), 2..24 decode steps each.  The pool is small
    enough that decodes run out of pages and get preempted."""
    rng = np.random.default_rng([seed, 9])
    arrival = np.sort(rng.integers(0, rounds // 2, size=n))
    arrival[0] = 0
    prompt = rng.integers(8, 301, size=n)
    cached = np.where(rng.random(n) < 1 / 3, (prompt * rng.uniform(0, 0.5, size=n)).astype(np.int64), 0)
    max_new = rng.integers(2, 25, size=n)
    Hq, Hkv, d = heads
    return ServeScenario(name=f"serving loop: {n} requests, pool {pool_pages} pages, tau={token_budget}",
                         seed=seed, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, page_size=16,
                         dtype=dtype, token_budget=token_budget, max_chunk=max_chunk,
                         chunk_align=chunk_align, num_pool_pages=pool_pages,
                         arrival=arrival.astype(np.int32), prompt_len=prompt.astype(np.int32),
                         num_cached=cached.astype(np.int32), max_new=max_new.astype(np.int32),
                         rounds=rounds)


def projection_inputs(T: int, hidden: int, n_out: int, seed: int, dtype: str = "bf16"):
    """Seeded hidden states x [T][hidden] ~ N(0, 1) and projection weights w [n_out][hidden] ~
    N(0, 1/hidden) (so each output is O(1)), both rounded to the storage type."""
    rng = np.random.default_rng([seed, 5])
    x = rng.standard_normal((T, hidden), dtype=np.float32)
    w = rng.standard_normal((n_out, hidden), dtype=np.float32) * np.float32(1.0 / math.sqrt(hidden))
    return round_to_storage(x, dtype), round_to_storage(w, dtype)
