"""Test/bench harness: lay workload inputs into the library's paged layout and read them back.

Page layout of the library (include/ca.h): k_cache [pool][Hkv][d/8][P][8],
v_cache [pool][Hkv][d/16][P/4][16][4].  The pool tensors are allocated with those shapes, so a
(page, slot) pair indexes them directly.  These helpers only move data (scatter / gather by
block table); they compute nothing.
"""
from __future__ import annotations

from typing import Iterable, Optional

import numpy as np


def torch_dtype(dt: str):
    import torch
    return torch.bfloat16 if dt == "bf16" else torch.float32


def alloc_pool(wl, device="cuda", fill: Optional[float] = float("nan")):
    import torch
    td = torch_dtype(wl.dtype)
    P, H, d = wl.page_size, wl.num_kv_heads, wl.head_dim
    k = torch.empty((wl.num_pool_pages, H, d // 8, P, 8), dtype=td, device=device)
    v = torch.empty((wl.num_pool_pages, H, d // 16, P // 4, 16, 4), dtype=td, device=device)
    if fill is not None:
        k.fill_(fill)
        v.fill_(fill)
    return k, v


def random_pool(wl, seed: int, device="cuda"):
    """Whole pool filled with N(0,1) values drawn on the device (background for big configs)."""
    import torch
    k, v = alloc_pool(wl, device, fill=None)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    for t in (k, v):
        flat = t.view(-1)
        step = 1 << 28
        for b in range(0, flat.numel(), step):
            e = min(b + step, flat.numel())
            flat[b:e] = torch.randn(e - b, generator=gen, device=device, dtype=torch.float32).to(t.dtype)
    return k, v


def _slots(table: np.ndarray, P: int, start: int, stop: int):
    pos = np.arange(start, stop)
    return table[pos // P].astype(np.int64), (pos % P).astype(np.int64)


def _scatter(k_cache, v_cache, pi, si, k, v):
    """Write dense k, v [n, Hkv, d] to (page pi[i], slot si[i])."""
    n, H, d = k.shape
    k_cache[pi, :, :, si, :] = k.reshape(n, H, d // 8, 8).to(k_cache.device, k_cache.dtype)
    v_cache[pi, :, :, si // 4, :, si % 4] = v.reshape(n, H, d // 16, 16).to(v_cache.device, v_cache.dtype)


def _gather(k_cache, v_cache, pi, si):
    """Read (page pi[i], slot si[i]) back as dense k, v [n, Hkv, d]."""
    k = k_cache[pi, :, :, si, :]
    v = v_cache[pi, :, :, si // 4, :, si % 4]
    n, H = k.shape[0], k.shape[1]
    return k.reshape(n, H, -1), v.reshape(n, H, -1)


def draw_histories(wl, requests: Iterable[int], threads: int = 16):
    """{r: wl.history(r)} drawn on a thread pool (each request has its own seeded generator, and
    numpy releases the GIL while it fills an array, so the draws run side by side)."""
    from concurrent.futures import ThreadPoolExecutor
    reqs = list(requests)
    with ThreadPoolExecutor(max(1, min(threads, len(reqs)))) as ex:
        return dict(zip(reqs, ex.map(wl.history, reqs)))


def write_history(wl, k_cache, v_cache, requests: Optional[Iterable[int]] = None, hist=None):
    """Scatter each request's drawn history (positions 0..nc-1) into its pages (hist: histories
    drawn ahead of time, {r: (k, v)}; default: drawn here)."""
    import torch
    reqs = range(wl.n) if requests is None else requests
    dev = k_cache.device
    for r in reqs:
        nc = int(wl.num_computed[r])
        if nc == 0:
            continue
        hk, hv = wl.history(r) if hist is None else hist[r]
        pages, slots = _slots(wl.block_tables[r], wl.page_size, 0, nc)
        pi = torch.from_numpy(pages).to(dev)
        si = torch.from_numpy(slots).to(dev)
        _scatter(k_cache, v_cache, pi, si, torch.from_numpy(hk), torch.from_numpy(hv))


def write_positions(k_cache, v_cache, table: np.ndarray, P: int, k: np.ndarray, v: np.ndarray):
    """Scatter dense k, v [n, Hkv, d] to positions 0..n-1 of a request with block table `table`."""
    import torch
    n = k.shape[0]
    if n == 0:
        return
    pages, slots = _slots(np.asarray(table), P, 0, n)
    dev = k_cache.device
    _scatter(k_cache, v_cache, torch.from_numpy(pages).to(dev), torch.from_numpy(slots).to(dev),
             torch.from_numpy(np.ascontiguousarray(k)), torch.from_numpy(np.ascontiguousarray(v)))


def read_dense(k_cache, v_cache, table: np.ndarray, P: int, kv_len: int):
    """Gather positions 0..kv_len-1 of one request back into dense [kv_len, Hkv, d] float64."""
    import torch
    pages, slots = _slots(table, P, 0, kv_len)
    pi = torch.from_numpy(pages).to(k_cache.device)
    si = torch.from_numpy(slots).to(k_cache.device)
    k, v = _gather(k_cache, v_cache, pi, si)
    return (k.float().cpu().numpy().astype(np.float64), v.float().cpu().numpy().astype(np.float64))


def read_positions(k_cache, v_cache, table: np.ndarray, P: int, start: int, stop: int):
    """Gather positions start..stop-1 of one request into dense [n, Hkv, d] float64."""
    pages, slots = _slots(np.asarray(table), P, start, stop)
    pi = __import__("torch").from_numpy(pages).to(k_cache.device)
    si = __import__("torch").from_numpy(slots).to(k_cache.device)
    k, v = _gather(k_cache, v_cache, pi, si)
    return (k.float().cpu().numpy().astype(np.float64), v.float().cpu().numpy().astype(np.float64))


def to_device(x: np.ndarray, dt: str, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device).to(torch_dtype(dt))


def ulp_distance(a: np.ndarray, b: np.ndarray, dt: str) -> np.ndarray:
    """|a - b| in units of the storage type's spacing at b (both hold storage-type values)."""
    mant = 7 if dt == "bf16" else 23
    b = np.asarray(b, dtype=np.float64)
    e = np.floor(np.log2(np.maximum(np.abs(b), 2.0 ** -126)))
    return np.abs(np.asarray(a, dtype=np.float64) - b) / np.exp2(e - mant)


def gpu_step(ctx, wl, plan, q_raw, k_raw, v_raw, k_cache, v_cache, want_lse=True, stream=None,
             packed=False):
    """One step through the C ABI: append + RoPE, then mixed attention.  Returns device tensors.
    packed: hand q, k, v over as one packed [T][Hq + 2 Hkv][d] array (ca_append_kv_rope_packed)."""
    import torch
    from chunked_prefill_paged_ca_amd import make_desc
    desc = make_desc(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.page_size, wl.dtype)
    if packed:
        qkv = to_device(np.concatenate([q_raw, k_raw, v_raw], axis=1), wl.dtype)
        q_out = torch.empty((qkv.shape[0], wl.num_q_heads, wl.head_dim), dtype=qkv.dtype, device=qkv.device)
        ctx.append_kv_rope_packed(desc, plan, qkv, q_out, k_cache, v_cache, wl.num_pool_pages,
                                  stream=stream)
        q_in = q_out
    else:
        q_in = to_device(q_raw, wl.dtype)
        k_in = to_device(k_raw, wl.dtype)
        v_in = to_device(v_raw, wl.dtype)
        q_out = torch.empty_like(q_in)
        ctx.append_kv_rope(desc, plan, q_in, q_out, k_in, v_in, k_cache, v_cache, wl.num_pool_pages,
                           stream=stream)
    o = torch.empty_like(q_out)
    lse = (torch.empty((plan.num_tokens, wl.num_q_heads), dtype=torch.float32, device=q_in.device)
           if want_lse else None)
    ctx.mixed_attention(desc, plan, q_out, k_cache, v_cache, wl.num_pool_pages, o, lse,
                        stream=stream)
    return q_out, o, lse


def lib_plan(wl, num_computed, num_prompt_left):
    import chunked_prefill_paged_ca_amd as ca
    return ca.plan_batch(num_computed, num_prompt_left, wl.block_tables, wl.token_budget,
                         wl.max_chunk, wl.page_size, wl.num_pool_pages, chunk_align=wl.chunk_align)
