"""Algorithmic work of one mixed step: the bytes and flops the method must move or compute.

These are the figures the benchmark divides by measured kernel time to place each kernel on its
roofline.  Masked-out causal work and padding are never counted.

Sources:
  * per-token KV bytes k = 2 * layers * H_kv * d_h * bytes -- magicnetworld.com
    "分块预填充与 Stall-free 调度", section 二、符号与术语约定;
  * the balance chunk C* = R (1 + D S k / 2P) - D and the memory floor (2P + D S k) / W -- same
    page, sections 四 and 六·补一;
  * causal prefill visits L (L + 1) / 2 (query, key) pairs whatever the chunking, and chunk k
    re-reads the (k - 1) c history tokens before it -- pinghaoyang.com.cn "Sarathi-Serve 完全拆解",
    section 为什么总 FLOPs 近似不变，显存流量却增加 (the formulas themselves are missing from the
    extracted text; the sums are the plain reading of the prose around them).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Sequence


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, bytes_per_elem: int) -> int:
    return 2 * layers * kv_heads * head_dim * bytes_per_elem


def memory_floor_seconds(two_p_bytes: float, decodes: int, context: int, kv_bytes: float,
                         bandwidth: float) -> float:
    """Weights read once plus every decode's history KV, over the memory bandwidth."""
    return (two_p_bytes + decodes * context * kv_bytes) / bandwidth


def balance_chunk(machine_balance: float, decodes: int, context: int, kv_bytes: float,
                  two_p_bytes: float) -> float:
    """Prefill tokens per step that make compute time equal memory time for the whole model."""
    return machine_balance * (1.0 + decodes * context * kv_bytes / two_p_bytes) - decodes


def visible_pairs(L: int) -> int:
    return L * (L + 1) // 2


def history_reread_tokens(L: int, c: int) -> int:
    """History tokens re-read over all chunks of one prompt of L tokens cut into chunks of c."""
    K = -(-L // c)
    return sum(min((k - 1) * c, L) for k in range(1, K + 1))


@dataclass
class Work:
    bytes: float = 0.0
    flops: float = 0.0

    def __iadd__(self, other: "Work"):
        self.bytes += other.bytes
        self.flops += other.flops
        return self


def decode_work(kv_len: int, hq: int, hkv: int, d: int, page_size: int, elem: int = 2) -> Work:
    """One decode row: read its whole K/V once, read q, write o, read its page ids."""
    npages = -(-kv_len // page_size)
    b = kv_len * 2 * hkv * d * elem + 2 * hq * d * elem + 4 * npages
    f = 4 * d * hq * kv_len
    return Work(b, f)


def chunk_work(history: int, q: int, hq: int, hkv: int, d: int, elem: int = 2) -> Work:
    """One prefill chunk of q rows on `history` cached tokens (keys 0..p for the row at p)."""
    b = (history + q) * 2 * hkv * d * elem + 2 * q * hq * d * elem
    f = 4 * d * hq * (q * history + q * (q + 1) // 2)
    return Work(b, f)


def plan_work(q_lens: Sequence[int], kv_lens: Sequence[int], num_decodes: int, hq: int, hkv: int,
              d: int, page_size: int, elem: int = 2):
    """(decode Work, chunk Work) of a planned step; sequences [0, num_decodes) are decodes."""
    dec, chk = Work(), Work()
    for s, (q, kv) in enumerate(zip(q_lens, kv_lens)):
        if s < num_decodes:
            dec += decode_work(int(kv), hq, hkv, d, page_size, elem)
        else:
            chk += chunk_work(int(kv) - int(q), int(q), hq, hkv, d, elem)
    return dec, chk


def append_bytes(T: int, hq: int, hkv: int, d: int, elem: int = 2) -> int:
    """Append + rotary: read q, k, v of T tokens, write rotated q and the cache rows."""
    return 2 * T * (hq + 2 * hkv) * d * elem
