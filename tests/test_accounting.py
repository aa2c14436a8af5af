"""Pins for the work accounting used by the benchmark's roofline figures."""
import json
import os

from chunked_prefill_paged_ca_amd import accounting as acc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_kv_bytes_and_worked_seconds():
    with open(os.path.join(GOLDEN, "accounting_worked_seconds.json"), encoding="utf-8") as f:
        g = json.load(f)
    kb = g["kv_bytes_per_token"]
    assert acc.kv_bytes_per_token(kb["layers"], kb["kv_heads"], kb["head_dim"],
                                  kb["bytes_per_elem"]) == kb["expected"]
    w = g["worked_seconds"]
    t = acc.memory_floor_seconds(w["two_P_bytes"], w["D"], w["S"], w["k"], w["W_bytes_per_s"])
    assert abs(t * 1e3 - w["expected_tau_mem_ms"]) < w["tolerance_ms"]
    R = w["F_flops"] / w["W_bytes_per_s"]
    c = acc.balance_chunk(R, w["D"], w["S"], w["k"], w["two_P_bytes"])
    assert abs(c - w["expected_C_star"]) < w["tolerance_C"]
    # TTFT = ceil(T / C) iterations of the memory floor
    assert round(-(-4096 // round(c)) * t * 1e3) == w["expected_TTFT_4096_at_Cstar_ms"]
    assert round(-(-4096 // 128) * t * 1e3) == w["expected_TTFT_4096_at_128_ms"]


def test_pairs_invariant_under_chunking():
    # brute-force count of visible (query, key) pairs for a chunked causal prefill
    for L, c in ((64, 16), (100, 7), (257, 256), (512, 512)):
        pairs = 0
        for s in range(0, L, c):
            for i in range(s, min(s + c, L)):
                pairs += i + 1
        assert pairs == acc.visible_pairs(L)
        # chunk_work flops over all chunks equal one-shot flops
        f = sum(acc.chunk_work(s, min(c, L - s), 2, 1, 8).flops for s in range(0, L, c))
        assert f == acc.chunk_work(0, L, 2, 1, 8).flops


def test_history_reread():
    for L, c in ((8192, 64), (8192, 512), (8192, 8192), (1000, 300)):
        K = -(-L // c)
        brute = sum(s for s in range(0, L, c))  # chunk starting at s re-reads s history tokens
        assert acc.history_reread_tokens(L, c) == brute
        if L % c == 0:
            assert brute == c * K * (K - 1) // 2
