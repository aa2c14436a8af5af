"""Pins for the CPU oracle: each test ties an oracle function to something other than itself.

Pins used (none re-types the oracle's own formula):
  * the pages' worked example of a 512-token budget (tests/golden/worked_example_512.json), also
    with chunk sizes aligned to 32 as the pages' tile-quantisation section describes, and a
    downward brute-force search for aligned chunk sizes;
  * the QKV projection: a triple-loop brute force, identity and row-selection weights, and a
    tie that shows one rounding of the exact sum;
  * the serving loop: the worked example over two rounds (P becomes a decode, Q gets 431), the
    pages' rounds-to-first-token example (tests/golden/rounds_to_first_token.json), and pool /
    preemption invariants over random arrivals;
  * brute force: a NumPy masked-softmax matrix formulation on tiny inputs;
  * closed forms: V == 1 gives 1, one-hot V gives the probability row, kv_len 1 gives v_0,
    K == 0 gives the prefix mean, two keys give a logistic weight (scipy.special.expit);
  * reductions to library routines: bf16 rounding against torch's float32 -> bfloat16
    conversion; split-half RoPE against complex multiplication by exp(i*angle);
  * invariants: causality under perturbation of later keys, GQA equal to MHA with replicated
    KV heads, rotation-group identities, chunked prefill equal to one-shot prefill.
"""
import json
import os

import numpy as np
import pytest
from scipy.special import expit, softmax

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


# ------------------------------------------------------------------------------------------
# Plan
# ------------------------------------------------------------------------------------------

def _tables(n, pages_each, pool_perm):
    it = iter(pool_perm)
    return [np.array([next(it) for _ in range(p)], dtype=np.int32) for p in pages_each]


def test_plan_worked_example(oracle_mod):
    g = _load("worked_example_512.json")
    nd = g["num_decodes"]
    rng = np.random.default_rng(0)
    ctx = rng.integers(10, 100, size=nd)
    nc = list(ctx - 1) + [500, 700]
    left = [0] * nd + g["prefills_left"]
    pages = [int(-(-(c + 1) // 16)) + 1 for c in nc[:nd]] + [100, 120]
    tables = _tables(len(nc), pages, rng.permutation(20000))
    p = oracle_mod.plan(nc, left, tables, g["token_budget"], 0, 16, 20000)
    assert p["status"] == 0
    q = np.diff(p["qo_indptr"])
    e1 = g["expected_step1_q"]
    assert list(q[:nd]) == [e1["decodes"]] * nd
    assert list(q[nd:]) == [e1["P"], e1["Q"]]
    assert p["num_tokens"] == e1["total"] and p["num_decodes"] == nd
    assert list(p["req_ids"]) == list(range(nd + 2))
    # Next step: P became a decode, Q continues.
    nc2 = [c + 1 for c in nc[:nd]] + [nc[nd] + 300, nc[nd + 1] + 132]
    left2 = [0] * (nd + 1) + [900 - 132]
    p2 = oracle_mod.plan(nc2, left2, tables, g["token_budget"], 0, 16, 20000)
    q2 = np.diff(p2["qo_indptr"])
    e2 = g["expected_step2_q"]
    assert p2["num_decodes"] == e2["decodes"]
    assert q2[-1] == e2["Q"] and p2["num_tokens"] == e2["total"]


def test_plan_worked_example_aligned(oracle_mod):
    g = _load("worked_example_512.json")
    nd = g["num_decodes"]
    nc = [40] * nd + [500, 700]
    left = [0] * nd + g["prefills_left"]
    tables = [np.arange(200 * i, 200 * i + 200, dtype=np.int32) for i in range(nd + 2)]
    p = oracle_mod.plan(nc, left, tables, g["token_budget"], 0, 16, 200 * (nd + 2), chunk_align=32)
    e = g["aligned_32"]["expected_step1_q"]
    q = np.diff(p["qo_indptr"])
    assert list(q[nd:]) == [e["P"], e["Q"]] and p["num_tokens"] == e["total"]
    # alignment 0 and 1 are the base rule
    for a in (0, 1):
        p1 = oracle_mod.plan(nc, left, tables, g["token_budget"], 0, 16, 200 * (nd + 2), chunk_align=a)
        assert list(np.diff(p1["qo_indptr"])[nd:]) == [300, 132]


def _aligned_chunks_brute_force(nc, left, tables, tau, mc, P, A):
    """Prefill chunk sizes by a downward search: the largest q <= every cap that is either a
    multiple of A or the whole rest of the prompt (no arithmetic shortcut)."""
    budget = tau - min(tau, sum(1 for x in left if x == 0))
    out = {}
    for r in range(len(nc)):
        if left[r] == 0 or budget <= 0:
            continue
        cap = min(left[r], budget, len(tables[r]) * P - nc[r])
        if mc:
            cap = min(cap, mc)
        q = cap
        while q > 0 and not (q == left[r] or q % A == 0):
            q -= 1
        if q > 0:
            out[r] = q
            budget -= q
    return out


def test_plan_alignment_brute_force(oracle_mod):
    rng = np.random.default_rng(11)
    P = 16
    for trial in range(300):
        n = int(rng.integers(1, 25))
        nc = rng.integers(0, 300, size=n).astype(np.int32)
        left = np.where(rng.random(n) < 0.4, 0, rng.integers(1, 400, size=n)).astype(np.int32)
        pages = [-(-(int(nc[i]) + max(1, int(left[i]))) // P) + int(rng.integers(0, 2)) - int(rng.random() < 0.2)
                 for i in range(n)]
        pages = [max(p_, -(-(int(nc[i]) + 1) // P)) for i, p_ in enumerate(pages)]
        tables = _tables(n, pages, rng.permutation(sum(pages) + 10))
        tau = int(rng.integers(1, 600))
        mc = int(rng.choice([0, 0, 40, 64]))
        A = int(rng.choice([2, 16, 32, 100]))
        p = oracle_mod.plan(nc, left, tables, tau, mc, P, sum(pages) + 10, chunk_align=A)
        assert p["status"] == 0
        q = np.diff(p["qo_indptr"])
        nd = p["num_decodes"]
        got = {int(r): int(x) for r, x in zip(p["req_ids"][nd:], q[nd:])}
        assert got == _aligned_chunks_brute_force(nc, left, tables, tau, mc, P, A)
        for r, x in got.items():
            assert x == left[r] or x % A == 0


def test_plan_aligned_sweep_shape(oracle_mod):
    # One prompt, budget c = 257 with 32-alignment: every chunk but the last is 256.
    L, c = 1000, 257
    nc, left = 0, L
    tab = [np.arange(-(-L // 16), dtype=np.int32)]
    qs = []
    while left > 0:
        p = oracle_mod.plan([nc], [left], tab, c, 0, 16, 1000, chunk_align=32)
        qs.append(int(p["num_tokens"]))
        nc += qs[-1]
        left -= qs[-1]
    assert qs == [256, 256, 256, 232]


# ------------------------------------------------------------------------------------------
# Serving loop (SchedModel)
# ------------------------------------------------------------------------------------------

def _running_decodes(m, n, ctx=2048, max_new=1000):
    """n requests that are decoding: one prefill round of their last prompt token first."""
    ids = [m.add(ctx + 1, max_new, ctx) for _ in range(n)]
    m.step()
    m.commit()
    assert all(m.reqs[i]["state"] == m.RUNNING for i in ids)
    return ids


def test_sched_worked_example_two_rounds(oracle_mod):
    g = _load("worked_example_512.json")
    nd = g["num_decodes"]
    m = oracle_mod.SchedModel(g["token_budget"], 0, 16, 20000)
    _running_decodes(m, nd, ctx=1)
    P = m.add(1500, 10, 1500 - g["prefills_left"][0])
    Q = m.add(2948, 10, 2948 - g["prefills_left"][1])
    e1, e2 = g["expected_step1_q"], g["expected_step2_q"]
    p = m.step()
    q = np.diff(p["qo_indptr"])
    assert p["num_decodes"] == nd and list(q[nd:]) == [e1["P"], e1["Q"]] and p["num_tokens"] == e1["total"]
    assert list(p["req_ids"][nd:]) == [P, Q]
    m.commit()
    assert m.reqs[P]["state"] == m.RUNNING and m.reqs[Q]["left"] == 900 - 132
    p = m.step()
    q = np.diff(p["qo_indptr"])
    assert p["num_decodes"] == e2["decodes"] and q[-1] == e2["Q"] and p["num_tokens"] == e2["total"]


def test_sched_rounds_to_first_token(oracle_mod):
    g = _load("rounds_to_first_token.json")
    D, C = g["decodes"], g["prefill_share"]
    m = oracle_mod.SchedModel(D + C, 0, 16, 100000)
    _running_decodes(m, D)
    r = m.add(g["prompt_len"], 5)
    rounds = 0
    while m.reqs[r]["state"] == m.WAITING:
        p = m.step()
        assert p["num_decodes"] == D
        m.commit()
        rounds += 1
    assert rounds == g["expected_rounds"]


def test_sched_invariants_random(oracle_mod):
    """Pool conservation, table sizes, what a preemption does, exactly max_new decode steps per
    finished request, budget per round."""
    rng = np.random.default_rng(21)
    P = 16
    preempted_total = 0
    for trial in range(40):
        N = int(rng.integers(4, 40))
        tau = int(rng.integers(1, 200))
        m = oracle_mod.SchedModel(tau, int(rng.choice([0, 0, 32])), P, N, int(rng.choice([0, 0, 16])))
        arrivals = sorted(rng.integers(0, 30, size=int(rng.integers(1, 12))).tolist())
        steps_run = {}
        for rnd in range(80):
            while arrivals and arrivals[0] <= rnd:
                L = int(rng.integers(1, 120))
                c = int(rng.integers(0, L)) if rng.random() < 0.3 else 0
                if len(m.free) < -(-c // P):
                    break
                arrivals.pop(0)
                m.add(L, int(rng.integers(0, 8)), c)
            states_before = [(r["state"], r["nc"]) for r in m.reqs]
            p = m.step()
            assert p["num_tokens"] <= tau
            for i, r in enumerate(m.reqs):
                if states_before[i][0] == m.RUNNING and r["state"] == m.WAITING:
                    preempted_total += 1
                    assert r["nc"] == 0 and r["left"] == states_before[i][1] and not r["pages"]
                    assert i not in p["req_ids"]
            for s, i in enumerate(p["req_ids"]):
                if s < p["num_decodes"]:
                    steps_run[i] = steps_run.get(i, 0) + 1
            m.commit()
            owned = [pg for r in m.reqs for pg in r["pages"]]
            assert len(owned) == len(set(owned)) and len(owned) + len(m.free) == N
            assert set(owned).isdisjoint(set(m.free))
            for r in m.reqs:
                if r["state"] == m.FINISHED:
                    assert not r["pages"]
                else:
                    assert len(r["pages"]) == -(-r["nc"] // P)
        for i, r in enumerate(m.reqs):
            assert steps_run.get(i, 0) == r["generated"]
            if r["state"] == m.FINISHED:
                assert r["generated"] == r["max_new"]
    assert preempted_total > 0  # the random pools are small enough to exercise preemption


# ------------------------------------------------------------------------------------------
# QKV projection
# ------------------------------------------------------------------------------------------

def test_linear_brute_force(oracle_mod):
    rng = np.random.default_rng(3)
    for T, K, N in ((1, 1, 1), (3, 5, 4), (7, 16, 9)):
        x = oracle_mod.round_to(rng.standard_normal((T, K)), "bf16")
        w = oracle_mod.round_to(rng.standard_normal((N, K)), "bf16")
        ref = np.zeros((T, N))
        for t in range(T):
            for n in range(N):
                acc = 0.0
                for k in range(K):
                    acc += x[t, k] * w[n, k]
                ref[t, n] = acc
        assert np.array_equal(oracle_mod.linear(x, w, "bf16"), oracle_mod.round_to(ref, "bf16"))
        assert np.array_equal(oracle_mod.linear(x, w, "fp32"), oracle_mod.round_to(ref, "fp32"))


def test_linear_identity_and_selection(oracle_mod):
    rng = np.random.default_rng(4)
    x = oracle_mod.round_to(rng.standard_normal((6, 8)), "bf16")
    assert np.array_equal(oracle_mod.linear(x, np.eye(8), "bf16"), x)
    perm = rng.permutation(8)
    assert np.array_equal(oracle_mod.linear(x, np.eye(8)[perm], "bf16"), x[:, perm])


def test_linear_single_rounding(oracle_mod):
    # 1 + 2^-8 is a tie between the bf16 neighbours 1 and 1 + 2^-7: nearest-even gives 1, and
    # 1 + 2^-8 + 2^-20 (a sum that a per-term rounding would lose) rounds up
    x = np.array([[1.0, 2.0 ** -8, 2.0 ** -20]])
    assert oracle_mod.linear(x[:, :2], np.ones((1, 2)), "bf16")[0, 0] == 1.0
    assert oracle_mod.linear(x, np.ones((1, 3)), "bf16")[0, 0] == 1.0 + 2.0 ** -7


def _check_plan_invariants(p, nc, left, tables, tau, max_chunk, P):
    q = np.diff(p["qo_indptr"])
    assert p["num_tokens"] == q.sum() <= tau
    nd = p["num_decodes"]
    rid = p["req_ids"]
    # decodes first, contiguous, each one token, in caller order; prefills after, in order
    assert all(left[r] == 0 for r in rid[:nd]) and all(q[:nd] == 1)
    assert all(left[r] > 0 for r in rid[nd:])
    assert list(rid[:nd]) == sorted(rid[:nd]) and list(rid[nd:]) == sorted(rid[nd:])
    for s, r in enumerate(rid):
        kv = nc[r] + q[s]
        npg = p["kv_page_indptr"][s + 1] - p["kv_page_indptr"][s]
        assert npg == -(-kv // P)
        assert 1 <= p["kv_last_page_len"][s] <= P
        assert (npg - 1) * P + p["kv_last_page_len"][s] == kv
        idx = p["kv_page_indices"][p["kv_page_indptr"][s]:p["kv_page_indptr"][s + 1]]
        assert np.array_equal(idx, tables[r][:npg])
        if s >= nd:
            assert q[s] <= left[r]
            if max_chunk:
                assert q[s] <= max_chunk
    # brute-force greedy: decodes take min(#decodes, tau); each prefill gets what was left
    decs = [r for r in range(len(nc)) if left[r] == 0]
    assert nd == min(len(decs), tau)
    assert p["num_deferred_decodes"] == len(decs) - nd


def test_plan_invariants_random(oracle_mod):
    rng = np.random.default_rng(7)
    P = 16
    for trial in range(300):
        n = int(rng.integers(0, 40))
        nc = rng.integers(0, 300, size=n).astype(np.int32)
        left = np.where(rng.random(n) < 0.6, 0, rng.integers(1, 400, size=n)).astype(np.int32)
        pages = [-(-(int(nc[i]) + max(1, int(left[i]))) // P) + int(rng.integers(0, 2))
                 for i in range(n)]
        tables = _tables(n, pages, rng.permutation(sum(pages) + 10))
        tau = int(rng.integers(1, 600))
        mc = int(rng.choice([0, 0, 8, 64]))
        p = oracle_mod.plan(nc, left, tables, tau, mc, P, sum(pages) + 10)
        assert p["status"] == 0
        _check_plan_invariants(p, nc, left, tables, tau, mc, P)
        # Greedy budget use: the first prefill that is not fully served got all that was left
        q = np.diff(p["qo_indptr"])
        used = p["num_decodes"]
        for s in range(p["num_decodes"], p["num_seqs"]):
            r = p["req_ids"][s]
            want = left[r] if not mc else min(left[r], mc)
            room = len(tables[r]) * P - nc[r]
            assert q[s] == min(want, tau - used, room)
            used += q[s]


def test_plan_sweep_shape(oracle_mod):
    # One prompt of L tokens, budget c, no decodes: K = ceil(L/c) chunks of c, last shorter.
    L = 1000
    for c in (64, 100, 256, 1000, 4096):
        nc, left = 0, L
        tab = [np.arange(-(-L // 16), dtype=np.int32)]
        qs = []
        while left > 0:
            p = oracle_mod.plan([nc], [left], tab, c, 0, 16, 1000)
            q = int(p["num_tokens"])
            qs.append(q)
            nc += q
            left -= q
        K = -(-L // c)
        assert len(qs) == K
        assert all(x == min(c, L) for x in qs[:-1]) and qs[-1] == L - (K - 1) * min(c, L)


def test_plan_errors_and_deferral(oracle_mod):
    tab = [np.array([0], dtype=np.int32), np.array([1], dtype=np.int32)]
    # decode at position 16 needs a second page
    assert oracle_mod.plan([16], [0], tab[:1], 8, 0, 16, 4)["status"] == oracle_mod.NO_PAGES
    # page id outside the pool
    assert oracle_mod.plan([3], [0], [np.array([9], np.int32)], 8, 0, 16, 4)["status"] == 1
    assert oracle_mod.plan([3], [0], tab[:1], 0, 0, 16, 4)["status"] == 1       # tau <= 0
    assert oracle_mod.plan([-1], [0], tab[:1], 8, 0, 16, 4)["status"] == 1      # negative
    # more decodes than budget: first tau run, the rest are deferred
    tabs = [np.array([i], dtype=np.int32) for i in range(5)]
    p = oracle_mod.plan([1] * 5, [0] * 5, tabs, 3, 0, 16, 5)
    assert p["status"] == 0 and p["num_decodes"] == 3 and p["num_deferred_decodes"] == 2
    assert list(p["req_ids"]) == [0, 1, 2]
    # capacity: counts are reported
    p = oracle_mod.plan([1] * 5, [0] * 5, tabs, 8, 0, 16, 5, cap_seqs=2)
    assert p["status"] == oracle_mod.CAPACITY and p["num_seqs"] == 5


# ------------------------------------------------------------------------------------------
# Rounding
# ------------------------------------------------------------------------------------------

def test_bf16_rounding_matches_torch(oracle_mod):
    import torch
    rng = np.random.default_rng(3)
    x32 = np.concatenate([rng.standard_normal(20000).astype(np.float32),
                          (rng.standard_normal(2000) * 1e-38).astype(np.float32),
                          (rng.standard_normal(2000) * 1e30).astype(np.float32)])
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle_mod.round_to(x32.astype(np.float64), "bf16")
    assert np.array_equal(got, ref)


def test_bf16_rounding_ties_and_neighbours(oracle_mod):
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties go to the even mantissa (1.0);
    # 1 + 3*2^-8 is halfway between 1+2^-7 and 1+2^-6: goes to 1 + 2^-6.
    assert oracle_mod.bf16_value(1 + 2 ** -8) == 1.0
    assert oracle_mod.bf16_value(1 + 3 * 2 ** -8) == 1 + 2 ** -6
    assert oracle_mod.bf16_value(1 + 2 ** -8 + 2 ** -40) == 1 + 2 ** -7
    # doubles strictly between fp32 values: result is the nearer bf16 neighbour
    rng = np.random.default_rng(4)
    for x in rng.standard_normal(2000) * 3:
        r = oracle_mod.bf16_value(x)
        e = np.floor(np.log2(abs(x)))
        ulp = 2.0 ** (e - 7)
        assert abs(r - x) <= ulp / 2 + 1e-300
        assert (r / ulp) == np.round(r / ulp)


def test_fp32_rounding(oracle_mod):
    x = np.random.default_rng(5).standard_normal(1000)
    assert np.array_equal(oracle_mod.round_to(x, "fp32"), x.astype(np.float32).astype(np.float64))


# ------------------------------------------------------------------------------------------
# Rotary embedding
# ------------------------------------------------------------------------------------------

def _complex_rope(x, pos, theta):
    """Split-half RoPE as complex multiplication: z_i = x_i + i x_{i+d/2} times e^{i p w_i}."""
    d = x.shape[-1]
    h = d // 2
    w = np.power(theta, -np.arange(h) * 2.0 / d)
    z = x[..., :h] + 1j * x[..., h:]
    z = z * np.exp(1j * pos[:, None, None] * w[None, None, :])
    return np.concatenate([z.real, z.imag], axis=-1)


def test_rope_properties(oracle_mod):
    rng = np.random.default_rng(11)
    d = 64
    x = rng.standard_normal((50, 3, d))
    pos = rng.integers(0, 40000, size=50).astype(np.int32)
    y = oracle_mod.rope(x, pos)
    # position 0 is the identity
    assert np.array_equal(oracle_mod.rope(x, np.zeros(50, np.int32)), x)
    # an isometry on every rotated pair
    h = d // 2
    assert np.allclose(x[..., :h] ** 2 + x[..., h:] ** 2, y[..., :h] ** 2 + y[..., h:] ** 2,
                       rtol=1e-12, atol=1e-12)
    # equal to complex multiplication (a library-level formulation of the same rotation)
    assert np.allclose(y, _complex_rope(x, pos.astype(np.float64), 10000.0), atol=1e-9)
    # relative position: <R(m) q, R(n) k> = <R(m - n) q, k>
    q = rng.standard_normal((1, 1, d))
    k = rng.standard_normal((1, 1, d))
    for m, n in ((5, 3), (1000, 17), (31000, 30000)):
        lhs = np.sum(oracle_mod.rope(q, np.array([m], np.int32)) *
                     oracle_mod.rope(k, np.array([n], np.int32)))
        rhs = np.sum(oracle_mod.rope(q, np.array([m - n], np.int32)) * k)
        assert abs(lhs - rhs) < 1e-9
    # composition: R(a) R(b) = R(a + b)
    a = oracle_mod.rope(oracle_mod.rope(q, np.array([123], np.int32)), np.array([456], np.int32))
    assert np.allclose(a, oracle_mod.rope(q, np.array([579], np.int32)), atol=1e-12)


# ------------------------------------------------------------------------------------------
# Attention
# ------------------------------------------------------------------------------------------

def _brute(q, pos, k, v, scale):
    """Masked-softmax matrix formulation, independent of the oracle's loop order."""
    nrows, hq, d = q.shape
    hkv = k.shape[1]
    G = hq // hkv
    out = np.empty_like(q)
    lse = np.empty((nrows, hq))
    for h in range(hq):
        K = k[:, h // G, :]
        V = v[:, h // G, :]
        S = (q[:, h, :] @ K.T) * scale
        mask = np.arange(k.shape[0])[None, :] > pos[:, None]
        S = np.where(mask, -np.inf, S)
        out[:, h, :] = softmax(S, axis=1) @ V
        mx = S.max(axis=1)
        lse[:, h] = mx + np.log(np.exp(S - mx[:, None]).sum(axis=1))
    return out, lse


@pytest.mark.parametrize("hq,hkv,d,kv_len", [(2, 2, 8, 1), (4, 2, 16, 37), (6, 3, 32, 70),
                                              (8, 1, 64, 130)])
def test_attention_brute_force(oracle_mod, hq, hkv, d, kv_len):
    rng = np.random.default_rng(hq * 1000 + kv_len)
    pos = np.sort(rng.choice(kv_len, size=min(kv_len, 9), replace=False)).astype(np.int32)
    q = rng.standard_normal((pos.size, hq, d)) * 2
    k = rng.standard_normal((kv_len, hkv, d))
    v = rng.standard_normal((kv_len, hkv, d))
    o, lse = oracle_mod.attention(q, pos, k, v)
    ob, lb = _brute(q, pos, k, v, 1.0 / np.sqrt(d))
    assert np.allclose(o, ob, atol=1e-12, rtol=1e-10)
    assert np.allclose(lse, lb, atol=1e-12, rtol=1e-12)


def test_attention_closed_forms(oracle_mod):
    rng = np.random.default_rng(21)
    hq, hkv, d, L = 4, 2, 16, 25
    q = rng.standard_normal((L, hq, d))
    k = rng.standard_normal((L, hkv, d))
    pos = np.arange(L, dtype=np.int32)
    # V == 1 -> every output is 1 (weights sum to one)
    o, _ = oracle_mod.attention(q, pos, k, np.ones((L, hkv, d)))
    assert np.allclose(o, 1.0, atol=1e-14)
    # one-hot V: output column j is the probability of key j; rows sum to 1, zero beyond pos
    v = np.zeros((L, hkv, L))
    for j in range(L):
        v[j, :, j] = 1.0
    qL = rng.standard_normal((L, hq, L))
    kL = rng.standard_normal((L, hkv, L))
    o, _ = oracle_mod.attention(qL, pos, kL, v)
    assert np.allclose(o.sum(axis=2), 1.0, atol=1e-13)
    assert np.all(o >= 0)
    for t in range(L):
        assert np.all(o[t, :, t + 1:] == 0.0)
    # kv_len 1 -> the single value
    o, lse = oracle_mod.attention(q[:1], np.array([0], np.int32), k[:1], k[:1] * 3)
    assert np.array_equal(o[0], np.repeat(k[:1] * 3, hq // hkv, axis=1)[0])
    # K == 0 -> uniform weights: prefix mean of V
    v = rng.standard_normal((L, hkv, d))
    o, lse = oracle_mod.attention(q, pos, np.zeros((L, hkv, d)), v)
    for t in range(L):
        mean = v[:t + 1].mean(axis=0)
        assert np.allclose(o[t], np.repeat(mean, hq // hkv, axis=0), atol=1e-13)
        assert np.allclose(lse[t], np.log(t + 1), atol=1e-13)
    # two keys, scale 1/sqrt(d): weight of key 0 is the logistic of the score gap
    d = 64
    a = 3.0
    q2 = np.zeros((1, 1, d)); q2[0, 0, 0] = a
    k2 = np.zeros((2, 1, d)); k2[0, 0, 0] = 1.0
    v2 = np.zeros((2, 1, d)); v2[0, 0, 1] = 1.0; v2[1, 0, 2] = 1.0
    o, _ = oracle_mod.attention(q2, np.array([1], np.int32), k2, v2)
    w0 = expit(a / np.sqrt(d))
    assert abs(o[0, 0, 1] - w0) < 1e-15 and abs(o[0, 0, 2] - (1 - w0)) < 1e-15


def test_attention_causality_and_gqa(oracle_mod):
    rng = np.random.default_rng(31)
    hq, hkv, d, L = 8, 2, 32, 40
    q = rng.standard_normal((L, hq, d))
    k = rng.standard_normal((L, hkv, d))
    v = rng.standard_normal((L, hkv, d))
    pos = np.arange(L, dtype=np.int32)
    o, lse = oracle_mod.attention(q, pos, k, v)
    # perturbing keys/values after position p leaves row p unchanged
    p0 = 17
    k2, v2 = k.copy(), v.copy()
    k2[p0 + 1:] += 5.0
    v2[p0 + 1:] -= 3.0
    o2, _ = oracle_mod.attention(q, pos, k2, v2)
    assert np.array_equal(o[:p0 + 1], o2[:p0 + 1])
    assert not np.allclose(o[p0 + 1:], o2[p0 + 1:])
    # GQA == MHA with each kv head replicated for its group of q heads (contiguous groups)
    G = hq // hkv
    om, lm = oracle_mod.attention(q, pos, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1))
    assert np.array_equal(o, om) and np.array_equal(lse, lm)


# ------------------------------------------------------------------------------------------
# Chunked prefill == one-shot prefill (in the oracle: bit for bit)
# ------------------------------------------------------------------------------------------

def _run_scenario(oracle_mod, wl):
    from chunked_prefill_paged_ca_amd.workload import StreamCursor
    sess = oracle_mod.Session(wl)
    cur = StreamCursor(wl)
    outs = []
    for _ in range(wl.steps):
        p = sess.plan()
        assert p["status"] == 0
        q, k, v = cur.take(p["req_ids"], np.diff(p["qo_indptr"]))
        r = sess.step(p, q, k, v)
        outs.append((p, r))
    return sess, outs


def test_chunked_equals_one_shot_tiny(oracle_mod):
    from chunked_prefill_paged_ca_amd.workload import make_config
    chunked = make_config(1)
    one = make_config(1, one_shot=True)
    s1, outs1 = _run_scenario(oracle_mod, chunked)
    s2, outs2 = _run_scenario(oracle_mod, one)
    prompt = 3  # request index of the prompt in the chunked scenario
    assert np.array_equal(s1.k[prompt], s2.k[0]) and np.array_equal(s1.v[prompt], s2.v[0])
    rows = []
    for p, r in outs1:
        nd = p["num_decodes"]
        # every step: 3 decodes first, then one chunk of 16 (max_chunk)
        assert nd == 3 and np.diff(p["qo_indptr"])[-1] == 16
        b = p["qo_indptr"][nd]
        rows.append((r["o"][b:], r["lse"][b:], r["pos"][b:]))
    o_c = np.concatenate([x[0] for x in rows])
    l_c = np.concatenate([x[1] for x in rows])
    pos_c = np.concatenate([x[2] for x in rows])
    assert np.array_equal(pos_c, np.arange(64))
    o_1, l_1 = outs2[0][1]["o"], outs2[0][1]["lse"]
    assert np.array_equal(o_c, o_1) and np.array_equal(l_c, l_1)
    # decodes: contexts 40, 57, 100 at step 1, one more key per step
    for step, (p, r) in enumerate(outs1):
        assert list(r["pos"][:3]) == [39 + step, 56 + step, 99 + step]
