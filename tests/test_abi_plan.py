"""CPU tests of the C ABI: the library loads, exports every declared symbol, and its host plan
equals the oracle's plan bit for bit (statuses, counts and every metadata array)."""
import ctypes

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import chunked_prefill_paged_ca_amd as ca
from chunked_prefill_paged_ca_amd import binding
from chunked_prefill_paged_ca_amd.workload import make_config


@pytest.fixture(scope="module")
def L():
    from __graft_entry__ import ensure_built
    ensure_built()
    return ca.lib()


def test_exports_every_header_symbol(L):
    syms = ca.header_symbols()
    assert {"ca_plan_batch", "ca_append_kv_rope", "ca_mixed_attention", "ca_create",
            "ca_destroy", "ca_status_string", "ca_last_error"} <= set(syms)
    for s in syms:
        assert hasattr(L, s), s


def test_library_leaves_none_of_its_own_symbols_undefined(L):
    """Every symbol of the library's own namespace is defined in libca.so (a kernel whose host
    handle was not emitted would otherwise only fail to load on a machine with a GPU)."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--undefined-only", binding.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    own = [ln for ln in out.splitlines() if "_ZN2ca" in ln or " ca_" in ln]
    assert own == [], own


def test_probe_library_exports_its_entry_point(L):
    """The measurement probe is its own library (not part of the ca_* ABI); it loads without a
    GPU and exports its one C entry point."""
    import ctypes
    from chunked_prefill_paged_ca_amd import peaks
    probe = ctypes.CDLL(peaks.PROBE_LIB)
    for sym in ("ca_probe_mfma_rate", "ca_probe_read_rate"):
        assert hasattr(probe, sym)
        assert not hasattr(L, sym)


def test_status_strings(L):
    for s in range(6):
        assert binding.status_string(s)


def _compare(oracle_mod, nc, left, tables, tau, mc, P, pool, cap_seqs=None, cap_pages=None,
             align=0):
    o = oracle_mod.plan(nc, left, tables, tau, mc, P, pool, cap_seqs=cap_seqs, cap_pages=cap_pages,
                        chunk_align=align)
    p = ca.plan_batch(nc, left, tables, tau, mc, P, pool, cap_seqs=cap_seqs, cap_pages=cap_pages,
                      raise_on_error=False, chunk_align=align)
    assert p.status == o["status"], (p.status, o["status"], binding.last_error())
    if o["status"] in (0, 3):
        for k in ("num_seqs", "num_decodes", "num_tokens", "num_pages", "num_deferred_decodes"):
            assert getattr(p, k) == o[k], k
    if o["status"] == 0:
        a = p.arrays()
        for k in ("req_ids", "qo_indptr", "kv_page_indptr", "kv_page_indices", "kv_last_page_len"):
            assert np.array_equal(a[k], o[k]), k
        assert p.generation > 0
    return p, o


@pytest.mark.parametrize("cfg", [1, 2, 4, 5])
@pytest.mark.parametrize("align", [0, 32])
def test_plan_matches_oracle_on_configs(L, oracle_mod, cfg, align):
    wl = make_config(cfg)
    p, o = _compare(oracle_mod, wl.num_computed, wl.num_prompt_left, wl.block_tables,
                    wl.token_budget, wl.max_chunk, wl.page_size, wl.num_pool_pages, align=align)
    assert o["status"] == 0 and o["num_tokens"] <= wl.token_budget


@pytest.mark.parametrize("c", [64, 256, 2048, 8192])
def test_plan_sweep_matches_oracle(L, oracle_mod, c):
    wl = make_config(3, chunk=c)
    nc, left = wl.num_computed.copy(), wl.num_prompt_left.copy()
    for _ in range(wl.steps):
        p, o = _compare(oracle_mod, nc, left, wl.block_tables, wl.token_budget, 0, 16,
                        wl.num_pool_pages)
        q = o["num_tokens"]
        assert q == min(c, int(left[0]))
        nc[0] += q
        left[0] -= q
    assert left[0] == 0


req = st.tuples(st.integers(0, 200), st.integers(0, 300), st.integers(0, 3))


@settings(max_examples=300, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(reqs=st.lists(req, min_size=0, max_size=30), tau=st.integers(1, 700),
       mc=st.sampled_from([0, 0, 1, 7, 64]), P=st.sampled_from([1, 16, 5]),
       decode_frac=st.floats(0, 1), seed=st.integers(0, 2 ** 31 - 1),
       bad_page=st.booleans(), cap_cut=st.integers(0, 3),
       align=st.sampled_from([0, 0, 1, 16, 32, 100]))
def test_plan_matches_oracle_random(L, oracle_mod, reqs, tau, mc, P, decode_frac, seed,
                                    bad_page, cap_cut, align):
    rng = np.random.default_rng(seed)
    nc, left, tables = [], [], []
    next_page = 0
    for (c, lft, extra) in reqs:
        is_dec = rng.random() < decode_frac
        lft = 0 if is_dec else max(1, lft)
        need = -(-(c + max(1, lft)) // P)
        npg = max(0, need + extra - 1)  # sometimes one page short (NO_PAGES / room cap)
        tables.append(np.arange(next_page, next_page + npg, dtype=np.int32))
        next_page += npg
        nc.append(c)
        left.append(lft)
    pool = max(next_page, 1)
    if bad_page and tables and tables[0].size:
        tables[0] = tables[0].copy()
        tables[0][0] = pool + 3
    cap_seqs = max(0, len(reqs) - cap_cut) if cap_cut == 3 else None
    _compare(oracle_mod, nc, left, tables, tau, mc, P, pool, cap_seqs=cap_seqs, align=align)


def test_plan_rejects_bad_params(L, oracle_mod):
    t = [np.array([0], np.int32)]
    for args in ((t, 0, 0, 16, 4), (t, 8, -1, 16, 4), (t, 8, 0, 0, 4), (t, 8, 0, 16, 0)):
        _compare(oracle_mod, [1], [0], *args)
    _compare(oracle_mod, [-3], [0], t, 8, 0, 16, 4)
    _compare(oracle_mod, [1], [0], t, 8, 0, 16, 4, align=-1)
    _compare(oracle_mod, [3], [-1], t, 8, 0, 16, 4)


def test_plan_validate_write_targets(L):
    """ca_plan_validate: two block tables that share a page both sequences append to are refused
    with CA_VALIDATE_WRITE_TARGETS (and pass the range checks without it); a shared read-only
    prefix page is fine; a table that lists a page twice collides with itself; a page id beyond
    a smaller pool is refused."""
    P = 16
    # A: 20-token prompt on pages [3, 5] (slots 0..15 of 3, 0..3 of 5); B: 10 tokens on [5]
    overlap = ca.plan_batch([0, 0], [20, 10], [np.array([3, 5]), np.array([5])], 64, 0, P, 8)
    overlap.validate(8)
    with pytest.raises(ca.CaError, match="sequences 0 and 1 both append to page 5 slot 0"):
        overlap.validate(8, write_targets=True)
    # two decodes whose tables end on the same page: both append position 16 to page 6 slot 0
    dec = ca.plan_batch([16, 16], [0, 0], [np.array([1, 6]), np.array([2, 6])], 64, 0, P, 8)
    dec.validate(8)
    with pytest.raises(ca.CaError, match="both append to page 6 slot 0"):
        dec.validate(8, write_targets=True)
    # a shared prefix page (read by both, written by neither) is consistent
    shared = ca.plan_batch([16, 16], [4, 4], [np.array([3, 6]), np.array([3, 7])], 64, 0, P, 8)
    shared.validate(8, write_targets=True)
    # one table naming page 2 twice: positions 0..3 and 16..19 land in the same slots
    twice = ca.plan_batch([0], [20], [np.array([2, 2])], 64, 0, P, 8)
    with pytest.raises(ca.CaError, match="sequences 0 and 0 both append to page 2 slot 0"):
        twice.validate(8, write_targets=True)
    # the pool bound is the caller's: page 7 is outside a 7-page pool
    with pytest.raises(ca.CaError, match="outside the pool"):
        shared.validate(7)
    with pytest.raises(ca.CaError, match="unknown flags"):
        lib_flags = 4
        binding._check(L.ca_plan_validate(ctypes.byref(shared.c), 8, lib_flags), "ca_plan_validate")


# ------------------------------------------------------------------------------------------
# ca_sched: the serving loop, library against the oracle's model, round by round
# ------------------------------------------------------------------------------------------

def _run_loop_both(oracle_mod, rng, N, tau, mc, align, rounds, arrivals, P=16):
    lib_s = ca.Scheduler(tau, mc, P, N, chunk_align=align)
    ref = oracle_mod.SchedModel(tau, mc, P, N, align)
    pending = list(arrivals)
    preempts = 0
    for rnd in range(rounds):
        while pending and pending[0][0] <= rnd:
            _, L, new, c = pending[0]
            assert lib_s.free_pages() == len(ref.free)
            if len(ref.free) < -(-c // P):
                break
            pending.pop(0)
            assert lib_s.add(L, new, c) == ref.add(L, new, c)
        p = lib_s.step()
        o = ref.step()
        for k in ("num_seqs", "num_decodes", "num_tokens", "num_pages", "num_deferred_decodes"):
            assert getattr(p, k) == o[k], (rnd, k)
        a = p.arrays()
        for k in ("req_ids", "qo_indptr", "kv_page_indptr", "kv_page_indices", "kv_last_page_len"):
            assert np.array_equal(a[k], o[k]), (rnd, k)
        lib_s.commit()
        ref.commit()
        for i, r in enumerate(ref.reqs):
            g = lib_s.get(i)
            assert g["state"] == r["state"] and g["num_computed"] == r["nc"], (rnd, i)
            assert g["num_generated"] == r["generated"] and g["num_preemptions"] == r["preemptions"]
            assert np.array_equal(g["block_table"], np.asarray(r["pages"], dtype=np.int32))
            preempts += r["preemptions"]
    return preempts


def test_sched_matches_oracle_random(L, oracle_mod):
    rng = np.random.default_rng(5)
    total_preempts = 0
    for trial in range(60):
        N = int(rng.integers(3, 60))
        tau = int(rng.integers(1, 300))
        mc = int(rng.choice([0, 0, 24, 64]))
        align = int(rng.choice([0, 0, 8, 32]))
        arr = []
        for _ in range(int(rng.integers(1, 16))):
            Lp = int(rng.integers(1, 200))
            c = int(rng.integers(0, Lp)) if rng.random() < 0.3 else 0
            arr.append((int(rng.integers(0, 40)), Lp, int(rng.integers(0, 10)), c))
        arr.sort(key=lambda x: x[0])
        total_preempts += _run_loop_both(oracle_mod, rng, N, tau, mc, align, 90, arr)
    assert total_preempts > 0


def test_sched_worked_example_library(L):
    s = ca.Scheduler(512, 0, 16, 20000)
    for _ in range(80):
        s.add(2, 10, 1)
    s.step()
    s.commit()
    P = s.add(1500, 10, 1200)
    Q = s.add(2948, 10, 2048)
    p = s.step()
    a = p.arrays()
    assert p.num_decodes == 80 and list(np.diff(a["qo_indptr"])[-2:]) == [300, 132]
    assert list(a["req_ids"][-2:]) == [P, Q]
    s.commit()
    p = s.step()
    assert p.num_decodes == 81 and p.num_tokens == 512


def test_sched_errors(L):
    s = ca.Scheduler(64, 0, 16, 4)
    with pytest.raises(binding.CaError):
        s.commit()                      # nothing planned
    with pytest.raises(binding.CaError):
        s.add(10, 1, 10)                # num_cached must stay below the prompt
    with pytest.raises(binding.CaError):
        s.add(0, 1)                     # empty prompt
    with pytest.raises(binding.CaError):
        s.add(100, 1, 80)               # prefix needs 5 pages, the pool has 4
    with pytest.raises(binding.CaError):
        s.add(40, 1, 20, cached_pages=np.array([1, 7], dtype=np.int32))  # page outside the pool
    r = s.add(40, 1, 20, cached_pages=np.array([2, 3], dtype=np.int32))
    assert s.free_pages() == 2 and list(s.get(r)["block_table"]) == [2, 3]
    with pytest.raises(binding.CaError):
        s.add(40, 1, 20, cached_pages=np.array([3, 0], dtype=np.int32))  # page 3 is taken
    assert s.free_pages() == 2
    s.step()
    with pytest.raises(binding.CaError):
        s.step()                        # the planned round is not committed
    with pytest.raises(binding.CaError):
        s.add(5, 1)                     # nor can requests join before the commit
    s.commit()
    with pytest.raises(binding.CaError):
        s.get(7)
    with pytest.raises(binding.CaError):
        ca.Scheduler(64, 0, 16, 4, chunk_align=-2)
