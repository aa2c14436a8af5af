"""ca_mixed_attention_noalloc against ca_mixed_attention, through the C ABI, on the same inputs.

The no-alloc entry point keeps its workspace in the library's static scratch array; its results
must match the ordinary entry point's to the attention bar (2e-2 in bf16, 1e-4 in fp32; lse 2e-3 /
1e-5), on consecutive calls that leave the previous call's contents in the array -- the second
call smaller than the first -- and on a step whose chunk partials do not fit in the array (the
no-alloc call then runs longer key splits).
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

TOL_O = {"bf16": 2e-2, "fp32": 1e-4}
TOL_LSE = {"bf16": 2e-3, "fp32": 1e-5}


@pytest.fixture(scope="module")
def ctx():
    import torch
    from __graft_entry__ import ensure_built
    ensure_built()
    import chunked_prefill_paged_ca_amd as ca
    assert torch.cuda.is_available()
    c = ca.create(0)
    yield c
    c.close()


def _step_both(ctx, wl, kc, vc, label):
    """Append once, then attention through both entry points; returns the worst differences."""
    import torch
    import chunked_prefill_paged_ca_amd as ca
    from chunked_prefill_paged_ca_amd.workload import StreamCursor
    from tests import harness as H
    plan = H.lib_plan(wl, wl.num_computed, wl.num_prompt_left)
    a = plan.arrays()
    q, k, v = StreamCursor(wl).take(a["req_ids"], np.diff(a["qo_indptr"]))
    desc = ca.make_desc(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.page_size, wl.dtype)
    q_in, k_in, v_in = (H.to_device(x, wl.dtype) for x in (q, k, v))
    q_rot = torch.empty_like(q_in)
    ctx.append_kv_rope(desc, plan, q_in, q_rot, k_in, v_in, kc, vc, wl.num_pool_pages)
    T = plan.num_tokens
    o_ref, o_na = torch.empty_like(q_rot), torch.full_like(q_rot, float("nan"))
    l_ref = torch.empty((T, wl.num_q_heads), dtype=torch.float32, device="cuda")
    l_na = torch.full_like(l_ref, float("nan"))
    ctx.mixed_attention(desc, plan, q_rot, kc, vc, wl.num_pool_pages, o_ref, l_ref)
    ctx.mixed_attention(desc, plan, q_rot, kc, vc, wl.num_pool_pages, o_na, l_na, no_alloc=True)
    torch.cuda.synchronize()
    assert torch.isfinite(o_na.float()).all() and torch.isfinite(l_na).all(), label
    err = (o_na.float() - o_ref.float()).abs().max().item()
    lerr = (l_na - l_ref).abs().max().item()
    print(f"[no-alloc {label}] T={T} seqs={plan.num_seqs} max|o_na - o|={err:.3e} "
          f"max|lse_na - lse|={lerr:.3e}", flush=True)
    assert err <= TOL_O[wl.dtype] and lerr <= TOL_LSE[wl.dtype], (label, err, lerr)


def test_noalloc_matches_ordinary_entry_point(ctx):
    """Two calls in a row: the Mistral-7B step (80 decodes + two chunks, 512 rows), then a much
    smaller mixed batch of another shape (6 sequences, 12/4 heads) on the array the first call
    left behind; then the tiny fp32 batch (the plain kernel's partials in the array)."""
    from chunked_prefill_paged_ca_amd.workload import Workload, make_config
    from tests import harness as H
    wl = make_config(2)
    kc, vc = H.random_pool(wl, seed=2)
    _step_both(ctx, wl, kc, vc, "mistral-7b step")
    del kc, vc
    nc = np.array([0, 15, 31, 0, 16, 40], np.int32)
    left = np.array([0, 0, 0, 1, 1, 33], np.int32)
    stream = np.array([1, 1, 1, 1, 1, 33], np.int32)
    pool = 64
    perm = np.random.default_rng(9).permutation(pool).astype(np.int32)
    tabs, it = [], 0
    for r in range(6):
        n = -(-int(nc[r] + stream[r]) // 16)
        tabs.append(perm[it:it + n]); it += n
    small = Workload(name="small", config=0, seed=77, num_q_heads=12, num_kv_heads=4, head_dim=128,
                     page_size=16, dtype="bf16", token_budget=64, max_chunk=0, num_pool_pages=pool,
                     num_computed=nc, num_prompt_left=left, block_tables=tabs, stream_len=stream)
    kc, vc = H.alloc_pool(small, fill=0.0)
    H.write_history(small, kc, vc)
    _step_both(ctx, small, kc, vc, "small batch")
    tiny = make_config(1)
    kc, vc = H.alloc_pool(tiny, fill=0.0)
    H.write_history(tiny, kc, vc)
    _step_both(ctx, tiny, kc, vc, "tiny fp32")


def test_noalloc_with_partials_beyond_the_array(ctx):
    """The Yi-34B step: its chunk rows' key splits need more partial space than the array holds,
    so the no-alloc call runs longer splits; same results to the bar."""
    from chunked_prefill_paged_ca_amd.workload import make_config
    from tests import harness as H
    wl = make_config(4)
    kc, vc = H.random_pool(wl, seed=4)
    _step_both(ctx, wl, kc, vc, "yi-34b step")
