"""GPU parity: the HIP path through the C ABI against the CPU oracle, on the same seeded inputs.

Bars (fixed before any kernel ran):
  * plan metadata and page indices: bit-exact;
  * rotated q and the appended K/V: at most 1 unit in the last place of the storage type (both
    sides round an fp64 rotation once; only a near-tie in the last bit may differ), history
    bit-exact;
  * attention output: max |o - o_oracle| <= 2e-2 in bf16 storage, <= 1e-4 in fp32 storage;
    lse within 2e-3 (bf16) / 1e-5 (fp32) -- scores are exact products of stored values summed in
    fp32, so lse error is fp32 summation error only.
Unused pool pages and the unused tail of every last page hold NaN, so a kernel that reads a
slot it should not see, or lets a masked slot's value through, fails.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

TOL_O = {"bf16": 2e-2, "fp32": 1e-4}
TOL_LSE = {"bf16": 2e-3, "fp32": 1e-5}


@pytest.fixture(scope="module")
def env():
    import torch
    from __graft_entry__ import ensure_built
    ensure_built()
    import chunked_prefill_paged_ca_amd as ca
    import oracle
    assert torch.cuda.is_available()
    ctx = ca.create(0)
    yield ctx, oracle
    ctx.close()


def _log(msg):
    print(msg, flush=True)


def run_and_check(ctx, oracle, wl, steps=None, rows_per_seq=None, track=None, pool=None,
                  check_cache=True, label="", packed=False):
    """Run `steps` steps on GPU and oracle; compare everything compared in the module docstring.

    rows_per_seq -- if set, attend-check only this many rows per sequence (sampled, incl. last).
    track        -- request indices the oracle keeps a cache for (default all).
    Returns per-step outputs for further checks.
    """
    import torch
    from chunked_prefill_paged_ca_amd.workload import StreamCursor
    from tests import harness as H

    dt = wl.dtype
    if pool is None:
        k_cache, v_cache = H.alloc_pool(wl)
        H.write_history(wl, k_cache, v_cache)
    else:
        k_cache, v_cache = pool
    sess = oracle.Session(wl, requests=track)
    cur = StreamCursor(wl)
    rng = np.random.default_rng(1234)
    results = []
    for step in range(steps or wl.steps):
        ref_plan = sess.plan()
        plan = H.lib_plan(wl, sess.num_computed, sess.num_prompt_left)
        a = plan.arrays()
        for k in ("req_ids", "qo_indptr", "kv_page_indptr", "kv_page_indices", "kv_last_page_len"):
            assert np.array_equal(a[k], ref_plan[k]), (label, step, k)
        q, k, v = cur.take(ref_plan["req_ids"], np.diff(ref_plan["qo_indptr"]))
        q_out, o, lse = H.gpu_step(ctx, wl, plan, q, k, v, k_cache, v_cache, packed=packed)
        torch.cuda.synchronize()
        rows = None
        if rows_per_seq is not None:
            sel = []
            qo = ref_plan["qo_indptr"]
            for s_ in range(len(qo) - 1):
                b, e = int(qo[s_]), int(qo[s_ + 1])
                pick = set([e - 1, b])
                if e - b > 2:
                    pick |= set(rng.choice(np.arange(b, e), size=min(rows_per_seq, e - b), replace=False).tolist())
                sel += sorted(pick)
            rows = np.asarray(sel)
        ref = sess.step(ref_plan, q, k, v, rows=rows)
        go = o.float().cpu().numpy().astype(np.float64)
        gl = lse.cpu().numpy().astype(np.float64)
        gq = q_out.float().cpu().numpy().astype(np.float64)
        uq = H.ulp_distance(gq, ref["q_rot"], dt)
        assert uq.max() <= 1.0, (label, step, "q_rot ulp", uq.max())
        # one rounding of the same fp64 value: only a last-bit difference of the device and host
        # sine/cosine can make a result differ, so mismatches are rare (a wrong rounding mode
        # would put them near one half)
        assert (uq > 0).mean() <= 1e-3, (label, step, "q_rot mismatch rate", (uq > 0).mean())
        mask = ~np.isnan(ref["o"][:, 0, 0])
        err = np.abs(go[mask] - ref["o"][mask]).max() if mask.any() else 0.0
        lerr = np.abs(gl[mask] - ref["lse"][mask]).max() if mask.any() else 0.0
        _log(f"[{label}] step {step}: T={plan.num_tokens} seqs={plan.num_seqs} "
             f"decodes={plan.num_decodes} rows checked={int(mask.sum())} max|do|={err:.3e} "
             f"max|dlse|={lerr:.3e} q-rot mismatches={int((uq > 0).sum())}")
        assert np.all(np.isfinite(go)), (label, step, "non-finite output")
        assert err <= TOL_O[dt], (label, step, err)
        assert lerr <= TOL_LSE[dt], (label, step, lerr)
        if check_cache:
            for r in (sess.k.keys()):
                kv_len = int(sess.num_computed[r])
                gk, gv = H.read_dense(k_cache, v_cache, wl.block_tables[r], wl.page_size, kv_len)
                uk = H.ulp_distance(gk, sess.k[r], dt)
                assert uk.max() <= 1.0, (label, step, r, "k cache ulp", uk.max())
                assert np.array_equal(gv, sess.v[r]), (label, step, r, "v cache")
        results.append((ref_plan, go, gl, ref))
    return results, (k_cache, v_cache), sess


def run_every_row(ctx, oracle, wl, k_cache, v_cache, hist, group=32, label=""):
    """One step of a large workload on the GPU, then EVERY row against the oracle.

    The GPU pool must already hold every request's history; `hist` holds the same histories as
    drawn ({r: (k, v)}).  The oracle keeps a dense fp64 cache per tracked request, so it is run
    in groups of `group` requests (a Session tracking only them, attending only their rows): its
    fp64 memory stays bounded while every decode row, every chunk row, and every appended K/V
    slot is compared.  Bars as in run_and_check."""
    import torch
    from chunked_prefill_paged_ca_amd.workload import StreamCursor
    from tests import harness as H

    dt = wl.dtype
    ref_plan = oracle.Session(wl, requests=[]).plan()
    plan = H.lib_plan(wl, wl.num_computed, wl.num_prompt_left)
    a = plan.arrays()
    for k in ("req_ids", "qo_indptr", "kv_page_indptr", "kv_page_indices", "kv_last_page_len"):
        assert np.array_equal(a[k], ref_plan[k]), (label, k)
    q, k, v = StreamCursor(wl).take(ref_plan["req_ids"], np.diff(ref_plan["qo_indptr"]))
    q_out, o, lse = H.gpu_step(ctx, wl, plan, q, k, v, k_cache, v_cache)
    torch.cuda.synchronize()
    go = o.float().cpu().numpy().astype(np.float64)
    gl = lse.cpu().numpy().astype(np.float64)
    gq = q_out.float().cpu().numpy().astype(np.float64)
    qo = ref_plan["qo_indptr"]
    req_ids = [int(r) for r in ref_plan["req_ids"]]
    seq_of = {r: s_ for s_, r in enumerate(req_ids)}
    checked = np.zeros(plan.num_tokens, dtype=bool)
    worst, lworst = 0.0, 0.0
    for g0 in range(0, len(req_ids), group):
        members = req_ids[g0:g0 + group]
        sess = oracle.Session(wl, requests=members, history=hist.__getitem__)
        rows = np.concatenate([np.arange(qo[seq_of[r]], qo[seq_of[r] + 1]) for r in members])
        ref = sess.step(ref_plan, q, k, v, rows=rows)
        if g0 == 0:
            uq = H.ulp_distance(gq, ref["q_rot"], dt)
            assert uq.max() <= 1.0 and (uq > 0).mean() <= 1e-3, (label, "q_rot", uq.max())
        err = np.abs(go[rows] - ref["o"][rows]).max()
        lerr = np.abs(gl[rows] - ref["lse"][rows]).max()
        assert np.all(np.isfinite(go[rows])), (label, g0, "non-finite output")
        assert err <= TOL_O[dt], (label, g0, err)
        assert lerr <= TOL_LSE[dt], (label, g0, lerr)
        worst, lworst = max(worst, err), max(lworst, lerr)
        checked[rows] = True
        _log(f"[{label}] requests {g0}..{g0 + len(members) - 1}: {rows.size} rows, max|do|={err:.3e} "
             f"max|dlse|={lerr:.3e}")
        # the slots this step appended, for every member
        for r in members:
            s_ = seq_of[r]
            n_new = int(qo[s_ + 1] - qo[s_])
            kv_len = int(sess.num_computed[r])
            gk, gv = H.read_positions(k_cache, v_cache, wl.block_tables[r], wl.page_size,
                                      kv_len - n_new, kv_len)
            uk = H.ulp_distance(gk, sess.k[r][kv_len - n_new:], dt)
            assert uk.max() <= 1.0, (label, r, "k cache ulp", uk.max())
            assert np.array_equal(gv, sess.v[r][kv_len - n_new:]), (label, r, "v cache")
        del sess, ref
    assert checked.all(), (label, "rows left unchecked", int((~checked).sum()))
    _log(f"[{label}] every row: T={plan.num_tokens} seqs={plan.num_seqs} decodes={plan.num_decodes} "
         f"max|do|={worst:.3e} max|dlse|={lworst:.3e}")
    return ref_plan, go, gl


@pytest.mark.parametrize("dt", ["fp32", "bf16"])
def test_tiny_chunked_matches_oracle_and_one_shot(env, dt):
    """Config 1: 4 steps of (3 decodes + a 16-row chunk), then the same prompt one-shot."""
    from chunked_prefill_paged_ca_amd.workload import make_config
    from tests import harness as H
    ctx, oracle = env
    wl = make_config(1, dtype=dt)
    res, (kc, vc), sess = run_and_check(ctx, oracle, wl, label=f"tiny-{dt}")
    one = make_config(1, one_shot=True, dtype=dt)
    res1, (kc1, vc1), sess1 = run_and_check(ctx, oracle, one, label=f"tiny-oneshot-{dt}")
    # chunked == one-shot on the GPU: the prompt's final cache bit-exact, outputs within tolerance
    gk, gv = H.read_dense(kc, vc, wl.block_tables[3], 16, 64)
    gk1, gv1 = H.read_dense(kc1, vc1, one.block_tables[0], 16, 64)
    assert np.array_equal(gk, gk1) and np.array_equal(gv, gv1)
    chunk_o = np.concatenate([go[p["qo_indptr"][p["num_decodes"]]:] for p, go, gl, ref in res])
    one_o = res1[0][1]
    assert np.abs(chunk_o - one_o).max() <= TOL_O[dt]


@pytest.mark.parametrize("variant", ["base", "peaky", "packed", "fp32"])
def test_mistral_mixed_full(env, variant):
    """Config 2 at full size: 80 decodes + P(300 on 1200) + Q(132 on 2048), every row checked
    (packed: q, k, v handed over as one packed projection-shaped array; fp32: the same step in
    fp32 storage, through the plain kernel, against the 1e-4 bar)."""
    from chunked_prefill_paged_ca_amd.workload import make_config
    ctx, oracle = env
    wl = make_config(2, peaky=(variant == "peaky"), dtype="fp32" if variant == "fp32" else None)
    res, _, _ = run_and_check(ctx, oracle, wl, label=f"mistral-{variant}", packed=(variant == "packed"))
    p = res[0][0]
    assert list(np.diff(p["qo_indptr"])[-2:]) == [300, 132] and p["num_tokens"] == 512


def test_mistral_value_one_every_row(env):
    """V == 1 everywhere: every output of every row must be exactly representable 1 (softmax
    weights sum to one) -- a property checked on all T x Hq x d outputs."""
    import torch
    from chunked_prefill_paged_ca_amd.workload import StreamCursor, make_config
    from tests import harness as H
    ctx, oracle = env
    wl = make_config(2, kv_value=1.0)
    kc, vc = H.alloc_pool(wl)
    H.write_history(wl, kc, vc)
    plan = H.lib_plan(wl, wl.num_computed, wl.num_prompt_left)
    q, k, v = StreamCursor(wl).take(plan.arrays()["req_ids"], np.diff(plan.arrays()["qo_indptr"]))
    _, o, lse = H.gpu_step(ctx, wl, plan, q, k, v, kc, vc)
    torch.cuda.synchronize()
    err = (o.float() - 1.0).abs().max().item()
    _log(f"[mistral V=1] max|o-1| = {err:.3e}")
    assert err <= 2 ** -8


def test_yi_share_every_row(env):
    """Config 4 at full size: 128 decodes + one 1920-row chunk at 14336 in the fused launch;
    every one of the 2048 rows (and every appended slot) against the oracle."""
    from chunked_prefill_paged_ca_amd.workload import make_config
    from tests import harness as H
    ctx, oracle = env
    wl = make_config(4)
    kc, vc = H.alloc_pool(wl)
    hist = H.draw_histories(wl, range(wl.n))
    H.write_history(wl, kc, vc, hist=hist)
    p, _, _ = run_every_row(ctx, oracle, wl, kc, vc, hist, label="yi-share")
    assert p["num_decodes"] == 128 and p["num_tokens"] == 2048


def test_yi_chunk_alone_whole_blocks(env):
    """The Yi-34B share's 1920-row chunk on 14336 cached keys with no decode rows beside it: its
    53 x 4 column blocks fill the device in one round with key ranges within 25 % of each other,
    so each block runs its whole key range in one workgroup (no split, no merge); sampled rows
    against the oracle."""
    from chunked_prefill_paged_ca_amd.workload import Workload, make_config
    ctx, oracle = env
    wl = make_config(4)
    keep = [r for r in range(wl.n) if not wl.is_decode(r)]
    uids = np.arange(wl.n) if wl.uids is None else wl.uids
    wl = Workload(**{**wl.__dict__, "num_computed": wl.num_computed[keep],
                     "num_prompt_left": wl.num_prompt_left[keep],
                     "block_tables": [wl.block_tables[r] for r in keep],
                     "stream_len": wl.stream_len[keep], "uids": uids[keep]})
    res, _, _ = run_and_check(ctx, oracle, wl, rows_per_seq=64, label="yi-chunk-alone")
    p = res[0][0]
    assert p["num_decodes"] == 0 and p["num_tokens"] == 1920


def test_llama70b_share_every_row(env):
    """Config 5 at full size on a fragmented 128K-page pool (unused pages hold device-drawn
    random values): 256 decodes + chunks 640@0, 512@6000, 128@30000; every one of the 1536 rows
    (and every appended slot) against the oracle, whose caches are built 32 requests at a time."""
    from chunked_prefill_paged_ca_amd.workload import make_config
    from tests import harness as H
    ctx, oracle = env
    wl = make_config(5)
    kc, vc = H.random_pool(wl, seed=5)
    hist = H.draw_histories(wl, range(wl.n))
    H.write_history(wl, kc, vc, hist=hist)
    p, _, _ = run_every_row(ctx, oracle, wl, kc, vc, hist, label="70b-share")
    assert p["num_decodes"] == 256 and p["num_tokens"] == 1536


@pytest.mark.parametrize("c,align", [(64, 0), (128, 0), (256, 0), (512, 0), (2048, 0), (257, 32)])
def test_sweep_chunked_vs_one_shot(env, c, align):
    """Config 3: one 8192-token prompt at token budget c (chunks snapped to multiples of `align`
    when set: 257 with 32 gives 32 chunks of 256) against the oracle (sampled rows each step),
    then against the GPU's own one-shot run: same final cache bit for bit."""
    from chunked_prefill_paged_ca_amd.workload import make_config
    from tests import harness as H
    ctx, oracle = env
    wl = make_config(3, chunk=c)
    wl.chunk_align = align
    if align:
        wl.steps = -(-8192 // (c - c % align))
    res, (kc, vc), _ = run_and_check(ctx, oracle, wl, rows_per_seq=6, check_cache=False,
                                     label=f"sweep-c{c}-a{align}")
    one = make_config(3, one_shot=True)
    res1, (kc1, vc1), _ = run_and_check(ctx, oracle, one, rows_per_seq=16, check_cache=False,
                                        label="sweep-oneshot")
    gk, gv = H.read_dense(kc, vc, wl.block_tables[0], 16, 8192)
    gk1, gv1 = H.read_dense(kc1, vc1, one.block_tables[0], 16, 8192)
    assert np.array_equal(gk, gk1) and np.array_equal(gv, gv1)
    chunk_o = np.concatenate([go for p, go, gl, ref in res])
    assert np.abs(chunk_o - res1[0][1]).max() <= TOL_O["bf16"]


def test_append_four_units_per_thread(env):
    """The append launch's widest layout: 2048 tokens of the Llama-13B shape (MHA, 40 + 40 heads)
    do not fit on the CUs at one rotation unit per thread, so each thread rotates four units and
    stores sixteen V elements.  The rotated q and every appended K/V slot against the oracle
    (attention sampled)."""
    from chunked_prefill_paged_ca_amd.workload import make_config
    ctx, oracle = env
    wl = make_config(3, chunk=2048)
    run_and_check(ctx, oracle, wl, steps=1, rows_per_seq=4, check_cache=True, label="append-u4")


@pytest.mark.parametrize("T,library", [(1, False), (7, False), (16, False), (17, False), (33, False),
                                       (80, False), (100, False), (256, False), (512, False),
                                       (523, False), (2048, False), (1, True), (80, True)])
def test_qkv_projection_matches_oracle(env, T, library):
    """The Mistral-7B q/k/v projection (hidden 4096 -> (32 + 2 x 8) x 128 features) over T
    tokens against the exact product rounded once.  T <= 16 runs the weight-streaming kernel
    (7: a ragged token tile), larger T the tiled MFMA kernel (17, 33, 80, 100: K split over
    several workgroups and summed; 523: a ragged last token block; 2048: many token blocks per
    weight tile) -- and in a context created with CA_PROJECTION_LIBRARY=1 the library GEMM.  The GPU sums K = 4096 exact bf16 products in
    fp32, whose error is at most K 2^-24 sum_k |x_k w_k| (the standard bound for a K-term
    floating-point sum); the bar is that bound plus one bf16 unit in the last place of the exact
    value.  Away from cancellation this means "equal or the neighbouring bf16 value"; an output
    near zero may be further off in ulps of its own tiny magnitude."""
    import torch
    import chunked_prefill_paged_ca_amd as ca
    from chunked_prefill_paged_ca_amd.workload import projection_inputs
    from tests import harness as H
    ctx, oracle = env
    Hq, Hkv, d, hidden = 32, 8, 128, 4096
    N = (Hq + 2 * Hkv) * d
    x, w = projection_inputs(T, hidden, N, seed=11 + T)
    desc = ca.make_desc(Hq, Hkv, d, 16, "bf16")
    out = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    if library:
        import os
        os.environ["CA_PROJECTION_LIBRARY"] = "1"
        try:
            pctx = ca.create(0)
        finally:
            del os.environ["CA_PROJECTION_LIBRARY"]
    else:
        pctx = ctx
    pctx.qkv_projection(desc, T, hidden, H.to_device(x, "bf16"), H.to_device(w, "bf16"), out)
    torch.cuda.synchronize()
    if library:
        pctx.close()
    _check_projection(oracle, x, w, out, f"T={T}")


def _check_projection(oracle, x, w, out, label):
    """The projection bar of test_qkv_projection_matches_oracle: the fp32 sum bound plus one bf16
    ulp of the exact value, and at most 1e-4 of the outputs more than one ulp off."""
    from tests import harness as H
    hidden = x.shape[1]
    got = out.float().cpu().numpy().astype(np.float64)
    ref = oracle.linear(x, w, "bf16")
    u = H.ulp_distance(got, ref, "bf16")
    sum_bound = hidden * 2.0 ** -24 * (np.abs(x.astype(np.float64)) @ np.abs(w.astype(np.float64)).T)
    allowed = sum_bound + np.abs(ref) * 2.0 ** -7 + 2.0 ** -133
    _log(f"[projection {label}] max ulp {u.max():.0f}, outputs not equal {(u > 0).mean():.5f}, "
         f"worst |err|/allowed {(np.abs(got - ref) / allowed).max():.3f}")
    assert np.all(np.abs(got - ref) <= allowed)
    assert (u > 1).mean() <= 1e-4


@pytest.mark.parametrize("bm,bn,split,T", [(128, 192, 1, 300), (128, 256, 2, 200), (256, 96, 2, 300),
                                           (256, 128, 1, 523), (32, 64, 5, 40), (96, 64, 7, 80),
                                           (64, 128, 3, 64)])
def test_projection_forced_tile_shapes(env, bm, bn, split, T):
    """Every tile shape the tiled projection kernel is built with, forced through
    CA_PROJECTION_TILE=bm,bn,split (a context created with it set), with ragged last token
    blocks (300 = 2 x 128 + 44, 523) and K splits that do not divide the 64 K stages evenly (5, 7,
    3: split i takes stages [64 i / n, 64 (i + 1) / n)), against the exact product at the bar of
    test_qkv_projection_matches_oracle."""
    import os
    import torch
    import chunked_prefill_paged_ca_amd as ca
    from chunked_prefill_paged_ca_amd.workload import projection_inputs
    from tests import harness as H
    _, oracle = env
    Hq, Hkv, d, hidden = 32, 8, 128, 4096
    N = (Hq + 2 * Hkv) * d
    x, w = projection_inputs(T, hidden, N, seed=101 + T + bm + bn + split)
    desc = ca.make_desc(Hq, Hkv, d, 16, "bf16")
    out = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    os.environ["CA_PROJECTION_TILE"] = f"{bm},{bn},{split}"
    try:
        pctx = ca.create(0)
    finally:
        del os.environ["CA_PROJECTION_TILE"]
    try:
        pctx.qkv_projection(desc, T, hidden, H.to_device(x, "bf16"), H.to_device(w, "bf16"), out)
        torch.cuda.synchronize()
    finally:
        pctx.close()
    _check_projection(oracle, x, w, out, f"tile {bm}x{bn} split {split} T={T}")


def test_projected_step_matches_oracle(env):
    """The Mistral-7B step fed from hidden states: projection, packed append, attention, against
    the oracle's projection (rounded once) -> RoPE -> attention.  The projections may differ in
    the last bf16 bit, so the bar here is on the attention output (2e-2) and lse (1e-2)."""
    import torch
    import chunked_prefill_paged_ca_amd as ca
    from chunked_prefill_paged_ca_amd.workload import make_config, projection_inputs
    from tests import harness as H
    ctx, oracle = env
    wl = make_config(2)
    Hq, Hkv, d, hidden = wl.num_q_heads, wl.num_kv_heads, wl.head_dim, 4096
    N = (Hq + 2 * Hkv) * d
    kc, vc = H.alloc_pool(wl)
    H.write_history(wl, kc, vc)
    sess = oracle.Session(wl)
    ref_plan = sess.plan()
    plan = H.lib_plan(wl, wl.num_computed, wl.num_prompt_left)
    T = plan.num_tokens
    x, w = projection_inputs(T, hidden, N, seed=29)
    desc = ca.make_desc(Hq, Hkv, d, wl.page_size, wl.dtype)
    qkv = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    ctx.qkv_projection(desc, T, hidden, H.to_device(x, "bf16"), H.to_device(w, "bf16"), qkv)
    q_rot = torch.empty((T, Hq, d), dtype=torch.bfloat16, device="cuda")
    ctx.append_kv_rope_packed(desc, plan, qkv, q_rot, kc, vc, wl.num_pool_pages)
    o = torch.empty_like(q_rot)
    lse = torch.empty((T, Hq), dtype=torch.float32, device="cuda")
    ctx.mixed_attention(desc, plan, q_rot, kc, vc, wl.num_pool_pages, o, lse)
    torch.cuda.synchronize()
    ref_qkv = oracle.linear(x, w, "bf16").reshape(T, Hq + 2 * Hkv, d)
    ref = sess.step(ref_plan, ref_qkv[:, :Hq], ref_qkv[:, Hq:Hq + Hkv], ref_qkv[:, Hq + Hkv:])
    err = np.abs(o.float().cpu().numpy() - ref["o"]).max()
    lerr = np.abs(lse.cpu().numpy() - ref["lse"]).max()
    _log(f"[projected step] T={T} max|do|={err:.3e} max|dlse|={lerr:.3e}")
    assert err <= TOL_O["bf16"] and lerr <= 1e-2


def test_serving_loop_matches_oracle(env):
    """ca_sched driving 60 rounds of a serving loop (arrivals, prefix hits, finishing requests
    and preemptions on a 48-page pool) through append + attention: every round's plan equals the
    oracle's loop bit for bit, every row's output is within tolerance, and the cache of every
    scheduled request holds exactly the oracle's tokens (recomputed ones included)."""
    import torch
    import chunked_prefill_paged_ca_amd as ca
    from chunked_prefill_paged_ca_amd.workload import make_serve_scenario
    from tests import harness as H
    ctx, oracle = env
    sc = make_serve_scenario()
    dt = sc.dtype
    sched = ca.Scheduler(sc.token_budget, sc.max_chunk, sc.page_size, sc.num_pool_pages, sc.chunk_align)
    serve = oracle.ServeSession(sc)
    k_cache, v_cache = H.alloc_pool(sc)
    added, preempted, rows = 0, 0, 0
    for rnd in range(sc.rounds):
        while added < sc.n and sc.arrival[added] <= rnd:
            assert sched.free_pages() == serve.free_pages()
            if serve.free_pages() < -(-int(sc.num_cached[added]) // sc.page_size):
                break
            rid = sched.add(int(sc.prompt_len[added]), int(sc.max_new[added]), int(sc.num_cached[added]))
            assert rid == serve.add(added) == added
            hk, hv = sc.history(added)
            H.write_positions(k_cache, v_cache, sched.get(rid)["block_table"], sc.page_size, hk, hv)
            added += 1
        ref_plan = serve.plan()
        plan = sched.step()
        a = plan.arrays()
        for k in ("req_ids", "qo_indptr", "kv_page_indptr", "kv_page_indices", "kv_last_page_len"):
            assert np.array_equal(a[k], ref_plan[k]), (rnd, k)
        if plan.num_tokens == 0:
            serve.step(ref_plan, *sc.take([], [], []))
            sched.commit()
            continue
        q, k, v = sc.take(ref_plan["req_ids"], serve.starts(ref_plan), np.diff(ref_plan["qo_indptr"]))
        q_out, o, lse = H.gpu_step(ctx, sc, plan, q, k, v, k_cache, v_cache)
        torch.cuda.synchronize()
        ref = serve.step(ref_plan, q, k, v)
        sched.commit()
        go = o.float().cpu().numpy().astype(np.float64)
        gl = lse.cpu().numpy().astype(np.float64)
        uq = H.ulp_distance(q_out.float().cpu().numpy().astype(np.float64), ref["q_rot"], dt)
        err = np.abs(go - ref["o"]).max()
        lerr = np.abs(gl - ref["lse"]).max()
        rows += plan.num_tokens
        _log(f"[serving] round {rnd}: T={plan.num_tokens} seqs={plan.num_seqs} decodes={plan.num_decodes} "
             f"free pages={sched.free_pages()} max|do|={err:.3e} max|dlse|={lerr:.3e}")
        assert uq.max() <= 1.0 and err <= TOL_O[dt] and lerr <= TOL_LSE[dt], (rnd, uq.max(), err, lerr)
        for i in ref_plan["req_ids"]:
            g = sched.get(int(i))
            if g["state"] == ca.CA_REQ_FINISHED:
                continue
            gk, gv = H.read_dense(k_cache, v_cache, g["block_table"], sc.page_size, g["num_computed"])
            assert H.ulp_distance(gk, serve.k[int(i)], dt).max() <= 1.0, (rnd, i, "k cache")
            assert np.array_equal(gv, serve.v[int(i)]), (rnd, i, "v cache")
    states = [sched.get(i)["state"] for i in range(added)]
    preempted = sum(sched.get(i)["num_preemptions"] for i in range(added))
    _log(f"[serving] {rows} rows, {states.count(ca.CA_REQ_FINISHED)} of {added} finished, {preempted} preemptions")
    assert added == sc.n and preempted > 0 and states.count(ca.CA_REQ_FINISHED) >= sc.n - 2


@pytest.mark.parametrize("mode", ["split", "few-decode-wgs", "eight-decode-waves", "decode-only"])
def test_attention_launch_layouts(env, mode):
    """The Mistral-7B step through the other layouts of the attention launch: decode and chunk
    rows as two launches (CA_SPLIT_ATTENTION=1), a mixed launch with only 8 decode workgroups (so
    every decode wave runs many items, crossing many (row, kv head) boundaries), 8 decode waves
    per workgroup instead of 4 (CA_DECODE_WAVES=8), and a step with decodes only (no chunk
    workgroups at all)."""
    import os
    import chunked_prefill_paged_ca_amd as ca
    from chunked_prefill_paged_ca_amd.workload import Workload, make_config
    _, oracle = env
    setting = {"split": ("CA_SPLIT_ATTENTION", "1"), "few-decode-wgs": ("CA_DECODE_WGS", "8"),
               "eight-decode-waves": ("CA_DECODE_WAVES", "8"), "decode-only": None}[mode]
    if setting:
        os.environ[setting[0]] = setting[1]
    try:
        ctx = ca.create(0)
    finally:
        if setting:
            del os.environ[setting[0]]
    try:
        wl = make_config(2)
        if mode == "decode-only":
            keep = [r for r in range(wl.n) if wl.is_decode(r)]
            uids = np.arange(wl.n) if wl.uids is None else wl.uids
            wl = Workload(**{**wl.__dict__, "num_computed": wl.num_computed[keep],
                             "num_prompt_left": wl.num_prompt_left[keep],
                             "block_tables": [wl.block_tables[r] for r in keep],
                             "stream_len": wl.stream_len[keep], "uids": uids[keep]})
        res, _, _ = run_and_check(ctx, oracle, wl, label=f"layout-{mode}")
        p = res[0][0]
        assert p["num_decodes"] == 80
        assert (p["num_seqs"] == 80) == (mode == "decode-only")
    finally:
        ctx.close()


@pytest.mark.parametrize("hq,hkv", [(32, 8), (64, 8), (16, 1)])
def test_long_decodes_split_and_merged(env, hq, hkv):
    """Three long decodes (contexts 30000, 20000 and 9000 keys) at d = 128, group sizes 4, 8 and
    16: every (row, kv head) is cut into dozens of pieces, one per decode wave it crosses, and the
    merge combines them.  Three steps on one context, so the work lists and partial slots are
    rebuilt for every step."""
    from chunked_prefill_paged_ca_amd.workload import Workload
    ctx, oracle = env
    steps = 3
    nc = np.array([29999, 19999, 8999], np.int32)
    left = np.zeros(3, np.int32)
    stream = np.full(3, steps, np.int32)
    pool = 4096
    perm = np.random.default_rng(31).permutation(pool).astype(np.int32)
    tabs, it = [], 0
    for r in range(3):
        n = -(-int(nc[r] + stream[r]) // 16)
        tabs.append(perm[it:it + n]); it += n
    wl = Workload(name="long-decodes", config=0, seed=79, num_q_heads=hq, num_kv_heads=hkv,
                  head_dim=128, page_size=16, dtype="bf16", token_budget=64, max_chunk=0,
                  num_pool_pages=pool, num_computed=nc, num_prompt_left=left, block_tables=tabs,
                  stream_len=stream, steps=steps)
    res, _, _ = run_and_check(ctx, oracle, wl, label=f"long-decodes-{hq}/{hkv}")
    assert len(res) == steps and all(r[0]["num_decodes"] == 3 for r in res)


def test_edge_cases(env):
    """kv_len 1 decode, a decode filling its last page exactly, 1-row chunks, a chunk starting
    on a page boundary, GQA group 8 with d = 64, and page-permutation invariance."""
    import torch
    from chunked_prefill_paged_ca_amd.workload import StreamCursor, Workload
    from tests import harness as H
    ctx, oracle = env
    for hq, hkv, d in ((8, 1, 64), (4, 4, 128), (12, 4, 128)):
        nc = np.array([0, 15, 31, 0, 16, 40], np.int32)
        left = np.array([0, 0, 0, 1, 1, 33], np.int32)
        stream = np.array([1, 1, 1, 1, 1, 33], np.int32)
        pool = 64
        perm = np.random.default_rng(9).permutation(pool).astype(np.int32)
        tabs, it = [], 0
        for r in range(6):
            n = -(-int(nc[r] + stream[r]) // 16)
            tabs.append(perm[it:it + n]); it += n
        wl = Workload(name="edge", config=0, seed=77, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                      page_size=16, dtype="bf16", token_budget=64, max_chunk=0,
                      num_pool_pages=pool, num_computed=nc, num_prompt_left=left,
                      block_tables=tabs, stream_len=stream)
        res, _, _ = run_and_check(ctx, oracle, wl, label=f"edge-{hq}/{hkv}/{d}")
        # same data on a different page placement: bit-identical outputs
        perm2 = np.random.default_rng(10).permutation(pool).astype(np.int32)
        tabs2, it = [], 0
        for r in range(6):
            tabs2.append(perm2[it:it + len(tabs[r])]); it += len(tabs[r])
        wl2 = Workload(**{**wl.__dict__, "block_tables": tabs2})
        res2, _, _ = run_and_check(ctx, oracle, wl2, label=f"edge-perm-{hq}/{hkv}/{d}")
        assert np.array_equal(res[0][1], res2[0][1]) and np.array_equal(res[0][2], res2[0][2])


@pytest.mark.parametrize("hq,hkv,d", [(16, 1, 64), (32, 2, 128), (8, 8, 64)])
def test_chunk_kernel_shapes(env, hq, hkv, d):
    """Chunk rows through many 128-key LDS stages for the group sizes and head dims the MFMA path
    takes -- G = 16 (its limit) at d = 64 and 128, G = 1 at d = 64 -- beside a decode in the same
    launch: a 100-row chunk on 700 cached keys (25 key blocks: six full stages and a partial
    one; at G = 16 its last column block holds 64 columns, so six of its eight waves only copy),
    a 37-row chunk from position 0, and a 1501-key decode."""
    from chunked_prefill_paged_ca_amd.workload import Workload
    ctx, oracle = env
    nc = np.array([1500, 0, 700], np.int32)
    left = np.array([0, 37, 100], np.int32)
    stream = np.array([1, 37, 100], np.int32)
    pool = 256
    perm = np.random.default_rng(21).permutation(pool).astype(np.int32)
    tabs, it = [], 0
    for r in range(3):
        n = -(-int(nc[r] + stream[r]) // 16)
        tabs.append(perm[it:it + n]); it += n
    wl = Workload(name="chunk-shapes", config=0, seed=78, num_q_heads=hq, num_kv_heads=hkv,
                  head_dim=d, page_size=16, dtype="bf16", token_budget=256, max_chunk=0,
                  num_pool_pages=pool, num_computed=nc, num_prompt_left=left, block_tables=tabs,
                  stream_len=stream)
    res, _, _ = run_and_check(ctx, oracle, wl, rows_per_seq=24, label=f"chunk-shapes-{hq}/{hkv}/{d}")
    assert res[0][0]["num_decodes"] == 1 and res[0][0]["num_tokens"] == 138


@pytest.mark.parametrize("split", [False, True])
def test_chunk_queue_mode(env, split):
    """Chunk items taken from the work queues (more items than free workgroup slots): a 300-row
    chunk on 2000 cached keys cut into 64-key splits (CA_CHUNK_SPLIT=64: ~1400 items, most of
    them claimed through the queue counters) beside three decodes, in one launch and (split)
    as a chunk-only launch.  Checked against the oracle, then the same attention launched four
    more times, the third and fifth through the allocation-free entry point: each launch must
    leave zeroed the counter set the next one claims from (the two sets alternate; with split,
    a decode-only launch sits between the queue-mode ones), and which worker ran which item
    must not change a bit
    (every item has its own partial slot, merged in a fixed order), so the ordinary launches
    agree bit for bit, and so do the two allocation-free ones (which lengthen the splits to fit
    their scratch, so they are held to the oracle's bar instead of to the others)."""
    import os
    import torch
    import chunked_prefill_paged_ca_amd as ca
    from chunked_prefill_paged_ca_amd import make_desc
    from chunked_prefill_paged_ca_amd.workload import StreamCursor, Workload
    from tests import harness as H
    _, oracle = env
    nc = np.array([1800, 2000, 2400, 1100], np.int32)
    left = np.array([0, 300, 0, 0], np.int32)
    stream = np.array([1, 300, 1, 1], np.int32)
    pool = 640
    perm = np.random.default_rng(31).permutation(pool).astype(np.int32)
    tabs, it = [], 0
    for r in range(4):
        n = -(-int(nc[r] + stream[r]) // 16)
        tabs.append(perm[it:it + n]); it += n
    wl = Workload(name="queue-mode", config=0, seed=91, num_q_heads=32, num_kv_heads=8,
                  head_dim=128, page_size=16, dtype="bf16", token_budget=512, max_chunk=0,
                  num_pool_pages=pool, num_computed=nc, num_prompt_left=left, block_tables=tabs,
                  stream_len=stream)
    env_set = {"CA_CHUNK_SPLIT": "64"}
    if split:
        env_set["CA_SPLIT_ATTENTION"] = "1"
    os.environ.update(env_set)
    try:
        qctx = ca.create(0)
    finally:
        for k in env_set:
            del os.environ[k]
    try:
        res, (k_cache, v_cache), _ = run_and_check(qctx, oracle, wl, rows_per_seq=40,
                                                   label=f"queue-mode-split{int(split)}")
        assert res[0][0]["num_decodes"] == 3
        # the step again on the appended caches: attention only, five launches
        sess = oracle.Session(wl)
        ref_plan = sess.plan()
        plan = H.lib_plan(wl, sess.num_computed, sess.num_prompt_left)
        q, _, _ = StreamCursor(wl).take(ref_plan["req_ids"], np.diff(ref_plan["qo_indptr"]))
        desc = make_desc(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.page_size, wl.dtype)
        q_in = H.to_device(q, wl.dtype)
        q_rot = torch.empty_like(q_in)
        # rotate q only: append_kv_rope into a scratch pool so the cache above stays as it is
        k0, v0 = H.alloc_pool(wl, fill=0.0)
        kn = torch.zeros((plan.num_tokens, wl.num_kv_heads, wl.head_dim), dtype=q_in.dtype, device="cuda")
        qctx.append_kv_rope(desc, plan, q_in, q_rot, kn, kn, k0, v0, wl.num_pool_pages)
        outs = []
        for i in range(5):
            o = torch.empty_like(q_rot)
            lse = torch.empty((plan.num_tokens, wl.num_q_heads), dtype=torch.float32, device="cuda")
            qctx.mixed_attention(desc, plan, q_rot, k_cache, v_cache, wl.num_pool_pages, o, lse,
                                 no_alloc=i in (2, 4))
            torch.cuda.synchronize()
            outs.append((o.cpu(), lse.cpu()))
        mask = ~np.isnan(res[0][3]["o"][:, 0, 0])
        for i in range(5):
            go = outs[i][0].float().numpy().astype(np.float64)
            assert np.abs(go[mask] - res[0][3]["o"][mask]).max() <= TOL_O["bf16"], ("launch", i)
        for i, j in ((1, 0), (3, 0), (4, 2)):
            assert torch.equal(outs[i][0], outs[j][0]), ("launch", i, "o differs from", j)
            assert torch.equal(outs[i][1], outs[j][1]), ("launch", i, "lse differs from", j)
        _log(f"[queue-mode-split{int(split)}] five launches within the bar; repeats bit-identical")
    finally:
        qctx.close()


@pytest.mark.parametrize("hq,hkv,d", [(64, 2, 128), (32, 1, 64)])
def test_wide_group_bf16(env, hq, hkv, d):
    """bf16 with 32 q heads per kv head (wider than one MFMA tile of 16 columns): these shapes
    run on the plain kernel with its split merge -- decodes of 1, 517 and 2100 keys, a 77-row
    chunk on 300 cached keys and a 40-row chunk from position 0 -- every row against the
    oracle."""
    from chunked_prefill_paged_ca_amd.workload import Workload
    ctx, oracle = env
    nc = np.array([0, 516, 2099, 300, 0], np.int32)
    left = np.array([0, 0, 0, 77, 40], np.int32)
    stream = np.array([1, 1, 1, 77, 40], np.int32)
    pool = 512
    perm = np.random.default_rng(41).permutation(pool).astype(np.int32)
    tabs, it = [], 0
    for r in range(5):
        n = -(-int(nc[r] + stream[r]) // 16)
        tabs.append(perm[it:it + n]); it += n
    wl = Workload(name="wide-group", config=0, seed=81, num_q_heads=hq, num_kv_heads=hkv,
                  head_dim=d, page_size=16, dtype="bf16", token_budget=256, max_chunk=0,
                  num_pool_pages=pool, num_computed=nc, num_prompt_left=left, block_tables=tabs,
                  stream_len=stream)
    res, _, _ = run_and_check(ctx, oracle, wl, label=f"wide-group-{hq}/{hkv}/{d}")
    assert res[0][0]["num_decodes"] == 3 and res[0][0]["num_tokens"] == 120


def test_debug_validate_refuses_colliding_writes(env):
    """With CA_DEBUG_VALIDATE=1 the append refuses a plan whose block tables make two sequences
    append to the same page slot, before anything is launched; a context without it runs the
    range checks only.  A plan first seen with a large pool is refused on a later call with a
    pool that no longer holds its pages (the cached device copy is not trusted blindly)."""
    import os
    import torch
    import chunked_prefill_paged_ca_amd as ca
    ctx, _ = env
    desc = ca.make_desc(2, 2, 64, 16, "bf16")
    plan = ca.plan_batch([0, 0], [20, 10], [np.array([3, 5]), np.array([5])], 64, 0, 16, 8)
    kc = torch.zeros((8, 2, 8, 16, 8), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros((8, 2, 4, 4, 16, 4), dtype=torch.bfloat16, device="cuda")
    x = torch.zeros((30, 2, 64), dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    os.environ["CA_DEBUG_VALIDATE"] = "1"
    try:
        dctx = ca.create(0)
    finally:
        del os.environ["CA_DEBUG_VALIDATE"]
    try:
        with pytest.raises(ca.CaError, match="both append to page 5 slot 0"):
            dctx.append_kv_rope(desc, plan, x, y, x, x, kc, vc, 8)
    finally:
        dctx.close()
    ok = ca.plan_batch([0, 0], [20, 10], [np.array([3, 5]), np.array([6])], 64, 0, 16, 8)
    ctx.append_kv_rope(desc, ok, x, y, x, x, kc, vc, 8)
    ctx.mixed_attention(desc, ok, y, kc, vc, 8, x)
    with pytest.raises(ca.CaError, match="outside the pool"):
        ctx.mixed_attention(desc, ok, y, kc[:6], vc[:6], 6, x)
    torch.cuda.synchronize()


def test_empty_step_is_noop(env):
    import torch
    import chunked_prefill_paged_ca_amd as ca
    ctx, _ = env
    plan = ca.plan_batch([], [], [], 16, 0, 16, 8)
    assert plan.num_tokens == 0
    desc = ca.make_desc(2, 2, 64, 16, "bf16")
    kc = torch.zeros((8, 2, 16, 64), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros((8, 2, 64, 16), dtype=torch.bfloat16, device="cuda")
    x = torch.zeros((1, 2, 64), dtype=torch.bfloat16, device="cuda")
    ctx.append_kv_rope(desc, plan, x, x, x[:, :2], x[:, :2], kc, vc, 8)
    ctx.mixed_attention(desc, plan, x, kc, vc, 8, x)
    torch.cuda.synchronize()


def test_profile_records_every_kernel(env):
    """The timing layer records one event pair per library launch, with positive durations."""
    import torch
    from chunked_prefill_paged_ca_amd.workload import StreamCursor, make_config
    from tests import harness as H
    ctx, _ = env
    wl = make_config(2)
    kc, vc = H.alloc_pool(wl, fill=0.0)
    plan = H.lib_plan(wl, wl.num_computed, wl.num_prompt_left)
    q, k, v = StreamCursor(wl).take(plan.arrays()["req_ids"], np.diff(plan.arrays()["qo_indptr"]))
    ctx.profile_read()
    ctx.profile_enable(True)
    H.gpu_step(ctx, wl, plan, q, k, v, kc, vc)
    torch.cuda.synchronize()
    ctx.profile_enable(False)
    recs = ctx.profile_read()
    names = [n for n, _ in recs]
    _log(f"[profile] {recs}")
    # the append launch copies the step's metadata itself; the attention call reuses it
    assert names == ["append_rope", "attention", "merge"], names
    assert "upload" not in names
    assert all(ms > 0 for _, ms in recs)
    assert ctx.profile_read() == []
    # an attention call that is the first to see a plan uploads it with its own launch
    plan2 = H.lib_plan(wl, wl.num_computed, wl.num_prompt_left)
    qd = torch.zeros((plan2.num_tokens, wl.num_q_heads, wl.head_dim), dtype=torch.bfloat16, device="cuda")
    od = torch.empty_like(qd)
    ctx.profile_enable(True)
    from chunked_prefill_paged_ca_amd import make_desc
    desc = make_desc(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.page_size, wl.dtype)
    ctx.mixed_attention(desc, plan2, qd, kc, vc, wl.num_pool_pages, od, None)
    torch.cuda.synchronize()
    ctx.profile_enable(False)
    names2 = [n for n, _ in ctx.profile_read()]
    assert names2[0] == "upload" and "attention" in names2, names2


def test_staging_ring_call_patterns(env):
    """The step metadata travels through a ring of pinned staging slots; a slot is refilled only
    once the launch that read it is known to have finished (reported by the next attention launch
    on the same stream, else by waiting for the device).  Thirty rounds of call patterns -- append
    then attention on one stream, the attention on a second stream ordered by an event, two appends
    before one attention, attention alone (its own upload), the attention repeated -- wrap the
    eight-slot ring several times; every round's outputs must equal a clean context's bit for
    bit."""
    import torch
    import chunked_prefill_paged_ca_amd as ca
    from chunked_prefill_paged_ca_amd.workload import StreamCursor, make_config
    from tests import harness as H
    ctx, _ = env
    wl = make_config(2)
    kc, vc = H.random_pool(wl, seed=5)
    desc = ca.make_desc(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.page_size, wl.dtype)
    batch = ca.RequestBatch(wl.num_computed, wl.num_prompt_left, wl.block_tables, wl.token_budget,
                            wl.max_chunk, wl.page_size, wl.num_pool_pages)
    plan0 = batch.plan()
    a = plan0.arrays()
    q_raw, k_raw, v_raw = StreamCursor(wl).take(a["req_ids"], np.diff(a["qo_indptr"]))
    q_in, k_in, v_in = (H.to_device(x, wl.dtype) for x in (q_raw, k_raw, v_raw))
    # reference: a fresh context, one append + attention (appending the same rows again
    # rewrites the same cache slots with the same values)
    ref_ctx = ca.create(0)
    q_ref = torch.empty_like(q_in)
    o_ref = torch.empty_like(q_in)
    ref_ctx.append_kv_rope(desc, plan0, q_in, q_ref, k_in, v_in, kc, vc, wl.num_pool_pages)
    ref_ctx.mixed_attention(desc, plan0, q_ref, kc, vc, wl.num_pool_pages, o_ref)
    torch.cuda.synchronize()
    ref_ctx.close()
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    for r in range(30):
        pattern = r % 5
        q_rot = torch.full_like(q_in, float("nan"))
        o = torch.full_like(q_in, float("nan"))
        if pattern == 0:
            ctx.append_kv_rope(desc, batch.plan(), q_in, q_rot, k_in, v_in, kc, vc, wl.num_pool_pages)
            # the same plan object again: its metadata is already on the device
            plan = batch.plan()
            ctx.append_kv_rope(desc, plan, q_in, q_rot, k_in, v_in, kc, vc, wl.num_pool_pages)
            ctx.mixed_attention(desc, plan, q_rot, kc, vc, wl.num_pool_pages, o)
        elif pattern == 1:
            plan = batch.plan()
            ctx.append_kv_rope(desc, plan, q_in, q_rot, k_in, v_in, kc, vc, wl.num_pool_pages)
            ev = torch.cuda.Event()
            ev.record(main)
            side.wait_event(ev)
            with torch.cuda.stream(side):
                ctx.mixed_attention(desc, plan, q_rot, kc, vc, wl.num_pool_pages, o, stream=side)
            ev2 = torch.cuda.Event()
            ev2.record(side)
            main.wait_event(ev2)
        elif pattern == 2:
            plan = batch.plan()
            ctx.append_kv_rope(desc, plan, q_in, q_rot, k_in, v_in, kc, vc, wl.num_pool_pages)
            ctx.mixed_attention(desc, plan, q_rot, kc, vc, wl.num_pool_pages, o)
        elif pattern == 3:
            q_rot.copy_(q_ref)
            ctx.mixed_attention(desc, batch.plan(), q_rot, kc, vc, wl.num_pool_pages, o)
        else:
            plan = batch.plan()
            ctx.append_kv_rope(desc, plan, q_in, q_rot, k_in, v_in, kc, vc, wl.num_pool_pages)
            ctx.mixed_attention(desc, plan, q_rot, kc, vc, wl.num_pool_pages, o)
            ctx.mixed_attention(desc, plan, q_rot, kc, vc, wl.num_pool_pages, o)
        torch.cuda.synchronize()
        assert torch.equal(q_rot, q_ref), ("staging", r, pattern, "q_rot")
        assert torch.equal(o, o_ref), ("staging", r, pattern, "o")
    _log("[staging] 30 rounds of 5 call patterns: outputs bit-identical to a clean context")


def test_misaligned_buffer_is_rejected(env):
    """Device buffers must be 16-byte aligned; a view shifted by one element is refused before
    anything is launched."""
    import torch
    import chunked_prefill_paged_ca_amd as ca
    ctx, _ = env
    plan = ca.plan_batch([0], [4], [np.arange(2, dtype=np.int32)], 16, 0, 16, 8)
    desc = ca.make_desc(2, 2, 64, 16, "bf16")
    kc = torch.zeros((8, 2, 16, 64), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros((8, 2, 64, 16), dtype=torch.bfloat16, device="cuda")
    base = torch.zeros(4 * 2 * 64 + 1, dtype=torch.bfloat16, device="cuda")
    shifted = base[1:].view(4, 2, 64)
    good = torch.zeros((4, 2, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ca.CaError, match="aligned"):
        ctx.append_kv_rope(desc, plan, shifted, good, good, good, kc, vc, 8)
    with pytest.raises(ca.CaError, match="aligned"):
        ctx.mixed_attention(desc, plan, good, kc, vc, 8, shifted)
    torch.cuda.synchronize()
