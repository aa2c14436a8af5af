"""Benchmark: one mixed chunked-prefill + decode step per iteration on one MI355X.

A step is the whole hot path over one batch: ca_plan_batch (host), ca_append_kv_rope and
ca_mixed_attention, on the Mistral-7B-shaped single-layer batch of the 512-token budget example
(32 q heads, 8 kv heads, d 128, bf16, page 16): 80 decodes with contexts uniform in [512, 4096],
prefill P getting 300 tokens on 1200 cached and prefill Q getting 132 on 2048, pages permuted
over a 64K-page pool.  Inputs are resident in HBM before the timed region starts.

Prints ONE JSON line.  `value` is tokens per second of whole steps over the timed region.
`roofline` places the dominant kernel -- the attention launch, which runs the decode rows and
the prefill-chunk rows side by side -- against the peak of the resource its algorithmic work
needs longest: reading the K/V pages at 8 TB/s HBM (the default workload and every
decode-heavy one), or the chunk rows' flops at 2.5 PFLOP/s bf16 MFMA (long prefill chunks),
using the launch's own duration (HIP events attached to that launch on the bench's stream, on
every tenth step of the timed region by default: each timed launch adds ~2 us to its step).
`traffic` is the HBM bytes the counters measured for that launch (profiles/), used only for the
workload they were taken on and while the kernel sources are unchanged.
`parts` times the decode and chunk work as two separate launches in a second, untimed pass, for
their own HBM and bf16 MFMA fractions.  `measured_peaks` re-measures, after the timed region,
what this device sustains (a 4 GiB read stream, a 1 GiB copy, an 8192^3 bf16 GEMM on random data) and
places the roofline launch against the matching one.  `cpu_baseline` times the CPU oracle on the same step.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_attention_mistral7b_mixed_step.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def stored_traffic(workload):
    """HBM bytes per attention launch from the committed counter summary, or None: the reading
    counts only for the workload it was taken on and while the kernel sources are unchanged."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    from chunked_prefill_paged_ca_amd.profiling import kernel_sources_sha256
    if t.get("workload") != workload or t.get("sources_sha256") != kernel_sources_sha256():
        return None
    return int(t["hbm_bytes_per_launch"])


def cpu_baseline(wl, min_seconds=10.0):
    """The oracle as it stands on the whole step (every row), repeated for at least min_seconds."""
    import oracle
    from chunked_prefill_paged_ca_amd.workload import StreamCursor
    sess = oracle.Session(wl)
    p = sess.plan()
    q, k, v = StreamCursor(wl).take(p["req_ids"], np.diff(p["qo_indptr"]))
    nd = p["num_decodes"]
    T = p["num_tokens"]
    threads = oracle.default_threads()
    times = []
    while sum(times) < min_seconds:
        fresh = sess.fork()
        t0 = time.perf_counter()
        fresh.step(p, q, k, v, nthreads=threads)
        times.append(time.perf_counter() - t0)
    dt = float(np.mean(times))
    return {"value": round(T / dt, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"the whole step: all {T} rows ({nd} decode rows + 2 prefill chunks), "
                      f"fp64 C oracle on {threads} threads, mean of {len(times)} runs "
                      f"({sum(times):.1f} s of work, {dt:.2f} s per step)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parts", action="store_true")
    ap.add_argument("--time-every", type=int, default=10,
                    help="attach the timing events to the attention launch of every N-th step of "
                         "the timed region (1: every step; each timed launch adds ~2 us to its "
                         "step, so the default times one step in ten)")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip re-measuring the HBM and bf16 GEMM rates this device sustains")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after the timed region, copy this many MiB device to device once (a "
                         "known-size reference for the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path has no cross-GPU exchange; see the sharding notes in the design doc)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from __graft_entry__ import ensure_built
    ensure_built()
    import chunked_prefill_paged_ca_amd as ca
    from chunked_prefill_paged_ca_amd import accounting as acc
    from chunked_prefill_paged_ca_amd.workload import StreamCursor, make_config
    from tests import harness as H

    torch.cuda.set_device(0)
    wl = make_config(args.config)
    log(f"workload: {wl.name}")
    kc, vc = H.random_pool(wl, seed=wl.seed)
    desc = ca.make_desc(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.page_size, wl.dtype)
    batch = ca.RequestBatch(wl.num_computed, wl.num_prompt_left, wl.block_tables, wl.token_budget,
                            wl.max_chunk, wl.page_size, wl.num_pool_pages)
    plan0 = batch.plan()
    a = plan0.arrays()
    q_lens = np.diff(a["qo_indptr"])
    q_raw, k_raw, v_raw = StreamCursor(wl).take(a["req_ids"], q_lens)
    q_in, k_in, v_in = (H.to_device(x, wl.dtype) for x in (q_raw, k_raw, v_raw))
    q_rot = torch.empty_like(q_in)
    o = torch.empty_like(q_in)
    lse = torch.empty((plan0.num_tokens, wl.num_q_heads), dtype=torch.float32, device="cuda")
    T = plan0.num_tokens
    nd = plan0.num_decodes
    kv_lens = np.array([int(wl.num_computed[r]) + int(q) for r, q in zip(a["req_ids"], q_lens)])
    dec_w, chk_w = acc.plan_work(q_lens, kv_lens, nd, wl.num_q_heads, wl.num_kv_heads,
                                 wl.head_dim, wl.page_size)
    stream = torch.cuda.current_stream()

    def run_steps(ctx, n, time_every=0):
        for i in range(n):
            plan = batch.plan()
            ctx.append_kv_rope(desc, plan, q_in, q_rot, k_in, v_in, kc, vc, wl.num_pool_pages, stream=stream)
            if time_every:
                ctx.profile_enable(ca.PROFILE_ATTENTION if i % time_every == 0 else False)
            ctx.mixed_attention(desc, plan, q_rot, kc, vc, wl.num_pool_pages, o, lse, stream=stream)

    def kernel_means(recs):
        per = {}
        for name, ms in recs:
            per.setdefault(name, []).append(ms)
        return {k: float(np.mean(v)) for k, v in per.items()}

    # ---- timed region: whole steps; the attention launch carries timing events ----
    ctx = ca.create(0)
    run_steps(ctx, args.warmup)
    torch.cuda.synchronize()
    ctx.profile_read()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_steps(ctx, args.steps, time_every=max(1, args.time_every))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ctx.profile_enable(False)
    recs0 = ctx.profile_read()
    km0 = kernel_means(recs0)
    attn_name = "attention" if "attention" in km0 else "generic"  # fp32 storage: plain kernel
    attn_ms = km0[attn_name]
    attn_all = np.array([ms for n, ms in recs0 if n == attn_name])
    ctx.close()
    ms_per_step = elapsed * 1e3 / args.steps
    value = T * args.steps / elapsed

    # The launch's bound is the resource its algorithmic work needs longest: K/V bytes at the HBM
    # peak, or the chunk rows' flops at the bf16 MFMA peak (long prefill chunks).
    attn_bytes = dec_w.bytes + chk_w.bytes
    t_hbm = attn_bytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = chk_w.flops / (BF16_PEAK_TFLOPS * 1e12)
    if t_mfma > t_hbm:
        achieved, peak, unit, bound = chk_w.flops / (attn_ms * 1e-3) / 1e12, BF16_PEAK_TFLOPS, "TFLOP/s", "mfma"
    else:
        achieved, peak, unit, bound = attn_bytes / (attn_ms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s", "hbm"
    traffic = stored_traffic(wl.name)
    out = {
        "metric": "mixed chunked-prefill+decode attn tokens/s; % HBM peak and % MFMA peak",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "tokens_per_step": T, "decodes": nd,
                   "token_budget": wl.token_budget, "page_size": wl.page_size,
                   "pool_pages": wl.num_pool_pages, "step": "plan + append_kv_rope + mixed_attention"},
        "roofline": {"bound": bound, "kernel": "attention (decode + chunk rows, one launch)",
                     "achieved": round(achieved, 1), "peak": peak, "unit": unit,
                     "frac": round(achieved / peak, 4), "traffic": traffic,
                     "alg_bytes_per_launch": int(attn_bytes),
                     "alg_flops_per_launch": int(chk_w.flops),
                     "launch_ms": round(attn_ms, 5),
                     "launch_ms_p10_p50_p90": [round(float(np.percentile(attn_all, x)), 5) for x in (10, 50, 90)],
                     "launches_timed": int(attn_all.size)},
    }

    # ---- second pass (not timed for `value`): decode and chunk as separate launches ----
    if not args.no_parts:
        os.environ["CA_SPLIT_ATTENTION"] = "1"
        ctx2 = ca.create(0)
        del os.environ["CA_SPLIT_ATTENTION"]
        run_steps(ctx2, args.warmup)
        torch.cuda.synchronize()
        ctx2.profile_read()
        ctx2.profile_enable(True)
        run_steps(ctx2, args.steps)
        torch.cuda.synchronize()
        ctx2.profile_enable(False)
        km = kernel_means(ctx2.profile_read())
        ctx2.close()
        parts = {"kernel_ms": {k: round(v, 5) for k, v in km.items()}}
        if "decode" in km:
            bw = dec_w.bytes / (km["decode"] * 1e-3) / 1e9
            parts["decode"] = {"bound": "hbm", "achieved": round(bw, 1), "peak": HBM_PEAK_GBS,
                               "unit": "GB/s", "frac": round(bw / HBM_PEAK_GBS, 4),
                               "alg_bytes_per_launch": int(dec_w.bytes)}
        if "chunk" in km:
            tf = chk_w.flops / (km["chunk"] * 1e-3) / 1e12
            parts["chunk"] = {"bound": "mfma", "achieved": round(tf, 2), "peak": BF16_PEAK_TFLOPS,
                              "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                              "alg_flops_per_launch": int(chk_w.flops)}
        out["parts"] = parts

    # ---- what this device sustains (after the timed region): the roofline above uses the
    # datasheet peaks; these put the same launch against measured ones ----
    if not args.no_peaks:
        from chunked_prefill_paged_ca_amd import peaks
        rd, cp, gm = peaks.hbm_read_gbs(), peaks.hbm_copy_gbs(), peaks.gemm_tflops("randn")
        r = out["roofline"]
        meas = rd if r["bound"] == "hbm" else gm
        out["measured_peaks"] = {"hbm_read_GBs": round(rd, 1), "hbm_copy_GBs": round(cp, 1),
                                 "bf16_gemm_8192_TFs": round(gm, 1),
                                 "roofline_frac_of_measured": round(r["achieved"] / meas, 4)}

    if args.copy_mib > 0:
        n = args.copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"reference copy: {args.copy_mib} MiB read + {args.copy_mib} MiB written")
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on the same step ...")
        out["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
