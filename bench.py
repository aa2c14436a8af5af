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
decode-heavy one), or the chunk rows' flops at 2.5 PFLOP/s bf16 MFMA (long prefill chunks).
Its duration comes from HIP events attached to that launch itself on the bench's stream: every
attention launch of the timed region carries them, and when the timed region has fewer than 50
steps the same stream of steps continues, still timed, until 50 launches have been timed
(mean and p10/p50/p90 over all of them).  `scrubbed` repeats 50 steps with a 512 MiB read
before each (outside the events), so L2 and the MALL hold none of the step's data: cold-HBM
launch times.
`traffic` is the HBM bytes the counters measured for that launch (profiles/), used only for the
workload they were taken on and while the sources that shape the launch are unchanged.
`parts` times the decode and chunk work as two separate launches in a second, untimed pass, for
their own HBM and bf16 MFMA fractions.  `per_config` runs the other workloads the same way
(Yi-34B and LLaMA2-70B one-GPU shares: whole steps; the Llama-13B 8192-token prompt: summed
kernel time over all of its chunks at each chunk size, against the one-shot prompt).
`measured_peaks` re-measures, after the timed region, what this device sustains (a 4 GiB read
stream, a 1 GiB copy, an 8192^3 bf16 GEMM on random data) and places the roofline launch against
the matching one.  `cpu_baseline` times the CPU oracle on the same step (all host threads, and
one thread).
"""
import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_attention_mistral7b_mixed_step.json")
MIN_TIMED_LAUNCHES = 50
SCRUB_MIB = 512


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def stored_traffic(workload):
    """HBM bytes per attention launch from the committed counter summary, or None: the reading
    counts only for the workload it was taken on and while the sources are unchanged."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    from chunked_prefill_paged_ca_amd.profiling import kernel_sources_sha256
    if t.get("workload") != workload or t.get("sources_sha256") != kernel_sources_sha256():
        return None
    return int(t["hbm_bytes_per_launch"])


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(wl, min_seconds=10.0):
    """The oracle as it stands on the whole step (every row): on every host thread, repeated for
    at least min_seconds, and once on one thread."""
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
    fresh = sess.fork()
    t0 = time.perf_counter()
    fresh.step(p, q, k, v, nthreads=1)
    dt1 = time.perf_counter() - t0
    return {"value": round(T / dt, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "one_thread": {"value": round(T / dt1, 2), "unit": "tokens/s", "seconds_per_step": round(dt1, 3)},
            "sample": f"the whole step: all {T} rows ({nd} decode rows + 2 prefill chunks), "
                      f"fp64 C oracle on {threads} threads, mean of {len(times)} runs "
                      f"({sum(times):.1f} s of work, {dt:.2f} s per step); one_thread: one run"}


def pct(a, ps=(10, 50, 90)):
    return [round(float(np.percentile(a, x)), 5) for x in ps]


def roofline_of(dec_w, chk_w, attn_ms):
    """The launch's bound is the resource its algorithmic work needs longest: K/V bytes at the
    HBM peak, or the chunk rows' flops at the bf16 MFMA peak (long prefill chunks)."""
    attn_bytes = dec_w.bytes + chk_w.bytes
    t_hbm = attn_bytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = chk_w.flops / (BF16_PEAK_TFLOPS * 1e12)
    if t_mfma > t_hbm:
        achieved, peak, unit, bound = chk_w.flops / (attn_ms * 1e-3) / 1e12, BF16_PEAK_TFLOPS, "TFLOP/s", "mfma"
    else:
        achieved, peak, unit, bound = attn_bytes / (attn_ms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s", "hbm"
    return {"bound": bound, "achieved": round(achieved, 1), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "alg_bytes_per_launch": int(attn_bytes),
            "alg_flops_per_launch": int(chk_w.flops)}


class Step:
    """One workload laid out on the device: pool, inputs, outputs and the request batch."""

    def __init__(self, wl, pool_fill="random"):
        import torch
        import chunked_prefill_paged_ca_amd as ca
        from chunked_prefill_paged_ca_amd import accounting as acc
        from chunked_prefill_paged_ca_amd.workload import StreamCursor
        from tests import harness as H
        self.ca, self.torch, self.wl = ca, torch, wl
        if pool_fill == "random":
            self.kc, self.vc = H.random_pool(wl, seed=wl.seed)
        else:
            self.kc, self.vc = H.alloc_pool(wl, fill=0.0)
        self.desc = ca.make_desc(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.page_size, wl.dtype)
        self.batch = ca.RequestBatch(wl.num_computed, wl.num_prompt_left, wl.block_tables,
                                     wl.token_budget, wl.max_chunk, wl.page_size, wl.num_pool_pages)
        plan0 = self.batch.plan()
        a = plan0.arrays()
        q_lens = np.diff(a["qo_indptr"])
        q_raw, k_raw, v_raw = StreamCursor(wl).take(a["req_ids"], q_lens)
        self.q_in, self.k_in, self.v_in = (H.to_device(x, wl.dtype) for x in (q_raw, k_raw, v_raw))
        self.q_rot = torch.empty_like(self.q_in)
        self.o = torch.empty_like(self.q_in)
        self.lse = torch.empty((plan0.num_tokens, wl.num_q_heads), dtype=torch.float32, device="cuda")
        self.T = plan0.num_tokens
        self.nd = plan0.num_decodes
        kv_lens = np.array([int(wl.num_computed[r]) + int(q) for r, q in zip(a["req_ids"], q_lens)])
        self.dec_w, self.chk_w = acc.plan_work(q_lens, kv_lens, self.nd, wl.num_q_heads,
                                               wl.num_kv_heads, wl.head_dim, wl.page_size)
        self.stream = torch.cuda.current_stream()
        self.scrub_buf = None

    def run(self, ctx, n, time_attention=False, scrub=False, every=1):
        """n whole steps (plan, append, attention); with time_attention every `every`-th attention
        launch carries timing events; with scrub a 512 MiB read precedes every step."""
        wl = self.wl
        if scrub and self.scrub_buf is None:
            self.scrub_buf = self.torch.ones(SCRUB_MIB << 18, dtype=self.torch.float32, device="cuda")
        for i in range(n):
            if scrub:
                # a read of 512 MiB evicts the step's data from L2 and the MALL and leaves
                # clean lines (a write would leave dirty ones for the next launch to write back)
                self.scrub_sum = self.scrub_buf.sum()
            plan = self.batch.plan()
            ctx.append_kv_rope(self.desc, plan, self.q_in, self.q_rot, self.k_in, self.v_in, self.kc,
                               self.vc, wl.num_pool_pages, stream=self.stream)
            # the last launch of every group of `every` carries the events: a timed launch costs
            # ~20 us of host time, which on the first step of a run would idle the device
            timed = time_attention and every > 0 and i % every == every - 1
            if timed:
                ctx.profile_enable(self.ca.PROFILE_ATTENTION)
            ctx.mixed_attention(self.desc, plan, self.q_rot, self.kc, self.vc, wl.num_pool_pages,
                                self.o, self.lse, stream=self.stream)
            if timed:
                ctx.profile_enable(False)

    def parts(self, warmup, steps):
        """Decode and chunk rows as two launches over the whole device, each timed."""
        ca, torch = self.ca, self.torch
        os.environ["CA_SPLIT_ATTENTION"] = "1"
        try:
            ctx2 = ca.create(0)
        finally:
            del os.environ["CA_SPLIT_ATTENTION"]
        self.run(ctx2, warmup)
        torch.cuda.synchronize()
        ctx2.profile_read()
        ctx2.profile_enable(True)
        self.run(ctx2, steps)
        torch.cuda.synchronize()
        ctx2.profile_enable(False)
        km = kernel_means(ctx2.profile_read())
        ctx2.close()
        parts = {"kernel_ms": {k: round(v, 5) for k, v in km.items()}}
        if "decode" in km:
            bw = self.dec_w.bytes / (km["decode"] * 1e-3) / 1e9
            parts["decode"] = {"bound": "hbm", "achieved": round(bw, 1), "peak": HBM_PEAK_GBS,
                               "unit": "GB/s", "frac": round(bw / HBM_PEAK_GBS, 4),
                               "alg_bytes_per_launch": int(self.dec_w.bytes)}
        if "chunk" in km:
            tf = self.chk_w.flops / (km["chunk"] * 1e-3) / 1e12
            parts["chunk"] = {"bound": "mfma", "achieved": round(tf, 2), "peak": BF16_PEAK_TFLOPS,
                              "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                              "alg_flops_per_launch": int(self.chk_w.flops)}
        return parts

    def release(self):
        for name in ("kc", "vc", "q_in", "k_in", "v_in", "q_rot", "o", "lse", "scrub_buf"):
            setattr(self, name, None)
        self.torch.cuda.empty_cache()


def kernel_means(recs):
    per = {}
    for name, ms in recs:
        per.setdefault(name, []).append(ms)
    return {k: float(np.mean(v)) for k, v in per.items()}


def attention_times(recs):
    names = {n for n, _ in recs}
    name = "attention" if "attention" in names else "generic"  # fp32 storage: plain kernel
    return name, np.array([ms for n, ms in recs if n == name])


def timed_steps(st, ctx, steps, warmup, every=1):
    """Warm-up, then `steps` timed whole steps with every `every`-th attention launch timed (0:
    none), continued outside the wall-clock region (every launch timed) until MIN_TIMED_LAUNCHES
    launches are timed."""
    torch = st.torch
    # the warm-up steps run exactly like the timed ones (events on every attention launch), so
    # the timing events are created and the first timed step pays nothing extra
    st.run(ctx, warmup, time_attention=True)
    torch.cuda.synchronize()
    ctx.profile_read()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    st.run(ctx, steps, time_attention=True, every=every)
    submitted = time.perf_counter() - t0  # host time to enqueue the steps
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    in_region = ctx.profile_read()
    n_region = sum(1 for n, _ in in_region if n in ("attention", "generic"))
    extra = []
    if n_region < MIN_TIMED_LAUNCHES:
        st.run(ctx, MIN_TIMED_LAUNCHES - n_region, time_attention=True)
        torch.cuda.synchronize()
        extra = ctx.profile_read()
    name, region_ms = attention_times(in_region) if in_region else ("attention", np.zeros(0))
    if extra:
        name, extra_ms = attention_times(extra)
    else:
        extra_ms = np.zeros(0)
    all_ms = np.concatenate([region_ms, extra_ms])
    return elapsed, submitted, name, region_ms, all_ms


def per_config_leg(n, steps=50, warmup=5):
    """A one-GPU share workload (Yi-34B: n = 4, LLaMA2-70B: n = 5): whole steps as in the main
    leg, plus the decode-only and chunk-only launches."""
    import chunked_prefill_paged_ca_amd as ca
    from chunked_prefill_paged_ca_amd.workload import make_config
    wl = make_config(n)
    st = Step(wl)
    ctx = ca.create(0)
    elapsed, _, name, region_ms, all_ms = timed_steps(st, ctx, steps, warmup)
    ctx.close()
    attn_ms = float(np.mean(all_ms))
    out = {"workload": wl.name, "tokens_per_step": st.T, "decodes": st.nd,
           "value": round(st.T * steps / elapsed, 1), "unit": "tokens/s",
           "ms_per_step": round(elapsed * 1e3 / steps, 4), "steps": steps,
           "roofline": {**roofline_of(st.dec_w, st.chk_w, attn_ms),
                        "kernel": f"{name} (decode + chunk rows, one launch)",
                        "launch_ms": round(attn_ms, 5), "launch_ms_p10_p50_p90": pct(all_ms),
                        "launches_timed": int(all_ms.size)}}
    out["parts"] = st.parts(warmup, 20)
    st.release()
    return out


def sweep_leg(chunks=(64, 128, 256, 512, 2048, 8192), reps=3):
    """The Llama-13B 8192-token prompt (MHA 40 x 128) prefilled in chunks of c (token budget c,
    8192 / c steps, each step appending its chunk and attending over the history before it):
    kernel time summed over all steps (median of `reps` passes), against the one-shot prompt
    (c = 8192).  Bytes are each step's unique K/V + q; flops the causal pairs (the same at every
    c); the bound is whichever needs longer at the peaks."""
    import torch
    import chunked_prefill_paged_ca_amd as ca
    from chunked_prefill_paged_ca_amd import accounting as acc
    from chunked_prefill_paged_ca_amd.workload import StreamCursor, make_config
    from tests import harness as H
    base = make_config(3, chunk=8192)
    q_raw, k_raw, v_raw = StreamCursor(base).take([0], [8192])
    q_all, k_all, v_all = (H.to_device(x, base.dtype) for x in (q_raw, k_raw, v_raw))
    q_rot = torch.empty_like(q_all)
    o = torch.empty_like(q_all)
    kc, vc = H.alloc_pool(base, fill=0.0)
    desc = ca.make_desc(base.num_q_heads, base.num_kv_heads, base.head_dim, base.page_size, base.dtype)
    ctx = ca.create(0)
    ctx.profile_enable(ca.PROFILE_ALL)
    res = {}
    for c in chunks:
        wl = make_config(3, chunk=c)
        work = acc.Work()
        for i in range(wl.steps):
            q = min(c, 8192 - i * c)
            work += acc.chunk_work(i * c, q, wl.num_q_heads, wl.num_kv_heads, wl.head_dim)
        totals, attn_totals = [], []
        for _ in range(reps + 1):  # the first pass warms up
            batch = ca.RequestBatch([0], [8192], wl.block_tables, c, 0, 16, wl.num_pool_pages)
            ctx.profile_read()
            done = 0
            for i in range(wl.steps):
                batch.update([done], [8192 - done])
                plan = batch.plan()
                t = plan.num_tokens
                sl = slice(done, done + t)
                ctx.append_kv_rope(desc, plan, q_all[sl], q_rot[sl], k_all[sl], v_all[sl], kc, vc,
                                   wl.num_pool_pages)
                ctx.mixed_attention(desc, plan, q_rot[sl], kc, vc, wl.num_pool_pages, o[sl])
                done += t
            torch.cuda.synchronize()
            recs = ctx.profile_read()
            totals.append(sum(ms for _, ms in recs))
            attn_totals.append(sum(ms for n, ms in recs if n in ("attention", "merge", "upload")))
        tot = float(np.median(totals[1:]))
        att = float(np.median(attn_totals[1:]))
        t_hbm = work.bytes / (HBM_PEAK_GBS * 1e9)
        t_mfma = work.flops / (BF16_PEAK_TFLOPS * 1e12)
        if t_mfma > t_hbm:
            ach, peak, unit, bound = work.flops / (att * 1e-3) / 1e12, BF16_PEAK_TFLOPS, "TFLOP/s", "mfma"
        else:
            ach, peak, unit, bound = work.bytes / (att * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s", "hbm"
        res[str(c)] = {"steps": wl.steps, "attention_merge_us": round(att * 1e3, 1),
                       "with_append_us": round(tot * 1e3, 1), "bound": bound,
                       "achieved": round(ach, 1), "unit": unit, "frac": round(ach / peak, 4),
                       "alg_bytes": int(work.bytes), "alg_flops": int(work.flops)}
    ctx.close()
    del q_all, k_all, v_all, q_rot, o, kc, vc
    torch.cuda.empty_cache()
    one = res[str(chunks[-1])]["attention_merge_us"]
    for c in chunks:
        res[str(c)]["vs_one_shot"] = round(res[str(c)]["attention_merge_us"] / one, 3)
    return {"workload": make_config(3).name.replace(" in chunks of c", ""),
            "note": "summed kernel time of the whole prompt per chunk size c (median of "
                    f"{reps} passes); attention_merge_us: the attention launches, their merges "
                    "and metadata uploads; with_append_us: plus the append launches",
            "chunks": res}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parts", action="store_true")
    ap.add_argument("--no-per-config", action="store_true",
                    help="skip the Yi-34B, LLaMA2-70B and Llama-13B sweep legs")
    ap.add_argument("--no-scrub", action="store_true", help="skip the cold-HBM (scrubbed) pass")
    ap.add_argument("--time-every", type=int, default=1,
                    help="attach timing events to every N-th attention launch of the timed region "
                         "(0: none; the launches timed after the region make up the 50)")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip re-measuring the HBM and bf16 GEMM rates this device sustains")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after the timed region, copy this many MiB device to device once (a "
                         "known-size reference for the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path has no cross-GPU exchange: it shards by heads or by requests, one independent "
              "launch per GPU)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from __graft_entry__ import ensure_built
    ensure_built()
    import chunked_prefill_paged_ca_amd as ca
    from chunked_prefill_paged_ca_amd.workload import make_config

    torch.cuda.set_device(0)
    wl = make_config(args.config)
    log(f"workload: {wl.name}")
    st = Step(wl)

    # ---- timed region: whole steps; every attention launch carries timing events ----
    ctx = ca.create(0)
    elapsed, submitted, attn_name, region_ms, all_ms = timed_steps(st, ctx, args.steps, args.warmup,
                                                                   every=args.time_every)
    ms_per_step = elapsed * 1e3 / args.steps
    value = st.T * args.steps / elapsed
    attn_ms = float(np.mean(all_ms))
    launches = args.warmup + args.steps + max(0, MIN_TIMED_LAUNCHES - int(region_ms.size))
    out = {
        "metric": "mixed chunked-prefill+decode attn tokens/s; % HBM peak and % MFMA peak",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        # host time per step to plan and enqueue it: below ms_per_step, the device is the bound
        "host_submit_ms_per_step": round(submitted * 1e3 / args.steps, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "tokens_per_step": st.T, "decodes": st.nd,
                   "token_budget": wl.token_budget, "page_size": wl.page_size,
                   "pool_pages": wl.num_pool_pages, "step": "plan + append_kv_rope + mixed_attention"},
        "roofline": {**roofline_of(st.dec_w, st.chk_w, attn_ms),
                     "kernel": f"{attn_name} (decode + chunk rows, one launch)",
                     "traffic": stored_traffic(wl.name),
                     "launch_ms": round(attn_ms, 5),
                     "launch_ms_p10_p50_p90": pct(all_ms),
                     "launches_timed": int(all_ms.size),
                     "launches_in_timed_region": int(region_ms.size),
                     "launch_ms_timed_region_mean": (round(float(np.mean(region_ms)), 5)
                                                     if region_ms.size else None),
                     "attention_launches_this_leg": launches},
    }
    if not args.no_scrub:
        st.run(ctx, MIN_TIMED_LAUNCHES, time_attention=True, scrub=True)
        torch.cuda.synchronize()
        _, cold = attention_times(ctx.profile_read())
        cm = float(np.mean(cold))
        out["roofline"]["scrubbed"] = {
            "note": f"{SCRUB_MIB} MiB read before every step, outside the events",
            "launch_ms": round(cm, 5), "launch_ms_p10_p50_p90": pct(cold),
            "launches_timed": int(cold.size),
            "frac": roofline_of(st.dec_w, st.chk_w, cm)["frac"]}
    ctx.close()

    # ---- second pass (not timed for `value`): decode and chunk as separate launches ----
    if not args.no_parts:
        out["parts"] = st.parts(args.warmup, max(args.steps, MIN_TIMED_LAUNCHES))
    st.release()

    # ---- the other workloads, one after the other ----
    if not args.no_per_config and args.config == 2:
        pc = {}
        for n in (4, 5):
            log(f"per-config leg: {make_config(n).name}")
            pc[str(n)] = per_config_leg(n)
        log("per-config leg: Llama-13B chunk-size sweep")
        pc["3"] = sweep_leg()
        out["per_config"] = pc

    # ---- what this device sustains (after the timed region): the roofline above uses the
    # datasheet peaks; these put the same launch against measured ones ----
    if not args.no_peaks:
        from chunked_prefill_paged_ca_amd import peaks
        rd, cp, gm = peaks.hbm_read_gbs(), peaks.hbm_copy_gbs(), peaks.gemm_tflops("randn")
        r = out["roofline"]
        meas = rd if r["bound"] == "hbm" else gm
        out["measured_peaks"] = {"hbm_read_nontemporal_GBs": round(rd, 1), "hbm_copy_GBs": round(cp, 1),
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
