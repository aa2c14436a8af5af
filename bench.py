"""Benchmark: one mixed chunked-prefill + decode step per iteration on one MI355X.

A step is the whole hot path over one batch: ca_plan_batch (host), ca_append_kv_rope and
ca_mixed_attention, on the Mistral-7B-shaped single-layer batch of the 512-token budget example
(32 q heads, 8 kv heads, d 128, bf16, page 16): 80 decodes with contexts uniform in [512, 4096],
prefill P getting 300 tokens on 1200 cached and prefill Q getting 132 on 2048, pages permuted
over a 64K-page pool.  Inputs are resident in HBM before the timed region starts.

Prints ONE JSON line (rank 0).  `roofline` places the dominant kernel (the decode attention,
HBM-bound) against the 8 TB/s HBM peak using algorithmic bytes and the kernel's own duration
(HIP events the library records around its launches on the bench's stream); `mfma` does the same
for the prefill-chunk kernel against the dense bf16 peak; `cpu_baseline` times the CPU oracle on
the same step.
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


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def cpu_baseline(wl):
    """The oracle as it stands on the whole step (every row), best of 3 runs."""
    import oracle
    from chunked_prefill_paged_ca_amd.workload import StreamCursor
    sess = oracle.Session(wl)
    p = sess.plan()
    q, k, v = StreamCursor(wl).take(p["req_ids"], np.diff(p["qo_indptr"]))
    nd = p["num_decodes"]
    T = p["num_tokens"]
    threads = oracle.default_threads()
    times = []
    for _ in range(3):
        fresh = sess.fork()
        t0 = time.perf_counter()
        fresh.step(p, q, k, v, nthreads=threads)
        times.append(time.perf_counter() - t0)
    dt = min(times)
    return {"value": round(T / dt, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"the whole step: all {T} rows ({nd} decode rows + 2 prefill chunks), "
                      f"fp64 C oracle on {threads} threads, best of 3 runs of {dt:.2f} s each"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
    ctx = ca.create(0)
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

    def step():
        plan = batch.plan()
        ctx.append_kv_rope(desc, plan, q_in, q_rot, k_in, v_in, kc, vc, wl.num_pool_pages, stream=stream)
        ctx.mixed_attention(desc, plan, q_rot, kc, vc, wl.num_pool_pages, o, lse, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ctx.profile_read()  # drop anything recorded so far
    ctx.profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ctx.profile_enable(False)
    recs = ctx.profile_read()
    per = {}
    for name, ms in recs:
        per.setdefault(name, []).append(ms)
    kern_ms = {k: float(np.mean(v)) for k, v in per.items()}
    ms_per_step = elapsed * 1e3 / args.steps
    value = T * args.steps / elapsed
    attn_ms = sum(kern_ms.get(k, 0.0) for k in ("chunk", "decode", "merge", "generic"))

    # dominant kernel: the decode split-KV kernel (HBM-bound); the chunk kernel is MFMA-bound
    dec_ms = kern_ms.get("decode", kern_ms.get("generic", float("nan")))
    achieved = dec_w.bytes / (dec_ms * 1e-3) / 1e9
    chunk_tflops = chk_w.flops / (kern_ms["chunk"] * 1e-3) / 1e12 if "chunk" in kern_ms else None
    out = {
        "metric": "mixed chunked-prefill+decode attn tokens/s; % HBM peak and % MFMA peak",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "tokens_per_step": T, "decodes": nd,
                   "token_budget": wl.token_budget, "page_size": wl.page_size,
                   "pool_pages": wl.num_pool_pages, "step": "plan + append_kv_rope + mixed_attention"},
        "kernel_ms": {k: round(v, 5) for k, v in kern_ms.items()},
        "attention_kernels_ms": round(attn_ms, 5),
        "roofline": {"bound": "hbm", "kernel": "decode", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None, "alg_bytes_per_launch": int(dec_w.bytes)},
        "mfma": {"kernel": "chunk", "alg_flops_per_launch": int(chk_w.flops),
                 "achieved_tflops": None if chunk_tflops is None else round(chunk_tflops, 2),
                 "peak_tflops": BF16_PEAK_TFLOPS,
                 "frac": None if chunk_tflops is None else round(chunk_tflops / BF16_PEAK_TFLOPS, 4)},
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on the same step ...")
        out["cpu_baseline"] = cpu_baseline(wl)
    ctx.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
