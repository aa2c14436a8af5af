"""Serving-loop measurement: ca_sched driving append + attention round after round on one MI355X.

    python -m chunked_prefill_paged_ca_amd.serve_bench [--rounds R] [--requests N]

Mistral-7B layer shapes (32 q heads, 8 kv heads, d 128, bf16, page 16), token budget 512, a
64K-page pool.  N requests arrive over the first half of the rounds (a few per round): prompts
log-uniform in [128, 4096] tokens, a fifth with a cached prefix of up to half the prompt, 32..256
decode steps each.  Each round: ca_sched_step (host), ca_append_kv_rope and ca_mixed_attention
on the plan (device), ca_sched_commit (host).  q/k/v are random device rows (the timing does not
depend on their values; correctness of the loop is tested against the oracle elsewhere).

Prints a markdown summary: whole-loop tokens per second (host and device work overlapping as
they do in a serving loop), the host time of each call per round in that loop (which includes
waiting for a free staging slot when the host runs ahead of the device), the device time of the
round's kernels (HIP events attached to the launches, a separate pass), and the calls' own host
cost (a third pass that lets the device drain after every round).
"""
from __future__ import annotations

import argparse
import math
import sys
import time

import numpy as np


def scenario(n: int, rounds: int, seed: int = 17):
    rng = np.random.default_rng([seed, 4])
    arrival = np.sort(rng.integers(0, max(1, rounds // 2), size=n))
    prompt = np.exp(rng.uniform(math.log(128), math.log(4096), size=n)).astype(np.int64)
    cached = np.where(rng.random(n) < 0.2, (prompt * rng.uniform(0, 0.5, size=n)).astype(np.int64), 0)
    max_new = rng.integers(32, 257, size=n)
    return arrival, prompt, cached, max_new


def run(rounds: int, n: int, timed_kernels: bool, sync_rounds: bool = False):
    """One pass of the loop.  sync_rounds: wait for the device at the end of every round (outside
    the timed host sections), so the host times below are the calls' own cost, without the waits
    for a free staging slot that a loop running ahead of the device meets."""
    import torch
    import chunked_prefill_paged_ca_amd as ca
    torch.cuda.set_device(0)
    Hq, Hkv, d, P, tau, pool = 32, 8, 128, 16, 512, 65536
    k_cache = torch.empty((pool, Hkv, d // 8, P, 8), dtype=torch.bfloat16, device="cuda").normal_()
    v_cache = torch.empty((pool, Hkv, d // 16, 4, 16, 4), dtype=torch.bfloat16, device="cuda").normal_()
    q = torch.randn((tau, Hq, d), device="cuda").to(torch.bfloat16)
    kn = torch.randn((tau, Hkv, d), device="cuda").to(torch.bfloat16)
    vn = torch.randn_like(kn)
    q_rot = torch.empty_like(q)
    o = torch.empty_like(q)
    lse = torch.empty((tau, Hq), dtype=torch.float32, device="cuda")
    desc = ca.make_desc(Hq, Hkv, d, P, "bf16")
    arrival, prompt, cached, max_new = scenario(n, rounds)
    sched = ca.Scheduler(tau, 0, P, pool)
    ctx = ca.create(0)
    if timed_kernels:
        ctx.profile_enable(True)
    added, tokens, decodes, host_step, host_commit, host_append, host_attn = 0, 0, 0, 0.0, 0.0, 0.0, 0.0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for rnd in range(rounds):
        while added < n and arrival[added] <= rnd:
            need = -(-int(cached[added]) // P)
            if sched.free_pages() < need:
                break
            sched.add(int(prompt[added]), int(max_new[added]), int(cached[added]))
            added += 1
        h0 = time.perf_counter()
        plan = sched.step()
        host_step += time.perf_counter() - h0
        T = plan.num_tokens
        if T:
            h0 = time.perf_counter()
            ctx.append_kv_rope(desc, plan, q, q_rot, kn, vn, k_cache, v_cache, pool)
            h1 = time.perf_counter()
            ctx.mixed_attention(desc, plan, q_rot, k_cache, v_cache, pool, o, lse)
            host_append += h1 - h0
            host_attn += time.perf_counter() - h1
        tokens += T
        decodes += plan.num_decodes
        h0 = time.perf_counter()
        sched.commit()
        host_commit += time.perf_counter() - h0
        if sync_rounds:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kernel_us = 0.0
    if timed_kernels:
        kernel_us = sum(ms for _, ms in ctx.profile_read()) * 1e3
    finished = sum(1 for i in range(added) if sched.get(i)["state"] == ca.CA_REQ_FINISHED)
    preempt = sum(sched.get(i)["num_preemptions"] for i in range(added))
    ctx.close()
    sched.close()
    return {"rounds": rounds, "admitted": added, "finished": finished, "preemptions": preempt,
            "tokens": tokens, "decode_tokens": decodes, "elapsed_s": elapsed,
            "host_step_us": host_step / rounds * 1e6, "host_commit_us": host_commit / rounds * 1e6,
            "host_append_us": host_append / rounds * 1e6, "host_attn_us": host_attn / rounds * 1e6,
            "kernel_us_per_round": kernel_us / rounds}


def main(argv):
    ap = argparse.ArgumentParser()
    ap.add_argument("--rounds", type=int, default=400)
    ap.add_argument("--requests", type=int, default=200)
    args = ap.parse_args(argv)
    free = run(args.rounds, args.requests, timed_kernels=False)
    timed = run(args.rounds, args.requests, timed_kernels=True)
    own = run(args.rounds, args.requests, timed_kernels=False, sync_rounds=True)
    own_total = own["host_step_us"] + own["host_append_us"] + own["host_attn_us"] + own["host_commit_us"]
    tps = free["tokens"] / free["elapsed_s"]
    out = [
        f"# Serving loop: Mistral-7B layer shapes, token budget 512, 64K-page pool, {args.requests} requests",
        "",
        f"Command (repository root, one MI355X): `python3 -m chunked_prefill_paged_ca_amd.serve_bench "
        f"--rounds {args.rounds} --requests {args.requests}`",
        "",
        "| quantity | value |",
        "|---|---|",
        f"| rounds | {free['rounds']} |",
        f"| requests admitted / finished | {free['admitted']} / {free['finished']} |",
        f"| preemptions | {free['preemptions']} |",
        f"| tokens processed (decode tokens) | {free['tokens']} ({free['decode_tokens']}) |",
        f"| mean tokens per round | {free['tokens'] / free['rounds']:.1f} |",
        f"| whole loop, host and device overlapping | {free['elapsed_s'] * 1e3:.1f} ms -> **{tps / 1e6:.2f} M tokens/s** |",
        f"| ca_sched_step host time per round | {free['host_step_us']:.1f} us |",
        f"| ca_sched_commit host time per round | {free['host_commit_us']:.1f} us |",
        f"| ca_append_kv_rope call, host time per round | {free['host_append_us']:.1f} us |",
        f"| ca_mixed_attention call, host time per round | {free['host_attn_us']:.1f} us |",
        f"| device time per round (upload + append + attention + merge; timed pass) | {timed['kernel_us_per_round']:.1f} us |",
        f"| host cost per round, device idle at every call (step / append / attention / commit) | "
        f"{own_total:.1f} us ({own['host_step_us']:.1f} / {own['host_append_us']:.1f} / "
        f"{own['host_attn_us']:.1f} / {own['host_commit_us']:.1f}) |",
    ]
    print("\n".join(out))
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
