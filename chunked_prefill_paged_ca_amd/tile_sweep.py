"""Tile quantisation of the prefill-chunk attention on one MI355X, and what chunk alignment buys.

Sarathi-Serve 完全拆解 (pinghaoyang.com.cn), section "257 为什么可能比 256 慢 32%": a chunk one
token past a tile multiple makes the kernel launch a whole extra row of tiles that does almost
no useful work, so planners snap chunk sizes to tile multiples.  Here the workload is the
Llama-13B prompt of 8192 tokens (MHA, 40 heads, d 128, bf16):

    python -m chunked_prefill_paged_ca_amd.tile_sweep single [c ...]
        one step: the last chunk of c rows on a history of 8192 - c; per-kernel times
    python -m chunked_prefill_paged_ca_amd.tile_sweep prompt [c ...]
        the whole prompt at token budget c, with chunk_align 0 and 32: the summed kernel time of
        all steps (append + attention + merge)
    python -m chunked_prefill_paged_ca_amd.tile_sweep sweep [c ...]
        the whole prompt at chunk size c against the one-shot prefill (c = 8192): attention time
        summed over the K = 8192/c steps, the K/V bytes it must read (the history is read again
        at every chunk) and the flops, each against its roofline

The sweep follows the chunk-size trade-off of [SS] "为什么总 FLOPs 近似不变，显存流量却增加":
the flops of the whole prompt do not depend on c, the K/V bytes read grow as c shrinks, so small
chunks are bound by HBM and large ones by MFMA.

Prints one markdown table per mode.  Needs the GPU library; uses random K/V (the timing does
not depend on the values).
"""
from __future__ import annotations

import sys

import numpy as np

DEFAULT_SINGLE = [224, 255, 256, 257, 288, 511, 512, 513]
DEFAULT_PROMPT = [256, 257, 512, 513]
DEFAULT_SWEEP = [64, 128, 256, 512, 2048, 8192]
HBM = 8.0e12
MFMA = 2.5e15


def _setup():
    import torch
    import chunked_prefill_paged_ca_amd as ca
    from chunked_prefill_paged_ca_amd.workload import make_config
    torch.cuda.set_device(0)
    wl = make_config(3, chunk=256)
    H, d = wl.num_kv_heads, wl.head_dim
    k = torch.randn((wl.num_pool_pages, H, d // 8, 16, 8), device="cuda").to(torch.bfloat16)
    v = torch.randn((wl.num_pool_pages, H, d // 16, 4, 16, 4), device="cuda").to(torch.bfloat16)
    desc = ca.make_desc(wl.num_q_heads, H, d, 16, "bf16")
    return torch, ca, wl, k, v, desc


def _run_step(torch, ca, ctx, wl, k, v, desc, plan, q, kn, vn):
    q_rot = torch.empty_like(q)
    o = torch.empty_like(q)
    ctx.append_kv_rope(desc, plan, q, q_rot, kn, vn, k, v, wl.num_pool_pages)
    ctx.mixed_attention(desc, plan, q_rot, k, v, wl.num_pool_pages, o, None)


def _inputs(torch, wl, T):
    q = torch.randn((T, wl.num_q_heads, wl.head_dim), device="cuda").to(torch.bfloat16)
    kn = torch.randn((T, wl.num_kv_heads, wl.head_dim), device="cuda").to(torch.bfloat16)
    return q, kn, torch.randn_like(kn)


def _kernel_us(recs):
    per = {}
    for name, ms in recs:
        per.setdefault(name, []).append(ms * 1e3)
    return per


def single(cs, reps=20):
    torch, ca, wl, k, v, desc = _setup()
    L = 8192
    rows = ["| c | attention us | merge us | attention us per row |", "|---|---|---|---|"]
    for c in cs:
        ctx = ca.create(0)
        plan = ca.plan_batch([L - c], [c], wl.block_tables, c, 0, 16, wl.num_pool_pages)
        q, kn, vn = _inputs(torch, wl, c)
        for _ in range(3):
            _run_step(torch, ca, ctx, wl, k, v, desc, plan, q, kn, vn)
        torch.cuda.synchronize()
        ctx.profile_read()
        ctx.profile_enable(True)
        for _ in range(reps):
            _run_step(torch, ca, ctx, wl, k, v, desc, plan, q, kn, vn)
        torch.cuda.synchronize()
        ctx.profile_enable(False)
        per = _kernel_us(ctx.profile_read())
        ctx.close()
        att = float(np.mean(per.get("attention", per.get("chunk", [0.0]))))
        mrg = float(np.mean(per.get("merge", [0.0])))
        rows.append(f"| {c} | {att:.1f} | {mrg:.1f} | {att / c:.3f} |")
        print(rows[-1], file=sys.stderr, flush=True)
    return "\n".join(rows) + "\n"


def prompt(cs, aligns=(0, 32)):
    torch, ca, wl, k, v, desc = _setup()
    L = 8192
    rows = ["| budget c | chunk_align | steps | chunk sizes | total kernel us |", "|---|---|---|---|---|"]
    for c in cs:
        for a in aligns:
            ctx = ca.create(0)
            nc, left, sizes, total = 0, L, [], 0.0
            while left > 0:
                plan = ca.plan_batch([nc], [left], wl.block_tables, c, 0, 16, wl.num_pool_pages,
                                     chunk_align=a)
                T = plan.num_tokens
                q, kn, vn = _inputs(torch, wl, T)
                _run_step(torch, ca, ctx, wl, k, v, desc, plan, q, kn, vn)  # warm this shape
                torch.cuda.synchronize()
                ctx.profile_read()
                ctx.profile_enable(True)
                _run_step(torch, ca, ctx, wl, k, v, desc, plan, q, kn, vn)
                torch.cuda.synchronize()
                ctx.profile_enable(False)
                total += sum(sum(x) for x in _kernel_us(ctx.profile_read()).values())
                sizes.append(T)
                nc += T
                left -= T
            ctx.close()
            uniq = sorted(set(sizes[:-1]))
            desc_sizes = f"{uniq} + last {sizes[-1]}" if len(sizes) > 1 else f"{sizes}"
            rows.append(f"| {c} | {a} | {len(sizes)} | {desc_sizes} | {total:.0f} |")
            print(rows[-1], file=sys.stderr, flush=True)
    return "\n".join(rows) + "\n"


def sweep(cs, reps=3):
    from chunked_prefill_paged_ca_amd import accounting as acc
    torch, ca, wl, k, v, desc = _setup()
    L, H, d = 8192, wl.num_kv_heads, wl.head_dim
    rows = ["| c | steps | attention + merge us | K/V bytes read GB | flops GF | TB/s | TF/s | "
            "roofline us (8 TB/s, 2.5 PF) | fraction of roofline | append + upload us |",
            "|---|---|---|---|---|---|---|---|---|---|"]
    for c in cs:
        ctx = ca.create(0)
        nc, steps, att, other, nbytes, flops = 0, 0, 0.0, 0.0, 0.0, 0.0
        t_roof = 0.0
        while nc < L:
            plan = ca.plan_batch([nc], [L - nc], wl.block_tables, c, 0, 16, wl.num_pool_pages)
            T = plan.num_tokens
            _, chk = acc.plan_work([T], [nc + T], 0, wl.num_q_heads, H, d, 16)
            q, kn, vn = _inputs(torch, wl, T)
            _run_step(torch, ca, ctx, wl, k, v, desc, plan, q, kn, vn)  # warm this shape
            torch.cuda.synchronize()
            ctx.profile_read()
            ctx.profile_enable(True)
            for _ in range(reps):
                _run_step(torch, ca, ctx, wl, k, v, desc, plan, q, kn, vn)
            torch.cuda.synchronize()
            ctx.profile_enable(False)
            per = _kernel_us(ctx.profile_read())
            att += sum(sum(per.get(n, [])) for n in ("attention", "chunk", "decode", "merge")) / reps
            other += sum(sum(per.get(n, [])) for n in ("append_rope", "upload")) / reps
            nbytes += chk.bytes
            flops += chk.flops
            t_roof += max(chk.bytes / HBM, chk.flops / MFMA)
            nc += T
            steps += 1
        ctx.close()
        rows.append(f"| {c} | {steps} | {att:.0f} | {nbytes / 1e9:.2f} | {flops / 1e9:.0f} | "
                    f"{nbytes / att / 1e6:.2f} | {flops / att / 1e6:.0f} | {t_roof * 1e6:.0f} | "
                    f"{t_roof * 1e6 / att:.2f} | {other:.0f} |")
        print(rows[-1], file=sys.stderr, flush=True)
    return "\n".join(rows) + "\n"


def main(argv):
    if not argv or argv[0] not in ("single", "prompt", "sweep"):
        print(__doc__, file=sys.stderr)
        return 2
    cs = [int(x) for x in argv[1:]]
    if argv[0] == "single":
        sys.stdout.write(single(cs or DEFAULT_SINGLE))
    elif argv[0] == "sweep":
        sys.stdout.write(sweep(cs or DEFAULT_SWEEP))
    else:
        sys.stdout.write(prompt(cs or DEFAULT_PROMPT))
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
