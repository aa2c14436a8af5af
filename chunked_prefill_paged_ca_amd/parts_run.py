"""Run one workload's steps with the decode and prefill-chunk rows as two separate launches.

    python -m chunked_prefill_paged_ca_amd.parts_run [--config N] [--steps K] [--warmup W]
                                                     [--copy-mib M]

Each step is the bench's step (plan, append + RoPE, attention, merge) with the attention call
split into a "chunk" launch followed by a "decode" launch of the same kernel (CA_SPLIT_ATTENTION=1),
so that counters taken by `rocprofv3 --pmc` attribute to each part on its own: in every step the
first attention dispatch is the chunk rows and the second the decode rows.  Prints one JSON line:
the mean event time of each launch kind, the algorithmic bytes of the decode rows and flops of
the chunk rows (accounting.py), and the launch order.  --copy-mib copies that many MiB device to
device once at the end, as a known-size reference for the HBM byte counters.
"""
from __future__ import annotations

import argparse
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", type=int, default=4)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--copy-mib", type=int, default=0)
    args = ap.parse_args(argv)

    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import torch
    import chunked_prefill_paged_ca_amd as ca
    from chunked_prefill_paged_ca_amd import accounting as acc
    from chunked_prefill_paged_ca_amd.workload import StreamCursor, make_config
    from tests import harness as H

    torch.cuda.set_device(0)
    wl = make_config(args.config)
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
    kv_lens = np.array([int(wl.num_computed[r]) + int(q) for r, q in zip(a["req_ids"], q_lens)])
    dec_w, chk_w = acc.plan_work(q_lens, kv_lens, plan0.num_decodes, wl.num_q_heads,
                                 wl.num_kv_heads, wl.head_dim, wl.page_size)
    stream = torch.cuda.current_stream()

    os.environ["CA_SPLIT_ATTENTION"] = "1"
    try:
        ctx = ca.create(0)
    finally:
        del os.environ["CA_SPLIT_ATTENTION"]

    def run(n):
        for _ in range(n):
            plan = batch.plan()
            ctx.append_kv_rope(desc, plan, q_in, q_rot, k_in, v_in, kc, vc, wl.num_pool_pages, stream=stream)
            ctx.mixed_attention(desc, plan, q_rot, kc, vc, wl.num_pool_pages, o, lse, stream=stream)

    run(args.warmup)
    torch.cuda.synchronize()
    ctx.profile_read()
    ctx.profile_enable(True)
    run(args.steps)
    torch.cuda.synchronize()
    ctx.profile_enable(False)
    per = {}
    order = []
    for name, ms in ctx.profile_read():
        per.setdefault(name, []).append(ms)
        if name in ("chunk", "decode") and len(order) < 2:
            order.append(name)
    ctx.close()
    if args.copy_mib > 0:
        src = torch.ones(args.copy_mib * (1 << 20) // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
    print(json.dumps({"workload": wl.name, "steps": args.steps,
                      "kernel_ms": {k: float(np.mean(v)) for k, v in per.items()},
                      "attention_launch_order": order,
                      "decode_alg_bytes": int(dec_w.bytes), "chunk_alg_flops": int(chk_w.flops),
                      "chunk_alg_bytes": int(chk_w.bytes), "copy_mib": args.copy_mib}), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
