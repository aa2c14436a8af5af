"""QKV projection on one MI355X: cost per token against the number of tokens sharing the weights.

    python -m chunked_prefill_paged_ca_amd.linear_bench [T ...]

bowenzhou.top "Sarathi：让解码搭上 prefill 的顺风车", section "Decode-maximal batching：顺车的账本":
decode tokens alone make the linear layers memory-bound (every weight is read for a handful of
tokens); riding along with a prefill chunk, they share one weight read with hundreds of tokens.
Here: the Mistral-7B q/k/v projection (hidden 4096 -> (32 + 2 x 8) x 128 = 6144 features, bf16)
through ca_qkv_projection for T tokens.  Eight weight copies are used in turn (400 MB, more than
the 256 MB last-level cache), so every call reads its weights from HBM as a real multi-layer
step does.  Times are HIP events around each call (CA_PROFILE_PROJECTION), mean of 40 calls.

Prints a markdown table: the path the library takes at that T (the weight-streaming kernel for
T <= 16, the tiled MFMA kernel above), time, TFLOP/s, GB/s (algorithmic bytes: weights + x + out),
the bound the roofline gives at that T (HBM at 8 TB/s or bf16 MFMA at 2.5 PFLOP/s) and the
fraction of it reached, the time per token, and the hipBLASLt GEMM's time at the same T
(a second context created with CA_PROJECTION_LIBRARY=1).
"""
from __future__ import annotations

import sys

import numpy as np

HBM = 8.0e12
MFMA = 2.5e15


def main(argv):
    import torch
    import chunked_prefill_paged_ca_amd as ca
    torch.cuda.set_device(0)
    Ts = [int(a) for a in argv] or [1, 16, 80, 160, 256, 512, 1024, 2048]
    Hq, Hkv, d, hidden = 32, 8, 128, 4096
    N = (Hq + 2 * Hkv) * d
    copies = 8
    ws = [torch.empty((N, hidden), dtype=torch.bfloat16, device="cuda").normal_(0.0, hidden ** -0.5)
          for _ in range(copies)]
    x = torch.randn((max(Ts), hidden), device="cuda").to(torch.bfloat16)
    out = torch.empty((max(Ts), N), dtype=torch.bfloat16, device="cuda")
    desc = ca.make_desc(Hq, Hkv, d, 16, "bf16")
    import os
    ctx = ca.create(0)
    os.environ["CA_PROJECTION_LIBRARY"] = "1"
    ctx_lib = ca.create(0)
    del os.environ["CA_PROJECTION_LIBRARY"]

    def time_calls(c, T):
        for i in range(2 * copies):  # plan this T and warm the library
            c.qkv_projection(desc, T, hidden, x, ws[i % copies], out)
        torch.cuda.synchronize()
        c.profile_read()
        c.profile_enable(ca.PROFILE_PROJECTION)
        reps = 40
        for i in range(reps):
            c.qkv_projection(desc, T, hidden, x, ws[i % copies], out)
        torch.cuda.synchronize()
        c.profile_enable(False)
        return float(np.mean([ms for _, ms in c.profile_read()])) * 1e3

    rows = ["| T | path | us per call | TFLOP/s | GB/s | roofline bound | fraction of bound | us per token "
            "| hipBLASLt us |",
            "|---|---|---|---|---|---|---|---|---|"]
    for T in Ts:
        us = time_calls(ctx, T)
        us_lib = time_calls(ctx_lib, T)
        path = "streaming kernel" if T <= 16 and hidden % 2048 == 0 and N % 32 == 0 else "tiled kernel"
        flops = 2.0 * T * hidden * N
        nbytes = 2.0 * (N * hidden + T * hidden + T * N)
        t_hbm, t_mfma = nbytes / HBM, flops / MFMA
        bound = "HBM" if t_hbm >= t_mfma else "MFMA"
        frac = max(t_hbm, t_mfma) / (us * 1e-6)
        rows.append(f"| {T} | {path} | {us:.1f} | {flops / us / 1e6:.0f} | {nbytes / us / 1e3:.0f} | "
                    f"{bound} | {frac:.2f} | {us / T:.3f} | {us_lib:.1f} |")
        print(rows[-1], file=sys.stderr, flush=True)
    ctx.close()
    ctx_lib.close()
    print(f"# QKV projection, Mistral-7B shapes (4096 -> 6144, bf16), weights read from HBM\n\n"
          f"Command (repository root, one MI355X): `python3 -m chunked_prefill_paged_ca_amd.linear_bench "
          f"{' '.join(argv)}`\n")
    print("\n".join(rows))
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
