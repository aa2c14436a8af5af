"""What this MI355X actually sustains, next to the datasheet peaks the roofline uses.

    python -m chunked_prefill_paged_ca_amd.peaks

Prints a markdown table:
  * bf16 MFMA issue rate (libca_probe.so: back-to-back v_mfma_f32_16x16x32_bf16 from registers,
    one workgroup per CU) for constant, zero, N(0, 1) and softmax-like operands -- the rate
    depends on the operand data on this part;
  * a large bf16 GEMM through torch.matmul (8192^3, hipBLASLt) on N(0, 1) and on all-ones data;
  * HBM: read streams of 800 MiB and 4 GiB with plain and with non-temporal loads
    (libca_probe.so: each wavefront reads whole 16 KB chunks, 16 loads of 16 bytes per lane in
    flight) and a 1 GiB device-to-device copy (read + write, torch).
The datasheet figures are 2.5 PFLOP/s dense bf16 and 8 TB/s HBM.
"""
from __future__ import annotations

import ctypes
import os
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
PROBE_LIB = os.path.join(PKG, "libca_probe.so")
MODES = ["ones", "zeros", "N(0, 1)", "exp(-|3z|), z ~ N(0, 1)"]


def _probe():
    if not os.path.exists(PROBE_LIB):
        raise RuntimeError(f"{PROBE_LIB} is not built (run the package build first)")
    lib = ctypes.CDLL(PROBE_LIB)
    lib.ca_probe_read_rate.restype = ctypes.c_int
    lib.ca_probe_read_rate.argtypes = [ctypes.c_size_t, ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
    lib.ca_probe_mfma_rate.restype = ctypes.c_int
    lib.ca_probe_mfma_rate.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                                       ctypes.POINTER(ctypes.c_float)]
    return lib


def mfma_rate(mode: int, iters: int = 4000):
    lib = _probe()
    tf, ms = ctypes.c_double(), ctypes.c_float()
    rc = lib.ca_probe_mfma_rate(mode, iters, ctypes.byref(tf), ctypes.byref(ms))
    if rc:
        raise RuntimeError(f"ca_probe_mfma_rate failed: HIP error {rc}")
    return tf.value, ms.value


def timed(fn, reps):
    import torch
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / reps


def gemm_tflops(kind: str, n: int = 8192) -> float:
    import torch
    if kind == "ones":
        a = torch.ones((n, n), dtype=torch.bfloat16, device="cuda")
        b = torch.ones((n, n), dtype=torch.bfloat16, device="cuda")
    else:
        g = torch.Generator(device="cuda").manual_seed(1)
        a = torch.randn((n, n), device="cuda", generator=g).to(torch.bfloat16)
        b = torch.randn((n, n), device="cuda", generator=g).to(torch.bfloat16)
    dt = timed(lambda: torch.matmul(a, b), 10)
    return 2.0 * n ** 3 / dt / 1e12


def hbm_copy_gbs(mib: int = 1024) -> float:
    import torch
    x = torch.ones(mib * (1 << 20) // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    dt = timed(lambda: y.copy_(x), 20)
    return 2.0 * x.numel() * 4 / dt / 1e9


def hbm_read_gbs(mib: int = 4096, nontemporal: bool = True) -> float:
    gbs = ctypes.c_double()
    rc = _probe().ca_probe_read_rate(mib * (1 << 20), int(nontemporal), ctypes.byref(gbs))
    if rc:
        raise RuntimeError(f"ca_probe_read_rate failed: HIP error {rc}")
    return gbs.value


def main(argv):
    import torch
    torch.cuda.set_device(0)
    rows = ["| what | measured | of datasheet peak |", "|---|---|---|"]
    for m, name in enumerate(MODES):
        tf, _ = mfma_rate(m)
        rows.append(f"| bf16 MFMA issue rate, operands {name} | {tf:.0f} TFLOP/s | {tf / 2500:.1%} |")
        print(rows[-1], file=sys.stderr, flush=True)
    for kind in ("N(0, 1)", "ones"):
        tf = gemm_tflops("ones" if kind == "ones" else "randn")
        rows.append(f"| torch.matmul bf16 8192^3, operands {kind} | {tf:.0f} TFLOP/s | {tf / 2500:.1%} |")
        print(rows[-1], file=sys.stderr, flush=True)
    c = hbm_copy_gbs()
    rows.append(f"| HBM copy 1 GiB (read + write) | {c:.0f} GB/s | {c / 8000:.1%} |")
    for mib in (800, 4096):
        for nt in (False, True):
            r = hbm_read_gbs(mib, nt)
            rows.append(f"| HBM read stream {mib} MiB, {'non-temporal' if nt else 'plain'} loads | {r:.0f} GB/s | {r / 8000:.1%} |")
            print(rows[-1], file=sys.stderr, flush=True)
    print("# Measured ceilings on one MI355X\n\nCommand (repository root): "
          "`python3 -m chunked_prefill_paged_ca_amd.peaks`\n")
    print("\n".join(rows))
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
