"""Build the HIP library libca.so in-tree for gfx950 (hipcc; no JIT, no torch extension).

Every kernel source and the host runtime are compiled into one shared library whose only
interface is the C ABI of include/ca.h.  A second, separate library, libca_probe.so, holds the
measurement probe of csrc/probe_mfma.hip (not part of the attention path).
"""
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libca.so")
SOURCES = ["api.hip", "plan.cpp", "sched.cpp", "linear.cpp", "linear_skinny.hip", "linear_tiled.hip",
           "append_rope.hip",
           "attn_generic.hip", "attn_mixed.hip", "merge.hip"]
LIBS = ["-L/opt/rocm/lib", "-lhipblaslt"]  # the QKV projection's GEMM
PROBE_LIB = os.path.join(PKG, "libca_probe.so")
PROBE_SOURCE = "probe_mfma.hip"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, jobs: int = 8) -> str:
    tmp = LIB + ".tmp"
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    common = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-Wall", "-Wno-unused-result", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    procs, objs = [], []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [hipcc()] + common + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
    failed = []
    for src, pr in procs:
        out, _ = pr.communicate()
        text = out.decode(errors="replace")
        # the host pass does not know the packed-fp32 feature flag; that warning is expected
        lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln]
        if lines and (verbose or pr.returncode):
            print("\n".join(lines), flush=True)
        if pr.returncode:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    link = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs + LIBS
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(tmp, LIB)
    probe = [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-x", "hip",
             os.path.join(CSRC, PROBE_SOURCE), "-o", PROBE_LIB + ".tmp"]
    if verbose:
        print(" ".join(probe), flush=True)
    pr = subprocess.run(probe, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if pr.returncode:
        print(pr.stdout.decode(errors="replace"), flush=True)
        raise RuntimeError(f"hipcc failed for {PROBE_SOURCE}")
    os.replace(PROBE_LIB + ".tmp", PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
