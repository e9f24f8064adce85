"""Build the gfx950 HIP library in-tree: weight_only_int4_stats_amd/libawq_gfx950.so.

Usage:  python -m weight_only_int4_stats_amd.build   (or build() from Python)

Every source is compiled with hipcc for gfx950 only, into _build/, then linked
into one shared library next to this file.  Flags:
  -ffp-contract=off      no implicit a*b+c -> fma: the quantizer's float steps
                         are each rounded as written (fma only where spelled out)
  -fhip-fp32-correctly-rounded-divide-sqrt   IEEE float division
  -Xclang -target-feature -Xclang -packed-fp32-ops   no packed fp32 VALU ops
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libawq_gfx950.so")
SOURCES = ["awq_api.cpp", "k_act_stats.hip", "k_quantize.hip", "k_search.hip", "k_gram.hip", "k_w4a16.hip",
           "k_gemv1.hip", "k_fold.hip", "k_salient.hip", "awq_noalloc.hip", "k_mid.hip", "k_skinny.hip", "k_stream.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build the library")


def flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-command-line-argument",
        "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
    ]


def build(verbose: bool = False, jobs: int = 4) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.rsplit(".", 1)[0] + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [cc] + flags() + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len(procs) >= jobs:
            _wait(procs.pop(0))
    for p in procs:
        _wait(p)
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    out = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if out.returncode != 0:
        raise RuntimeError(f"link failed:\n{out.stdout}")
    os.replace(tmp, LIB)
    return LIB


def _wait(item) -> None:
    src, p = item
    out, _ = p.communicate()
    text = out.decode(errors="replace")
    lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if p.returncode != 0:
        raise RuntimeError(f"compile of {src} failed:\n" + "\n".join(lines))
    if lines:
        print(f"[{src}]\n" + "\n".join(lines), file=sys.stderr)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
