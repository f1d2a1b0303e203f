"""Build libcider.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Every source is compiled in-tree into ``_build/`` and linked into
``w4a8_quantized_linear_amd/libcider.so``.  Packed-fp32 instructions are
disabled for the device code (-packed-fp32-ops); division and sqrt keep
their correctly rounded default lowering (no fast-math), which the
quantizers rely on.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIBRARY = os.path.join(PKG, "libcider.so")
SOURCES = ["api.hip", "quantize.hip", "clip.hip", "smooth.hip", "decode.hip", "gemm.hip", "gemm_few.hip", "gemm_skinny.hip", "gemv.hip"]
HEADERS = ["cider_kernels.h", "quant_common.h"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
    "-Wall", "-Wno-unused-result",
]


def _stale(out: str, deps: list[str]) -> bool:
    if not os.path.exists(out):
        return True
    t = os.path.getmtime(out)
    return any(os.path.getmtime(d) > t for d in deps)


def build(force: bool = True, verbose: bool = False) -> str:
    """Compile and link.  force=False skips sources whose object is newer
    than the source and the shared headers."""
    os.makedirs(BUILD, exist_ok=True)
    headers = [os.path.join(CSRC, h) for h in HEADERS] + [os.path.join(ROOT, "include", "cider.h")]
    procs = []
    objs = []
    for src in SOURCES:
        s = os.path.join(CSRC, src)
        o = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(o)
        if force or _stale(o, [s] + headers):
            cmd = [HIPCC, *FLAGS, "-c", s, "-o", o]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l]
        if p.returncode != 0:
            failed.append(src)
            sys.stderr.write("\n".join(lines) + "\n")
        elif verbose and lines:
            print("\n".join(lines))
    if failed:
        raise RuntimeError("hipcc failed for " + ", ".join(failed))
    if force or procs or _stale(LIBRARY, objs):
        tmp = LIBRARY + ".tmp%d" % os.getpid()
        subprocess.run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp, *objs],
                       check=True)
        os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    build(force="--incremental" not in sys.argv, verbose=True)
