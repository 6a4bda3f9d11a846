"""Build libtileq.so (all HIP kernels + the C ABI host runtime) for gfx950.

    python -m bit_rank_post_amd.build        # or __graft_entry__.build()

Every source is compiled with hipcc for --offload-arch=gfx950 in parallel into
_build/, then linked into bit_rank_post_amd/libtileq.so (in-tree, so it ships
with the source tree)."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libtileq.so")
# (source, object name, extra flags): the prefill GEMM is compiled once per
# residual code width
SOURCES = [("route.hip", "route", []), ("colproj.hip", "colproj", []),
           ("gemm_prefill.hip", "gemm_prefill2", ["-DTQ_PREFILL_BITS=2"]),
           ("gemm_prefill.hip", "gemm_prefill3", ["-DTQ_PREFILL_BITS=3"]),
           ("gemm_decode.hip", "gemm_decode", []), ("decode_stages.hip", "decode_stages", []),
           ("combine.hip", "combine", []), ("upload.hip", "upload", []),
           ("router.hip", "router", []), ("pack.hip", "pack", []),
           ("tileq_host.cpp", "tileq_host", [])]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def flags():
    return ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    procs = []
    objs = []
    for src, name, extra in SOURCES:
        obj = os.path.join(BUILD, name + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmd = [cc] + flags() + extra + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((src, cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                 stderr=subprocess.STDOUT)))
    failed = []
    for src, cmd, p in procs:
        out = p.communicate()[0].decode(errors="replace")
        out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed.append((src, out))
        elif verbose and out.strip():
            print(out)
    if failed:
        msg = "\n".join(f"--- {s}\n{o}" for s, o in failed)
        raise RuntimeError("hipcc failed:\n" + msg)
    tmp = LIB + ".tmp"
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout.decode(errors="replace"))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
