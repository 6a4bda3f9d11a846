"""Build libtileq.so (all HIP kernels + the C ABI host runtime) for gfx950.

    python -m bit_rank_post_amd.build        # or __graft_entry__.build()
    python -m bit_rank_post_amd.build --asan # host-sanitized variant (CPU tests)

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
           ("router.hip", "router", []), ("pack.hip", "pack", []), ("calib.hip", "calib", []),
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


ASAN_DIR = os.path.join(BUILD, "asan")
ASAN_LIB = os.path.join(ASAN_DIR, "libtileq_asan.so")


def asan_runtime() -> str:
    """Path of the compiler's AddressSanitizer runtime (preloaded into the
    uninstrumented Python that loads the sanitizer build)."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang++")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang++"
    out = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                         stdout=subprocess.PIPE, check=True).stdout.decode().strip()
    if not os.path.isabs(out) or not os.path.exists(out):
        raise RuntimeError("AddressSanitizer runtime not found")
    return out


def build_asan() -> str:
    """Host-sanitized variant of the library: the host runtime (argument
    checks, planning, allocation, launch set-up) compiled with
    AddressSanitizer and UndefinedBehaviorSanitizer, linked with the ordinary
    kernel objects.  The sanitizers apply to host code only; it is meant for
    CPU runs of the host-side tests (TILEQ_LIB_PATH=<this library>, the
    runtime of asan_runtime() preloaded)."""
    if not all(os.path.exists(os.path.join(BUILD, n + ".o")) for _, n, _ in SOURCES):
        build()
    os.makedirs(ASAN_DIR, exist_ok=True)
    cc = hipcc()
    obj = os.path.join(ASAN_DIR, "tileq_host.o")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-g"]
    cmd = [cc] + flags() + san + ["-x", "hip", "-c", os.path.join(CSRC, "tileq_host.cpp"), "-o", obj]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        raise RuntimeError("hipcc (sanitized host) failed:\n" + r.stdout.decode(errors="replace"))
    objs = [obj] + [os.path.join(BUILD, n + ".o") for _, n, _ in SOURCES if n != "tileq_host"]
    tmp = ASAN_LIB + ".tmp"
    r = subprocess.run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs,
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout.decode(errors="replace"))
    os.replace(tmp, ASAN_LIB)
    return ASAN_LIB


if __name__ == "__main__":
    if "--asan" in sys.argv:
        print(build_asan())
    else:
        print(build(verbose="-v" in sys.argv))
