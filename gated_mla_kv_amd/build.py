"""Build libgmla.so (the HIP kernels and the C ABI) in-tree for gfx950 with hipcc.

Every call recompiles all sources (objects in gated_mla_kv_amd/_build/, built in parallel) and
links gated_mla_kv_amd/libgmla.so atomically. It also links two variants from the same objects:
* libgmla_debug.so: kv_append, the top-k kernels and the C ABI built with GMLA_DEBUG_CHECKS, whose
  device-side bound checks record violations that mla_debug_flags reports;
* _build/asan/libgmla_asan.so (build_asan(), on request): the C ABI's host code built with
  AddressSanitizer (device code unchanged), for running the host-side validation under ASan.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgmla.so")

ARCH = os.environ.get("GMLA_ARCH", "gfx950")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops stay off: ordinary float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wno-unused-command-line-argument",
]
SOURCES = ["api.cpp", "gemm.hip", "norm_append.hip", "prefill_attn.hip", "prefill_attn_k3.hip",
           "decode_attn.hip",
           "decode_attn_k3.hip", "dsa_expanded.hip", "scores.hip"]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


DEBUG_SOURCES = ["api.cpp", "norm_append.hip", "dsa_expanded.hip"]  # the files with debug checks
DEBUG_LIB = os.path.join(PKG, "libgmla_debug.so")
ASAN_LIB = os.path.join(OUT_DIR, "asan", "libgmla_asan.so")


def _compile(src: str, verbose: bool, out_dir: str = OUT_DIR, extra: tuple = ()) -> str:
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs: list, out: str) -> str:
    tmp = out + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


def build(verbose: bool = False, jobs: int | None = None) -> str:
    dbg_dir = os.path.join(OUT_DIR, "debug")
    os.makedirs(dbg_dir, exist_ok=True)
    jobs = jobs or min(len(SOURCES) + len(DEBUG_SOURCES), os.cpu_count() or 4, 16)
    with cf.ThreadPoolExecutor(jobs) as ex:
        rel = [ex.submit(_compile, s, verbose) for s in SOURCES]
        dbg = {s: ex.submit(_compile, s, verbose, dbg_dir, ("-DGMLA_DEBUG_CHECKS",)) for s in DEBUG_SOURCES}
        objs = [f.result() for f in rel]
        dbg_objs = [dbg[s].result() if s in dbg else o for s, o in zip(SOURCES, objs)]
    _link(dbg_objs, DEBUG_LIB)
    return _link(objs, LIB)


def build_asan(verbose: bool = False) -> str:
    """libgmla_asan.so: the release objects with api.cpp's host code built with AddressSanitizer.
    A process that loads it needs the ASan runtime preloaded (asan_runtime())."""
    asan_dir = os.path.dirname(ASAN_LIB)
    os.makedirs(asan_dir, exist_ok=True)
    objs = [os.path.join(OUT_DIR, s + ".o") for s in SOURCES]
    if not all(os.path.exists(o) for o in objs):
        build(verbose)
    # -Xarch_host: only the host code is instrumented; the device code is the release code
    api = _compile("api.cpp", verbose, asan_dir,
                   ("-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"))
    return _link([api if o.endswith("api.cpp.o") else o for o in objs], ASAN_LIB)


def asan_runtime() -> str:
    """Path of the compiler's shared ASan runtime (to preload into a process using ASAN_LIB)."""
    r = subprocess.run([_hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the compiler's ASan runtime (libclang_rt.asan-x86_64.so) was not found")
    return path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
