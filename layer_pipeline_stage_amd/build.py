"""Build liblps.so (the C-ABI library with the gfx950 kernels) in-tree with hipcc.

    python -m layer_pipeline_stage_amd.build [--jobs N]
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "liblps.so")
BUILD = os.path.join(PKG, "_build")
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build liblps)")


FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed FP32 instructions stay off: the compiler may not form v_pk_* f32 ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-result",
]


# Host-only sanitizers (AddressSanitizer + UndefinedBehaviorSanitizer) for the
# library's CPU paths: each -fsanitize= applies to the host pass alone; the device
# code is built as usual.  The result is loaded with the ASan runtime preloaded.
SAN_FLAGS = [
    "-O1", "-g", "-fno-omit-frame-pointer", "-shared-libsan",
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
]
SAN_BUILD = os.path.join(PKG, "_build_san")
SAN_OUT = os.path.join(SAN_BUILD, "liblps_san.so")


def asan_runtime() -> str:
    """The clang ASan runtime that a sanitized liblps needs preloaded."""
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("the clang ASan runtime is not installed under /opt/rocm/llvm")
    return hits[-1]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def build(jobs: int | None = None, verbose: bool = False, sanitize: bool = False) -> str:
    out_dir, out = (SAN_BUILD, SAN_OUT) if sanitize else (BUILD, OUT)
    os.makedirs(out_dir, exist_ok=True)
    cc = hipcc()
    srcs = sources()
    flags = [f for f in FLAGS if f != "-O3"] + SAN_FLAGS if sanitize else FLAGS

    def compile_one(src):
        obj = os.path.join(out_dir, os.path.basename(src) + ".o")
        cmd = [cc, *flags, "-c", src, "-o", obj]
        if src.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                        if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{msg}")
        if verbose and msg.strip():
            print(msg, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(jobs or min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = out + ".tmp"
    link = [cc, "-shared", f"--offload-arch={ARCH}"]
    if sanitize:
        link += ["-shared-libsan", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    r = subprocess.run([*link, "-o", tmp, *objs], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("-v", "--verbose", action="store_true")
    ap.add_argument("--sanitize", action="store_true",
                    help="build _build_san/liblps_san.so with host ASan + UBSan")
    a = ap.parse_args()
    print(build(a.jobs, a.verbose, a.sanitize))
