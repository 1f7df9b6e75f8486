"""Build the gfx950 HIP library in-tree: quantized_moe_weight_amd/libpqmoe.so.

Every ``csrc/*.hip`` file is compiled for gfx950 only, in parallel, and linked
into one shared library with a plain C ABI (include/pq.h).  Packed-fp32 VALU
instructions are disabled for the device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libpqmoe.so")
BUILD_DIR = os.path.join(ROOT, "_build", "pqmoe")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
COMMON = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build of the same
# sources (device code is compiled as usual, without sanitizers), for running
# the host validation and planning code under the sanitizers on a CPU machine.
SAN_DIR = os.path.join(ROOT, "_build", "san")
SAN_OUT = os.path.join(SAN_DIR, "libpqmoe_san.so")
SAN_FLAGS = ["-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]


def _compile(src: str, out_dir: str = BUILD_DIR, extra=()) -> str:
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    flags = [f for f in COMMON if f != "-O3"] if extra else COMMON
    cmd = [HIPCC, *flags, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False, sanitize: bool = False) -> str:
    out_dir, out = (SAN_DIR, SAN_OUT) if sanitize else (BUILD_DIR, OUT)
    extra = SAN_FLAGS if sanitize else ()
    os.makedirs(out_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4)), 16)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda f: _compile(f, out_dir, extra), srcs))
    tmp = out + ".tmp"
    link_extra = [f for f in extra if f.startswith("-fsanitize") or f == "-Xarch_host"][:4] if sanitize else []
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *link_extra, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out} from {len(srcs)} sources", file=sys.stderr)
    return out


def sanitizer_runtime() -> str:
    """Path of the AddressSanitizer runtime that a process must preload to load
    the sanitized library."""
    r = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        cands = glob.glob(os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "llvm", "lib", "clang", "*", "lib",
                                       "linux", "libclang_rt.asan-x86_64.so"))
        if not cands:
            raise RuntimeError("AddressSanitizer runtime not found")
        path = cands[0]
    return path


if __name__ == "__main__":
    build(verbose=True, sanitize="--sanitize" in sys.argv)
