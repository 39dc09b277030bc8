"""Build libnvfp4.so (gfx950) in-tree with hipcc.

Usage: python -m precision_moe_gemm_amd.build
"""
from __future__ import annotations

import hashlib
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "libnvfp4.hip")
LIB = os.path.join(HERE, "libnvfp4.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # bit-exact quantization: no fused multiply-add contraction
    "-ffp-contract=off",
    # keep the compiler from forming packed fp32 ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def source_hash() -> str:
    """Hash of everything the library is built from (its sources, the public
    header and the compiler flags): stamped into the library at build time
    and compared by the loader, so a stale binary is never used."""
    h = hashlib.sha256()
    files = []
    for d in (os.path.join(HERE, "csrc"), os.path.join(ROOT, "include")):
        files += [os.path.join(d, f) for f in sorted(os.listdir(d)) if f.endswith((".h", ".hip"))]
    for f in files:
        h.update(os.path.relpath(f, ROOT).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    h.update(" ".join(HIPCC_FLAGS).encode())
    return h.hexdigest()[:16]


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return p


# The host layer (argument checks, workspace layout, dispatch) built with
# AddressSanitizer and UndefinedBehaviorSanitizer on the host side only; the
# device code is the same.  Loaded by the CPU tests through NVFP4_LIB_PATH
# with the sanitizer runtime preloaded.
SAN_DIR = os.path.join(ROOT, "_build", "sanitize")
SAN_LIB = os.path.join(SAN_DIR, "libnvfp4.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-shared-libasan", "-g"]


def _cmd(out: str, extra=()) -> list:
    stamp = source_hash()
    return [hipcc(), *HIPCC_FLAGS, *extra, f"-DNVFP4_BUILD_STAMP=\"{stamp}\"", "-I", os.path.join(ROOT, "include"),
            "-o", out, SRC]


def sanitizer_runtime() -> str:
    """The clang AddressSanitizer runtime that the sanitized library needs
    preloaded (it also carries the UndefinedBehaviorSanitizer handlers)."""
    out = subprocess.run([hipcc(), "--print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                         text=True).stdout.strip()
    if os.path.isabs(out) and os.path.exists(out):
        return out
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("clang AddressSanitizer runtime not found")
    return hits[-1]


def start_sanitized_build():
    """Start the sanitizer build in the background (a Popen); None when the
    library there already carries the current source stamp."""
    if sanitized_is_current():
        return None
    os.makedirs(SAN_DIR, exist_ok=True)
    tmp = SAN_LIB + ".tmp%d" % os.getpid()
    stamp = source_hash()  # the sources as they are when the compiler reads them
    proc = subprocess.Popen(_cmd(tmp, SAN_FLAGS), stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
    proc.nvfp4_tmp = tmp
    proc.nvfp4_stamp = stamp
    return proc


def finish_sanitized_build(proc) -> str:
    if proc is not None:
        _, err = proc.communicate()
        if proc.returncode != 0:
            if os.path.exists(proc.nvfp4_tmp):
                os.remove(proc.nvfp4_tmp)
            err = "\n".join(l for l in err.splitlines() if "packed-fp32-ops" not in l)
            raise RuntimeError("sanitizer build failed:\n" + err)
        os.replace(proc.nvfp4_tmp, SAN_LIB)
        with open(SAN_LIB + ".stamp", "w") as f:
            f.write(proc.nvfp4_stamp)
    return SAN_LIB


def sanitized_is_current() -> bool:
    stamp_file = SAN_LIB + ".stamp"
    try:
        with open(stamp_file) as f:
            return f.read().strip() == source_hash() and os.path.exists(SAN_LIB)
    except OSError:
        return False


def build_sanitized() -> str:
    """The sanitizer build of the current sources (rebuilt only when stale)."""
    return finish_sanitized_build(start_sanitized_build())


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = _cmd(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("hipcc failed:\n" + err)
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


# The HBM read probe that bench.py times beside the kernels (the achievable
# read rate of the streaming GEMM's access patterns); not part of libnvfp4.
PROBE_SRC = os.path.join(HERE, "csrc", "probe", "hbm_read.hip")
PROBE_LIB = os.path.join(HERE, "libhbmprobe.so")


def start_probe_build():
    tmp = PROBE_LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, "-o", tmp, PROBE_SRC]
    proc = subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
    proc.nvfp4_tmp = tmp
    return proc


def finish_probe_build(proc) -> str:
    _, err = proc.communicate()
    if proc.returncode != 0:
        if os.path.exists(proc.nvfp4_tmp):
            os.remove(proc.nvfp4_tmp)
        err = "\n".join(l for l in err.splitlines() if "packed-fp32-ops" not in l)
        raise RuntimeError("probe build failed:\n" + err)
    os.replace(proc.nvfp4_tmp, PROBE_LIB)
    return PROBE_LIB


def build_all(verbose: bool = False) -> str:
    """The library and, concurrently, its sanitizer build (when stale) and
    the read probe."""
    proc = start_sanitized_build()
    probe = start_probe_build()
    try:
        lib = build(verbose)
    finally:
        finish_sanitized_build(proc)
        finish_probe_build(probe)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
