"""Compile the lutq HIP library (liblutq.so) for gfx950, in-tree.

Usage: ``python -m weight_only_lut_amd.build`` or ``build()`` from Python.
Always recompiles; writes ``weight_only_lut_amd/liblutq.so`` atomically.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
# (source, extra flags): the matmul is compiled once per code width
SOURCES = [("lutq_api.cpp", []), ("lutq_layout.hip", []), ("lutq_quantize.hip", []),
           ("lutq_static.hip", []), ("lutq_peaks.hip", []),
           ("lutq_matmul.hip", ["-DLUTQ_MATMUL_BITS=2"]), ("lutq_matmul.hip", ["-DLUTQ_MATMUL_BITS=3"]),
           ("lutq_matmul.hip", ["-DLUTQ_MATMUL_BITS=4"])]
LIB = os.path.join(HERE, "liblutq.so")
# The same library with AddressSanitizer and UndefinedBehaviorSanitizer in
# its host code only (argument validation, planning, scratch management);
# device code is compiled exactly as in LIB. Loaded by the host-sanitizer
# test in place of LIB, with the clang ASan runtime preloaded.
SAN_LIB = os.path.join(HERE, "liblutq_san.so")
ARCH = "gfx950"
# each -fsanitize= applies to the host pass only (-Xarch_host right before it)
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-shared-libasan", "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # no packed-FP32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build liblutq.so)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops"  # host pass does not know the device-only feature
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    return res.returncode, msgs


def build(verbose: bool = False, sanitized: bool = True) -> str:
    """Compile every source to an object (in parallel), then link liblutq.so
    and, with `sanitized`, liblutq_san.so (host code under ASan + UBSan)."""
    import tempfile
    from concurrent.futures import ThreadPoolExecutor
    cc = hipcc()
    inc = ["-I", os.path.join(ROOT, "include")]
    variants = [(LIB, [])] + ([(SAN_LIB, SAN_FLAGS)] if sanitized else [])
    with tempfile.TemporaryDirectory(prefix="lutq_build_") as tmpdir:
        jobs, objs = [], {lib: [] for lib, _ in variants}
        for v, (lib, vflags) in enumerate(variants):
            for i, (src, extra) in enumerate(SOURCES):
                obj = os.path.join(tmpdir, f"{v}_{i}_{os.path.splitext(src)[0]}.o")
                cflags = [f for f in FLAGS if f != "-shared"] + vflags
                jobs.append((obj, [cc, *cflags, *extra, *inc, "-c", "-o", obj, os.path.join(CSRC, src)]))
                objs[lib].append(obj)
        workers = max(1, min(len(jobs), os.cpu_count() or 1, 8))
        with ThreadPoolExecutor(max_workers=workers) as ex:
            results = list(ex.map(lambda j: _run(j[1], verbose), jobs))
        errors = [m for rc, m in results if rc != 0]
        if errors:
            raise RuntimeError("hipcc failed:\n" + "\n".join(ln for m in errors for ln in m))
        if verbose:
            for rc, m in results:
                if m:
                    print("\n".join(m))
        for lib, vflags in variants:
            tmp = lib + f".tmp{os.getpid()}"
            rc, msgs = _run([cc, *FLAGS, *vflags, "-o", tmp, *objs[lib]], verbose)
            if rc != 0:
                if os.path.exists(tmp):
                    os.remove(tmp)
                raise RuntimeError("hipcc link failed:\n" + "\n".join(msgs))
            os.replace(tmp, lib)
    return LIB


def asan_runtime() -> str | None:
    """The clang AddressSanitizer runtime that liblutq_san.so links against."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang")
    for cand in (clang, shutil.which("clang"), "/opt/rocm/llvm/bin/clang"):
        if not cand or not os.path.exists(cand):
            continue
        res = subprocess.run([cand, "-print-resource-dir"], capture_output=True, text=True)
        path = os.path.join(res.stdout.strip(), "lib", "linux", "libclang_rt.asan-x86_64.so")
        if res.returncode == 0 and os.path.exists(path):
            return path
    return None


# Sources of the matmul device code: a stored kernel profile is current while
# their digest is unchanged (host-side planning lives in lutq_api.cpp; the
# profile also records the plan it was taken with).
KERNEL_SOURCES = ["lutq_device.h", "lutq_internal.h", "lutq_matmul.hip"]


# Sources of the quantizer's device code, likewise.
QUANT_SOURCES = ["lutq_device.h", "lutq_internal.h", "lutq_quant.h", "lutq_quantize.hip"]


def source_digest(names=None) -> str:
    """SHA-256 over kernel sources (to tell whether a stored profile is
    current): the matmul's by default, or the files named."""
    import hashlib
    h = hashlib.sha256()
    for name in names or KERNEL_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
