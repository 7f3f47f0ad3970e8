"""Builds libgdn.so in-tree with hipcc for gfx950.

    python -m gated_deltanet_recurrence_conv_amd.build

Every HIP source under csrc/ is compiled and linked into one shared library
next to this file; the ceiling loops under ceiling/ (measurement
infrastructure, not the path) go into a second one, libgdn_ceiling.so.  Packed-fp32 VALU instructions are disabled on the device
(-packed-fp32-ops off); hipcc's host pass warns that it does not know that
feature, which is harmless.  MFMA accumulators are kept in ordinary VGPRs
where possible (-amdgpu-mfma-vgpr-form), so the fp32 state that the prefill
scan updates with both VALU and MFMA is not copied between register files.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgdn.so")
CEILING_SRC = os.path.join(HERE, "ceiling")
CEILING_LIB = os.path.join(HERE, "libgdn_ceiling.so")
ARCH = "gfx950"


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build libgdn.so")
    return path


FLAGS = ["--offload-arch=" + ARCH, "-mcode-object-version=5", "-O3", "-std=c++17", "-fPIC",
         "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form"]
OBJDIR = os.path.join(HERE, "_build")


def _run(cmd, verbose: bool) -> str:
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in proc.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed (%d):\n%s" % (proc.returncode, out))
    return out


def _link(srcs, lib, incs, verbose: bool) -> str:
    """Compiles each source to an object (in parallel), then links them."""
    import concurrent.futures as cf
    os.makedirs(OBJDIR, exist_ok=True)
    inc_flags = []
    for inc in incs:
        inc_flags += ["-I", inc]
    objs = [os.path.join(OBJDIR, os.path.splitext(os.path.basename(s))[0] + ".o") for s in srcs]
    jobs = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        outs = list(ex.map(lambda so: _run([hipcc()] + FLAGS + inc_flags + ["-c", so[0], "-o", so[1]],
                                            verbose), zip(srcs, objs)))
    tmp = lib + ".tmp%d" % os.getpid()
    try:
        outs.append(_run([hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs, verbose))
    except RuntimeError:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise
    for out in outs:
        if out.strip() and verbose:
            print(out)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    """Builds libgdn.so and libgdn_ceiling.so; returns the path of libgdn.so."""
    inc = os.path.join(ROOT, "include")
    _link(sorted(glob.glob(os.path.join(CSRC, "*.hip"))), LIB, [inc, CSRC], verbose)
    _link(sorted(glob.glob(os.path.join(CEILING_SRC, "*.hip"))), CEILING_LIB, [inc], verbose)
    return LIB


def build_host_sanitized(lib: str, verbose: bool = False) -> str:
    """libgdn.so with the host code of the C ABI (gdn_api.hip: argument
    validation, status codes, launch geometry) built with AddressSanitizer and
    UndefinedBehaviorSanitizer; device code and the other sources as in
    build().  Each -fsanitize= applies to the host pass only (-Xarch_host).
    The process that loads it must preload the clang sanitizer runtime."""
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(OBJDIR, os.path.splitext(os.path.basename(s))[0] + ".o") for s in srcs]
    if not all(os.path.exists(o) for o in objs):
        build(verbose)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    api = os.path.join(CSRC, "gdn_api.hip")
    api_obj = lib + ".api.o"
    _run([hipcc()] + FLAGS + inc + ["-g", "-fno-omit-frame-pointer",
                                    "-Xarch_host", "-fsanitize=address",
                                    "-Xarch_host", "-fsanitize=undefined",
                                    "-Xarch_host", "-fno-sanitize-recover=all",
                                    "-c", api, "-o", api_obj], verbose)
    others = [o for s, o in zip(srcs, objs) if s != api]
    _run([hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", lib, api_obj] + others, verbose)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
