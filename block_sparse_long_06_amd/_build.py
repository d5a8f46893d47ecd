"""Build libmsa.so (HIP, gfx950) in-tree.

All HIP code is compiled with packed-fp32 instructions disabled
(-Xclang -target-feature -Xclang -packed-fp32-ops); hipcc's host pass warns that it
does not know the feature, which is harmless.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmsa.so")
ARCH = os.environ.get("MSA_OFFLOAD_ARCH", "gfx950")

HIPFLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # matrix-core accumulators in ordinary VGPRs: the epilogues read every element
            "-mllvm", "-amdgpu-mfma-vgpr-form=true",
            "-Wall", "-Wno-unused-function", "-I" + os.path.join(ROOT, "include")]


# backward.hip keeps its matrix-core accumulators in AGPRs: the attention backward holds
# ~180 of them (dK, dV, S, dP, dQ), and in the VGPR form they crowd out the registers its
# LDS operand reads need (measured: 2 % faster this way)
AGPR_ACCUMULATORS = {"backward.hip"}


def flags_for(src: str) -> list:
    if os.path.basename(src) not in AGPR_ACCUMULATORS:
        return list(HIPFLAGS)
    f = list(HIPFLAGS)
    i = f.index("-amdgpu-mfma-vgpr-form=true")
    del f[i - 1:i + 1]
    return f


# The host-sanitizer variant (libmsa_san.so): AddressSanitizer and UndefinedBehaviorSanitizer
# on the HOST code only (argument validation, workspace layouts, launch set-up); the device
# code is built as usual.  It loads only into a process that preloads clang's ASan runtime
# (tests/test_sanitizers.py runs the CPU suite that way).
SAN_HOST_FLAGS = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined".split() + [
    "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]
LIB_SAN = os.path.join(HERE, "libmsa_san.so")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, jobs: int = 8, sanitize: bool = False) -> str:
    """Compile every csrc/*.hip to an object (in parallel) and link libmsa.so (with
    sanitize=True: the host-sanitizer variant libmsa_san.so)."""
    objdir = os.path.join(HERE, "_build", "san") if sanitize else os.path.join(HERE, "_build")
    lib = LIB_SAN if sanitize else LIB
    os.makedirs(objdir, exist_ok=True)
    procs = []
    objs = []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = ["hipcc", *flags_for(src), *(SAN_HOST_FLAGS if sanitize else []), "-c", src, "-o", obj]
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len(procs) >= jobs:
            _drain(procs, verbose)
    _drain(procs, verbose)
    tmp = lib + ".tmp%d" % os.getpid()
    subprocess.run(["hipcc", "-shared", "--offload-arch=" + ARCH, *objs, "-o", tmp], check=True)
    missing = undefined_kernel_stubs(tmp)
    if missing:
        os.remove(tmp)
        raise RuntimeError("libmsa links kernels whose host launch stubs were not emitted (a kernel body the "
                           "host pass rejected?): " + ", ".join(missing[:4]))
    os.replace(tmp, lib)
    return lib


def undefined_kernel_stubs(lib: str) -> list:
    """Kernel launch stubs the shared library references but does not define.  The host
    pass of hipcc drops a template kernel's stub without an error when the instantiated
    body uses device-only builtins inside host-device code (a lambda), and a shared library
    links with the reference unresolved, so only loading it would fail."""
    try:
        out = subprocess.run(["nm", "-D", "--undefined-only", lib], check=True, capture_output=True, text=True).stdout
    except (OSError, subprocess.CalledProcessError):
        return []  # no nm: nothing to check with
    return [line.split()[-1] for line in out.splitlines() if "__device_stub__" in line]


def _drain(procs, verbose):
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed.append((src, text))
        elif verbose and text.strip():
            print(text, file=sys.stderr)
    procs.clear()
    if failed:
        for src, text in failed:
            print("=== %s\n%s" % (src, text), file=sys.stderr)
        raise RuntimeError("hipcc failed for: " + ", ".join(os.path.basename(s) for s, _ in failed))


if __name__ == "__main__":
    print(build(verbose=True))
