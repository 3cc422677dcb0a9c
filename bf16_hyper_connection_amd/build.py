"""Build libhcr.so (the HIP kernels and the C ABI) in-tree for gfx950 with hipcc."""

import hashlib
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libhcr.so")

SOURCES = ["hcr_kernels.hip", "hcr_matvec.hip", "hcr_api.cpp"]
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed FP32 instructions in device code (the host pass ignores the feature)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def source_hash():
    """sha256 over the library's sources (csrc/ and include/hcr.h); measurements taken with
    hardware counters are valid only for the sources they were taken on."""
    h = hashlib.sha256()
    files = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".h", ".cpp")))
    for name in files:
        with open(os.path.join(CSRC, name), "rb") as fh:
            h.update(name.encode() + b"\0" + fh.read())
    with open(os.path.join(ROOT, "include", "hcr.h"), "rb") as fh:
        h.update(b"hcr.h\0" + fh.read())
    return h.hexdigest()


def hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def build(verbose=False):
    """Compile every source into libhcr.so (always recompiles); returns the library path."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + HIPCC_FLAGS + ["-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", tmp] + \
          [os.path.join(CSRC, s) for s in SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in line)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + out)
    if verbose and out.strip():
        print(out, flush=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
