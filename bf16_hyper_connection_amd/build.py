"""Build libhcr.so (the HIP kernels and the C ABI) in-tree for gfx950 with hipcc, and the plain C
caller of the ABI that the tests run (tests/c_caller/hcr_read_file, built with the host C compiler)."""

import hashlib
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libhcr.so")
C_CALLER_SRC = os.path.join(ROOT, "tests", "c_caller", "hcr_read_file.c")
C_CALLER = os.path.join(ROOT, "tests", "c_caller", "hcr_read_file")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
# C11 with every warning an error: include/hcr.h must stay plain C
C_FLAGS = ["-std=c11", "-O2", "-Wall", "-Wextra", "-Wpedantic", "-Werror",
           "-D__HIP_PLATFORM_AMD__"]  # selects the AMD half of the HIP runtime header

SOURCES = ["hcr_kernels.hip", "hcr_matvec.hip", "hcr_api.cpp"]
# the calibration kernels (include/hcr_calib.h): a library of their own, measurement only
CALIB_LIB = os.path.join(PKG, "libhcr_calib.so")
CALIB_SOURCES = ["hcr_calib.hip"]
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed FP32 instructions in device code (the host pass ignores the feature)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the first 16 dwords of each kernel's arguments arrive in SGPRs (gfx950 kernarg preloading), so a
    # kernel's first loads and its stores do not wait for scalar loads of the argument segment.  Measured on
    # MI355X (cold read, one process, alternating with a build without it, 3 rounds): 0.08 us less per read
    # on the mean over T = 1..8
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    # matrix-core results in VGPRs rather than accumulation registers, so that the Q8_0 up kernel's per-block
    # scaling reads them without a v_accvgpr_read each.  Measured on MI355X (bench.py --ab, one process,
    # alternating builds, 3-4 rounds): the Q8_0 read 0.04-0.09 us faster per read from T = 4, BF16 level
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
]


def _code_only(text):
    """C/C++ source without comments and with whitespace collapsed (string literals kept)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c == '"' or c == "'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            i = text.find("\n", i)
            i = n if i < 0 else i
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_hash():
    """sha256 over the code of libhcr.so's sources (its csrc/ files and headers, and include/hcr.h; not the
    calibration library's), comments and whitespace left out, and the compiler flags; measurements taken
    with hardware counters are valid only for the code they were taken on."""
    h = hashlib.sha256()
    files = sorted(f for f in os.listdir(CSRC)
                   if f.endswith((".hip", ".h", ".cpp")) and f not in CALIB_SOURCES)
    paths = [os.path.join(CSRC, f) for f in files] + [os.path.join(ROOT, "include", "hcr.h")]
    for path in paths:
        with open(path) as fh:
            h.update(os.path.basename(path).encode() + b"\0" + _code_only(fh.read()).encode() + b"\0")
    h.update(" ".join(HIPCC_FLAGS).encode())  # the code the compiler makes of them
    return h.hexdigest()


def hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def c_compiler():
    for cand in (os.environ.get("CC"), shutil.which("gcc"), shutil.which("cc")):
        if cand and shutil.which(cand):
            return cand
    raise RuntimeError("no host C compiler (gcc or cc): the C caller cannot be built")


def build_c_caller(verbose=False):
    """Compile the C caller against include/hcr.h and link it to the built libhcr.so and the HIP
    runtime; returns its path."""
    tmp = C_CALLER + ".tmp%d" % os.getpid()
    cmd = [c_compiler()] + C_FLAGS + ["-I", os.path.join(ROOT, "include"), "-isystem", os.path.join(ROCM, "include"),
           C_CALLER_SRC, "-o", tmp, "-L", PKG, "-lhcr", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath," + os.path.relpath(PKG, os.path.dirname(C_CALLER)).join(["$ORIGIN/", ""]),
           "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("the C caller did not compile:\n" + res.stdout + res.stderr)
    os.replace(tmp, C_CALLER)
    return C_CALLER


def _hipcc_shared(path, sources, verbose):
    tmp = path + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + HIPCC_FLAGS + ["-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", tmp] + \
          [os.path.join(CSRC, s) for s in sources]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in line)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + out)
    if verbose and out.strip():
        print(out, flush=True)
    os.replace(tmp, path)


def build(verbose=False):
    """Compile every source into libhcr.so and the calibration kernels into libhcr_calib.so, then the
    C caller (always recompiles); returns the library path."""
    _hipcc_shared(LIB, SOURCES, verbose)
    _hipcc_shared(CALIB_LIB, CALIB_SOURCES, verbose)
    build_c_caller(verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
