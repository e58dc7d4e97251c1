"""Build the HIP library `libvspec_verify.so` in-tree for gfx950.

Run `python -m draft_token_verification_packed_amd.build` (or call build())
on any machine with ROCm's hipcc; no GPU is needed to compile.
"""
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(os.path.dirname(PKG), "include")
LIB = os.path.join(PKG, "libvspec_verify.so")
SOURCES = ["abi.cpp", "verify.hip", "confidence.hip"]
ARCH = "gfx950"
# Packed-FP32 VALU forms are kept out of the code objects: the compiler would
# otherwise fuse float pairs into v_pk_* instructions.
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=" + ARCH,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


def hipcc():
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found: ROCm is required to build the library")
    return p


def build(extra_flags=(), out=LIB, verbose=False):
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    cmd = [hipcc()] + FLAGS + list(extra_flags) + ["-I", CSRC, "-I", INCLUDE] + srcs + ["-o", out + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + msgs)
    if verbose and msgs.strip():
        print(msgs, file=sys.stderr)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
