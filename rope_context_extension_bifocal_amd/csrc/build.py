"""Build libbifocal.so (HIP for gfx950) in-tree, next to the Python binding.

    python -m rope_context_extension_bifocal_amd.csrc.build

Every HIP source is compiled with packed fp32 arithmetic disabled (the host
pass warns that it does not know the feature; that is harmless) and without
IEEE NaN quieting in min/max (no kernel relies on NaN propagation; masked
scores use -inf, which is still honoured).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libbifocal.so")
SOURCES = ["capi.cpp", "prefill.hip", "decode.hip", "rope.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose=False):
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-mno-amdgpu-ieee", "-fno-honor-nans",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", HERE,
           "-o", LIB + ".tmp"] + [os.path.join(HERE, s) for s in SOURCES]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError("hipcc failed building libbifocal.so")
    if verbose and out.strip():
        sys.stderr.write(out + "\n")
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
