"""Build libbifocal.so (HIP for gfx950) in-tree, next to the Python binding.

    python -m rope_context_extension_bifocal_amd.csrc.build          (libbifocal.so)
    python -m rope_context_extension_bifocal_amd.csrc.build --asan   (libbifocal_asan.so)

Every HIP source is compiled with packed fp32 arithmetic disabled (the host
pass warns that it does not know the feature; that is harmless) and without
IEEE NaN quieting in min/max (no kernel relies on NaN propagation; masked
scores use -inf, which is still honoured).

--asan builds the host code (argument validation, schedules, launch set-up)
with AddressSanitizer into libbifocal_asan.so, for CPU-side test runs with the
ASan runtime preloaded (load it by setting BIFOCAL_LIB to its path); the GPU
code is built as usual.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libbifocal.so")
LIB_ASAN = os.path.join(PKG, "libbifocal_asan.so")
SOURCES = ["capi.cpp", "prefill.hip", "decode.hip", "rope.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose=False, asan=False):
    out = LIB_ASAN if asan else LIB
    host_san = (["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]
                if asan else [])
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-mno-amdgpu-ieee", "-fno-honor-nans",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", HERE] + host_san + [
           "-o", out + ".tmp"] + [os.path.join(HERE, s) for s in SOURCES]
    res = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        sys.stderr.write(msg + "\n")
        raise RuntimeError("hipcc failed building " + os.path.basename(out))
    if verbose and msg.strip():
        sys.stderr.write(msg + "\n")
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True, asan="--asan" in sys.argv[1:]))
