"""Build libgdla.so (the HIP kernels and the C ABI of include/gdla.h) for gfx950.

hipcc compiles every ``csrc/*.hip`` file for gfx950 only and links them into
one shared library next to this file.  Packed-fp32 instruction selection is
switched off for the device code.
"""
import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(HERE, "libgdla.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build_library(extra_flags=(), out=None, quiet=False):
    out = out or LIBRARY
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    cmd = [hipcc] + HIPCC_FLAGS + list(extra_flags) + sources() + ["-o", out + ".tmp"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    if not quiet:
        msg = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                        if "packed-fp32-ops" not in l)
        if msg.strip():
            print(msg)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build_library())
