"""Build the CPU oracle (test infrastructure) with gcc.

The oracle is plain C compiled without fast-math, so every sum runs in the
order the source gives.  ``build_oracle()`` writes ``liboracle.so`` next to
this file (fp64 arithmetic); ``build_oracle(fp32=True)`` writes
``liboracle_fp32.so``, the same source with the prefill and decode
definitions carried in fp32 (the plain fp32 CPU reference timed beside the
GPU); ``build_oracle(mutant=k, out_dir=...)`` builds a copy with planted
mistake number k, which the tests use to show that their pins catch it.
Extra compiler flags (e.g. sanitizers) go in ``extra``.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "gdla_oracle.c")
LIBRARY = os.path.join(HERE, "liboracle.so")
LIBRARY_FP32 = os.path.join(HERE, "liboracle_fp32.so")


def build_oracle(out_dir=None, mutant=0, quiet=True, fp32=False, extra=(), out=None):
    if out is None:
        if out_dir is not None:
            out = os.path.join(out_dir, "liboracle_mutant%d.so" % mutant)
        else:
            out = LIBRARY_FP32 if fp32 else LIBRARY
    cmd = ["gcc", "-std=c11", "-O3", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-Werror",
           "-DORACLE_MUTANT=%d" % mutant] + (["-DORACLE_FP32"] if fp32 else []) + list(extra) + [
           SOURCE, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True, capture_output=quiet)
    os.replace(out + ".tmp", out)
    return out


def build_all():
    """Both arithmetic builds; returns their paths."""
    return [build_oracle(), build_oracle(fp32=True)]


if __name__ == "__main__":
    print(build_all())
