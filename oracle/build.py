"""Build the CPU oracle (test infrastructure) with gcc.

The oracle is plain C compiled without fast-math, so every sum runs in the
order the source gives.  ``build_oracle()`` writes ``liboracle.so`` next to
this file; ``build_oracle(mutant=k, out_dir=...)`` builds a copy with planted
mistake number k, which the tests use to show that their pins catch it.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "gdla_oracle.c")
LIBRARY = os.path.join(HERE, "liboracle.so")


def build_oracle(out_dir=None, mutant=0, quiet=True):
    out = LIBRARY if out_dir is None else os.path.join(out_dir, "liboracle_mutant%d.so" % mutant)
    cmd = ["gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-Werror",
           "-DORACLE_MUTANT=%d" % mutant, SOURCE, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True, capture_output=quiet)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build_oracle(quiet=False))
