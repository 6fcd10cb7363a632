"""Builds the oracle's shared library (test infrastructure only).

The oracle is a plain C file compiled with gcc: -O2, no fast-math and no
floating-point contraction, OpenMP for row parallelism.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mk_oracle.c")
LIB = os.path.join(HERE, "libmk_oracle.so")


def build(verbose: bool = False, mutant: int = 0, out: str = None) -> str:
    """Compiles mk_oracle.c. mutant > 0 builds a planted-mistake variant (tests only)."""
    out = out or LIB
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-shared",
           "-fPIC", "-Wall", "-Wextra", f"-DMKO_MUTANT={int(mutant)}", "-o", out + ".tmp", SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
