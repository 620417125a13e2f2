"""Compile the C oracle (test infrastructure) with gcc into oracle/_build/.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg use
the result.  `-fno-fast-math` keeps IEEE double semantics; FMA contraction
cannot change results because every BF16*BF16 product is exact in double.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
BUILD = os.path.join(HERE, "_build")
SRC = os.path.join(HERE, "oracle.c")


def lib_path(mutant: int = 0) -> str:
    name = "liboracle.so" if mutant == 0 else f"liboracle_mutant{mutant}.so"
    return os.path.join(BUILD, name)


def build(mutant: int = 0, out: str | None = None) -> str:
    out = out or lib_path(mutant)
    os.makedirs(os.path.dirname(out), exist_ok=True)
    cmd = ["gcc", "-O2", "-fno-fast-math", "-std=c11", "-Wall", "-Wextra",
           "-shared", "-fPIC", "-pthread", f"-DORACLE_MUTANT={int(mutant)}",
           SRC, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(int(sys.argv[1]) if len(sys.argv) > 1 else 0))
