"""Build the fp64 CPU oracle (plain C, gcc, OpenMP).  Test infrastructure only."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "kda_oracle.c")


def library_path() -> str:
    return os.path.join(HERE, "libkda_oracle.so")


def build_oracle(source: str = SOURCE, output: str | None = None, extra=()) -> str:
    """Compile ``source`` into a shared library (``-O2``, no fast-math)."""
    output = output or library_path()
    tmp = output + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra",
           "-o", tmp, source, "-lm", *extra]
    subprocess.run(cmd, check=True)
    os.replace(tmp, output)
    return output


if __name__ == "__main__":
    print(build_oracle(*sys.argv[1:2]))
