"""Build step for the fp64 CPU oracle (test infrastructure only).

Compiles ``oracle.c`` into ``liboracle.so`` next to this file with the system C compiler.
Plain -O2, no target-specific flags, so the library built in one container runs on another
x86-64 host.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(src: str = SRC, out: str = LIB, extra_flags=()) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-Wall", "-Wextra",
           *extra_flags, src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    print(build())
    sys.exit(0)
