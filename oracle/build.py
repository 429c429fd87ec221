"""Build the CPU oracle library (test infrastructure only).

`build()` compiles ``kvq_oracle.c`` with gcc into ``liboracle.so`` next to it.
`build(plant=n)` compiles a copy with planted mistake n into a scratch path;
the tests use those copies to show that the oracle's pins catch mistakes.
"""
import os
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kvq_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-Wall", "-ffp-contract=off", "-fno-fast-math",
          "-fopenmp", "-shared", "-fPIC"]


def build(plant=0, out=None):
    """Compile the oracle; returns the path of the shared library."""
    if out is None:
        out = LIB if plant == 0 else os.path.join(
            tempfile.gettempdir(), f"kvq_oracle_plant{plant}_{os.getpid()}.so")
    tmp = out + ".tmp"
    cmd = ["gcc", *CFLAGS, f"-DORA_PLANT={int(plant)}", "-o", tmp, SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def ensure_built():
    """Build the oracle only if no library exists yet."""
    if not os.path.exists(LIB):
        build()
    return LIB


if __name__ == "__main__":
    print(build())
