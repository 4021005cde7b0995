"""Build the CPU oracle (plain C, gcc) into oracle/libkvq_oracle.so.

Test infrastructure: the oracle is compiled here and loaded only by the test
suite, the package smoke check and the benchmark's CPU-baseline leg.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kvq_oracle.c")
LIB = os.path.join(HERE, "libkvq_oracle.so")

# -ffp-contract=off: no fused multiply-add, so every float operation rounds
# exactly once as written; no -ffast-math; IEEE binary32 on x86-64 SSE.
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
          "-fPIC", "-shared", "-pthread", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile the oracle; returns the path of the shared library."""
    if not force and os.path.exists(LIB) and \
            os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp"
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, SRC, "-lm"], check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
