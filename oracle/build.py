"""Build the CPU oracle (plain C, gcc) into oracle/libmoe_oracle.so.

Test infrastructure: the library is loaded only by the tests, the smoke
check and the CPU-baseline leg of the benchmark.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
LIB = os.path.join(HERE, "libmoe_oracle.so")

# -ffp-contract=off and no fast-math: every fp64/fp32 operation rounds exactly
# as written in the source.
CFLAGS = ["-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off", "-fno-fast-math",
          "-fopenmp", "-fPIC", "-shared"]


def build(extra_flags=None, out=LIB):
    cmd = ["gcc", *CFLAGS, *(extra_flags or []), SRC, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True, cwd=HERE)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build())
