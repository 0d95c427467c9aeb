"""Compile the CPU oracle (plain C, gcc) into two shared libraries.

_moe_oracle_f32.so accumulates the FFN arithmetic in fp32, _moe_oracle_f64.so
in fp64. Both are test infrastructure (see moe_oracle.c).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
# No fast-math and no contraction: every multiply and add is the one written,
# and fmaf() is the only fused operation. -mavx2 -mfma lets gcc vectorise the
# independent per-element chains without changing any of them.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off", "-fno-math-errno",
          "-mavx2", "-mfma", "-Wall", "-Wextra", "-Wno-unused-parameter"]
VARIANTS = {"f32": "float", "f64": "double"}


def lib_path(variant: str) -> str:
    return os.path.join(HERE, f"_moe_oracle_{variant}.so")


def build(verbose: bool = False) -> None:
    for v, real in VARIANTS.items():
        out = lib_path(v)
        cmd = ["gcc", *CFLAGS, f"-DORACLE_REAL={real}", SRC, "-o", out + ".tmp", "-lm"]
        if verbose:
            print(" ".join(cmd))
        subprocess.run(cmd, check=True)
        os.replace(out + ".tmp", out)


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
