"""Build the oracle's C part (liboz2_oracle.so) with gcc.

Test infrastructure only; called by __graft_entry__.build().  The flags keep
every floating-point operation separately rounded (-ffp-contract=off) so the
alpha/beta epilogue is evaluated exactly as written.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "oz2_oracle.c")
    out = os.path.join(HERE, "liboz2_oracle.so")
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", out + ".tmp", src, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True), file=sys.stderr)
