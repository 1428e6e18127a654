"""Build liboracle_hclrmix.so, the CPU oracle (test infrastructure only)."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))


def build(verbose: bool = False) -> str:
    out = os.path.join(HERE, "libhclrmix_oracle.so")
    tmp = out + ".tmp"
    # -ffp-contract=off: no fused multiply-add, every product and sum rounds to fp32
    # separately, as the pages' composition of standard operators does.
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
           "-fno-fast-math", "-fno-finite-math-only",
           os.path.join(HERE, "hclrmix_oracle.c"), "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
