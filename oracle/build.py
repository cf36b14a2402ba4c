"""Build the CPU oracle (test infrastructure) in-tree: liboracle.so (gcc)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def build():
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-std=gnu11", "-fopenmp", "-ffp-contract=off",
           "-Wall", "-o", "liboracle.so", "ds4_oracle.c", "ds4_encode.c", "-lquadmath", "-lm"]
    r = subprocess.run(cmd, cwd=HERE, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("oracle build failed:\n%s\n%s" % (r.stdout, r.stderr))


if __name__ == "__main__":
    build()
