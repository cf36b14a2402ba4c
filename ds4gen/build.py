"""Build the synthetic-input generator libraries in-tree.

libds4gen.so      host generator (gcc)
libds4gen_dev.so  device block fill for gfx950 (hipcc)
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-ffp-contract=off",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd):
    r = subprocess.run(cmd, cwd=HERE, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))


def build(device=True):
    _run(["gcc", "-O2", "-fPIC", "-shared", "-std=c11", "-ffp-contract=off", "-Wall",
          "-o", "libds4gen.so", "ds4gen_host.c", "-lm"])
    if device:
        _run([HIPCC] + HIP_FLAGS + ["-o", "libds4gen_dev.so", "ds4gen_fill.hip"])


if __name__ == "__main__":
    build()
