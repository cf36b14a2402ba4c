"""Build libds4moe.so (HIP, gfx950) in-tree."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]


def build(extra=()):
    out = os.path.join(HERE, "libds4moe.so")
    cmd = [HIPCC] + FLAGS + list(extra) + ["-o", out, os.path.join(HERE, "csrc", "ds4moe_api.hip")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("libds4moe build failed:\n%s\n%s" % (r.stdout, r.stderr[-8000:]))
    return r.stderr


if __name__ == "__main__":
    print(build())
