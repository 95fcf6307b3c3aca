"""Builds tests/devmath/libdevmath.so (test support: the device math probe)
with the library's compile flags, in-tree, for gfx950."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
LIB = os.path.join(HERE, "libdevmath.so")


def build() -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    arch = os.environ.get("LA_OFFLOAD_ARCH", "gfx950")
    csrc = os.path.join(ROOT, "linear_attention_recurrent_amd", "csrc")
    cmd = [hipcc, "-shared", "-fPIC", "-O3", "-std=c++17", f"--offload-arch={arch}",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", csrc,
           "-o", LIB + ".tmp", os.path.join(HERE, "probe.hip")]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for the device math probe:\n" + r.stdout.decode())
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build())
