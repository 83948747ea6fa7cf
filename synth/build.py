"""Build the seeded-input libraries: libsynth.so (host, gcc + OpenMP) and
libsynth_dev.so (HIP, gfx950)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build failed: " + " ".join(cmd) + "\n" + r.stdout + r.stderr)


def build(verbose=False):
    out = os.path.join(HERE, "libsynth.so")
    _run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", os.path.join(HERE, "synth.c"), "-o", out, "-lm"])
    out_dev = os.path.join(HERE, "libsynth_dev.so")
    _run([HIPCC] + HIP_FLAGS + [os.path.join(HERE, "synth_dev.hip"), "-o", out_dev])
    if verbose:
        print("built", out, out_dev)


if __name__ == "__main__":
    build(verbose=True)
