"""Build libvstep.so (HIP, gfx950) in-tree from csrc/*.hip."""
import concurrent.futures
import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I" + os.path.join(ROOT, "include")]
LIB = os.path.join(HERE, "libvstep.so")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build failed: " + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    return r.stderr


def build(verbose=False, jobs=8):
    srcs = sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.basename(s)[:-4] + ".o") for s in srcs]
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        logs = list(ex.map(lambda so: _run([HIPCC] + FLAGS + ["-c", so[0], "-o", so[1]]), zip(srcs, objs)))
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs)
    os.replace(tmp, LIB)
    if verbose:
        for s, l in zip(srcs, logs):
            w = [x for x in l.splitlines() if "warning" in x and "packed-fp32-ops" not in x]
            if w:
                print(os.path.basename(s), "\n".join(w[:20]))
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
