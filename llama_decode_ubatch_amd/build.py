"""Build libubd.so (HIP kernels + host runtime + C ABI) for gfx950, in-tree.

    python -m llama_decode_ubatch_amd.build

Objects go to llama_decode_ubatch_amd/_build/, the library next to this
file.  Every HIP compile disables packed-FP32 instruction selection.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libubd.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC,
          "-Wall", "-Wno-unused-function"]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines()
                    if "packed-fp32-ops" not in l)   # host-pass notice only
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def compile_library(sources, out, extra=(), jobs=8):
    bdir = os.path.join(os.path.dirname(out), "_build")
    os.makedirs(bdir, exist_ok=True)
    objs = []
    cmds = []
    for src in sources:
        obj = os.path.join(bdir, os.path.basename(src) + ".o")
        objs.append(obj)
        cmds.append([HIPCC, *COMMON, *extra, "-c", src, "-o", obj])
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for log in ex.map(_run, cmds):
            if log.strip():
                print(log)
    tmp = out + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, out)
    return out


def build(verbose=True):
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".cpp", ".hip")))
    compile_library(srcs, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build()
    sys.exit(0)
