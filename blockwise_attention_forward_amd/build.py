"""Build libbwattn.so (HIP, gfx950) in-tree from csrc/*.hip with hipcc.

Usage: ``python -m blockwise_attention_forward_amd.build`` or ``build()``.
Every call recompiles every source.
"""

import concurrent.futures
import glob
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libbwattn.so")
PROBE_LIB = os.path.join(HERE, "libbwa_probe.so")  # measurement helper (matrix-core peak)
ARCH = os.environ.get("BWATTN_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-I" + os.path.join(ROOT, "include"),
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def _link(hipcc, srcs, objdir, lib, ex):
    objs = [os.path.join(objdir, os.path.basename(s) + ".o") for s in srcs]
    outs = list(ex.map(lambda so: _run([hipcc, *FLAGS, "-c", so[0], "-o", so[1]]), zip(srcs, objs)))
    tmp = lib + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, lib)
    return outs


def build(verbose=False):
    hipcc = _hipcc()
    srcs = sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))
    probe_srcs = sorted(glob.glob(os.path.join(HERE, "probe", "*.hip")))
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", "8")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        outs = _link(hipcc, srcs, objdir, LIB, ex)
        outs += _link(hipcc, probe_srcs, objdir, PROBE_LIB, ex)
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
