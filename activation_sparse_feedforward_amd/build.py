"""Build libtwell.so (HIP kernels for gfx950 + the C ABI) in-tree.

    python -m activation_sparse_feedforward_amd.build

Every HIP source is compiled with hipcc for gfx950 only, with packed-fp32
instruction selection disabled (-packed-fp32-ops), then linked into
activation_sparse_feedforward_amd/libtwell.so; the measurement probes of
csrc/probe/ (used by bench.py only) go to libtwell_probe.so.  Always rebuilds.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build", "libtwell")
LIB = os.path.join(PKG, "libtwell.so")
# measurement probes (bench.py only; the library never calls them)
PROBE_DIR = os.path.join(CSRC, "probe")
PROBE_LIB = os.path.join(PKG, "libtwell_probe.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", f"-I{ROOT}/include"]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _sources():
    return sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str, folder: str = CSRC) -> str:
    obj = os.path.join(BUILD, os.path.basename(folder) + "_" + src + ".o")
    cmd = [HIPCC, *COMMON]
    if src.endswith(".hip"):
        cmd += ["-x", "hip", *DEVICE]
    cmd += ["-c", os.path.join(folder, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    srcs = _sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    shutil.move(tmp, LIB)
    probes = sorted(f for f in os.listdir(PROBE_DIR) if f.endswith(".hip"))
    pobjs = [_compile(f, PROBE_DIR) for f in probes]
    tmp = PROBE_LIB + ".tmp"
    r = subprocess.run([HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *pobjs], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed (probes)\n{r.stdout}\n{r.stderr}")
    shutil.move(tmp, PROBE_LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources and {PROBE_LIB} from {len(probes)}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
