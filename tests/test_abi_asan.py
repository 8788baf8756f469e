"""The C-ABI host layer under AddressSanitizer (CPU only).

twell_api.cpp -- argument validation, size queries, workspace layouts, status
strings -- is compiled with g++ -fsanitize=address and linked with the HIP
kernel objects of the normal build into a separate library; tests/test_abi.py
then runs against that library in a child process with the ASan runtime
preloaded.  None of those tests launches a kernel, so no GPU is needed; an
out-of-bounds or use-after-free access in the host layer aborts the child.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OBJS = sorted(glob.glob(os.path.join(ROOT, "_build", "libtwell", "csrc_*.hip.o")))
GXX = shutil.which("g++")

pytestmark = pytest.mark.skipif(GXX is None or not OBJS or not os.path.isdir("/opt/rocm/include"),
                                reason="needs g++, ROCm headers and the kernel objects of a normal build")


def _asan_library(out_dir):
    obj = os.path.join(out_dir, "twell_api_asan.o")
    lib = os.path.join(out_dir, "libtwell_asan.so")
    src = os.path.join(ROOT, "activation_sparse_feedforward_amd", "csrc", "twell_api.cpp")
    subprocess.run([GXX, "-std=c++17", "-O1", "-g", "-fsanitize=address", "-fno-omit-frame-pointer", "-fPIC",
                    "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", f"-I{ROOT}/include", "-c", src, "-o", obj],
                   check=True, capture_output=True, text=True)
    subprocess.run([GXX, "-shared", "-fsanitize=address", "-o", lib, obj, *OBJS, "-L/opt/rocm/lib", "-lamdhip64",
                    "-Wl,-rpath,/opt/rocm/lib"], check=True, capture_output=True, text=True)
    return lib


def test_abi_host_layer_under_asan(tmp_path):
    lib = _asan_library(str(tmp_path))
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report_load" in syms, "the host layer was not instrumented"
    asan_rt = subprocess.run([GXX, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    env = dict(os.environ, LD_PRELOAD=asan_rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    code = ("import sys; sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r});"
            "from activation_sparse_feedforward_amd import twell as T; T.LIB_PATH = {lib!r};"
            "import pytest; sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', '-m', 'not gpu', {t!r}]))"
            ).format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib,
                     t=os.path.join(ROOT, "tests", "test_abi.py"))
    r = subprocess.run([sys.executable, "-c", code], env=env, cwd=str(tmp_path), capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert " passed" in r.stdout
