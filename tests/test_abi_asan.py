"""The C ABI's host-side validation under AddressSanitizer (CPU only).

api.hip (argument checks, mask resolution, plans) is rebuilt with the host
pass instrumented, linked with the kernels' objects from the in-tree build,
and tests/test_abi.py runs against that library in a child process with the
sanitizer runtime preloaded.  Only host code is instrumented; nothing is
launched (every call in test_abi.py returns before a launch).
"""

import glob
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "blockwise_attention_forward_amd")
HIPCC = "/opt/rocm/bin/hipcc"
ASAN_RT = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))

DRIVER = r"""
import sys
sys.path.insert(0, {root!r})
import blockwise_attention_forward_amd as bw
bw.lib_path = {lib!r}
bw._lib = bw._load()
import pytest
sys.exit(pytest.main([{tests!r}, "-q", "-p", "no:cacheprovider", "-x"]))
"""


@pytest.mark.slow
def test_abi_validation_under_address_sanitizer():
    objs = [o for o in glob.glob(os.path.join(PKG, "_build", "*.hip.o")) if not o.endswith("api.hip.o")]
    if not (os.path.exists(HIPCC) and ASAN_RT and objs):
        pytest.skip("needs hipcc, the sanitizer runtime and an in-tree build")
    with tempfile.TemporaryDirectory() as d:
        api_o = os.path.join(d, "api.o")
        lib = os.path.join(d, "libbwattn_asan.so")
        flags = ["--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17", "-I" + os.path.join(ROOT, "include"),
                 "-fno-omit-frame-pointer", "-Xarch_host", "-fsanitize=address"]
        subprocess.run([HIPCC, *flags, "-c", os.path.join(PKG, "csrc", "api.hip"), "-o", api_o], check=True,
                       capture_output=True)
        subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                        api_o, *objs, "-o", lib], check=True, capture_output=True)
        env = dict(os.environ, LD_PRELOAD=ASAN_RT[-1], ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
        code = DRIVER.format(root=ROOT, lib=lib, tests=os.path.join(ROOT, "tests", "test_abi.py"))
        p = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, cwd=ROOT,
                           timeout=600)
        assert p.returncode == 0, p.stdout[-3000:] + p.stderr[-3000:]
        assert "AddressSanitizer" not in p.stderr
        assert " passed" in p.stdout
