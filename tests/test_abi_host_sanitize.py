"""CPU: the C-ABI layer (abi.cpp and the block manager's host layout code)
built with g++ under AddressSanitizer and UndefinedBehaviorSanitizer, linked
against a stub of the HIP calls it makes and of the kernel launchers
(tests/host_abi/hip_host_stub.cpp), and driven through every entry point
(tests/host_abi/abi_host_test.cpp): shapes swept for every decode form, cache
write, prefill, local attention, the block manager and the page read, plus
invalid arguments.  Each stub launcher writes or reads every byte its kernel
may touch per the parameters it was given, so a workspace or an extent
computed wrongly on the host is a sanitizer error here."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_183_amd", "csrc")
HOST = os.path.join(ROOT, "tests", "host_abi")
ROCM_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INCLUDE),
                    reason="needs g++ and the ROCm headers")
def test_abi_layer_under_asan_ubsan():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "abi_host_test")
        cmd = ["g++", "-O1", "-g", "-std=c++20", "-fsanitize=address,undefined",
               "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
               "-D__HIP_PLATFORM_AMD__",
               # the two HIP-language spellings abi.cpp uses, outside HIP mode
               "-D__align__(n)=__attribute__((aligned(n)))", "-DHIP_SYMBOL(x)=x",
               "-I", ROCM_INCLUDE, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
               os.path.join(CSRC, "abi.cpp"), os.path.join(CSRC, "block_manager_layout.cpp"),
               os.path.join(HOST, "hip_host_stub.cpp"), os.path.join(HOST, "abi_host_test.cpp"),
               "-o", exe]
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
        assert r.returncode == 0, r.stderr[-4000:]
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
        out = r.stdout + r.stderr
        assert r.returncode == 0, out[-4000:]
        assert "Sanitizer" not in out and "runtime error" not in out, out[-4000:]
        assert " 0 ABI check failures, 0 launch check failures" in out
