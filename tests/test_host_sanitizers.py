"""The C-ABI layer (argument validation, layouts, workspace plans, kernel-timing
records) built for the host alone with AddressSanitizer and
UndefinedBehaviorSanitizer, kernel launchers replaced by stand-ins
(tests/host_stubs.cpp), and the ABI tests run against it in a child process.
Any out-of-bounds access, use after free or undefined behaviour in the host
code those tests reach aborts the child."""
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "video_model_kv_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _runtime(name: str) -> str:
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else ""


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(os.path.join(ROCM, "include", "hip")),
                    reason="needs g++ and the HIP headers")
def test_abi_layer_under_address_and_ub_sanitizers():
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("sanitizer runtimes not found")
    with tempfile.TemporaryDirectory() as tmp:
        lib = os.path.join(tmp, "libqkv.so")
        srcs = [os.path.join(CSRC, f) for f in ("qkv_host.cpp", "timing.cpp")]
        srcs.append(os.path.join(ROOT, "tests", "host_stubs.cpp"))
        subprocess.run(["g++", "-std=c++17", "-g", "-O1", "-fPIC", "-shared", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
                        "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), "-I", CSRC, *srcs,
                        "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lpthread", "-o", lib], check=True)
        env = dict(os.environ, QKV_LIB_PATH=lib, LD_PRELOAD=f"{asan} {ubsan}", ASAN_OPTIONS="detect_leaks=0",
                   UBSAN_OPTIONS="print_stacktrace=1")
        check = ("import video_model_kv_amd._binding as B; import sys; "
                 f"assert B.LIB_PATH == {lib!r}; B.lib(); print('sanitized build loaded')")
        r = subprocess.run([sys.executable, "-c", check], cwd=ROOT, env=env, capture_output=True, text=True,
                           timeout=300)
        assert r.returncode == 0, r.stdout + r.stderr
        r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                            "tests/test_abi.py", "tests/test_zz_no_alloc.py"],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
        print(r.stdout[-2000:])
        assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
        assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
