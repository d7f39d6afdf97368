"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two sanitized builds are made with gcc/g++ in a temporary directory:
  * the fp64 oracle (oracle/ssd_oracle.c), and
  * the C ABI's host side (api.cpp + shapes.cpp, with the kernel launchers
    replaced by stubs that never launch: tests/sanitize/abi_stubs.cpp).
The oracle pins (test_oracle.py) and the ABI validation tests (test_abi.py)
then run again in a child interpreter that loads those builds (SSD_ORACLE_LIB,
SSD_LIB) with the ASan runtime preloaded.  Any sanitizer report fails the
run (halt_on_error)."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "ssd_chunked_scan_chunk_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
       "-g", "-O1", "-fPIC", "-shared"]


def _asan_runtime():
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None, reason="needs gcc/g++")
def test_oracle_and_abi_under_asan_ubsan(tmp_path):
    asan = _asan_runtime()
    if asan is None:
        pytest.skip("gcc has no AddressSanitizer runtime here")
    ora = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-std=c11"] + SAN + [os.path.join(ROOT, "oracle", "ssd_oracle.c"), "-o", ora,
                    "-lm", "-lpthread"], check=True)
    abi = str(tmp_path / "libssd_host_san.so")
    subprocess.run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC] + SAN +
                   [os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "shapes.cpp"),
                    os.path.join(ROOT, "tests", "sanitize", "abi_stubs.cpp"), "-o", abi], check=True)
    env = dict(os.environ)
    env.update({"SSD_ORACLE_LIB": ora, "SSD_LIB": abi, "LD_PRELOAD": asan,
                "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:log_path=" + str(tmp_path / "asan"),
                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"})
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-s", "-p", "no:cacheprovider",
                        "-m", "not gpu", os.path.join(ROOT, "tests", "test_oracle.py"),
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    for f in sorted(tmp_path.glob("asan*")):     # reports written by the ASan runtime
        out += "\n" + f.read_text()
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out, out[-2000:]
