"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The C ABI's host side (gdn_abi.cpp: argument checks, size queries, workspace carving) is
built host-only with ASan + UBSan, its kernel launchers replaced by stubs that return success
(tests/sanitize/gdn_host_stubs.cpp); the float64 oracle (gdn_oracle.c) is built with the same
sanitizers. Then the ABI host tests and the oracle's pins run against those builds in a child
process with the sanitizer runtime preloaded: any out-of-bounds access, use after free or
undefined behaviour in either ends the child with an error report.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]


def _asan_runtime():
    r = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def test_abi_host_and_oracle_pins_under_sanitizers(tmp_path):
    rt = _asan_runtime()
    if not (os.path.exists(HIPCC) and rt):
        pytest.skip("no hipcc / clang sanitizer runtime")
    csrc = os.path.join(ROOT, "gated_delta_rule_34_amd", "csrc")
    lib = str(tmp_path / "libgdn_sanitized.so")
    subprocess.run([HIPCC, "-xhip", "--offload-host-only", *SAN, "-shared-libasan", "-fno-omit-frame-pointer", "-g",
                    "-O1", "-std=c++17", "-fPIC", "-shared", f"-I{ROOT}/include", f"-I{csrc}",
                    os.path.join(csrc, "gdn_abi.cpp"), os.path.join(ROOT, "tests", "sanitize", "gdn_host_stubs.cpp"),
                    "-o", lib], check=True)
    olib = str(tmp_path / "liboracle_sanitized.so")
    subprocess.run([CLANG, "-fsanitize=address,undefined", "-shared-libasan", "-fno-omit-frame-pointer", "-g", "-O1",
                    "-std=c11", "-ffp-contract=off", "-shared", "-fPIC", "-pthread",
                    os.path.join(ROOT, "oracle", "gdn_oracle.c"), "-o", olib], check=True)
    env = dict(os.environ, LD_PRELOAD=rt, GDN_LIBRARY=lib, GDN_ORACLE_LIBRARY=olib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    probe = ("import sys; sys.path.insert(0, '.'); import gated_delta_rule_34_amd, oracle; oracle._load(); "
             "print(open('/proc/self/maps').read())")
    maps = subprocess.run([sys.executable, "-c", probe], env=env, cwd=ROOT, capture_output=True, text=True).stdout
    assert lib in maps and olib in maps and os.path.basename(rt) in maps  # the child runs the sanitized builds
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
           os.path.join(ROOT, "tests", "test_abi_host.py"), os.path.join(ROOT, "tests", "test_oracle.py")]
    r = subprocess.run(cmd, env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
    assert " passed" in r.stdout, tail
