"""The CPU oracle and the library's host code under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

tests/sanitize/oracle_driver.c runs every oracle entry point on small problems,
contract violations included; tests/sanitize/host_driver.cpp runs every C-ABI entry
point's argument checks, split heuristic and workspace planning over millions of
argument combinations (valid, invalid and extreme), which without a device end
before any launch.  Both must run to completion with no sanitizer report.  The
host code is rebuilt with the sanitizers for the host pass only (device code is
not instrumented); the kernels' objects come from the regular build.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "paged_kv_decode_amd", "csrc")
BUILD = os.path.join(ROOT, "paged_kv_decode_amd", "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, timeout):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=timeout, env=ENV)
    return r.returncode, r.stdout + r.stderr


def test_oracle_under_sanitizers(tmp_path):
    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("no gcc")
    exe = str(tmp_path / "oracle_asan")
    rc, log = _run([cc, "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", os.path.join(HERE, "oracle_driver.c"), "-o", exe, "-lm",
                    "-lpthread"], 300)
    assert rc == 0, log
    rc, log = _run([exe], 300)
    assert rc == 0 and log.startswith("ok"), log


def test_host_code_under_sanitizers(tmp_path):
    kernels = ["decode_d32", "decode_d64", "decode_d128", "decode_d256", "split_kv_decode", "lse_merge", "kv_append",
               "decode_metadata"]
    objs = [os.path.join(BUILD, k + ".o") for k in kernels]
    if not os.path.exists(HIPCC) or not all(os.path.exists(o) for o in objs):
        pytest.skip("hipcc or the library's build objects missing (run __graft_entry__.build())")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host",
           "-fno-sanitize-recover=all"]
    common = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
              "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    host = [(os.path.join(CSRC, "api.cpp"), []), (os.path.join(HERE, "host_driver.cpp"), [])] + \
        [(os.path.join(CSRC, f + ".hip"), ["-x", "hip"]) for f in ("noalloc", "stream_read", "valu_decode", "lds_decode")]
    built = []
    for src, lang in host:
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        rc, log = _run([HIPCC] + common + san + lang + ["-c", src, "-o", obj], 600)
        assert rc == 0, log
        built.append(obj)
    exe = str(tmp_path / "host_asan")
    rc, log = _run([HIPCC, "--offload-arch=gfx950"] + san + ["-o", exe] + built + objs, 600)
    assert rc == 0, log
    rc, log = _run([exe], 600)
    assert rc == 0 and log.startswith("ok") and "runtime error" not in log, log[-3000:]
