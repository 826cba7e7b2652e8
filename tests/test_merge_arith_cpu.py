"""Host-only checks of the arithmetic the kernels share with the host
(pkd_internal.hpp), compiled with hipcc for the host and run on the CPU:

- the in-place merge's counter words: from any stale word (garbage, another
  call's part-way count, a completed call's reset word, this call's own reset
  word) exactly the last of a segment's pieces sees the count complete and
  leaves the reset word, which the next call counts from; call tags wrap at
  2^40 and are never 0, and the largest tag leaves the count's 24 bits intact;
- the balanced partition's pieces: walking each workgroup's range as the
  kernel does gives, for every segment, the first workgroup and the piece count
  that segment_pieces computes in closed form (the merge kernel and the
  in-place merge both use it), and every slot w + s is used once;
- the paired deal of whole items: each item goes to exactly one workgroup, at
  most two each, pairs fold the 2E shortest and the rest run alone.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def test_shared_kernel_arithmetic(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("no hipcc")
    exe = str(tmp_path / "merge_arith")
    src = os.path.join(ROOT, "tests", "host", "merge_arith_driver.cpp")
    r = subprocess.run([HIPCC, "-O1", "-std=c++17", "-I", os.path.join(ROOT, "paged_kv_decode_amd", "csrc"),
                        src, "-o", exe], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr
