"""Host-side pieces of bench.py that need no GPU: the multi-GPU refusal, the
algorithmic byte count, and the readers of the committed profile summaries."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from paged_kv_decode_amd import workloads as wl  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_bytes_by_hand():
    """K/V rows of exactly the tokens seen, q, out, lse, the block-table entries
    used and the lengths, counted by hand for the two-sequence workload."""
    w = wl.make_workload(wl.WORKLOADS["tiny_b2_d64_ps16"], tail="zero")
    s = w.spec
    lens = [int(x) for x in w.seq_lens]
    kv = sum(lens) * s.num_kv_heads * s.head_dim * 2 * 2
    q = out = s.batch * s.num_q_heads * s.head_dim * 2
    lse = s.batch * s.num_q_heads * 4
    bt = sum(-(-L // s.page_size) for L in lens) * 4
    assert bench.algorithmic_bytes(w) == kv + q + out + lse + bt + s.batch * 4


def test_trace_average_is_read_from_the_committed_summary():
    path = os.path.join(ROOT, "profiles", "kernel_trace_llama_b32_d128_ps64.md")
    rows = [l for l in open(path, encoding="utf-8") if l.startswith("| `pkd::")]
    assert rows, "the B = 32 trace summary lists the library's kernel"
    name = rows[0].split("|")[1].strip().strip("`")
    want = float(rows[0].split("|")[3])
    assert bench.trace_avg_from_profiles("llama_b32_d128_ps64", name.split("<")[0]) == want
    assert bench.trace_avg_from_profiles("llama_b32_d128_ps64", "no_such_kernel") is None
    assert bench.trace_avg_from_profiles("no_such_workload", "pkd::") is None


def test_read_requests_give_the_read_bytes():
    """The L2's own read-request count in the committed B = 32 counter summary,
    times the 128-byte request size, is the step's algorithmic bytes to within
    1% (the step reads each K/V byte once; q, the block table and the lengths are
    a few hundred KB), and agrees with the calibrated FETCH_SIZE figure."""
    from paged_kv_decode_amd import workloads as wl
    rd = bench.rdreq_bytes_from_profiles("llama_b32_d128_ps64")
    assert rd is not None
    alg = bench.algorithmic_bytes(wl.make_workload(wl.WORKLOADS["llama_b32_d128_ps64"], tail="zero"))
    assert abs(rd / alg - 1) < 0.01, (rd, alg)
    rec = __import__("json").load(open(os.path.join(ROOT, "profiles", "traffic_llama_b32_d128_ps64.json")))
    fetch = rec["fetch_kib_per_dispatch"] * 1024 * rec["fetch_scale"]
    assert abs(rd / fetch - 1) < 0.01, (rd, fetch)
    assert bench.rdreq_bytes_from_profiles("no_such_workload") is None


def test_traffic_is_dropped_when_the_kernel_sources_change(tmp_path, monkeypatch):
    """A traffic figure under profiles/ is used only while the digest of the
    kernels' sources matches the one it was taken with."""
    prof = tmp_path / "profiles"
    prof.mkdir()
    rec = {"workload": "llama_b32_d128_ps64", "bytes_per_launch": 123456789.0,
           "kernel_source_sha256": bench._source_digest()}
    (prof / "traffic_llama_b32_d128_ps64.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_from_profiles("llama_b32_d128_ps64") == 123456789.0
    (prof / "traffic_llama_b32_d128_ps64.json").write_text(json.dumps(dict(rec, kernel_source_sha256="0" * 64)))
    assert bench.traffic_from_profiles("llama_b32_d128_ps64") is None
    assert bench.traffic_from_profiles("no_such_workload") is None


@pytest.mark.parametrize("src", ["/* a comment */\n", "// another\n", "\n\n   \n"])
def test_digest_ignores_comments_and_whitespace(tmp_path, monkeypatch, src):
    want = bench._source_digest()
    files = []
    for f in bench.KERNEL_SRCS:
        p = tmp_path / os.path.basename(f)
        p.write_text(open(f, encoding="utf-8").read() + src)
        files.append(str(p))
    monkeypatch.setattr(bench, "KERNEL_SRCS", files)
    assert bench._source_digest() == want


def test_digest_changes_with_the_code(tmp_path, monkeypatch):
    want = bench._source_digest()
    files = []
    for i, f in enumerate(bench.KERNEL_SRCS):
        p = tmp_path / os.path.basename(f)
        p.write_text(open(f, encoding="utf-8").read() + ("\nint extra_symbol;\n" if i == 0 else ""))
        files.append(str(p))
    monkeypatch.setattr(bench, "KERNEL_SRCS", files)
    assert bench._source_digest() != want
