"""paged_decode_ext_noalloc, the entry whose workspace is the library's fixed
device array, against paged_decode_ext with a caller workspace (needs an MI355X).

Both run the same kernels on the same inputs, so the outputs must agree bit for
bit.  Each case makes two calls in a row, the second with a smaller problem, so
the second runs on the array as the first left it.
"""
import pytest
import torch

from paged_kv_decode_amd import workloads as wl

pytestmark = pytest.mark.gpu

BAL = -1000  # PKD_SPLITS_BALANCED
PAIR = -1001  # PKD_SPLITS_PAIRED


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_decode_amd import binding
    return binding


def _dev(w):
    cuda = torch.device("cuda:0")
    t = dict(q=w.q.to(cuda), k=w.k_cache.to(cuda), v=w.v_cache.to(cuda),
             bt=w.block_table.to(cuda), lens=w.seq_lens.to(cuda))
    t["ks"] = None if w.k_scale is None else w.k_scale.to(cuda)
    t["vs"] = None if w.v_scale is None else w.v_scale.to(cuda)
    t["sinks"] = None if getattr(w, "sinks", None) is None else w.sinks.to(cuda)
    return t


def _both(B, w, S):
    """(noalloc out, lse), (ext out, lse) for workload w in split mode S."""
    t = _dev(w)
    dims = B.dims_for(t["q"], t["k"], t["bt"])
    ext = B.ext_for(t["q"], causal=w.spec.causal, window=w.spec.window)
    h = B.current_stream_handle(0)
    res = []
    for noalloc in (True, False):
        out = torch.full(t["q"].shape, float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full(t["q"].shape[:-1], float("nan"), dtype=torch.float32, device="cuda")
        if noalloc:
            st = B.paged_decode_ext_noalloc(dims, ext, t["q"], t["k"], t["v"], t["bt"], t["lens"], t["ks"], t["vs"],
                                            t["sinks"], w.scale, out, lse, S, h)
        else:
            need = B.paged_decode_workspace_bytes_ext(dims, ext, S)
            ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
            st = B.paged_decode_ext(dims, ext, t["q"], t["k"], t["v"], t["bt"], t["lens"], t["ks"], t["vs"],
                                    t["sinks"], w.scale, out, lse, S, ws if need else None, need, h)
        assert st == 0, (noalloc, S, B.paged_decode_status_string(st))
        torch.cuda.synchronize()
        res.append((out.cpu(), lse.cpu()))
    return res


def _lens(n, hi, seed):
    return [(i * 7919 + seed * 131) % hi + 1 for i in range(n)]


# (name, S, batch, Hq, Hkv, D, ps, dtype, q_len, causal, window, sinks, first lengths, second lengths)
CASES = [
    ("balanced in-place merge", BAL, 40, 32, 8, 128, 64, "bf16", 1, False, 0, False,
     _lens(40, 4000, 1), _lens(33, 2500, 2)),
    ("balanced with merge kernel", BAL, 5, 32, 8, 128, 64, "bf16", 1, False, 0, False,
     [700, 2, 0, 3000, 64], [300, 1]),
    ("grid splits", 4, 12, 16, 2, 64, 16, "bf16", 1, False, 0, False, _lens(12, 3000, 3), _lens(7, 900, 4)),
    ("direct output", 1, 8, 32, 8, 128, 64, "bf16", 1, False, 0, False, _lens(8, 2000, 5), _lens(3, 500, 6)),
    ("heuristic, fp8", 0, 24, 64, 8, 128, 64, "fp8_e4m3", 1, False, 0, False, _lens(24, 3000, 7),
     _lens(9, 1500, 8)),
    ("verify, window, sinks", BAL, 10, 16, 2, 128, 64, "bf16", 4, True, 500, True, _lens(10, 3000, 9),
     _lens(4, 800, 10)),
    # whole items paired by length (40 and 36 sequences of 8 KV heads: between one and two
    # items per compute unit), and the same mode falling back to the equal ranges with the
    # in-place merge (equal lengths)
    ("paired mode", PAIR, 40, 32, 8, 64, 64, "bf16", 1, False, 0, False, _lens(40, 3000, 11),
     _lens(36, 2000, 12)),
    ("paired mode, fallback", PAIR, 33, 32, 8, 64, 64, "bf16", 1, False, 0, False, [900] * 33, [700] * 34),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_ext_twice(B, case):
    name, S, bq, hq, hkv, d, ps, dtype, q_len, causal, window, sinks, lens1, lens2 = case
    for call, lens in enumerate((lens1, lens2)):
        w = wl.custom_workload(len(lens), hq, hkv, d, ps, lens, dtype, seed=900 + call, q_len=q_len,
                               causal=causal, window=window, sinks=sinks)
        (o1, l1), (o2, l2) = _both(B, w, S)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), (name, call)
        assert torch.equal(l1.view(torch.int32), l2.view(torch.int32)), (name, call)


def test_noalloc_rejects_a_mode_beyond_the_array(B):
    """A grid mode whose partials exceed the fixed array returns PKD_ERR_SCRATCH_LIMIT
    and writes nothing."""
    lens = _lens(64, 4000, 11)
    w = wl.custom_workload(len(lens), 32, 8, 128, 64, lens, "bf16", seed=950)
    t = _dev(w)
    dims = B.dims_for(t["q"], t["k"], t["bt"])
    S = 64
    assert B.paged_decode_workspace_bytes_ext(dims, None, S) > B.PKD_NOALLOC_SCRATCH_BYTES
    out = torch.zeros(t["q"].shape, dtype=torch.bfloat16, device="cuda")
    st = B.paged_decode_ext_noalloc(dims, None, t["q"], t["k"], t["v"], t["bt"], t["lens"], None, None, None,
                                    w.scale, out, None, S, B.current_stream_handle(0))
    assert st == B.PKD_ERR_SCRATCH_LIMIT
    torch.cuda.synchronize()
    assert int(out.view(torch.int16).count_nonzero()) == 0
