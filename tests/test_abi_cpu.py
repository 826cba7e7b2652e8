"""C-ABI checks that need no GPU: the library loads, exports every declared
symbol, and rejects bad arguments on the host before anything is enqueued.

No compute call is made here: pointer arguments are fake non-NULL addresses,
which the library never dereferences on an argument error.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "paged_kv_decode.h")

b = pytest.importorskip("paged_kv_decode_amd.binding",
                        reason="HIP library not built (run __graft_entry__.build())")

FAKE = 0x1000  # a non-NULL address that is never dereferenced on these paths


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int32_t|size_t|const char\*)\s+(\w+)\s*\(", text, flags=re.M)))


def header_defines():
    vals = {}
    for name, val in re.findall(r"#define\s+(PKD_\w+)\s+\(?(-?\d+)\)?", open(HEADER).read()):
        vals[name] = int(val)
    return vals


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert set(names) == set(b.EXPORTED)
    lib = ctypes.CDLL(b.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_binding_constants_match_header():
    vals = header_defines()
    for name, v in vals.items():
        if hasattr(b, name):
            assert getattr(b, name) == v, name
    assert vals["PKD_OK"] == 0 and vals["PKD_MAX_SPLITS"] == b.PKD_MAX_SPLITS


def test_dims_struct_layout():
    assert ctypes.sizeof(b.pkd_dims) == 11 * 4


def test_status_strings_are_distinct():
    codes = [0, -1, -2, -3, -4, -5, -6, -7, -8, -9, -10, -11]
    texts = [b.paged_decode_status_string(c) for c in codes]
    assert len(set(texts)) == len(texts)
    assert b.paged_decode_status_string(-12345) == "unknown status"


def dims(**kw):
    base = dict(batch=2, num_q_heads=4, num_kv_heads=1, head_dim=64, page_size=16, num_pages=10,
                max_pages_per_seq=7, kv_dtype=b.PKD_DTYPE_BF16, q_len=1, causal=0, window=0)
    base.update(kw)
    return b.pkd_dims(*[base[f] for f, _ in b.pkd_dims._fields_])


def call(d, q=FAKE, k=FAKE, v=FAKE, bt=FAKE, lens=FAKE, ks=None, vs=None, scale=0.125, out=FAKE,
         lse=None, S=1, ws=None, ws_bytes=0, sinks=None):
    return b.paged_decode(d, q, k, v, bt, lens, ks, vs, sinks, scale, out, lse, S, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(batch=-1), b.PKD_ERR_BAD_DIMS),
    (dict(num_q_heads=0), b.PKD_ERR_BAD_DIMS),
    (dict(num_kv_heads=0), b.PKD_ERR_BAD_DIMS),
    (dict(page_size=0), b.PKD_ERR_BAD_DIMS),
    (dict(num_pages=0), b.PKD_ERR_BAD_DIMS),
    (dict(max_pages_per_seq=0), b.PKD_ERR_BAD_DIMS),
    (dict(num_q_heads=6, num_kv_heads=4), b.PKD_ERR_GQA),
    (dict(head_dim=96), b.PKD_ERR_HEAD_DIM),
    (dict(head_dim=512), b.PKD_ERR_HEAD_DIM),
    (dict(kv_dtype=7), b.PKD_ERR_DTYPE),
    (dict(max_pages_per_seq=2**20, page_size=2**12), b.PKD_ERR_BAD_DIMS),
    (dict(q_len=0), b.PKD_ERR_BAD_DIMS),
    (dict(q_len=b.PKD_MAX_Q_LEN + 1), b.PKD_ERR_BAD_DIMS),
    (dict(causal=2), b.PKD_ERR_BAD_DIMS),
    (dict(causal=-1), b.PKD_ERR_BAD_DIMS),
    (dict(window=-1), b.PKD_ERR_BAD_DIMS),
])
def test_bad_dims_are_rejected(kw, status):
    d = dims(**kw)
    assert call(d) == status
    assert b.paged_decode_num_splits(d, 0) == status
    assert b.paged_decode_workspace_bytes(d, 2) == 0


def test_null_pointers_are_rejected():
    d = dims()
    assert b.paged_decode(None, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, 0.1, FAKE, None, 1, None, 0,
                          None) == b.PKD_ERR_NULL_POINTER
    for kw in ("q", "k", "v", "bt", "lens", "out"):
        assert call(d, **{kw: None}) == b.PKD_ERR_NULL_POINTER, kw


def test_fp8_scales_rules():
    d8 = dims(kv_dtype=b.PKD_DTYPE_FP8_E4M3)
    assert call(d8) == b.PKD_ERR_SCALES
    assert call(d8, ks=FAKE) == b.PKD_ERR_SCALES
    assert call(d8, vs=FAKE) == b.PKD_ERR_SCALES
    assert call(dims(), ks=FAKE, vs=FAKE) == b.PKD_ERR_SCALES


def test_misaligned_pointers_are_rejected():
    d = dims()
    for kw in ("q", "k", "v", "out"):
        assert call(d, **{kw: FAKE + 8}) == b.PKD_ERR_ALIGNMENT, kw
    for kw in ("bt", "lens"):
        assert call(d, **{kw: FAKE + 2}) == b.PKD_ERR_ALIGNMENT, kw
    assert call(d, lse=FAKE + 1) == b.PKD_ERR_ALIGNMENT
    assert call(d, sinks=FAKE + 2) == b.PKD_ERR_ALIGNMENT
    need = b.paged_decode_workspace_bytes(d, 3)
    assert call(d, S=3, ws=FAKE + 8, ws_bytes=need) == b.PKD_ERR_ALIGNMENT
    args = (FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0.1)
    assert b.paged_decode_partials(d, *args, 2, FAKE + 4, FAKE, None) == b.PKD_ERR_ALIGNMENT
    assert b.paged_decode_merge(8, 2, 64, FAKE + 2, FAKE, FAKE, None, None) == b.PKD_ERR_ALIGNMENT
    assert b.paged_decode_merge(8, 2, 64, FAKE, FAKE, FAKE + 1, None, None) == b.PKD_ERR_ALIGNMENT
    assert b.paged_decode_check_tables(d, FAKE + 2, FAKE, FAKE, None) == b.PKD_ERR_ALIGNMENT


def test_window_bounds_the_split_count():
    """With a sliding window the splits cover only the visible span, so the
    heuristic asks for no more splits than that span needs (a page size that
    is not a multiple of 16 keeps it on the grid mode)."""
    d = dims(batch=1, num_q_heads=8, num_kv_heads=8, page_size=8, max_pages_per_seq=4096, num_pages=4096)
    full = b.paged_decode_num_splits(d, 0)
    dw = dims(batch=1, num_q_heads=8, num_kv_heads=8, page_size=8, max_pages_per_seq=4096, num_pages=4096,
              window=256)
    windowed = b.paged_decode_num_splits(dw, 0)
    assert 1 <= windowed < full
    assert windowed <= (256 + 15 + 255) // 256


def test_non_finite_scale_is_rejected():
    assert call(dims(), scale=float("nan")) == b.PKD_ERR_BAD_DIMS
    assert call(dims(), scale=float("inf")) == b.PKD_ERR_BAD_DIMS


def test_num_splits_and_workspace_rules():
    d = dims()
    assert call(d, S=b.PKD_MAX_SPLITS + 1) == b.PKD_ERR_NUM_SPLITS
    assert call(d, S=-5) == b.PKD_ERR_NUM_SPLITS
    assert b.paged_decode_workspace_bytes(d, -5) == 0
    need = b.paged_decode_workspace_bytes(d, 3)
    # [B][Hq][S][D] fp32 + [B][Hq][S] fp32, each rounded up to 256 bytes
    assert need == 2 * 4 * 3 * 64 * 4 + 256
    assert call(d, S=3) == b.PKD_ERR_WORKSPACE
    assert call(d, S=3, ws=FAKE, ws_bytes=need - 1) == b.PKD_ERR_WORKSPACE
    assert b.paged_decode_workspace_bytes(d, 1) == 0
    assert b.paged_decode_workspace_bytes(d, b.PKD_MAX_SPLITS + 1) == 0


def test_workspace_grows_with_query_tokens():
    """Several query tokens per sequence: grid partials are [B][q_len][Hq][S][D]; the
    balanced mode packs the q_len * G rows of a KV head 16 to a head group."""
    d3 = dims(q_len=3, causal=1)
    # [B][q_len][Hq][S][D] fp32 + [B][q_len][Hq][S] fp32 (288 B, rounded up to 512)
    assert b.paged_decode_workspace_bytes(d3, 3) == 2 * 3 * 4 * 3 * 64 * 4 + 512
    # G = 4, q_len = 3: 12 rows per KV head, one head group of 12 rows per slot
    one = b.paged_decode_workspace_bytes(dims(), b.PKD_SPLITS_BALANCED)
    three = b.paged_decode_workspace_bytes(d3, b.PKD_SPLITS_BALANCED)
    assert three > one
    # G = 4, q_len = 5: 20 rows, two head groups per KV head
    d5 = dims(q_len=5)
    assert b.paged_decode_launches(d5, 4) == 2
    assert b.paged_decode_workspace_bytes(d5, b.PKD_SPLITS_BALANCED) > three
    assert call(dims(q_len=b.PKD_MAX_Q_LEN), S=3) == b.PKD_ERR_WORKSPACE  # accepted shape, no workspace


def test_valid_call_without_gpu_reports_no_device():
    """With correct arguments and no usable GPU the library reports it instead of
    computing anything (with a GPU present this case is covered by the GPU tests)."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    d = dims()
    assert call(d) == b.PKD_ERR_DEVICE
    need = b.paged_decode_workspace_bytes(d, 3)
    assert call(d, S=3, ws=FAKE, ws_bytes=need) == b.PKD_ERR_DEVICE
    assert call(dims(batch=0)) == b.PKD_OK  # an empty batch enqueues nothing


def test_partials_and_merge_argument_checks():
    d = dims()
    args = (FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0.1)
    assert b.paged_decode_partials(d, *args, 0, FAKE, FAKE, None) == b.PKD_ERR_NUM_SPLITS
    assert b.paged_decode_partials(d, *args, 2, None, FAKE, None) == b.PKD_ERR_NULL_POINTER
    assert b.paged_decode_merge(8, 2, 100, FAKE, FAKE, FAKE, None, None) == b.PKD_ERR_HEAD_DIM
    assert b.paged_decode_merge(8, 0, 64, FAKE, FAKE, FAKE, None, None) == b.PKD_ERR_NUM_SPLITS
    assert b.paged_decode_merge(-1, 2, 64, FAKE, FAKE, FAKE, None, None) == b.PKD_ERR_BAD_DIMS
    assert b.paged_decode_merge(8, 2, 64, FAKE, None, FAKE, None, None) == b.PKD_ERR_NULL_POINTER
    assert b.paged_decode_merge(0, 2, 64, FAKE, FAKE, FAKE, None, None) == b.PKD_OK
    assert b.paged_decode_check_tables(d, None, FAKE, FAKE, None) == b.PKD_ERR_NULL_POINTER


def test_two_phase_argument_checks():
    d = dims()
    args = (FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0.1)
    # direct output has no split phases
    assert b.paged_decode_partition(d, *args, 1, FAKE, 1 << 20, None) == b.PKD_ERR_NUM_SPLITS
    assert b.paged_decode_finish(d, 1, FAKE, 1 << 20, None, FAKE, None, None) == b.PKD_ERR_NUM_SPLITS
    need = b.paged_decode_workspace_bytes(d, 4)
    assert b.paged_decode_partition(d, *args, 4, FAKE, need - 1, None) == b.PKD_ERR_WORKSPACE
    assert b.paged_decode_finish(d, 4, None, need, None, FAKE, None, None) == b.PKD_ERR_WORKSPACE
    assert b.paged_decode_finish(d, 4, FAKE, need, None, None, None, None) == b.PKD_ERR_NULL_POINTER
    assert b.paged_decode_partition(d, *args, -7, FAKE, need, None) == b.PKD_ERR_NUM_SPLITS


def test_heuristic_choices():
    """Without a device (so without the one-item-per-compute-unit rule, which
    the GPU tests cover): one split when no sequence can show more than 256
    tokens; the balanced partition wherever it applies; otherwise one split
    when the (sequence, KV-head) items already fill the device, else a split
    count bounded by the cap and by the length hint."""
    b128 = dims(batch=128, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=128,
                num_pages=2048, max_pages_per_seq=16)
    assert b.paged_decode_num_splits(b128, 0) == b.PKD_SPLITS_BALANCED
    big = dims(batch=2048, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=128,
               num_pages=32768, max_pages_per_seq=16)
    assert b.paged_decode_num_splits(big, 0) == 1
    b32 = dims(batch=32, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=64,
               num_pages=1500, max_pages_per_seq=64)
    assert b.paged_decode_num_splits(b32, 0) == b.PKD_SPLITS_BALANCED
    odd = dims(batch=32, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=24,
               num_pages=6000, max_pages_per_seq=171)
    s_odd = b.paged_decode_num_splits(odd, 0)
    assert 2 <= s_odd <= 16
    long1 = dims(batch=1, num_q_heads=16, num_kv_heads=2, head_dim=128, page_size=40,
                 num_pages=3277, max_pages_per_seq=3277)
    s1 = b.paged_decode_num_splits(long1, 0)
    assert s_odd < s1 <= b.PKD_MAX_SPLITS
    assert b.paged_decode_num_splits(long1, 256) == 1  # a short hint caps the split count
    tiny = dims()  # 7 pages of 16 tokens
    assert b.paged_decode_num_splits(tiny, 0) == 1
    assert b.paged_decode_num_splits(dims(max_pages_per_seq=16), 0) == 1  # 256 tokens
    assert b.paged_decode_num_splits(dims(max_pages_per_seq=17), 0) == b.PKD_SPLITS_BALANCED
    # a window bounds the span: 200 + 1 + 14 = 215 visible tokens of a 4096-token table
    assert b.paged_decode_num_splits(dims(max_pages_per_seq=256, num_pages=512, window=200), 0) == 1
    assert b.paged_decode_num_splits(dims(max_pages_per_seq=256, num_pages=512, window=300), 0) == \
        b.PKD_SPLITS_BALANCED


def test_balanced_mode_rules():
    ok = dims(batch=4, page_size=16)
    need = b.paged_decode_workspace_bytes(ok, b.PKD_SPLITS_BALANCED)
    assert need > 0
    assert call(ok, S=b.PKD_SPLITS_BALANCED) == b.PKD_ERR_WORKSPACE
    assert call(ok, S=b.PKD_SPLITS_BALANCED, ws=FAKE, ws_bytes=need - 1) == b.PKD_ERR_WORKSPACE
    odd_ps = dims(batch=4, page_size=24)
    assert b.paged_decode_workspace_bytes(odd_ps, b.PKD_SPLITS_BALANCED) == 0
    assert call(odd_ps, S=b.PKD_SPLITS_BALANCED, ws=FAKE, ws_bytes=1 << 30) == b.PKD_ERR_NUM_SPLITS
    too_many = dims(batch=b.PKD_BALANCED_MAX_BATCH + 1, page_size=16)
    assert call(too_many, S=b.PKD_SPLITS_BALANCED, ws=FAKE, ws_bytes=1 << 30) == b.PKD_ERR_NUM_SPLITS


def test_one_hip_runtime_in_process():
    """The library binds to PyTorch's HIP runtime instead of mapping a second one."""
    assert len(b._hip_runtimes_mapped()) <= 1


def test_launch_counts():
    """Direct output is one kernel; grid splits two; the balanced mode one where
    segments are at least as many as workgroups (it merges in place), else two."""
    b32 = dims(batch=32, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=64,
               num_pages=1500, max_pages_per_seq=64)
    assert b.paged_decode_launches(b32, 1) == 1
    assert b.paged_decode_launches(b32, 4) == 2
    assert b.paged_decode_launches(b32, b.PKD_SPLITS_BALANCED) == 1
    assert b.paged_decode_launches(b32, 0) == 1
    long1 = dims(batch=1, num_q_heads=16, num_kv_heads=2, head_dim=64, page_size=64,
                 num_pages=2048, max_pages_per_seq=2048)
    assert b.paged_decode_launches(long1, b.PKD_SPLITS_BALANCED) == 2
    assert b.paged_decode_launches(b32, -5) == b.PKD_ERR_NUM_SPLITS
    assert b.paged_decode_launches(dims(head_dim=96), 1) == b.PKD_ERR_HEAD_DIM


# ---- paged_decode_metadata argument checks ----------------------------------

def meta(**kw):
    base = dict(batch=4, req_rows=8, req_stride=256, page_size=16, max_pages_per_seq=16, q_len=1, window=0,
                extend=1)
    base.update(kw)
    return b.pkd_meta_dims(*[base[f] for f, _ in b.pkd_meta_dims._fields_])


def meta_call(md, rt=FAKE, rp=FAKE, sl=FAKE, cs=FAKE, cu=FAKE, pt=FAKE, ss=None, sp=None, err=None):
    return b.paged_decode_metadata(md, rt, rp, sl, cs, cu, pt, ss, sp, err, None)


def test_meta_dims_struct_layout():
    assert ctypes.sizeof(b.pkd_meta_dims) == 8 * 4


@pytest.mark.parametrize("kw", [dict(batch=-1), dict(batch=65536), dict(req_rows=0), dict(req_stride=0),
                                dict(page_size=0), dict(max_pages_per_seq=0), dict(q_len=0),
                                dict(q_len=b.PKD_MAX_Q_LEN + 1), dict(window=-1), dict(extend=-1),
                                dict(batch=65535, max_pages_per_seq=4096, page_size=16)])
def test_metadata_bad_dims(kw):
    assert meta_call(meta(**kw)) == b.PKD_ERR_BAD_DIMS


def test_metadata_pointer_rules():
    assert meta_call(None) == b.PKD_ERR_NULL_POINTER
    for i in range(6):
        args = [FAKE] * 6
        args[i] = None
        assert meta_call(meta(), *args) == b.PKD_ERR_NULL_POINTER, i
    assert meta_call(meta(window=8)) == b.PKD_ERR_NULL_POINTER  # window tables required
    assert meta_call(meta(window=8), ss=FAKE) == b.PKD_ERR_NULL_POINTER
    assert meta_call(meta(), rp=FAKE + 4) == b.PKD_ERR_ALIGNMENT
    assert meta_call(meta(), pt=FAKE + 2) == b.PKD_ERR_ALIGNMENT
    assert meta_call(meta(), err=FAKE + 1) == b.PKD_ERR_ALIGNMENT
    # An empty batch needs cu_seqlens_k only.
    assert meta_call(meta(batch=0, window=3), None, None, None, None, FAKE, None) == b.PKD_ERR_DEVICE
    assert meta_call(meta(batch=0), cu=None) == b.PKD_ERR_NULL_POINTER
    # Valid arguments reach the device check (no device here).
    assert meta_call(meta()) == b.PKD_ERR_DEVICE
    assert meta_call(meta(window=8), ss=FAKE, sp=FAKE, err=FAKE) == b.PKD_ERR_DEVICE


# ---- contiguous_decode argument checks ----------------------------------------

def cdims(**kw):
    base = dict(batch=2, num_q_heads=4, num_kv_heads=2, head_dim=64, max_seq_len=100, kv_dtype=b.PKD_DTYPE_BF16,
                q_len=1, causal=0, window=0, reserved=0, q_strides=(256, 256, 64), kv_strides=(12800, 128, 64),
                out_strides=(256, 256, 64))
    base.update(kw)
    arr = ctypes.c_int64 * 3
    vals = [arr(*base[f]) if f.endswith("strides") else base[f] for f, _ in b.pkd_contig_dims._fields_]
    return b.pkd_contig_dims(*vals)


def ccall(cd, q=FAKE, k=FAKE, v=FAKE, lens=FAKE, ks=None, vs=None, sinks=None, out=FAKE, lse=None, S=1, ws=None,
          ws_bytes=0):
    return b.contiguous_decode(cd, q, k, v, lens, ks, vs, sinks, 0.125, out, lse, S, ws, ws_bytes, None)


def test_contig_dims_struct_layout():
    assert ctypes.sizeof(b.pkd_contig_dims) == 10 * 4 + 9 * 8


@pytest.mark.parametrize("kw,status", [
    (dict(max_seq_len=0), b.PKD_ERR_BAD_DIMS),
    (dict(reserved=1), b.PKD_ERR_BAD_DIMS),
    (dict(batch=-1), b.PKD_ERR_BAD_DIMS),
    (dict(head_dim=48), b.PKD_ERR_HEAD_DIM),
    (dict(num_q_heads=3), b.PKD_ERR_GQA),
    (dict(window=-2), b.PKD_ERR_BAD_DIMS),
    (dict(q_strides=(256, -8, 64)), b.PKD_ERR_BAD_DIMS),
    (dict(kv_strides=(12800, 1 << 27, 64)), b.PKD_ERR_BAD_DIMS),   # 16 token rows overflow 32-bit offsets
    (dict(q_strides=(256, 256, 68)), b.PKD_ERR_ALIGNMENT),          # q rows not 16-byte aligned
    (dict(out_strides=(260, 256, 64)), b.PKD_ERR_ALIGNMENT),
    (dict(kv_strides=(12800, 132, 64)), b.PKD_ERR_ALIGNMENT),
    (dict(kv_dtype=b.PKD_DTYPE_FP8_E4M3, kv_strides=(12800, 136, 64)), b.PKD_ERR_ALIGNMENT),  # 136 B: not 16-aligned
])
def test_contiguous_bad_dims(kw, status):
    cd = cdims(**kw)
    assert ccall(cd) == status
    assert b.contiguous_decode_workspace_bytes(cd, 3) == 0


def test_contiguous_pointer_and_scale_rules():
    assert ccall(None) == b.PKD_ERR_NULL_POINTER
    for kw in ("q", "k", "v", "lens", "out"):
        assert ccall(cdims(), **{kw: None}) == b.PKD_ERR_NULL_POINTER, kw
    assert ccall(cdims(), ks=FAKE, vs=FAKE) == b.PKD_ERR_SCALES
    assert ccall(cdims(kv_dtype=b.PKD_DTYPE_FP8_E4M3, kv_strides=(12800, 128, 64))) == b.PKD_ERR_SCALES
    assert ccall(cdims(), q=FAKE + 8) == b.PKD_ERR_ALIGNMENT
    assert ccall(cdims(), sinks=FAKE + 2) == b.PKD_ERR_ALIGNMENT
    need = b.contiguous_decode_workspace_bytes(cdims(), 3)
    assert need > 0
    assert ccall(cdims(), S=3, ws=None, ws_bytes=0) == b.PKD_ERR_WORKSPACE
    assert ccall(cdims()) == b.PKD_ERR_DEVICE  # valid arguments reach the device check
    assert ccall(cdims(batch=0)) == b.PKD_OK
