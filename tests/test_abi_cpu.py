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
    """Every function declared in the public headers (include/*.h)."""
    names = set()
    inc = os.path.join(ROOT, "include")
    for h in sorted(os.listdir(inc)):
        if not h.endswith(".h"):
            continue
        text = re.sub(r"/\*.*?\*/", "", open(os.path.join(inc, h)).read(), flags=re.S)
        names |= set(re.findall(r"^\s*(?:int32_t|size_t|const char\*)\s+(\w+)\s*\(", text, flags=re.M))
    return sorted(names)


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
    assert ctypes.sizeof(b.pkd_dims) == 8 * 4
    assert ctypes.sizeof(b.pkd_ext) == 4 * 4


def test_status_strings_are_distinct():
    codes = [0, -1, -2, -3, -4, -5, -6, -7, -8, -9, -10, -11, -12]
    texts = [b.paged_decode_status_string(c) for c in codes]
    assert len(set(texts)) == len(texts)
    assert b.paged_decode_status_string(-12345) == "unknown status"


def dims(**kw):
    base = dict(batch=2, num_q_heads=4, num_kv_heads=1, head_dim=64, page_size=16, num_pages=10,
                max_pages_per_seq=7, kv_dtype=b.PKD_DTYPE_BF16)
    base.update(kw)
    return b.pkd_dims(*[base[f] for f, _ in b.pkd_dims._fields_])


def ext(q_len=1, causal=0, window=0, reserved=0):
    return b.pkd_ext(q_len, causal, window, reserved)


def call(d, q=FAKE, k=FAKE, v=FAKE, bt=FAKE, lens=FAKE, ks=None, vs=None, scale=0.125, out=FAKE,
         lse=None, S=1, ws=None, ws_bytes=0):
    """paged_decode, the plain entry."""
    return b.paged_decode(d, q, k, v, bt, lens, ks, vs, scale, out, lse, S, ws, ws_bytes, None)


def call_ext(d, e=None, q=FAKE, k=FAKE, v=FAKE, bt=FAKE, lens=FAKE, ks=None, vs=None, scale=0.125, out=FAKE,
             lse=None, S=1, ws=None, ws_bytes=0, sinks=None):
    """paged_decode_ext, the entry with the extended forms and special split modes."""
    return b.paged_decode_ext(d, e, q, k, v, bt, lens, ks, vs, sinks, scale, out, lse, S, ws, ws_bytes, None)


# The plain entry's prototype as the boundary's contract writes it (scope table,
# part (b)): dims, q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale,
# scale, out, lse, num_splits, workspace, workspace_bytes, stream.
CONTRACT_PARAMS = ["const pkd_dims*", "const void*", "const void*", "const void*", "const int32_t*",
                   "const int32_t*", "const float*", "const float*", "float", "void*", "float*", "int32_t",
                   "void*", "size_t", "void*"]
CONTRACT_DIMS = ["batch", "num_q_heads", "num_kv_heads", "head_dim", "page_size", "num_pages",
                 "max_pages_per_seq", "kv_dtype"]


def _prototype_params(name):
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    m = re.search(r"\b" + name + r"\s*\(([^)]*)\)\s*;", text)
    assert m, name
    params = []
    for part in m.group(1).split(","):
        part = " ".join(part.split())
        typ = re.sub(r"\s*\b\w+$", "", part)  # drop the parameter name
        params.append(typ.replace(" *", "*"))
    return params


def test_plain_entry_matches_the_contract_prototype():
    """The header declares paged_decode and pkd_dims exactly as the contract
    writes them: the same parameter types in the same order, and the same
    eight int32 fields."""
    assert _prototype_params("paged_decode") == CONTRACT_PARAMS
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef struct \{([^}]*)\} pkd_dims;", text).group(1)
    assert re.findall(r"int32_t\s+(\w+);", body) == CONTRACT_DIMS
    assert [f for f, _ in b.pkd_dims._fields_] == CONTRACT_DIMS


def test_contract_prototype_compiles_against_the_header(tmp_path):
    """A C caller written to the contract: its function-pointer type must accept
    &paged_decode without a conversion (gcc with incompatible pointer types an
    error), and its pkd_dims must be 32 bytes."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "caller.c"
    src.write_text(
        '#include "paged_kv_decode.h"\n'
        "typedef int32_t (*contract_fn)(const pkd_dims*, const void*, const void*, const void*,\n"
        "                               const int32_t*, const int32_t*, const float*, const float*, float,\n"
        "                               void*, float*, int32_t, void*, size_t, void*);\n"
        "contract_fn entry = &paged_decode;\n"
        "typedef char dims_is_32_bytes[sizeof(pkd_dims) == 32 ? 1 : -1];\n")
    r = subprocess.run([cc, "-std=c11", "-fsyntax-only", "-Werror=incompatible-pointer-types",
                        "-I", os.path.join(ROOT, "include"), str(src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_contract_prototype_called_through_ctypes():
    """Calls the exported symbol through a prototype built from the contract alone
    (not the binding's), so a drift in the argument order would show."""
    lib = ctypes.CDLL(b.LIB_PATH)
    fn = lib.paged_decode
    P = ctypes.c_void_p

    class Dims(ctypes.Structure):
        _fields_ = [(n, ctypes.c_int32) for n in CONTRACT_DIMS]

    fn.argtypes = [ctypes.POINTER(Dims), P, P, P, P, P, P, P, ctypes.c_float, P, P, ctypes.c_int32, P,
                   ctypes.c_size_t, P]
    fn.restype = ctypes.c_int32
    d = Dims(2, 4, 1, 64, 16, 10, 7, b.PKD_DTYPE_BF16)
    ok = (ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None, None)
    assert fn(None, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0.125, FAKE, None, 1, None, 0, None) == \
        b.PKD_ERR_NULL_POINTER
    # the float scale sits in its own position: a NaN there is rejected
    assert fn(*ok, float("nan"), FAKE, None, 1, None, 0, None) == b.PKD_ERR_BAD_DIMS
    # lse is the eleventh argument: a misaligned lse is rejected
    assert fn(*ok, 0.125, FAKE, FAKE + 1, 1, None, 0, None) == b.PKD_ERR_ALIGNMENT
    # num_splits above the cap is rejected; a workspace too small for 3 splits is rejected
    assert fn(*ok, 0.125, FAKE, None, b.PKD_MAX_SPLITS + 1, None, 0, None) == b.PKD_ERR_NUM_SPLITS
    assert fn(*ok, 0.125, FAKE, None, 3, FAKE, 16, None) == b.PKD_ERR_WORKSPACE
    # FP8 without scales is rejected
    d8 = Dims(2, 4, 1, 64, 16, 10, 7, b.PKD_DTYPE_FP8_E4M3)
    assert fn(ctypes.byref(d8), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0.125, FAKE, None, 1, None, 0, None) == \
        b.PKD_ERR_SCALES


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
    (dict(num_q_heads=2**25, num_kv_heads=1), b.PKD_ERR_BAD_DIMS),
    (dict(num_q_heads=2**31 - 1, num_kv_heads=1), b.PKD_ERR_BAD_DIMS),
])
def test_bad_dims_are_rejected(kw, status):
    d = dims(**kw)
    assert call(d) == status
    assert call_ext(d) == status
    assert b.paged_decode_num_splits(d, 0) == status
    assert b.paged_decode_workspace_bytes(d, 2) == 0


@pytest.mark.parametrize("kw", [dict(q_len=0), dict(q_len=b.PKD_MAX_Q_LEN + 1), dict(causal=2),
                                dict(causal=-1), dict(window=-1), dict(reserved=1)])
def test_bad_ext_is_rejected(kw):
    d, e = dims(), ext(**kw)
    assert call_ext(d, e) == b.PKD_ERR_BAD_DIMS
    assert b.paged_decode_num_splits_ext(d, e, 0) == b.PKD_ERR_BAD_DIMS
    assert b.paged_decode_workspace_bytes_ext(d, e, 2) == 0
    assert b.paged_decode_launches(d, e, 1) == b.PKD_ERR_BAD_DIMS


def test_null_ext_is_plain_decode():
    """ext NULL and ext {1, 0, 0, 0} describe the same problem."""
    d = dims(batch=32, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=64, num_pages=1500,
             max_pages_per_seq=64)
    for S in (1, 3, 0, b.PKD_SPLITS_BALANCED):
        assert b.paged_decode_workspace_bytes_ext(d, None, S) == b.paged_decode_workspace_bytes_ext(d, ext(), S)
        assert b.paged_decode_launches(d, None, S) == b.paged_decode_launches(d, ext(), S)
    assert b.paged_decode_num_splits_ext(d, None, 0) == b.paged_decode_num_splits(d, 0)
    assert b.paged_decode_num_splits_ext(d, ext(), 0) == b.paged_decode_num_splits(d, 0)


def test_null_pointers_are_rejected():
    d = dims()
    assert b.paged_decode(None, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0.1, FAKE, None, 1, None, 0,
                          None) == b.PKD_ERR_NULL_POINTER
    assert call_ext(None) == b.PKD_ERR_NULL_POINTER
    for kw in ("q", "k", "v", "bt", "lens", "out"):
        assert call(d, **{kw: None}) == b.PKD_ERR_NULL_POINTER, kw
        assert call_ext(d, **{kw: None}) == b.PKD_ERR_NULL_POINTER, kw


def test_noalloc_argument_checks():
    """paged_decode_ext_noalloc: argument errors as paged_decode_ext's, a mode
    whose workspace exceeds the fixed array rejected before anything else is
    touched, and, without a GPU, a valid call reports the missing device."""
    def na(d, e=None, q=FAKE, S=1, out=FAKE, sinks=None):
        return b.paged_decode_ext_noalloc(d, e, q, FAKE, FAKE, FAKE, FAKE, None, None, sinks, 0.125, out, None, S,
                                          None)
    assert na(None) == b.PKD_ERR_NULL_POINTER
    assert na(dims(head_dim=96)) == b.PKD_ERR_HEAD_DIM
    assert na(dims(), ext(reserved=1)) == b.PKD_ERR_BAD_DIMS
    assert na(dims(), q=None) == b.PKD_ERR_NULL_POINTER
    assert na(dims(), S=3, out=None) == b.PKD_ERR_NULL_POINTER
    assert na(dims(), S=-5) == b.PKD_ERR_NUM_SPLITS
    big = dims(batch=64, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=64, num_pages=4096,
               max_pages_per_seq=64)
    assert b.paged_decode_workspace_bytes_ext(big, None, 64) > b.PKD_NOALLOC_SCRATCH_BYTES
    assert na(big, S=64) == b.PKD_ERR_SCRATCH_LIMIT
    import torch
    if not torch.cuda.is_available():
        assert na(dims()) == b.PKD_ERR_DEVICE
        assert na(dims(), S=3) == b.PKD_ERR_DEVICE
        assert na(big, S=b.PKD_SPLITS_BALANCED) == b.PKD_ERR_DEVICE


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
    assert call_ext(d, sinks=FAKE + 2) == b.PKD_ERR_ALIGNMENT
    need = b.paged_decode_workspace_bytes(d, 3)
    assert call(d, S=3, ws=FAKE + 8, ws_bytes=need) == b.PKD_ERR_ALIGNMENT
    args = (FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0.1)
    assert b.paged_decode_partials(d, None, *args, 2, FAKE + 4, FAKE, None) == b.PKD_ERR_ALIGNMENT
    assert b.paged_decode_merge(8, 2, 64, FAKE + 2, FAKE, FAKE, None, None) == b.PKD_ERR_ALIGNMENT
    assert b.paged_decode_merge(8, 2, 64, FAKE, FAKE, FAKE + 1, None, None) == b.PKD_ERR_ALIGNMENT
    assert b.paged_decode_check_tables(d, FAKE + 2, FAKE, FAKE, None) == b.PKD_ERR_ALIGNMENT


def test_window_bounds_the_split_count():
    """With a sliding window the splits cover only the visible span, so the
    heuristic asks for no more splits than that span needs (a page size that
    is not a multiple of 16 keeps it on the grid mode)."""
    d = dims(batch=1, num_q_heads=8, num_kv_heads=8, page_size=8, max_pages_per_seq=4096, num_pages=4096)
    full = b.paged_decode_num_splits(d, 0)
    windowed = b.paged_decode_num_splits_ext(d, ext(window=256), 0)
    assert 1 <= windowed < full
    assert windowed <= (256 + 15 + 255) // 256


def test_non_finite_scale_is_rejected():
    assert call(dims(), scale=float("nan")) == b.PKD_ERR_BAD_DIMS
    assert call(dims(), scale=float("inf")) == b.PKD_ERR_BAD_DIMS


def test_num_splits_and_workspace_rules():
    d = dims()
    assert call(d, S=b.PKD_MAX_SPLITS + 1) == b.PKD_ERR_NUM_SPLITS
    assert call_ext(d, S=b.PKD_MAX_SPLITS + 1) == b.PKD_ERR_NUM_SPLITS
    # paged_decode: every num_splits <= 0 is the heuristic; paged_decode_ext: only
    # PKD_SPLITS_AUTO and PKD_SPLITS_BALANCED are accepted below 1
    assert call(d, S=-5) == call(d, S=0) == call(d, S=b.PKD_SPLITS_BALANCED)
    assert call_ext(d, S=-5) == b.PKD_ERR_NUM_SPLITS
    assert b.paged_decode_workspace_bytes(d, -5) == b.paged_decode_workspace_bytes(d, 0)
    assert b.paged_decode_workspace_bytes_ext(d, None, -5) == 0
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
    d, e3 = dims(), ext(q_len=3, causal=1)
    # [B][q_len][Hq][S][D] fp32 + [B][q_len][Hq][S] fp32 (288 B, rounded up to 512)
    assert b.paged_decode_workspace_bytes_ext(d, e3, 3) == 2 * 3 * 4 * 3 * 64 * 4 + 512
    # G = 4, q_len = 3: 12 rows per KV head, one head group of 12 rows per slot
    one = b.paged_decode_workspace_bytes_ext(d, None, b.PKD_SPLITS_BALANCED)
    three = b.paged_decode_workspace_bytes_ext(d, e3, b.PKD_SPLITS_BALANCED)
    assert three > one
    # G = 4, q_len = 5: 20 rows, two head groups per KV head
    e5 = ext(q_len=5)
    assert b.paged_decode_launches(d, e5, 4) == 2
    assert b.paged_decode_workspace_bytes_ext(d, e5, b.PKD_SPLITS_BALANCED) > three
    assert call_ext(d, ext(q_len=b.PKD_MAX_Q_LEN), S=3) == b.PKD_ERR_WORKSPACE  # accepted shape, no workspace


def test_valid_call_without_gpu_reports_no_device():
    """With correct arguments and no usable GPU the library reports it instead of
    computing anything (with a GPU present this case is covered by the GPU tests)."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    d = dims()
    assert call(d) == b.PKD_ERR_DEVICE
    assert call_ext(d, ext(q_len=2, causal=1)) == b.PKD_ERR_DEVICE
    need = b.paged_decode_workspace_bytes(d, 3)
    assert call(d, S=3, ws=FAKE, ws_bytes=need) == b.PKD_ERR_DEVICE
    assert call(dims(batch=0)) == b.PKD_OK  # an empty batch enqueues nothing
    assert call_ext(dims(batch=0)) == b.PKD_OK


def test_partials_and_merge_argument_checks():
    d = dims()
    args = (FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0.1)
    assert b.paged_decode_partials(d, None, *args, 0, FAKE, FAKE, None) == b.PKD_ERR_NUM_SPLITS
    assert b.paged_decode_partials(d, None, *args, 2, None, FAKE, None) == b.PKD_ERR_NULL_POINTER
    assert b.paged_decode_partials(d, ext(reserved=3), *args, 2, FAKE, FAKE, None) == b.PKD_ERR_BAD_DIMS
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
    assert b.paged_decode_partition(d, None, *args, 1, FAKE, 1 << 20, None) == b.PKD_ERR_NUM_SPLITS
    assert b.paged_decode_finish(d, None, 1, FAKE, 1 << 20, None, FAKE, None, None) == b.PKD_ERR_NUM_SPLITS
    need = b.paged_decode_workspace_bytes(d, 4)
    assert b.paged_decode_partition(d, None, *args, 4, FAKE, need - 1, None) == b.PKD_ERR_WORKSPACE
    assert b.paged_decode_finish(d, None, 4, None, need, None, FAKE, None, None) == b.PKD_ERR_WORKSPACE
    assert b.paged_decode_finish(d, None, 4, FAKE, need, None, None, None, None) == b.PKD_ERR_NULL_POINTER
    assert b.paged_decode_partition(d, None, *args, -7, FAKE, need, None) == b.PKD_ERR_NUM_SPLITS
    # the workspace of 3 query tokens is larger than that of one
    e3 = ext(q_len=3)
    need3 = b.paged_decode_workspace_bytes_ext(d, e3, 4)
    assert need3 > need
    assert b.paged_decode_partition(d, e3, *args, 4, FAKE, need, None) == b.PKD_ERR_WORKSPACE
    assert b.paged_decode_finish(d, e3, 4, FAKE, need, None, FAKE, None, None) == b.PKD_ERR_WORKSPACE


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
    wide = dims(max_pages_per_seq=256, num_pages=512)
    assert b.paged_decode_num_splits_ext(wide, ext(window=200), 0) == 1
    assert b.paged_decode_num_splits_ext(wide, ext(window=300), 0) == b.PKD_SPLITS_BALANCED


def test_balanced_mode_rules():
    ok = dims(batch=4, page_size=16)
    need = b.paged_decode_workspace_bytes_ext(ok, None, b.PKD_SPLITS_BALANCED)
    assert need > 0
    assert call_ext(ok, S=b.PKD_SPLITS_BALANCED) == b.PKD_ERR_WORKSPACE
    assert call_ext(ok, S=b.PKD_SPLITS_BALANCED, ws=FAKE, ws_bytes=need - 1) == b.PKD_ERR_WORKSPACE
    odd_ps = dims(batch=4, page_size=24)
    assert b.paged_decode_workspace_bytes_ext(odd_ps, None, b.PKD_SPLITS_BALANCED) == 0
    assert call_ext(odd_ps, S=b.PKD_SPLITS_BALANCED, ws=FAKE, ws_bytes=1 << 30) == b.PKD_ERR_NUM_SPLITS
    too_many = dims(batch=b.PKD_BALANCED_MAX_BATCH + 1, page_size=16)
    assert call_ext(too_many, S=b.PKD_SPLITS_BALANCED, ws=FAKE, ws_bytes=1 << 30) == b.PKD_ERR_NUM_SPLITS


def test_valu_entry_argument_checks():
    """pkd_decode_valu takes a bf16 cache, head_dim 64 or 128, G in {1, 2, 4} and
    page sizes that are multiples of 16; everything else is rejected on the host."""
    def v(d, q=FAKE, lse=None, out=FAKE):
        return b.pkd_decode_valu(d, q, FAKE, FAKE, FAKE, FAKE, 0.125, out, lse, None)
    assert v(None) == b.PKD_ERR_NULL_POINTER
    assert v(dims(head_dim=256)) == b.PKD_ERR_HEAD_DIM
    assert v(dims(head_dim=32)) == b.PKD_ERR_HEAD_DIM
    assert v(dims(kv_dtype=b.PKD_DTYPE_FP8_E4M3)) == b.PKD_ERR_DTYPE
    assert v(dims(num_q_heads=8, num_kv_heads=1)) == b.PKD_ERR_BAD_DIMS  # G = 8
    assert v(dims(num_q_heads=6, num_kv_heads=4)) == b.PKD_ERR_GQA
    assert v(dims(page_size=24)) == b.PKD_ERR_BAD_DIMS
    assert v(dims(), q=None) == b.PKD_ERR_NULL_POINTER
    assert v(dims(), q=FAKE + 8) == b.PKD_ERR_ALIGNMENT
    assert v(dims(), lse=FAKE + 2) == b.PKD_ERR_ALIGNMENT
    assert v(dims(batch=0)) == b.PKD_OK
    import torch
    if not torch.cuda.is_available():
        assert v(dims()) == b.PKD_ERR_DEVICE


def test_lds_entry_argument_checks():
    """pkd_decode_lds takes a bf16 cache, head_dim 128, G <= 16, page sizes that are
    multiples of 16 and at most 512 pages per sequence; everything else is rejected
    on the host."""
    def v(d, q=FAKE, lse=None, out=FAKE):
        return b.pkd_decode_lds(d, q, FAKE, FAKE, FAKE, FAKE, 0.125, out, lse, None)

    def d128(**kw):
        return dims(**{"head_dim": 128, **kw})
    assert v(None) == b.PKD_ERR_NULL_POINTER
    assert v(d128(head_dim=64)) == b.PKD_ERR_HEAD_DIM
    assert v(d128(head_dim=256)) == b.PKD_ERR_HEAD_DIM
    assert v(d128(kv_dtype=b.PKD_DTYPE_FP8_E4M3)) == b.PKD_ERR_DTYPE
    assert v(d128(num_q_heads=32, num_kv_heads=1)) == b.PKD_ERR_BAD_DIMS  # G = 32
    assert v(d128(num_q_heads=6, num_kv_heads=4)) == b.PKD_ERR_GQA
    assert v(d128(page_size=24)) == b.PKD_ERR_BAD_DIMS
    assert v(d128(max_pages_per_seq=513)) == b.PKD_ERR_BAD_DIMS
    assert v(d128(), q=None) == b.PKD_ERR_NULL_POINTER
    assert v(d128(), q=FAKE + 8) == b.PKD_ERR_ALIGNMENT
    assert v(d128(), lse=FAKE + 2) == b.PKD_ERR_ALIGNMENT
    assert v(d128(batch=0)) == b.PKD_OK
    import torch
    if not torch.cuda.is_available():
        assert v(d128()) == b.PKD_ERR_DEVICE
        assert v(d128(num_q_heads=16, num_kv_heads=1, max_pages_per_seq=512)) == b.PKD_ERR_DEVICE


def test_one_hip_runtime_in_process():
    """The library binds to PyTorch's HIP runtime instead of mapping a second one."""
    assert len(b._hip_runtimes_mapped()) <= 1


def test_launch_counts():
    """Direct output is one kernel; grid splits two; the balanced mode one where
    segments are at least as many as workgroups (it merges in place), else two."""
    b32 = dims(batch=32, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=64,
               num_pages=1500, max_pages_per_seq=64)
    assert b.paged_decode_launches(b32, None, 1) == 1
    assert b.paged_decode_launches(b32, None, 4) == 2
    assert b.paged_decode_launches(b32, None, b.PKD_SPLITS_BALANCED) == 1
    assert b.paged_decode_launches(b32, None, 0) == 1
    long1 = dims(batch=1, num_q_heads=16, num_kv_heads=2, head_dim=64, page_size=64,
                 num_pages=2048, max_pages_per_seq=2048)
    assert b.paged_decode_launches(long1, None, b.PKD_SPLITS_BALANCED) == 2
    assert b.paged_decode_launches(b32, None, -5) == b.PKD_ERR_NUM_SPLITS
    assert b.paged_decode_launches(dims(head_dim=96), None, 1) == b.PKD_ERR_HEAD_DIM


def test_paged_decode_path():
    """The path query agrees with the launch counts; without a device the
    LDS-staged direct kernel (which depends on the compute-unit count) is never
    reported, and bad arguments give statuses."""
    b32 = dims(batch=32, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=64,
               num_pages=1500, max_pages_per_seq=64)
    assert b.paged_decode_path(b32, None, 1) == b.PKD_PATH_DIRECT
    assert b.paged_decode_path(b32, None, 4) == b.PKD_PATH_SPLITS
    assert b.paged_decode_path(b32, None, b.PKD_SPLITS_BALANCED) == b.PKD_PATH_BALANCED
    long1 = dims(batch=1, num_q_heads=16, num_kv_heads=2, head_dim=64, page_size=64,
                 num_pages=2048, max_pages_per_seq=2048)
    assert b.paged_decode_path(long1, None, b.PKD_SPLITS_BALANCED) == b.PKD_PATH_BALANCED_MERGE
    for S in (0, 1, 3, b.PKD_SPLITS_BALANCED):
        for d in (b32, long1):
            path = b.paged_decode_path(d, None, S)
            want = 1 if path in (b.PKD_PATH_DIRECT, b.PKD_PATH_DIRECT_LDS, b.PKD_PATH_BALANCED) else 2
            assert b.paged_decode_launches(d, None, S) == want
    assert b.paged_decode_path(None, None, 1) == b.PKD_ERR_NULL_POINTER
    assert b.paged_decode_path(b32, None, -5) == b.PKD_ERR_NUM_SPLITS
    assert b.paged_decode_path(dims(head_dim=96), None, 1) == b.PKD_ERR_HEAD_DIM


def test_registers_entry_argument_checks():
    """pkd_decode_registers checks its arguments as paged_decode does (bf16 only)."""
    def v(d, q=FAKE, lse=None, out=FAKE):
        return b.pkd_decode_registers(d, q, FAKE, FAKE, FAKE, FAKE, 0.125, out, lse, None)
    assert v(None) == b.PKD_ERR_NULL_POINTER
    assert v(dims(head_dim=96)) == b.PKD_ERR_HEAD_DIM
    assert v(dims(kv_dtype=b.PKD_DTYPE_FP8_E4M3)) == b.PKD_ERR_SCALES
    assert v(dims(num_q_heads=6, num_kv_heads=4)) == b.PKD_ERR_GQA
    assert v(dims(), q=None) == b.PKD_ERR_NULL_POINTER
    assert v(dims(), out=None) == b.PKD_ERR_NULL_POINTER
    assert v(dims(), q=FAKE + 8) == b.PKD_ERR_ALIGNMENT
    assert v(dims(), lse=FAKE + 2) == b.PKD_ERR_ALIGNMENT
    assert v(dims(batch=0)) == b.PKD_OK
    import torch
    if not torch.cuda.is_available():
        assert v(dims()) == b.PKD_ERR_DEVICE


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


def test_stream_read_argument_checks():
    """The measurement stream kernel rejects bad shapes on the host."""
    sink = FAKE
    ok = dict(buf=FAKE, nbytes=1 << 20, row_bytes=2048, chunk_bytes=256, pattern=0, workgroups=8, waves=4,
              batch_kb=8, nontemporal=1, sink=sink, stream=None)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return b.pkd_stream_read(a["buf"], a["nbytes"], a["row_bytes"], a["chunk_bytes"], a["pattern"],
                                 a["workgroups"], a["waves"], a["batch_kb"], a["nontemporal"], a["sink"], a["stream"])
    assert call(buf=None) == b.PKD_ERR_NULL_POINTER
    assert call(sink=None) == b.PKD_ERR_NULL_POINTER
    assert call(buf=FAKE + 8) == b.PKD_ERR_ALIGNMENT
    for kw in (dict(chunk_bytes=48), dict(chunk_bytes=8), dict(row_bytes=1000), dict(nbytes=2048 * 3 + 1024),
               dict(pattern=3), dict(pattern=-1), dict(waves=9), dict(workgroups=0), dict(batch_kb=12),
               dict(nontemporal=2), dict(pattern=1, chunk_bytes=32), dict(pattern=1, nbytes=2048 * 8),
               dict(pattern=2, waves=8, batch_kb=16), dict(pattern=2, waves=4, batch_kb=32)):
        assert call(**kw) == b.PKD_ERR_BAD_DIMS, kw
    # valid shapes reach the device check (no GPU here)
    for kw in (dict(), dict(pattern=1), dict(pattern=2), dict(pattern=2, waves=8, batch_kb=8),
               dict(pattern=2, waves=4, batch_kb=16)):
        assert call(**kw) == b.PKD_ERR_DEVICE, kw
    assert b.pkd_stream_read_sink_bytes(256, 4) == 256 * 4 * 64 * 4
    assert b.pkd_stream_read_sink_bytes(0, 4) == 0
