"""Thin ctypes binding over libpaged_kv_decode.so, with the C ABI's names.

Argument marshalling only: every step of the decode runs in the library's HIP
kernels.  Pointer arguments accept a torch tensor (its data_ptr() is passed), a
plain integer address, or None (NULL).  The raw functions return the library's
integer status; `decode` is a convenience that infers the dimensions from torch
tensors, allocates out / lse / workspace with torch.empty on the tensors'
device and raises PkdError on a negative status.

The library must have been built (paged_kv_decode_amd/build.py); if it is
missing this module raises on import.  There is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpaged_kv_decode.so")

PKD_OK = 0
PKD_ERR_NULL_POINTER = -1
PKD_ERR_BAD_DIMS = -2
PKD_ERR_GQA = -3
PKD_ERR_HEAD_DIM = -4
PKD_ERR_DTYPE = -5
PKD_ERR_SCALES = -6
PKD_ERR_NUM_SPLITS = -7
PKD_ERR_WORKSPACE = -8
PKD_ERR_LAUNCH = -9
PKD_ERR_DEVICE = -10
PKD_ERR_ALIGNMENT = -11
PKD_ERR_SCRATCH_LIMIT = -12
PKD_MAX_SPLITS = 512
PKD_NOALLOC_SCRATCH_BYTES = 16 << 20
PKD_MAX_Q_LEN = 64
PKD_SPLIT_ALIGN = 64
PKD_SPLITS_AUTO = 0
PKD_SPLITS_BALANCED = -1000
PKD_BALANCED_MAX_BATCH = 1024
PKD_SPLITS_PAIRED = -1001
PKD_PAIRED_MAX_BATCH = 256
PKD_PATH_DIRECT = 1
PKD_PATH_DIRECT_LDS = 2
PKD_PATH_SPLITS = 3
PKD_PATH_BALANCED = 4
PKD_PATH_BALANCED_MERGE = 5
PKD_PATH_PAIRED = 6
PKD_DTYPE_BF16 = 0
PKD_DTYPE_FP8_E4M3 = 1

EXPORTED = ("paged_decode", "paged_decode_ext", "paged_decode_partition", "paged_decode_finish",
            "paged_decode_num_splits", "paged_decode_num_splits_ext", "paged_decode_launches", "paged_decode_path",
            "paged_decode_workspace_bytes", "paged_decode_workspace_bytes_ext", "paged_decode_partials",
            "paged_decode_merge",
            "paged_decode_check_tables", "paged_kv_append", "paged_decode_metadata", "contiguous_decode",
            "contiguous_decode_workspace_bytes", "paged_decode_status_string", "pkd_stream_read",
            "pkd_stream_read_sink_bytes", "paged_decode_ext_noalloc", "pkd_decode_valu",
            "pkd_decode_lds", "pkd_decode_registers")


class PkdError(RuntimeError):
    def __init__(self, status: int):
        super().__init__(f"paged_kv_decode status {status}: {paged_decode_status_string(status)}")
        self.status = status


class pkd_dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("max_pages_per_seq", ctypes.c_int32), ("kv_dtype", ctypes.c_int32)]


class pkd_ext(ctypes.Structure):
    _fields_ = [("q_len", ctypes.c_int32), ("causal", ctypes.c_int32), ("window", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class pkd_meta_dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("req_rows", ctypes.c_int32), ("req_stride", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32), ("q_len", ctypes.c_int32),
                ("window", ctypes.c_int32), ("extend", ctypes.c_int32)]


class pkd_contig_dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("max_seq_len", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
                ("q_len", ctypes.c_int32), ("causal", ctypes.c_int32), ("window", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("q_strides", ctypes.c_int64 * 3), ("kv_strides", ctypes.c_int64 * 3),
                ("out_strides", ctypes.c_int64 * 3)]


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run paged_kv_decode_amd/build.py "
                      "(or __graft_entry__.build()) first")

# PyTorch bundles its own HIP runtime (SONAME libamdhip64.so.7).  Loading torch
# first makes the library's libamdhip64.so.7 dependency resolve to that same
# runtime, so torch's device pointers and stream handles are valid in the
# library's calls.  Loading the library first would map a second HIP runtime
# from /opt/rocm next to torch's, which cannot share streams or devices.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)


def _hip_runtimes_mapped():
    paths = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    paths.add(os.path.realpath(line.split()[-1]))
    except OSError:
        pass
    return paths


if len(_hip_runtimes_mapped()) > 1:
    raise ImportError("two HIP runtimes are mapped in this process "
                      f"({sorted(_hip_runtimes_mapped())}); import torch before loading "
                      "libpaged_kv_decode.so")

_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_dims_p = ctypes.POINTER(pkd_dims)
_ext_p = ctypes.POINTER(pkd_ext)

_lib.paged_decode.argtypes = [_dims_p, _p, _p, _p, _p, _p, _p, _p, ctypes.c_float, _p, _p, _i32,
                              _p, ctypes.c_size_t, _p]
_lib.paged_decode.restype = _i32
_lib.paged_decode_ext.argtypes = [_dims_p, _ext_p, _p, _p, _p, _p, _p, _p, _p, _p, ctypes.c_float, _p, _p, _i32,
                                  _p, ctypes.c_size_t, _p]
_lib.paged_decode_ext.restype = _i32
_lib.paged_decode_ext_noalloc.argtypes = [_dims_p, _ext_p, _p, _p, _p, _p, _p, _p, _p, _p, ctypes.c_float, _p, _p,
                                          _i32, _p]
_lib.paged_decode_ext_noalloc.restype = _i32
_lib.paged_decode_partition.argtypes = [_dims_p, _ext_p, _p, _p, _p, _p, _p, _p, _p, ctypes.c_float, _i32,
                                        _p, ctypes.c_size_t, _p]
_lib.paged_decode_partition.restype = _i32
_lib.paged_decode_finish.argtypes = [_dims_p, _ext_p, _i32, _p, ctypes.c_size_t, _p, _p, _p, _p]
_lib.paged_decode_finish.restype = _i32
_lib.paged_decode_num_splits.argtypes = [_dims_p, _i32]
_lib.paged_decode_num_splits.restype = _i32
_lib.paged_decode_num_splits_ext.argtypes = [_dims_p, _ext_p, _i32]
_lib.paged_decode_num_splits_ext.restype = _i32
_lib.paged_decode_launches.argtypes = [_dims_p, _ext_p, _i32]
_lib.paged_decode_launches.restype = _i32
_lib.paged_decode_path.argtypes = [_dims_p, _ext_p, _i32]
_lib.paged_decode_path.restype = _i32
_lib.paged_decode_workspace_bytes.argtypes = [_dims_p, _i32]
_lib.paged_decode_workspace_bytes.restype = ctypes.c_size_t
_lib.paged_decode_workspace_bytes_ext.argtypes = [_dims_p, _ext_p, _i32]
_lib.paged_decode_workspace_bytes_ext.restype = ctypes.c_size_t
_lib.paged_decode_partials.argtypes = [_dims_p, _ext_p, _p, _p, _p, _p, _p, _p, _p, ctypes.c_float, _i32,
                                       _p, _p, _p]
_lib.paged_decode_partials.restype = _i32
_lib.paged_decode_merge.argtypes = [ctypes.c_int64, _i32, _i32, _p, _p, _p, _p, _p]
_lib.paged_decode_merge.restype = _i32
_lib.paged_decode_check_tables.argtypes = [_dims_p, _p, _p, _p, _p]
_lib.paged_decode_check_tables.restype = _i32
_lib.paged_kv_append.argtypes = [_dims_p, ctypes.c_int64, _p, _p, _p, _p, _p, _i32, _p, _p, _p, _p, _p]
_lib.paged_kv_append.restype = _i32
_lib.paged_decode_metadata.argtypes = [ctypes.POINTER(pkd_meta_dims)] + [_p] * 10
_lib.paged_decode_metadata.restype = _i32
_lib.contiguous_decode.argtypes = [ctypes.POINTER(pkd_contig_dims), _p, _p, _p, _p, _p, _p, _p, ctypes.c_float,
                                   _p, _p, _i32, _p, ctypes.c_size_t, _p]
_lib.contiguous_decode.restype = _i32
_lib.contiguous_decode_workspace_bytes.argtypes = [ctypes.POINTER(pkd_contig_dims), _i32]
_lib.contiguous_decode_workspace_bytes.restype = ctypes.c_size_t
_lib.pkd_decode_valu.argtypes = [_dims_p, _p, _p, _p, _p, _p, ctypes.c_float, _p, _p, _p]
_lib.pkd_decode_valu.restype = _i32
_lib.pkd_decode_lds.argtypes = [_dims_p, _p, _p, _p, _p, _p, ctypes.c_float, _p, _p, _p]
_lib.pkd_decode_lds.restype = _i32
_lib.pkd_decode_registers.argtypes = [_dims_p, _p, _p, _p, _p, _p, ctypes.c_float, _p, _p, _p]
_lib.pkd_decode_registers.restype = _i32
_lib.pkd_stream_read.argtypes = [_p, ctypes.c_int64, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _p, _p]
_lib.pkd_stream_read.restype = _i32
_lib.pkd_stream_read_sink_bytes.argtypes = [_i32, _i32]
_lib.pkd_stream_read_sink_bytes.restype = ctypes.c_size_t
_lib.paged_decode_status_string.argtypes = [_i32]
_lib.paged_decode_status_string.restype = ctypes.c_char_p


def lib() -> ctypes.CDLL:
    return _lib


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _dims_ref(dims):
    if dims is None:
        return None
    return ctypes.byref(dims)


def paged_decode(dims, q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale, scale, out, lse,
                 num_splits, workspace, workspace_bytes, stream) -> int:
    return _lib.paged_decode(_dims_ref(dims), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                             _ptr(seq_lens), _ptr(k_scale), _ptr(v_scale), float(scale), _ptr(out), _ptr(lse),
                             int(num_splits), _ptr(workspace), int(workspace_bytes), _ptr(stream))


def paged_decode_ext(dims, ext, q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale, sinks, scale, out,
                     lse, num_splits, workspace, workspace_bytes, stream) -> int:
    return _lib.paged_decode_ext(_dims_ref(dims), _dims_ref(ext), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                 _ptr(block_table), _ptr(seq_lens), _ptr(k_scale), _ptr(v_scale), _ptr(sinks),
                                 float(scale), _ptr(out), _ptr(lse), int(num_splits), _ptr(workspace),
                                 int(workspace_bytes), _ptr(stream))


def paged_decode_ext_noalloc(dims, ext, q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale, sinks, scale,
                             out, lse, num_splits, stream) -> int:
    return _lib.paged_decode_ext_noalloc(_dims_ref(dims), _dims_ref(ext), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                         _ptr(block_table), _ptr(seq_lens), _ptr(k_scale), _ptr(v_scale),
                                         _ptr(sinks), float(scale), _ptr(out), _ptr(lse), int(num_splits),
                                         _ptr(stream))


def paged_decode_partition(dims, ext, q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale, scale,
                           num_splits, workspace, workspace_bytes, stream) -> int:
    return _lib.paged_decode_partition(_dims_ref(dims), _dims_ref(ext), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                       _ptr(block_table), _ptr(seq_lens), _ptr(k_scale), _ptr(v_scale),
                                       float(scale), int(num_splits), _ptr(workspace), int(workspace_bytes),
                                       _ptr(stream))


def paged_decode_finish(dims, ext, num_splits, workspace, workspace_bytes, sinks, out, lse, stream) -> int:
    return _lib.paged_decode_finish(_dims_ref(dims), _dims_ref(ext), int(num_splits), _ptr(workspace),
                                    int(workspace_bytes), _ptr(sinks), _ptr(out), _ptr(lse), _ptr(stream))


def paged_decode_num_splits(dims, max_seq_len_hint: int = 0) -> int:
    return _lib.paged_decode_num_splits(_dims_ref(dims), int(max_seq_len_hint))


def paged_decode_num_splits_ext(dims, ext, max_seq_len_hint: int = 0) -> int:
    return _lib.paged_decode_num_splits_ext(_dims_ref(dims), _dims_ref(ext), int(max_seq_len_hint))


def paged_decode_launches(dims, ext, num_splits: int) -> int:
    return _lib.paged_decode_launches(_dims_ref(dims), _dims_ref(ext), int(num_splits))


def paged_decode_path(dims, ext, num_splits: int) -> int:
    return _lib.paged_decode_path(_dims_ref(dims), _dims_ref(ext), int(num_splits))


def paged_decode_workspace_bytes(dims, num_splits: int) -> int:
    return _lib.paged_decode_workspace_bytes(_dims_ref(dims), int(num_splits))


def paged_decode_workspace_bytes_ext(dims, ext, num_splits: int) -> int:
    return _lib.paged_decode_workspace_bytes_ext(_dims_ref(dims), _dims_ref(ext), int(num_splits))


def paged_decode_partials(dims, ext, q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale, scale,
                          num_splits, o_part, lse_part, stream) -> int:
    return _lib.paged_decode_partials(_dims_ref(dims), _dims_ref(ext), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                      _ptr(block_table), _ptr(seq_lens), _ptr(k_scale), _ptr(v_scale),
                                      float(scale), int(num_splits), _ptr(o_part), _ptr(lse_part),
                                      _ptr(stream))


def paged_decode_merge(rows, num_splits, head_dim, o_part, lse_part, out, lse, stream) -> int:
    return _lib.paged_decode_merge(int(rows), int(num_splits), int(head_dim), _ptr(o_part),
                                   _ptr(lse_part), _ptr(out), _ptr(lse), _ptr(stream))


def paged_decode_check_tables(dims, block_table, seq_lens, d_error_count, stream) -> int:
    return _lib.paged_decode_check_tables(_dims_ref(dims), _ptr(block_table), _ptr(seq_lens),
                                          _ptr(d_error_count), _ptr(stream))


def paged_kv_append(dims, num_tokens, k_new, v_new, slot_mapping, positions, cos_sin, max_position, k_cache,
                    v_cache, k_scale, v_scale, stream) -> int:
    return _lib.paged_kv_append(_dims_ref(dims), int(num_tokens), _ptr(k_new), _ptr(v_new), _ptr(slot_mapping),
                                _ptr(positions), _ptr(cos_sin), int(max_position), _ptr(k_cache), _ptr(v_cache),
                                _ptr(k_scale), _ptr(v_scale), _ptr(stream))


def paged_decode_metadata(md, req_to_token, req_pool_indices, seq_lens, cache_seqlens, cu_seqlens_k, page_table,
                          swa_seqlens, swa_page_table, d_error_count, stream) -> int:
    return _lib.paged_decode_metadata(None if md is None else ctypes.byref(md), _ptr(req_to_token),
                                      _ptr(req_pool_indices), _ptr(seq_lens), _ptr(cache_seqlens),
                                      _ptr(cu_seqlens_k), _ptr(page_table), _ptr(swa_seqlens),
                                      _ptr(swa_page_table), _ptr(d_error_count), _ptr(stream))


def contiguous_decode(cd, q, k, v, seq_lens, k_scale, v_scale, sinks, scale, out, lse, num_splits, workspace,
                      workspace_bytes, stream) -> int:
    return _lib.contiguous_decode(None if cd is None else ctypes.byref(cd), _ptr(q), _ptr(k), _ptr(v),
                                  _ptr(seq_lens), _ptr(k_scale), _ptr(v_scale), _ptr(sinks), float(scale), _ptr(out),
                                  _ptr(lse), int(num_splits), _ptr(workspace), int(workspace_bytes), _ptr(stream))


def contiguous_decode_workspace_bytes(cd, num_splits: int) -> int:
    return _lib.contiguous_decode_workspace_bytes(None if cd is None else ctypes.byref(cd), int(num_splits))


def pkd_decode_valu(dims, q, k_cache, v_cache, block_table, seq_lens, scale, out, lse, stream) -> int:
    return _lib.pkd_decode_valu(_dims_ref(dims), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                _ptr(seq_lens), float(scale), _ptr(out), _ptr(lse), _ptr(stream))


def pkd_decode_lds(dims, q, k_cache, v_cache, block_table, seq_lens, scale, out, lse, stream) -> int:
    return _lib.pkd_decode_lds(_dims_ref(dims), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                _ptr(seq_lens), float(scale), _ptr(out), _ptr(lse), _ptr(stream))


def pkd_decode_registers(dims, q, k_cache, v_cache, block_table, seq_lens, scale, out, lse, stream) -> int:
    return _lib.pkd_decode_registers(_dims_ref(dims), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                _ptr(seq_lens), float(scale), _ptr(out), _ptr(lse), _ptr(stream))


def pkd_stream_read(buf, nbytes, row_bytes, chunk_bytes, pattern, workgroups, waves, batch_kb, nontemporal, sink,
                    stream) -> int:
    return _lib.pkd_stream_read(_ptr(buf), int(nbytes), int(row_bytes), int(chunk_bytes), int(pattern),
                                int(workgroups), int(waves), int(batch_kb), int(nontemporal), _ptr(sink),
                                _ptr(stream))


def pkd_stream_read_sink_bytes(workgroups, waves) -> int:
    return _lib.pkd_stream_read_sink_bytes(int(workgroups), int(waves))


def paged_decode_status_string(status: int) -> str:
    return _lib.paged_decode_status_string(int(status)).decode()


# ---- torch conveniences (memory and streams only) ---------------------------

def dims_for(q, k_cache, block_table) -> pkd_dims:
    """pkd_dims from torch tensors q [B,Hq,D] (or [B,q_len,Hq,D]), k_cache [P,ps,Hkv,D],
    block_table [B,MP]."""
    import torch
    if q.dim() == 4:
        B, _, hq, d = q.shape
    else:
        B, hq, d = q.shape
    num_pages, ps, hkv, d2 = k_cache.shape
    if d2 != d:
        raise ValueError("q and k_cache head_dim differ")
    if k_cache.dtype == torch.bfloat16:
        kvd = PKD_DTYPE_BF16
    elif k_cache.dtype == torch.float8_e4m3fn:
        kvd = PKD_DTYPE_FP8_E4M3
    else:
        raise TypeError(f"unsupported KV-cache dtype {k_cache.dtype}")
    return pkd_dims(B, hq, hkv, d, ps, num_pages, block_table.shape[1], kvd)


def ext_for(q, causal: bool = False, window: int = 0) -> Optional[pkd_ext]:
    """pkd_ext for q [B,Hq,D] or [B,q_len,Hq,D] with the causal mask when `causal` and a
    sliding window of `window` tokens (0: none); None for plain decode."""
    q_len = q.shape[1] if q.dim() == 4 else 1
    if q_len == 1 and not causal and window == 0:
        return None
    return pkd_ext(q_len, int(bool(causal)), int(window), 0)


def current_stream_handle(device) -> int:
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def decode(q, k_cache, v_cache, block_table, seq_lens, scale: float, k_scale=None, v_scale=None,
           num_splits: int = 0, out=None, lse=None, workspace=None, stream: Optional[int] = None,
           causal: bool = False, window: int = 0, sinks=None):
    """Run the decode on torch device tensors; returns (out bf16 shaped like q, lse fp32
    [B,Hq] or [B,q_len,Hq]).  q is [B,Hq,D], or [B,q_len,Hq,D] for several query tokens
    per sequence (with the causal mask when `causal`); `window` > 0 is a sliding window
    in tokens and `sinks` an fp32 [Hq] device tensor of sink logits.  Plain decode with
    num_splits in 1..PKD_MAX_SPLITS or 0 (the heuristic) goes through paged_decode, the
    rest through paged_decode_ext."""
    import torch
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache),
                    ("block_table", block_table), ("seq_lens", seq_lens)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if q.dtype != torch.bfloat16:
        raise TypeError("q must be bfloat16")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise TypeError("block_table and seq_lens must be int32")
    if v_cache.dtype != k_cache.dtype or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must match")
    if sinks is not None and (not sinks.is_cuda or sinks.dtype != torch.float32 or sinks.numel() != q.shape[-2]):
        raise ValueError("sinks must be an fp32 device tensor of num_q_heads values")
    dims = dims_for(q, k_cache, block_table)
    ext = ext_for(q, causal, window)
    dev = q.device
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=dev)
    S = num_splits if num_splits != PKD_SPLITS_AUTO else paged_decode_num_splits_ext(dims, ext, 0)
    if -11 <= S < 0:
        raise PkdError(S)
    need = paged_decode_workspace_bytes_ext(dims, ext, S)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if stream is None:
        stream = current_stream_handle(dev)
    if ext is None and sinks is None and 1 <= S <= PKD_MAX_SPLITS:
        st = paged_decode(dims, q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale, scale, out, lse, S,
                          workspace, ws_bytes, stream)
    else:
        st = paged_decode_ext(dims, ext, q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale, sinks,
                              scale, out, lse, S, workspace, ws_bytes, stream)
    if st != PKD_OK:
        raise PkdError(st)
    return out, lse


def append(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale=None, v_scale=None, positions=None,
           cos_sin=None, stream: Optional[int] = None):
    """Run paged_kv_append on torch device tensors (k_cache / v_cache updated in place)."""
    import torch
    n, hkv, d = k_new.shape
    num_pages, ps, hkv2, d2 = k_cache.shape
    if (hkv2, d2) != (hkv, d) or v_new.shape != k_new.shape or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch between new rows and caches")
    if k_new.dtype != torch.bfloat16 or v_new.dtype != torch.bfloat16:
        raise TypeError("k_new and v_new must be bfloat16")
    kvd = PKD_DTYPE_FP8_E4M3 if k_cache.dtype == torch.float8_e4m3fn else PKD_DTYPE_BF16
    dims = pkd_dims(0, hkv, hkv, d, ps, num_pages, 1, kvd)
    max_pos = 0 if cos_sin is None else cos_sin.shape[0]
    if stream is None:
        stream = current_stream_handle(k_new.device)
    st = paged_kv_append(dims, n, k_new, v_new, slot_mapping, positions, cos_sin, max_pos, k_cache, v_cache,
                         k_scale, v_scale, stream)
    if st != PKD_OK:
        raise PkdError(st)


def metadata(req_to_token, req_pool_indices, seq_lens, page_size: int, max_pages: int, q_len: int = 1,
             window: int = 0, extend: int = 0, stream: Optional[int] = None):
    """Run paged_decode_metadata on torch device tensors (req_to_token int32 [R, C],
    req_pool_indices and seq_lens int64 [B]).  Returns a dict of device tensors:
    cache_seqlens, cu_seqlens_k, page_table and, with a window, swa_seqlens and
    swa_page_table, plus error_count (int32 [1])."""
    import torch
    for name, t, dt in (("req_to_token", req_to_token, torch.int32), ("req_pool_indices", req_pool_indices,
                        torch.int64), ("seq_lens", seq_lens, torch.int64)):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != dt:
            raise ValueError(f"{name} must be a contiguous {dt} device tensor")
    R, C = req_to_token.shape
    B = req_pool_indices.shape[0]
    dev = req_to_token.device
    res = dict(cache_seqlens=torch.empty(B, dtype=torch.int32, device=dev),
               cu_seqlens_k=torch.empty(B + 1, dtype=torch.int32, device=dev),
               page_table=torch.empty(B, max_pages, dtype=torch.int32, device=dev),
               error_count=torch.empty(1, dtype=torch.int32, device=dev))
    if window > 0:
        res["swa_seqlens"] = torch.empty(B, dtype=torch.int32, device=dev)
        res["swa_page_table"] = torch.empty(B, max_pages, dtype=torch.int32, device=dev)
    md = pkd_meta_dims(B, R, C, page_size, max_pages, q_len, window, extend)
    if stream is None:
        stream = current_stream_handle(dev)
    st = paged_decode_metadata(md, req_to_token, req_pool_indices, seq_lens, res["cache_seqlens"],
                               res["cu_seqlens_k"], res["page_table"], res.get("swa_seqlens"),
                               res.get("swa_page_table"), res["error_count"], stream)
    if st != PKD_OK:
        raise PkdError(st)
    return res


def contig_dims_for(q, k, out, causal: bool = False, window: int = 0) -> pkd_contig_dims:
    """pkd_contig_dims from torch views q and out [B, Hq, D] or [B, q_len, Hq, D] and
    k [B, L_max, Hkv, D] (any strides; the last dimension contiguous)."""
    import torch
    q4 = q if q.dim() == 4 else q.unsqueeze(1)
    o4 = out if out.dim() == 4 else out.unsqueeze(1)
    B, q_len, hq, d = q4.shape
    _, cap, hkv, d2 = k.shape
    if d2 != d or q.stride(-1) != 1 or k.stride(-1) != 1 or out.stride(-1) != 1:
        raise ValueError("head dims differ or are not contiguous")
    kvd = PKD_DTYPE_FP8_E4M3 if k.dtype == torch.float8_e4m3fn else PKD_DTYPE_BF16
    arr = ctypes.c_int64 * 3
    return pkd_contig_dims(B, hq, hkv, d, cap, kvd, q_len, int(bool(causal)), int(window), 0,
                           arr(*q4.stride()[:3]), arr(*k.stride()[:3]), arr(*o4.stride()[:3]))


def contiguous(q, k, v, seq_lens, scale: float, k_scale=None, v_scale=None, num_splits: int = 0, out=None,
               lse=None, stream: Optional[int] = None, causal: bool = False, window: int = 0, sinks=None):
    """Run contiguous_decode on torch device views q ([B, Hq, D] or [B, q_len, Hq, D]) and
    k, v ([B, L_max, Hkv, D], any strides: e.g. a permuted [B, Hkv, L_max, D] tensor).
    out defaults to a dense tensor shaped like q; returns (out, lse)."""
    import torch
    if k.stride() != v.stride() or k.shape != v.shape or k.dtype != v.dtype:
        raise ValueError("k and v must share shape, strides and dtype")
    dev = q.device
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=dev)
    cd = contig_dims_for(q, k, out, causal, window)
    need = contiguous_decode_workspace_bytes(cd, num_splits)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if stream is None:
        stream = current_stream_handle(dev)
    st = contiguous_decode(cd, q, k, v, seq_lens, k_scale, v_scale, sinks, scale, out, lse, num_splits, ws, need,
                           stream)
    if st != PKD_OK:
        raise PkdError(st)
    return out, lse
