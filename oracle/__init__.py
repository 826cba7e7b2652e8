"""fp64 CPU oracle for paged decode attention (ctypes wrapper over paged_attention_ref.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may use this package; the GPU library never does.  It imports
nothing from the library.  Inputs are host arrays (numpy, or CPU torch tensors
whose raw storage is read): q as bf16, K/V caches as bf16 or FP8 E4M3FN codes.

Every function computes the plain definition written out in
paged_attention_ref.c (scaled dot-product attention of one query token per
sequence over the K/V rows its block table points to; natural-log LSE).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_lib = None

_c_int = ctypes.c_int
_c_double = ctypes.c_double
_p = ctypes.c_void_p

_STATUS = {0: "ok", -1: "bad argument", -2: "block-table entry outside the page pool",
           -3: "sequence length outside [0, max_pages * page_size]", -4: "out of memory"}


def lib():
    """The loaded oracle library.  PKD_ORACLE_LIB, when set, names another build of
    paged_attention_ref.c to load instead (the mutation tests point it at copies
    with planted mistakes); otherwise the in-tree build is used, built on demand."""
    global _lib
    if _lib is None:
        path = os.environ.get("PKD_ORACLE_LIB")
        if not path:
            path = _build.LIB
            if not os.path.exists(path):
                _build.build()
        L = ctypes.CDLL(path)
        common = [_c_int] * 8 + [_p] * 7 + [_c_double]
        L.pkd_oracle_paged_decode.argtypes = common + [_p, _p, _c_int]
        L.pkd_oracle_paged_decode.restype = _c_int
        L.pkd_oracle_paged_decode_split.argtypes = common + [_c_int, _p, _p, _c_int]
        L.pkd_oracle_paged_decode_split.restype = _c_int
        L.pkd_oracle_paged_decode_rows.argtypes = common + [_c_int, _p, _p, _p]
        L.pkd_oracle_paged_decode_rows.restype = _c_int
        L.pkd_oracle_paged_decode_ranges.argtypes = common + [_p, _p, _p, _p]
        L.pkd_oracle_paged_decode_ranges.restype = _c_int
        multi = [_c_int] * 10 + [_p] * 7 + [_c_double]
        L.pkd_oracle_paged_decode_multi.argtypes = multi + [_p, _p, _c_int]
        L.pkd_oracle_paged_decode_multi.restype = _c_int
        L.pkd_oracle_paged_decode_multi_rows.argtypes = multi + [_c_int, _p, _p, _p]
        L.pkd_oracle_paged_decode_multi_rows.restype = _c_int
        ext = [_c_int] * 11 + [_p] * 8 + [_c_double]
        L.pkd_oracle_paged_decode_ext.argtypes = ext + [_p, _p, _c_int]
        L.pkd_oracle_paged_decode_ext.restype = _c_int
        L.pkd_oracle_paged_decode_ext_rows.argtypes = ext + [_c_int, _p, _p, _p]
        L.pkd_oracle_paged_decode_ext_rows.restype = _c_int
        L.pkd_oracle_lse_merge.argtypes = [ctypes.c_int64, _c_int, _c_int, _p, _p, _p, _p]
        L.pkd_oracle_lse_merge.restype = None
        L.pkd_oracle_bf16_value.argtypes = [ctypes.c_uint16]
        L.pkd_oracle_bf16_value.restype = _c_double
        L.pkd_oracle_fp8e4m3_value.argtypes = [ctypes.c_uint8]
        L.pkd_oracle_fp8e4m3_value.restype = _c_double
        L.pkd_oracle_fp8e4m3_encode.argtypes = [ctypes.c_float]
        L.pkd_oracle_fp8e4m3_encode.restype = ctypes.c_uint8
        L.pkd_oracle_bf16_round.argtypes = [ctypes.c_float]
        L.pkd_oracle_bf16_round.restype = ctypes.c_uint16
        L.pkd_oracle_kv_append.argtypes = [_c_int] * 5 + [ctypes.c_int64] + [_p] * 5 + [_c_int] + [_p] * 4
        L.pkd_oracle_kv_append.restype = _c_int
        L.pkd_oracle_decode_metadata.argtypes = [_c_int] * 8 + [_p] * 8
        L.pkd_oracle_decode_metadata.restype = _c_int
        L.pkd_oracle_contiguous_decode.argtypes = [_c_int] * 9 + [_p] * 9 + [_c_double, _p, _p, _c_int]
        L.pkd_oracle_contiguous_decode.restype = _c_int
        _lib = L
    return _lib


def _raw(x, dtype):
    """Contiguous numpy view of x's raw storage, reinterpreted as `dtype`."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor on the CPU
        x = x.detach().contiguous()
        import torch
        if x.dtype in (torch.bfloat16, torch.float16):
            x = x.view(torch.int16)
        elif x.dtype == torch.float8_e4m3fn:
            x = x.view(torch.uint8)
        x = x.numpy()
    x = np.ascontiguousarray(x)
    if x.dtype.itemsize != np.dtype(dtype).itemsize:
        raise TypeError(f"expected {np.dtype(dtype)} storage, got {x.dtype}")
    return x.view(dtype)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_p)


def _check(st):
    if st != 0:
        raise ValueError(f"oracle: {_STATUS.get(st, st)}")


class _Args:
    def __init__(self, q, k_cache, v_cache, block_table, seq_lens, scale, k_scale=None, v_scale=None,
                 kv_fp8=None):
        self.q = _raw(q, np.uint16)
        if self.q.ndim == 4:  # [B][q_len][Hq][D]: several query tokens per sequence
            B, self.q_len, hq, d = self.q.shape
        else:
            B, hq, d = self.q.shape
            self.q_len = 1
        kv_fp8 = (np.asarray(k_cache).dtype.itemsize == 1 if not hasattr(k_cache, "element_size")
                  else k_cache.element_size() == 1) if kv_fp8 is None else kv_fp8
        self.fp8 = bool(kv_fp8)
        self.k = _raw(k_cache, np.uint8 if self.fp8 else np.uint16)
        self.v = _raw(v_cache, np.uint8 if self.fp8 else np.uint16)
        num_pages, ps, hkv, d2 = self.k.shape
        assert d2 == d and self.v.shape == self.k.shape
        self.bt = _raw(block_table, np.int32)
        self.lens = _raw(seq_lens, np.int32)
        assert self.bt.shape[0] == B and self.lens.shape == (B,)
        self.ks = _raw(k_scale, np.float32)
        self.vs = _raw(v_scale, np.float32)
        self.dims = (B, hq, hkv, d, ps, num_pages, self.bt.shape[1], 1 if self.fp8 else 0)
        self.scale = float(scale)

    def head(self):
        assert self.q_len == 1, "single-token entry points take q as [B][Hq][D]"
        return list(self.dims) + [_ptr(self.q), _ptr(self.k), _ptr(self.v), _ptr(self.bt),
                                  _ptr(self.lens), _ptr(self.ks), _ptr(self.vs), self.scale]

    def head_ext(self, causal, window, sinks):
        self.sinks = _raw(sinks, np.float32)
        return list(self.dims) + [self.q_len, int(bool(causal)), int(window), _ptr(self.sinks)] + [
            _ptr(self.q), _ptr(self.k), _ptr(self.v), _ptr(self.bt), _ptr(self.lens), _ptr(self.ks),
            _ptr(self.vs), self.scale]

    def head_multi(self, causal):
        return list(self.dims) + [self.q_len, int(bool(causal))] + [
            _ptr(self.q), _ptr(self.k), _ptr(self.v), _ptr(self.bt), _ptr(self.lens), _ptr(self.ks),
            _ptr(self.vs), self.scale]


def paged_decode(q, k_cache, v_cache, block_table, seq_lens, scale, k_scale=None, v_scale=None,
                 nthreads: int = 1):
    """Plain definition.  Returns (out [B,Hq,D] float64, lse [B,Hq] float64)."""
    a = _Args(q, k_cache, v_cache, block_table, seq_lens, scale, k_scale, v_scale)
    B, hq, _, d = a.dims[:4]
    out = np.empty((B, hq, d), np.float64)
    lse = np.empty((B, hq), np.float64)
    _check(lib().pkd_oracle_paged_decode(*a.head(), _ptr(out), _ptr(lse), int(nthreads)))
    return out, lse


def paged_decode_split(q, k_cache, v_cache, block_table, seq_lens, scale, num_splits,
                       k_scale=None, v_scale=None, nthreads: int = 1):
    """Split form: ceil(L/S)-token ranges recombined by the LSE merge."""
    a = _Args(q, k_cache, v_cache, block_table, seq_lens, scale, k_scale, v_scale)
    B, hq, _, d = a.dims[:4]
    out = np.empty((B, hq, d), np.float64)
    lse = np.empty((B, hq), np.float64)
    _check(lib().pkd_oracle_paged_decode_split(*a.head(), int(num_splits), _ptr(out), _ptr(lse),
                                               int(nthreads)))
    return out, lse


def paged_decode_rows(q, k_cache, v_cache, block_table, seq_lens, scale, rows,
                      k_scale=None, v_scale=None):
    """Plain definition for rows = b * Hq + h only.  Returns (out [n, D], lse [n])."""
    a = _Args(q, k_cache, v_cache, block_table, seq_lens, scale, k_scale, v_scale)
    d = a.dims[3]
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    out = np.empty((rows.size, d), np.float64)
    lse = np.empty((rows.size,), np.float64)
    _check(lib().pkd_oracle_paged_decode_rows(*a.head(), int(rows.size), _ptr(rows), _ptr(out),
                                              _ptr(lse)))
    return out, lse


def paged_decode_ranges(q, k_cache, v_cache, block_table, seq_lens, scale, t_begin, t_end,
                        k_scale=None, v_scale=None):
    """Plain definition over tokens [t_begin[b], t_end[b]) of each sequence."""
    a = _Args(q, k_cache, v_cache, block_table, seq_lens, scale, k_scale, v_scale)
    B, hq, _, d = a.dims[:4]
    tb = np.ascontiguousarray(np.asarray(t_begin, dtype=np.int32))
    te = np.ascontiguousarray(np.asarray(t_end, dtype=np.int32))
    assert tb.shape == (B,) and te.shape == (B,)
    out = np.empty((B, hq, d), np.float64)
    lse = np.empty((B, hq), np.float64)
    _check(lib().pkd_oracle_paged_decode_ranges(*a.head(), _ptr(tb), _ptr(te), _ptr(out), _ptr(lse)))
    return out, lse


def paged_decode_multi(q, k_cache, v_cache, block_table, seq_lens, scale, causal, k_scale=None,
                       v_scale=None, nthreads: int = 1):
    """Several query tokens per sequence: q [B, q_len, Hq, D]; query token i is at
    position L - q_len + i and, with causal, sees tokens up to that position only.
    Returns (out [B, q_len, Hq, D] float64, lse [B, q_len, Hq] float64)."""
    a = _Args(q, k_cache, v_cache, block_table, seq_lens, scale, k_scale, v_scale)
    B, hq, _, d = a.dims[:4]
    out = np.empty((B, a.q_len, hq, d), np.float64)
    lse = np.empty((B, a.q_len, hq), np.float64)
    _check(lib().pkd_oracle_paged_decode_multi(*a.head_multi(causal), _ptr(out), _ptr(lse), int(nthreads)))
    return out, lse


def paged_decode_multi_rows(q, k_cache, v_cache, block_table, seq_lens, scale, causal, rows,
                            k_scale=None, v_scale=None):
    """paged_decode_multi for rows = (b * q_len + i) * Hq + h only.  Returns (out [n, D], lse [n])."""
    a = _Args(q, k_cache, v_cache, block_table, seq_lens, scale, k_scale, v_scale)
    d = a.dims[3]
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    out = np.empty((rows.size, d), np.float64)
    lse = np.empty((rows.size,), np.float64)
    _check(lib().pkd_oracle_paged_decode_multi_rows(*a.head_multi(causal), int(rows.size), _ptr(rows),
                                                    _ptr(out), _ptr(lse)))
    return out, lse


def paged_decode_ext(q, k_cache, v_cache, block_table, seq_lens, scale, causal=False, window=0, sinks=None,
                     k_scale=None, v_scale=None, nthreads: int = 1):
    """Several query tokens with causal mask, sliding window and sinks (see
    paged_attention_ref.c).  q [B, Hq, D] or [B, q_len, Hq, D]; sinks float32 [Hq] or None.
    Returns (out [B, q_len, Hq, D], lse [B, q_len, Hq]) as float64."""
    a = _Args(q, k_cache, v_cache, block_table, seq_lens, scale, k_scale, v_scale)
    B, hq, _, d = a.dims[:4]
    out = np.empty((B, a.q_len, hq, d), np.float64)
    lse = np.empty((B, a.q_len, hq), np.float64)
    _check(lib().pkd_oracle_paged_decode_ext(*a.head_ext(causal, window, sinks), _ptr(out), _ptr(lse),
                                             int(nthreads)))
    return out, lse


def paged_decode_ext_rows(q, k_cache, v_cache, block_table, seq_lens, scale, rows, causal=False, window=0,
                          sinks=None, k_scale=None, v_scale=None):
    """paged_decode_ext for rows = (b * q_len + i) * Hq + h only.  Returns (out [n, D], lse [n])."""
    a = _Args(q, k_cache, v_cache, block_table, seq_lens, scale, k_scale, v_scale)
    d = a.dims[3]
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    out = np.empty((rows.size, d), np.float64)
    lse = np.empty((rows.size,), np.float64)
    _check(lib().pkd_oracle_paged_decode_ext_rows(*a.head_ext(causal, window, sinks), int(rows.size), _ptr(rows),
                                                  _ptr(out), _ptr(lse)))
    return out, lse


def lse_merge(o_part, lse_part):
    """o_part [R, S, D], lse_part [R, S] (float64) -> (out [R, D], lse [R])."""
    o = np.ascontiguousarray(o_part, dtype=np.float64)
    l = np.ascontiguousarray(lse_part, dtype=np.float64)
    R, S, D = o.shape
    assert l.shape == (R, S)
    out = np.empty((R, D), np.float64)
    lse = np.empty((R,), np.float64)
    lib().pkd_oracle_lse_merge(R, S, D, _ptr(o), _ptr(l), _ptr(out), _ptr(lse))
    return out, lse


def fp8e4m3_encode(x: float) -> int:
    """E4M3FN code of an fp32 value within [-448, 448]: nearest, ties to the even code."""
    return int(lib().pkd_oracle_fp8e4m3_encode(float(x)))


def bf16_round(x: float) -> int:
    """bf16 bits of an fp32 value, round to nearest even."""
    return int(lib().pkd_oracle_bf16_round(float(x)))


def kv_append(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale=None, v_scale=None, positions=None,
              cos_sin=None):
    """Paged KV append (see paged_attention_ref.c).  k_new, v_new: bf16 [N, Hkv, D];
    slot_mapping: int64 [N]; k_cache, v_cache: [num_pages, ps, Hkv, D] bf16 or float8_e4m3fn
    (not modified); optional RoPE: positions int64 [N] and cos_sin float32 [max_position, D].
    Returns the updated caches as raw numpy arrays (uint16 bf16 bits or uint8 FP8 codes)."""
    kv_fp8 = (k_cache.element_size() if hasattr(k_cache, "element_size") else np.asarray(k_cache).dtype.itemsize) == 1
    kn = _raw(k_new, np.uint16)
    vn = _raw(v_new, np.uint16)
    n, hkv, d = kn.shape
    assert vn.shape == kn.shape
    kc = _raw(k_cache, np.uint8 if kv_fp8 else np.uint16).copy()
    vc = _raw(v_cache, np.uint8 if kv_fp8 else np.uint16).copy()
    num_pages, ps, hkv2, d2 = kc.shape
    assert (hkv2, d2) == (hkv, d) and vc.shape == kc.shape
    sm = _raw(slot_mapping, np.int64)
    pos = None if positions is None else _raw(positions, np.int64)
    cs = None if cos_sin is None else _raw(cos_sin, np.float32)
    max_pos = 0 if cs is None else cs.shape[0]
    ks = _raw(k_scale, np.float32)
    vs = _raw(v_scale, np.float32)
    _check(lib().pkd_oracle_kv_append(hkv, d, ps, num_pages, 1 if kv_fp8 else 0, n, _ptr(kn), _ptr(vn), _ptr(sm),
                                      _ptr(pos), _ptr(cs), max_pos, _ptr(kc), _ptr(vc), _ptr(ks), _ptr(vs)))
    return kc, vc


def decode_metadata(req_to_token, req_pool_indices, seq_lens, page_size, max_pages, q_len=1, window=0,
                    extend=0):
    """Decode metadata preparation (see paged_attention_ref.c).  req_to_token int32
    [req_rows, req_stride]; req_pool_indices, seq_lens int64 [B].  Returns (dict of numpy
    arrays cache_seqlens [B], cu_seqlens_k [B + 1], page_table [B, max_pages] and, with a
    window, swa_seqlens [B], swa_page_table [B, max_pages]; count of invalid entries)."""
    rt = np.ascontiguousarray(_raw(req_to_token, np.int32))
    rp = np.ascontiguousarray(_raw(req_pool_indices, np.int64))
    sl = np.ascontiguousarray(_raw(seq_lens, np.int64))
    R, C = rt.shape
    B = rp.shape[0]
    assert sl.shape == (B,)
    res = dict(cache_seqlens=np.empty(B, np.int32), cu_seqlens_k=np.empty(B + 1, np.int32),
               page_table=np.empty((B, max_pages), np.int32))
    if window > 0:
        res["swa_seqlens"] = np.empty(B, np.int32)
        res["swa_page_table"] = np.empty((B, max_pages), np.int32)
    bad = lib().pkd_oracle_decode_metadata(B, R, C, int(page_size), int(max_pages), int(q_len), int(window),
                                           int(extend), _ptr(rt), _ptr(rp), _ptr(sl), _ptr(res["cache_seqlens"]),
                                           _ptr(res["cu_seqlens_k"]), _ptr(res["page_table"]),
                                           _ptr(res.get("swa_seqlens")), _ptr(res.get("swa_page_table")))
    _check(min(bad, 0))
    return res, bad


def _strided(x, dtype):
    """(numpy array over x's whole storage as raw `dtype`, element offset of x, x's strides)
    for a CPU torch tensor view whose last dimension is contiguous."""
    import torch
    assert x.stride(-1) == 1, "the head dimension must be contiguous"
    flat = torch.empty(0, dtype=x.dtype).set_(x.untyped_storage())
    return _raw(flat, dtype), x.storage_offset(), x.stride()


def contiguous_decode(q, k_cache, v_cache, seq_lens, scale, causal=False, window=0, sinks=None, k_scale=None,
                      v_scale=None, nthreads: int = 1):
    """Decode over contiguous, strided K/V (see paged_attention_ref.c).  k_cache, v_cache:
    CPU tensor views shaped [B, L_max, Hkv, D] with any strides (the last one 1), e.g. a
    permuted [B, Hkv, L_max, D] tensor or a slice of a larger one; q a view shaped
    [B, Hq, D] or [B, q_len, Hq, D], also any strides.  Returns (out [B, q_len, Hq, D],
    lse [B, q_len, Hq]) as float64."""
    kv_fp8 = k_cache.element_size() == 1
    kt = np.uint8 if kv_fp8 else np.uint16
    kb, ko, ks_ = _strided(k_cache, kt)
    vb, vo, vs_ = _strided(v_cache, kt)
    assert ks_ == vs_ and k_cache.shape == v_cache.shape, "k and v must share shape and strides"
    q4 = q if q.dim() == 4 else q.unsqueeze(1)
    qb, qo, qs_ = _strided(q4, np.uint16)
    B, q_len, hq, d = q4.shape
    _, max_len, hkv, d2 = k_cache.shape
    assert d2 == d
    kv_str = np.array([ks_[0], ks_[1], ks_[2]], np.int64)
    q_str = np.array([qs_[0], qs_[1], qs_[2]], np.int64)
    lens = np.ascontiguousarray(_raw(seq_lens, np.int32))
    sk = None if sinks is None else np.ascontiguousarray(_raw(sinks, np.float32))
    ksc = _raw(k_scale, np.float32)
    vsc = _raw(v_scale, np.float32)
    out = np.empty((B, q_len, hq, d), np.float64)
    lse = np.empty((B, q_len, hq), np.float64)
    at = lambda a, off: ctypes.c_void_p(a.ctypes.data + off * a.itemsize)
    _check(lib().pkd_oracle_contiguous_decode(B, hq, hkv, d, max_len, 1 if kv_fp8 else 0, q_len, int(bool(causal)),
                                              int(window), _ptr(sk), at(qb, qo), _ptr(q_str), at(kb, ko), at(vb, vo),
                                              _ptr(kv_str), _ptr(lens), _ptr(ksc), _ptr(vsc), float(scale),
                                              _ptr(out), _ptr(lse), int(nthreads)))
    return out, lse


def bf16_value(bits: int) -> float:
    return lib().pkd_oracle_bf16_value(int(bits) & 0xFFFF)


def fp8e4m3_value(code: int) -> float:
    return lib().pkd_oracle_fp8e4m3_value(int(code) & 0xFF)


def run_workload(w, nthreads: int = 1, num_splits: int = 0):
    """Oracle over a drawn workload object (q, k_cache, v_cache, block_table,
    seq_lens, scale, k_scale, v_scale attributes)."""
    args = (w.q, w.k_cache, w.v_cache, w.block_table, w.seq_lens, w.scale)
    if getattr(w.spec, "window", 0) or getattr(w, "sinks", None) is not None:
        assert not num_splits
        return paged_decode_ext(*args, w.spec.causal, w.spec.window, w.sinks, w.k_scale, w.v_scale, nthreads)
    if getattr(w.spec, "q_len", 1) > 1 or getattr(w.spec, "causal", False):
        assert not num_splits
        return paged_decode_multi(*args, w.spec.causal, w.k_scale, w.v_scale, nthreads)
    if num_splits:
        return paged_decode_split(*args, num_splits, w.k_scale, w.v_scale, nthreads)
    return paged_decode(*args, w.k_scale, w.v_scale, nthreads)
