"""Seeded synthetic inputs for paged decode attention.

This module only draws and lays out inputs; it holds none of the attention
arithmetic.  Both the GPU library's tests and the CPU oracle's tests take their
inputs from here, and nothing here imports either of them.

A workload is drawn on the CPU with one ``torch.Generator`` in a fixed order:
sequence lengths, then the physical page permutation, then q, then the logical
(per-token) K rows, then the logical V rows.  Values are N(0, 1) in float32,
rounded to bfloat16 (round-to-nearest-even).  For an FP8 cache every KV head
gets its own fp32 scale, amax / 448 over that head's values, and the values are
divided by the scale, clamped to +-448 and rounded to OCP FP8 E4M3FN
(``torch.float8_e4m3fn``).

The logical rows are then scattered into a page pool ``[num_pages, page_size,
Hkv, D]``: sequence b's i-th logical page goes to physical page
``perm[first_page_of_b + i]``.  The pool holds exactly the pages the sequences
use (sum of ceil(L_b / page_size)); slots past a sequence's length in its last
page are filled with NaN (``tail="nan"``, used by parity runs so that any read
of them shows) or zeros (``tail="zero"``).  Block-table entries past a
sequence's last page are -1.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np
import torch

FP8_E4M3_MAX = 448.0


@dataclasses.dataclass(frozen=True)
class WorkloadSpec:
    """Shape and draw recipe of one synthetic decode step."""
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    kv_dtype: str                      # "bf16" or "fp8_e4m3"
    seed: int
    seq_lens: Optional[tuple] = None   # fixed lengths, or
    len_range: Optional[tuple] = None  # inclusive uniform integer range (lo, hi)
    max_len: int = 0                   # longest length the block table must allow
    q_len: int = 1                     # query tokens per sequence (the last q_len positions)
    causal: bool = False               # query token i sees positions <= L - q_len + i only
    window: int = 0                    # > 0: query token at position p sees positions > p - window only
    sinks: bool = False                # draw a sink logit per query head (U[0, 8])

    @property
    def max_pages_per_seq(self) -> int:
        return -(-self.max_len // self.page_size)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


def _spec(name, B, hq, hkv, d, ps, dtype, seed, seq_lens=None, len_range=None, q_len=1, causal=False,
          window=0, sinks=False):
    max_len = max(seq_lens) if seq_lens is not None else len_range[1]
    return WorkloadSpec(name, B, hq, hkv, d, ps, dtype, seed,
                        tuple(seq_lens) if seq_lens is not None else None,
                        tuple(len_range) if len_range is not None else None, max_len, q_len, causal,
                        window, sinks)


# The decode shapes the method is exercised on: a tiny case, a Llama-style
# B=32 step, a B=128 step, long-context head-dim sweeps and an FP8 cache; and
# the B=32 shape verifying 4 speculative tokens per sequence under the causal
# mask (several query tokens per sequence); and the B=32 shape with a
# 1024-token sliding window and a sink logit per query head (the window size
# is a choice: the variant's source names none).
WORKLOADS = {w.name: w for w in [
    _spec("tiny_b2_d64_ps16", 2, 4, 1, 64, 16, "bf16", 1, seq_lens=(37, 100)),
    _spec("llama_b32_d128_ps64", 32, 32, 8, 128, 64, "bf16", 2, len_range=(1024, 4096)),
    _spec("batch128_d128_ps128", 128, 32, 8, 128, 128, "bf16", 3, seq_lens=(2048,) * 128),
    _spec("longctx_b1_d32", 1, 16, 2, 32, 64, "bf16", 41, seq_lens=(131072,)),
    _spec("longctx_b1_d64", 1, 16, 2, 64, 64, "bf16", 42, seq_lens=(131072,)),
    _spec("longctx_b1_d256", 1, 16, 2, 256, 64, "bf16", 43, seq_lens=(131072,)),
    _spec("longctx_b16_d32", 16, 16, 2, 32, 64, "bf16", 44, len_range=(8192, 32768)),
    _spec("longctx_b16_d64", 16, 16, 2, 64, 64, "bf16", 45, len_range=(8192, 32768)),
    _spec("longctx_b16_d256", 16, 16, 2, 256, 64, "bf16", 46, len_range=(8192, 32768)),
    _spec("fp8kv_b64_d128_ps64", 64, 64, 8, 128, 64, "fp8_e4m3", 5, len_range=(512, 8192)),
    _spec("verify_b32_q4_d128_ps64", 32, 32, 8, 128, 64, "bf16", 6, len_range=(1024, 4096),
          q_len=4, causal=True),
    _spec("window1k_sinks_b32_d128_ps64", 32, 32, 8, 128, 64, "bf16", 7, len_range=(1024, 4096),
          window=1024, sinks=True),
]}


@dataclasses.dataclass
class Workload:
    """Host (CPU) tensors of one decode step plus the logical rows they came from."""
    spec: WorkloadSpec
    seq_lens: torch.Tensor       # [B] int32
    block_table: torch.Tensor    # [B, max_pages] int32, -1 past the used pages
    num_pages: int
    q: torch.Tensor              # [B, Hq, D] bfloat16, or [B, q_len, Hq, D] when q_len > 1
    k_cache: torch.Tensor        # [num_pages, ps, Hkv, D] bfloat16 or float8_e4m3fn
    v_cache: torch.Tensor
    k_scale: Optional[torch.Tensor]  # [Hkv] float32 (fp8 only)
    v_scale: Optional[torch.Tensor]
    k_logical: torch.Tensor      # [sum L, Hkv, D] in the cache dtype, sequence-major
    v_logical: torch.Tensor
    token_offsets: torch.Tensor  # [B + 1] int64 prefix sums of seq_lens
    perm: torch.Tensor           # [num_pages] int64 physical page of each logical page
    sinks: Optional[torch.Tensor] = None  # [Hq] float32 sink logits (natural log), or None

    @property
    def scale(self) -> float:
        return self.spec.scale

    def kv_bytes(self) -> int:
        """Bytes of the K and V rows the step reads: sum_b L_b * Hkv * D * 2 * elem."""
        e = self.k_cache.element_size()
        return int(self.seq_lens.to(torch.int64).sum()) * self.spec.num_kv_heads * self.spec.head_dim * 2 * e


def _quantize_fp8_per_head(x: torch.Tensor):
    """x: [T, Hkv, D] float32 -> (codes float8_e4m3fn, scale [Hkv] float32)."""
    amax = x.abs().amax(dim=(0, 2)).to(torch.float32)
    scale = torch.where(amax > 0, amax / FP8_E4M3_MAX, torch.ones_like(amax))
    codes = (x / scale.view(1, -1, 1)).clamp(-FP8_E4M3_MAX, FP8_E4M3_MAX).to(torch.float8_e4m3fn)
    return codes, scale


def _nan_fill(dtype):
    if dtype == torch.float8_e4m3fn:
        return torch.tensor([0x7F], dtype=torch.uint8).view(torch.float8_e4m3fn)[0]
    return torch.tensor(float("nan"), dtype=dtype)


def scatter_to_pages(k_logical: torch.Tensor, v_logical: torch.Tensor, seq_lens: Sequence[int],
                     page_size: int, perm: torch.Tensor, max_pages: int, tail: str = "nan"):
    """Lay logical rows out in a page pool.

    k_logical, v_logical: [sum L, Hkv, D] rows of all sequences, sequence-major.
    perm: physical page of each logical page (a permutation of range(num_pages)).
    Returns (k_cache, v_cache, block_table).
    """
    lens = [int(x) for x in seq_lens]
    B = len(lens)
    npages = [-(-L // page_size) for L in lens]
    num_pages = sum(npages)
    assert perm.numel() == num_pages
    hkv, d = k_logical.shape[1], k_logical.shape[2]
    dtype = k_logical.dtype
    shape = (num_pages, page_size, hkv, d)
    if tail == "nan":
        fill = _nan_fill(dtype)
        k_cache = torch.empty(shape, dtype=dtype)
        v_cache = torch.empty(shape, dtype=dtype)
        if dtype == torch.float8_e4m3fn:
            k_cache.view(torch.uint8).fill_(0x7F)
            v_cache.view(torch.uint8).fill_(0x7F)
        else:
            k_cache.fill_(fill)
            v_cache.fill_(fill)
    elif tail == "zero":
        k_cache = torch.zeros(shape, dtype=dtype) if dtype != torch.float8_e4m3fn else \
            torch.zeros(shape, dtype=torch.uint8).view(torch.float8_e4m3fn)
        v_cache = k_cache.clone()
    else:
        raise ValueError(f"tail must be 'nan' or 'zero', got {tail!r}")

    block_table = torch.full((B, max_pages), -1, dtype=torch.int32)
    rows = []
    first = 0
    for b, L in enumerate(lens):
        assert npages[b] <= max_pages, "sequence longer than the block table allows"
        phys = perm[first:first + npages[b]]
        block_table[b, :npages[b]] = phys.to(torch.int32)
        t = torch.arange(L, dtype=torch.int64)
        rows.append(phys[t // page_size] * page_size + t % page_size)
        first += npages[b]
    if rows:
        rows = torch.cat(rows)
        if dtype == torch.float8_e4m3fn:
            k_cache.view(torch.uint8).view(-1, hkv, d)[rows] = k_logical.view(torch.uint8)
            v_cache.view(torch.uint8).view(-1, hkv, d)[rows] = v_logical.view(torch.uint8)
        else:
            k_cache.view(-1, hkv, d)[rows] = k_logical
            v_cache.view(-1, hkv, d)[rows] = v_logical
    return k_cache, v_cache, block_table


def draw_seq_lens(spec: WorkloadSpec, g: torch.Generator) -> torch.Tensor:
    if spec.seq_lens is not None:
        return torch.tensor(spec.seq_lens, dtype=torch.int32)
    lo, hi = spec.len_range
    lens = torch.randint(lo, hi + 1, (spec.batch,), generator=g, dtype=torch.int64)
    if spec.kv_dtype == "fp8_e4m3" and spec.batch >= 2:
        # The FP8 case must hold lengths that are and are not page multiples.
        mult = (lens % spec.page_size) == 0
        if not bool(mult.any()):
            lens[0] = max(spec.page_size, min(hi - hi % spec.page_size,
                                              int(lens[0]) - int(lens[0]) % spec.page_size))
        if bool(((lens % spec.page_size) == 0).all()):
            lens[1] = lens[1] - 1 if int(lens[1]) > lo else lens[1] + 1
    return lens.to(torch.int32)


def make_workload(spec: WorkloadSpec, tail: str = "nan",
                  seq_lens: Optional[Sequence[int]] = None) -> Workload:
    """Draw one decode step from `spec` (optionally overriding its lengths)."""
    g = torch.Generator().manual_seed(spec.seed)
    lens = torch.tensor(list(seq_lens), dtype=torch.int32) if seq_lens is not None \
        else draw_seq_lens(spec, g)
    B, hq, hkv, d, ps = spec.batch, spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.page_size
    assert lens.numel() == B
    max_pages = max(spec.max_pages_per_seq, max((-(-int(L) // ps) for L in lens), default=0), 1)
    num_pages = sum(-(-int(L) // ps) for L in lens)
    perm = torch.randperm(num_pages, generator=g)
    qshape = (B, hq, d) if spec.q_len == 1 else (B, spec.q_len, hq, d)
    q = torch.randn(*qshape, generator=g).to(torch.bfloat16)
    total = int(lens.to(torch.int64).sum())
    k32 = torch.randn(total, hkv, d, generator=g)
    v32 = torch.randn(total, hkv, d, generator=g)
    k_scale = v_scale = None
    if spec.kv_dtype == "bf16":
        k_log, v_log = k32.to(torch.bfloat16), v32.to(torch.bfloat16)
    elif spec.kv_dtype == "fp8_e4m3":
        k_log, k_scale = _quantize_fp8_per_head(k32)
        v_log, v_scale = _quantize_fp8_per_head(v32)
    else:
        raise ValueError(spec.kv_dtype)
    del k32, v32
    sinks = (torch.rand(hq, generator=g) * 8).to(torch.float32) if spec.sinks else None
    k_cache, v_cache, bt = scatter_to_pages(k_log, v_log, lens.tolist(), ps, perm, max_pages, tail)
    offs = torch.zeros(B + 1, dtype=torch.int64)
    offs[1:] = torch.cumsum(lens.to(torch.int64), 0)
    return Workload(spec, lens, bt, num_pages, q, k_cache, v_cache, k_scale, v_scale,
                    k_log, v_log, offs, perm, sinks)


def custom_workload(batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int, page_size: int,
                    seq_lens: Sequence[int], kv_dtype: str = "bf16", seed: int = 0,
                    tail: str = "nan", max_pages: Optional[int] = None, name: str = "custom",
                    q_len: int = 1, causal: bool = False, window: int = 0, sinks: bool = False) -> Workload:
    """A one-off workload with explicit lengths (edge cases, small parity cases)."""
    lens = [int(x) for x in seq_lens]
    max_len = max(lens + [1])
    if max_pages is not None:
        max_len = max(max_len, max_pages * page_size)
    spec = WorkloadSpec(name, batch, num_q_heads, num_kv_heads, head_dim, page_size, kv_dtype, seed,
                        tuple(lens), None, max_len, q_len, causal, window, sinks)
    return make_workload(spec, tail=tail)


def rebuild_with_rows(w: Workload, q: Optional[torch.Tensor] = None,
                      k_logical: Optional[torch.Tensor] = None,
                      v_logical: Optional[torch.Tensor] = None,
                      perm: Optional[torch.Tensor] = None, tail: str = "nan") -> Workload:
    """Same pages and lengths as `w`, with some of q / logical K / logical V / the
    page permutation replaced (values are used as given; the dtypes must match)."""
    q = w.q if q is None else q
    k_log = w.k_logical if k_logical is None else k_logical
    v_log = w.v_logical if v_logical is None else v_logical
    perm = w.perm if perm is None else perm
    k_cache, v_cache, bt = scatter_to_pages(k_log, v_log, w.seq_lens.tolist(), w.spec.page_size,
                                            perm, w.block_table.shape[1], tail)
    return dataclasses.replace(w, q=q, k_cache=k_cache, v_cache=v_cache, block_table=bt,
                               k_logical=k_log, v_logical=v_log, perm=perm)


def as_numpy_bits(t: torch.Tensor) -> np.ndarray:
    """Raw storage of a bf16 / fp8 tensor as a contiguous numpy integer array."""
    t = t.contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()


@dataclasses.dataclass
class AppendWorkload:
    """Host tensors of one paged KV append: new K/V rows for N tokens, where they go,
    optional RoPE inputs, and a cache pool with prior contents."""
    k_new: torch.Tensor          # [N, Hkv, D] bfloat16
    v_new: torch.Tensor
    slot_mapping: torch.Tensor   # [N] int64: page * page_size + position; -1 (padding) and past-the-pool entries
    positions: Optional[torch.Tensor]  # [N] int64 or None
    cos_sin: Optional[torch.Tensor]    # [max_position, D] float32: cos of the D/2 angles, then their sin
    k_cache: torch.Tensor        # [num_pages, ps, Hkv, D] bfloat16 or float8_e4m3fn (prior contents)
    v_cache: torch.Tensor
    k_scale: Optional[torch.Tensor]    # [Hkv] float32 (fp8)
    v_scale: Optional[torch.Tensor]


def rope_table(max_position: int, head_dim: int, base: float = 10000.0) -> torch.Tensor:
    """Standard rotary table: angle p * base^(-2i/D) for i < D/2; cos values, then sin values."""
    inv = base ** (-torch.arange(0, head_dim // 2, dtype=torch.float64) * 2.0 / head_dim)
    ang = torch.arange(max_position, dtype=torch.float64)[:, None] * inv[None, :]
    return torch.cat([torch.cos(ang), torch.sin(ang)], dim=1).to(torch.float32).contiguous()


def append_workload(n_tokens: int, num_kv_heads: int, head_dim: int, page_size: int, num_pages: int,
                    kv_dtype: str = "bf16", rope: bool = False, seed: int = 0, pad_every: int = 0,
                    scale_range=(0.002, 0.02)) -> AppendWorkload:
    """N tokens to distinct random slots of a random pool; every pad_every-th token is padding
    (slot -1) and one token (if N > 2) points past the pool.  New values are N(0, 1) * 2 in bf16;
    FP8 scales are drawn per KV head from scale_range, small enough that some values saturate."""
    g = torch.Generator().manual_seed(seed)
    capacity = num_pages * page_size
    assert n_tokens <= capacity
    slots = torch.randperm(capacity, generator=g)[:n_tokens].to(torch.int64)
    if pad_every:
        slots[::pad_every] = -1
    if n_tokens > 2:
        slots[1] = capacity + 5
    k_new = (torch.randn(n_tokens, num_kv_heads, head_dim, generator=g) * 2).to(torch.bfloat16)
    v_new = (torch.randn(n_tokens, num_kv_heads, head_dim, generator=g) * 2).to(torch.bfloat16)
    positions = cos_sin = None
    if rope:
        max_pos = 4096
        positions = torch.randint(0, max_pos, (n_tokens,), generator=g, dtype=torch.int64)
        if n_tokens > 3:
            positions[2] = max_pos + 1  # outside the table: that token writes nothing
        cos_sin = rope_table(max_pos, head_dim)
    shape = (num_pages, page_size, num_kv_heads, head_dim)
    k_scale = v_scale = None
    if kv_dtype == "bf16":
        k_cache = torch.randn(*shape, generator=g).to(torch.bfloat16)
        v_cache = torch.randn(*shape, generator=g).to(torch.bfloat16)
    else:
        lo, hi = scale_range
        k_scale = (lo + (hi - lo) * torch.rand(num_kv_heads, generator=g)).to(torch.float32)
        v_scale = (lo + (hi - lo) * torch.rand(num_kv_heads, generator=g)).to(torch.float32)
        codes = torch.randint(0, 256, shape, generator=g, dtype=torch.int32).to(torch.uint8)
        codes[(codes & 0x7F) == 0x7F] = 0  # no NaN codes among the prior contents
        k_cache = codes.view(torch.float8_e4m3fn)
        v_cache = torch.randint(0, 126, shape, generator=g, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    return AppendWorkload(k_new, v_new, slots, positions, cos_sin, k_cache, v_cache, k_scale, v_scale)


@dataclasses.dataclass
class MetadataWorkload:
    """Host tensors of one decode-metadata preparation: a runtime's token map
    holding the block tables of a decode workload in shuffled request rows."""
    req_to_token: torch.Tensor      # [req_rows, req_stride] int32 KV slots
    req_pool_indices: torch.Tensor  # [B] int64
    seq_lens: torch.Tensor          # [B] int64, before the step's `extend` tokens
    block_table: torch.Tensor       # [B, MP] int32, what the page table must come out as
    page_size: int
    max_pages: int
    extend: int


def metadata_workload(w: Workload, req_rows: int, extend: int = 1, seed: int = 0) -> MetadataWorkload:
    """The token map of decode workload w: sequence b sits in a random request
    row of a pool of req_rows rows, token t at slot bt[b][t // ps] * ps + t % ps;
    every other cell holds a random slot.  seq_lens are w's lengths minus extend
    (the step adds them back)."""
    g = torch.Generator().manual_seed(seed)
    bt = w.block_table
    B, MP = bt.shape
    ps = w.spec.page_size
    stride = MP * ps
    rt = torch.randint(0, int(w.k_cache.shape[0]) * ps, (req_rows, stride), generator=g, dtype=torch.int32)
    rows = torch.randperm(req_rows, generator=g)[:B].to(torch.int64)
    for b in range(B):
        L = int(w.seq_lens[b])
        t = torch.arange(L)
        rt[rows[b], :L] = (bt[b, t // ps].to(torch.int64) * ps + t % ps).to(torch.int32)
    lens = (w.seq_lens.to(torch.int64) - extend).clamp(min=0)
    return MetadataWorkload(rt, rows, lens, bt, ps, MP, extend)


def contiguous_kv(w: Workload, layout: str = "blhd", capacity: Optional[int] = None):
    """K and V of workload w in contiguous tensors, returned as views shaped
    [B, capacity, Hkv, D] (capacity defaults to the longest length):
      "blhd"         a dense [B, capacity, Hkv, D] tensor;
      "bhld"         a dense [B, Hkv, capacity, D] tensor, permuted;
      "blhd_padded"  a slice of a [B, capacity + 5, Hkv + 1, D] tensor.
    Token t < L_b of sequence b holds the sequence's logical row t; every other
    element (tokens past L_b, padding) is NaN, so that a read of one shows."""
    B = w.spec.batch
    hkv, d = w.spec.num_kv_heads, w.spec.head_dim
    lens = [int(x) for x in w.seq_lens]
    cap = capacity if capacity is not None else max(max(lens), 1)
    fp8 = w.k_cache.dtype == torch.float8_e4m3fn
    out = []
    for logical in (w.k_logical, w.v_logical):
        if layout == "blhd":
            shape = (B, cap, hkv, d)
        elif layout == "bhld":
            shape = (B, hkv, cap, d)
        elif layout == "blhd_padded":
            shape = (B, cap + 5, hkv + 1, d)
        else:
            raise ValueError(layout)
        if fp8:
            buf = torch.full(shape, 0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn)  # 0x7F: an E4M3FN NaN
        else:
            buf = torch.full(shape, float("nan"), dtype=logical.dtype)
        view = buf.permute(0, 2, 1, 3) if layout == "bhld" else buf[:, :cap, :hkv]
        for b in range(B):
            o = int(w.token_offsets[b])
            if lens[b]:
                if fp8:
                    view.view(torch.uint8)[b, :lens[b]] = logical[o:o + lens[b]].view(torch.uint8)
                else:
                    view[b, :lens[b]] = logical[o:o + lens[b]]
        out.append(view)
    return out[0], out[1]


def strided_q(q: torch.Tensor) -> torch.Tensor:
    """q ([B, Hq, D] or [B, q_len, Hq, D]) copied into a slice of a larger NaN-filled
    tensor (two extra heads, one extra query token), so its strides are not dense."""
    q4 = q if q.dim() == 4 else q.unsqueeze(1)
    B, ql, hq, d = q4.shape
    buf = torch.full((B, ql + 1, hq + 2, d), float("nan"), dtype=q.dtype)
    view = buf[:, :ql, 1:hq + 1]
    view.copy_(q4)
    return view if q.dim() == 4 else view[:, 0]
