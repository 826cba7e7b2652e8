"""Pins of the fp64 oracle to things other than itself (CPU only).

The pages print no worked example, so every pin is a brute-force library
computation, a closed form, an invariant or a special case that the definition
of paged decode attention fixes.  Each is chosen so that a plausible slip in the
oracle (a dropped term, a wrong sign, a wrong page/slot index, a transposed
operand, the wrong KV head for a query head, a base-2 LSE) fails one of them.
"""
import dataclasses
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from paged_kv_decode_amd import workloads as wl


def _f64(t):
    return t.to(torch.float64).numpy() if t.dtype != torch.float8_e4m3fn else t.to(torch.float32).to(torch.float64).numpy()


def brute_force(w):
    """Dense attention over the logical (pre-scatter) rows with scipy's softmax and
    logsumexp; never sees the page pool or the block table."""
    B, hq, d = w.q.shape
    hkv = w.spec.num_kv_heads
    G = hq // hkv
    q = _f64(w.q)
    K = _f64(w.k_logical)
    V = _f64(w.v_logical)
    if w.k_scale is not None:
        K = K * w.k_scale.double().numpy()[None, :, None]
        V = V * w.v_scale.double().numpy()[None, :, None]
    out = np.zeros((B, hq, d))
    lse = np.full((B, hq), -np.inf)
    for b in range(B):
        t0, t1 = int(w.token_offsets[b]), int(w.token_offsets[b + 1])
        if t1 == t0:
            continue
        for h in range(hq):
            g = h // G
            s = w.scale * (K[t0:t1, g, :] @ q[b, h])
            out[b, h] = scipy.special.softmax(s) @ V[t0:t1, g, :]
            lse[b, h] = scipy.special.logsumexp(s)
    return out, lse


def _close(a, b, tol):
    a, b = np.asarray(a), np.asarray(b)
    both_inf = np.isneginf(a) & np.isneginf(b)
    with np.errstate(invalid="ignore"):
        diff = np.where(both_inf, 0.0, np.abs(a - b))
    return bool(np.all(diff <= tol * (1.0 + np.abs(np.where(both_inf, 0.0, b)))))


SMALL_CASES = [
    # (B, Hq, Hkv, D, ps, seq_lens, dtype, seed)
    (1, 1, 1, 8, 1, [5], "bf16", 11),
    (2, 4, 2, 16, 3, [7, 50], "bf16", 12),
    (3, 4, 1, 32, 16, [1, 33, 48], "bf16", 13),
    (3, 8, 4, 16, 3, [49, 2, 17], "bf16", 14),
    (2, 4, 4, 8, 16, [16, 31], "bf16", 15),
    (2, 4, 2, 16, 3, [20, 45], "fp8_e4m3", 16),
    (3, 4, 1, 32, 16, [9, 50, 16], "fp8_e4m3", 17),
]


@pytest.mark.parametrize("case", SMALL_CASES)
def test_p1_matches_dense_brute_force(case):
    B, hq, hkv, d, ps, lens, dtype, seed = case
    w = wl.custom_workload(B, hq, hkv, d, ps, lens, dtype, seed)
    out, lse = oracle.run_workload(w)
    ref_out, ref_lse = brute_force(w)
    assert _close(out, ref_out, 1e-12)
    assert _close(lse, ref_lse, 1e-12)


def test_p1_tiny_named_workload():
    w = wl.make_workload(wl.WORKLOADS["tiny_b2_d64_ps16"])
    assert w.num_pages == 10 and w.block_table.shape == (2, 7)
    assert sorted(w.block_table[w.block_table >= 0].tolist()) == list(range(10))
    out, lse = oracle.run_workload(w)
    ref_out, ref_lse = brute_force(w)
    assert _close(out, ref_out, 1e-12) and _close(lse, ref_lse, 1e-12)


def test_closed_form_two_tokens():
    """q = (1, 0), k0 = (0, 0), k1 = (2, 0), scale 1/2: s = (0, 1); with v0 = (1, 0)
    and v1 = (0, 1), out = (1, e) / (1 + e) and lse = ln(1 + e)."""
    w = wl.custom_workload(1, 1, 1, 2, 1, [2], "bf16", 0)
    bf = torch.bfloat16
    q = torch.tensor([[[1.0, 0.0]]], dtype=bf)
    K = torch.tensor([[[0.0, 0.0]], [[2.0, 0.0]]], dtype=bf)
    V = torch.tensor([[[1.0, 0.0]], [[0.0, 1.0]]], dtype=bf)
    w = wl.rebuild_with_rows(w, q=q, k_logical=K, v_logical=V)
    out, lse = oracle.paged_decode(w.q, w.k_cache, w.v_cache, w.block_table, w.seq_lens, 0.5)
    e = math.e
    assert abs(out[0, 0, 0] - 1 / (1 + e)) < 1e-15
    assert abs(out[0, 0, 1] - e / (1 + e)) < 1e-15
    assert abs(lse[0, 0] - math.log1p(e)) < 1e-15


@pytest.mark.parametrize("dtype", ["bf16", "fp8_e4m3"])
def test_p2_single_token_returns_its_value_row(dtype):
    w = wl.custom_workload(3, 8, 2, 32, 16, [1, 1, 1], dtype, 21)
    out, lse = oracle.run_workload(w)
    V = _f64(w.v_logical)
    K = _f64(w.k_logical)
    if w.v_scale is not None:
        V = V * w.v_scale.double().numpy()[None, :, None]
        K = K * w.k_scale.double().numpy()[None, :, None]
    q = _f64(w.q)
    for b in range(3):
        for h in range(8):
            g = h // 4
            assert np.array_equal(out[b, h], V[b, g])  # exp(0)/1 * v0
            s = w.scale * float(np.dot(q[b, h], K[b, g]))
            assert abs(lse[b, h] - s) <= 1e-13 * (1 + abs(s))


def test_p3_constant_values_return_the_constant():
    w = wl.custom_workload(2, 4, 2, 16, 3, [40, 13], "bf16", 31)
    V = torch.full_like(w.v_logical, 0.7109375)  # exactly representable in bf16
    w = wl.rebuild_with_rows(w, v_logical=V)
    out, _ = oracle.run_workload(w)
    assert np.max(np.abs(out - 0.7109375)) <= 1e-15


def test_p4_zero_query_gives_mean_and_log_length():
    w = wl.custom_workload(2, 4, 1, 16, 16, [37, 100], "bf16", 41)
    w = wl.rebuild_with_rows(w, q=torch.zeros_like(w.q))
    out, lse = oracle.run_workload(w)
    V = _f64(w.v_logical)
    for b in range(2):
        t0, t1 = int(w.token_offsets[b]), int(w.token_offsets[b + 1])
        mean = V[t0:t1, 0, :].mean(axis=0)
        for h in range(4):
            assert np.max(np.abs(out[b, h] - mean)) <= 1e-13
            assert abs(lse[b, h] - math.log(t1 - t0)) <= 1e-13


def test_p5_identical_keys_give_dot_plus_log_length():
    w = wl.custom_workload(2, 4, 2, 16, 3, [25, 8], "bf16", 51)
    K = w.k_logical.clone()
    K[:] = K[0:1]
    w = wl.rebuild_with_rows(w, k_logical=K)
    out, lse = oracle.run_workload(w)
    q = _f64(w.q)
    k = _f64(K[0])
    for b in range(2):
        L = int(w.seq_lens[b])
        for h in range(4):
            s = w.scale * float(np.dot(q[b, h], k[h // 2]))
            assert abs(lse[b, h] - (s + math.log(L))) <= 1e-12 * (1 + abs(s))


@pytest.mark.parametrize("dtype", ["bf16", "fp8_e4m3"])
def test_p6_page_permutation_invariance_is_bitwise(dtype):
    w = wl.custom_workload(3, 8, 2, 32, 4, [29, 64, 3], dtype, 61)
    out1, lse1 = oracle.run_workload(w)
    g = torch.Generator().manual_seed(999)
    perm2 = torch.randperm(w.num_pages, generator=g)
    assert not torch.equal(perm2, w.perm)
    w2 = wl.rebuild_with_rows(w, perm=perm2)
    assert not torch.equal(w2.block_table, w.block_table)
    out2, lse2 = oracle.run_workload(w2)
    assert np.array_equal(out1, out2) and np.array_equal(lse1, lse2)


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 64])
def test_p7_split_count_invariance(splits):
    w = wl.custom_workload(3, 8, 2, 16, 5, [37, 6, 51], "bf16", 71)
    out, lse = oracle.run_workload(w)
    out_s, lse_s = oracle.run_workload(w, num_splits=splits)
    assert _close(out_s, out, 1e-12) and _close(lse_s, lse, 1e-12)


def test_p8_gqa_mapping_consecutive_heads_share_a_kv_head():
    B, hq, hkv = 2, 8, 4  # G = 2: heads 0,1 -> kv 0; 2,3 -> kv 1; ...
    w = wl.custom_workload(B, hq, hkv, 16, 4, [10, 19], "bf16", 81)
    consts = torch.tensor([0.5, -1.25, 2.0, 3.5], dtype=torch.bfloat16)
    V = consts.view(1, hkv, 1).expand_as(w.v_logical).contiguous()
    w = wl.rebuild_with_rows(w, v_logical=V)
    out, _ = oracle.run_workload(w)
    for h in range(hq):
        assert np.max(np.abs(out[:, h, :] - float(consts[h // 2]))) <= 1e-15


def test_zero_length_sequence_gives_zero_and_minus_inf():
    w = wl.custom_workload(3, 4, 2, 16, 4, [0, 9, 0], "bf16", 91)
    out, lse = oracle.run_workload(w)
    assert np.all(out[0] == 0) and np.all(out[2] == 0)
    assert np.all(np.isneginf(lse[0])) and np.all(np.isneginf(lse[2]))
    assert np.all(np.isfinite(lse[1]))
    out_s, lse_s = oracle.run_workload(w, num_splits=3)
    assert _close(out_s, out, 1e-12) and _close(lse_s, lse, 1e-12)


def test_thread_count_does_not_change_bits():
    w = wl.custom_workload(4, 8, 2, 32, 16, [100, 3, 77, 64], "bf16", 95)
    a = oracle.run_workload(w, nthreads=1)
    b = oracle.run_workload(w, nthreads=5)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_rows_entry_matches_full_oracle():
    w = wl.custom_workload(3, 8, 2, 32, 16, [40, 3, 77], "fp8_e4m3", 96)
    out, lse = oracle.run_workload(w)
    rows = [0, 5, 9, 23, 17]
    o_r, l_r = oracle.paged_decode_rows(w.q, w.k_cache, w.v_cache, w.block_table, w.seq_lens,
                                        w.scale, rows, w.k_scale, w.v_scale)
    flat_o, flat_l = out.reshape(-1, 32), lse.reshape(-1)
    assert np.array_equal(o_r, flat_o[rows]) and np.array_equal(l_r, flat_l[rows])


def test_nan_tail_slots_are_never_read():
    """Parity inputs poison every slot past L; the oracle output stays finite."""
    w = wl.custom_workload(2, 4, 1, 16, 16, [5, 17], "bf16", 97)
    assert torch.isnan(w.k_cache.float()).any()
    out, lse = oracle.run_workload(w)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))


def test_bad_block_table_entry_is_reported():
    w = wl.custom_workload(1, 2, 1, 8, 4, [9], "bf16", 98)
    bt = w.block_table.clone()
    bt[0, 2] = w.num_pages  # outside the pool
    with pytest.raises(ValueError):
        oracle.paged_decode(w.q, w.k_cache, w.v_cache, bt, w.seq_lens, w.scale)


# ---- the log-sum-exp merge ------------------------------------------------

def test_merge_matches_logsumexp_weighting():
    rng = np.random.default_rng(5)
    R, S, D = 7, 5, 12
    o = rng.standard_normal((R, S, D))
    l = rng.standard_normal((R, S)) * 3
    l[2, 1] = -np.inf
    l[4, :] = -np.inf
    out, lse = oracle.lse_merge(o, l)
    for r in range(R):
        if r == 4:
            assert np.isneginf(lse[r]) and np.all(out[r] == 0)
            continue
        ref_lse = scipy.special.logsumexp(l[r])
        w = scipy.special.softmax(l[r])
        assert abs(lse[r] - ref_lse) <= 1e-13 * (1 + abs(ref_lse))
        assert np.max(np.abs(out[r] - w @ o[r])) <= 1e-13


def test_merge_of_one_partial_is_identity():
    rng = np.random.default_rng(6)
    o = rng.standard_normal((3, 1, 8))
    l = rng.standard_normal((3, 1))
    out, lse = oracle.lse_merge(o, l)
    assert np.allclose(out, o[:, 0], rtol=0, atol=1e-15) and np.allclose(lse, l[:, 0], rtol=0, atol=1e-15)


# ---- scalar decoders ------------------------------------------------------

def test_p10_fp8_e4m3fn_decoder_matches_torch_on_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).to(torch.float64).numpy()
    ours = np.array([oracle.fp8e4m3_value(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours)) and nan.sum() == 2  # 0x7F and 0xFF
    assert np.array_equal(ours[~nan], ref[~nan])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9  # largest normal, smallest subnormal


def test_bf16_decoder_matches_torch_on_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    ours = np.array([oracle.bf16_value(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(ours[~nan], ref[~nan])


def test_ranges_entry_pieces_recombine_to_full():
    """Oracle over explicit ranges: the two halves of each sequence, merged with the
    LSE merge, give the full result; full ranges reproduce the plain entry bitwise."""
    w = wl.custom_workload(3, 4, 2, 16, 5, [37, 1, 64], "bf16", 99)
    full_o, full_l = oracle.run_workload(w)
    L = w.seq_lens.numpy()
    args = (w.q, w.k_cache, w.v_cache, w.block_table, w.seq_lens, w.scale)
    o_all, l_all = oracle.paged_decode_ranges(*args, np.zeros(3), L)
    assert np.array_equal(o_all, full_o) and np.array_equal(l_all, full_l)
    mid = L // 2
    o1, l1 = oracle.paged_decode_ranges(*args, np.zeros(3), mid)
    o2, l2 = oracle.paged_decode_ranges(*args, mid, L)
    parts_o = np.stack([o1, o2], axis=2).reshape(-1, 2, 16)
    parts_l = np.stack([l1, l2], axis=2).reshape(-1, 2)
    mo, ml = oracle.lse_merge(parts_o, parts_l)
    assert _close(mo.reshape(full_o.shape), full_o, 1e-12)
    assert _close(ml.reshape(full_l.shape), full_l, 1e-12)


# ---- several query tokens per sequence (speculative verify / extend) -------

def brute_force_multi(w):
    """Dense attention for q [B, q_len, Hq, D] over the logical rows, with the causal
    mask written as an explicit position comparison (query token i of a length-L
    sequence sits at position L - q_len + i); scipy's softmax and logsumexp."""
    B, QL, hq, d = w.q.shape
    hkv = w.spec.num_kv_heads
    G = hq // hkv
    q = _f64(w.q)
    K = _f64(w.k_logical)
    V = _f64(w.v_logical)
    if w.k_scale is not None:
        K = K * w.k_scale.double().numpy()[None, :, None]
        V = V * w.v_scale.double().numpy()[None, :, None]
    out = np.zeros((B, QL, hq, d))
    lse = np.full((B, QL, hq), -np.inf)
    for b in range(B):
        t0, t1 = int(w.token_offsets[b]), int(w.token_offsets[b + 1])
        L = t1 - t0
        pos = np.arange(L)
        for i in range(QL):
            visible = pos <= L - QL + i if w.spec.causal else np.ones(L, bool)
            if not visible.any():
                continue
            for h in range(hq):
                g = h // G
                s = w.scale * (K[t0:t1, g, :] @ q[b, i, h])
                s = s[visible]
                out[b, i, h] = scipy.special.softmax(s) @ V[t0:t1, g, :][visible]
                lse[b, i, h] = scipy.special.logsumexp(s)
    return out, lse


MULTI_CASES = [
    # (B, Hq, Hkv, D, ps, seq_lens, q_len, causal, dtype, seed)
    (2, 4, 2, 16, 3, [7, 20], 3, True, "bf16", 201),
    (3, 8, 2, 16, 16, [5, 33, 2], 4, True, "bf16", 202),   # L = 2 < q_len: two rows see nothing
    (2, 4, 1, 32, 4, [9, 17], 2, False, "bf16", 203),
    (2, 4, 2, 16, 16, [12, 40], 5, True, "fp8_e4m3", 204),
    (1, 2, 2, 8, 1, [6], 6, True, "bf16", 205),             # L = q_len: token 0 sees one row
]


@pytest.mark.parametrize("case", MULTI_CASES)
def test_multi_matches_dense_brute_force_with_explicit_mask(case):
    B, hq, hkv, d, ps, lens, ql, causal, dtype, seed = case
    w = wl.custom_workload(B, hq, hkv, d, ps, lens, dtype, seed, q_len=ql, causal=causal)
    out, lse = oracle.run_workload(w)
    ref_o, ref_l = brute_force_multi(w)
    assert _close(out, ref_o, 1e-12) and _close(lse, ref_l, 1e-12)


def test_multi_with_one_query_token_is_single_token_decode_bitwise():
    w1 = wl.custom_workload(3, 8, 2, 32, 16, [40, 3, 77], "bf16", 211)
    out1, lse1 = oracle.run_workload(w1)
    for causal in (False, True):
        q4 = w1.q.unsqueeze(1).contiguous()  # [B, 1, Hq, D]
        o, l = oracle.paged_decode_multi(q4, w1.k_cache, w1.v_cache, w1.block_table, w1.seq_lens,
                                         w1.scale, causal)
        assert np.array_equal(o[:, 0], out1) and np.array_equal(l[:, 0], lse1)


@pytest.mark.parametrize("causal", [False, True])
def test_multi_token_i_is_single_token_decode_over_its_visible_prefix(causal):
    """Query token i (causal) is the single-token definition over the first
    L - q_len + i + 1 tokens of the same pages; without the mask, over all L."""
    ql = 3
    w = wl.custom_workload(3, 8, 4, 16, 5, [14, 30, 9], "bf16", 212, q_len=ql, causal=causal)
    out, lse = oracle.run_workload(w)
    L = w.seq_lens.to(torch.int64)
    for i in range(ql):
        vis = torch.clamp(L - ql + i + 1, min=0) if causal else L
        o, l = oracle.paged_decode(w.q[:, i].contiguous(), w.k_cache, w.v_cache, w.block_table,
                                   vis.to(torch.int32), w.scale)
        assert np.array_equal(out[:, i], o) and np.array_equal(lse[:, i], l)


def test_multi_first_token_of_a_just_filled_sequence_sees_only_token_zero():
    """Causal, L = q_len: query token 0 sees token 0 alone, so out = V_0 exactly
    and lse = s_0 (closed form)."""
    w = wl.custom_workload(1, 4, 2, 16, 4, [5], "bf16", 213, q_len=5, causal=True)
    out, lse = oracle.run_workload(w)
    q = _f64(w.q)
    K = _f64(w.k_logical)
    V = _f64(w.v_logical)
    for h in range(4):
        g = h // 2
        assert np.array_equal(out[0, 0, h], V[0, g])
        assert abs(lse[0, 0, h] - w.scale * float(K[0, g] @ q[0, 0, h])) <= 1e-15


def test_multi_rows_without_visible_tokens_are_zero_and_minus_inf():
    w = wl.custom_workload(2, 4, 1, 16, 4, [2, 0], "bf16", 214, q_len=4, causal=True)
    out, lse = oracle.run_workload(w)
    # sequence 0 (L = 2): tokens 0 and 1 see nothing, tokens 2 and 3 see 1 and 2 rows
    assert np.all(out[0, :2] == 0) and np.all(np.isneginf(lse[0, :2]))
    assert np.all(np.isfinite(lse[0, 2:]))
    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1]))


def test_multi_rows_entry_matches_full_oracle():
    w = wl.custom_workload(3, 8, 2, 32, 16, [40, 3, 77], "fp8_e4m3", 215, q_len=3, causal=True)
    out, lse = oracle.run_workload(w)
    rows = [0, 5, 9, 23, 17, 40, 71]
    o_r, l_r = oracle.paged_decode_multi_rows(w.q, w.k_cache, w.v_cache, w.block_table, w.seq_lens,
                                              w.scale, True, rows, w.k_scale, w.v_scale)
    flat_o, flat_l = out.reshape(-1, 32), lse.reshape(-1)
    assert np.array_equal(o_r, flat_o[rows]) and np.array_equal(l_r, flat_l[rows])


# ---- paged KV append (quantised cache write with optional RoPE) -----------------

dataclasses_replace = dataclasses.replace


def _append(w, **kw):
    return oracle.kv_append(w.k_new, w.v_new, w.slot_mapping, w.k_cache, w.v_cache, w.k_scale, w.v_scale,
                            w.positions, w.cos_sin, **kw)


def test_append_bf16_copies_rows_to_their_slots_and_nothing_else():
    w = wl.append_workload(40, 3, 16, 8, 12, "bf16", seed=301, pad_every=7)
    kc, vc = _append(w)
    k0 = wl.as_numpy_bits(w.k_cache).copy()
    v0 = wl.as_numpy_bits(w.v_cache).copy()
    ps = 8
    kn = wl.as_numpy_bits(w.k_new)
    vn = wl.as_numpy_bits(w.v_new)
    written = np.zeros(k0.shape[:2], bool)
    for n, slot in enumerate(w.slot_mapping.tolist()):
        if slot < 0 or slot >= 12 * ps:
            continue
        written[slot // ps, slot % ps] = True
        assert np.array_equal(kc[slot // ps, slot % ps], kn[n]) and np.array_equal(vc[slot // ps, slot % ps], vn[n])
    assert written.sum() == sum(1 for s in w.slot_mapping.tolist() if 0 <= s < 12 * ps)
    assert np.array_equal(kc[~written], k0[~written]) and np.array_equal(vc[~written], v0[~written])


def test_fp8_encoder_matches_torch_rounding():
    """Nearest E4M3FN code with ties to even, against torch's float8_e4m3fn conversion, on
    every bf16 value in [-448, 448], all exact midpoints between codes, and random floats."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    xs = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float32)
    xs = xs[torch.isfinite(xs) & (xs.abs() <= 448)]
    codes = torch.arange(0x7F, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float32)
    mids = (codes[1:] + codes[:-1]) / 2
    rnd = torch.empty(20000).uniform_(-448, 448, generator=torch.Generator().manual_seed(5))
    xs = torch.cat([xs, mids, -mids, rnd]).to(torch.float32)
    ref = xs.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = np.array([oracle.fp8e4m3_encode(float(x)) for x in xs.numpy()], dtype=np.uint8)
    assert np.array_equal(ours, ref)


def test_append_fp8_quantises_with_each_heads_scale_and_saturates():
    w = wl.append_workload(30, 4, 32, 4, 10, "fp8_e4m3", seed=302)
    kc, vc = _append(w)
    kn = w.k_new.to(torch.float32).numpy()
    vn = w.v_new.to(torch.float32).numpy()
    ks, vs = w.k_scale.numpy(), w.v_scale.numpy()
    saturated = 0
    for n, slot in enumerate(w.slot_mapping.tolist()):
        if slot < 0 or slot >= 40:
            continue
        for h in range(4):
            qk = np.clip(kn[n, h] / ks[h], -448, 448).astype(np.float32)  # fp32 division, as specified
            saturated += int((np.abs(kn[n, h] / ks[h]) > 448).sum())
            exp_k = torch.from_numpy(qk).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            qv = np.clip(vn[n, h] / vs[h], -448, 448).astype(np.float32)
            exp_v = torch.from_numpy(qv).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(kc[slot // 4, slot % 4, h], exp_k)
            assert np.array_equal(vc[slot // 4, slot % 4, h], exp_v)
    assert saturated > 0  # the draw exercises the clamp


def test_rope_identity_and_quarter_turn():
    """cos = 1, sin = 0 leaves K unchanged; cos = 0, sin = 1 maps (k[d], k[d + D/2]) to
    (-k[d + D/2], k[d]) exactly (rotate-half pairing)."""
    w = wl.append_workload(12, 2, 16, 4, 6, "bf16", seed=303, rope=True)
    D = 16
    table = torch.zeros(2, D)
    table[0, : D // 2] = 1.0          # position 0: identity
    table[1, D // 2:] = 1.0           # position 1: a quarter turn
    pos = torch.tensor([n % 2 for n in range(12)], dtype=torch.int64)
    w2 = dataclasses_replace(w, positions=pos, cos_sin=table.contiguous())
    kc, _ = _append(w2)
    kn = wl.as_numpy_bits(w.k_new)
    kf = w.k_new.to(torch.float32).numpy()
    for n, slot in enumerate(w.slot_mapping.tolist()):
        if slot < 0 or slot >= 24:
            continue
        row = kc[slot // 4, slot % 4]
        if n % 2 == 0:
            assert np.array_equal(row, kn[n])
        else:
            expect = np.concatenate([-kf[n, :, D // 2:], kf[n, :, : D // 2]], axis=1)
            got = torch.from_numpy(row.view(np.int16).copy()).view(torch.bfloat16).to(torch.float32).numpy()
            assert np.array_equal(got, expect)


def test_rope_rotations_compose_and_keep_pair_norms():
    """Rotating by the table row of angle a and then of angle b matches one rotation by
    a + b, and every (d, d + D/2) pair keeps its length, within fp32/bf16 rounding."""
    D = 32
    w = wl.append_workload(8, 1, D, 8, 1, "bf16", seed=304)
    slots = torch.arange(8, dtype=torch.int64)
    rng = np.random.default_rng(9)
    a, b = rng.uniform(-3, 3, D // 2), rng.uniform(-3, 3, D // 2)
    def table(ang):
        return torch.from_numpy(np.concatenate([np.cos(ang), np.sin(ang)])[None, :].astype(np.float32))
    zero = torch.zeros(8, dtype=torch.int64)
    def rotate(k_new, ang):
        ww = dataclasses_replace(w, k_new=k_new, slot_mapping=slots, positions=zero, cos_sin=table(ang))
        kc, _ = _append(ww)
        return torch.from_numpy(kc.view(np.int16).copy()).view(torch.bfloat16).reshape(8, 1, D)
    once = rotate(rotate(w.k_new, a), b).to(torch.float64).numpy()
    both = rotate(w.k_new, a + b).to(torch.float64).numpy()
    assert np.max(np.abs(once - both)) <= 0.05 * (1 + np.abs(both).max())
    x = w.k_new.to(torch.float64).numpy()
    r = rotate(w.k_new, a).to(torch.float64).numpy()
    n0 = x[..., : D // 2] ** 2 + x[..., D // 2:] ** 2
    n1 = r[..., : D // 2] ** 2 + r[..., D // 2:] ** 2
    assert np.allclose(n1, n0, rtol=2e-2, atol=1e-3)
    # and the rotation really moved the rows
    assert np.max(np.abs(r - x)) > 0.1


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3"])
def test_rope_append_within_one_code_of_the_fp64_rotation(kv_dtype):
    """The append's fp32 recipe (a product, then one fused multiply-add, then the cache
    rounding) against the rotation computed in fp64: every stored value is within half
    a code step plus the fp32 recipe's error bound of the exact value, every code is the
    exact code or a neighbour where that fp32 error is under a quarter step (no
    cancellation), and nearly all codes are the exact value's code."""
    import rope_reference as rr
    w = wl.append_workload(300, 4, 64, 16, 40, kv_dtype, seed=310, rope=True, scale_range=(0.01, 0.05))
    kc, _ = _append(w)
    worst, exact_share, dist = rr.check(w, kc, kv_dtype)
    assert worst <= 1.0, f"error / derived bound {worst:.3g}"
    assert dist <= 1
    assert exact_share > 0.99


def test_rope_row_is_selected_by_position_and_out_of_table_positions_write_nothing():
    w = wl.append_workload(20, 2, 16, 4, 10, "bf16", seed=305, rope=True)
    kc, _ = _append(w)
    k0 = wl.as_numpy_bits(w.k_cache)
    for n, slot in enumerate(w.slot_mapping.tolist()):
        if slot < 0 or slot >= 40:
            continue
        p = int(w.positions[n])
        if p >= w.cos_sin.shape[0]:
            assert np.array_equal(kc[slot // 4, slot % 4], k0[slot // 4, slot % 4])
            continue
        # the same token appended alone with a one-row table holding row p
        ww = dataclasses_replace(w, k_new=w.k_new[n:n + 1].contiguous(), v_new=w.v_new[n:n + 1].contiguous(),
                                 slot_mapping=torch.tensor([0]), positions=torch.tensor([0]),
                                 cos_sin=w.cos_sin[p:p + 1].contiguous())
        one, _ = _append(ww)
        assert np.array_equal(kc[slot // 4, slot % 4], one[0, 0])


def test_bf16_rounding_matches_torch():
    """fp32 -> bf16 round to nearest even, against torch, on random values across the exponent
    range and on exact midpoints between bf16 neighbours (both tie directions)."""
    g = torch.Generator().manual_seed(11)
    x = torch.randn(20000, generator=g) * torch.exp2(torch.randint(-60, 60, (20000,), generator=g).float())
    lo = torch.randn(5000, generator=g).to(torch.bfloat16)
    lo_bits = lo.view(torch.int16).to(torch.int32) & 0xFFFF
    mids = ((lo_bits << 16) | 0x8000).to(torch.int32).view(torch.float32)  # halfway to the next bf16
    xs = torch.cat([x, mids])
    ref = xs.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = np.array([oracle.bf16_round(float(v)) for v in xs.numpy()], dtype=np.uint16)
    assert np.array_equal(ours, ref)


# ---- sliding window and attention sinks -------------------------------------------

def brute_force_ext(w):
    """Dense attention with the visible set written as explicit position tests (window
    lower end, causal upper end) and the sink as one more logit with no value row."""
    q = _f64(w.q)
    if q.ndim == 3:
        q = q[:, None]
    B, QL, hq, d = q.shape
    G = hq // w.spec.num_kv_heads
    K, V = _f64(w.k_logical), _f64(w.v_logical)
    if w.k_scale is not None:
        K = K * w.k_scale.double().numpy()[None, :, None]
        V = V * w.v_scale.double().numpy()[None, :, None]
    W = w.spec.window
    sinks = None if w.sinks is None else w.sinks.double().numpy()
    out = np.zeros((B, QL, hq, d))
    lse = np.full((B, QL, hq), -np.inf)
    for b in range(B):
        t0, t1 = int(w.token_offsets[b]), int(w.token_offsets[b + 1])
        L = t1 - t0
        pos = np.arange(L)
        for i in range(QL):
            p = L - QL + i
            vis = np.ones(L, bool)
            if w.spec.causal:
                vis &= pos <= p
            if W:
                vis &= pos > p - W
            for h in range(hq):
                s = w.scale * (K[t0:t1, h // G, :] @ q[b, i, h])[vis]
                logits = s if sinks is None else np.append(s, sinks[h])
                if logits.size == 0:
                    continue
                lse[b, i, h] = scipy.special.logsumexp(logits)
                wts = np.exp(s - lse[b, i, h])
                out[b, i, h] = wts @ V[t0:t1, h // G, :][vis]
    return out, lse


EXT_CASES = [
    # (B, Hq, Hkv, D, ps, lens, q_len, causal, window, sinks, dtype, seed)
    (3, 4, 2, 16, 4, [20, 7, 33], 1, False, 8, False, "bf16", 401),
    (2, 8, 2, 16, 16, [40, 5], 3, True, 6, True, "bf16", 402),
    (2, 4, 1, 32, 3, [11, 0], 1, False, 0, True, "bf16", 403),
    (2, 4, 2, 16, 16, [30, 18], 4, False, 5, True, "fp8_e4m3", 404),
    (1, 2, 1, 8, 4, [9], 2, True, 1, True, "bf16", 405),
]


@pytest.mark.parametrize("case", EXT_CASES)
def test_window_and_sinks_match_brute_force(case):
    B, hq, hkv, d, ps, lens, ql, causal, window, sinks, dtype, seed = case
    w = wl.custom_workload(B, hq, hkv, d, ps, lens, dtype, seed, q_len=ql, causal=causal, window=window,
                           sinks=sinks)
    out, lse = oracle.run_workload(w)
    ref_o, ref_l = brute_force_ext(w)
    assert _close(out, ref_o, 1e-12) and _close(lse, ref_l, 1e-12)


def test_no_window_and_no_sinks_is_the_multi_token_entry_bitwise():
    w = wl.custom_workload(3, 8, 2, 16, 4, [19, 40, 2], "bf16", 406, q_len=3, causal=True)
    ref = oracle.run_workload(w)
    args = (w.q, w.k_cache, w.v_cache, w.block_table, w.seq_lens, w.scale)
    for window in (0, 10 ** 6):
        out, lse = oracle.paged_decode_ext(*args, True, window, None)
        assert np.array_equal(out, ref[0]) and np.array_equal(lse, ref[1])
    minus_inf = torch.full((8,), float("-inf"))
    out, lse = oracle.paged_decode_ext(*args, True, 0, minus_inf)
    assert np.array_equal(out, ref[0]) and np.array_equal(lse, ref[1])


def test_decode_window_is_attention_over_the_last_window_tokens():
    w = wl.custom_workload(3, 4, 2, 16, 5, [30, 4, 17], "bf16", 407)
    L = w.seq_lens.numpy()
    args = (w.q, w.k_cache, w.v_cache, w.block_table, w.seq_lens, w.scale)
    for window in (1, 6, 17):
        out, lse = oracle.paged_decode_ext(*args, False, window, None)
        o_r, l_r = oracle.paged_decode_ranges(*args, np.maximum(L - window, 0), L)
        assert np.array_equal(out[:, 0], o_r) and np.array_equal(lse[:, 0], l_r)


def test_sink_closed_form_and_empty_rows():
    """One visible token: out = v0 e^s0 / (e^s0 + e^sink), lse = ln(e^s0 + e^sink); no
    visible token: out = 0, lse = sink."""
    w = wl.custom_workload(2, 2, 1, 8, 4, [1, 0], "bf16", 408, sinks=True)
    out, lse = oracle.run_workload(w)
    q, K, V = _f64(w.q), _f64(w.k_logical), _f64(w.v_logical)
    sk = w.sinks.double().numpy()
    for h in range(2):
        s0 = w.scale * float(K[0, 0] @ q[0, h])
        z = math.exp(s0) + math.exp(sk[h])
        assert np.max(np.abs(out[0, 0, h] - V[0, 0] * math.exp(s0) / z)) <= 1e-13
        assert abs(lse[0, 0, h] - math.log(z)) <= 1e-13
        assert np.all(out[1, 0, h] == 0) and lse[1, 0, h] == np.float32(sk[h])


# ---- decode metadata preparation --------------------------------------------

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_metadata_hand_worked_example():
    """The oracle reproduces a case worked by hand (tests/golden), with and
    without the sliding-window tables."""
    with open(os.path.join(GOLDEN, "decode_metadata_hand_example.json")) as f:
        g = json.load(f)
    rt = np.array(g["req_to_token"], np.int32)
    rp = np.array(g["req_pool_indices"], np.int64)
    sl = np.array(g["seq_lens"], np.int64)
    e = g["expected"]
    res, bad = oracle.decode_metadata(rt, rp, sl, g["page_size"], g["max_pages"], extend=g["extend"])
    assert bad == e["invalid"]
    assert res["cache_seqlens"].tolist() == e["cache_seqlens"]
    assert res["cu_seqlens_k"].tolist() == e["cu_seqlens_k"]
    assert res["page_table"].tolist() == e["page_table"]
    for c in g["swa_cases"]:
        r2, bad2 = oracle.decode_metadata(rt, rp, sl, g["page_size"], g["max_pages"], q_len=c["q_len"],
                                          window=c["window"], extend=g["extend"])
        assert bad2 == e["invalid"]
        assert r2["page_table"].tolist() == e["page_table"]
        assert r2["swa_seqlens"].tolist() == c["swa_seqlens"], c["why"]
        assert r2["swa_page_table"].tolist() == c["swa_page_table"], c["why"]


def token_map_from_block_table(bt, lens, ps, req_rows, stride, seed):
    """A req_to_token pool holding the given block tables in shuffled request
    rows: token t of sequence b is slot bt[b][t // ps] * ps + t % ps; every
    other cell is random garbage.  Returns (req_to_token, req_pool_indices)."""
    rng = np.random.default_rng(seed)
    B = bt.shape[0]
    rt = rng.integers(-5, 10 ** 6, size=(req_rows, stride)).astype(np.int32)
    rows = rng.permutation(req_rows)[:B]
    for b in range(B):
        for t in range(int(lens[b])):
            rt[rows[b], t] = bt[b, t // ps] * ps + t % ps
    return rt, rows.astype(np.int64)


@pytest.mark.parametrize("ps", [1, 16, 24, 64])
def test_metadata_recovers_the_block_table_and_lengths(ps):
    """Built from a token map that was itself built from a block table, the
    page table is that block table (then -1), the lengths are the lengths plus
    the extension, and the prefix sums step by them."""
    rng = np.random.default_rng(ps)
    B, MP, extend = 9, 7, 2
    lens = rng.integers(0, MP * ps - extend + 1, size=B)
    lens[0], lens[1] = 0, MP * ps - extend
    bt = rng.permutation(B * MP * 3)[:B * MP].reshape(B, MP).astype(np.int32)
    rt, rows = token_map_from_block_table(bt, lens + extend, ps, 2 * B + 3, MP * ps + 5, seed=ps)
    res, bad = oracle.decode_metadata(rt, rows, lens.astype(np.int64), ps, MP, extend=extend)
    assert bad == 0
    L = lens + extend
    assert res["cache_seqlens"].tolist() == L.tolist()
    cu = res["cu_seqlens_k"].astype(np.int64)
    assert cu[0] == 0 and np.diff(cu).tolist() == L.tolist()
    for b in range(B):
        n = -(-int(L[b]) // ps)
        assert res["page_table"][b, :n].tolist() == bt[b, :n].tolist()
        assert (res["page_table"][b, n:] == -1).all()


@pytest.mark.parametrize("ps,q_len,window", [(16, 1, 40), (16, 3, 17), (64, 1, 100), (24, 2, 50), (1, 1, 5)])
def test_metadata_swa_tables_drop_only_pages_below_the_window(ps, q_len, window):
    """The SWA tables drop whole pages that hold no visible position and nothing
    else, and the oracle's decode over them (same window) equals its decode
    over the full tables bit for bit."""
    lens = [0, 1, window - 1, window, window + q_len, 3 * window + 7, 500]
    w = wl.custom_workload(len(lens), 8, 2, 64, ps, lens, "bf16", seed=ps + window, q_len=q_len, causal=True,
                           window=window, sinks=True)
    MP = w.block_table.shape[1]
    bt = w.block_table.numpy()
    rt, rows = token_map_from_block_table(bt, lens, ps, len(lens) + 4, MP * ps, seed=window)
    res, bad = oracle.decode_metadata(rt, rows, np.array(lens, np.int64), ps, MP, q_len=q_len, window=window)
    assert bad == 0
    for b, L in enumerate(lens):
        lo = max(L - q_len - window + 1, 0)
        dropped = L - int(res["swa_seqlens"][b])
        assert dropped % ps == 0 and dropped <= lo < dropped + ps
        n = -(-L // ps)
        f = dropped // ps
        assert res["swa_page_table"][b, :n - f].tolist() == bt[b, f:n].tolist()
        assert (res["swa_page_table"][b, n - f:] == -1).all()
    full = oracle.paged_decode_ext(w.q, w.k_cache, w.v_cache, torch.from_numpy(res["page_table"]),
                                   torch.from_numpy(res["cache_seqlens"]), w.scale, True, window, w.sinks)
    swa = oracle.paged_decode_ext(w.q, w.k_cache, w.v_cache, torch.from_numpy(res["swa_page_table"]),
                                  torch.from_numpy(res["swa_seqlens"]), w.scale, True, window, w.sinks)
    assert np.array_equal(full[0], swa[0]) and np.array_equal(full[1], swa[1])


def test_metadata_invalid_entries_are_counted_and_blanked():
    rt = np.arange(4 * 32, dtype=np.int32).reshape(4, 32)
    rp = np.array([0, -1, 4, 3, 2], np.int64)
    sl = np.array([5, 5, 5, 40, -1], np.int64)  # 40 > 4 pages of 8 tokens; -1 < 0
    res, bad = oracle.decode_metadata(rt, rp, sl, 8, 4, window=3)
    assert bad == 4
    assert res["cache_seqlens"].tolist() == [5, 0, 0, 0, 0]
    assert res["cu_seqlens_k"].tolist() == [0, 5, 5, 5, 5, 5]
    assert res["page_table"][0].tolist() == [0, -1, -1, -1]
    assert (res["page_table"][1:] == -1).all() and (res["swa_page_table"][1:] == -1).all()
    assert res["swa_seqlens"].tolist() == [5, 0, 0, 0, 0]


# ---- contiguous (strided) KV decode ------------------------------------------

CONTIG_CASES = [
    # (B, Hq, Hkv, D, ps, seq_lens, q_len, causal, window, sinks, dtype, seed)
    (3, 8, 2, 64, 16, [37, 1, 100], 1, False, 0, False, "bf16", 601),
    (3, 8, 2, 64, 16, [0, 50, 9], 3, True, 20, True, "bf16", 602),
    (2, 4, 4, 32, 24, [70, 33], 2, False, 0, True, "fp8_e4m3", 603),
]


@pytest.mark.parametrize("case", CONTIG_CASES)
@pytest.mark.parametrize("layout", ["blhd", "bhld", "blhd_padded"])
def test_contiguous_equals_paged_on_the_same_rows(case, layout):
    """Decode over the sequences' rows laid out contiguously (three layouts, a
    strided q; NaN in every element that is not a sequence row) gives the same
    bits as the paged decode of the same rows."""
    bq, hq, hkv, d, ps, lens, ql, causal, win, sinks, dtype, seed = case
    w = wl.custom_workload(bq, hq, hkv, d, ps, lens, dtype, seed, q_len=ql, causal=causal, window=win, sinks=sinks)
    paged = oracle.paged_decode_ext(w.q, w.k_cache, w.v_cache, w.block_table, w.seq_lens, w.scale, causal, win,
                                    w.sinks, w.k_scale, w.v_scale)
    k, v = wl.contiguous_kv(w, layout, capacity=max(lens) + 3)
    got = oracle.contiguous_decode(wl.strided_q(w.q), k, v, w.seq_lens, w.scale, causal, win, w.sinks,
                                   w.k_scale, w.v_scale)
    assert np.array_equal(got[0], paged[0].reshape(got[0].shape)) and np.array_equal(got[1], paged[1].reshape(got[1].shape))


def test_contiguous_layout_reads_each_stride():
    """Swapping two tokens, two KV heads or two sequences in the contiguous
    tensor changes exactly the rows that read them."""
    lens = [40, 40]
    w = wl.custom_workload(2, 4, 2, 32, 16, lens, "bf16", seed=610)
    k, v = wl.contiguous_kv(w, "bhld")
    base = oracle.contiguous_decode(w.q, k, v, w.seq_lens, w.scale)
    k2, v2 = k.clone(), v.clone()
    k2[0, [3, 7]] = k2[0, [7, 3]]  # two tokens of sequence 0 (K and V rows): the sum is order-free
    v2[0, [3, 7]] = v2[0, [7, 3]]
    same = oracle.contiguous_decode(w.q, k2, v2, w.seq_lens, w.scale)
    assert np.allclose(same[0], base[0], atol=1e-12) and not torch.equal(k2[0, 3], k[0, 3])
    v2 = v.clone()
    v2[0, 5] = v2[0, 5] + 1.0      # one value row of sequence 0, both heads
    moved = oracle.contiguous_decode(w.q, k, v2, w.seq_lens, w.scale)
    assert not np.allclose(moved[0][0], base[0][0]) and np.array_equal(moved[0][1], base[0][1])
    k3 = k.clone()
    k3[1, :, 0] = k3[1, :, 1].clone()  # KV head 0 of sequence 1 := KV head 1
    heads = oracle.contiguous_decode(w.q, k3, v, w.seq_lens, w.scale)
    assert np.array_equal(heads[0][0], base[0][0])
    assert np.array_equal(heads[0][1, :, 2:], base[0][1, :, 2:])  # query heads 2, 3 read KV head 1
    assert not np.allclose(heads[0][1, :, :2], base[0][1, :, :2])
