"""Parity of the HIP path against the fp64 oracle (needs an MI355X).

Every call goes through the C ABI (paged_kv_decode_amd.binding).  Acceptance:
|out - ref| <= 1e-2 + 1e-2 * |ref| element-wise on the bf16 output and
|lse - ref| <= 1e-3, with ref the oracle on the same seeded inputs.  Index work
is checked bit-exactly by one-hot probes; tails are NaN-poisoned and unused
block-table entries are -1 so that any stray read shows.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
from paged_kv_decode_amd import workloads as wl

pytestmark = pytest.mark.gpu

BAL = -1000  # PKD_SPLITS_BALANCED
PAIR = -1001  # PKD_SPLITS_PAIRED
OUT_ATOL = 1e-2
OUT_RTOL = 1e-2
LSE_ATOL = 1e-3


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_decode_amd import binding
    return binding


def dev(w):
    cuda = torch.device("cuda:0")
    t = dict(q=w.q.to(cuda), k=w.k_cache.to(cuda), v=w.v_cache.to(cuda),
             bt=w.block_table.to(cuda), lens=w.seq_lens.to(cuda))
    t["ks"] = None if w.k_scale is None else w.k_scale.to(cuda)
    t["vs"] = None if w.v_scale is None else w.v_scale.to(cuda)
    t["sinks"] = None if getattr(w, "sinks", None) is None else w.sinks.to(cuda)
    return t


def run(B, w, S=0, t=None, scale=None):
    t = t or dev(w)
    out, lse = B.decode(t["q"], t["k"], t["v"], t["bt"], t["lens"], w.scale if scale is None else scale,
                        t["ks"], t["vs"], num_splits=S, causal=w.spec.causal, window=w.spec.window,
                        sinks=t["sinks"])
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def check(out, lse, ref_out, ref_lse, what=""):
    o = out.to(torch.float64).numpy().reshape(ref_out.shape)
    l = lse.to(torch.float64).numpy().reshape(ref_lse.shape)
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    err = np.abs(o - ref_out)
    bound = OUT_ATOL + OUT_RTOL * np.abs(ref_out)
    assert np.all(err <= bound), f"{what}: out max err {err.max():.3g} (worst ratio {(err / bound).max():.3g})"
    inf_ref = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(l), inf_ref), f"{what}: -inf pattern of lse differs"
    lerr = np.abs(np.where(inf_ref, 0.0, l - np.where(inf_ref, 0.0, ref_lse)))
    assert np.all(lerr <= LSE_ATOL), f"{what}: lse max err {lerr.max():.3g}"
    return float(err.max()), float(lerr.max())


def oracle_full(w):
    return oracle.run_workload(w, nthreads=min(16, max(1, len(__import__("os").sched_getaffinity(0)))))


# ---- the small case, direct and split -------------------------------------

@pytest.mark.parametrize("S", [1, 3, 0, BAL])
def test_tiny_workload(B, S):
    w = wl.make_workload(wl.WORKLOADS["tiny_b2_d64_ps16"])
    ref = oracle_full(w)
    out, lse = run(B, w, S)
    check(out, lse, *ref, what=f"tiny S={S}")


# ---- shapes, page sizes, edge lengths ---------------------------------------

EDGE_LENS = lambda ps: [1, ps - 1 if ps > 1 else 2, ps, ps + 1, 37, 200, 0, 513]


@pytest.mark.parametrize("dtype", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("d", [32, 64, 128, 256])
@pytest.mark.parametrize("ps", [16, 24, 64])
def test_head_dims_page_sizes_edge_lengths(B, dtype, d, ps):
    lens = EDGE_LENS(ps)
    w = wl.custom_workload(len(lens), 8, 2, d, ps, lens, dtype, seed=1000 + d + ps)
    ref = oracle_full(w)
    t = dev(w)
    for S in (1, 4, 11) + ((BAL,) if ps % 16 == 0 else ()):
        out, lse = run(B, w, S, t)
        check(out, lse, *ref, what=f"{dtype} D={d} ps={ps} S={S}")


@pytest.mark.parametrize("hq,hkv", [(4, 4), (16, 2), (16, 1), (32, 1), (40, 2)])
def test_gqa_group_sizes(B, hq, hkv):
    """G = 1, 8, 16, 32 (two head groups) and 20 (a partial second group)."""
    lens = [5, 130, 64, 1]
    w = wl.custom_workload(len(lens), hq, hkv, 64, 16, lens, "bf16", seed=hq * 10 + hkv)
    ref = oracle_full(w)
    t = dev(w)
    for S in (1, 3, BAL):
        out, lse = run(B, w, S, t)
        check(out, lse, *ref, what=f"Hq={hq} Hkv={hkv} S={S}")


def test_split_count_larger_than_tiles(B):
    lens = [37, 3, 64, 65]
    w = wl.custom_workload(len(lens), 8, 2, 128, 16, lens, "bf16", seed=7)
    ref = oracle_full(w)
    t = dev(w)
    for S in (2, 7, 64, 512, BAL):
        out, lse = run(B, w, S, t)
        check(out, lse, *ref, what=f"S={S}")


def test_all_zero_lengths(B):
    """Every sequence empty: out = 0 and lse = -inf, and no page is read (the block
    table holds only -1)."""
    cuda = torch.device("cuda:0")
    q = torch.randn(3, 4, 64).to(torch.bfloat16).to(cuda)
    k = torch.full((1, 16, 1, 64), float("nan"), dtype=torch.bfloat16, device=cuda)
    bt = torch.full((3, 2), -1, dtype=torch.int32, device=cuda)
    lens = torch.zeros(3, dtype=torch.int32, device=cuda)
    for S in (1, 5, BAL):
        out, lse = B.decode(q, k, k.clone(), bt, lens, 0.125, num_splits=S)
        torch.cuda.synchronize()
        assert torch.all(out.float() == 0) and torch.all(torch.isneginf(lse))


# ---- bit-exact indexing probe -------------------------------------------------

def one_hot_workload(lens, hq, hkv, d, ps, dtype, seed):
    """q = e_0 for every head; K[t][0] = 0 except one chosen token t* per sequence
    with K[t*][0] = 4096 (exact in bf16; in fp8 it is the head's amax, code 448).
    Scores are 0 except 4096 * scale >= 256 at t*, so exp(s_t - s_t*) underflows to 0
    and the output must be exactly bf16(V[t*]) (for fp8: bf16(code * v_scale))."""
    w = wl.custom_workload(len(lens), hq, hkv, d, ps, lens, dtype, seed)
    g = torch.Generator().manual_seed(seed + 1)
    q = torch.zeros_like(w.q)
    q[..., 0] = 1.0
    K32 = torch.randn(w.k_logical.shape, generator=g)
    K32[..., 0] = 0.0
    tstar = []
    for b, L in enumerate(lens):
        if L == 0:
            tstar.append(-1)
            continue
        choices = [0, ps - 1, ps, L - 1, int(torch.randint(0, L, (1,), generator=g))]
        ts = min(choices[b % len(choices)], L - 1)
        tstar.append(ts)
        K32[int(w.token_offsets[b]) + ts, :, 0] = 4096.0
    if dtype == "bf16":
        K = K32.to(torch.bfloat16)
        w2 = wl.rebuild_with_rows(w, q=q, k_logical=K)
    else:
        codes, kscale = wl._quantize_fp8_per_head(K32)
        w2 = wl.rebuild_with_rows(w, q=q, k_logical=codes)
        w2.k_scale = kscale
    return w2, tstar


@pytest.mark.parametrize("dtype", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("d,ps", [(64, 16), (128, 64), (32, 64), (256, 64), (128, 24), (128, 128)])
def test_bit_exact_one_hot_probe(B, dtype, d, ps):
    lens = [ps * 3 + 5, ps, 1, ps * 7 - 1, 2 * ps + 1, 77]
    hq, hkv = 8, 2
    w, tstar = one_hot_workload(lens, hq, hkv, d, ps, dtype, seed=d * 7 + ps)
    t = dev(w)
    V = w.v_logical
    for S in (1, 3, 0) + ((BAL,) if ps % 16 == 0 else ()):
        out, lse = run(B, w, S, t)
        for b, ts in enumerate(tstar):
            row = V[int(w.token_offsets[b]) + ts]  # [Hkv, D]
            for h in range(hq):
                kv = h // (hq // hkv)
                if dtype == "bf16":
                    want = row[kv].clone()
                else:
                    want = (row[kv].to(torch.float32) * w.v_scale[kv]).to(torch.bfloat16)
                got = out[b, h]
                assert torch.equal(got.float(), want.float()), \
                    f"b={b} h={h} t*={ts} S={S}: output is not V[t*] exactly"
        ref = oracle_full(w)
        check(out, lse, *ref, what=f"one-hot S={S}")


# The full-size shapes the probe and the determinism check also run at: the
# B=32, B=128 and FP8 B=64 workloads' heads, page sizes and lengths.
FULL_SHAPES = {
    "tiny": ("tiny_b2_d64_ps16", "bf16"),
    "llama_b32": ("llama_b32_d128_ps64", "bf16"),
    "batch128": ("batch128_d128_ps128", "bf16"),
    "longctx_b1_d32": ("longctx_b1_d32", "bf16"),
    "longctx_b16_d256": ("longctx_b16_d256", "bf16"),
    "fp8kv_b64": ("fp8kv_b64_d128_ps64", "fp8_e4m3"),
}


def full_shape_modes(spec):
    return (1, 8, 0, BAL)


@pytest.mark.parametrize("shape", list(FULL_SHAPES))
def test_bit_exact_one_hot_probe_at_full_shapes(B, shape):
    """The indexing probe at full size: one token t* per sequence (its first,
    a page's last or first slot, its last, or a random one) dominates every
    head, so every output row must be exactly that token's V row."""
    name, dtype = FULL_SHAPES[shape]
    spec = wl.WORKLOADS[name]
    lens = wl.make_workload(spec, tail="zero").seq_lens.tolist()
    w, tstar = one_hot_workload(lens, spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.page_size, dtype,
                                seed=spec.seed + 500)
    t = dev(w)
    G = spec.num_q_heads // spec.num_kv_heads
    rows = torch.stack([w.v_logical[int(w.token_offsets[b]) + ts] for b, ts in enumerate(tstar)])  # [B, Hkv, D]
    if dtype == "bf16":
        want = rows.repeat_interleave(G, dim=1)
    else:
        want = (rows.to(torch.float32) * w.v_scale.view(1, -1, 1)).to(torch.bfloat16).repeat_interleave(G, dim=1)
    for S in full_shape_modes(spec):
        out, _ = run(B, w, S, t)
        # Exact equality of values (the other tokens' zero weights times V add +0,
        # so a -0 element of V[t*] comes out as +0, the same value).
        bad = (out.float() != want.float()).any(dim=-1)
        assert not bad.any(), f"S={S}: rows {bad.nonzero()[:5].tolist()} are not V[t*] exactly"


@pytest.mark.parametrize("shape", list(FULL_SHAPES))
def test_bitwise_deterministic_at_full_shapes(B, shape):
    name, _ = FULL_SHAPES[shape]
    spec = wl.WORKLOADS[name]
    w = wl.make_workload(spec, tail="nan")
    t = dev(w)
    for S in full_shape_modes(spec):
        a = run(B, w, S, t)
        b_ = run(B, w, S, t)
        assert torch.equal(a[0].view(torch.int16), b_[0].view(torch.int16)) and torch.equal(a[1], b_[1]), S


# ---- poisoned tails, determinism, dtype interleaving --------------------------

@pytest.mark.parametrize("dtype", ["bf16", "fp8_e4m3"])
def test_nan_tails_and_padding_are_never_read(B, dtype):
    lens = [37, 100, 1, 16, 15]
    w_nan = wl.custom_workload(len(lens), 8, 2, 64, 16, lens, dtype, seed=31, tail="nan")
    w_zero = wl.custom_workload(len(lens), 8, 2, 64, 16, lens, dtype, seed=31, tail="zero")
    assert (w_nan.block_table == -1).any()
    for S in (1, 3, BAL):
        a = run(B, w_nan, S)
        z = run(B, w_zero, S)
        assert torch.isfinite(a[0].float()).all()
        assert torch.equal(a[0].view(torch.int16), z[0].view(torch.int16))
        assert torch.equal(a[1], z[1])


def test_bitwise_deterministic(B):
    w = wl.custom_workload(6, 32, 8, 128, 64, [300, 2049, 1, 64, 999, 4000], "bf16", seed=41)
    t = dev(w)
    for S in (1, 5, BAL):
        a = run(B, w, S, t)
        b_ = run(B, w, S, t)
        assert torch.equal(a[0].view(torch.int16), b_[0].view(torch.int16)) and torch.equal(a[1], b_[1])


def test_bf16_and_fp8_interleaved_at_one_shape(B):
    """The same shape in both cache dtypes, called alternately, so one compiled
    variant cannot silently serve the other."""
    lens = [513, 64, 1000]
    wb = wl.custom_workload(3, 16, 2, 128, 64, lens, "bf16", seed=51)
    wf = wl.custom_workload(3, 16, 2, 128, 64, lens, "fp8_e4m3", seed=51)
    rb, rf = oracle_full(wb), oracle_full(wf)
    for S in (2, BAL, 2):
        check(*run(B, wb, S), *rb, what=f"bf16 S={S}")
        check(*run(B, wf, S), *rf, what=f"fp8 S={S}")


def test_fp8_every_finite_code_decodes_exactly(B):
    """Single-token sequences whose V rows hold every finite E4M3FN code with
    v_scale = 1: the output is the decoded code itself, exactly."""
    codes = [c for c in range(256) if c not in (0x7F, 0xFF)]
    d = 128
    nseq = -(-len(codes) // d)
    w = wl.custom_workload(nseq, 2, 1, d, 16, [1] * nseq, "fp8_e4m3", seed=61)
    flat = torch.tensor(codes + [0] * (nseq * d - len(codes)), dtype=torch.uint8)
    V = flat.view(nseq, 1, d).view(torch.float8_e4m3fn)
    w = wl.rebuild_with_rows(w, v_logical=V)
    w.v_scale = torch.ones(1)
    w.k_scale = torch.ones(1)
    out, _ = run(B, w, 1)
    want = V.view(nseq, d).to(torch.float32)
    for h in range(2):
        assert torch.equal(out[:, h].to(torch.float32), want)


def test_sharpened_attention(B):
    """q scaled by 4: attention is far from flat, so the absolute tolerance is not
    what makes the check pass.  Besides the acceptance bound, every element must
    meet the bound derived from the kernels' arithmetic.  The softmax weights
    enter the PV matrix product rounded to bf16 (relative error at most
    u = 2^-8 each) and the output is rounded to bf16 (at most u |out|); every
    other step is fp32.  So |out - ref| <= u (sum_t w_t |v_t| + |ref|) plus fp32
    accumulation, where w_t are the exact softmax weights; sum_t w_t |v_t| is the
    oracle run on |V|.  (With a dominant token this is about u |v_t*|: up to
    0.016 for |v| near 4, which is why a flat 4e-3 bound does not hold.)"""
    w = wl.custom_workload(4, 32, 8, 128, 64, [2048, 1024, 3000, 77], "bf16", seed=71)
    w = wl.rebuild_with_rows(w, q=(w.q.float() * 4).to(torch.bfloat16))
    ref = oracle_full(w)
    w_abs = wl.rebuild_with_rows(w, v_logical=w.v_logical.abs())
    wabs, _ = oracle_full(w_abs)
    u = 2.0 ** -8
    bound = 1.1 * u * (wabs + np.abs(ref[0])) + 1e-5
    for S in (1, 4, BAL):
        out, lse = run(B, w, S)
        check(out, lse, *ref, what=f"sharp S={S}")
        err = np.abs(out.double().numpy() - ref[0])
        assert np.all(err <= bound), f"S={S}: worst error / derived bound {(err / bound).max():.3g}"
        rms_err = float(np.sqrt(np.mean(err ** 2)))
        rms_ref = float(np.sqrt(np.mean(ref[0] ** 2)))
        assert rms_err <= 5e-3 * rms_ref, f"S={S}: rms error {rms_err:.3g} vs rms output {rms_ref:.3g}"


def test_partials_entry_matches_oracle_per_split(B):
    lens = [37, 300, 0, 64, 1025]
    w = wl.custom_workload(len(lens), 8, 2, 64, 16, lens, "bf16", seed=81)
    t = dev(w)
    dims = B.dims_for(t["q"], t["k"], t["bt"])
    S = 4
    R = len(lens) * 8
    o_part = torch.empty(R * S * 64, dtype=torch.float32, device="cuda")
    l_part = torch.empty(R * S, dtype=torch.float32, device="cuda")
    st = B.paged_decode_partials(dims, None, t["q"], t["k"], t["v"], t["bt"], t["lens"], None, None, w.scale,
                                 S, o_part, l_part, B.current_stream_handle(0))
    assert st == 0
    torch.cuda.synchronize()
    o_part = o_part.cpu().view(len(lens), 8, S, 64).double().numpy()
    l_part = l_part.cpu().view(len(lens), 8, S).double().numpy()
    cap = w.block_table.shape[1] * w.spec.page_size
    c = B.PKD_SPLIT_ALIGN * (-(-(-(-cap // S)) // B.PKD_SPLIT_ALIGN))
    for j in range(S):
        tb = [min(j * c, L) for L in lens]
        te = [min((j + 1) * c, L) for L in lens]
        ref_o, ref_l = oracle.paged_decode_ranges(w.q, w.k_cache, w.v_cache, w.block_table,
                                                  w.seq_lens, w.scale, tb, te)
        assert np.all(np.abs(o_part[:, :, j] - ref_o) <= 1e-2 + 1e-2 * np.abs(ref_o))
        inf = np.isneginf(ref_l)
        assert np.array_equal(np.isneginf(l_part[:, :, j]), inf)
        assert np.all(np.abs(np.where(inf, 0, l_part[:, :, j] - np.where(inf, 0, ref_l))) <= 1e-3)


@pytest.mark.parametrize("S", [9, 37, 100])
@pytest.mark.parametrize("d", [32, 64, 128, 256])
def test_merge_entry_matches_oracle(B, d, S):
    """S = 9, 37, 100 take the one-, four- and sixteen-waves-per-row merges."""
    rng = np.random.default_rng(d + S)
    R = 37
    o = rng.standard_normal((R, S, d)).astype(np.float32)
    l = (rng.standard_normal((R, S)) * 4).astype(np.float32)
    l[3, 2] = -np.inf
    l[5, :] = -np.inf
    l[7, :-1] = -np.inf
    l[9, 1:] = -np.inf
    out = torch.empty(R, d, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(R, dtype=torch.float32, device="cuda")
    st = B.paged_decode_merge(R, S, d, torch.from_numpy(o).cuda(), torch.from_numpy(l).cuda(), out, lse,
                              B.current_stream_handle(0))
    assert st == 0
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.lse_merge(o.astype(np.float64), l.astype(np.float64))
    check(out.cpu(), lse.cpu(), ref_o, ref_l, what=f"merge D={d}")
    assert torch.all(out[5].float().cpu() == 0)


def test_check_tables(B):
    w = wl.custom_workload(3, 4, 1, 64, 16, [37, 100, 0], "bf16", seed=91, max_pages=8)
    t = dev(w)
    dims = B.dims_for(t["q"], t["k"], t["bt"])
    cnt = torch.full((1,), -5, dtype=torch.int32, device="cuda")
    assert B.paged_decode_check_tables(dims, t["bt"], t["lens"], cnt, B.current_stream_handle(0)) == 0
    torch.cuda.synchronize()
    assert int(cnt.item()) == 0
    bt = t["bt"].clone()
    bt[0, 1] = w.num_pages   # a used entry out of range
    bt[1, 6] = -1            # a used entry of the second sequence
    bt[2, 0] = 12345         # unused (length 0): not inspected
    lens = t["lens"].clone()
    lens[2] = 10 ** 6        # longer than the block table allows
    assert B.paged_decode_check_tables(dims, bt, lens, cnt, B.current_stream_handle(0)) == 0
    torch.cuda.synchronize()
    assert int(cnt.item()) == 3


# ---- the balanced partition ---------------------------------------------------

@pytest.mark.parametrize("case", [
    # (lens, Hq, Hkv, D, ps, dtype)
    ([0, 5, 0, 3000, 1, 16, 17, 0], 8, 2, 128, 16, "bf16"),   # empty and one-group sequences
    ([1] * 300, 8, 8, 64, 16, "bf16"),                         # fewer groups than waves
    ([33] * 700 + [2000, 0, 1], 4, 1, 64, 64, "bf16"),         # many segments per wave
    ([4096, 1, 4095], 40, 2, 128, 64, "bf16"),                 # two head groups, the second partial
    ([513, 8192, 64, 700], 64, 8, 128, 64, "fp8_e4m3"),        # fp8, G = 8
    ([12000, 5], 16, 2, 256, 64, "bf16"),                      # D = 256
    ([3000] * 4, 16, 2, 32, 128, "fp8_e4m3"),                  # fp8 D = 32
])
def test_balanced_partition(B, case):
    lens, hq, hkv, d, ps, dtype = case
    w = wl.custom_workload(len(lens), hq, hkv, d, ps, lens, dtype, seed=len(lens) + d + ps)
    ref = oracle_full(w)
    out, lse = run(B, w, BAL)
    check(out, lse, *ref, what=f"balanced {case[1:]}")


def test_balanced_largest_batch(B):
    lens = [(i * 37) % 300 for i in range(1024)]
    w = wl.custom_workload(1024, 4, 2, 64, 32, lens, "bf16", seed=3)
    ref = oracle_full(w)
    check(*run(B, w, BAL), *ref, what="balanced B=1024")


# ---- whole items paired by length (PKD_SPLITS_PAIRED) ------------------------

def _paired_cases(cus):
    """(name, batch, Hq, Hkv, D, ps, lens, dtype, extra) around one and two items
    per compute unit: folded pairs, one item each, the equal-length and the
    more-than-two-per-unit fallbacks to the equal ranges, empty sequences."""
    b1 = cus // 8  # sequences with 8 KV heads that give one item per unit
    ragged = lambda n, lo, hi, seed: [int(x) for x in
                                      np.random.default_rng(seed).integers(lo, hi + 1, size=n)]
    return [
        ("pairs", b1 + 3, 32, 8, 128, 64, ragged(b1 + 3, 1, 900, 1), "bf16", {}),
        ("pairs_all", 2 * b1, 32, 8, 128, 64, ragged(2 * b1, 1, 700, 2), "bf16", {}),
        ("one_each", b1 - 5, 32, 8, 128, 64, ragged(b1 - 5, 1, 700, 3), "bf16", {}),
        ("equal_fallback", b1 + 1, 32, 8, 128, 64, [320] * (b1 + 1), "bf16", {}),
        ("over_two", 2 * b1 + 3, 16, 8, 64, 16, ragged(2 * b1 + 3, 1, 300, 4), "bf16", {}),
        ("empties", b1 + 6, 32, 8, 128, 64, [0, 0] + ragged(b1 + 4, 1, 600, 5), "bf16", {}),
        ("fp8", b1 + 9, 64, 8, 128, 64, ragged(b1 + 9, 1, 900, 6), "fp8_e4m3", {}),
        ("d32_wide_heads", b1 + 2, 16, 8, 32, 64, ragged(b1 + 2, 1, 800, 7), "bf16", {}),
        ("d256", b1 + 1, 16, 8, 256, 16, ragged(b1 + 1, 1, 300, 8), "bf16", {}),
        ("window_sinks", b1 + 4, 32, 8, 128, 64, ragged(b1 + 4, 1, 900, 9), "bf16",
         dict(window=200, sinks=True)),
        ("verify_causal", b1 + 2, 16, 8, 64, 64, ragged(b1 + 2, 4, 700, 10), "bf16",
         dict(q_len=3, causal=True)),
    ]


@pytest.mark.parametrize("idx", range(11))
def test_paired_mode(B, idx):
    """PKD_SPLITS_PAIRED against the oracle, in every branch of the device's
    plan (folded pairs, one item each, fallbacks to the equal ranges), with
    empty sequences, FP8, paired KV heads, windows, sinks and several query
    tokens; one launch, and its path query names it."""
    name, bq, hq, hkv, d, ps, lens, dtype, extra = _paired_cases(_cu_count())[idx]
    w = wl.custom_workload(bq, hq, hkv, d, ps, lens, dtype, seed=500 + idx, **extra)
    ref = oracle_full(w)
    t = dev(w)
    dims = B.dims_for(t["q"], t["k"], t["bt"])
    ext = B.ext_for(t["q"], w.spec.causal, w.spec.window)
    assert B.paged_decode_path(dims, ext, PAIR) == B.PKD_PATH_PAIRED
    assert B.paged_decode_launches(dims, ext, PAIR) == 1
    out, lse = run(B, w, PAIR, t)
    check(out, lse, *ref, what=f"paired {name}")
    # a second call on the same workspace contents gives the same bits
    out2, lse2 = run(B, w, PAIR, t)
    assert torch.equal(out2.view(torch.int16), out.view(torch.int16)) and torch.equal(lse2, lse)


def test_paired_mode_rejected_by_two_phases(B):
    """The two-phase entries take no paired mode: PKD_ERR_NUM_SPLITS, nothing written."""
    w = wl.custom_workload(4, 8, 2, 64, 16, [30, 1, 0, 90], "bf16", seed=31)
    t = dev(w)
    dims = B.dims_for(t["q"], t["k"], t["bt"])
    nbytes = B.paged_decode_workspace_bytes_ext(dims, None, PAIR)
    assert nbytes > 0
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    h = B.current_stream_handle(0)
    assert B.paged_decode_partition(dims, None, t["q"], t["k"], t["v"], t["bt"], t["lens"], None, None, w.scale,
                                    PAIR, ws, nbytes, h) == B.PKD_ERR_NUM_SPLITS
    torch.cuda.synchronize()
    assert int(ws.count_nonzero()) == 0


# ---- full-size workloads: every output element against the oracle -----------

FULL = ["llama_b32_d128_ps64", "batch128_d128_ps128", "longctx_b1_d32", "longctx_b1_d64",
        "longctx_b1_d256", "longctx_b16_d32", "longctx_b16_d64", "longctx_b16_d256",
        "fp8kv_b64_d128_ps64", "verify_b32_q4_d128_ps64", "window1k_sinks_b32_d128_ps64"]


def full_modes(spec):
    """The launch configurations a full-size workload is checked in: the
    library's own choice (the one the benchmark times), direct output, a fixed
    split count, the balanced partition and whole items paired by length."""
    return [0, 1, 8, BAL, PAIR]


@pytest.mark.parametrize("name", FULL)
def test_full_size_workload_every_row(B, name):
    """Every output row and LSE of each full-size workload, in every launch
    configuration, against the fp64 oracle on the same inputs (NaN tails,
    -1 padding)."""
    spec = wl.WORKLOADS[name]
    w = wl.make_workload(spec, tail="nan")
    t = dev(w)
    ref = oracle_full(w)
    for S in full_modes(spec):
        out, lse = run(B, w, S, t)
        check(out, lse, *ref, what=f"{name} S={S}")


TWO_PHASE_CASES = {
    "small": (5, 16, 2, 128, 64, [700, 1, 0, 3000, 64]),  # few segments: partition + merge kernel
    "b32": (32, 32, 8, 128, 64, [(i * 613) % 3500 + 1 for i in range(30)] + [0, 64]),
    "b24": (24, 32, 8, 128, 64, [(i * 613) % 3500 + 1 for i in range(22)] + [0, 64]),
}


@pytest.mark.parametrize("S,case", [(4, "small"), (BAL, "small"), (BAL, "b32"), (BAL, "b24")])
def test_two_phases_equal_paged_decode(B, S, case):
    """paged_decode_partition then paged_decode_finish is exactly paged_decode,
    also where paged_decode merges inside the partition kernel (b32)."""
    bq, hq, hkv, d, ps, lens = TWO_PHASE_CASES[case]
    w = wl.custom_workload(bq, hq, hkv, d, ps, lens, "bf16", seed=123)
    t = dev(w)
    ref_out, ref_lse = run(B, w, S, t)
    dims = B.dims_for(t["q"], t["k"], t["bt"])
    nbytes = B.paged_decode_workspace_bytes_ext(dims, None, S)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(t["q"])
    lse = torch.empty(t["q"].shape[:2], dtype=torch.float32, device="cuda")
    h = B.current_stream_handle(0)
    assert B.paged_decode_partition(dims, None, t["q"], t["k"], t["v"], t["bt"], t["lens"], None, None, w.scale,
                                    S, ws, nbytes, h) == 0
    assert B.paged_decode_finish(dims, None, S, ws, nbytes, None, out, lse, h) == 0
    torch.cuda.synchronize()
    assert torch.equal(out.cpu().view(torch.int16), ref_out.view(torch.int16))
    assert torch.equal(lse.cpu(), ref_lse)


def _cu_count():
    return torch.cuda.get_device_properties(0).multi_processor_count


@pytest.mark.parametrize("hkv,d,dtype,expect,above", [(8, 128, "bf16", 1, 1), (8, 64, "bf16", 1, PAIR),
                                                       (8, 32, "bf16", BAL, PAIR), (8, 128, "fp8_e4m3", BAL, 1),
                                                       (8, 64, "fp8_e4m3", BAL, PAIR)])
def test_auto_mode_around_one_item_per_cu(B, hkv, d, dtype, expect, above):
    """PKD_SPLITS_AUTO picks direct output for a bf16 cache with head rows of at
    least 128 bytes when the (sequence, KV head, head group) items number between
    three quarters of the compute units and all of them (one whole item per unit,
    nothing to merge); above that, up to two items per unit, whole items paired
    by length (the LDS-staged direct kernel's pairs form for D = 128, else the
    paired mode); elsewhere the balanced partition."""
    cus = _cu_count()
    if cus % hkv:
        pytest.skip("compute units not a multiple of the KV heads")
    kvd = B.PKD_DTYPE_FP8_E4M3 if dtype == "fp8_e4m3" else B.PKD_DTYPE_BF16
    for batch, want in ((cus // hkv // 2, BAL), (3 * cus // 4 // hkv, expect), (cus // hkv - 1, expect),
                        (cus // hkv, expect), (cus // hkv + 1, above), (2 * cus // hkv, above),
                        (2 * cus // hkv + 1, BAL)):
        dims = B.pkd_dims(batch, 4 * hkv, hkv, d, 64, 4096, 64, kvd)
        assert B.paged_decode_num_splits(dims, 0) == want, (batch, hkv, d, dtype)
        if want == 1 and d == 128:
            assert B.paged_decode_path(dims, None, 0) == B.PKD_PATH_DIRECT_LDS


def test_auto_few_long_items(B):
    """PKD_SPLITS_AUTO for at most one item per 64 compute units (a few long
    sequences): grid splits, about one workgroup per unit (units / items), capped
    by the longest sequence at 256 tokens per split; with more items, or short
    sequences, the other rules."""
    cus = _cu_count()
    if cus < 128:
        pytest.skip("fewer than 128 compute units")
    for hkv, mp in ((2, 2048), (1, 2048), (2, 40)):
        dims = B.pkd_dims(1, 16, hkv, 64, 64, 4096, mp, B.PKD_DTYPE_BF16)
        want = min(cus // hkv, -(-(mp * 64) // 256), B.PKD_MAX_SPLITS)  # hkv items
        assert B.paged_decode_num_splits(dims, 0) == want, (hkv, mp, want)
        assert B.paged_decode_path(dims, None, 0) == B.PKD_PATH_SPLITS
    # no sequence longer than 256 tokens: direct output comes first
    dims = B.pkd_dims(1, 16, 2, 64, 64, 4096, 4, B.PKD_DTYPE_BF16)
    assert B.paged_decode_num_splits(dims, 0) == 1
    # 16 sequences of 2 KV heads: 32 items, above one per 64 units -> balanced
    dims = B.pkd_dims(16, 16, 2, 64, 64, 8192, 512, B.PKD_DTYPE_BF16)
    if 32 * 64 > cus:
        assert B.paged_decode_num_splits(dims, 0) == BAL


def _lds_pairs_cases(cus):
    """(name, batch, Hq, Hkv, ps, lens, sinks) with between one and two (sequence,
    KV head) items per compute unit, for the LDS-staged kernel's pairs form."""
    b1 = cus // 8
    ragged = lambda n, lo, hi, seed: [int(x) for x in
                                      np.random.default_rng(seed).integers(lo, hi + 1, size=n)]
    return [
        ("ragged", b1 + 1, 32, 8, 64, ragged(b1 + 1, 1024, 4096, 11), False),
        ("two_per_unit", 2 * b1, 32, 8, 64, ragged(2 * b1, 1, 3000, 12), False),
        ("equal", b1 + 3, 32, 8, 64, [700] * (b1 + 3), False),
        ("empty_and_short", b1 + 5, 32, 8, 16, [0, 1, 0, 15, 16, 17] + ragged(b1 - 1, 1, 900, 13), False),
        ("sinks", b1 + 7, 32, 8, 64, ragged(b1 + 7, 1, 1500, 14), True),
        ("hkv2_g16", cus // 2 + 9, 32, 2, 48, ragged(cus // 2 + 9, 1, 400, 15), False),
    ]


@pytest.mark.parametrize("idx", range(6))
def test_lds_pairs_direct(B, idx):
    """Direct output for bf16 D = 128 with more items than compute units: the
    LDS-staged kernel deals one or two whole items per workgroup, paired by
    length on the device.  Against the oracle (NaN tails, -1 padding), and bit
    for bit against the same kernel launched one workgroup per item."""
    name, bq, hq, hkv, ps, lens, sinks = _lds_pairs_cases(_cu_count())[idx]
    w = wl.custom_workload(bq, hq, hkv, 128, ps, lens, "bf16", seed=700 + idx, sinks=sinks)
    t = dev(w)
    dims = B.dims_for(t["q"], t["k"], t["bt"])
    assert B.paged_decode_num_splits(dims, 0) == 1
    assert B.paged_decode_path(dims, None, 1) == B.PKD_PATH_DIRECT_LDS
    out, lse = run(B, w, 0, t)
    check(out, lse, *oracle_full(w), what=f"lds pairs {name}")
    if not sinks:
        out1, lse1 = run_lds(B, w, t)
        assert torch.equal(out.view(torch.int16), out1.view(torch.int16)) and torch.equal(lse, lse1)


def test_two_phases_reject_auto_direct(B):
    """Where PKD_SPLITS_AUTO resolves to direct output, the two-phase entries
    return PKD_ERR_NUM_SPLITS and write nothing."""
    cus = _cu_count()
    if cus % 8:
        pytest.skip("compute units not a multiple of 8")
    bq = cus // 8
    w = wl.custom_workload(bq, 32, 8, 128, 64, [(i * 613) % 3500 + 1 for i in range(bq)], "bf16", seed=124)
    t = dev(w)
    dims = B.dims_for(t["q"], t["k"], t["bt"])
    assert B.paged_decode_num_splits(dims, 0) == 1
    ws = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    h = B.current_stream_handle(0)
    assert B.paged_decode_partition(dims, None, t["q"], t["k"], t["v"], t["bt"], t["lens"], None, None, w.scale,
                                    0, ws, ws.numel(), h) == B.PKD_ERR_NUM_SPLITS
    torch.cuda.synchronize()
    assert int(ws.count_nonzero()) == 0
    # and paged_decode itself, with AUTO, matches the oracle
    out, lse = run(B, w, 0, t)
    check(out, lse, *oracle_full(w), what="AUTO direct at one item per compute unit")


@pytest.mark.parametrize("case", ["b32", "b5", "long"])
def test_plain_entry_heuristic(B, case):
    """paged_decode, the plain entry, with num_splits <= 0: every such value is
    the heuristic's choice, the workspace paged_decode_workspace_bytes gives for
    it suffices, and the result equals paged_decode_ext in the mode the heuristic
    names, bit for bit, and the oracle."""
    shapes = {"b32": (32, 32, 8, 128, 64, [(i * 613) % 3500 + 1 for i in range(32)]),
              "b5": (5, 32, 8, 128, 64, [700, 2, 0, 3000, 64]),
              "long": (1, 16, 2, 64, 64, [20000])}
    bq, hq, hkv, d, ps, lens = shapes[case]
    w = wl.custom_workload(bq, hq, hkv, d, ps, lens, "bf16", seed=125)
    t = dev(w)
    dims = B.dims_for(t["q"], t["k"], t["bt"])
    chosen = B.paged_decode_num_splits(dims, 0)
    nbytes = B.paged_decode_workspace_bytes(dims, 0)
    assert nbytes == B.paged_decode_workspace_bytes_ext(dims, None, chosen)
    h = B.current_stream_handle(0)
    ref_out, ref_lse = run(B, w, chosen, t)
    for S in (0, -1, -77):
        ws = torch.full((max(nbytes, 1),), 0xA5, dtype=torch.uint8, device="cuda")
        out = torch.empty_like(t["q"])
        lse = torch.empty(t["q"].shape[:2], dtype=torch.float32, device="cuda")
        assert B.paged_decode(dims, t["q"], t["k"], t["v"], t["bt"], t["lens"], None, None, w.scale, out, lse, S,
                              ws if nbytes else None, nbytes, h) == 0
        torch.cuda.synchronize()
        assert torch.equal(out.cpu().view(torch.int16), ref_out.view(torch.int16)), (case, S)
        assert torch.equal(lse.cpu().view(torch.int32), ref_lse.view(torch.int32)), (case, S)
    check(ref_out, ref_lse, *oracle_full(w), what=f"plain entry heuristic {case}")


@pytest.mark.parametrize("S,nseq", [(BAL, 32), (4, 32), (1, 32), (PAIR, 32), (PAIR, 40), (0, 40)])
def test_graph_replays(B, S, nseq):
    """A captured decode replays correctly several times, with eager work and
    synchronisations between the replays, and matches the eager call bitwise.
    The call tag of the in-place merge's counters is fixed at capture, so every
    replay reuses it (the paired mode's fallback at 32 sequences merges in
    place; at 40 sequences it deals pairs, and AUTO runs the LDS-staged pairs
    form)."""
    lens = [(i * 1543) % 6000 + 100 for i in range(nseq)]
    w = wl.custom_workload(nseq, 32, 8, 128, 64, lens, "bf16", seed=21)
    t = dev(w)
    dims = B.dims_for(t["q"], t["k"], t["bt"])
    nbytes = B.paged_decode_workspace_bytes_ext(dims, None, S)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(t["q"])
    lse = torch.empty(t["q"].shape[:2], dtype=torch.float32, device="cuda")
    eager_out, eager_lse = run(B, w, S, t)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            st = B.paged_decode_ext(dims, None, t["q"], t["k"], t["v"], t["bt"], t["lens"], None, None, None,
                                    w.scale, out, lse, S, ws if nbytes else None, nbytes,
                                    B.current_stream_handle(0))
    torch.cuda.current_stream().wait_stream(side)
    assert st == 0
    for i in range(4):
        out.fill_(0)
        lse.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.cpu().view(torch.int16), eager_out.view(torch.int16)), f"replay {i}: out"
        assert torch.equal(lse.cpu().view(torch.int32), eager_lse.view(torch.int32)), f"replay {i}: lse"


def test_in_kernel_merge_ignores_workspace_contents(B):
    """The balanced mode that merges in place needs no initialised workspace:
    garbage, zeros and the words a previous call left give the same bits."""
    lens = [(i * 997) % 4000 + 1 for i in range(40)] + [0] * 3
    w = wl.custom_workload(len(lens), 32, 8, 128, 64, lens, "bf16", seed=77)
    t = dev(w)
    dims = B.dims_for(t["q"], t["k"], t["bt"])
    assert B.paged_decode_launches(dims, None, BAL) == 1
    nbytes = B.paged_decode_workspace_bytes_ext(dims, None, BAL)
    outs = []
    for fill in (0xFF, 0x00, None, 0x5A):
        ws = torch.full((nbytes,), fill if fill is not None else 0, dtype=torch.uint8, device="cuda")
        if fill is None:  # a workspace that a previous call has used
            B.decode(t["q"], t["k"], t["v"], t["bt"], t["lens"], w.scale, num_splits=BAL, workspace=ws)
        out, lse = B.decode(t["q"], t["k"], t["v"], t["bt"], t["lens"], w.scale, num_splits=BAL, workspace=ws)
        torch.cuda.synchronize()
        outs.append((out.cpu().view(torch.int16), lse.cpu().view(torch.int32)))
    for o, l in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1])
    check(outs[0][0].view(torch.bfloat16), outs[0][1].view(torch.float32), *oracle_full(w), what="in-kernel merge")


# ---- several query tokens per sequence (speculative verify / extend) --------

MULTI_CASES = [
    # (B, Hq, Hkv, D, ps, seq_lens, q_len, causal, dtype, seed)
    (4, 8, 2, 64, 16, [1, 3, 37, 200], 4, True, "bf16", 301),      # L < q_len: rows that see nothing
    (3, 32, 8, 128, 64, [700, 64, 2], 4, True, "bf16", 302),      # G = 4, q_len = 4: one full group of 16
    (3, 16, 2, 128, 16, [100, 513, 17], 3, True, "bf16", 303),    # G = 8, q_len = 3: 24 rows, partial 2nd group
    (2, 8, 8, 64, 24, [50, 77], 5, True, "bf16", 304),            # ps = 24: per-row page lookups
    (3, 8, 2, 128, 64, [0, 130, 65], 2, False, "bf16", 305),      # no mask, an empty sequence
    (3, 16, 2, 128, 64, [40, 300, 7], 8, True, "fp8_e4m3", 306),  # FP8, 64 rows per KV head
    (2, 4, 1, 256, 16, [33, 90], 16, True, "bf16", 307),          # D = 256, q_len = 16
    (2, 4, 4, 32, 16, [20, 45], 6, True, "bf16", 308),            # G = 1, D = 32
]


@pytest.mark.parametrize("case", MULTI_CASES)
def test_multi_token_parity(B, case):
    bq, hq, hkv, d, ps, lens, ql, causal, dtype, seed = case
    w = wl.custom_workload(bq, hq, hkv, d, ps, lens, dtype, seed, q_len=ql, causal=causal)
    ref = oracle_full(w)
    t = dev(w)
    for S in (1, 3, 0) + ((BAL,) if ps % 16 == 0 else ()):
        out, lse = run(B, w, S, t)
        assert out.shape == (bq, ql, hq, d) and lse.shape == (bq, ql, hq)
        check(out, lse, *ref, what=f"multi {case} S={S}")


def test_multi_with_one_query_token_is_decode_bitwise(B):
    lens = [5, 130, 64, 1, 700]
    w = wl.custom_workload(len(lens), 32, 8, 128, 64, lens, "bf16", seed=311)
    t = dev(w)
    q4 = t["q"].unsqueeze(1).contiguous()
    for S in (1, 4, BAL):
        ref_o, ref_l = run(B, w, S, t)
        for causal in (False, True):
            o, l = B.decode(q4, t["k"], t["v"], t["bt"], t["lens"], w.scale, num_splits=S, causal=causal)
            torch.cuda.synchronize()
            assert torch.equal(o.cpu()[:, 0].view(torch.int16), ref_o.view(torch.int16))
            assert torch.equal(l.cpu()[:, 0].view(torch.int32), ref_l.view(torch.int32))


def test_multi_token_one_hot_probe_sees_exactly_its_prefix(B):
    """Causal bit-exact probe: K[t][0] = 4096 at two tokens of each sequence, the
    last position (visible to the last query token only) and position L - q_len
    (visible to all).  With q = e_0 every query token but the last must return
    V at L - q_len bit for bit, and the last the bf16 mean of the two V rows is
    not bit-defined, so it is checked against the oracle instead."""
    ql = 4
    lens = [4, 37, 64, 129]
    d = 64
    w = wl.custom_workload(len(lens), 8, 2, d, 16, lens, "bf16", seed=312, q_len=ql, causal=True)
    q = torch.zeros_like(w.q)
    q[..., 0] = 1.0
    k = torch.zeros_like(w.k_logical)
    offs = w.token_offsets
    for b, L in enumerate(lens):
        k[int(offs[b]) + L - ql, :, 0] = 4096.0
        k[int(offs[b]) + L - 1, :, 0] = 4096.0
    w = wl.rebuild_with_rows(w, q=q, k_logical=k)
    t = dev(w)
    ref_o, ref_l = oracle_full(w)
    for S in (1, 3, BAL):
        out, lse = run(B, w, S, t)
        check(out, lse, ref_o, ref_l, what=f"multi one-hot S={S}")
        for b, L in enumerate(lens):
            vrow = w.v_logical[int(offs[b]) + L - ql]  # [Hkv, D]
            for i in range(ql - 1):
                for h in range(8):
                    assert torch.equal(out[b, i, h].view(torch.int16), vrow[h // 4].view(torch.int16)), (S, b, i, h)


def test_multi_verify_workload_modes(B):
    """The B=32 verify step (4 query tokens per sequence, causal) at full size:
    every row against the oracle in every mode, and AUTO runs exactly the mode
    it resolves to."""
    spec = wl.WORKLOADS["verify_b32_q4_d128_ps64"]
    w = wl.make_workload(spec, tail="nan")
    t = dev(w)
    ref = oracle_full(w)
    dims, e = B.dims_for(t["q"], t["k"], t["bt"]), B.ext_for(t["q"], causal=True)
    assert B.paged_decode_launches(dims, e, BAL) == 1  # 256 segments: merged in place
    outs = {}
    for S in (BAL, 0, 1, 8):
        out, lse = run(B, w, S, t)
        check(out, lse, *ref, what=f"verify S={S}")
        outs[S] = (out, lse)
    s_auto = B.paged_decode_num_splits_ext(dims, e, 0)
    assert s_auto in outs
    assert torch.equal(outs[s_auto][0].view(torch.int16), outs[0][0].view(torch.int16))


@pytest.mark.parametrize("lens", [[(i * 613) % 3500 + 1 for i in range(30)] + [0, 3], [700, 2, 0, 3000, 64]])
def test_multi_two_phases_equal_paged_decode(B, lens):
    """Balanced mode with several query tokens: partition + finish equals
    paged_decode bitwise, whether paged_decode merges in place (32 sequences) or
    not (5 sequences)."""
    w = wl.custom_workload(len(lens), 32, 8, 128, 64, lens, "bf16", seed=313, q_len=4, causal=True)
    t = dev(w)
    ref_out, ref_lse = run(B, w, BAL, t)
    dims, e = B.dims_for(t["q"], t["k"], t["bt"]), B.ext_for(t["q"], causal=True)
    nbytes = B.paged_decode_workspace_bytes_ext(dims, e, BAL)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(t["q"])
    lse = torch.empty(t["q"].shape[:-1], dtype=torch.float32, device="cuda")
    h = B.current_stream_handle(0)
    assert B.paged_decode_partition(dims, e, t["q"], t["k"], t["v"], t["bt"], t["lens"], None, None, w.scale, BAL,
                                    ws, nbytes, h) == 0
    assert B.paged_decode_finish(dims, e, BAL, ws, nbytes, None, out, lse, h) == 0
    torch.cuda.synchronize()
    assert torch.equal(out.cpu().view(torch.int16), ref_out.view(torch.int16))
    assert torch.equal(lse.cpu().view(torch.int32), ref_lse.view(torch.int32))
    check(out.cpu(), lse.cpu(), *oracle_full(w), what="multi two phases")


# ---- balanced mode: more segment and piece structures --------------------------

BALANCED_CASES = [
    # (B, Hq, Hkv, D, ps, seq_lens, seed): what the case exercises
    (8, 32, 8, 128, 64, [0, 1, 15, 16, 17, 700, 0, 3000], 401),                  # edge lengths, merge kernel
    (40, 32, 8, 64, 16, [(i * 977) % 500 + 1 for i in range(36)] + [0] * 4, 402),  # in-place merge
    (4, 128, 4, 128, 16, [33, 1000, 0, 5], 403),                                   # G = 32: two head groups
    (34, 16, 16, 32, 32, [(i * 331) % 900 + 1 for i in range(34)], 404),           # G = 1 at 16 KV heads
    (1, 64, 8, 128, 16, [100000], 405),                                            # one sequence over all workgroups
    (32, 32, 8, 128, 64, [60000] + [16] * 31, 406),                                # in place, > 8 partials per row
]


@pytest.mark.parametrize("case", BALANCED_CASES)
def test_balanced_structures_parity(B, case):
    bq, hq, hkv, d, ps, lens, seed = case
    w = wl.custom_workload(bq, hq, hkv, d, ps, lens, "bf16", seed)
    ref = oracle_full(w)
    t = dev(w)
    out, lse = run(B, w, BAL, t)
    check(out, lse, *ref, what=f"balanced {case[:5]}")
    # the two phases give the same bits as paged_decode
    dims = B.dims_for(t["q"], t["k"], t["bt"])
    nbytes = B.paged_decode_workspace_bytes_ext(dims, None, BAL)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    o2 = torch.empty_like(t["q"])
    l2 = torch.empty(t["q"].shape[:-1], dtype=torch.float32, device="cuda")
    h = B.current_stream_handle(0)
    assert B.paged_decode_partition(dims, None, t["q"], t["k"], t["v"], t["bt"], t["lens"], None, None, w.scale,
                                    BAL, ws, nbytes, h) == 0
    assert B.paged_decode_finish(dims, None, BAL, ws, nbytes, None, o2, l2, h) == 0
    torch.cuda.synchronize()
    assert torch.equal(o2.cpu().view(torch.int16), out.view(torch.int16))
    assert torch.equal(l2.cpu().view(torch.int32), lse.view(torch.int32))


# ---- paged KV append (quantised cache write with optional RoPE) --------------------

APPEND_CASES = [
    # (N, Hkv, D, page_size, num_pages, kv dtype, rope, seed)
    (37, 2, 32, 16, 4, "bf16", False, 501),
    (64, 8, 128, 64, 3, "bf16", True, 502),
    (50, 4, 64, 16, 8, "fp8_e4m3", False, 503),
    (129, 8, 128, 64, 4, "fp8_e4m3", True, 504),
    (20, 1, 256, 16, 2, "fp8_e4m3", True, 505),
    (700, 2, 256, 128, 8, "bf16", True, 506),
]


def _dev_append(w):
    c = torch.device("cuda:0")
    d = lambda t: None if t is None else t.to(c)
    return dict(k_new=d(w.k_new), v_new=d(w.v_new), slot_mapping=d(w.slot_mapping), positions=d(w.positions),
                cos_sin=d(w.cos_sin), k_cache=d(w.k_cache).clone(), v_cache=d(w.v_cache).clone(),
                k_scale=d(w.k_scale), v_scale=d(w.v_scale))


@pytest.mark.parametrize("case", APPEND_CASES)
def test_append_matches_oracle_bitwise(B, case):
    n, hkv, d, ps, pages, dtype, rope, seed = case
    w = wl.append_workload(n, hkv, d, ps, pages, dtype, rope=rope, seed=seed, pad_every=9)
    ref_k, ref_v = oracle.kv_append(w.k_new, w.v_new, w.slot_mapping, w.k_cache, w.v_cache, w.k_scale,
                                    w.v_scale, w.positions, w.cos_sin)
    t = _dev_append(w)
    B.append(**t)
    torch.cuda.synchronize()
    got_k = wl.as_numpy_bits(t["k_cache"].cpu())
    got_v = wl.as_numpy_bits(t["v_cache"].cpu())
    assert np.array_equal(got_k, ref_k.reshape(got_k.shape)), f"K cache differs {case}"
    assert np.array_equal(got_v, ref_v.reshape(got_v.shape)), f"V cache differs {case}"


@pytest.mark.parametrize("dtype", ["bf16", "fp8_e4m3"])
def test_append_rope_against_fp64_rotation(B, dtype):
    """The kernel's rotated K rows against the rotation computed in fp64 (not only against
    the oracle's fp32 recipe): every stored value within half a code step plus the fp32
    recipe's error bound, codes within one of the exact code where the two terms do not
    cancel, and nearly all exactly the exact code."""
    import rope_reference as rr
    w = wl.append_workload(2000, 8, 128, 64, 40, dtype, rope=True, seed=512, scale_range=(0.01, 0.05))
    t = _dev_append(w)
    B.append(**t)
    torch.cuda.synchronize()
    worst, exact_share, dist = rr.check(w, wl.as_numpy_bits(t["k_cache"].cpu()), dtype)
    assert worst <= 1.0, f"error / derived bound {worst:.3g}"
    assert dist <= 1
    assert exact_share > 0.99


def test_append_fp8_conversion_on_every_bf16_value(B):
    """Scale 1: every bf16 value in [-448, 448], including exact midpoints between FP8 codes,
    is encoded by the kernel exactly as by the oracle's nearest-code, ties-to-even rule."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16)
    f = vals.to(torch.float32)
    vals = vals[torch.isfinite(f) & (f.abs() <= 448)]
    d = 128
    rows = -(-vals.numel() // d)
    padded = torch.zeros(rows * d, dtype=torch.bfloat16)
    padded[: vals.numel()] = vals
    k_new = padded.view(rows, 1, d)
    w = wl.append_workload(rows, 1, d, 16, -(-rows // 16), "fp8_e4m3", seed=507)
    w.k_new, w.v_new = k_new, k_new.flip(0).contiguous()
    w.slot_mapping = torch.arange(rows, dtype=torch.int64)
    w.k_scale = torch.ones(1)
    w.v_scale = torch.ones(1)
    ref_k, ref_v = oracle.kv_append(w.k_new, w.v_new, w.slot_mapping, w.k_cache, w.v_cache, w.k_scale, w.v_scale)
    t = _dev_append(w)
    B.append(**t)
    torch.cuda.synchronize()
    assert np.array_equal(wl.as_numpy_bits(t["k_cache"].cpu()), ref_k)
    assert np.array_equal(wl.as_numpy_bits(t["v_cache"].cpu()), ref_v)


def test_append_then_decode(B):
    """Fill a cache by appending every token of three sequences (FP8, RoPE off), then decode:
    the result matches the oracle decode of the oracle-filled cache."""
    lens = [37, 100, 64]
    ps, hkv, hq, d = 16, 2, 8, 64
    w = wl.custom_workload(len(lens), hq, hkv, d, ps, lens, "fp8_e4m3", seed=508)
    # the logical rows as bf16 values to append, and the slot of every token
    kl = (w.k_logical.to(torch.float32) * w.k_scale.view(1, -1, 1)).to(torch.bfloat16)
    vl = (w.v_logical.to(torch.float32) * w.v_scale.view(1, -1, 1)).to(torch.bfloat16)
    slots = []
    for b, L in enumerate(lens):
        for tok in range(L):
            slots.append(int(w.block_table[b, tok // ps]) * ps + tok % ps)
    slots = torch.tensor(slots, dtype=torch.int64)
    empty = torch.zeros_like(w.k_cache.view(torch.uint8)).view(torch.float8_e4m3fn)
    ref_k, ref_v = oracle.kv_append(kl, vl, slots, empty, empty, w.k_scale, w.v_scale)
    c = torch.device("cuda:0")
    kc, vc = empty.to(c).clone(), empty.to(c).clone()
    B.append(kl.to(c), vl.to(c), slots.to(c), kc, vc, w.k_scale.to(c), w.v_scale.to(c))
    torch.cuda.synchronize()
    assert np.array_equal(wl.as_numpy_bits(kc.cpu()), ref_k) and np.array_equal(wl.as_numpy_bits(vc.cpu()), ref_v)
    ref_o, ref_l = oracle.paged_decode(w.q, kc.cpu(), vc.cpu(), w.block_table, w.seq_lens, w.scale, w.k_scale,
                                       w.v_scale)
    out, lse = B.decode(w.q.to(c), kc, vc, w.block_table.to(c), w.seq_lens.to(c), w.scale, w.k_scale.to(c),
                        w.v_scale.to(c), num_splits=0)
    torch.cuda.synchronize()
    check(out.cpu(), lse.cpu(), ref_o, ref_l, what="append then decode")


# ---- sliding window and attention sinks ------------------------------------

WINDOW_CASES = [
    # (B, Hq, Hkv, D, ps, seq_lens, q_len, causal, window, sinks, dtype, seed)
    (8, 16, 4, 128, 16, [0, 1, 63, 64, 65, 200, 1000, 17], 1, False, 64, False, "bf16", 401),
    (4, 8, 2, 64, 16, [1, 2, 17, 300], 1, False, 1, True, "bf16", 402),        # the last token only
    (3, 32, 4, 128, 64, [700, 50, 0], 1, False, 100, True, "bf16", 403),       # window not a multiple of 16
    (3, 16, 4, 128, 16, [3, 40, 500], 4, True, 32, True, "bf16", 404),         # q_len 4 under the causal mask
    (3, 8, 2, 128, 64, [90, 600, 5], 3, False, 20, True, "fp8_e4m3", 405),     # no mask, FP8
    (3, 8, 2, 128, 24, [50, 333, 1], 2, True, 50, True, "bf16", 406),          # ps 24: per-row page lookups
    (3, 8, 2, 64, 16, [10, 300, 0], 1, False, 10000, True, "bf16", 407),       # window past every length
    (2, 4, 4, 32, 16, [20, 45], 1, False, 16, False, "bf16", 408),             # D 32, G 1
    (2, 8, 1, 256, 64, [129, 700], 8, True, 70, True, "bf16", 409),            # D 256, q_len 8
    (3, 8, 2, 128, 64, [4, 300, 0], 6, True, 0, True, "bf16", 410),            # sinks alone; L < q_len
]


def first_group(L, q_len, window):
    """First token a sequence's splits start at: its lowest window start rounded
    down to a multiple of 16 (0 without a window)."""
    return (max(L - q_len - window + 1, 0) // 16) * 16 if window > 0 else 0


def poison_below_window(w):
    """NaN in every K and V row below each sequence's first visible 16-token
    group: the kernels must never read them (the oracle does not either)."""
    kc, vc = w.k_cache.clone(), w.v_cache.clone()
    nan = float("nan")
    ps = w.spec.page_size
    for b, L in enumerate(w.seq_lens.tolist()):
        for t_ in range(first_group(L, w.spec.q_len, w.spec.window)):
            page = int(w.block_table[b, t_ // ps])
            if kc.dtype == torch.float8_e4m3fn:
                kc.view(torch.uint8)[page, t_ % ps] = 0x7F  # an E4M3FN NaN code
                vc.view(torch.uint8)[page, t_ % ps] = 0x7F
            else:
                kc[page, t_ % ps] = nan
                vc[page, t_ % ps] = nan
    return kc, vc


@pytest.mark.parametrize("case", WINDOW_CASES)
def test_window_and_sinks_parity(B, case):
    """Every split mode against the oracle, with K/V below the window poisoned."""
    bq, hq, hkv, d, ps, lens, ql, causal, win, sinks, dtype, seed = case
    w = wl.custom_workload(bq, hq, hkv, d, ps, lens, dtype, seed, q_len=ql, causal=causal, window=win,
                           sinks=sinks)
    kc, vc = poison_below_window(w)
    w = dataclasses.replace(w, k_cache=kc, v_cache=vc)
    ref = oracle_full(w)
    t = dev(w)
    for S in (1, 3, 0) + ((BAL,) if ps % 16 == 0 else ()):
        out, lse = run(B, w, S, t)
        check(out, lse, *ref, what=f"window {case} S={S}")
    if sinks:
        # Empty rows carry the sink as their LSE and a zero output.
        ref_l = ref[1].reshape(bq, ql, hq)
        for b, L in enumerate(lens):
            if L == 0:
                assert np.allclose(ref_l[b], w.sinks.numpy()[None, :].astype(np.float64), atol=1e-6)


def test_window_ignores_pages_below_it_bitwise(B):
    """With a window of W, dropping the whole pages below each sequence's window
    (shifting its block-table row and length) changes no bit of the result."""
    ps, win = 16, 48  # window a multiple of the page size: the shifted table is whole pages
    lens = [300, 48, 49, 500, 17]
    w = wl.custom_workload(len(lens), 16, 4, 128, ps, lens, "bf16", seed=420, window=win)
    t = dev(w)
    bt_short = torch.full_like(w.block_table, -1)
    lens_short = []
    for b, L in enumerate(lens):
        drop = max(L - win, 0) // ps  # whole pages below the window
        n = -(-L // ps) - drop
        bt_short[b, :n] = w.block_table[b, drop:drop + n]
        lens_short.append(L - drop * ps)
    t2 = dict(t, bt=bt_short.cuda(), lens=torch.tensor(lens_short, dtype=torch.int32, device="cuda"))
    for S in (1, BAL):
        o1, l1 = run(B, w, S, t)
        o2, l2 = run(B, w, S, t2)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), S
        assert torch.equal(l1, l2), S


@pytest.mark.parametrize("S", [4, BAL])
def test_two_phases_fold_sinks(B, S):
    """paged_decode_finish folds the sinks in exactly as paged_decode does."""
    lens = [700, 1, 0, 3000, 64]
    w = wl.custom_workload(len(lens), 16, 2, 128, 64, lens, "bf16", seed=430, window=500, sinks=True)
    t = dev(w)
    ref_out, ref_lse = run(B, w, S, t)
    dims, e = B.dims_for(t["q"], t["k"], t["bt"]), B.ext_for(t["q"], window=500)
    nbytes = B.paged_decode_workspace_bytes_ext(dims, e, S)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(t["q"])
    lse = torch.empty(t["q"].shape[:2], dtype=torch.float32, device="cuda")
    h = B.current_stream_handle(0)
    assert B.paged_decode_partition(dims, e, t["q"], t["k"], t["v"], t["bt"], t["lens"], None, None, w.scale, S,
                                    ws, nbytes, h) == 0
    assert B.paged_decode_finish(dims, e, S, ws, nbytes, t["sinks"], out, lse, h) == 0
    torch.cuda.synchronize()
    assert torch.equal(out.cpu().view(torch.int16), ref_out.view(torch.int16))
    assert torch.equal(lse.cpu(), ref_lse)


def test_window_sinks_workload_poisoned_below_window(B):
    """The B=32 step with a 1024-token window and sinks at full size, with every
    K/V row below each sequence's window start set to NaN: every row against the
    oracle in every mode (a read below the window would show as NaN)."""
    spec = wl.WORKLOADS["window1k_sinks_b32_d128_ps64"]
    w = wl.make_workload(spec, tail="nan")
    kc, vc = poison_below_window(w)
    w = dataclasses.replace(w, k_cache=kc, v_cache=vc)
    t = dev(w)
    ref = oracle_full(w)
    for S in (BAL, 0, 1, 8):
        out, lse = run(B, w, S, t)
        check(out, lse, *ref, what=f"window S={S}")


# ---- decode metadata preparation ---------------------------------------------

def token_map(bt, lens, ps, req_rows, stride, seed):
    """req_to_token pool holding block tables bt in shuffled request rows (token t
    of sequence b at slot bt[b][t // ps] * ps + t % ps), random elsewhere."""
    rng = np.random.default_rng(seed)
    B = bt.shape[0]
    rt = rng.integers(-5, 10 ** 6, size=(req_rows, stride)).astype(np.int32)
    rows = rng.permutation(req_rows)[:B]
    for b in range(B):
        L = int(lens[b])
        t = np.arange(L)
        rt[rows[b], :L] = bt[b, t // ps] * ps + t % ps
    return rt, rows.astype(np.int64)


def meta_device(B, rt, rows, lens, ps, MP, q_len=1, window=0, extend=0):
    cuda = torch.device("cuda:0")
    res = B.metadata(torch.from_numpy(rt).to(cuda), torch.from_numpy(rows).to(cuda),
                     torch.from_numpy(np.asarray(lens, np.int64)).to(cuda), ps, MP, q_len=q_len, window=window,
                     extend=extend)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in res.items()}


META_CASES = [
    # (B, ps, MP, q_len, window, extend, seed)
    (5, 16, 8, 1, 0, 1, 501),
    (7, 1, 40, 1, 9, 0, 502),
    (9, 24, 6, 3, 50, 2, 503),
    (300, 64, 16, 1, 200, 1, 504),     # more entries than one scan chunk
    (1000, 16, 4, 4, 7, 0, 505),       # several chunks
    (0, 16, 4, 1, 5, 0, 506),          # empty batch
]


@pytest.mark.parametrize("case", META_CASES)
def test_metadata_matches_oracle_bitwise(B, case):
    bq, ps, MP, ql, win, ext, seed = case
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, MP * ps - ext + 1, size=bq)
    if bq > 2:
        lens[0], lens[1] = 0, MP * ps - ext
    bt = rng.integers(0, 5000, size=(bq, MP)).astype(np.int32)
    rt, rows = token_map(bt, lens + ext, ps, bq + 5, MP * ps + 3, seed)
    if bq > 4:
        rows[2] = bq + 5          # invalid request row
        lens[3] = MP * ps         # too long once extended (when ext > 0)
        rows[4] = -1
    ref, bad = oracle.decode_metadata(rt, rows, lens.astype(np.int64), ps, MP, q_len=ql, window=win, extend=ext)
    got = meta_device(B, rt, rows, lens, ps, MP, ql, win, ext)
    for k, v in ref.items():
        assert np.array_equal(got[k], v), k
    assert int(got["error_count"][0]) == bad


def test_metadata_feeds_decode_bitwise(B):
    """Decode on device-built tables equals decode on the original ones, and the
    window tables decode to the same bits as the full tables with the window."""
    lens = [(i * 997) % 3000 + 1 for i in range(24)] + [0, 64, 4096]
    w = wl.custom_workload(len(lens), 32, 8, 128, 64, lens, "bf16", seed=510, window=700, sinks=True)
    t = dev(w)
    MP = w.block_table.shape[1]
    bt = w.block_table.numpy()
    rt, rows = token_map(np.where(bt < 0, 0, bt), lens, 64, len(lens) + 7, MP * 64, seed=511)
    m = meta_device(B, rt, rows, lens, 64, MP, window=700)
    assert int(m["error_count"][0]) == 0
    for S in (1, BAL, 0):
        ref_o, ref_l = run(B, w, S, t)
        for bt_key, len_key in (("page_table", "cache_seqlens"), ("swa_page_table", "swa_seqlens")):
            t2 = dict(t, bt=torch.from_numpy(m[bt_key]).cuda(), lens=torch.from_numpy(m[len_key]).cuda())
            o, l = run(B, w, S, t2)
            assert torch.equal(o.view(torch.int16), ref_o.view(torch.int16)), (S, bt_key)
            assert torch.equal(l, ref_l), (S, bt_key)


# ---- contiguous K/V with stride-based addressing -------------------------------

CONTIG_GPU_CASES = [
    # (B, Hq, Hkv, D, seq_lens, q_len, causal, window, sinks, dtype, seed)
    (4, 8, 2, 128, [1, 37, 200, 0], 1, False, 0, False, "bf16", 701),
    (3, 16, 2, 64, [513, 17, 90], 3, True, 40, True, "bf16", 702),
    (3, 8, 2, 128, [300, 64, 5], 2, False, 0, True, "fp8_e4m3", 703),
    (2, 4, 4, 256, [129, 33], 4, True, 0, False, "bf16", 704),
    (2, 8, 8, 32, [70, 1], 1, False, 16, True, "bf16", 705),
]


def contig_dev(w, layout, strided_out):
    cuda = torch.device("cuda:0")
    k, v = wl.contiguous_kv(w, layout, capacity=int(w.seq_lens.max()) + 5)
    # Keep the views' strides on the device: move whole storages, then re-view.
    def to_dev(x):
        base = torch.empty(0, dtype=x.dtype).set_(x.untyped_storage()).to(cuda)
        return base.as_strided(x.shape, x.stride(), x.storage_offset())
    q = wl.strided_q(w.q)
    t = dict(q=to_dev(q), k=to_dev(k), v=to_dev(v), lens=w.seq_lens.to(cuda))
    t["ks"] = None if w.k_scale is None else w.k_scale.to(cuda)
    t["vs"] = None if w.v_scale is None else w.v_scale.to(cuda)
    t["sinks"] = None if w.sinks is None else w.sinks.to(cuda)
    if strided_out:
        buf = torch.full(w.q.shape[:-2] + (w.q.shape[-2] + 3, w.q.shape[-1]), float("nan"), dtype=torch.bfloat16,
                         device=cuda)
        t["out"] = buf[..., 2:2 + w.q.shape[-2], :]
    else:
        t["out"] = None
    return t, k, v, q


def run_contig(B, w, t, S):
    out, lse = B.contiguous(t["q"], t["k"], t["v"], t["lens"], w.scale, t["ks"], t["vs"], num_splits=S,
                            out=t["out"], causal=w.spec.causal, window=w.spec.window, sinks=t["sinks"])
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


@pytest.mark.parametrize("case", CONTIG_GPU_CASES)
@pytest.mark.parametrize("layout", ["blhd", "bhld", "blhd_padded"])
def test_contiguous_parity(B, case, layout):
    """Every split mode against the oracle in three K/V layouts, with a strided
    q and (padded layout) a strided out; NaN in every element that is not a
    sequence row, so that any stray read shows."""
    bq, hq, hkv, d, lens, ql, causal, win, sinks, dtype, seed = case
    w = wl.custom_workload(bq, hq, hkv, d, 16, lens, dtype, seed, q_len=ql, causal=causal, window=win, sinks=sinks)
    t, k, v, q = contig_dev(w, layout, strided_out=layout == "blhd_padded")
    ref = oracle.contiguous_decode(q, k, v, w.seq_lens, w.scale, causal, win, w.sinks, w.k_scale, w.v_scale)
    for S in (1, 3, 0, BAL):
        out, lse = run_contig(B, w, t, S)
        check(out.contiguous(), lse, *ref, what=f"contiguous {layout} {case} S={S}")


def test_contiguous_equals_paged_bitwise(B):
    """Direct output and the balanced mode give the same bits on contiguous K/V
    as on the same rows in pages (the same tokens meet in the same order)."""
    lens = [(i * 613) % 3000 + 1 for i in range(14)] + [0, 64]
    w = wl.custom_workload(len(lens), 32, 8, 128, 64, lens, "bf16", seed=720, window=900, sinks=True)
    tp = dev(w)
    t, _, _, _ = contig_dev(w, "bhld", strided_out=True)
    for S in (1, BAL):
        po, pl = run(B, w, S, tp)
        co, cl = run_contig(B, w, t, S)
        assert torch.equal(co.contiguous().view(torch.int16), po.view(torch.int16)), S
        assert torch.equal(cl, pl), S


# ---- HIP graph capture of the other entry points -------------------------------

def _capture(fn):
    """Capture fn() into a HIP graph on a side stream; returns the graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("S", [BAL, 1, 3])
def test_graph_replays_window_sinks_and_contiguous(B, S):
    """Captured window/sink decodes (paged) and contiguous decodes replay several
    times, with eager work between, bitwise equal to the eager calls."""
    lens = [(i * 613) % 3000 + 1 for i in range(30)] + [0, 64]
    w = wl.custom_workload(len(lens), 32, 8, 128, 64, lens, "bf16", seed=740, window=500, sinks=True)
    t = dev(w)
    eager_o, eager_l = run(B, w, S, t)
    out = torch.empty_like(t["q"])
    lse = torch.empty(t["q"].shape[:2], dtype=torch.float32, device="cuda")
    dims, e = B.dims_for(t["q"], t["k"], t["bt"]), B.ext_for(t["q"], window=500)
    nbytes = B.paged_decode_workspace_bytes_ext(dims, e, S)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    tc, _, _, _ = contig_dev(w, "bhld", strided_out=True)
    co_eager, cl_eager = run_contig(B, w, tc, S)
    cd = B.contig_dims_for(tc["q"], tc["k"], tc["out"], window=500)
    cbytes = B.contiguous_decode_workspace_bytes(cd, S)
    cws = torch.empty(max(cbytes, 1), dtype=torch.uint8, device="cuda")
    clse = torch.empty(t["q"].shape[:2], dtype=torch.float32, device="cuda")
    st = []

    def body():
        h = B.current_stream_handle(0)
        st.append(B.paged_decode_ext(dims, e, t["q"], t["k"], t["v"], t["bt"], t["lens"], None, None, t["sinks"],
                                     w.scale, out, lse, S, ws if nbytes else None, nbytes, h))
        st.append(B.contiguous_decode(cd, tc["q"], tc["k"], tc["v"], tc["lens"], None, None, tc["sinks"], w.scale,
                                      tc["out"], clse, S, cws if cbytes else None, cbytes, h))
    g = _capture(body)
    assert st == [0, 0]
    for i in range(4):
        out.fill_(0)
        lse.fill_(0)
        tc["out"].fill_(0)
        clse.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.cpu().view(torch.int16), eager_o.view(torch.int16)), f"replay {i}"
        assert torch.equal(lse.cpu(), eager_l), f"replay {i}"
        assert torch.equal(tc["out"].cpu().contiguous().view(torch.int16), co_eager.contiguous().view(torch.int16))
        assert torch.equal(clse.cpu(), cl_eager), f"replay {i}"


def test_graph_replays_append_and_metadata(B):
    """A captured append (FP8, RoPE) and metadata preparation replay several
    times onto reset buffers, bitwise equal to the oracle each time."""
    aw = wl.append_workload(300, 8, 128, 64, 16, "fp8_e4m3", rope=True, seed=750, pad_every=7)
    ref_k, ref_v = oracle.kv_append(aw.k_new, aw.v_new, aw.slot_mapping, aw.k_cache, aw.v_cache, aw.k_scale,
                                    aw.v_scale, aw.positions, aw.cos_sin)
    t = _dev_append(aw)
    k0, v0 = t["k_cache"].clone(), t["v_cache"].clone()
    rng = np.random.default_rng(751)
    lens = rng.integers(0, 16 * 64, size=40)
    bt = rng.integers(0, 5000, size=(40, 16)).astype(np.int32)
    rt, rows = token_map(bt, lens, 64, 50, 16 * 64, seed=752)
    ref_m, bad = oracle.decode_metadata(rt, rows, lens.astype(np.int64), 64, 16, window=100)
    cuda = torch.device("cuda:0")
    rt_d, rows_d = torch.from_numpy(rt).to(cuda), torch.from_numpy(rows).to(cuda)
    lens_d = torch.from_numpy(lens.astype(np.int64)).to(cuda)
    m_out = {}

    def body():
        B.append(**t)
        m_out.update(B.metadata(rt_d, rows_d, lens_d, 64, 16, window=100))
    g = _capture(body)
    for i in range(3):
        t["k_cache"].copy_(k0)
        t["v_cache"].copy_(v0)
        for v in m_out.values():
            v.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_k, got_v = wl.as_numpy_bits(t["k_cache"].cpu()), wl.as_numpy_bits(t["v_cache"].cpu())
        assert np.array_equal(got_k, ref_k.reshape(got_k.shape)), f"replay {i}: K"
        assert np.array_equal(got_v, ref_v.reshape(got_v.shape)), f"replay {i}: V"
        for k, v in ref_m.items():
            assert np.array_equal(m_out[k].cpu().numpy(), v), f"replay {i}: {k}"
        assert int(m_out["error_count"].cpu()[0]) == bad


def test_largest_q_len_with_causal_window_and_sinks(B):
    """q_len at its maximum (64 query tokens: 64 and 128 packed rows per KV head,
    i.e. 4 and 8 head groups) under the causal mask with a window and sinks,
    in every split mode, against the oracle."""
    for hq, hkv in ((4, 4), (8, 4)):
        lens = [64, 200, 3, 700]
        w = wl.custom_workload(len(lens), hq, hkv, 64, 16, lens, "bf16", seed=760 + hq, q_len=64, causal=True,
                               window=40, sinks=True)
        ref = oracle_full(w)
        t = dev(w)
        for S in (1, 3, BAL):
            out, lse = run(B, w, S, t)
            check(out, lse, *ref, what=f"q_len 64 Hq={hq} S={S}")


# ---- the vector-ALU inner loop (measurement entry) ------------------------------

VALU_CASES = [
    # (B, Hq, Hkv, D, ps, seq_lens, seed)
    (5, 32, 8, 128, 64, [700, 2, 0, 3000, 64], 901),
    (4, 16, 8, 64, 16, [1, 17, 300, 33], 902),
    (3, 8, 8, 128, 32, [5000, 31, 129], 903),
    (6, 8, 4, 64, 48, [95, 96, 97, 1, 480, 0], 904),
]


def run_valu(B, w, t):
    dims = B.dims_for(t["q"], t["k"], t["bt"])
    out = torch.full(t["q"].shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full(t["q"].shape[:-1], float("nan"), dtype=torch.float32, device="cuda")
    st = B.pkd_decode_valu(dims, t["q"], t["k"], t["v"], t["bt"], t["lens"], w.scale, out, lse,
                           B.current_stream_handle(0))
    assert st == 0, B.paged_decode_status_string(st)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


@pytest.mark.parametrize("case", VALU_CASES)
def test_valu_entry_matches_oracle(B, case):
    """The vector-ALU kernel against the oracle (NaN tails, -1 padding), G = 4, 2, 1
    and page sizes 16 to 64."""
    bq, hq, hkv, d, ps, lens, seed = case
    w = wl.custom_workload(bq, hq, hkv, d, ps, lens, "bf16", seed)
    out, lse = run_valu(B, w, dev(w))
    check(out, lse, *oracle_full(w), what=f"valu {case[:5]}")


@pytest.mark.parametrize("name", ["llama_b32_d128_ps64", "batch128_d128_ps128"])
def test_valu_entry_full_size(B, name):
    """Every row of the B=32 and B=128 steps, as timed beside the matrix-core kernels."""
    w = wl.make_workload(wl.WORKLOADS[name], tail="nan")
    out, lse = run_valu(B, w, dev(w))
    check(out, lse, *oracle_full(w), what=f"valu {name}")


# ---- tiles staged by direct-to-LDS loads (measurement entry) --------------------

LDS_CASES = [
    # (B, Hq, Hkv, D, ps, seq_lens, seed): G = 4, 1, 16, 6, 8; ragged tails, empty
    # and one-token sequences, more tiles than waves and fewer.
    (5, 32, 8, 128, 64, [700, 2, 0, 3000, 64], 911),
    (4, 16, 16, 128, 16, [1, 17, 300, 33], 912),
    (3, 16, 1, 128, 32, [5000, 31, 129], 913),
    (6, 24, 4, 128, 48, [95, 96, 97, 1, 480, 0], 914),
    (2, 8, 1, 128, 128, [8191, 4097], 915),
]


def run_lds(B, w, t):
    dims = B.dims_for(t["q"], t["k"], t["bt"])
    out = torch.full(t["q"].shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full(t["q"].shape[:-1], float("nan"), dtype=torch.float32, device="cuda")
    st = B.pkd_decode_lds(dims, t["q"], t["k"], t["v"], t["bt"], t["lens"], w.scale, out, lse,
                          B.current_stream_handle(0))
    assert st == 0, B.paged_decode_status_string(st)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


@pytest.mark.parametrize("case", LDS_CASES)
def test_lds_entry_matches_oracle_and_grid_kernel(B, case):
    """The LDS-staged kernel against the oracle (NaN tails, -1 padding), and bit for
    bit against paged_decode with num_splits = 1, whose arithmetic it shares."""
    bq, hq, hkv, d, ps, lens, seed = case
    w = wl.custom_workload(bq, hq, hkv, d, ps, lens, "bf16", seed)
    t = dev(w)
    out, lse = run_lds(B, w, t)
    check(out, lse, *oracle_full(w), what=f"lds {case[:5]}")
    out1, lse1 = run(B, w, 1, t)
    assert torch.equal(out.view(torch.int16), out1.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lse1.view(torch.int32))


def test_direct_output_path_choice(B):
    """paged_decode runs the LDS-staged direct kernel (bf16 or FP8) for up to two
    rounds of D = 128 items of one query token without a window (two in its
    pairs form), and the register-staged one otherwise; for bf16 both give the
    same bits, so the switch is invisible in the results."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    b32 = B.pkd_dims(32, 32, 8, 128, 64, 1500, 64, B.PKD_DTYPE_BF16)
    lds = B.PKD_PATH_DIRECT_LDS if 32 * 8 <= 2 * cus else B.PKD_PATH_DIRECT
    assert B.paged_decode_path(b32, None, 1) == lds
    assert B.paged_decode_path(b32, B.pkd_ext(1, 1, 0, 0), 1) == lds  # causal, one token: no mask
    assert B.paged_decode_path(b32, B.pkd_ext(4, 1, 0, 0), 1) == B.PKD_PATH_DIRECT  # 4 query tokens
    assert B.paged_decode_path(b32, B.pkd_ext(1, 0, 512, 0), 1) == B.PKD_PATH_DIRECT  # window
    b64 = B.pkd_dims(64, 32, 8, 128, 64, 1500, 64, B.PKD_DTYPE_BF16)
    assert B.paged_decode_path(b64, None, 1) == (B.PKD_PATH_DIRECT_LDS if 64 * 8 <= 2 * cus else B.PKD_PATH_DIRECT)
    b128 = B.pkd_dims(128, 32, 8, 128, 128, 4100, 32, B.PKD_DTYPE_BF16)
    assert B.paged_decode_path(b128, None, 1) == B.PKD_PATH_DIRECT  # four rounds
    fp8 = B.pkd_dims(32, 32, 8, 128, 64, 1500, 64, B.PKD_DTYPE_FP8_E4M3)
    assert B.paged_decode_path(fp8, None, 1) == lds
    fp8_d64 = B.pkd_dims(32, 32, 8, 64, 64, 1500, 64, B.PKD_DTYPE_FP8_E4M3)
    assert B.paged_decode_path(fp8_d64, None, 1) == B.PKD_PATH_DIRECT


@pytest.mark.parametrize("bq,hq,lens_seed,sinks", [(20, 64, 1, False), (33, 64, 2, True), (64, 64, 3, False),
                                                   (40, 8, 4, True)])
def test_fp8_lds_direct_matches_oracle(B, bq, hq, lens_seed, sinks):
    """FP8 direct output on the LDS-staged kernel (one workgroup per item, or the
    pairs form above one item per compute unit) against the oracle, and against
    the same call with a window longer than every sequence, which changes no
    score but runs the register-staged grid kernel.  Its eight waves group the
    tiles differently from the grid kernel's four, so the two agree to rounding
    (a few bf16 ulps), not bit for bit; a repeated call gives the same bits."""
    lens = [int(x) for x in np.random.default_rng(lens_seed).integers(0, 2500, size=bq)]
    w = wl.custom_workload(bq, hq, 8, 128, 64, lens, "fp8_e4m3", 4100 + lens_seed, sinks=sinks)
    t = dev(w)
    dims = B.dims_for(t["q"], t["k"], t["bt"])
    assert B.paged_decode_path(dims, None, 1) == B.PKD_PATH_DIRECT_LDS
    big = w.spec.max_pages_per_seq * w.spec.page_size + 64
    assert B.paged_decode_path(dims, B.ext_for(t["q"], False, big), 1) == B.PKD_PATH_DIRECT
    out_w, lse_w = B.decode(t["q"], t["k"], t["v"], t["bt"], t["lens"], w.scale, t["ks"], t["vs"], num_splits=1,
                            window=big, sinks=t["sinks"])
    out, lse = run(B, w, 1, t)
    torch.cuda.synchronize()
    ref = oracle_full(w)
    check(out, lse, *ref, what=f"fp8 lds direct B={bq}")
    check(out_w.cpu(), lse_w.cpu(), *ref, what=f"fp8 grid direct B={bq}")
    d = (out.float() - out_w.cpu().float()).abs()
    assert float(d.max()) <= 4 * 2.0 ** -8 * float(out.float().abs().max()) + 1e-6
    out2, lse2 = run(B, w, 1, t)
    assert torch.equal(out2.view(torch.int16), out.view(torch.int16)) and torch.equal(lse2, lse)


@pytest.mark.parametrize("q_len,causal,sinks", [(1, False, True), (1, True, True), (1, False, False),
                                                 (4, True, True)])
def test_lds_direct_equals_grid_kernel_with_sinks(B, q_len, causal, sinks):
    """Direct output at the B = 32 shape (LDS-staged where one round fits, for one
    query token) against the same call with a window longer than every sequence,
    which changes no score but runs the register-staged grid kernel: the bits
    must agree, with and without sinks (and for four causal query tokens, which
    both calls send to the grid kernel)."""
    lens = [1024 + 97 * i for i in range(31)] + [3]  # a sequence shorter than q_len too
    w = wl.custom_workload(32, 32, 8, 128, 64, lens, "bf16", 1234 + q_len, q_len=q_len, causal=causal,
                           sinks=sinks)
    t = dev(w)
    dims = B.dims_for(t["q"], t["k"], t["bt"])
    big = w.spec.max_pages_per_seq * w.spec.page_size + 64
    assert B.paged_decode_path(dims, B.ext_for(t["q"], causal, big), 1) == B.PKD_PATH_DIRECT
    out_w, lse_w = B.decode(t["q"], t["k"], t["v"], t["bt"], t["lens"], w.scale, num_splits=1, causal=causal,
                            window=big, sinks=t["sinks"])
    out, lse = run(B, w, 1, t)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out_w.cpu().view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lse_w.cpu().view(torch.int32))
    check(out, lse, *oracle_full(w), what=f"lds direct q_len={q_len} causal={causal} sinks={sinks}")


@pytest.mark.parametrize("case", LDS_CASES)
def test_registers_entry_equals_paged_decode(B, case):
    """pkd_decode_registers (the grid kernel whatever the shape) against the oracle
    and bit for bit against paged_decode with num_splits = 1."""
    bq, hq, hkv, d, ps, lens, seed = case
    w = wl.custom_workload(bq, hq, hkv, d, ps, lens, "bf16", seed)
    t = dev(w)
    dims = B.dims_for(t["q"], t["k"], t["bt"])
    out = torch.full(t["q"].shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full(t["q"].shape[:-1], float("nan"), dtype=torch.float32, device="cuda")
    st = B.pkd_decode_registers(dims, t["q"], t["k"], t["v"], t["bt"], t["lens"], w.scale, out, lse,
                                B.current_stream_handle(0))
    assert st == 0, B.paged_decode_status_string(st)
    torch.cuda.synchronize()
    out, lse = out.cpu(), lse.cpu()
    check(out, lse, *oracle_full(w), what=f"registers {case[:5]}")
    out1, lse1 = run(B, w, 1, t)
    assert torch.equal(out.view(torch.int16), out1.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lse1.view(torch.int32))


def test_lds_and_register_direct_kernels_agree_on_random_shapes(B):
    """24 seeded random shapes (batch, G, page size, ragged and empty lengths, NaN
    tails): the LDS-staged kernel (pkd_decode_lds) and the register-staged grid
    kernel (pkd_decode_registers) give the same bits."""
    rng = np.random.default_rng(20261203)
    for case in range(24):
        hkv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.choice([1, 2, 3, 4, 8, 16]))
        bq = int(rng.integers(1, 33))
        ps = int(rng.choice([16, 32, 48, 64, 128]))
        lens = [int(x) for x in rng.integers(0, 2500, size=bq)]
        lens[int(rng.integers(0, bq))] = int(rng.choice([0, 1, 15, 16, 17]))
        w = wl.custom_workload(bq, hkv * G, hkv, 128, ps, lens, "bf16", 7000 + case)
        t = dev(w)
        dims = B.dims_for(t["q"], t["k"], t["bt"])
        outs = []
        for fn in (B.pkd_decode_lds, B.pkd_decode_registers):
            out = torch.full(t["q"].shape, float("nan"), dtype=torch.bfloat16, device="cuda")
            lse = torch.full(t["q"].shape[:-1], float("nan"), dtype=torch.float32, device="cuda")
            st = fn(dims, t["q"], t["k"], t["v"], t["bt"], t["lens"], w.scale, out, lse, B.current_stream_handle(0))
            assert st == 0, B.paged_decode_status_string(st)
            outs.append((out, lse))
        torch.cuda.synchronize()
        (o1, l1), (o2, l2) = outs
        what = f"case {case}: B={bq} Hkv={hkv} G={G} ps={ps}"
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), what
        assert torch.equal(l1.view(torch.int32), l2.view(torch.int32)), what


@pytest.mark.parametrize("name", ["llama_b32_d128_ps64", "batch128_d128_ps128"])
def test_lds_entry_full_size(B, name):
    """Every row of the B=32 and B=128 steps, as timed beside the register-staged kernel."""
    w = wl.make_workload(wl.WORKLOADS[name], tail="nan")
    t = dev(w)
    out, lse = run_lds(B, w, t)
    check(out, lse, *oracle_full(w), what=f"lds {name}")
    out1, lse1 = run(B, w, 1, t)
    assert torch.equal(out.view(torch.int16), out1.view(torch.int16))


# ---- FP8 on the LDS-staged pipeline (balanced kernel, D = 128) -------------------

FP8_LDS_CASES = [
    # (B, Hq, Hkv, ps, seq_lens, q_len, causal, sinks, seed): G = 8, 1, 16, 4; page
    # sizes 16..128 (32-token tiles straddling pages), ragged, empty and short
    # sequences, causal query tokens, pieces starting on odd 16-token groups.
    (64, 64, 8, 64, None, 1, False, False, 1601),
    (5, 32, 4, 16, [700, 2, 0, 3001, 64], 1, False, True, 1602),
    (4, 16, 16, 32, [1, 17, 300, 33], 1, False, False, 1603),
    (3, 16, 1, 48, [5000, 31, 129], 3, True, False, 1604),
    (6, 32, 8, 128, [95, 96, 97, 1, 480, 15], 2, True, True, 1605),
    (2, 16, 4, 16, [8191, 4097], 1, False, False, 1606),
]


@pytest.mark.parametrize("case", FP8_LDS_CASES)
def test_fp8_lds_pipeline_equals_register_path(B, case):
    """FP8 K/V, D = 128, balanced mode: the tiles go through the LDS-staged pipeline.
    The same call with a window longer than every sequence changes no score but
    runs the register-staged tile loop; the bits must agree, and both must match
    the oracle."""
    bq, hq, hkv, ps, lens, q_len, causal, sinks, seed = case
    if lens is None:
        lens = [int(x) for x in np.random.default_rng(seed).integers(512, 8193, size=bq)]
    w = wl.custom_workload(bq, hq, hkv, 128, ps, lens, "fp8_e4m3", seed, q_len=q_len, causal=causal,
                           sinks=sinks)
    t = dev(w)
    big = w.spec.max_pages_per_seq * w.spec.page_size + 64
    out, lse = run(B, w, B.PKD_SPLITS_BALANCED, t)
    out_w, lse_w = B.decode(t["q"], t["k"], t["v"], t["bt"], t["lens"], w.scale, t["ks"], t["vs"],
                            num_splits=B.PKD_SPLITS_BALANCED, causal=causal, window=big, sinks=t["sinks"])
    torch.cuda.synchronize()
    what = f"fp8 lds {case[:4]} q_len={q_len}"
    assert torch.equal(out.view(torch.int16), out_w.cpu().view(torch.int16)), what
    assert torch.equal(lse.view(torch.int32), lse_w.cpu().view(torch.int32)), what
    check(out, lse, *oracle_full(w), what=what)


# ---- the read-only stream kernel (measurement entry) ----------------------------

@pytest.mark.parametrize("pattern", [0, 1])
def test_stream_read_folds_every_word_once(B, pattern):
    """Patterns 0 and 1 cover the buffer exactly once: the XOR of every thread's
    sink word equals the XOR of the whole buffer (each wave's block count is a
    multiple of the batch, so no block is folded twice)."""
    g = torch.Generator().manual_seed(77 + pattern)
    words = torch.randint(-2**31, 2**31 - 1, ((1 << 20) // 4,), dtype=torch.int64, generator=g).to(torch.int32)
    buf = words.cuda()
    wgs, waves, kb = 8, 4, 8  # 1024 blocks: 32 per wave
    sink = torch.zeros(B.pkd_stream_read_sink_bytes(wgs, waves) // 4, dtype=torch.int32, device="cuda")
    st = B.pkd_stream_read(buf, 1 << 20, 2048, 256, pattern, wgs, waves, kb, 1, sink, B.current_stream_handle(0))
    assert st == 0, B.paged_decode_status_string(st)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(words.numpy().view(np.uint32))
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == want


@pytest.mark.parametrize("waves,kb", [(4, 4), (4, 8), (8, 8), (4, 16)])
def test_stream_read_direct_to_lds_lands_in_lds(B, waves, kb):
    """Pattern 2's loads write LDS: over a buffer of one repeated word, every
    thread of a wave with blocks reads that word back from its ring."""
    c = 0x01020304
    buf = torch.full(((1 << 20) // 4,), c, dtype=torch.int32, device="cuda")
    wgs = 8  # 1024 blocks: at least 16 per wave
    sink = torch.zeros(B.pkd_stream_read_sink_bytes(wgs, waves) // 4, dtype=torch.int32, device="cuda")
    st = B.pkd_stream_read(buf, 1 << 20, 2048, 256, 2, wgs, waves, kb, 1, sink, B.current_stream_handle(0))
    assert st == 0, B.paged_decode_status_string(st)
    torch.cuda.synchronize()
    assert bool((sink.cpu() == c).all())
