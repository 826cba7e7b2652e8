"""An fp64 reference for the rotated K rows of the paged KV append, shared by the
oracle pin and the GPU test.

The append rotates each new K row in the rotate-half form: for d < D/2, with
c = cos_sin[pos][d] and s = cos_sin[pos][D/2 + d],
k'[d] = k[d] c - k[d + D/2] s and k'[d + D/2] = k[d + D/2] c + k[d] s.
Here k' is computed in fp64, where the bf16 and fp32 inputs and their products
are exact and each sum is rounded once, far below any bf16 or FP8 step.

The implementations compute k' in fp32 (a product, then one fused multiply-add)
and round it to the cache's code.  Their k' differs from the exact one by at most
the product's rounding and the fused add's rounding, each at most 2^-24 of the
terms' magnitude m = |k[d] c| + |k[d + D/2] s|, so the stored value may differ
from the exact one by at most half a code step plus 2^-23 m (plus, for FP8, the
fp32 division by the scale, 2^-24 of the quotient).  Where that fp32 error is far
below a code step (no cancellation between the two terms) the stored code is the
exact value's code or a neighbour of it.
"""
import numpy as np
import torch


def rotated_fp64(w):
    """(k' [N, Hkv, D] fp64, m [N, Hkv, D]: the terms' magnitude) of append workload w;
    rows of tokens whose position lies outside the table are returned unrotated."""
    k = w.k_new.to(torch.float64).numpy()
    n, hkv, d = k.shape
    half = d // 2
    cs = w.cos_sin.to(torch.float64).numpy()
    out = k.copy()
    mag = np.abs(k)
    for i in range(n):
        p = int(w.positions[i])
        if p < 0 or p >= cs.shape[0]:
            continue
        c, s = cs[p, :half], cs[p, half:]
        a, b = k[i, :, :half], k[i, :, half:]
        out[i, :, :half] = a * c - b * s
        out[i, :, half:] = b * c + a * s
        mag[i, :, :half] = np.abs(a * c) + np.abs(b * s)
        mag[i, :, half:] = np.abs(b * c) + np.abs(a * s)
    return out, mag


def _bf16_key(bits):
    """Monotone integer order of bf16 bit patterns (negative values below positive)."""
    b = bits.astype(np.int64) & 0xFFFF
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def _fp8_key(codes):
    c = codes.astype(np.int64) & 0xFF
    return np.where(c & 0x80, -(c & 0x7F), c)


def _bf16_step(x):
    """Spacing of bf16 values at |x| (normal range)."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 2.0 ** (e - 7)


def _fp8_step(x):
    """Spacing of E4M3FN values at |x| (subnormal spacing 2^-9 below 2^-6)."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -6)))
    return 2.0 ** (e - 3)


def check(w, k_cache_bits, kv_dtype):
    """Compares the rows an append wrote (k_cache_bits: the updated K cache as raw bits
    [P, ps, Hkv, D]) with the fp64 rotation.  Returns (worst error / derived bound, share
    of codes equal to the exact value's code, worst code distance where the fp32 error
    bound is under a quarter of a code step)."""
    exact, mag = rotated_fp64(w)
    num_pages, ps = k_cache_bits.shape[:2]
    cap = num_pages * ps
    rows, idx = [], []
    for i, slot in enumerate(w.slot_mapping.tolist()):
        p = int(w.positions[i])
        if slot < 0 or slot >= cap or p < 0 or p >= w.cos_sin.shape[0]:
            continue
        rows.append(k_cache_bits[slot // ps, slot % ps])
        idx.append(i)
    stored = np.stack(rows).astype(np.int64)
    e, m = exact[idx], mag[idx]
    fp32_err = 2.0 ** -23 * m
    if kv_dtype == "bf16":
        val = torch.from_numpy((stored & 0xFFFF).astype(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
        want = torch.from_numpy(e).to(torch.bfloat16).view(torch.int16).numpy().astype(np.int64) & 0xFFFF
        step = np.maximum(_bf16_step(e), _bf16_step(val))
        err = np.abs(val - e)
        key = _bf16_key
    else:
        sc = w.k_scale.to(torch.float64).numpy()[None, :, None]
        x = np.clip(e / sc, -448.0, 448.0)
        val = torch.from_numpy((stored & 0xFF).astype(np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy().astype(np.int64)
        step = np.maximum(_fp8_step(x), _fp8_step(val))
        err = np.abs(val - x)
        fp32_err = fp32_err / sc + 2.0 ** -24 * np.abs(x)
        key = _fp8_key
    bound = 0.5 * step + fp32_err + 1e-30
    well = fp32_err < 0.25 * step
    dist = np.abs(key(stored) - key(want))
    return float(np.max(err / bound)), float(np.mean(stored == want)), int(np.max(dist[well]))
