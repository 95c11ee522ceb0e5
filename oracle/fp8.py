"""Oracle for per-page-scaled fp8 KV pages -- test infrastructure only.

cann-recipes-infer page, section 5.2: KV values are scaled before they are stored in the pages
and the scale factor is kept in each page's metadata, to be multiplied back on reading. Here the
pages hold fp8 codes and every (block, kv head) page has one scale per tensor.

Readings taken where the page leaves the step open:
  * format: OCP E4M3FN (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; subnormals
    m/8 * 2^-6; the largest finite value is 448; code 0x7F / 0xFF is NaN, there is no infinity);
  * a page's scale is a power of two, 2^k with the smallest integer k >= -120 such that every
    valid value of the page satisfies |x| <= 448 * 2^k (k = 0 for an all-zero page); dividing by
    it is exact (2^-120 is a normal fp32 number), so rounding the scaled value to the nearest
    code (ties to the even code) is the only rounding;
  * a cache write that touches a page rescales the whole page: its valid rows -- the ones cached
    before (decoded with the old scale) and the ones this step writes (bf16 inputs) -- set the new
    scale, and all of them are encoded again with it; rows past the context are not touched;
  * attention reads code * scale, exactly.
"""
from __future__ import annotations

import numpy as np

FP8_MAX = 448.0


def _e4m3_value(c):
    """The format's definition of the value of codes c (int array) as float64; NaN codes give
    NaN."""
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = (1.0 + m / 8.0) * np.exp2(e - 7.0)
    sub = (m / 8.0) * 2.0 ** -6
    v = sign * np.where(e == 0, sub, normal)
    return np.where((e == 15) & (m == 7), np.nan, v)


# the definition evaluated once for each of the 256 codes
_VALUES = _e4m3_value(np.arange(256, dtype=np.int64))


def decode_e4m3(codes):
    """Values of E4M3FN codes (uint8 array) as float64; NaN codes give NaN. Each code's value
    is the definition's (_e4m3_value), looked up, so large page pools decode in one pass."""
    return _VALUES[np.asarray(codes, dtype=np.uint8)]


# the 127 finite non-negative values, ascending (codes 0x00 .. 0x7E)
_POS = decode_e4m3(np.arange(0x7F))


def encode_e4m3(x):
    """Nearest E4M3FN code of each value (ties to the code with an even last bit); magnitudes
    above 448 are out of range here (the scale rule keeps every stored value within it)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    if np.any(a > FP8_MAX) or np.any(np.isnan(x)):
        raise ValueError("value outside the finite fp8 range")
    hi = np.clip(np.searchsorted(_POS, a, side="left"), 0, len(_POS) - 1)   # first >= a
    lo = np.clip(hi - 1, 0, len(_POS) - 1)
    dlo, dhi = a - _POS[lo], _POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0) & (hi != lo))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == _POS[hi], hi, code)
    neg = np.signbit(x)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


K_MIN = -120


def page_scale(amax):
    """2^k with the smallest integer k >= -120 such that amax <= 448 * 2^k (1.0 when amax is 0)."""
    amax = float(amax)
    if amax == 0.0:
        return 1.0
    k = int(np.floor(np.log2(amax / FP8_MAX)))
    while FP8_MAX * 2.0 ** k < amax:
        k += 1
    while k > K_MIN and FP8_MAX * 2.0 ** (k - 1) >= amax:
        k -= 1
    return 2.0 ** max(k, K_MIN)


def reshape_and_cache_fp8(k_new, v_new, k_codes, v_codes, k_scales, v_scales, block_table, q_lens,
                          context_lens):
    """Write this step's rows into fp8 pages, rescaling every page the step touches.

    k_new, v_new [T, Hkv, D] (the bf16 inputs as float values); k_codes, v_codes uint8
    [NB, Hkv, bs, D]; k_scales, v_scales [NB, Hkv] float. Returns new copies of the four page
    arrays. Sequence s owns rows cu[s] .. cu[s+1]-1 at positions P .. ctx-1 (P = ctx - q_len).
    """
    kc, vc = k_codes.copy(), v_codes.copy()
    ks, vs = np.asarray(k_scales, dtype=np.float64).copy(), np.asarray(v_scales, dtype=np.float64).copy()
    bs = kc.shape[2]
    hkv = kc.shape[1]
    cu = np.concatenate([[0], np.cumsum(np.asarray(q_lens, dtype=np.int64))])
    for s in range(len(q_lens)):
        ctx = int(context_lens[s])
        P = ctx - int(q_lens[s])
        for lb in range(P // bs, (ctx - 1) // bs + 1):
            b = int(block_table[s][lb])
            lo = lb * bs
            n_valid = min(ctx, lo + bs) - lo
            for codes, scales, new in ((kc, ks, k_new), (vc, vs, v_new)):
                for g in range(hkv):
                    vals = decode_e4m3(codes[b, g, :n_valid]) * scales[b, g]
                    for j in range(n_valid):
                        pos = lo + j
                        if pos >= P:
                            vals[j] = np.asarray(new[cu[s] + pos - P, g], dtype=np.float64)
                    sc = page_scale(np.max(np.abs(vals)) if vals.size else 0.0)
                    codes[b, g, :n_valid] = encode_e4m3(vals / sc)
                    scales[b, g] = sc
    return kc, vc, ks, vs


def dequantize_pages(codes, scales):
    """code * scale per (block, kv head) page, float64 [NB, Hkv, bs, D]."""
    return decode_e4m3(codes) * np.asarray(scales, dtype=np.float64)[:, :, None, None]
