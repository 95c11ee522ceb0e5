"""Pins for the fp8 page oracle (OCP E4M3FN codes with power-of-two page scales). CPU only."""
import numpy as np
import pytest

from oracle import fp8


def test_decode_matches_the_format_definition():
    d = fp8.decode_e4m3(np.arange(256))
    assert d[0x38] == 1.0                    # exponent field 7 = bias, mantissa 0
    assert d[0x7E] == 448.0                  # largest finite: 1.75 * 2^8
    assert d[0x08] == 2.0 ** -6              # smallest normal
    assert d[0x07] == 7 / 8 * 2.0 ** -6      # largest subnormal
    assert d[0x01] == 2.0 ** -9              # smallest subnormal
    assert d[0x40] == 2.0 and d[0x3F] == 1.875
    assert np.isnan(d[0x7F]) and np.isnan(d[0xFF])
    assert d[0x80] == 0.0 and np.signbit(d[0x80])
    assert np.array_equal(d[0x80:0xFF], -d[0x00:0x7F])
    assert np.all(np.diff(d[:0x7F]) > 0)     # codes 0..126 ascending


def test_encode_inverts_decode_on_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(fp8.encode_e4m3(fp8.decode_e4m3(codes)), codes)


def test_ties_go_to_the_even_code():
    v = fp8.decode_e4m3(np.arange(0x7F))
    mids = (v[:-1] + v[1:]) / 2              # exact in float64
    got = fp8.encode_e4m3(mids).astype(int)
    lo = np.arange(0x7E)
    expect = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(got, expect)
    assert fp8.encode_e4m3(np.array([1.0625]))[0] == 0x38    # between 1 and 1.125 -> 1
    assert fp8.encode_e4m3(np.array([2.0 ** -10]))[0] == 0x00  # half the smallest subnormal


def test_encode_is_the_nearest_code_by_brute_force():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(3000) * 2.0 ** rng.integers(-12, 9, 3000)
    x = x[np.abs(x) <= 448]
    got = fp8.decode_e4m3(fp8.encode_e4m3(x))
    allv = fp8.decode_e4m3(np.arange(0x7F))
    allv = np.concatenate([allv, -allv])
    best = np.min(np.abs(x[:, None] - allv[None, :]), axis=1)
    assert np.array_equal(np.abs(got - x), best)


@pytest.mark.parametrize("amax", [1e-30, 2.0 ** -20, 0.3, 1.0, 3.5, 224.0, 448.0, 449.0, 1e6])
def test_page_scale_is_the_smallest_fitting_power_of_two(amax):
    s = fp8.page_scale(amax)
    assert np.log2(s) == np.round(np.log2(s))
    assert amax <= 448.0 * s and amax > 224.0 * s
    assert fp8.page_scale(0.0) == 1.0


def test_page_scale_floor():
    # below 448 * 2^-121 the exponent stops at -120 (a normal fp32 power of two)
    assert fp8.page_scale(1e-38) == 2.0 ** -120
    assert fp8.page_scale(448.0 * 2.0 ** -120) == 2.0 ** -120
    assert fp8.page_scale(448.0 * 2.0 ** -120 * 1.0001) == 2.0 ** -119


def _pages(nb, hkv, bs, d):
    codes = np.full((nb, hkv, bs, d), 0x7F, dtype=np.uint8)     # NaN sentinels everywhere
    return codes, codes.copy(), np.ones((nb, hkv)), np.ones((nb, hkv))


def test_first_write_encodes_rows_with_the_page_scale():
    rng = np.random.default_rng(1)
    hkv, bs, d = 2, 16, 8
    kc, vc, ks, vs = _pages(3, hkv, bs, d)
    k_new = rng.standard_normal((5, hkv, d)).astype(np.float32)
    v_new = rng.standard_normal((5, hkv, d)).astype(np.float32)
    table = np.array([[2, -1]])
    kc2, vc2, ks2, vs2 = fp8.reshape_and_cache_fp8(k_new, v_new, kc, vc, ks, vs, table, [5], [5])
    for g in range(hkv):
        s = fp8.page_scale(np.abs(k_new[:, g]).max())
        assert ks2[2, g] == s
        assert np.array_equal(kc2[2, g, :5], fp8.encode_e4m3(k_new[:, g] / s))
    assert np.all(kc2[2, :, 5:] == 0x7F) and np.all(kc2[:2] == 0x7F)   # nothing else written
    # dequantized rows are within half a code step (relative 2^-4) for normal magnitudes
    deq = fp8.dequantize_pages(kc2, ks2)[2, :, :5].transpose(1, 0, 2)
    big = np.abs(k_new) > 2.0 ** -6 * ks2[2].max()
    assert np.all(np.abs(deq - k_new)[big] <= np.abs(k_new)[big] * 2.0 ** -4)


def test_append_keeps_codes_when_the_page_max_does_not_grow_and_rescales_when_it_does():
    hkv, bs, d = 1, 16, 4
    kc, vc, ks, vs = _pages(1, hkv, bs, d)
    table = np.array([[0]])
    first = np.array([[[1.0, -3.0, 0.5, 2.0]]], dtype=np.float32)
    kc, vc, ks, vs = fp8.reshape_and_cache_fp8(first, first, kc, vc, ks, vs, table, [1], [1])
    codes0 = kc[0, 0, 0].copy()
    small = np.array([[[0.25, 1.0, -1.5, 0.0]]], dtype=np.float32)           # |x| <= 3
    kc, vc, ks, vs = fp8.reshape_and_cache_fp8(small, small, kc, vc, ks, vs, table, [1], [2])
    assert np.array_equal(kc[0, 0, 0], codes0) and ks[0, 0] == fp8.page_scale(3.0)
    big = np.array([[[100.0, 0.0, 0.0, 0.0]]], dtype=np.float32)
    kc, vc, ks, vs = fp8.reshape_and_cache_fp8(big, big, kc, vc, ks, vs, table, [1], [3])
    s = fp8.page_scale(100.0)
    assert ks[0, 0] == s
    old = fp8.decode_e4m3(codes0) * fp8.page_scale(3.0)          # re-encoded with the new scale
    assert np.array_equal(kc[0, 0, 0], fp8.encode_e4m3(old / s))
    assert np.array_equal(kc[0, 0, 2], fp8.encode_e4m3(big[0, 0] / s))
    assert np.all(kc[0, 0, 3:] == 0x7F)
