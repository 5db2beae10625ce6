"""Pins for the CPU oracle against facts the pages and mathematics fix.

[review]     "[arXiv 2606.20474] UltraQuant: 컨텍스트가 긴 에이전트를 위한 4비트 KV 캐싱"
[commentary] pheeree.github.io "kv-cache-4bit-serving-residency-collapse"
[tq-guide]   "TurboQuant 완전 정리 - 이론 최적에 근접한 KV 캐시·벡터 검색 양자화와 vLLM 실측"

Each pin uses an independent route (exact rational arithmetic, a library
routine, a closed form, an invariant or a printed value), never a re-typing of
the oracle's own formula.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg
import torch

import oracle as O
from bit_kv_cache_wht_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- rotation
@pytest.mark.parametrize("d", [1, 2, 4, 8, 16, 32, 64, 128, 256])
def test_hadamard_orthogonal(d):
    h = O.sylvester_hadamard(d)
    assert np.array_equal(h @ h.T, d * np.eye(d, dtype=np.int64))      # H H^T = d I
    assert np.array_equal(h, h.T)


@pytest.mark.parametrize("d", [2, 8, 64, 128])
def test_hadamard_is_library_sylvester(d):
    assert np.array_equal(O.sylvester_hadamard(d), scipy.linalg.hadamard(d))


def test_wht_scale_is_correctly_rounded_sqrt():
    assert O.wht_scale(64) == 0.125
    c = O.wht_scale(128)
    half_ulp = Fraction(math.ulp(c)) / 2
    lo, hi = Fraction(c) - half_ulp, Fraction(c) + half_ulp
    assert lo * lo < Fraction(1, 128) < hi * hi            # c is the nearest double to sqrt(1/128)


def test_wht_orthogonality_invariants():
    rng = np.random.default_rng(0)
    x, y = rng.standard_normal((2, 50, 128))
    wx, wy = O.wht(x), O.wht(y)
    np.testing.assert_allclose(O.wht(wx), x, rtol=0, atol=1e-13)                # self-inverse
    np.testing.assert_allclose(np.linalg.norm(wx, axis=1), np.linalg.norm(x, axis=1), rtol=1e-14)
    # [tq-guide] "직교성을 이용한 내적 보존": <Mx, My> = <x, y>
    np.testing.assert_allclose((wx * wy).sum(1), (x * y).sum(1), rtol=1e-12, atol=1e-12)
    e0 = np.zeros(128); e0[0] = 1.0
    np.testing.assert_allclose(O.wht(e0), np.full(128, O.wht_scale(128)), rtol=0, atol=0)
    np.testing.assert_allclose(O.wht(np.ones(128)), np.sqrt(128.0) * e0, rtol=1e-15, atol=1e-15)


def _exact_hadamard_row(vals):
    """H v in exact rational arithmetic (fast transform over Fractions)."""
    v = [Fraction(float(t)) for t in vals]
    h = 1
    while h < len(v):
        for i in range(0, len(v), 2 * h):
            for j in range(i, i + h):
                a, b = v[j], v[j + h]
                v[j], v[j + h] = a + b, a - b
        h *= 2
    return v


def test_wht_float64_sums_are_exact_on_bf16_rows():
    # The oracle and the GPU sum in different orders; both are exact when the
    # row's exponent span allows it.  Check against exact rationals.
    wl = W.make_workload("pin", 1, 8, 8, 128, [24], [24], seed=42)
    x = O.bf16_bits_to_f64(wl.k.reshape(-1, 128))
    c = O.wht_scale(128)
    got = O.wht(x)
    for r in range(x.shape[0]):
        exact = _exact_hadamard_row(x[r])
        assert all(float(e) == e for e in exact)            # every sum representable
        assert np.array_equal(got[r], np.array([float(e) * c for e in exact]))


def test_exact_sum_rows_boundary():
    # The criterion at its edge, built from explicit values: multiples of 2^u
    # whose magnitudes sum to 2^(u+53) - 2^u keep every partial sum exact; one
    # more 2^u (a sum of 2^(u+53), where the spacing of doubles becomes 2^(u+1))
    # does not.
    for u in (-149, -30, 0, 40):
        unit = 2.0 ** u
        row = np.zeros(128)
        row[0] = 2.0 ** (u + 52)
        row[1] = 2.0 ** (u + 52) - 2 * unit
        row[2] = unit
        assert O.exact_sum_rows(row[None])[0]            # sum 2^(u+53) - 2^u
        row[3] = unit
        assert not O.exact_sum_rows(row[None])[0]        # sum 2^(u+53)
    assert O.exact_sum_rows(np.zeros((1, 64)))[0]
    # bf16 rows: exponent spans of 38 binades are inside, 39 and more may not be
    r = np.zeros((2, 128))
    r[:, :127] = 1.9921875                                # 0x3FFF: bf16 with all 8 significand bits
    r[0, 127] = 1.9921875 * 2.0 ** -38
    r[1, 127] = 1.9921875 * 2.0 ** -39
    assert list(O.exact_sum_rows(r)) == [True, False]


def test_wht_outside_the_exact_sum_domain_is_the_exact_sum_rounded_once():
    # Rows with a span far beyond the domain: the oracle's value must be the
    # exact Hadamard sum (here by the fast transform over Fractions) times c_d,
    # rounded once, whatever the float64 matrix product gives.
    rng = np.random.default_rng(77)
    for d in (64, 128):
        x = rng.standard_normal((6, d)).astype(np.float32).astype(np.float64)
        x[:, 0] *= 2.0 ** 60
        x[1, 1:] *= 2.0 ** -70
        x[2, 1::3] = 0.0
        x[3] *= 2.0 ** -100                                # float32 subnormals beside normals
        assert not O.exact_sum_rows(x).any()
        c = Fraction(O.wht_scale(d))
        got = O.wht(x)
        for r in range(x.shape[0]):
            want = np.array([float(c * e) for e in _exact_hadamard_row(x[r])]) + 0.0
            assert np.array_equal(got[r], want)
        assert not np.array_equal(got, O.wht(x, exact=False))   # the float64 product rounds here


def test_wht_exact_zero_outputs_are_positive_zero():
    # Reading R2: an output whose exact sum is zero carries no sign.  Rows of
    # signed zeros, and rows whose Hadamard sums cancel exactly, give +0 there.
    d = 64
    z = np.zeros((3, d))
    z[0] = -0.0
    z[1, ::2] = -0.0
    z[2, 0], z[2, 1] = 1.5, -1.5                 # H row k sums to 0 where H[0,k] == H[1,k]
    got = O.wht(z)
    h = O.sylvester_hadamard(d)
    zero = np.zeros_like(got, dtype=bool)
    zero[:2] = True
    zero[2] = h[0] == h[1]
    assert np.all(got[zero] == 0.0) and not np.any(np.signbit(got[zero]))
    assert np.all(np.abs(got[2][~zero[2]]) == 3.0 * O.wht_scale(d))
    codes, _ = O.quantize_fp4(got)
    assert not np.any(codes[zero])                  # code 0, not the negative-zero code 8


# ---------------------------------------------------------------- UE8M0 exponent
def _least_exponent(m: float) -> int:
    """Brute force: smallest integer E with m <= 6 * 2**E, exact rationals."""
    fm = Fraction(m)
    e = math.floor(math.log2(m)) - 4 if m > 0 else -2000
    while Fraction(6) * Fraction(2) ** e < fm:
        e += 1
    while Fraction(6) * Fraction(2) ** (e - 1) >= fm:
        e -= 1
    return e


def test_scale_exponent_against_brute_force():
    vals = [0.0, 5e-324, 1e-310, 2.0 ** -1022, 1e-40, 6 * 2.0 ** -127, 6 * 2.0 ** -128, 1e-3, 0.5,
            1.0, 1.5, 3.0, 5.999999999, 6.0, 6.000000001, 7.5, 12.0, 1e30, 6 * 2.0 ** 127,
            6 * 2.0 ** 127 * (1 + 2 ** -52), 1e300]
    for k in range(-140, 140, 7):
        b = 6.0 * 2.0 ** k
        vals += [b, np.nextafter(b, 0), np.nextafter(b, np.inf)]
        f = 1.5 * 2.0 ** k                      # boundary of the closed form at fraction 1.5
        vals += [f, np.nextafter(f, 0), np.nextafter(f, np.inf)]
    rng = np.random.default_rng(1)
    vals += list(np.exp(rng.uniform(-100, 100, 500)))
    vals = np.array(vals)
    got = O.scale_exponent(vals)
    for m, e in zip(vals, got):
        want = -127 if m == 0 else min(127, max(-127, _least_exponent(float(m))))
        assert e == want, (m, e, want)


def test_scale_exponent_never_clips_in_range():
    rng = np.random.default_rng(2)
    m = np.exp(rng.uniform(-60, 60, 10000))
    e = O.scale_exponent(m)
    assert np.all(m <= np.ldexp(6.0, e)) and np.all(m > np.ldexp(6.0, e - 1))


# ---------------------------------------------------------------- constOpt scale (R9)
def test_sqrt2_up_brackets_sqrt2():
    # SQRT2_UP is the least double above sqrt(2): its square exceeds 2 and the
    # previous double's square is below 2 (exact rational arithmetic)
    up = Fraction(O.SQRT2_UP)
    below = Fraction(float(np.nextafter(O.SQRT2_UP, 0.0)))
    assert up * up > 2 > below * below


def _nearest_log2(s: float) -> int:
    """The integer nearest to log2(s) for a double s > 0, by exact comparison of
    s^2 with 2^(2k+1) (sqrt(2) is irrational, so there are no ties)."""
    q = Fraction(s)
    k = math.floor(math.log2(s))
    while Fraction(2) ** k > q:
        k -= 1
    while Fraction(2) ** (k + 1) <= q:
        k += 1
    return k + 1 if q * q > Fraction(2) ** (2 * k + 1) else k


def test_constopt_exponent_against_exact_log2_rounding():
    rng = np.random.default_rng(11)
    for c in (O.CONSTOPT_C, 0.195, 1.0):
        m = list(np.exp(rng.uniform(-80, 80, 400)))
        for k in range(-130, 130, 9):        # products just either side of sqrt(2) * 2^k
            t = O.SQRT2_UP * 2.0 ** k / c
            m += [t, np.nextafter(t, 0), np.nextafter(t, np.inf), 2.0 ** k / c]
        m = np.array(m)
        got = O.scale_exponent_constopt(m, c)
        for mi, e in zip(m, got):
            s = float(np.float64(c) * mi)
            want = -127 if s == 0 else min(127, max(-127, _nearest_log2(s)))
            assert e == want, (c, mi, s, e, want)


def test_constopt_worked_values_log_domain():
    # c = 1: s = m.  0.72 is nearer 1 than 0.5 in log2 (-0.47) though nearer 0.5
    # on the line; 0.70 is nearer 0.5 in both.  1.4 -> 2^0, 1.5 -> 2^1.
    e = O.scale_exponent_constopt(np.array([0.72, 0.70, 1.0, 1.4, 1.5, 0.0, 1e300, 1e-300]), 1.0)
    assert list(e) == [0, -1, 0, 0, 1, -127, 127, -127]


def test_constopt_codes_saturate_at_six():
    # absmax m = 1 / 0.156 gives s = c m = 1 (E = 0): the absmax element
    # (6.41 before scaling) saturates to the top code, 6.0
    m = 1.0 / O.CONSTOPT_C
    x = np.zeros((1, 32))
    x[0, 0], x[0, 1], x[0, 2] = m, -m, 1.25
    codes, sb = O.quantize_fp4(x, "constopt")
    assert sb[0, 0] == 127
    assert codes[0, 0] == 7 and codes[0, 1] == 15 and codes[0, 2] == 2     # 1.25 -> 1.0 (tie to even)
    assert O.dequantize_fp4(codes, sb)[0, 0] == 6.0
    # the absmax rule never clips: the same group gets E = 1 (6.41 <= 12)
    codes2, sb2 = O.quantize_fp4(x)
    assert sb2[0, 0] == 128 and codes2[0, 0] == 5                            # 6.41 / 2 = 3.2 -> 3.0 (code 5)


def test_constopt_power_of_two_optimum_matches_pages():
    # [review] §3.3 / §6.2, [commentary] footnote 13: c = 0.195 is the optimum of
    # the power-of-two rule (0.156 being the optimum of an unconstrained scale).
    # On rotated unit vectors the quantizer's MSE under R9 is least at 0.195; the
    # paper's default 0.156 and raw absmax (c = 1) are worse under the same rule.
    g = golden("constopt_constants.json")
    rng = np.random.default_rng(12)
    x = rng.standard_normal((2000, 128))
    y = O.wht(x / np.linalg.norm(x, axis=1, keepdims=True))

    def mse(c):
        codes, sb = O.quantize_fp4(y, "constopt", c)
        return np.mean(np.sum((O.dequantize_fp4(codes, sb) - y) ** 2, axis=1))

    cs = np.round(np.arange(0.180, 0.2101, 0.005), 3)
    errs = [mse(c) for c in cs]
    best = cs[int(np.argmin(errs))]
    assert abs(best - g["c_power_of_two_optimal"]) <= 0.005, (best, errs)
    assert mse(g["c_default_mse_optimal"]) > min(errs)
    assert mse(g["c_raw_absmax"]) > mse(g["c_default_mse_optimal"])


# ---------------------------------------------------------------- E2M1
def _e2m1_from_bits(code):
    """Value of an E2M1 bit pattern from the format: 1 sign, 2 exponent (bias 1),
    1 mantissa bit; exponent 0 is subnormal."""
    s = -1.0 if code & 8 else 1.0
    e, m = (code >> 1) & 3, code & 1
    return s * (m * 0.5 if e == 0 else (1 + m / 2) * 2.0 ** (e - 1))


def test_e2m1_levels_follow_bit_format():
    for c in range(16):
        assert O.e2m1_decode(c) == _e2m1_from_bits(c)
        assert np.signbit(O.e2m1_decode(c)) == bool(c & 8)


def test_e2m1_round_to_nearest_even_exhaustive():
    levels = [_e2m1_from_bits(c) for c in range(8)]
    for c, lv in enumerate(levels):
        assert O.e2m1_encode(lv) == c and O.e2m1_encode(-lv) == c | 8
    for c in range(7):
        lo, hi = levels[c], levels[c + 1]
        mid = (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        assert O.e2m1_encode(mid) == even
        assert O.e2m1_encode(-mid) == even | 8
        assert O.e2m1_encode(np.nextafter(mid, 0)) == c
        assert O.e2m1_encode(np.nextafter(mid, 10)) == c + 1
    assert O.e2m1_encode(6.5) == 7 and O.e2m1_encode(1e9) == 7 and O.e2m1_encode(-7.0) == 15
    assert O.e2m1_encode(-0.0) == 8 and O.e2m1_encode(-0.1) == 8 and O.e2m1_encode(0.0) == 0


def test_fp4_roundtrip_on_grid():
    # North-star pin: values already on the E2M1 x 2^k grid come back exactly.
    rng = np.random.default_rng(3)
    mags = np.array([_e2m1_from_bits(c) for c in range(8)])
    k = rng.integers(-20, 20, size=(2000, 1))
    x = rng.choice(mags, size=(2000, 32)) * rng.choice([-1.0, 1.0], size=(2000, 32))
    x = np.ldexp(x, k)
    codes, sb = O.quantize_fp4(x)
    assert np.array_equal(O.dequantize_fp4(codes, sb), x)


def test_fp4_quantizer_distortion_vs_published_bounds():
    # [tq-guide] 이론적 보장: D_mse >= 1/4^b; FP4 plus one scale byte per 32 is
    # 4.25 bits per element.  The fixed grid sits above TurboQuant's 4-bit value.
    g = golden("tq_distortion.json")
    rng = np.random.default_rng(4)
    x = rng.standard_normal((20000, 128))
    x /= np.linalg.norm(x, axis=1, keepdims=True)
    y = O.wht(x)
    codes, sb = O.quantize_fp4(y)
    mse = np.mean(np.sum((O.dequantize_fp4(codes, sb) - y) ** 2, axis=1))
    assert mse >= 4.0 ** -4.25
    assert mse >= g["lower_bound"][3] and mse >= g["turboquant_mse"][3]
    assert mse < 0.03


# ---------------------------------------------------------------- packing / format
def test_pack_unpack_identity_all_bytes():
    b = np.arange(256, dtype=np.uint8).reshape(1, 256)
    assert np.array_equal(O.pack_nibbles(O.unpack_nibbles(b)), b)
    assert np.array_equal(O.unpack_nibbles(np.array([0x21], np.uint8)), [1, 2])  # low nibble first


def test_format_facts_printed_on_pages():
    f = golden("format_facts.json")
    d = 128
    blk = O.head_block_bytes(O.FMT_FP4, d)
    groups = O.PAGE_SIZE * d // f["group_channels"]
    assert blk == groups * f["bytes_per_group"]
    assert 8 * blk / (O.PAGE_SIZE * d) == f["bits_per_element"]
    assert 1 - f["code_bits"] / f["bits_per_element"] < f["within_fraction_of_ideal_4bit"]
    T, H = 65536, 8
    assert T // O.PAGE_SIZE * O.page_bytes(O.FMT_FP4, H, d) == T * H * d * 17 // 32
    assert O.head_block_bytes(O.FMT_FP8, d) * 2 == O.head_block_bytes(O.FMT_BF16, d)


@pytest.mark.parametrize("fmt", [O.FMT_FP4, O.FMT_FP8, O.FMT_BF16])
@pytest.mark.parametrize("d", [64, 128])
def test_page_layout_is_a_bijection(fmt, d):
    """Writing all 16 slots of a page touches every byte of each head block exactly
    once, for K and for V: the offset helpers tile the block."""
    counts = {}
    for is_v in (False, True):
        cnt = np.zeros(O.head_block_bytes(fmt, d), np.int64)
        tok = np.arange(16)[:, None]
        if fmt == O.FMT_FP4:
            code = (O.fp4_v_code_offset if is_v else O.fp4_k_code_offset)(tok, np.arange(d // 2)[None], d)
            sc = (O.fp4_v_scale_offset if is_v else O.fp4_k_scale_offset)(tok, np.arange(d // 32)[None], d)
            np.add.at(cnt, code.ravel(), 1)
            np.add.at(cnt, sc.ravel(), 1)
        elif fmt == O.FMT_FP8:
            off = (O.fp8_v_offset if is_v else O.fp8_k_offset)(tok, np.arange(d)[None], d)
            np.add.at(cnt, off.ravel(), 1)
        else:
            idx = (O.bf16_v_index if is_v else O.bf16_k_index)(tok, np.arange(d)[None], d)
            np.add.at(cnt, (2 * idx).ravel(), 1)
            np.add.at(cnt, (2 * idx + 1).ravel(), 1)
        counts[is_v] = cnt
        assert np.all(cnt == 1)


@pytest.mark.parametrize("H", [1, 2, 3, 4, 5, 8])
def test_fp4_block_positions_permute_heads_and_rotate_pairs(H):
    # Reading R8: in every page the heads' blocks take each position once; for
    # an even H_kv the heads of a pair stay adjacent and the pairs rotate by one
    # pair position from page to page, so over H_kv / 2 consecutive pages every
    # pair starts at every pair position.
    for page in list(range(12)) + [2 ** 30 + 3, 2 ** 31 - 1]:
        pos = O.fp4_block_position(np.arange(H), page, H)
        assert sorted(pos.tolist()) == list(range(H))
        if H % 2 == 0:
            assert np.all(pos[1::2] == pos[0::2] + 1) and np.all(pos[0::2] % 2 == 0)
            assert np.array_equal(pos[0::2] // 2, (np.arange(H // 2) + page) % (H // 2))
    assert O.fp4_block_position(3, 0, 8) == 3


@pytest.mark.parametrize("H", [1, 3, 8])
@pytest.mark.parametrize("d", [64, 128])
def test_fp8_page_rotation_tiles_the_page_like_a_256_byte_stride(H, d):
    # Reading R8: the FP8 page's bytes (blocks back to back) rotate by 256 bytes
    # per page id.  Each page is covered once, and a byte's address modulo
    # 16 KB equals the one a page stride of page_bytes + 256 would give it
    # (when the page is 16 KB).
    pb = O.page_bytes(O.FMT_FP8, H, d)
    tok, ch = np.arange(16)[:, None], np.arange(d)[None, :]
    for page in (0, 1, 5, 63, 64, 1000, 2 ** 31 - 1):
        cnt = np.zeros(pb, np.int64)
        for h in range(H):
            for fn in (O.fp8_k_offset, O.fp8_v_offset):
                np.add.at(cnt, O.fp8_page_offset(h, fn(tok, ch, d), page, H, d).ravel(), 1)
        assert np.all(cnt == 2)                  # K and V offsets each tile the page once
    if pb == 16384:
        b = np.arange(pb)
        h, within = b // O.head_block_bytes(O.FMT_FP8, d), b % O.head_block_bytes(O.FMT_FP8, d)
        for page in (0, 3, 77):
            rotated = page * pb + O.fp8_page_offset(h, within, page, H, d)
            strided = page * (pb + 256) + b
            assert np.array_equal(rotated % 16384, strided % 16384)


# ---------------------------------------------------------------- E4M3 / bf16
def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3_decode(codes)
    nan = (codes & 0x7F) == 0x7F
    assert np.all(np.isnan(got[nan])) and np.all(np.isnan(ref[nan]))
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


def test_e4m3_encode_roundtrip_and_ties():
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    assert np.array_equal(O.e4m3_encode(O.e4m3_decode(finite)), finite)
    pos = O.e4m3_decode(np.arange(0x7F))
    mids = (pos[:-1] + pos[1:]) / 2
    enc = O.e4m3_encode(mids)
    lower = np.arange(0x7E)
    assert np.array_equal(enc, np.where(lower % 2 == 0, lower, lower + 1))    # ties to even
    assert O.e4m3_encode(449.0) == 0x7E and O.e4m3_encode(1e6) == 0x7E and O.e4m3_encode(-1e6) == 0xFE
    assert O.e4m3_encode(-0.0) == 0x80


def test_e4m3_encode_matches_torch_cast():
    rng = np.random.default_rng(5)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(10.0) ** rng.integers(-4, 3, 200000),
        (O.e4m3_decode(np.arange(0x7E)) + O.e4m3_decode(np.arange(1, 0x7F))) / 2,   # midpoints
    ]).astype(np.float32)
    x = np.concatenate([x, -x])
    x = x[np.abs(x) < 464]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_encode(x.astype(np.float64)), ref)


def test_bf16_round_matches_torch_cast():
    rng = np.random.default_rng(6)
    x = rng.standard_normal(100000).astype(np.float32)
    ties = ((x.view(np.uint32) & 0xFFFF0000) | 0x8000).view(np.float32)     # exact halfway cases
    x = np.concatenate([x, ties, -ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.bf16_round_bits(x), ref)


# ---------------------------------------------------------------- cache write / read
def _grid_workload(d=64, T=48, H=2, seed=7):
    """Inputs whose rotation lands exactly on the FP4 grid (d = 64: c_d = 1/8 makes
    the WHT exactly invertible), so the whole write path must be lossless."""
    rng = np.random.default_rng(seed)
    mags = np.array([_e2m1_from_bits(c) for c in range(8)])
    y = rng.choice(mags, size=(T, H, d)) * rng.choice([-1.0, 1.0], size=(T, H, d))
    y = np.ldexp(y.reshape(T, H, d // 32, 32), rng.integers(-3, 3, size=(T, H, d // 32, 1))).reshape(T, H, d)
    x = O.wht(y)                                       # exact: y dyadic, c = 1/8
    assert np.array_equal(x.astype(np.float32).astype(np.float64), x)
    assert np.array_equal(O.wht(x), y)
    return x.astype(np.float32), y


def test_append_fp4_end_to_end_exact_on_d64():
    x, y = _grid_workload()
    T, H, d = x.shape
    rng = np.random.default_rng(8)
    pages = rng.permutation(8)
    slots = (pages[np.arange(T) // 16] * 16 + np.arange(T) % 16).astype(np.int32)
    kp, vp = O.new_pool(O.FMT_FP4, 8, H, d), O.new_pool(O.FMT_FP4, 8, H, d)
    O.append(O.FMT_FP4, kp, vp, x, x, slots, in_dtype="f32")
    table = pages[:3]
    for h in range(H):
        for is_v, pool in ((False, kp), (True, vp)):
            assert np.array_equal(O.gather_dequant(O.FMT_FP4, pool, table, T, h, d, is_v), y[:, h])


def test_append_skips_negative_slots_and_writes_nothing_else():
    x, _ = _grid_workload(T=16, H=1)
    kp, vp = O.new_pool(O.FMT_FP4, 2, 1, 64), O.new_pool(O.FMT_FP4, 2, 1, 64)
    slots = np.full(16, -1, np.int32)
    slots[3] = 16 + 5
    O.append(O.FMT_FP4, kp, vp, x, x, slots, in_dtype="f32")
    assert not kp[0].any() and not vp[0].any()
    blk = kp[1, 0]
    touched = np.concatenate([O.fp4_k_code_offset(5, np.arange(32), 64), O.fp4_k_scale_offset(5, np.arange(2), 64)])
    mask = np.zeros(blk.size, bool); mask[touched] = True
    assert not blk[~mask].any()


# ---------------------------------------------------------------- attention
def _brute_attention(q, K, V, scale):
    """Plain loops in Python floats: softmax(scale q.k) weighted sum of v."""
    s = [scale * sum(a * b for a, b in zip(q, k)) for k in K]
    mx = max(s)
    w = [math.exp(t - mx) for t in s]
    tot = sum(w)
    return [sum(w[j] * V[j][c] for j in range(len(V))) / tot for c in range(len(q))]


def test_fp4_decode_equals_plain_attention_on_exact_inputs():
    # Quantizer bypassed in effect: inputs are exact on the FP4 / E4M3 grids, so the
    # rotated-and-unrotated FP4 path must equal attention on the original vectors.
    d, T, H, G = 64, 40, 2, 3
    x_k, _ = _grid_workload(d=d, T=T, H=H, seed=9)
    x_v, _ = _grid_workload(d=d, T=T, H=H, seed=10)
    rng = np.random.default_rng(11)
    q_rot = rng.choice([0.0, 0.5, 1.0, -1.0, 2.0, -1.5, 0.25, -3.0], size=(2, H * G, d))
    q = O.wht(q_rot).astype(np.float32)
    assert np.array_equal(O.wht(q.astype(np.float64)), q_rot)
    lens = np.array([T, 17])
    pages = rng.permutation(6)
    table = np.stack([pages[:3], pages[3:6]])
    kp, vp = O.new_pool(O.FMT_FP4, 6, H, d), O.new_pool(O.FMT_FP4, 6, H, d)
    for b in range(2):
        L = lens[b]
        slots = table[b][np.arange(L) // 16] * 16 + np.arange(L) % 16
        O.append(O.FMT_FP4, kp, vp, x_k[:L], x_v[:L], slots, in_dtype="f32")
    scale = 1 / math.sqrt(d)
    out = O.decode_attention(O.FMT_FP4, kp, vp, H, d, q, table, lens, scale, in_dtype="f32")
    for b in range(2):
        for h in range(H * G):
            ref = _brute_attention(q[b, h].astype(np.float64), x_k[:lens[b], h // G].astype(np.float64),
                                   x_v[:lens[b], h // G].astype(np.float64), scale)
            np.testing.assert_allclose(out[b, h], ref, rtol=0, atol=1e-12)


def test_fp4_prefill_equals_causal_attention_on_exact_inputs():
    # R10 on inputs exact on the FP4 / E4M3 grids: every chunk row equals plain
    # causal attention (a triangular mask over the chunk) on the original vectors.
    d, T, H, G = 64, 40, 2, 3
    x_k, _ = _grid_workload(d=d, T=T, H=H, seed=19)
    x_v, _ = _grid_workload(d=d, T=T, H=H, seed=20)
    rng = np.random.default_rng(21)
    lens, chunks = np.array([T, 21]), np.array([7, 21])               # a chunk after a prefix; a whole prompt
    q_rot = rng.choice([0.0, 0.5, 1.0, -1.0, 2.0, -1.5, 0.25, -3.0], size=(int(chunks.sum()), H * G, d))
    q = O.wht(q_rot).astype(np.float32)
    pages = rng.permutation(6)
    table = np.stack([pages[:3], pages[3:6]])
    kp, vp = O.new_pool(O.FMT_FP4, 6, H, d), O.new_pool(O.FMT_FP4, 6, H, d)
    for b in range(2):
        L = lens[b]
        slots = table[b][np.arange(L) // 16] * 16 + np.arange(L) % 16
        O.append(O.FMT_FP4, kp, vp, x_k[:L], x_v[:L], slots, in_dtype="f32")
    scale = 1 / math.sqrt(d)
    out = O.prefill_attention(O.FMT_FP4, kp, vp, H, d, q, chunks, table, lens, scale, in_dtype="f32")
    row = 0
    for b in range(2):
        for j in range(chunks[b]):
            P = lens[b] - chunks[b] + j                                 # the token's position
            for h in range(H * G):
                Kx = x_k[:P + 1, h // G].astype(np.float64)
                Vx = x_v[:P + 1, h // G].astype(np.float64)
                ref = _brute_attention(q[row, h].astype(np.float64), Kx, Vx, scale)
                np.testing.assert_allclose(out[row, h], ref, rtol=0, atol=1e-12)
            row += 1
    # causality: changing keys and values after a token's position leaves its row alone
    x_k2, x_v2 = x_k.copy(), x_v.copy()
    x_k2[36:], x_v2[36:] = x_k[36:] * 2, -x_v[36:]
    kp2, vp2 = O.new_pool(O.FMT_FP4, 6, H, d), O.new_pool(O.FMT_FP4, 6, H, d)
    for b in range(2):
        L = lens[b]
        slots = table[b][np.arange(L) // 16] * 16 + np.arange(L) % 16
        O.append(O.FMT_FP4, kp2, vp2, x_k2[:L], x_v2[:L], slots, in_dtype="f32")
    out2 = O.prefill_attention(O.FMT_FP4, kp2, vp2, H, d, q, chunks, table, lens, scale, in_dtype="f32")
    keep = 36 - (lens[0] - chunks[0])                                 # sequence 0's chunk tokens before position 36
    assert keep == 3
    assert np.array_equal(out2[:keep], out[:keep])                    # positions 33 .. 35
    assert all(not np.array_equal(out2[r], out[r]) for r in range(keep, chunks[0]))
    assert np.array_equal(out2[chunks[0]:], out[chunks[0]:])          # sequence 1 is 21 tokens long


@pytest.mark.parametrize("d", [64, 128])
def test_signed_rotation_is_library_hadamard_times_sign_diagonal(d):
    # R12: R = c_d H_d diag(s), built here from scipy's Hadamard matrix; R is
    # orthogonal and unrotate is its transpose.
    rng = np.random.default_rng(40 + d)
    s = rng.choice([-1.0, 1.0], size=d)
    R = scipy.linalg.hadamard(d).astype(np.float64) / math.sqrt(d) @ np.diag(s)
    x = rng.standard_normal((5, d))
    np.testing.assert_allclose(O.rotate(x, s), x @ R.T, rtol=0, atol=1e-14)
    np.testing.assert_allclose(O.unrotate(x, s), x @ R, rtol=0, atol=1e-14)
    np.testing.assert_allclose(O.unrotate(O.rotate(x, s), s), x, rtol=0, atol=1e-14)
    np.testing.assert_allclose(R.T @ R, np.eye(d), rtol=0, atol=1e-14)
    assert np.array_equal(O.rotate(x, np.ones(d)), O.wht(x))
    with pytest.raises(ValueError):
        O.rotate(x, np.full(d, 0.5))


def test_all_negative_signs_flip_every_nonzero_code():
    # s = -1 everywhere makes R x = -(c_d H_d x): the same scale bytes, and every
    # code's sign bit flipped except where the rotated value is exactly zero (+0
    # in both, R2).  Rows: d = 64 grid rows scaled off the grid, so the codes
    # include exact zeros, small values of both signs and saturated ones.
    d = 64
    x, _ = _grid_workload(d=d, T=16, H=2, seed=41)
    x = (x.astype(np.float64) * 1.37).astype(np.float32)
    zero = (x.astype(np.float64) @ scipy.linalg.hadamard(d).astype(np.float64)) == 0.0   # [16][2][d]
    assert zero.any() and not zero.all()
    slots = np.arange(16, dtype=np.int32)
    pools = {}
    for name, sg in (("plain", None), ("neg", -np.ones(d))):
        kp, vp = O.new_pool(O.FMT_FP4, 1, 2, d), O.new_pool(O.FMT_FP4, 1, 2, d)
        O.append(O.FMT_FP4, kp, vp, x, x, slots, in_dtype="f32", signs=sg)
        pools[name] = (kp, vp)
    cj = np.arange(d // 2)
    for pool_i, is_v in ((0, False), (1, True)):
        cf = O.fp4_v_code_offset if is_v else O.fp4_k_code_offset
        sf = O.fp4_v_scale_offset if is_v else O.fp4_k_scale_offset
        for h in range(2):
            a = pools["plain"][pool_i].reshape(1, 2, -1)[0, h]
            b = pools["neg"][pool_i].reshape(1, 2, -1)[0, h]
            for t in range(16):
                ca = O.unpack_nibbles(a[cf(t, cj, d)])
                cb = O.unpack_nibbles(b[cf(t, cj, d)])
                assert np.array_equal(np.where(zero[t, h], ca, ca ^ 8), cb)
                assert np.array_equal(ca[zero[t, h]], np.zeros(int(zero[t, h].sum()), np.uint8))
                assert np.array_equal(a[sf(t, np.arange(d // 32), d)], b[sf(t, np.arange(d // 32), d)])


@pytest.mark.parametrize("variant", ["signs", "k_only", "k_only_signs"])
def test_fp4_rotation_variants_equal_plain_attention_on_exact_inputs(variant):
    # R11 / R12 on inputs exact on the FP4 / E4M3 grids after the variant's
    # rotation (K and the query through R = c_d H_d diag(s), V through R or left
    # as it is): decode and prefill must equal plain attention on the original
    # vectors.  A sign left out anywhere, or V rotated under k_only, puts the
    # rows off the grid and fails by the quantization error.
    d, T, H, G = 64, 40, 2, 3
    k_only = variant.startswith("k_only")
    rng = np.random.default_rng(50 + len(variant))
    s = rng.choice([-1.0, 1.0], size=d) if variant.endswith("signs") else None
    sv = np.ones(d) if s is None else s
    _, y_k = _grid_workload(d=d, T=T, H=H, seed=51)
    _, y_v = _grid_workload(d=d, T=T, H=H, seed=52)
    x_k = (sv * O.wht(y_k)).astype(np.float32)                  # R^T y: exact at d = 64
    x_v = (y_v if k_only else sv * O.wht(y_v)).astype(np.float32)
    assert np.array_equal(O.rotate(x_k.astype(np.float64), s), y_k)
    q_rot = rng.choice([0.0, 0.5, 1.0, -1.0, 2.0, -1.5, 0.25, -3.0], size=(2, H * G, d))
    q = (sv * O.wht(q_rot)).astype(np.float32)
    lens = np.array([T, 17])
    pages = rng.permutation(6)
    table = np.stack([pages[:3], pages[3:6]])
    kp, vp = O.new_pool(O.FMT_FP4, 6, H, d), O.new_pool(O.FMT_FP4, 6, H, d)
    for b in range(2):
        L = lens[b]
        slots = table[b][np.arange(L) // 16] * 16 + np.arange(L) % 16
        O.append(O.FMT_FP4, kp, vp, x_k[:L], x_v[:L], slots, in_dtype="f32", k_only=k_only, signs=s)
    for h in range(H):
        assert np.array_equal(O.gather_dequant(O.FMT_FP4, vp, table[0], T, h, d, True), y_v[:, h])
    scale = 1 / math.sqrt(d)
    out = O.decode_attention(O.FMT_FP4, kp, vp, H, d, q, table, lens, scale, in_dtype="f32", k_only=k_only,
                             signs=s)
    for b in range(2):
        for h in range(H * G):
            ref = _brute_attention(q[b, h].astype(np.float64), x_k[:lens[b], h // G].astype(np.float64),
                                   x_v[:lens[b], h // G].astype(np.float64), scale)
            np.testing.assert_allclose(out[b, h], ref, rtol=0, atol=1e-12)
    # prefill: a 5-token chunk at the end of sequence 0
    qc = np.repeat(q[:1], 5, axis=0)
    pf = O.prefill_attention(O.FMT_FP4, kp, vp, H, d, qc, np.array([5, 0]), table, lens, scale, in_dtype="f32",
                             k_only=k_only, signs=s)
    for j in range(5):
        P = T - 5 + j
        for h in range(H * G):
            ref = _brute_attention(qc[j, h].astype(np.float64), x_k[:P + 1, h // G].astype(np.float64),
                                   x_v[:P + 1, h // G].astype(np.float64), scale)
            np.testing.assert_allclose(pf[j, h], ref, rtol=0, atol=1e-12)
    with pytest.raises(ValueError):
        O.append(O.FMT_FP8, O.new_pool(O.FMT_FP8, 6, H, d), O.new_pool(O.FMT_FP8, 6, H, d), x_k[:1], x_v[:1],
                 np.zeros(1, np.int32), in_dtype="f32", k_only=True)


def _small_pools(fmt, seed=12, B=3, H=2, G=4, d=128, lens=(1, 33, 70)):
    wl = W.make_workload("attn", B, H * G, H, d, list(lens), list(lens), seed=seed)
    kp, vp = O.new_pool(fmt, wl.num_pages, H, d), O.new_pool(fmt, wl.num_pages, H, d)
    O.append(fmt, kp, vp, wl.k, wl.v, wl.slot_mapping)
    return wl, kp, vp


@pytest.mark.parametrize("fmt", [O.FMT_FP4, O.FMT_FP8, O.FMT_BF16])
def test_attention_special_cases(fmt):
    wl, kp, vp = _small_pools(fmt)
    d, H = wl.head_dim, wl.num_kv_heads
    scale = 1 / math.sqrt(d)
    out = O.decode_attention(fmt, kp, vp, H, d, wl.q, wl.page_table, wl.seq_lens, scale)
    unrot = O.wht if fmt == O.FMT_FP4 else (lambda v: v)
    G = wl.num_q_heads // H
    for h in range(wl.num_q_heads):     # seq_len 1: output is that token's value row
        v0 = O.gather_dequant(fmt, vp, wl.page_table[0], 1, h // G, d, True)[0]
        np.testing.assert_allclose(out[0, h], unrot(v0), rtol=0, atol=1e-12)
    # q = 0: equal logits, output is the mean of the value rows
    q0 = np.zeros_like(wl.q)
    out0 = O.decode_attention(fmt, kp, vp, H, d, q0, wl.page_table, wl.seq_lens, scale)
    for b in range(wl.batch):
        V = O.gather_dequant(fmt, vp, wl.page_table[b], wl.seq_lens[b], 0, d, True)
        np.testing.assert_allclose(out0[b, 0], unrot(V.mean(0)), rtol=0, atol=1e-12)
    # empty sequence gives a zero row
    lens0 = wl.seq_lens.copy(); lens0[1] = 0
    oz = O.decode_attention(fmt, kp, vp, H, d, wl.q, wl.page_table, lens0, scale)
    assert not oz[1].any()


def _baseline_pools(fmt, k, v, lens, H, d, in_dtype, seed):
    rng = np.random.default_rng(seed)
    npg = [(L + 15) // 16 for L in lens]
    pages = rng.permutation(sum(npg))
    table = np.zeros((len(lens), max(npg)), np.int64)
    kp, vp = O.new_pool(fmt, sum(npg), H, d), O.new_pool(fmt, sum(npg), H, d)
    off = 0
    for b, L in enumerate(lens):
        table[b, :npg[b]] = pages[off:off + npg[b]]
        off += npg[b]
        slots = table[b][np.arange(L) // 16] * 16 + np.arange(L) % 16
        O.append(fmt, kp, vp, k[b, :L], v[b, :L], slots.astype(np.int32), in_dtype=in_dtype)
    return kp, vp, table


@pytest.mark.parametrize("fmt", [O.FMT_FP8, O.FMT_BF16])
def test_baseline_decode_equals_plain_attention_on_grid_inputs(fmt):
    # The FP8 / BF16 branch of the decode: q, K and V exactly on the format's
    # grid (E4M3 values from torch's float8_e4m3fn, or bf16 values), so the
    # oracle must equal plain attention on the given vectors, unrotated.
    H, G, d, T = 2, 3, 64, 40
    lens = [T, 23]
    g = torch.Generator().manual_seed(31 + fmt)
    if fmt == O.FMT_FP8:
        def grid(*shape):
            b = torch.randint(0, 256, shape, generator=g, dtype=torch.int32).to(torch.uint8)
            b[(b & 0x7F) == 0x7F] = 0x3A                                  # no NaN codes
            b &= 0xBF                                                       # exponent field < 8: |x| < 2
            return b.view(torch.float8_e4m3fn).to(torch.float32).numpy()
        k, v, q = grid(2, T, H, d), grid(2, T, H, d), grid(2, H * G, d)
        args = dict(in_dtype="f32")
        kx, vx, qx = k, v, q
    else:
        def grid(*shape):
            t = torch.randn(*shape, generator=g).to(torch.bfloat16)
            return t.view(torch.int16).numpy().view(np.uint16), t.to(torch.float64).numpy()
        (k, kx), (v, vx), (q, qx) = grid(2, T, H, d), grid(2, T, H, d), grid(2, H * G, d)
        args = dict(in_dtype="bf16")
    kp, vp, table = _baseline_pools(fmt, k, v, lens, H, d, args["in_dtype"], seed=32)
    scale = 1 / math.sqrt(d)
    out = O.decode_attention(fmt, kp, vp, H, d, q, table, np.array(lens), scale, **args)
    for b in range(2):
        for h in range(H * G):
            ref = _brute_attention(np.asarray(qx[b, h], np.float64), np.asarray(kx[b, :lens[b], h // G], np.float64),
                                   np.asarray(vx[b, :lens[b], h // G], np.float64), scale)
            np.testing.assert_allclose(out[b, h], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("fmt", [O.FMT_FP8, O.FMT_BF16])
def test_baseline_decode_rounds_off_grid_inputs_like_torch(fmt):
    # Off-grid inputs: the FP8 baseline rounds q, K and V to E4M3 (no rotation,
    # no query scale), the BF16 baseline stores float32 K and V rounded to bf16
    # and takes the bf16 query as it is; the expected values come from torch's
    # float8_e4m3fn / bfloat16 casts and plain attention.
    H, G, d, T = 2, 4, 128, 37
    lens = [T, 9]
    rng = np.random.default_rng(41 + fmt)
    k = (rng.standard_normal((2, T, H, d)) * 3).astype(np.float32)
    v = (rng.standard_normal((2, T, H, d)) * 3).astype(np.float32)
    k[..., 5] *= 20                                           # outlier channel, still below 448
    q32 = rng.standard_normal((2, H * G, d)).astype(np.float32)
    kp, vp, table = _baseline_pools(fmt, k, v, lens, H, d, "f32", seed=42)
    if fmt == O.FMT_FP8:
        cast = lambda a: torch.from_numpy(a).to(torch.float8_e4m3fn).to(torch.float64).numpy()
        q, args, qx = q32, dict(in_dtype="f32"), cast(q32)
    else:
        cast = lambda a: torch.from_numpy(a).to(torch.bfloat16).to(torch.float64).numpy()
        qt = torch.from_numpy(q32).to(torch.bfloat16)
        q, args, qx = qt.view(torch.int16).numpy().view(np.uint16), dict(in_dtype="bf16"), qt.to(torch.float64).numpy()
    kx, vx = cast(k), cast(v)
    scale = 1 / math.sqrt(d)
    out = O.decode_attention(fmt, kp, vp, H, d, q, table, np.array(lens), scale, **args)
    for b in range(2):
        for h in range(H * G):
            ref = _brute_attention(qx[b, h], kx[b, :lens[b], h // G], vx[b, :lens[b], h // G], scale)
            np.testing.assert_allclose(out[b, h], ref, rtol=0, atol=1e-11)
    # a rotation anywhere in the branch would move the rows far from these values
    rot = O.decode_attention(O.FMT_FP4, *_baseline_pools(O.FMT_FP4, k, v, lens, H, d, "f32", seed=42)[:2], H, d,
                             q32, table, np.array(lens), scale, in_dtype="f32")
    assert np.abs(rot - out).max() > 1e-3


def test_attention_weights_sum_to_one_and_gqa_mapping():
    wl, kp, vp = _small_pools(O.FMT_FP4, seed=13)
    d, H, G = wl.head_dim, wl.num_kv_heads, wl.num_q_heads // wl.num_kv_heads
    # softmax weights sum to 1: with every value row equal to ones the output is ones
    K = np.random.default_rng(0).standard_normal((50, d))
    qh = np.random.default_rng(1).standard_normal((3, d))
    np.testing.assert_allclose(O.attention(qh, K, np.ones((50, d)), 0.3), 1.0, rtol=1e-14)
    # duplicated query heads give identical rows; GQA equals MHA with repeated KV
    q = wl.q.copy()
    q[:, 1] = q[:, 0]
    out = O.decode_attention(O.FMT_FP4, kp, vp, H, d, q, wl.page_table, wl.seq_lens, 0.1)
    assert np.array_equal(out[:, 0], out[:, 1])
    b = 2
    for h in range(wl.num_q_heads):
        qhat = O.e4m3_decode(O.rotate_quantize_query(q[b, h]))
        K = O.gather_dequant(O.FMT_FP4, kp, wl.page_table[b], wl.seq_lens[b], h // G, d, False)
        V = O.gather_dequant(O.FMT_FP4, vp, wl.page_table[b], wl.seq_lens[b], h // G, d, True)
        np.testing.assert_allclose(out[b, h], O.wht(O.attention(qhat[None], K, V, 0.1)[0]), rtol=0, atol=1e-14)


# ---------------------------------------------------------------- PV operand precision
def test_fold_p_fp8_exact_when_exponents_match_and_p_on_grid():
    # Closed form: with one V exponent per 32-token block and p on the E4M3 grid,
    # the folded FP8 operand is p itself and the scaled PV is the exact product.
    rng = np.random.default_rng(60)
    T, d = 96, 64
    grid = np.array([1.0, 0.75, 0.5, 0.375, 0.25, 0.125, 0.0625, 0.015625])
    p = rng.choice(grid, size=(3, T))
    e_blk = rng.integers(-6, 6, size=(T // 32, d // 32))
    sb = (np.repeat(e_blk, 32, axis=0) + 127).astype(np.uint8)          # [T][d/32]
    codes = rng.integers(0, 16, size=(T, d)).astype(np.uint8)
    for g in range(d // 32):
        e = sb[:, g].astype(np.int64) - 127
        assert np.array_equal(O.fold_p_fp8(p, e), np.ldexp(p, e[None, :]))        # p 2^E_t, unrounded
    np.testing.assert_array_equal(O.pv_fp8_scaled(p, codes, sb), p @ O.dequantize_fp4(codes, sb))


def test_fold_p_fp8_error_within_e4m3_half_ulp():
    # E4M3 has 3 fraction bits: a folded value in the normal range [2^-6, 448]
    # rounds within 2^-4 relative; below half the least subnormal (2^-10) to 0.
    rng = np.random.default_rng(61)
    p = rng.uniform(0.0, 1.0, size=(4, 128))
    e = rng.integers(-20, 3, size=128)
    out = O.fold_p_fp8(p, e)
    M = np.repeat([e[i:i + 32].max() for i in range(0, 128, 32)], 32)
    folded = np.ldexp(p, e - M)
    normal = folded >= 2.0 ** -6
    assert normal.any() and (~normal).any()
    want = np.ldexp(p, e[None, :])                     # p 2^E_t
    rel = np.abs(out - want) / want
    assert np.all(rel[normal] <= 2.0 ** -4)
    assert np.all(out[folded < 2.0 ** -10] == 0.0)


def test_fold_p_fp8_with_headroom_rounds_like_torch_fp8():
    # R13's fold: block scale 2^M with M = (largest E of the 32-token block) - 8,
    # at least -127; the folded values P 2^(E_t - M) (at most 2^8) rounded by
    # torch's float8_e4m3fn cast.
    rng = np.random.default_rng(64)
    T = 80                                             # two whole blocks and a block of 16
    p = rng.uniform(0.0, 1.0, size=(3, T))
    p[:, 5] = 1.0
    e = rng.integers(-40, 6, size=T)
    e[64:] = rng.integers(-127, -121, size=T - 64)     # a block whose M is clamped to -127
    want = np.zeros_like(p)
    for b0 in range(0, T, 32):
        blk = range(b0, min(b0 + 32, T))
        M = max(max(int(e[t]) for t in blk) - 8, -127)
        for r in range(p.shape[0]):
            for t in blk:
                x = torch.tensor(math.ldexp(float(p[r, t]), int(e[t]) - M), dtype=torch.float64)
                want[r, t] = math.ldexp(float(x.to(torch.float8_e4m3fn).to(torch.float64)), M)
    got = O.fold_p_fp8(p, e, headroom=O.SPV_HEADROOM)
    np.testing.assert_array_equal(got, want)
    assert (got == 0).any() and (got > 0).any()


def _spv_case(rng, L, d, G=3, spread=(100, 141)):
    k = rng.standard_normal((L, d))
    vc = rng.integers(0, 16, size=(L, d)).astype(np.uint8)
    vs = rng.integers(spread[0], spread[1], size=(L, d // 32)).astype(np.uint8)
    q = rng.standard_normal((G, d))
    return q, k, vc, vs


@pytest.mark.parametrize("step", [128, 32, 7])
def test_scaled_pv_decode_without_rounding_is_plain_attention(step):
    # Closed form: the step-wise combination (each step against its own maximum,
    # weighted by exp(m_s - m)) is an identity of the softmax, so with the fold
    # left unrounded the result is the plain attention.
    rng = np.random.default_rng(65 + step)
    q, k, vc, vs = _spv_case(rng, 300, 64)
    got = O.attention_pv_scaled(q, k, vc, vs, 0.3, step=step, fold=False)
    want = O.attention(q, k, O.dequantize_fp4(vc, vs), 0.3)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


def test_scaled_pv_decode_uniform_probabilities_closed_form():
    # q = 0: every logit is 0, so every probability is exactly 1 and the fold
    # rounds only exact powers of two: 2^(E_t - M) for E_t - M >= -9 (down to the
    # least E4M3 subnormal), 0 below (2^-10 is a tie and rounds to the even 0).
    # The output is the mean over tokens of the values that survive.
    rng = np.random.default_rng(66)
    L, d = 300, 64
    _, k, vc, vs = _spv_case(rng, L, d, spread=(96, 141))      # exponent spreads up to 44 within a block
    vs[256:288] = rng.integers(0, 9, size=(32, d // 32))        # E <= -119: M clamped to -127
    q = np.zeros((2, d))
    vals = O.dequantize_fp4(vc, vs)
    e = vs.astype(np.int64) - 127
    want = np.zeros(d)
    for t in range(L):
        b0 = 32 * (t // 32)                                     # 32-token blocks of 128-token steps
        for c in range(d):
            g = c // 32
            M = max(max(int(e[u, g]) for u in range(b0, min(b0 + 32, L))) - 8, -127)
            if e[t, g] - M >= -9:
                want[c] += vals[t, c]
    want /= L
    dropped = sum(int(e[t, g] - max(e[32 * (t // 32):32 * (t // 32) + 32, g].max() - 8, -127) < -9)
                  for t in range(L) for g in range(d // 32))
    assert dropped > 0
    got = O.attention_pv_scaled(q, k, vc, vs, 1.0)
    np.testing.assert_allclose(got, np.tile(want, (2, 1)), rtol=1e-12, atol=1e-12 * np.abs(want).max())


def test_scaled_pv_decode_rows_gather_and_rotate_back():
    # On a cache written by append with q = 0 (probabilities exactly 1) and V's
    # exponents within 17 binades of each block's largest, every fold is exact,
    # so the scaled-PV decode rows equal the plain decode rows (same gather of
    # V, same rotation back).
    wl = W.make_workload("spv_rows", 2, 8, 2, 128, [200, 37], [200, 37], seed=67)
    kp = O.new_pool(O.FMT_FP4, wl.num_pages, 2, 128)
    vp = O.new_pool(O.FMT_FP4, wl.num_pages, 2, 128)
    O.append(O.FMT_FP4, kp, vp, wl.k, wl.v, wl.slot_mapping)
    q = np.zeros_like(wl.q)
    plain = O.decode_attention(O.FMT_FP4, kp, vp, 2, 128, q, wl.page_table, wl.seq_lens, 0.1)
    spv = O.decode_attention(O.FMT_FP4, kp, vp, 2, 128, q, wl.page_table, wl.seq_lens, 0.1, pv_scaled=True)
    np.testing.assert_allclose(spv, plain, rtol=0, atol=1e-12 * np.abs(plain).max())
    assert np.abs(plain).max() > 0
    with pytest.raises(ValueError):
        O.decode_attention(O.FMT_FP8, kp, vp, 2, 128, q, wl.page_table, wl.seq_lens, 0.1, pv_scaled=True)


def test_pv_f16_hi_lo_carries_22_bits():
    rng = np.random.default_rng(62)
    p = rng.uniform(2.0 ** -10, 1.0, size=(4, 200))
    v = O.dequantize_fp4(rng.integers(0, 16, size=(200, 64)).astype(np.uint8),
                         rng.integers(120, 133, size=(200, 2)).astype(np.uint8))
    # hi + lo is p to 2^-22 relative, or to 2^-25 absolute where lo is an f16
    # subnormal; V is exact in f16
    bound = (2.0 ** -22 * p + 2.0 ** -25) @ np.abs(v)
    err = np.abs(O.pv_f16_hi_lo(p, v) - p @ v)
    assert np.all(err <= bound * (1 + 1e-9) + 1e-12)
    hi_only = p.astype(np.float16).astype(np.float64) @ v
    assert np.all(np.abs(hi_only - p @ v) <= 2.0 ** -11 * p @ np.abs(v) * (1 + 1e-9))


def test_pv_precision_choice_on_decode_statistics():
    # What the PV operand precision costs on decode statistics (8 query heads of
    # one KV head, 8192 tokens, d = 128, K/V with outlier channels, rotated
    # cache): f16 hi + lo P stays far inside the 1e-3 relative-L2 output
    # tolerance; FP8 P with V's exponents folded in (the fully scaled-MFMA PV)
    # does not.
    wl = W.make_workload("pv_prec", 1, 8, 1, 128, [8192], [8192], seed=63)
    k = O.bf16_bits_to_f64(wl.k[:, 0])
    v = O.bf16_bits_to_f64(wl.v[:, 0])
    kc, ksb = O.quantize_fp4(O.wht(k))
    vc, vsb = O.quantize_fp4(O.wht(v))
    K, V = O.dequantize_fp4(kc, ksb), O.dequantize_fp4(vc, vsb)
    qhat = O.e4m3_decode(O.rotate_quantize_query(wl.q[0]))                # [8][128]
    s = (qhat @ K.T) / math.sqrt(128)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    l = p.sum(axis=1, keepdims=True)
    exact = O.wht(p @ V / l)
    res = {}
    for name, got in (("f16_hi_lo", O.pv_f16_hi_lo(p, V)), ("fp8_scaled", O.pv_fp8_scaled(p, vc, vsb))):
        o = O.wht(got / l)
        res[name] = (np.linalg.norm(o - exact) / np.linalg.norm(exact), np.abs(o - exact).max())
    # R13's decode: 128-token steps against their own maxima, headroom 8
    vcodes = O.unpack_nibbles(O.pack_nibbles(vc))
    o = O.wht(O.attention_pv_scaled(qhat, K, vcodes, vsb, 1 / math.sqrt(128)))
    res["r13_decode"] = (np.linalg.norm(o - exact) / np.linalg.norm(exact), np.abs(o - exact).max())
    print("PV precision (rel-L2, max-abs):", res)
    assert res["f16_hi_lo"][0] < 1e-5 and res["f16_hi_lo"][1] < 1e-4
    assert res["fp8_scaled"][0] > 1e-3
    assert 1e-3 < res["r13_decode"][0] < res["fp8_scaled"][0]
