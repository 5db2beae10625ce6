"""Plain float64 reference for the UltraQuant FP4 KV-cache write path and decode.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the library.

Sources, cited by page title and section:
  [review]      "[arXiv 2606.20474] UltraQuant: 컨텍스트가 긴 에이전트를 위한 4비트 KV 캐싱"
                (manon006.tistory.com/395)
  [commentary]  "kv-cache-4bit-serving-residency-collapse" commentary on the same
                paper (pheeree.github.io, 2026-09-01), whose footnotes quote the paper
  [tq-guide]    "TurboQuant 완전 정리 - 이론 최적에 근접한 KV 캐시·벡터 검색 양자화와
                vLLM 실측" (juhoplayground.github.io)

What the method computes ([review] §3.1, §3.2; [commentary] footnote 2):
  write path   x = WHT(row); per 32-channel group m = max|x_i|; scale exponent E
               stored as the UE8M0 byte E + 127; each x_i / 2**E rounded to an
               FP4 E2M1 level; 32 codes packed two per byte plus the scale byte,
               17 bytes per group (4.25 bits per element).
  dequant      value = code * 2**(byte - 127).
  decode       the query is rotated into the key basis and rounded to FP8 E4M3
               ([review] §3.2, §4.2); attention runs over the dequantized cache.

Readings where the pages are silent (each listed with its reason in the design doc):
  R1  K and V are both rotated; the attention output is rotated back.
  R2  WHT = Sylvester Hadamard in natural order, scaled by c_d = sqrt(1/d),
      over the whole head_dim, no random signs.  Each rotated value is the
      exact Hadamard sum times c_d (the double nearest sqrt(1/d)), rounded once
      to float64.  A rotated value whose exact sum is zero is +0: the exact
      transform has no signed zeros.
  R3  E = the least integer with m <= 6 * 2**E (never clips), clamped to
      [-127, 127]; an all-zero group gets E = -127.
  R4  E2M1 rounding is to nearest, ties to the even code; the sign bit is the
      sign of the value, so a negative value that rounds to zero is code 8.
  R5  Every rounding decision is taken on the float64 value (no float32 step).
  R6  FP8 is OCP E4M3 (bias 7, max 448), round to nearest even, saturating at
      448, sign copied for zero; no query scale.
  R7  sm_scale multiplies the logits; GQA maps query head h to KV head
      h // (H_q / H_kv).
  R8  Cache page layout: see ``head_block_bytes`` and the ``*_offset`` helpers.
  R10 Chunked prefill over the cache: a sequence's chunk of q_lens[b] query
      tokens holds its last positions (the chunk is written to the cache
      first); chunk token j at position P = seq_lens[b] - q_lens[b] + j attends
      to positions 0 .. P, each row exactly as the decode over that prefix.
  R9  constOpt scale mode (``scale_mode="constopt"``): s = c * m rounded once to
      float64 (c = 0.156 by default), E = the integer nearest to log2(s) (the
      log domain: the pages' "power-of-two-optimal" constant 0.195 is the
      optimum of that rule on rotated unit vectors, where linear-domain rounding
      would put it near 0.207), clamped to [-127, 127], m == 0 giving -127;
      codes then saturate at +-6 as in R4.
  R11 K-only rotation (``k_only=True``; [review] §3.1 table "Rotation": the
      Walsh-Hadamard rotation is applied to K; [commentary] footnote 1:
      "asymmetric K/V treatment"): K is rotated as in R1/R2, V is quantized in
      its own basis (a zero channel stored as +0, like a rotated zero in R2),
      and the attention output is not rotated back.
  R12 Randomized-sign Hadamard (``signs``; [tq-guide] "알고리즘 원리", "랜덤 회전과
      Beta 분포": a random +-1 diagonal times the Hadamard matrix): the rotation
      is R = c_d H_d diag(s) with one caller-drawn s in {+1, -1}^d per cache,
      applied to K, V and the query alike; the output goes back through
      R^T = diag(s) c_d H_d.  Without signs R is the plain R2 transform.
  R13 Scaled-MFMA PV (``pv_scaled``; [review] §3.2 "dequantization rule과
      scaled-MFMA", §6.3 optimization ladder; [commentary] footnote 2: the
      scaled matrix instruction takes FP4 codes with UE8M0 scales, so values
      are never widened to BF16).  V's scales run along head_dim while PV
      contracts over tokens, so they enter the product folded into FP8
      probabilities: per 32-channel group and block of 32 tokens, P * 2^(E_t - M)
      rounded to E4M3 with the block scale 2^M, M = the block's largest V
      exponent minus 8 (at least -127).  For the rounding not to depend on the
      order in which steps are visited, P is taken within each 128-token step
      (positions 128 s .. 128 s + 127) against that step's largest logit; the
      steps are combined as in the online softmax, with unrounded sums of P.

Parity pins: tests/test_oracle_pins.py (no function here is "parity unpinned").
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "PAGE_SIZE", "GROUP", "FMT_FP4", "FMT_FP8", "FMT_BF16",
    "sylvester_hadamard", "wht_scale", "exact_sum_rows", "wht", "rotate", "unrotate",
    "scale_exponent", "CONSTOPT_C", "SQRT2_UP", "scale_exponent_constopt",
    "E2M1_LEVELS", "e2m1_encode", "e2m1_decode",
    "quantize_fp4", "dequantize_fp4", "pack_nibbles", "unpack_nibbles",
    "e4m3_decode", "e4m3_encode", "bf16_bits_to_f64", "f32_to_f64", "bf16_round_bits",
    "head_block_bytes", "page_bytes", "new_pool", "prefill_attention",
    "fp4_block_position", "fp4_k_code_offset", "fp4_k_scale_offset", "fp4_v_code_offset", "fp4_v_scale_offset",
    "fp8_k_offset", "fp8_v_offset", "fp8_page_offset", "bf16_k_index", "bf16_v_index",
    "append", "gather_dequant", "rotate_quantize_query", "attention",
    "decode_attention", "decode_attention_rows",
    "pv_f16_hi_lo", "fold_p_fp8", "pv_fp8_scaled", "SPV_STEP", "SPV_HEADROOM", "attention_pv_scaled",
    "gather_fp4_codes",
]

PAGE_SIZE = 16          # tokens per page (vLLM-style paged cache; [review] §6.5.1)
GROUP = 32              # channels per scale group ([review] §3.1 table: "Group size")
FMT_FP4, FMT_FP8, FMT_BF16 = 0, 1, 2


# --------------------------------------------------------------------------
# Rotation ([review] §3.1: Walsh-Hadamard rotation; reading R2)
# --------------------------------------------------------------------------
def sylvester_hadamard(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix: H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]."""
    if d < 1 or d & (d - 1):
        raise ValueError("Hadamard order must be a power of two")
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def wht_scale(d: int) -> float:
    """c_d = sqrt(1/d): makes c_d * H_d orthogonal (and, H being symmetric, self-inverse)."""
    return float(np.sqrt(1.0 / d))


def exact_sum_rows(x) -> np.ndarray:
    """Per row of x (last axis): True when every partial sum of the values with
    any signs is exactly representable in float64, so that a float64 sum of them
    in any order and grouping is exact.

    Criterion: all values are integer multiples of 2**u (u = the lowest set bit
    of any of them) and sum |x_i| < 2**(u + 53); then every partial sum is such a
    multiple below that bound.  For bf16 rows this holds when the nonzero
    exponents span at most 38 binades, for float32 rows 22.  The float64 sum of
    the |x_i| used for the test is itself exact below the bound and, rounding
    being monotone, at or above it otherwise, so the test is exact.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    frac, ex = np.frexp(a)                                  # a = frac * 2**ex, frac in [0.5, 1)
    mant = np.ldexp(frac, 53).astype(np.int64)              # 53-bit integer significand (0 for a = 0)
    low = mant & -mant                                      # its lowest set bit
    lowexp = np.where(a > 0, np.frexp(low.astype(np.float64))[1] - 1 + ex - 53, 1 << 20)
    u = lowexp.min(axis=-1)                                 # 2**20: an all-zero row
    bound = np.ldexp(1.0, np.minimum(u + 53, 1023))
    return (a.sum(axis=-1) < bound) | (u == 1 << 20)


def _wht_exact_row(row: np.ndarray, c: float) -> np.ndarray:
    """RN(c * (H row)_k) + 0 for one row, the Hadamard sums in exact integer
    arithmetic (every float64 is a dyadic rational) and rounded once."""
    from fractions import Fraction
    fr = [Fraction(float(t)) for t in row]
    den = max(f.denominator for f in fr)                    # a power of two
    n = np.array([int(f * den) for f in fr], dtype=object)
    sums = sylvester_hadamard(row.size).astype(object) @ n  # exact Python integers
    cf = Fraction(c)
    return np.array([float(cf * int(s) / den) for s in sums], dtype=np.float64) + 0.0


def wht(x, exact=True) -> np.ndarray:
    """Normalized Walsh-Hadamard transform over the last axis: x -> c_d * (H_d x).

    exact=True (the write path and the query): each output is the exact sum
    S = (H_d x)_k multiplied by c_d and rounded once to float64, plus +0 (an
    exact zero is +0 whatever the signs of the inputs, reading R2).  Rows for
    which ``exact_sum_rows`` holds take the float64 matrix product, whose sums
    are then exact in any order; the other rows take exact integer arithmetic.

    exact=False (outputs compared within a tolerance): the float64 matrix
    product for every row, whose rounding errors are of order 2**-53 times the
    row's L1 norm.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    h = sylvester_hadamard(d).astype(np.float64)
    c = wht_scale(d)
    out = (x @ h) * c + 0.0                  # H symmetric: (H x)^T = x^T H
    if exact:
        flat_x, flat_o = x.reshape(-1, d), out.reshape(-1, d)
        for r in np.nonzero(~exact_sum_rows(flat_x))[0]:
            flat_o[r] = _wht_exact_row(flat_x[r], c)
    return out


def rotate(x, signs=None) -> np.ndarray:
    """R x over the last axis with R = c_d H_d diag(s) (reading R12): channel i
    negated where signs[i] = -1, then the normalized WHT; signs None is R2's R."""
    x = np.asarray(x, dtype=np.float64)
    if signs is not None:
        s = np.asarray(signs, dtype=np.float64)
        if s.shape != (x.shape[-1],) or not np.all(np.abs(s) == 1.0):
            raise ValueError("signs must be a +-1 vector of length head_dim")
        x = x * s
    return wht(x)


def unrotate(y, signs=None) -> np.ndarray:
    """R^T y = diag(s) c_d H_d y (the inverse of ``rotate``: c_d H_d is symmetric
    and orthogonal, diag(s) its own inverse)."""
    o = wht(y, exact=False)
    return o if signs is None else o * np.asarray(signs, dtype=np.float64)


# --------------------------------------------------------------------------
# UE8M0 group scale ([review] §3.1, §3.2; [commentary] footnote 2; reading R3)
# --------------------------------------------------------------------------
def scale_exponent(m) -> np.ndarray:
    """Least integer E with m <= 6 * 2**E, clamped to [-127, 127]; m == 0 gives -127.

    A float estimate ceil(log2(m/6)) is corrected with exact comparisons against
    6 * 2**E (exact in float64 for |E| <= 129) until E satisfies the definition:
    m <= 6 * 2**E and m > 6 * 2**(E-1).
    """
    m = np.asarray(m, dtype=np.float64)
    out = np.full(m.shape, -127, dtype=np.int64)
    nz = m > 0
    mz = m[nz]
    with np.errstate(divide="ignore"):
        e = np.ceil(np.log2(mz / 6.0))
    e = np.clip(e, -128, 129).astype(np.int64)
    for _ in range(4):
        too_small = mz > np.ldexp(6.0, e)                    # definition violated: raise E
        e = np.where(too_small & (e < 129), e + 1, e)
        not_least = (e > -128) & (mz <= np.ldexp(6.0, e - 1))  # a smaller E also works
        e = np.where(not_least, e - 1, e)
    out[nz] = np.clip(e, -127, 127)
    return out


# --------------------------------------------------------------------------
# constOpt group scale ([review] §3.1 and §3.3 "constant-optimized scaling": the
# absmax times a global constant c, stored as the nearest power of two, c = 0.156
# from offline calibration; §6.2 ablation of c; [commentary] footnote 13; R9)
# --------------------------------------------------------------------------
CONSTOPT_C = 0.156
SQRT2_UP = float.fromhex("0x1.6a09e667f3bcdp+0")     # the least double above sqrt(2)


def scale_exponent_constopt(m, c=CONSTOPT_C) -> np.ndarray:
    """The integer nearest to log2(s), s = c * m rounded once to float64, clamped to
    [-127, 127]; m == 0 gives -127.

    With s = M * 2**e, M in [1, 2): E = e + 1 when M > sqrt(2), else e.  sqrt(2)
    is irrational, so no double equals it (no ties) and M > sqrt(2) exactly when
    M >= SQRT2_UP.
    """
    m = np.asarray(m, dtype=np.float64)
    s = np.float64(c) * m
    out = np.full(m.shape, -127, dtype=np.int64)
    nz = s > 0
    frac, ex = np.frexp(s[nz])                               # s = frac * 2**ex, frac in [0.5, 1)
    e = (ex - 1).astype(np.int64) + (2.0 * frac >= SQRT2_UP)
    out[nz] = np.clip(e, -127, 127)
    return out


# --------------------------------------------------------------------------
# FP4 E2M1 codes ([review] §3.1 table "Code grid", §6.5; readings R4, R5)
# --------------------------------------------------------------------------
E2M1_LEVELS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])  # magnitude codes 0..7


def _nearest_even(a: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Index of the entry of the increasing ``table`` nearest to a >= 0, ties to the
    even index; values above the last entry map to the last index (saturation)."""
    a = np.asarray(a, dtype=np.float64)
    i = np.searchsorted(table, a, side="right") - 1          # table[i] <= a
    i = np.clip(i, 0, len(table) - 1)
    top = i == len(table) - 1
    j = np.minimum(i + 1, len(table) - 1)
    below = a - table[i]                                     # distance to the lower neighbour
    above = table[j] - a                                     # distance to the upper neighbour
    pick_up = (above < below) | ((above == below) & (i % 2 == 1))
    res = np.where(pick_up & ~top, j, i)
    return res.astype(np.int64)


def e2m1_encode(r) -> np.ndarray:
    """FP4 E2M1 code of a value already divided by its group scale.

    Bit 3 is the sign of r (signbit, so -0.0 and small negatives give 8); bits
    0..2 index the nearest level, ties to the even code; |r| > 6 saturates to 6.
    """
    r = np.asarray(r, dtype=np.float64)
    mag = _nearest_even(np.abs(r), E2M1_LEVELS)
    return (mag | (np.signbit(r).astype(np.int64) << 3)).astype(np.uint8)


def e2m1_decode(code) -> np.ndarray:
    code = np.asarray(code, dtype=np.int64)
    mag = E2M1_LEVELS[code & 7]
    return np.where(code & 8, -mag, mag)


def quantize_fp4(x, scale_mode="absmax", c=CONSTOPT_C):
    """Quantize rotated rows x[..., d] per 32-channel group; the scale exponent is
    R3's (``scale_mode="absmax"``) or R9's (``"constopt"``, constant c).

    Returns (codes [..., d] uint8 in 0..15, scale bytes [..., d/32] uint8).
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    g = x.reshape(x.shape[:-1] + (d // GROUP, GROUP))
    m = np.max(np.abs(g), axis=-1)                    # group absmax
    if scale_mode == "absmax":
        e = scale_exponent(m)
    elif scale_mode == "constopt":
        e = scale_exponent_constopt(m, c)
    else:
        raise ValueError(scale_mode)
    r = np.ldexp(g, -e[..., None])                    # exact division by 2**E
    codes = e2m1_encode(r).reshape(x.shape)
    return codes, (e + 127).astype(np.uint8)


def dequantize_fp4(codes, scale_bytes) -> np.ndarray:
    """value = code * 2**(byte - 127) ([review] §3.2; [commentary] footnote 2)."""
    codes = np.asarray(codes)
    d = codes.shape[-1]
    v = e2m1_decode(codes).reshape(codes.shape[:-1] + (d // GROUP, GROUP))
    e = np.asarray(scale_bytes, dtype=np.int64) - 127
    return np.ldexp(v, e[..., None]).reshape(codes.shape)


def pack_nibbles(codes) -> np.ndarray:
    """Two codes per byte: element 2j in the low nibble, 2j+1 in the high nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = b & 15
    out[..., 1::2] = b >> 4
    return out


# --------------------------------------------------------------------------
# FP8 E4M3 (OCP) for the query ([review] §3.2, §4.2) and the FP8 baseline; R6
# --------------------------------------------------------------------------
def e4m3_decode(b) -> np.ndarray:
    """OCP E4M3: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0 is
    subnormal (m/8 * 2**-6); S.1111.111 is NaN; no infinities."""
    b = np.asarray(b, dtype=np.int64)
    s = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 15
    m = (b & 7).astype(np.float64)
    val = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    val = np.where((e == 15) & ((b & 7) == 7), np.nan, val)
    return s * val


_E4M3_POS = e4m3_decode(np.arange(0x7F))      # codes 0x00..0x7E, increasing, max 448


def e4m3_encode(v) -> np.ndarray:
    """Round float64 to OCP E4M3: nearest, ties to even code, |v| > 448 saturates
    to 448 (0x7E / 0xFE), sign bit copied (so -0.0 gives 0x80).  Inputs are finite."""
    v = np.asarray(v, dtype=np.float64)
    mag = _nearest_even(np.abs(v), _E4M3_POS)
    return (mag | (np.signbit(v).astype(np.int64) << 7)).astype(np.uint8)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) to float64, exactly."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def f32_to_f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def bf16_round_bits(x32) -> np.ndarray:
    """float32 values to bf16 bits, round to nearest, ties to even (finite inputs):
    choose the nearer of the two bf16 neighbours of x."""
    x = np.asarray(x32, dtype=np.float32)
    u = x.view(np.uint32)
    lo_bits = (u >> 16).astype(np.uint32)                     # truncation toward zero
    lo = bf16_bits_to_f64(lo_bits.astype(np.uint16))
    hi = bf16_bits_to_f64((lo_bits + 1).astype(np.uint16))    # next bf16 away from zero
    a = np.abs(x.astype(np.float64))
    d_lo, d_hi = a - np.abs(lo), np.abs(hi) - a
    up = (d_hi < d_lo) | ((d_hi == d_lo) & (lo_bits & 1 == 1))
    return np.where(up, lo_bits + 1, lo_bits).astype(np.uint16)


# --------------------------------------------------------------------------
# Paged cache layout (reading R8).  Pools are uint8 [num_pages][H_kv][block]:
# a page is H_kv blocks back to back, 17 bytes per 32 elements for FP4, with no
# padding.  The order of bytes inside a page is not fixed by the pages; the
# layout below serves the decode's operand loads, and the FP4 block positions
# and the FP8 page bytes rotate with the page id, so that blocks start at
# different offsets from page to page.
#   FP4: KV head h's block at position (h + 2 page) mod H_kv of page `page`
#   FP4 K block: codes[16 tok][d/2] (token-major) then scales[tok % 4][d/32][tok // 4]
#   FP4 V block: codes[d/2 rows][16 tok] (channel pair c in row 16*(c % (d/32)) + c // (d/32))
#                then scales[d/32 groups][16 tok]
#   FP8 K block: [16 tok][d] bytes;  FP8 V block: [d][16 tok] bytes; the FP8 page
#                (blocks back to back) rotated by 256 * page bytes, fp8_page_offset
#   BF16 K block: [16 tok][d] bf16;  BF16 V block: [d][16 tok] bf16 (little endian)
# --------------------------------------------------------------------------
def head_block_bytes(fmt: int, d: int) -> int:
    if fmt == FMT_FP4:
        return PAGE_SIZE * (d // 2) + PAGE_SIZE * (d // GROUP)   # 17 bytes per 32 elements
    if fmt == FMT_FP8:
        return PAGE_SIZE * d
    if fmt == FMT_BF16:
        return PAGE_SIZE * d * 2
    raise ValueError(fmt)


def page_bytes(fmt: int, num_kv_heads: int, d: int) -> int:
    return num_kv_heads * head_block_bytes(fmt, d)


def new_pool(fmt: int, num_pages: int, num_kv_heads: int, d: int) -> np.ndarray:
    return np.zeros((num_pages, num_kv_heads, head_block_bytes(fmt, d)), dtype=np.uint8)


def fp4_block_position(head, page, num_kv_heads):
    """Position of KV head `head`'s block inside page `page` of an FP4 pool:
    (head + 2 * page) mod H_kv.  For an even H_kv the two heads of a pair stay
    adjacent and pair p sits at pair position (p + page) mod (H_kv / 2), so the
    pairs' blocks start at different offsets from page to page (reading R8)."""
    H = int(num_kv_heads)
    return (np.asarray(head, np.int64) + 2 * (np.asarray(page, np.int64) % H)) % H


def fp4_k_code_offset(tok, byte, d):
    return tok * (d // 2) + byte


def fp4_k_scale_offset(tok, group, d):
    # scale bytes ordered [slot % 4][group][slot // 4]
    return PAGE_SIZE * (d // 2) + ((tok % 4) * (d // GROUP) + group) * 4 + tok // 4


def fp4_v_code_offset(tok, pair, d):
    # 16-byte rows (one per channel pair, byte = slot); channel pair c sits in
    # row 16 * (c % (d/32)) + c // (d/32)
    cpl = d // GROUP
    return ((pair % cpl) * 16 + pair // cpl) * PAGE_SIZE + tok


def fp4_v_scale_offset(tok, group, d):
    return PAGE_SIZE * (d // 2) + group * PAGE_SIZE + tok


def fp8_k_offset(tok, ch, d):
    return tok * d + ch


def fp8_v_offset(tok, ch, d):
    return ch * PAGE_SIZE + tok


def fp8_page_offset(head, offset, page, num_kv_heads, d):
    """Byte of an FP8 page holding byte `offset` of KV head `head`'s block: the
    page is its blocks back to back, rotated by 256 * page bytes (mod the page
    size) -- byte b of the unrotated page sits at (b + 256 page) mod page_bytes,
    so every byte keeps the address modulo 16 KB that a page stride of 16 KB +
    256 would give it (reading R8)."""
    pb = num_kv_heads * head_block_bytes(FMT_FP8, d)
    units = pb // 256
    b = np.asarray(head, np.int64) * head_block_bytes(FMT_FP8, d) + np.asarray(offset, np.int64)
    return (b + 256 * (np.asarray(page, np.int64) % units)) % pb


def bf16_k_index(tok, ch, d):      # index into the block viewed as uint16
    return tok * d + ch


def bf16_v_index(tok, ch, d):
    return ch * PAGE_SIZE + tok


def append(fmt, k_pool, v_pool, k_new, v_new, slot_mapping, in_dtype="bf16", scale_mode="absmax",
           k_only=False, signs=None):
    """Write new tokens into the paged pools in place.

    k_new, v_new: [T][H_kv][d] as bf16 bits (uint16, in_dtype "bf16") or float32
    (in_dtype "f32").  slot_mapping[t] = page * 16 + offset; a negative slot skips
    the token.  FP4 rotates and quantizes ([review] §3.1; ``scale_mode`` as in
    ``quantize_fp4``, constOpt with c = 0.156; ``k_only`` leaves V unrotated, R11;
    ``signs`` makes the rotation R12's); FP8 rounds each value to E4M3 with
    scale 1; BF16 stores the value (float32 input rounded to bf16).
    """
    if fmt != FMT_FP4 and (k_only or signs is not None):
        raise ValueError("rotation variants apply to the FP4 cache only")
    k_new = np.asarray(k_new)
    T, H, d = k_new.shape
    to64 = bf16_bits_to_f64 if in_dtype == "bf16" else f32_to_f64
    slots = np.asarray(slot_mapping, dtype=np.int64)
    keep = np.nonzero(slots >= 0)[0]
    page, off = slots[keep] // PAGE_SIZE, slots[keep] % PAGE_SIZE
    for pool, src, is_v in ((k_pool, k_new, False), (v_pool, np.asarray(v_new), True)):
        flat = pool.reshape(pool.shape[0], H, -1)
        x = to64(src[keep])                                   # [n][H][d] exact
        if fmt == FMT_FP4:
            y = x + 0.0 if (is_v and k_only) else rotate(x, signs)
            codes, sbytes = quantize_fp4(y, scale_mode)       # [n][H][d], [n][H][d/32]
            packed = pack_nibbles(codes)                      # [n][H][d/2]
            j = np.arange(d // 2)
            g = np.arange(d // GROUP)
            for h in range(H):
                pos = fp4_block_position(h, page, H)[:, None]
                if is_v:
                    flat[page[:, None], pos, fp4_v_code_offset(off[:, None], j[None, :], d)] = packed[:, h]
                    flat[page[:, None], pos, fp4_v_scale_offset(off[:, None], g[None, :], d)] = sbytes[:, h]
                else:
                    flat[page[:, None], pos, fp4_k_code_offset(off[:, None], j[None, :], d)] = packed[:, h]
                    flat[page[:, None], pos, fp4_k_scale_offset(off[:, None], g[None, :], d)] = sbytes[:, h]
        elif fmt == FMT_FP8:
            b = e4m3_encode(x)
            c = np.arange(d)
            fn = fp8_v_offset if is_v else fp8_k_offset
            flat_p = pool.reshape(pool.shape[0], -1)
            for h in range(H):
                pos = fp8_page_offset(h, fn(off[:, None], c[None, :], d), page[:, None], H, d)
                flat_p[page[:, None], pos] = b[:, h]
        elif fmt == FMT_BF16:
            bits = src[keep].astype(np.uint16) if in_dtype == "bf16" else bf16_round_bits(src[keep])
            c = np.arange(d)
            fn = bf16_v_index if is_v else bf16_k_index
            f16 = flat.view(np.uint16)
            for h in range(H):
                f16[page[:, None], h, fn(off[:, None], c[None, :], d)] = bits[:, h]
        else:
            raise ValueError(fmt)


def gather_fp4_codes(pool, page_row, seq_len, head, d, is_v):
    """FP4 codes [seq_len][d] (0..15) and scale bytes [seq_len][d/32] of one KV
    head of one sequence: token t lives in page page_row[t // 16] at offset t % 16."""
    t = np.arange(seq_len)
    page = np.asarray(page_row, dtype=np.int64)[t // PAGE_SIZE][:, None]
    off = (t % PAGE_SIZE)[:, None]
    H = pool.shape[1]
    flat = pool.reshape(pool.shape[0], H, -1)
    j = np.arange(d // 2)[None, :]
    g = np.arange(d // GROUP)[None, :]
    pos = fp4_block_position(head, page, H)
    if is_v:
        packed = flat[page, pos, fp4_v_code_offset(off, j, d)]
        sb = flat[page, pos, fp4_v_scale_offset(off, g, d)]
    else:
        packed = flat[page, pos, fp4_k_code_offset(off, j, d)]
        sb = flat[page, pos, fp4_k_scale_offset(off, g, d)]
    return unpack_nibbles(packed), sb


def gather_dequant(fmt, pool, page_row, seq_len, head, d, is_v) -> np.ndarray:
    """Dequantized [seq_len][d] rows of one KV head of one sequence: token t lives
    in page page_row[t // 16] at offset t % 16."""
    t = np.arange(seq_len)
    page = np.asarray(page_row, dtype=np.int64)[t // PAGE_SIZE][:, None]
    off = (t % PAGE_SIZE)[:, None]
    H = pool.shape[1]
    flat = pool.reshape(pool.shape[0], H, -1)
    if fmt == FMT_FP4:
        return dequantize_fp4(*gather_fp4_codes(pool, page_row, seq_len, head, d, is_v))
    c = np.arange(d)[None, :]
    if fmt == FMT_FP8:
        fn = fp8_v_offset if is_v else fp8_k_offset
        flat_p = pool.reshape(pool.shape[0], -1)
        return e4m3_decode(flat_p[page, fp8_page_offset(head, fn(off, c, d), page, H, d)])
    if fmt == FMT_BF16:
        fn = bf16_v_index if is_v else bf16_k_index
        return bf16_bits_to_f64(flat.view(np.uint16)[page, head, fn(off, c, d)])
    raise ValueError(fmt)


def rotate_quantize_query(q, in_dtype="bf16", signs=None) -> np.ndarray:
    """E4M3 bytes of the rotated query ([review] §3.2: the query is rotated into the
    key basis and rounded to FP8 E4M3), rounded directly from float64 (R5); with
    ``signs`` the rotation is R12's."""
    to64 = bf16_bits_to_f64 if in_dtype == "bf16" else f32_to_f64
    return e4m3_encode(rotate(to64(q), signs))


def attention(qhat, k, v, sm_scale) -> np.ndarray:
    """softmax(sm_scale * qhat k^T) v in float64 for one KV head: qhat [G][d],
    k, v [L][d] -> [G][d]."""
    s = sm_scale * (qhat @ k.T)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ v


# --------------------------------------------------------------------------
# PV operand precision: the f16 hi + lo probabilities the kernels use, and the
# fully scaled-MFMA alternative ([review] §3.2 and [commentary] footnote 2: FP4
# value codes and UE8M0 scales fed to the scaled matrix instruction).  Models of
# operand rounding only (products summed exactly), for measuring what each
# choice costs against the float64 result.
# --------------------------------------------------------------------------
def _f16(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def pv_f16_hi_lo(p, v) -> np.ndarray:
    """sum_t P[r, t] V[t, c] with P split into f16 hi = f16(p) and lo = f16(p - hi)
    and V as f16 (exact for dequantized FP4 within the f16 range): p [R][T],
    v [T][d] -> [R][d]."""
    p = np.asarray(p, dtype=np.float64)
    hi = _f16(p)
    lo = _f16(p - hi)
    v16 = _f16(v)
    return hi @ v16 + lo @ v16


def fold_p_fp8(p, exps, block=32, headroom=0) -> np.ndarray:
    """The B operand of a scaled-MFMA PV for one 32-channel group: V's per-token
    exponent E_t folded into the probabilities, normalized by M = (the largest E
    of each block of 32 tokens) - ``headroom``, at least -127 (that block's
    UE8M0 operand scale 2^M), and rounded to E4M3.  p [R][T], exps [T] (V's
    group exponents) -> the rounded operand times 2^M, [R][T] (so that
    sum_t result[r, t] * code[t] is the PV)."""
    p = np.asarray(p, dtype=np.float64)
    e = np.asarray(exps, dtype=np.int64)
    T = e.size
    nb = -(-T // block)
    padded = np.full(nb * block, -(1 << 20), dtype=np.int64)          # below every exponent
    padded[:T] = e
    M = np.maximum(padded.reshape(nb, block).max(axis=1) - headroom, -127)
    Mt = np.repeat(M, block)[:T]
    folded = np.ldexp(p, (e - Mt)[None, :])
    return np.ldexp(e4m3_decode(e4m3_encode(folded)), Mt[None, :])


def pv_fp8_scaled(p, codes, scale_bytes, headroom=0) -> np.ndarray:
    """sum_t P[r, t] V[t, c] computed as the scaled-MFMA PV would: FP4 codes as the
    A operand (scale 1), and per 32-channel group g the probabilities folded with
    V's exponents of that group (``fold_p_fp8``) as the FP8 B operand.
    p [R][T], codes [T][d] (0..15), scale_bytes [T][d/32] -> [R][d]."""
    codes = np.asarray(codes)
    T, d = codes.shape
    vals = e2m1_decode(codes)
    e = np.asarray(scale_bytes, dtype=np.int64) - 127
    out = np.zeros((np.asarray(p).shape[0], d))
    for g in range(d // GROUP):
        cs = slice(GROUP * g, GROUP * (g + 1))
        out[:, cs] = fold_p_fp8(p, e[:, g], headroom=headroom) @ vals[:, cs]
    return out


# The decode with the scaled-MFMA PV (reading R13): softmax steps of SPV_STEP
# tokens at positions SPV_STEP * s .. of the sequence; the largest folded
# probability is 2^SPV_HEADROOM (E4M3 reaches 448).
SPV_STEP = 128
SPV_HEADROOM = 8


def attention_pv_scaled(qhat, k, v_codes, v_scale_bytes, sm_scale, step=SPV_STEP, fold=True) -> np.ndarray:
    """softmax(sm_scale * qhat k^T) V for one KV head with the PV of each step of
    ``step`` tokens on the scaled FP8 x FP4 product (R13): within the step the
    probabilities are taken against the step's own largest logit of each row, so
    that each is at most 1; per 32-channel group and 32-token block they are
    folded with V's exponents (headroom SPV_HEADROOM) and rounded to E4M3, and
    multiplied by V's FP4 codes.  The steps' products and their unrounded
    probability sums are then combined, each weighted by exp(its maximum minus
    the overall maximum), and the output is their quotient.  ``fold=False``
    takes the exact product instead (no rounding), which makes the result the
    plain softmax attention.  qhat [G][d], k [L][d], v_codes [L][d] (0..15),
    v_scale_bytes [L][d/32] -> [G][d]."""
    if fold and step % GROUP:
        raise ValueError("the 32-token blocks of the fold must tile the steps")
    s = sm_scale * (np.asarray(qhat, dtype=np.float64) @ np.asarray(k, dtype=np.float64).T)   # [G][L]
    G, L = s.shape
    codes = np.asarray(v_codes)
    d = codes.shape[1]
    nS = -(-L // step)
    sp = np.full((G, nS * step), -np.inf)
    sp[:, :L] = s
    ms = sp.reshape(G, nS, step).max(axis=2)                          # [G][steps], each step has a token
    p = np.exp(sp - np.repeat(ms, step, axis=1))                       # 0 past the sequence
    if fold:
        vals = e2m1_decode(codes)
        e = np.asarray(v_scale_bytes, dtype=np.int64) - 127
        ops = [fold_p_fp8(p[:, :L], e[:, g], headroom=SPV_HEADROOM) for g in range(d // GROUP)]
    else:
        vals = dequantize_fp4(codes, v_scale_bytes)
        ops = [p[:, :L]] * (d // GROUP)
    vp = np.zeros((nS * step, d))
    vp[:L] = vals
    vp = vp.reshape(nS, step, d)
    ostep = np.zeros((G, nS, d))                                       # each step's product
    for g, op in enumerate(ops):
        cs = slice(GROUP * g, GROUP * (g + 1))
        opp = np.zeros((G, nS * step))
        opp[:, :L] = op
        ostep[:, :, cs] = np.einsum("gst,stc->gsc", opp.reshape(G, nS, step), vp[:, :, cs])
    lstep = p.reshape(G, nS, step).sum(axis=2)
    w = np.exp(ms - ms.max(axis=1, keepdims=True))                     # exp(m_s - m)
    o = np.einsum("gs,gsc->gc", w, ostep)
    l = (w * lstep).sum(axis=1)
    return o / l[:, None]


def decode_attention_rows(fmt, k_pool, v_pool, num_kv_heads, d, q, page_table, seq_lens,
                          sm_scale, rows, in_dtype="bf16", k_only=False, signs=None, pv_scaled=False) -> np.ndarray:
    """Output rows for the (sequence, query head) pairs in ``rows`` ([n][2]).

    FP4: q rotated and rounded to E4M3, output rotated back with the transpose of
    the rotation (R2's normalized WHT is its own inverse); with ``k_only`` (R11)
    the output stays as attended, V being unrotated; ``signs`` as in R12;
    ``pv_scaled`` takes the scaled-MFMA PV of R13 (``attention_pv_scaled``).
    FP8: q rounded to E4M3, no rotation; BF16: q as given.  A sequence of length
    0 gives a zero row.
    """
    if fmt != FMT_FP4 and (k_only or signs is not None or pv_scaled):
        raise ValueError("rotation variants and the scaled PV apply to the FP4 cache only")
    q = np.asarray(q)
    Hq = q.shape[1]
    group = Hq // num_kv_heads
    to64 = bf16_bits_to_f64 if in_dtype == "bf16" else f32_to_f64
    out = np.zeros((len(rows), d))
    cache = {}
    for n, (b, h) in enumerate(rows):
        L = int(seq_lens[b])
        if L == 0:
            continue
        hk = h // group
        key = (b, hk)
        if key not in cache:
            V = (gather_fp4_codes(v_pool, page_table[b], L, hk, d, True) if pv_scaled
                 else gather_dequant(fmt, v_pool, page_table[b], L, hk, d, True))
            cache = {key: (gather_dequant(fmt, k_pool, page_table[b], L, hk, d, False), V)}
        K, V = cache[key]
        if fmt == FMT_FP4:
            qhat = e4m3_decode(rotate_quantize_query(q[b, h], in_dtype, signs))
        elif fmt == FMT_FP8:
            qhat = e4m3_decode(e4m3_encode(to64(q[b, h])))
        else:
            qhat = to64(q[b, h])
        if pv_scaled:
            o = attention_pv_scaled(qhat[None, :], K, V[0], V[1], float(sm_scale))[0]
        else:
            o = attention(qhat[None, :], K, V, float(sm_scale))[0]
        out[n] = unrotate(o, signs) if (fmt == FMT_FP4 and not k_only) else o
    return out


def prefill_attention(fmt, k_pool, v_pool, num_kv_heads, d, q, q_lens, page_table, seq_lens,
                      sm_scale, in_dtype="bf16", k_only=False, signs=None, pv_scaled=False) -> np.ndarray:
    """Causal attention of chunks of query tokens over the cache ([review] §1 and
    §5.4: a new turn's tokens read the resident prefix instead of re-prefilling
    it; reading R10).  q [T_q][H_q][d] holds sequence 0's chunk, then sequence
    1's, ...; the row of chunk token j of sequence b is the decode of that row
    over positions 0 .. seq_lens[b] - q_lens[b] + j.  Returns [T_q][H_q][d]."""
    q = np.asarray(q)
    q_lens = np.asarray(q_lens, dtype=np.int64)
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    b_of = np.repeat(np.arange(q_lens.size), q_lens)                   # sequence of each query token
    j_of = np.arange(q.shape[0]) - np.repeat(np.cumsum(q_lens) - q_lens, q_lens)
    prefix = seq_lens[b_of] - q_lens[b_of] + j_of + 1                  # positions 0 .. P
    table = np.asarray(page_table)[b_of]
    return decode_attention(fmt, k_pool, v_pool, num_kv_heads, d, q, table, prefix, sm_scale, in_dtype,
                            k_only, signs, pv_scaled)


def decode_attention(fmt, k_pool, v_pool, num_kv_heads, d, q, page_table, seq_lens,
                     sm_scale, in_dtype="bf16", k_only=False, signs=None, pv_scaled=False) -> np.ndarray:
    """All output rows [B][H_q][d] (float64)."""
    q = np.asarray(q)
    B, Hq = q.shape[0], q.shape[1]
    rows = [(b, h) for b in range(B) for h in range(Hq)]
    out = decode_attention_rows(fmt, k_pool, v_pool, num_kv_heads, d, q, page_table,
                                seq_lens, sm_scale, rows, in_dtype, k_only, signs, pv_scaled)
    return out.reshape(B, Hq, d)
