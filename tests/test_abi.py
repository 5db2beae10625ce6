"""CPU checks of the C ABI: the library loads, exports every symbol that
include/uq.h declares, and its host-side validation returns the documented
status before touching the GPU (no compute call is made here)."""
import ctypes
import os
import re

import numpy as np
import pytest

import bit_kv_cache_wht_amd as uq
from bit_kv_cache_wht_amd import _binding as B
import oracle as O

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "uq.h")
FAKE = 0x10000          # non-null placeholder; validation fails before any use


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(uq_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) == 19, names
    h = uq.lib()
    for n in names:
        assert hasattr(h, n), n
    assert set(names) == set(B._SIGS)


def cache(fmt=B.UQ_KV_FP4, pages=4, heads=2, d=128, page_size=16, k=FAKE, v=FAKE, rot=0, signs=(0, 0, 0, 0)):
    return B._Cache(fmt, pages, page_size, heads, d, k, v, rot, (ctypes.c_uint32 * 4)(*signs))


def test_cache_struct_layout():
    # uq_kv_cache: five int32, two pointers, the rotation word, four sign words
    assert ctypes.sizeof(B._Cache) == 64
    assert B._Cache.rotation.offset == 40 and B._Cache.rotation_signs.offset == 44


def _rotation_cases(fmt, d):
    """(cache, expected status of a call that would otherwise succeed)."""
    out = [(cache(fmt, d=d, rot=4), B.UQ_ERR_INVALID_ARG),                         # unknown bit
           (cache(fmt, d=d, signs=(1, 0, 0, 0)), B.UQ_ERR_INVALID_ARG)]            # signs without UQ_ROT_SIGNS
    if fmt == B.UQ_KV_FP4:
        out += [(cache(fmt, d=d, rot=B.UQ_ROT_K_ONLY), B.UQ_OK),
                (cache(fmt, d=d, rot=B.UQ_ROT_SIGNS, signs=(0xFFFFFFFF, 1, 0, 0)), B.UQ_OK),
                (cache(fmt, d=d, rot=3, signs=(0, 0x80000000, 0, 0)), B.UQ_OK),
                (cache(fmt, d=d, rot=B.UQ_ROT_SIGNS, signs=(0, 0, 1 if d == 64 else 0, 1 if d == 64 else 0)),
                 B.UQ_ERR_INVALID_ARG if d == 64 else B.UQ_OK)]                    # bits at or above head_dim
    else:
        out += [(cache(fmt, d=d, rot=B.UQ_ROT_K_ONLY), B.UQ_ERR_INVALID_ARG),       # FP4 caches only
                (cache(fmt, d=d, rot=B.UQ_ROT_SIGNS, signs=(1, 0, 0, 0)), B.UQ_ERR_INVALID_ARG)]
    return out


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("name,fmt", [("uq_quantize_append", 0), ("uq_append_fp8", 1), ("uq_append_bf16", 2)])
def test_rotation_variant_validation(name, fmt, d):
    f = getattr(uq.lib(), name)
    for c, want in _rotation_cases(fmt, d):
        # an empty append reaches the end of validation without a launch
        assert f(ctypes.byref(c), None, None, 0, None, 0, 0, None) == want, (c.rotation, list(c.rotation_signs))
    dec = {0: uq.lib().uq_decode_attention, 1: uq.lib().uq_decode_attention_fp8,
           2: uq.lib().uq_decode_attention_bf16}[fmt]
    for c, want in _rotation_cases(fmt, d):
        assert dec(ctypes.byref(c), None, 0, None, 8, None, 0, 16, 0.1, None, None, 0, 0, None) == want
    if fmt == 0:
        pf = uq.lib().uq_prefill_attention
        for c, want in _rotation_cases(fmt, d):
            assert pf(ctypes.byref(c), None, 0, None, 0, None, 8, None, 3, 16, 0.1, None, 0, None) == want


def test_sign_words_packing():
    s = np.ones(128)
    s[[0, 31, 32, 127]] = -1
    assert uq.sign_words(s, 128) == (0x80000001, 1, 0, 0x80000000)
    assert uq.sign_words(np.ones(64), 64) == (0, 0, 0, 0)
    with pytest.raises(ValueError):
        uq.sign_words(np.ones(64), 128)
    with pytest.raises(ValueError):
        uq.sign_words(np.zeros(64), 64)


@pytest.mark.parametrize("fmt", [0, 1, 2])
@pytest.mark.parametrize("d", [64, 128])
def test_block_sizes_match_oracle_layout(fmt, d):
    assert uq.uq_head_block_bytes(fmt, d) == O.head_block_bytes(fmt, d)
    for heads in (1, 3, 4, 8):
        c = cache(fmt, heads=heads, d=d)
        # a page is its head blocks back to back, nothing more
        assert uq.lib().uq_page_bytes(ctypes.byref(c)) == O.page_bytes(fmt, heads, d) == heads * O.head_block_bytes(fmt, d)


def test_page_bytes_at_the_benchmark_shapes():
    # FP4: exactly 17/32 bytes per element (4.25 bits: [commentary] footnote 2;
    # [review] §3.1 table "Stored footprint"); FP8 one byte; BF16 two.
    for heads in (8, 4):
        c = cache(B.UQ_KV_FP4, heads=heads, d=128)
        assert uq.lib().uq_page_bytes(ctypes.byref(c)) == heads * 16 * (64 + 4) == heads * 16 * 128 * 17 // 32
        assert uq.lib().uq_page_bytes(ctypes.byref(cache(B.UQ_KV_FP8, heads=heads, d=128))) == heads * 16 * 128
        assert uq.lib().uq_page_bytes(ctypes.byref(cache(B.UQ_KV_BF16, heads=heads, d=128))) == heads * 16 * 128 * 2
    c = cache(B.UQ_KV_FP4, heads=8, d=128)
    assert uq.lib().uq_page_bytes(ctypes.byref(c)) == 8704


def test_block_sizes_invalid():
    assert uq.uq_head_block_bytes(0, 96) == 0
    assert uq.uq_head_block_bytes(7, 128) == 0
    c = cache(page_size=32)
    assert uq.lib().uq_page_bytes(ctypes.byref(c)) == 0
    assert uq.lib().uq_page_bytes(None) == 0


APPENDS = [("uq_quantize_append", B.UQ_KV_FP4), ("uq_append_fp8", B.UQ_KV_FP8), ("uq_append_bf16", B.UQ_KV_BF16)]


@pytest.mark.parametrize("name,fmt", APPENDS)
def test_append_validation(name, fmt):
    f = getattr(uq.lib(), name)
    ok = cache(fmt)
    call = lambda c=ok, k=FAKE, v=FAKE, dt=0, s=FAKE, n=4, fl=0: f(ctypes.byref(c) if c is not None else None,
                                                                    k, v, dt, s, n, fl, None)
    assert call(c=None) == B.UQ_ERR_INVALID_ARG
    other = (fmt + 1) % 3
    assert call(c=cache(other)) == B.UQ_ERR_INVALID_ARG          # format mismatch
    assert call(c=cache(fmt, page_size=8)) == B.UQ_ERR_UNSUPPORTED
    assert call(c=cache(fmt, d=96)) == B.UQ_ERR_UNSUPPORTED
    assert call(c=cache(fmt, heads=0)) == B.UQ_ERR_INVALID_ARG
    assert call(c=cache(fmt, k=None)) == B.UQ_ERR_INVALID_ARG
    assert call(k=None) == B.UQ_ERR_INVALID_ARG
    assert call(v=None) == B.UQ_ERR_INVALID_ARG
    assert call(s=None) == B.UQ_ERR_INVALID_ARG
    assert call(dt=5) == B.UQ_ERR_INVALID_ARG
    assert call(n=-1) == B.UQ_ERR_INVALID_ARG
    assert call(fl=1) == B.UQ_ERR_INVALID_ARG
    assert call(fl=4) == B.UQ_ERR_INVALID_ARG
    if fmt == B.UQ_KV_FP4:                                          # constOpt accepted for FP4 writes only
        assert call(fl=B.UQ_FLAG_SCALE_CONSTOPT, k=None) == B.UQ_ERR_INVALID_ARG
        assert call(fl=B.UQ_FLAG_SCALE_CONSTOPT, n=0, k=None, v=None, s=None) == B.UQ_OK
    else:
        assert call(fl=B.UQ_FLAG_SCALE_CONSTOPT, n=0, k=None, v=None, s=None) == B.UQ_ERR_INVALID_ARG
    assert call(n=0, k=None, v=None, s=None) == B.UQ_OK            # empty append is a no-op
    # 2 T H rows are indexed in 32 bits
    assert call(c=cache(fmt, heads=1), n=1 << 30) == B.UQ_ERR_UNSUPPORTED
    assert call(c=cache(fmt, heads=4), n=(1 << 28) + 1) == B.UQ_ERR_UNSUPPORTED


def test_query_validation():
    f = uq.lib().uq_rotate_quantize_query
    assert f(FAKE, 3, FAKE, 4, 128, None) == B.UQ_ERR_INVALID_ARG
    assert f(FAKE, 0, FAKE, 4, 96, None) == B.UQ_ERR_UNSUPPORTED
    assert f(None, 0, FAKE, 4, 128, None) == B.UQ_ERR_INVALID_ARG
    assert f(FAKE, 0, None, 4, 128, None) == B.UQ_ERR_INVALID_ARG
    assert f(FAKE, 0, FAKE, -1, 128, None) == B.UQ_ERR_INVALID_ARG
    assert f(None, 0, None, 0, 128, None) == B.UQ_OK


DECODES = [("uq_decode_attention", B.UQ_KV_FP4), ("uq_decode_attention_fp8", B.UQ_KV_FP8),
           ("uq_decode_attention_bf16", B.UQ_KV_BF16)]


@pytest.mark.parametrize("name,fmt", DECODES)
def test_decode_validation(name, fmt):
    f = getattr(uq.lib(), name)
    ok = cache(fmt, heads=2)
    ws = uq.lib().uq_decode_workspace_bytes(ctypes.byref(ok), 3, 16, 8)
    assert ws > 0

    def call(c=ok, q=FAKE, qd=0, pt=FAKE, mp=8, sl=FAKE, B_=3, Hq=16, scale=0.1, out=FAKE, w=FAKE, wb=ws, fl=0):
        return f(ctypes.byref(c) if c is not None else None, q, qd, pt, mp, sl, B_, Hq, scale, out, w, wb, fl, None)

    assert call(c=None) == B.UQ_ERR_INVALID_ARG
    assert call(c=cache((fmt + 1) % 3, heads=2)) == B.UQ_ERR_INVALID_ARG
    assert call(c=cache(fmt, heads=2, d=256)) == B.UQ_ERR_UNSUPPORTED
    assert call(Hq=15) == B.UQ_ERR_UNSUPPORTED                   # H_q % H_kv != 0
    assert call(Hq=34) == B.UQ_ERR_UNSUPPORTED                   # group of 17 > 16
    assert call(B_=-1) == B.UQ_ERR_INVALID_ARG
    assert call(mp=0) == B.UQ_ERR_INVALID_ARG
    assert call(q=None) == B.UQ_ERR_INVALID_ARG
    assert call(pt=None) == B.UQ_ERR_INVALID_ARG
    assert call(sl=None) == B.UQ_ERR_INVALID_ARG
    assert call(out=None) == B.UQ_ERR_INVALID_ARG
    assert call(qd=9) == B.UQ_ERR_INVALID_ARG
    assert call(scale=float("nan")) == B.UQ_ERR_INVALID_ARG
    assert call(scale=0.0) == B.UQ_ERR_INVALID_ARG
    assert call(scale=-0.1) == B.UQ_ERR_INVALID_ARG
    assert call(scale=float("inf")) == B.UQ_ERR_INVALID_ARG
    assert call(w=None) == B.UQ_ERR_WORKSPACE
    assert call(wb=ws - 1) == B.UQ_ERR_WORKSPACE
    assert call(fl=2) == B.UQ_ERR_INVALID_ARG
    assert call(fl=16) == B.UQ_ERR_INVALID_ARG
    assert call(fl=B.UQ_FLAG_CHECK, w=None) == B.UQ_ERR_WORKSPACE                # accepted by every format
    if fmt == B.UQ_KV_FP4:
        assert call(fl=B.UQ_FLAG_OUT_ROTATED, w=None) == B.UQ_ERR_WORKSPACE     # flags accepted
        assert call(fl=B.UQ_FLAG_PV_SCALED, w=None) == B.UQ_ERR_WORKSPACE
    else:
        assert call(fl=B.UQ_FLAG_OUT_ROTATED) == B.UQ_ERR_INVALID_ARG
        assert call(fl=B.UQ_FLAG_PV_SCALED) == B.UQ_ERR_INVALID_ARG
    if fmt == B.UQ_KV_BF16:
        assert call(qd=B.UQ_IN_F32) == B.UQ_ERR_UNSUPPORTED
    assert call(B_=0, q=None, pt=None, sl=None, out=None, w=None) == B.UQ_OK
    # a step's index inside its item is kept in 20 bits: at most 2^21 pages per sequence
    assert call(B_=1, mp=(1 << 21) + 1) == B.UQ_ERR_UNSUPPORTED
    wbig = uq.lib().uq_decode_workspace_bytes(ctypes.byref(ok), 1, 16, 1 << 21)
    assert call(B_=1, mp=1 << 21, w=None, wb=wbig) == B.UQ_ERR_WORKSPACE      # the limit itself passes


def test_fused_step_validation():
    f = uq.lib().uq_append_decode_attention
    ok = cache(B.UQ_KV_FP4, heads=2)
    ws = uq.lib().uq_decode_workspace_bytes(ctypes.byref(ok), 3, 16, 8)

    def call(c=ok, k=FAKE, v=FAKE, q=FAKE, dt=0, pt=FAKE, mp=8, sl=FAKE, B_=3, Hq=16, scale=0.1, out=FAKE, w=FAKE,
             wb=ws, fl=0):
        return f(ctypes.byref(c) if c is not None else None, k, v, q, dt, pt, mp, sl, B_, Hq, scale, out, w, wb, fl,
                 None)

    assert call(c=None) == B.UQ_ERR_INVALID_ARG
    assert call(c=cache(B.UQ_KV_FP8, heads=2)) == B.UQ_ERR_INVALID_ARG    # FP4 caches only
    assert call(k=None) == B.UQ_ERR_INVALID_ARG
    assert call(v=None) == B.UQ_ERR_INVALID_ARG
    assert call(q=None) == B.UQ_ERR_INVALID_ARG
    assert call(dt=4) == B.UQ_ERR_INVALID_ARG
    assert call(Hq=15) == B.UQ_ERR_UNSUPPORTED
    assert call(w=None) == B.UQ_ERR_WORKSPACE
    assert call(fl=16) == B.UQ_ERR_INVALID_ARG
    assert call(fl=B.UQ_FLAG_OUT_ROTATED, w=None) == B.UQ_ERR_WORKSPACE
    assert call(fl=B.UQ_FLAG_PV_SCALED | B.UQ_FLAG_SCALE_CONSTOPT, w=None) == B.UQ_ERR_WORKSPACE
    assert call(fl=B.UQ_FLAG_SCALE_CONSTOPT | B.UQ_FLAG_OUT_ROTATED, w=None) == B.UQ_ERR_WORKSPACE
    assert call(fl=B.UQ_FLAG_CHECK | B.UQ_FLAG_SCALE_CONSTOPT, w=None) == B.UQ_ERR_WORKSPACE
    assert call(B_=0, k=None, v=None, q=None, pt=None, sl=None, out=None, w=None) == B.UQ_OK


def test_noalloc_decode_validation():
    # every argument check runs before the static scratch array is set up, so
    # none of these reaches the device
    f = uq.lib().uq_decode_attention_noalloc
    ok = cache(B.UQ_KV_FP4, heads=2)

    def call(c=ok, q=FAKE, qd=0, pt=FAKE, mp=8, sl=FAKE, B_=3, Hq=16, scale=0.1, out=FAKE, fl=0):
        return f(ctypes.byref(c) if c is not None else None, q, qd, pt, mp, sl, B_, Hq, scale, out, fl, None)

    assert call(c=None) == B.UQ_ERR_INVALID_ARG
    assert call(c=cache(B.UQ_KV_FP8, heads=2)) == B.UQ_ERR_INVALID_ARG       # FP4 caches only
    assert call(Hq=15) == B.UQ_ERR_UNSUPPORTED
    assert call(q=None) == B.UQ_ERR_INVALID_ARG
    assert call(scale=0.0) == B.UQ_ERR_INVALID_ARG
    assert call(fl=2) == B.UQ_ERR_INVALID_ARG
    assert call(fl=B.UQ_FLAG_CHECK) == B.UQ_ERR_INVALID_ARG      # its error word would be in the hidden scratch
    assert call(fl=B.UQ_FLAG_PV_SCALED, Hq=15) == B.UQ_ERR_UNSUPPORTED   # the flag passes, the shape does not
    assert call(mp=(1 << 21) + 1, B_=1) == B.UQ_ERR_UNSUPPORTED
    # more (sequence, KV head) items than the static array's 65,536 counters
    assert call(c=cache(B.UQ_KV_FP4, heads=9), B_=8000, Hq=9) == B.UQ_ERR_WORKSPACE
    assert call(B_=0, q=None, pt=None, sl=None, out=None) == B.UQ_OK


def test_workspace_bytes_grow_with_shape():
    c = cache(B.UQ_KV_FP4, heads=8)
    w1 = uq.lib().uq_decode_workspace_bytes(ctypes.byref(c), 64, 64, 512)
    w2 = uq.lib().uq_decode_workspace_bytes(ctypes.byref(c), 128, 64, 512)
    assert 0 < w1 < w2 and w1 % 256 == 0
    assert uq.lib().uq_decode_workspace_bytes(None, 1, 1, 1) == 0
    assert uq.lib().uq_decode_workspace_bytes(ctypes.byref(c), 1, 0, 1) == 0


def test_status_strings():
    for s in (0, -1, -2, -3, -4):
        assert uq.uq_status_string(s) != "unknown status"
    assert uq.uq_status_string(99) == "unknown status"
    assert uq.uq_last_hip_error() == 0


def test_profile_events_validation():
    f = uq.lib().uq_profile_next_decode
    assert f(FAKE, None) == B.UQ_ERR_INVALID_ARG
    assert f(None, FAKE) == B.UQ_ERR_INVALID_ARG
    assert f(None, None) == B.UQ_OK


def test_query_rotation_of_a_cache_validation():
    f = uq.lib().uq_rotate_quantize_query_cache
    ok = cache(B.UQ_KV_FP4, heads=2)
    assert f(None, FAKE, 0, FAKE, 4, None) == B.UQ_ERR_INVALID_ARG
    assert f(ctypes.byref(cache(B.UQ_KV_FP8, heads=2)), FAKE, 0, FAKE, 4, None) == B.UQ_ERR_INVALID_ARG
    assert f(ctypes.byref(ok), FAKE, 7, FAKE, 4, None) == B.UQ_ERR_INVALID_ARG
    assert f(ctypes.byref(ok), FAKE, 0, FAKE, -1, None) == B.UQ_ERR_INVALID_ARG
    assert f(ctypes.byref(ok), None, 0, FAKE, 4, None) == B.UQ_ERR_INVALID_ARG
    assert f(ctypes.byref(ok), None, 0, None, 0, None) == B.UQ_OK       # no rows: no launch


def test_profile_clock_cancel():
    # NULL clocks and no rate wanted: a pending request is cancelled, no device call
    assert uq.lib().uq_profile_next_decode_clock(None, None) == B.UQ_OK


def test_stream_read_validation():
    f = uq.lib().uq_stream_read
    assert f(None, 0, None, None) == B.UQ_OK                  # nothing to read: no launch
    assert f(None, 16, FAKE, None) == B.UQ_ERR_INVALID_ARG
    assert f(FAKE, 16, None, None) == B.UQ_ERR_INVALID_ARG
    assert f(FAKE + 4, 16, FAKE, None) == B.UQ_ERR_INVALID_ARG   # src not 16-byte aligned
    assert f(FAKE, 20, FAKE, None) == B.UQ_ERR_INVALID_ARG       # not a multiple of 16 bytes
    assert f(FAKE, 16, FAKE + 2, None) == B.UQ_ERR_INVALID_ARG   # sink not 4-byte aligned


def test_prefill_validation():
    f = uq.lib().uq_prefill_attention
    ok = cache(B.UQ_KV_FP4, heads=2)

    def call(c=ok, q=FAKE, dt=0, cu=FAKE, tq=10, pt=FAKE, mp=8, sl=FAKE, B_=3, Hq=16, scale=0.1, out=FAKE, fl=0):
        return f(ctypes.byref(c) if c is not None else None, q, dt, cu, tq, pt, mp, sl, B_, Hq, scale, out, fl, None)

    assert call(c=None) == B.UQ_ERR_INVALID_ARG
    assert call(c=cache(B.UQ_KV_FP8, heads=2)) == B.UQ_ERR_INVALID_ARG     # FP4 caches only
    assert call(fl=1) == B.UQ_ERR_INVALID_ARG
    assert call(dt=3) == B.UQ_ERR_INVALID_ARG
    assert call(B_=-1) == B.UQ_ERR_INVALID_ARG
    assert call(tq=-1) == B.UQ_ERR_INVALID_ARG
    assert call(mp=0) == B.UQ_ERR_INVALID_ARG
    assert call(Hq=15) == B.UQ_ERR_UNSUPPORTED                  # not a multiple of the KV heads
    assert call(Hq=2 * 129) == B.UQ_ERR_UNSUPPORTED             # more than 128 query heads per KV head
    assert call(B_=4097) == B.UQ_ERR_UNSUPPORTED
    assert call(scale=0.0) == B.UQ_ERR_INVALID_ARG
    assert call(scale=float("nan")) == B.UQ_ERR_INVALID_ARG
    for name in ("q", "cu", "pt", "sl", "out"):
        assert call(**{name: None}) == B.UQ_ERR_INVALID_ARG
    assert call(tq=0, q=None, cu=None, pt=None, sl=None, out=None) == B.UQ_OK     # nothing to do
    assert call(B_=0, q=None, cu=None, pt=None, sl=None, out=None) == B.UQ_OK
