"""GPU parity: libuq (through its C ABI) against the CPU oracle on the same seeded
inputs.  Cache bytes (FP4 codes, UE8M0 scale bytes, FP8 and BF16 values) and
E4M3 query bytes must be bit-exact; attention outputs must be within relative
L2 1e-3 and max-abs 5e-3 of the oracle's float64 result computed from the
identical quantized cache.
"""
import zlib

import numpy as np
import pytest

import oracle as O
from bit_kv_cache_wht_amd import workloads as W

from gpu_util import (FORMATS, announce, assert_close, dev, gpu_append, gpu_cache, gpu_decode, oracle_append,
                      oracle_decode, pools_np, torch_mod, uq)

pytestmark = pytest.mark.gpu


def _wl(name):
    """Small workloads that still span several 4-page steps and ragged tails."""
    if name == "tiny":
        return W.tiny()
    specs = {
        "edge_lens": dict(batch=4, num_q_heads=64, num_kv_heads=8, head_dim=128, seq_lens=[1, 15, 16, 17]),
        "gqa_ragged": dict(batch=3, num_q_heads=32, num_kv_heads=4, head_dim=128, seq_lens=[300, 1000, 77]),
        "mha_5heads": dict(batch=2, num_q_heads=5, num_kv_heads=5, head_dim=128, seq_lens=[129, 40]),
        "group16_d64": dict(batch=2, num_q_heads=16, num_kv_heads=1, head_dim=64, seq_lens=[200, 33]),
        "empty_seqs": dict(batch=5, num_q_heads=8, num_kv_heads=2, head_dim=128, seq_lens=[0, 5, 0, 64, 65]),
        "one_long": dict(batch=1, num_q_heads=8, num_kv_heads=1, head_dim=128, seq_lens=[5000]),
        "d64_bf16": dict(batch=3, num_q_heads=12, num_kv_heads=3, head_dim=64, seq_lens=[90, 64, 250]),
        # enough steps that every wave of every workgroup takes several, crossing
        # item boundaries inside a workgroup's share
        "multi_step": dict(batch=8, num_q_heads=64, num_kv_heads=8, head_dim=128, seq_lens=[2048] * 8),
        # mixed lengths: shares cut items between workgroups after several steps each
        "multi_ragged": dict(batch=6, num_q_heads=32, num_kv_heads=4, head_dim=128,
                             seq_lens=[3000, 1500, 7000, 64, 2500, 5000]),
    }
    s = specs[name]
    return W.make_workload(name, s["batch"], s["num_q_heads"], s["num_kv_heads"], s["head_dim"], s["seq_lens"],
                           s["seq_lens"], seed=zlib.crc32(name.encode()) % 1000 + 7)


SMALL = ["tiny", "edge_lens", "gqa_ragged", "mha_5heads", "group16_d64", "empty_seqs", "one_long", "d64_bf16",
         "multi_step", "multi_ragged"]


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("name", SMALL)
def test_append_bit_exact(fmt, name):
    wl = _wl(name)
    announce(f"append {fmt} {name} T={wl.total_tokens} H={wl.num_kv_heads} d={wl.head_dim}")
    got = pools_np(gpu_append(fmt, wl))
    want = oracle_append(fmt, wl)
    for g, w, kv in zip(got, want, "KV"):
        bad = np.nonzero(g != w)
        assert bad[0].size == 0, f"{kv} pool: {bad[0].size} bytes differ, first at {[int(x[0]) for x in bad]}"


def _edge_rows(d, rng):
    """float32 K/V rows that reach every rounding regime of the FP4 write: group
    scales from 2^-127 to 2^127 (including the ends the float32 hardware
    rounding does not cover), float32 subnormal inputs, zero and negative-zero
    groups, and rows whose rotated values sit within float32 rounding of E2M1
    decision points (the inverse rotation of grid midpoints, rounded to
    float32; for d = 64, c_d = 1/8 and some land exactly on them).

    The scaled rows draw their magnitudes within 2^13 of each other, so they
    lie inside the exact-sum domain stated in uq.h; the near-tie rows fall on
    either side of it.  Returns (inside, outside), split by the oracle's
    criterion."""
    from scipy.linalg import hadamard
    Hn = hadamard(d).astype(np.float64) / np.sqrt(d)
    rows = []
    for k in (-149, -140, -130, -125, -120, -110, -102, -101, -100, -99, -60, 0, 60, 99, 100, 101, 102, 110, 120, 125):
        mag = (1.0 + rng.random(d)) * 2.0 ** (k + rng.integers(-12, 1, d))
        rows.append(mag * rng.choice([-1.0, 1.0], d))
    z = np.zeros(d); z[: d // 2] = -0.0; rows.append(z)
    z = rng.choice([-1.0, 1.0], d) * (1.0 + rng.random(d)); z[32:64] = 0.0; rows.append(z)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0])
    for e in (-90, -30, -3, 0, 7, 40, 95):
        for _ in range(3):
            y = rng.choice(mids, d) * rng.choice([-1.0, 1.0], d) * 2.0 ** e
            y[::32] = 6.0 * 2.0 ** e                       # fixes each group's scale at e
            rows.append(Hn @ y)
    x = np.clip(np.array(rows, dtype=np.float64), -3.0e38, 3.0e38).astype(np.float32)
    inside = O.exact_sum_rows(x.astype(np.float64))
    return x[inside], x[~inside]


def _append_rows(d, xs, many, name):
    """FP4-appends the rows (as K, and reversed and negated as V; `many` repeats
    them past the small-batch threshold so that the large-batch kernel runs
    too); returns the workload and the GPU pools."""
    H = 2
    xs = np.tile(xs, (1600 if many else 1, 1))
    T = xs.shape[0] // H
    wl = W.make_workload(name, 1, H, H, d, [T], [T], in_dtype="f32", seed=9)
    wl.k = np.ascontiguousarray(xs[: T * H].reshape(T, H, d))
    wl.v = np.ascontiguousarray(-xs[::-1][: T * H].reshape(T, H, d))
    announce(f"append fp4 {name} d={d} T={T} H={H}")
    return wl, pools_np(gpu_append("fp4", wl))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("many", [False, True])
def test_append_extreme_scales_and_near_ties(d, many):
    rng = np.random.default_rng(d + (7 if many else 0))
    inside, _ = _edge_rows(d, rng)
    assert inside.shape[0] >= 30
    wl, got = _append_rows(d, inside, many, "extreme")
    want = oracle_append("fp4", wl)
    for g, w, kv in zip(got, want, "KV"):
        bad = np.nonzero(g != w)
        assert bad[0].size == 0, f"{kv} pool: {bad[0].size} bytes differ, first at {[int(x[0]) for x in bad]}"


def _stated_bound(x, d):
    """uq.h's bound on how far a rotated value may be from the exact one outside
    the exact-sum domain, per float32 row: (log2(d) + 2) 2^-53 c_d sum |x_i|."""
    return (np.log2(d) + 2) * 2.0 ** -53 * O.wht_scale(d) * np.abs(x.astype(np.float64)).sum(-1)


def check_fp4_within_stated_bound(wl, pools):
    """Every group scale and every code of the workload's rows in the FP4 pools
    are the rounding decisions of some values within the stated bound of the
    exact rotated rows: the scale lies between the exponents of the group
    absmax minus and plus the bound, and each dequantized value between the
    roundings, at that scale, of the exact value minus and plus the bound."""
    d, H = wl.head_dim, wl.num_kv_heads
    T = wl.total_tokens
    t = np.arange(T)
    page = wl.page_table[0][t // 16]
    for pool, src, is_v in ((pools[0], wl.k, False), (pools[1], wl.v, True)):
        blk = pool.reshape(pool.shape[0], H, -1)
        off = O.fp4_v_scale_offset if is_v else O.fp4_k_scale_offset
        for h in range(H):
            rows = src[:, h]
            vals = O.gather_dequant(O.FMT_FP4, pool, wl.page_table[0], T, h, d, is_v)
            pos = O.fp4_block_position(h, page, H)[:, None]
            E = blk[page[:, None], pos, off((t % 16)[:, None], np.arange(d // 32)[None, :], d)].astype(np.int64) - 127
            y = O.wht(rows.astype(np.float64))
            delta = _stated_bound(rows, d)[:, None]
            m = np.abs(y).reshape(T, d // 32, 32).max(2)
            lo_e, hi_e = O.scale_exponent(np.maximum(m - delta, 0.0)), O.scale_exponent(m + delta)
            assert np.all((E >= lo_e) & (E <= hi_e)), "a group scale outside the stated bound"
            Ee = np.repeat(E, 32, axis=1)
            q = lambda v: np.ldexp(O.e2m1_decode(O.e2m1_encode(np.ldexp(v, -Ee))), Ee)
            assert np.all((vals >= q(y - delta)) & (vals <= q(y + delta))), "a code outside the stated bound"


def outside_domain_rows(d, rng):
    """The near-tie rows outside the exact-sum domain plus rows spanning up to
    2^100 (one large channel beside full-precision float32 values, float32
    subnormals beside normals); all outside the domain."""
    _, outside = _edge_rows(d, rng)
    extra = rng.standard_normal((40, d))
    extra[:, 0] *= 2.0 ** rng.integers(30, 100, 40)
    extra[10:20] *= 2.0 ** -100
    extra[20:30, 1:] *= 2.0 ** -40
    x = np.concatenate([outside, extra.astype(np.float32)])
    return x[~O.exact_sum_rows(x.astype(np.float64))]


@pytest.mark.parametrize("d", [64, 128])
def test_append_outside_exact_sum_domain_within_stated_bound(d):
    # uq.h: outside the exact-sum domain each rotated value is within
    # (log2 d + 2) 2^-53 c_d sum|x| of the exact one, and the stored bytes are
    # the rounding decisions of such a value.
    x = outside_domain_rows(d, np.random.default_rng(300 + d))
    assert x.shape[0] >= 40
    wl, got = _append_rows(d, x, False, "outside_domain")
    check_fp4_within_stated_bound(wl, got)


@pytest.mark.parametrize("d", [64, 128])
def test_query_rotation_outside_exact_sum_domain_within_stated_bound(d):
    torch = torch_mod()
    rng = np.random.default_rng(400 + d)
    x = rng.standard_normal((64, d))
    x[:, 0] *= 2.0 ** rng.integers(35, 60, 64)
    x = x.astype(np.float32)
    x = x[~O.exact_sum_rows(x.astype(np.float64))]
    assert x.shape[0] >= 60
    out = torch.empty(x.shape, dtype=torch.uint8, device="cuda")
    announce(f"query rotation outside the exact-sum domain d={d}")
    uq().uq_rotate_quantize_query(dev(x, "f32"), out)
    torch.cuda.synchronize()
    got = O.e4m3_decode(out.cpu().numpy())
    y = O.wht(x.astype(np.float64))
    delta = _stated_bound(x, d)[:, None]
    lo, hi = O.e4m3_decode(O.e4m3_encode(y - delta)), O.e4m3_decode(O.e4m3_encode(y + delta))
    assert np.all((got >= lo) & (got <= hi))


@pytest.mark.parametrize("fmt", FORMATS)
def test_append_skips_negative_slots_and_partial_calls(fmt):
    wl = _wl("gqa_ragged")
    announce(f"append {fmt} with skipped slots")
    rng = np.random.default_rng(0)
    slots = wl.slot_mapping.copy()
    slots[rng.random(slots.size) < 0.3] = -1
    cache = gpu_cache(fmt, wl)
    half = wl.total_tokens // 2
    gpu_append(fmt, wl, cache, idx=np.arange(half), slots=slots[:half])          # two calls
    gpu_append(fmt, wl, cache, idx=np.arange(half, wl.total_tokens), slots=slots[half:])
    want = oracle_append(fmt, wl, slots=slots)
    for g, w in zip(pools_np(cache), want):
        assert np.array_equal(g, w)


@pytest.mark.parametrize("in_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
def test_query_rotation_bytes(in_dtype, d):
    torch = torch_mod()
    rng = np.random.default_rng(d)
    rows = 333
    x = (rng.standard_normal((rows, d)) * 10.0 ** rng.integers(-6, 3, (rows, 1))).astype(np.float32)
    x[0] = 0.0
    x[1] = 1e4                                   # saturates after rotation
    x[2, :] = 0; x[2, 0] = -3e-3                 # subnormal E4M3 range, negative
    if in_dtype == "bf16":
        arr = W._to_bf16_bits(x)
    else:
        arr = x
    announce(f"query rotation {in_dtype} d={d} rows={rows}")
    out = torch.empty((rows, d), dtype=torch.uint8, device="cuda")
    uq().uq_rotate_quantize_query(dev(arr, in_dtype), out)
    torch.cuda.synchronize()
    want = O.rotate_quantize_query(arr, in_dtype=in_dtype)
    assert np.array_equal(out.cpu().numpy(), want)


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("name", SMALL)
def test_decode_on_oracle_cache(fmt, name):
    wl = _wl(name)
    if fmt == "bf16" and wl.in_dtype != "bf16":
        pytest.skip("the BF16 baseline takes a bf16 query")
    pools = oracle_append(fmt, wl)
    announce(f"decode {fmt} {name} B={wl.batch} Hq={wl.num_q_heads} Hkv={wl.num_kv_heads} lens={list(wl.seq_lens)}")
    got = gpu_decode(fmt, wl, gpu_cache(fmt, wl, pools))
    want = oracle_decode(fmt, wl, pools)
    assert_close(got, want, f"{fmt} {name}")
    for b in np.nonzero(wl.seq_lens == 0)[0]:
        assert not got[b].any()


def _many_short():
    """240 sequences, mostly short with a few long ones (about 65K tokens): with
    unequal lengths the decode charges each item a fixed cost when it divides the
    steps between workgroups, so shares here hold many items (several rounds)
    and cut items at uneven step counts."""
    rng = np.random.default_rng(77)
    lens = rng.choice([17, 40, 90, 130, 300, 600], size=240)
    lens[::37] = 2048 + rng.integers(0, 1500, size=lens[::37].size)
    return W.make_workload("many_short", 240, 32, 4, 128, list(lens), list(lens), seed=78)


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])     # 8- and 4-wave workgroups
def test_decode_many_short_sequences(fmt):
    wl = _many_short()
    pools = oracle_append(fmt, wl)
    announce(f"decode {fmt} many_short B={wl.batch} tokens={wl.total_tokens}")
    got = gpu_decode(fmt, wl, gpu_cache(fmt, wl, pools))
    assert_close(got, oracle_decode(fmt, wl, pools), f"{fmt} many_short")


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("name", ["tiny", "gqa_ragged", "one_long"])
def test_end_to_end(fmt, name):
    wl = _wl(name)
    if fmt == "bf16" and wl.in_dtype != "bf16":
        pytest.skip("the BF16 baseline takes a bf16 query")
    announce(f"end-to-end {fmt} {name}")
    got = gpu_decode(fmt, wl, gpu_append(fmt, wl))
    want = oracle_decode(fmt, wl, oracle_append(fmt, wl))
    assert_close(got, want, f"e2e {fmt} {name}")


def test_fp4_out_rotated_flag():
    wl = _wl("gqa_ragged")
    pools = oracle_append("fp4", wl)
    announce("decode fp4 OUT_ROTATED")
    got = gpu_decode("fp4", wl, gpu_cache("fp4", wl, pools), flags=uq().UQ_FLAG_OUT_ROTATED)
    want = O.wht(oracle_decode("fp4", wl, pools))        # normalized WHT is self-inverse
    assert_close(got, want, "out rotated")


def test_decode_repeatable_and_stream_ordered():
    # One step per workgroup here, so the same call twice gives identical bits.
    # With several steps per workgroup the waves claim steps dynamically, and
    # which wave's running sums a step joins changes between calls: the results
    # then differ at float32 rounding level only.
    wl = _wl("one_long")
    cache = gpu_append("fp4", wl)
    announce("decode fp4 repeat")
    a = gpu_decode("fp4", wl, cache)
    b = gpu_decode("fp4", wl, cache)
    assert np.array_equal(a, b)
    wl = _wl("multi_step")
    cache = gpu_append("fp4", wl)
    a = gpu_decode("fp4", wl, cache)
    b = gpu_decode("fp4", wl, cache)
    assert np.linalg.norm(a - b) <= 1e-6 * np.linalg.norm(a)


def test_fp4_decode_with_disparate_group_scales():
    # Rows whose rotated groups differ by 2^20 in magnitude: the scaled MFMA must
    # keep the small group's contribution (its UE8M0 block scale differs per lane).
    rng = np.random.default_rng(11)
    T, H, d = 96, 1, 64
    y = rng.standard_normal((T, H, d))
    y[..., :32] *= 2.0 ** 10
    y[..., 32:] *= 2.0 ** -10
    x = O.wht(y).astype(np.float32)
    wl = W.make_workload("wide", 1, 4, 1, d, [T], [T], in_dtype="f32", seed=3)
    wl.k[:] = x
    wl.v[:] = x[::-1]
    wl.q[:] = (rng.standard_normal((1, 4, d)) * 2.0 ** -8).astype(np.float32)
    pools = oracle_append("fp4", wl)
    announce("decode fp4 with group scales 2^10 / 2^-10")
    got = gpu_decode("fp4", wl, gpu_cache("fp4", wl, pools))
    want = oracle_decode("fp4", wl, pools)
    # compare per output element relative to that row's scale
    assert_close(got / np.abs(want).max(), want / np.abs(want).max(), "fp4 wide scales (normalized)")


def _scale_bf16_bits(bits, k):
    """bf16 bit patterns times 2^k (exact: normal values stay normal here)."""
    f = (np.asarray(bits).astype(np.uint32) << 16).view(np.float32) * np.float32(2.0 ** k)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def test_bf16_decode_outside_the_float16_range():
    # The BF16 baseline takes K, q and V into bf16 matrix products as stored:
    # values far outside float16's range (V near 2^60, K near 2^-60, q near 2^60)
    # must give the oracle's result, scaled.
    wl = _wl("gqa_ragged")
    wl.k = _scale_bf16_bits(wl.k, -60)
    wl.v = _scale_bf16_bits(wl.v, 60)
    wl.q = _scale_bf16_bits(wl.q, 60)
    pools = oracle_append("bf16", wl)
    announce("decode bf16 with |V| ~ 2^60, |K| ~ 2^-60")
    got = gpu_decode("bf16", wl, gpu_cache("bf16", wl, pools))
    want = oracle_decode("bf16", wl, pools)
    assert np.abs(want).max() > 2.0 ** 55
    assert_close(got * 2.0 ** -60, want * 2.0 ** -60, "bf16 outside the float16 range (scaled by 2^-60)")
