"""GPU parity of the constOpt scale mode (UQ_FLAG_SCALE_CONSTOPT): group scale
E = the integer nearest to log2(0.156 * m) (log domain), codes saturating at 6.

- The FP4 append with the flag must equal the oracle's constOpt append bit for
  bit: on the small workloads, on rows that reach every rounding regime, and on
  rows whose group absmax puts 0.156 * m within float32 rounding of a log-domain
  decision point sqrt(2) * 2^k (both sides).
- The fused step with the flag writes the same bytes and attends over them
  (output within relative L2 1e-3 and max-abs 5e-3 of the oracle).
"""
import numpy as np
import pytest

import oracle as O
from bit_kv_cache_wht_amd import workloads as W

from gpu_util import (announce, assert_close, dev, gpu_append, gpu_cache, oracle_append, oracle_decode, pools_np,
                      torch_mod, uq)
from test_gpu_fused import _new_rows, _split
from test_gpu_parity import SMALL, _edge_rows, _wl

pytestmark = pytest.mark.gpu


def _flag():
    return uq().UQ_FLAG_SCALE_CONSTOPT


def _assert_pools_equal(got, want, what):
    for g, w, kv in zip(got, want, "KV"):
        bad = np.nonzero(g != w)
        assert bad[0].size == 0, f"{what}: {kv} pool: {bad[0].size} bytes differ, first at {[int(x[0]) for x in bad]}"


@pytest.mark.parametrize("name", SMALL)
def test_constopt_append_bit_exact(name):
    wl = _wl(name)
    announce(f"append fp4 constOpt {name} T={wl.total_tokens} H={wl.num_kv_heads} d={wl.head_dim}")
    got = pools_np(gpu_append("fp4", wl, flags=_flag()))
    want = oracle_append("fp4", wl, scale_mode="constopt")
    _assert_pools_equal(got, want, f"constOpt {name}")
    # the rule differs from the absmax rule: some scale bytes must differ
    assert any((g != w).any() for g, w in zip(got, oracle_append("fp4", wl)))


def _rows_wl(x, d, H=2):
    T = x.shape[0] // H
    wl = W.make_workload("constopt_rows", 1, H, H, d, [T], [T], in_dtype="f32", seed=9)
    wl.k = np.ascontiguousarray(x[: T * H].reshape(T, H, d))
    wl.v = np.ascontiguousarray(-x[::-1][: T * H].reshape(T, H, d))
    return wl


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("many", [False, True])
def test_constopt_append_extreme_scales(d, many):
    # `many` repeats the rows past the small-batch threshold (large-batch kernel)
    rng = np.random.default_rng(100 + d + (7 if many else 0))
    x = np.tile(_edge_rows(d, rng)[0], (1600 if many else 1, 1))   # rows inside the exact-sum domain
    wl = _rows_wl(x, d)
    announce(f"append fp4 constOpt extreme scales d={d} T={wl.total_tokens}")
    _assert_pools_equal(pools_np(gpu_append("fp4", wl, flags=_flag())),
                        oracle_append("fp4", wl, scale_mode="constopt"), f"constOpt extreme d={d}")


def test_constopt_append_exponent_decision_points():
    # d = 64: the normalized WHT is H / 8, so the input row m/8 * (1, ..., 1)
    # rotates exactly to (m, 0, ..., 0): group 0 has absmax m, group 1 is zero.
    # m runs over the float32 values next to sqrt(2) * 2^k / 0.156 (the products
    # 0.156 * m then fall within float32 rounding of the decision point, on both
    # sides), exponents -120 .. 125.
    d = 64
    ms = []
    for k in range(-117, 123, 3):                      # 2^-120 < m < 2^125
        t = np.float32(O.SQRT2_UP * 2.0 ** k / O.CONSTOPT_C)
        ms += [t, np.nextafter(t, np.float32(0)), np.nextafter(t, np.float32(np.inf))]
    ms = np.array(ms, dtype=np.float32)
    assert np.all(np.isfinite(ms)) and ms.min() > 2.0 ** -120 and ms.max() < 2.0 ** 125
    x = np.repeat((ms / np.float32(8.0))[:, None], d, axis=1).astype(np.float32)
    sign = np.where(np.arange(ms.size) % 2 == 0, 1.0, -1.0).astype(np.float32)[:, None]
    x = x * sign
    if x.shape[0] % 2:
        x = x[:-1]
    wl = _rows_wl(x, d)
    e = O.scale_exponent_constopt(ms.astype(np.float64))
    assert len(set(e.tolist())) > 50                   # many exponents, both sides of the decision
    s = np.float64(O.CONSTOPT_C) * ms.astype(np.float64)
    up = 2.0 * np.frexp(s)[0] >= O.SQRT2_UP
    assert 0 < up.sum() < up.size
    announce(f"append fp4 constOpt exponent decision points ({x.shape[0]} rows)")
    _assert_pools_equal(pools_np(gpu_append("fp4", wl, flags=_flag())),
                        oracle_append("fp4", wl, scale_mode="constopt"), "constOpt decision points")


@pytest.mark.parametrize("name", ["edge_lens", "gqa_ragged", "d64_bf16", "multi_step"])
def test_constopt_fused_step(name):
    torch = torch_mod()
    m = uq()
    wl = _wl(name)
    pre, new, has = _split(wl)
    announce(f"fused fp4 constOpt {name} lens={list(wl.seq_lens)}")
    cache = gpu_cache("fp4", wl)
    if pre.size:
        gpu_append("fp4", wl, cache, idx=pre, flags=_flag())
    k_new, v_new = _new_rows(wl, new, has)
    B, Hq, d = wl.batch, wl.num_q_heads, wl.head_dim
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.zeros(m.uq_decode_workspace_bytes(cache, B, Hq, wl.page_table.shape[1]), dtype=torch.uint8,
                     device="cuda")
    m.uq_append_decode_attention(cache, dev(k_new, wl.in_dtype), dev(v_new, wl.in_dtype), dev(wl.q, wl.in_dtype),
                                 dev(np.ascontiguousarray(wl.page_table, dtype=np.int32)),
                                 dev(np.ascontiguousarray(wl.seq_lens, dtype=np.int32)),
                                 float(np.float32(1.0 / np.sqrt(d))), out, ws, flags=_flag())
    torch.cuda.synchronize()
    want_pools = oracle_append("fp4", wl, scale_mode="constopt")
    _assert_pools_equal(pools_np(cache), want_pools, f"fused constOpt {name}")
    assert_close(out.cpu().numpy().astype(np.float64), oracle_decode("fp4", wl, want_pools), f"fused constOpt {name}")
