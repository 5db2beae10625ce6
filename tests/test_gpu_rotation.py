"""GPU parity of the FP4 cache's rotation variants (UQ_ROT_K_ONLY: V stored in
its own basis, output not rotated back; UQ_ROT_SIGNS: R = c_d H diag(s) for K,
V and the query, output through R^T) and of caches of different formats and
variants side by side (BF16 boundary layers around FP4 layers).

- Append: bytes equal to the oracle's, through the small-batch and the
  large-batch kernels, bf16 and f32 inputs, d = 64 and 128.
- Decode, fused append + decode and chunked prefill: outputs within relative
  L2 1e-3 and max-abs 5e-3 of the oracle's, on caches the GPU wrote.
"""
import numpy as np
import pytest

import oracle as O
from bit_kv_cache_wht_amd import workloads as W

from gpu_util import (FMT_ID, announce, assert_close, dev, gpu_append, gpu_cache, gpu_decode, oracle_append,
                      oracle_decode, pools_np, sm_scale, torch_mod, uq)
from test_gpu_fused import _new_rows, _split
from test_gpu_parity import _wl

pytestmark = pytest.mark.gpu

VARIANTS = {"k_only": (True, False), "signs": (False, True), "k_only_signs": (True, True)}


def _variant(name, d, seed=3001):
    k_only, signed = VARIANTS[name]
    return k_only, (W.rotation_signs(d, seed) if signed else None)


def _assert_pools_equal(got, want, what):
    for g, w, kv in zip(got, want, "KV"):
        bad = np.nonzero(g != w)
        assert bad[0].size == 0, f"{what}: {kv} pool: {bad[0].size} bytes differ, first at {[int(x[0]) for x in bad]}"


@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("name", ["tiny", "edge_lens", "gqa_ragged", "d64_bf16", "multi_ragged"])
def test_variant_append_bit_exact(variant, name):
    wl = _wl(name)
    k_only, signs = _variant(variant, wl.head_dim, seed=len(name))
    announce(f"append fp4 {variant} {name} T={wl.total_tokens} H={wl.num_kv_heads} d={wl.head_dim} {wl.in_dtype}")
    cache = gpu_append("fp4", wl, cache=gpu_cache("fp4", wl, k_only=k_only, signs=signs))
    _assert_pools_equal(pools_np(cache), oracle_append("fp4", wl, k_only=k_only, signs=signs), f"{variant} {name}")


@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("name", ["tiny", "edge_lens", "gqa_ragged", "mha_5heads", "group16_d64", "empty_seqs",
                                  "d64_bf16", "multi_ragged"])
def test_variant_decode(variant, name):
    wl = _wl(name)
    k_only, signs = _variant(variant, wl.head_dim, seed=7 + len(name))
    announce(f"decode fp4 {variant} {name} lens={list(wl.seq_lens)} Hq={wl.num_q_heads} Hkv={wl.num_kv_heads}")
    cache = gpu_append("fp4", wl, cache=gpu_cache("fp4", wl, k_only=k_only, signs=signs))
    pools = oracle_append("fp4", wl, k_only=k_only, signs=signs)
    _assert_pools_equal(pools_np(cache), pools, f"{variant} {name}")
    got = gpu_decode("fp4", wl, cache)
    assert_close(got, oracle_decode("fp4", wl, pools, k_only=k_only, signs=signs), f"decode {variant} {name}")


def test_signed_out_rotated_flag():
    # UQ_FLAG_OUT_ROTATED leaves the output in the rotated basis: R o; with
    # K-only rotation the output is in the original basis either way.
    wl = _wl("gqa_ragged")
    signs = W.rotation_signs(wl.head_dim, 5)
    pools = oracle_append("fp4", wl, signs=signs)
    announce("decode fp4 signs OUT_ROTATED")
    got = gpu_decode("fp4", wl, gpu_cache("fp4", wl, pools, signs=signs), flags=uq().UQ_FLAG_OUT_ROTATED)
    want = O.rotate(oracle_decode("fp4", wl, pools, signs=signs), signs)
    assert_close(got, want, "signs out rotated")
    pools = oracle_append("fp4", wl, k_only=True)
    got = gpu_decode("fp4", wl, gpu_cache("fp4", wl, pools, k_only=True), flags=uq().UQ_FLAG_OUT_ROTATED)
    assert_close(got, oracle_decode("fp4", wl, pools, k_only=True), "k_only out rotated")


@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("name", ["edge_lens", "multi_step"])
def test_variant_fused_step(variant, name):
    torch = torch_mod()
    m = uq()
    wl = _wl(name)
    k_only, signs = _variant(variant, wl.head_dim, seed=3 + len(name))
    pre, new, has = _split(wl)
    announce(f"fused fp4 {variant} {name} lens={list(wl.seq_lens)}")
    cache = gpu_cache("fp4", wl, k_only=k_only, signs=signs)
    if pre.size:
        gpu_append("fp4", wl, cache, idx=pre)
    k_new, v_new = _new_rows(wl, new, has)
    B, Hq, d = wl.batch, wl.num_q_heads, wl.head_dim
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.zeros(m.uq_decode_workspace_bytes(cache, B, Hq, wl.page_table.shape[1]), dtype=torch.uint8,
                     device="cuda")
    m.uq_append_decode_attention(cache, dev(k_new, wl.in_dtype), dev(v_new, wl.in_dtype), dev(wl.q, wl.in_dtype),
                                 dev(np.ascontiguousarray(wl.page_table, dtype=np.int32)),
                                 dev(np.ascontiguousarray(wl.seq_lens, dtype=np.int32)),
                                 float(np.float32(1.0 / np.sqrt(d))), out, ws)
    torch.cuda.synchronize()
    want_pools = oracle_append("fp4", wl, k_only=k_only, signs=signs)
    _assert_pools_equal(pools_np(cache), want_pools, f"fused {variant} {name}")
    assert_close(out.cpu().numpy().astype(np.float64),
                 oracle_decode("fp4", wl, want_pools, k_only=k_only, signs=signs), f"fused {variant} {name}")


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_variant_prefill(variant):
    wl = W.make_workload("pf_rot", 3, 32, 4, 128, [700, 300, 129], [256, 40, 129], seed=77)
    q, cu = W.prefill_queries(wl, seed=78)
    k_only, signs = _variant(variant, wl.head_dim, seed=79)
    announce(f"prefill fp4 {variant} lens={list(wl.seq_lens)} chunks={list(np.diff(cu))}")
    torch = torch_mod()
    cache = gpu_append("fp4", wl, cache=gpu_cache("fp4", wl, k_only=k_only, signs=signs))
    out = torch.full((q.shape[0], wl.num_q_heads, wl.head_dim), float("nan"), dtype=torch.float32, device="cuda")
    uq().uq_prefill_attention(cache, dev(q, wl.in_dtype), dev(cu), dev(np.ascontiguousarray(wl.page_table)),
                              dev(np.ascontiguousarray(wl.seq_lens)), sm_scale(wl.head_dim), out)
    torch.cuda.synchronize()
    kp, vp = oracle_append("fp4", wl, k_only=k_only, signs=signs)
    want = O.prefill_attention(FMT_ID["fp4"], kp, vp, wl.num_kv_heads, wl.head_dim, q, np.diff(cu), wl.page_table,
                               wl.seq_lens, sm_scale(wl.head_dim), in_dtype=wl.in_dtype, k_only=k_only, signs=signs)
    assert_close(out.cpu().numpy().astype(np.float64), want, f"prefill {variant}")


def test_mixed_layer_formats():
    # Six attention layers of one model on one stream: the first two and the last
    # two keep BF16 caches, the middle ones FP4 (one plain, one with signs); each
    # layer's cache descriptor selects its own format and rotation.
    layers = [("bf16", False, None), ("bf16", False, None), ("fp4", False, None),
              ("fp4", False, W.rotation_signs(128, 9)), ("bf16", False, None), ("bf16", False, None)]
    base = _wl("gqa_ragged")
    outs, wants = [], []
    for i, (fmt, k_only, signs) in enumerate(layers):
        wl = W.make_workload(f"layer{i}", base.batch, base.num_q_heads, base.num_kv_heads, base.head_dim,
                             list(base.seq_lens), list(base.seq_lens), seed=500 + i)
        announce(f"layer {i}: {fmt} signs={signs is not None}")
        cache = gpu_append(fmt, wl, cache=gpu_cache(fmt, wl, k_only=k_only, signs=signs))
        outs.append(gpu_decode(fmt, wl, cache))
        pools = oracle_append(fmt, wl, k_only=k_only, signs=signs)
        wants.append(oracle_decode(fmt, wl, pools, k_only=k_only, signs=signs))
    for i, (g, w) in enumerate(zip(outs, wants)):
        assert_close(g, w, f"layer {i} ({layers[i][0]})")


@pytest.mark.parametrize("variant", ["plain", "k_only", "signs", "k_only_signs"])
@pytest.mark.parametrize("in_dtype,d", [("bf16", 128), ("f32", 64)])
def test_query_rotation_of_a_cache(variant, in_dtype, d):
    # uq_rotate_quantize_query_cache: the E4M3 bytes of R q with the cache's R
    # (c_d H diag(s) for a signed cache; K-only caches rotate queries as usual)
    torch = torch_mod()
    k_only, signs = (False, None) if variant == "plain" else _variant(variant, d, seed=d + 5)
    rng = np.random.default_rng(d + 11)
    rows = 257
    x = (rng.standard_normal((rows, d)) * 10.0 ** rng.integers(-4, 2, (rows, 1))).astype(np.float32)
    arr = W._to_bf16_bits(x) if in_dtype == "bf16" else x
    wl = W.make_workload("qrot", 1, 1, 1, d, [16], [16], in_dtype=in_dtype, seed=1)
    cache = gpu_cache("fp4", wl, k_only=k_only, signs=signs)
    out = torch.empty((rows, d), dtype=torch.uint8, device="cuda")
    announce(f"query rotation of a {variant} cache, {in_dtype} d={d}")
    uq().uq_rotate_quantize_query_cache(cache, dev(arr, in_dtype), out)
    torch.cuda.synchronize()
    want = O.rotate_quantize_query(arr, in_dtype=in_dtype, signs=signs)
    assert np.array_equal(out.cpu().numpy(), want)
    if signs is not None:                              # the plain rotation differs
        assert not np.array_equal(want, O.rotate_quantize_query(arr, in_dtype=in_dtype))
