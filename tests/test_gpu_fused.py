"""GPU parity of the fused FP4 decode step (uq_append_decode_attention): the
newest token of every sequence is written into the cache and attended over in
one launch.

- The cache after the call must equal, bit for bit, the oracle's cache holding
  every token (small cases: whole pools; full size: sampled pages, always
  including pages that received a new token).
- The output must agree with the unfused decode (uq_decode_attention) run
  afterwards on the same cache to within float32 rounding (rel-L2 1e-6: the
  waves' dynamic step claims may group the sums differently between calls).
  Before the call the new token's slot holds another token with its V scaled
  by 2^10, so a read of the slot before the write would move the output by far
  more than that (about 2^10 / context length relative).
- The output must match the oracle within relative L2 1e-3 and max-abs 5e-3.

Small cases have one to a few steps per workgroup (the write is ordered by a
barrier before any claim); the full-size cases give every workgroup hundreds
of steps, so the item's last step is claimed after the main-loop barrier.
"""
import numpy as np
import pytest

import oracle as O
from bit_kv_cache_wht_amd import workloads as W

from gpu_util import (FMT_ID, announce, assert_close, dev, gpu_append, gpu_cache, gpu_decode, oracle_append,
                      oracle_decode, oracle_decode_rows_from_inputs, page_blocks_np, pools_np, torch_mod, uq)
from test_gpu_parity import SMALL, _wl

pytestmark = pytest.mark.gpu


def _split(wl):
    """(prefix token indices, newest token index of each non-empty sequence, the
    sequences that have one)."""
    lens = wl.seq_lens.astype(np.int64)
    has = np.nonzero(lens > 0)[0]
    new = wl.tok_offsets[has] + lens[has] - 1
    pre = np.setdiff1d(np.arange(wl.total_tokens), new)
    return pre, new, has


def _new_rows(wl, new, has):
    """k_new, v_new [B][H_kv][d] in the workload's input dtype (zero rows for empty
    sequences)."""
    shape = (wl.batch, wl.num_kv_heads, wl.head_dim)
    k = np.zeros(shape, wl.k.dtype)
    v = np.zeros(shape, wl.v.dtype)
    k[has], v[has] = wl.k[new], wl.v[new]
    return k, v


def _fused_call(wl, cache, k_new, v_new):
    torch = torch_mod()
    m = uq()
    B, Hq, d = wl.batch, wl.num_q_heads, wl.head_dim
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.zeros(m.uq_decode_workspace_bytes(cache, B, Hq, wl.page_table.shape[1]), dtype=torch.uint8,
                     device="cuda")
    m.uq_append_decode_attention(cache, dev(k_new, wl.in_dtype), dev(v_new, wl.in_dtype), dev(wl.q, wl.in_dtype),
                                 dev(np.ascontiguousarray(wl.page_table, dtype=np.int32)),
                                 dev(np.ascontiguousarray(wl.seq_lens, dtype=np.int32)),
                                 float(np.float32(1.0 / np.sqrt(d))), out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def _scaled(x, in_dtype, f):
    if in_dtype == "bf16":
        return W._to_bf16_bits((x.astype(np.uint32) << 16).view(np.float32) * np.float32(f))
    return (x * np.float32(f)).astype(np.float32)


def _prepared_cache(wl, pre, new):
    """GPU cache with the prefix written and, at each new token's slot, another
    token whose V is scaled by 2^10."""
    torch = torch_mod()
    cache = gpu_cache("fp4", wl)
    for i in range(0, pre.size, 1 << 18):
        gpu_append("fp4", wl, cache, idx=pre[i:i + (1 << 18)])
    if new.size:
        decoy = (new + 1) % wl.total_tokens
        uq().uq_quantize_append(cache, dev(wl.k[decoy], wl.in_dtype),
                                dev(_scaled(wl.v[decoy], wl.in_dtype, 1024.0), wl.in_dtype),
                                dev(np.ascontiguousarray(wl.slot_mapping[new], dtype=np.int32)))
        torch.cuda.synchronize()
    return cache


def _assert_same_as_unfused(got, wl, cache, what):
    again = gpu_decode("fp4", wl, cache)
    rel = np.linalg.norm(got - again) / max(np.linalg.norm(again), 1e-30)
    announce(f"{what}: fused vs unfused rel-L2 {rel:.2e}")
    assert rel <= 1e-6, f"{what}: fused output differs from the unfused decode of the same cache ({rel:.2e})"


@pytest.mark.parametrize("name", SMALL)
def test_fused_step_small(name):
    wl = _wl(name)
    pre, new, has = _split(wl)
    announce(f"fused fp4 {name} B={wl.batch} Hq={wl.num_q_heads} Hkv={wl.num_kv_heads} d={wl.head_dim} "
             f"lens={list(wl.seq_lens)}")
    cache = _prepared_cache(wl, pre, new)
    got = _fused_call(wl, cache, *_new_rows(wl, new, has))
    want_pools = oracle_append("fp4", wl)
    for g, w, kv in zip(pools_np(cache), want_pools, "KV"):
        bad = np.nonzero(g != w)
        assert bad[0].size == 0, f"{kv} pool: {bad[0].size} bytes differ, first at {[int(x[0]) for x in bad]}"
    _assert_same_as_unfused(got, wl, cache, f"fused {name}")
    assert_close(got, oracle_decode("fp4", wl, want_pools), f"fused {name}")
    for b in np.nonzero(wl.seq_lens == 0)[0]:
        assert not got[b].any()


def _check_new_pages(wl, cache, seqs, extra, seed):
    """Pages holding the new tokens of `seqs` plus `extra` random pages, whole,
    against the oracle's pages built from the tokens that live in them."""
    rng = np.random.default_rng(seed)
    lens = wl.seq_lens.astype(np.int64)
    page_of = wl.slot_mapping // 16
    new_pages = wl.page_table[seqs, (lens[seqs] - 1) // 16]
    pages = np.unique(np.concatenate([new_pages, rng.choice(np.unique(page_of), size=extra, replace=False)]))
    tok = np.nonzero(np.isin(page_of, pages))[0]
    # a pool of the full page count: the FP4 block positions depend on the page id
    kp = O.new_pool(FMT_ID["fp4"], wl.num_pages, wl.num_kv_heads, wl.head_dim)
    vp = O.new_pool(FMT_ID["fp4"], wl.num_pages, wl.num_kv_heads, wl.head_dim)
    O.append(FMT_ID["fp4"], kp, vp, wl.k[tok], wl.v[tok], wl.slot_mapping[tok], in_dtype=wl.in_dtype)
    got_k = page_blocks_np(cache, cache.k_pool, pages)
    got_v = page_blocks_np(cache, cache.v_pool, pages)
    announce(f"fused {wl.name}: {pages.size} sampled pages ({len(seqs)} with new tokens)")
    assert np.array_equal(got_k, kp[pages]), "K pages differ from the oracle"
    assert np.array_equal(got_v, vp[pages]), "V pages differ from the oracle"


@pytest.mark.parametrize("which", ["decode_gqa", "ragged"])
def test_fused_step_fullsize(which):
    wl = W.decode_gqa() if which == "decode_gqa" else W.ragged()
    pre, new, has = _split(wl)
    announce(f"fused fp4 {wl.name}: B={wl.batch} tokens={wl.total_tokens}")
    cache = _prepared_cache(wl, pre, new)
    got = _fused_call(wl, cache, *_new_rows(wl, new, has))
    rng = np.random.default_rng(61)
    seqs = np.sort(rng.choice(has, size=min(16, has.size), replace=False))
    _check_new_pages(wl, cache, seqs, 16, seed=62)
    _assert_same_as_unfused(got, wl, cache, f"fused {wl.name}")
    G = wl.num_q_heads // wl.num_kv_heads
    pairs = [(int(seqs[0]), 0), (int(seqs[-1]), wl.num_kv_heads - 1)]
    rows = [(b, hk * G + g) for b, hk in pairs for g in range(G)]
    want = oracle_decode_rows_from_inputs("fp4", wl, rows)
    assert_close(np.array([got[b, h] for b, h in rows]), want, f"fused {wl.name} rows of {pairs}")
    del cache
    torch_mod().cuda.empty_cache()
