"""UQ_FLAG_CHECK on the GPU: the decode entry points validate sequence lengths
and page ids and report them in the workspace's error word.

The pools are allocated with four pages more than the cache descriptor
declares, and the bad page ids used here are num_pages and num_pages + 3, so
even an unchecked read would stay inside the pool allocation; the error word
and the outputs show whether the check replaced them.  Bad lengths are clamped
to the page-table row with or without the check.
"""
import numpy as np
import pytest

import oracle as O
from bit_kv_cache_wht_amd import workloads as W

from gpu_util import (FMT_ID, announce, assert_close, dev, gpu_append, oracle_append, oracle_decode, sm_scale,
                      torch_mod, uq)

pytestmark = pytest.mark.gpu

SLACK = 4


def _wl():
    return W.make_workload("check", 4, 16, 2, 128, [300, 1000, 77, 500], [1] * 4, seed=901)


def _cache(fmt, wl):
    """A cache whose pools hold SLACK pages more than its descriptor declares."""
    m = uq()
    c = m.KvCache.allocate(FMT_ID[fmt], wl.num_pages + SLACK, wl.num_kv_heads, wl.head_dim)
    c.num_pages = wl.num_pages
    return gpu_append(fmt, wl, c)


def _decode(fmt, wl, cache, page_table, seq_lens, flags):
    torch = torch_mod()
    m = uq()
    B, Hq, d = wl.batch, wl.num_q_heads, wl.head_dim
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.zeros(m.uq_decode_workspace_bytes(cache, B, Hq, page_table.shape[1]), dtype=torch.uint8,
                     device="cuda")
    fn = {"fp4": m.uq_decode_attention, "fp8": m.uq_decode_attention_fp8, "bf16": m.uq_decode_attention_bf16}[fmt]
    fn(cache, dev(wl.q, wl.in_dtype), dev(np.ascontiguousarray(page_table, dtype=np.int32)),
       dev(np.ascontiguousarray(seq_lens, dtype=np.int32)), sm_scale(wl.head_dim), out, ws, flags=flags)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), m.decode_check_word(ws)


@pytest.mark.parametrize("fmt", ["fp4", "fp8", "bf16"])
def test_check_on_valid_contents_reports_nothing(fmt):
    wl = _wl()
    announce(f"check {fmt}: valid page table and lengths")
    cache = _cache(fmt, wl)
    got, word = _decode(fmt, wl, cache, wl.page_table, wl.seq_lens, uq().UQ_FLAG_CHECK)
    assert word == 0
    assert_close(got, oracle_decode(fmt, wl, oracle_append(fmt, wl)), f"{fmt} checked decode")


@pytest.mark.parametrize("fmt", ["fp4", "fp8", "bf16"])
def test_check_reports_bad_page_ids_and_lengths(fmt):
    m = uq()
    wl = _wl()
    cache = _cache(fmt, wl)
    want = oracle_decode(fmt, wl, oracle_append(fmt, wl))
    N = wl.num_pages
    bad_pt = wl.page_table.copy()
    bad_pt[1, 2] = N                                   # one past the last page
    bad_pt[2, 0] = N + SLACK - 1
    announce(f"check {fmt}: page ids {N} and {N + SLACK - 1} in sequences 1 and 2")
    got, word = _decode(fmt, wl, cache, bad_pt, wl.seq_lens, m.UQ_FLAG_CHECK)
    assert word == m.UQ_CHECK_BAD_PAGE
    # the sequences without a bad id are untouched
    assert_close(got[[0, 3]], want[[0, 3]], f"{fmt}: rows of the sequences with valid pages")
    assert np.all(np.isfinite(got))
    bad_len = wl.seq_lens.copy()
    bad_len[0] = -3
    bad_len[3] = 16 * wl.page_table.shape[1] + 5
    announce(f"check {fmt}: lengths {list(bad_len)}")
    got, word = _decode(fmt, wl, cache, wl.page_table, bad_len, m.UQ_FLAG_CHECK)
    assert word == m.UQ_CHECK_BAD_LEN
    assert not got[0].any()                            # -3 is used as 0: an empty sequence
    assert_close(got[[1, 2]], want[[1, 2]], f"{fmt}: rows of the sequences with valid lengths")
    got, word = _decode(fmt, wl, cache, bad_pt, bad_len, m.UQ_FLAG_CHECK)
    assert word == m.UQ_CHECK_BAD_LEN | m.UQ_CHECK_BAD_PAGE


def test_check_fused_step_writes_nothing_into_a_bad_page():
    torch = torch_mod()
    m = uq()
    wl = _wl()
    B, Hq, Hkv, d = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    cache = _cache("fp4", wl)
    before_k, before_v = cache.k_pool.cpu().numpy().copy(), cache.v_pool.cpu().numpy().copy()
    bad_pt = wl.page_table.copy()
    last = (wl.seq_lens - 1) // 16
    bad_pt[1, last[1]] = wl.num_pages                  # the page of sequence 1's newest token
    rng = np.random.default_rng(5)
    kn = W._to_bf16_bits(rng.standard_normal((B, Hkv, d)).astype(np.float32))
    vn = W._to_bf16_bits(rng.standard_normal((B, Hkv, d)).astype(np.float32))
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.zeros(m.uq_decode_workspace_bytes(cache, B, Hq, bad_pt.shape[1]), dtype=torch.uint8, device="cuda")
    announce("check fused fp4: newest token's page id out of the pool")
    m.uq_append_decode_attention(cache, dev(kn, "bf16"), dev(vn, "bf16"), dev(wl.q, "bf16"),
                                 dev(np.ascontiguousarray(bad_pt)), dev(np.ascontiguousarray(wl.seq_lens)),
                                 sm_scale(d), out, ws, flags=m.UQ_FLAG_CHECK)
    torch.cuda.synchronize()
    assert m.decode_check_word(ws) == m.UQ_CHECK_BAD_PAGE
    after_k, after_v = cache.k_pool.cpu().numpy(), cache.v_pool.cpu().numpy()
    # the slack pages past the declared pool are never written
    assert np.array_equal(after_k[wl.num_pages:], before_k[wl.num_pages:])
    assert np.array_equal(after_v[wl.num_pages:], before_v[wl.num_pages:])
    # the other sequences' newest tokens were written: their pages changed
    for b in (0, 2, 3):
        pg = wl.page_table[b, last[b]]
        assert not np.array_equal(after_k[pg], before_k[pg])
