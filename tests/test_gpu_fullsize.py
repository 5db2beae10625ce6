"""GPU parity at the full configured sizes, through the same C-ABI calls the bench
times (the library picks its launch configuration from the shapes alone).

- Cache bytes: every page of the GPU pools must equal, bit for bit, the page the
  oracle builds from the raw inputs (append 65,536 tokens x 8 heads; decode
  64 x 8,192 and 8 x 65,536 with 64 / 8 heads; ragged 128 sequences of
  1,024..131,072 tokens with 32 / 4 heads).
- Attention: the whole output tensor of each decode must be within relative L2
  1e-3 (over all rows) and max-abs 5e-3 (over every element) of the oracle's
  decode over its own pools -- FP4 on all three decode workloads, the FP8 and
  BF16 baselines on 64 x 8,192.
- Chunked prefill (ragged, the last 256 tokens of each sequence as the chunk):
  sampled rows of the longest, the shortest and a median sequence against the
  oracle's decode of that row over its causal prefix (the whole tensor would
  take the float64 oracle hours).

The oracle runs on up to 16 host threads (token chunks for the cache, (sequence,
KV head) pairs for the decode).
"""
import numpy as np
import pytest

import oracle as O
from bit_kv_cache_wht_amd import workloads as W

from gpu_util import (announce, assert_close, gpu_append, gpu_decode, oracle_append_all, oracle_decode_all,
                      oracle_threads, pools_np, sm_scale, torch_mod, uq)

pytestmark = pytest.mark.gpu


def _free():
    torch = torch_mod()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _whole(fmt, wl, decode=True):
    """GPU append of every token, then (decode) the GPU decode; every page and
    (decode) the whole output tensor against the oracle."""
    announce(f"{fmt} {wl.name}: B={wl.batch} tokens={wl.total_tokens} Hq={wl.num_q_heads} "
             f"Hkv={wl.num_kv_heads} (oracle on {oracle_threads()} threads)")
    cache = gpu_append(fmt, wl)
    got = gpu_decode(fmt, wl, cache) if decode else None
    gk, gv = pools_np(cache)
    del cache
    _free()
    kp, vp = oracle_append_all(fmt, wl)
    nk, nv = int(np.count_nonzero(gk != kp)), int(np.count_nonzero(gv != vp))
    announce(f"{fmt} {wl.name}: {kp.shape[0]} pages compared, {nk} K and {nv} V bytes differ")
    assert nk == 0 and nv == 0, f"{fmt} {wl.name}: {nk} K and {nv} V cache bytes differ from the oracle"
    del gk, gv
    if decode:
        want = oracle_decode_all(fmt, wl, (kp, vp))
        assert_close(got, want, f"{fmt} {wl.name} whole output")
        for b in np.nonzero(wl.seq_lens == 0)[0]:
            assert not got[b].any()


def test_append_65536x8x128_all_pages_exact():
    _whole("fp4", W.append_only(), decode=False)


@pytest.mark.parametrize("fmt", ["fp4", "fp8", "bf16"])
def test_decode_gqa_64x8192_whole(fmt):
    _whole(fmt, W.decode_gqa())


def test_long_context_8x65536_fp4_whole():
    _whole("fp4", W.long_context())


def test_ragged_128_fp4_whole():
    _whole("fp4", W.ragged())


def test_prefill_ragged_128_fp4():
    # The bench's prefill call: the last 256 tokens of each of the 128 ragged
    # sequences attend causally to their cache.  Sampled chunk rows (first, middle
    # and last token of the chunk; all query heads of one KV head) of the longest,
    # the shortest and a median sequence against the oracle's decode of that row
    # over its causal prefix, from a private cache of the pair's raw inputs.
    torch = torch_mod()
    wl = W.ragged()
    q, cu = W.prefill_queries(wl)
    lens = wl.seq_lens
    announce(f"prefill fp4 {wl.name}: B={wl.batch} lens {int(lens.min())}..{int(lens.max())} Tq={q.shape[0]}")
    cache = gpu_append("fp4", wl)
    out = torch.full((q.shape[0], wl.num_q_heads, wl.head_dim), float("nan"), dtype=torch.float32, device="cuda")
    dv = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    qd = dv(q.view(np.int16)).view(torch.bfloat16)
    uq().uq_prefill_attention(cache, qd, dv(cu), dv(wl.page_table), dv(wl.seq_lens), sm_scale(wl.head_dim), out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    del cache, out, qd
    _free()
    assert np.isfinite(got).all()
    G, d = wl.num_q_heads // wl.num_kv_heads, wl.head_dim
    order = np.argsort(lens)
    for b, hk in [(int(order[-1]), 3), (int(order[0]), 0), (int(order[len(order) // 2]), 2)]:
        L, ql, t0 = int(lens[b]), int(cu[b + 1] - cu[b]), int(wl.tok_offsets[b])
        npg = (L + 15) // 16
        kp, vp = O.new_pool(O.FMT_FP4, npg, 1, d), O.new_pool(O.FMT_FP4, npg, 1, d)
        O.append(O.FMT_FP4, kp, vp, wl.k[t0:t0 + L, hk:hk + 1], wl.v[t0:t0 + L, hk:hk + 1],
                 np.arange(L, dtype=np.int32), in_dtype=wl.in_dtype)
        for j in (0, ql // 2, ql - 1):
            row = int(cu[b]) + j
            qrows = q[row:row + 1, hk * G:(hk + 1) * G].reshape(1, G, d)
            want = O.decode_attention_rows(O.FMT_FP4, kp, vp, 1, d, qrows, np.arange(npg)[None, :],
                                           np.array([L - ql + j + 1]), sm_scale(d), [(0, g) for g in range(G)],
                                           in_dtype=wl.in_dtype)
            assert_close(got[row, hk * G:(hk + 1) * G], want, f"prefill ragged seq {b} (L={L}) token {j} kv {hk}")
