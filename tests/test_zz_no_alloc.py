"""The no-allocation FP4 decode (uq_decode_attention_noalloc, for callers that
cannot allocate) against the workspace decode (uq_decode_attention) on the same
caches, and against the oracle: two calls in a row, the second with a smaller
input, so that the second call runs on the static scratch array as the first
left it (counters back at zero, stale partials of another shape)."""
import numpy as np
import pytest

from bit_kv_cache_wht_amd import workloads as W

from gpu_util import (announce, assert_close, dev, gpu_append, gpu_decode, oracle_append, oracle_decode, sm_scale,
                      torch_mod, uq)

pytestmark = pytest.mark.gpu


def _noalloc(wl, cache):
    torch = torch_mod()
    B, Hq, d = wl.batch, wl.num_q_heads, wl.head_dim
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    uq().uq_decode_attention_noalloc(cache, dev(wl.q, wl.in_dtype), dev(np.ascontiguousarray(wl.page_table)),
                                     dev(np.ascontiguousarray(wl.seq_lens)), sm_scale(d), out)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def test_noalloc_decode_matches_workspace_decode_on_two_calls():
    # both shapes cut their items between workgroups, so both calls write and
    # merge split partials and use the arrival counters
    big = W.make_workload("noalloc_big", 6, 32, 4, 128, [3000, 1500, 7000, 64, 2500, 5000],
                          [1] * 6, seed=811)
    small = W.make_workload("noalloc_small", 2, 8, 2, 128, [900, 4100], [1] * 2, seed=812)
    for wl in (big, small):
        announce(f"noalloc decode {wl.name}: B={wl.batch} Hq={wl.num_q_heads} Hkv={wl.num_kv_heads} "
                 f"lens={list(wl.seq_lens)}")
        cache = gpu_append("fp4", wl)
        got = _noalloc(wl, cache)
        want = gpu_decode("fp4", wl, cache)
        assert_close(got, want, f"noalloc vs workspace decode, {wl.name}")
        assert_close(got, oracle_decode("fp4", wl, oracle_append("fp4", wl)), f"noalloc vs oracle, {wl.name}")
