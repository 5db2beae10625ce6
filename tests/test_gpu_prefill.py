"""GPU parity of the chunked-prefill attention over the FP4 cache
(uq_prefill_attention): each sequence's chunk holds its last q_len positions,
already in the cache; chunk token j at position P attends to positions 0 .. P.
Outputs are compared with the oracle (each row = the decode over its causal
prefix) within relative L2 1e-3 and max-abs 5e-3.

Cases: chunks after a prefix and whole prompts, chunk lengths that are not
multiples of a workgroup's tokens, empty chunks, GQA groups of 1, 4, 5, 6, 8, 16, 32
and 128 (5 and 6 do not divide a workgroup's 256 rows; 128 is the largest the
boundary takes),
whole prompts of several hundred tokens with one query head per KV head, 600
sequences (the workgroups' plan in several chunks),
d = 64 and 128, bf16 and f32 inputs, and single-token chunks (which must also
agree with the decode entry point itself)."""
import numpy as np
import pytest

import oracle as O
from bit_kv_cache_wht_amd import workloads as W

from gpu_util import FMT_ID, announce, assert_close, dev, gpu_append, gpu_decode, oracle_append, sm_scale, torch_mod, uq

pytestmark = pytest.mark.gpu

CASES = {
    # name: (B, Hq, Hkv, d, seq_lens, chunk lens, in_dtype)
    "chunk_after_prefix": (3, 32, 4, 128, [700, 300, 1290], [256, 40, 77], "bf16"),
    "whole_prompts": (2, 16, 2, 128, [200, 33], [200, 33], "bf16"),
    "single_tokens": (4, 64, 8, 128, [1, 17, 400, 1000], [1, 1, 1, 1], "bf16"),
    "mha_d64_f32": (2, 4, 4, 64, [150, 90], [64, 90], "f32"),
    "group16": (2, 16, 1, 128, [520, 64], [129, 1], "bf16"),
    "empty_chunks": (4, 8, 2, 128, [100, 50, 300, 16], [0, 50, 0, 16], "bf16"),
    # one query head per KV head: a workgroup's 256 rows are 256 consecutive
    # positions, so its waves reach the diagonal at different steps
    "mha_long_prompts": (3, 2, 2, 128, [1000, 531, 777], [300, 531, 777], "bf16"),
    # query groups that do not divide a workgroup's 256 rows: 42 tokens x 6 heads
    # (4 padding rows) and 51 x 5 (1), so row / G and row % G cross token
    # boundaries inside a 16-row block
    "group6": (3, 12, 2, 128, [600, 257, 90], [300, 257, 45], "bf16"),
    "group5_d64_f32": (2, 10, 2, 64, [333, 129], [200, 129], "f32"),
    # the largest group the boundary takes (128 query heads per KV head: two
    # chunk tokens per workgroup), and 32
    "group128_d64": (2, 128, 1, 64, [90, 40], [20, 40], "bf16"),
    "group32": (2, 64, 2, 128, [300, 77], [100, 77], "bf16"),
}


def _case(name):
    B, Hq, Hkv, d, lens, chunks, dt = CASES[name]
    wl = W.make_workload(name, B, Hq, Hkv, d, lens, chunks, in_dtype=dt, seed=sum(map(ord, name)))
    q, cu = W.prefill_queries(wl, seed=len(name))
    return wl, q, cu


def _gpu_prefill(wl, q, cu, cache):
    torch = torch_mod()
    out = torch.full((q.shape[0], wl.num_q_heads, wl.head_dim), float("nan"), dtype=torch.float32, device="cuda")
    uq().uq_prefill_attention(cache, dev(q, wl.in_dtype), dev(cu), dev(np.ascontiguousarray(wl.page_table)),
                              dev(np.ascontiguousarray(wl.seq_lens)), sm_scale(wl.head_dim), out)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("name", list(CASES))
def test_prefill_matches_oracle(name):
    wl, q, cu = _case(name)
    announce(f"prefill fp4 {name} lens={list(wl.seq_lens)} chunks={list(np.diff(cu))} Hq={wl.num_q_heads} "
             f"Hkv={wl.num_kv_heads} d={wl.head_dim}")
    cache = gpu_append("fp4", wl)
    got = _gpu_prefill(wl, q, cu, cache)
    kp, vp = oracle_append("fp4", wl)
    want = O.prefill_attention(FMT_ID["fp4"], kp, vp, wl.num_kv_heads, wl.head_dim, q, np.diff(cu),
                               wl.page_table, wl.seq_lens, sm_scale(wl.head_dim), in_dtype=wl.in_dtype)
    assert_close(got, want, f"prefill {name}")


def test_many_sequences_across_plan_chunks():
    # 600 sequences: the workgroups' plan scans lengths 512 at a time, and orders
    # them by length octave (1 .. 256 tokens here: nine octaves) with the blocks of
    # each sequence last-first; some chunks are empty, some whole sequences
    rng = np.random.default_rng(700)
    B = 600
    lens = np.exp2(rng.uniform(0, 8, B)).astype(np.int64)
    chunks = np.minimum(rng.integers(0, 12, B), lens)
    chunks[rng.random(B) < 0.1] = 0
    whole = rng.random(B) < 0.05
    chunks[whole] = lens[whole]
    wl = W.make_workload("many_seqs", B, 4, 2, 128, lens.tolist(), chunks.tolist(), seed=701)
    q, cu = W.prefill_queries(wl, seed=702)
    announce(f"prefill fp4 many_seqs B={B} lens {int(lens.min())}..{int(lens.max())} Tq={q.shape[0]}")
    cache = gpu_append("fp4", wl)
    got = _gpu_prefill(wl, q, cu, cache)
    kp, vp = oracle_append("fp4", wl)
    want = O.prefill_attention(FMT_ID["fp4"], kp, vp, wl.num_kv_heads, wl.head_dim, q, np.diff(cu),
                               wl.page_table, wl.seq_lens, sm_scale(wl.head_dim), in_dtype=wl.in_dtype)
    assert_close(got, want, "prefill many_seqs")


def test_single_token_chunks_equal_decode():
    wl, q, cu = _case("single_tokens")
    cache = gpu_append("fp4", wl)
    got = _gpu_prefill(wl, q, cu, cache)
    dec = gpu_decode("fp4", wl, cache, q=q)                    # one query per sequence: the same rows
    rel = np.linalg.norm(got - dec) / np.linalg.norm(dec)
    announce(f"prefill of single tokens vs decode: rel-L2 {rel:.2e}")
    assert rel <= 1e-5                                          # float32 sums in another order
