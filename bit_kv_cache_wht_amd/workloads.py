"""Seeded synthetic workloads for the FP4 KV-cache hot path.

This module only draws inputs: Gaussian K/V/q with a few fixed high-magnitude
channels per KV head (the channel-wise key outliers that the rotation is meant
to spread, [review] §2.2 and §3.1), token lengths, and a random page
permutation.  It holds none of the method's arithmetic and is shared by the
tests, the bench and the CPU oracle's callers.

[review] = "[arXiv 2606.20474] UltraQuant: 컨텍스트가 긴 에이전트를 위한 4비트 KV 캐싱"
(manon006.tistory.com/395).

Draw order for a seed (numpy PCG64 main stream): context lengths (ragged
workload only), outlier channels for K then V (per KV head, without
replacement), q values, page permutation.  K and V values come from separate
streams, one per block of 65,536 tokens, seeded with SeedSequence(seed,
spawn_key=(1 for K / 2 for V, block)), so that large workloads can be drawn in
parallel.  All values are float32 standard normals, multiplied by the outlier
factor on the chosen channels and, for bf16 inputs, rounded to the nearest
bf16 (ties to even).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

PAGE_SIZE = 16


@dataclass
class Workload:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    in_dtype: str                 # "bf16" (uint16 bit patterns) or "f32"
    seq_lens: np.ndarray          # [B] tokens in the cache at decode time
    new_lens: np.ndarray          # [B] trailing tokens written by the timed append
    k: np.ndarray                 # [T][H_kv][d], sequences concatenated in order
    v: np.ndarray
    q: np.ndarray                 # [B][H_q][d]
    tok_offsets: np.ndarray       # [B+1] start of each sequence in k/v
    page_table: np.ndarray        # [B][max_pages] int32, unused tail entries 0
    slot_mapping: np.ndarray      # [T] int32 = page * 16 + offset
    num_pages: int
    meta: dict = field(default_factory=dict)

    @property
    def total_tokens(self) -> int:
        return int(self.tok_offsets[-1])

    def new_token_index(self) -> np.ndarray:
        """Indices (into k/v/slot_mapping) of the tokens written by the timed append."""
        idx = [np.arange(self.tok_offsets[b + 1] - self.new_lens[b], self.tok_offsets[b + 1])
               for b in range(self.batch)]
        return np.concatenate(idx) if idx else np.zeros(0, np.int64)

    def prefix_token_index(self) -> np.ndarray:
        idx = [np.arange(self.tok_offsets[b], self.tok_offsets[b + 1] - self.new_lens[b])
               for b in range(self.batch)]
        return np.concatenate(idx) if idx else np.zeros(0, np.int64)


CHUNK = 1 << 16     # tokens per K/V random stream


def _to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Nearest bf16 (ties to even) of finite float32 values, as uint16 bits."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def _draw_kv(seed, which, T, H, d, outlier_ch, factor, in_dtype):
    """[T][H][d] values; token block c comes from its own stream (seed, which, c)."""
    from concurrent.futures import ThreadPoolExecutor
    import os
    out = np.empty((T, H, d), dtype=np.uint16 if in_dtype == "bf16" else np.float32)
    mult = np.ones((H, d), dtype=np.float32)
    for h in range(H):
        mult[h, outlier_ch[h]] = factor

    def block(c):
        t0 = c * CHUNK
        n = min(CHUNK, T - t0)
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(which, c))))
        x = rng.standard_normal((n, H, d), dtype=np.float32)
        x *= mult
        out[t0:t0 + n] = _to_bf16_bits(x) if in_dtype == "bf16" else x

    nblocks = (T + CHUNK - 1) // CHUNK
    workers = max(1, min(16, len(os.sched_getaffinity(0)), nblocks))
    if workers == 1:
        for c in range(nblocks):
            block(c)
    else:
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(block, range(nblocks)))
    return out


def make_workload(name, batch, num_q_heads, num_kv_heads, head_dim, seq_lens, new_lens,
                  in_dtype="bf16", n_outliers=4, outlier_factor=15.0, seed=0,
                  draw_lengths=None) -> Workload:
    """Generic generator.  ``draw_lengths(rng)`` (optional) replaces ``seq_lens`` and
    is called first so that lengths come from the same seed."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if draw_lengths is not None:
        seq_lens, new_lens = draw_lengths(rng)
    seq_lens = np.asarray(seq_lens, dtype=np.int64).reshape(batch)
    new_lens = np.minimum(np.asarray(new_lens, dtype=np.int64).reshape(batch), seq_lens)
    H, d = num_kv_heads, head_dim
    out_k = [rng.choice(d, size=n_outliers, replace=False) for _ in range(H)]
    out_v = [rng.choice(d, size=n_outliers, replace=False) for _ in range(H)]
    tok_offsets = np.concatenate([[0], np.cumsum(seq_lens)]).astype(np.int64)
    T = int(tok_offsets[-1])
    k = _draw_kv(seed, 1, T, H, d, out_k, outlier_factor, in_dtype)
    v = _draw_kv(seed, 2, T, H, d, out_v, outlier_factor, in_dtype)
    q32 = rng.standard_normal((batch, num_q_heads, d), dtype=np.float32)
    q = _to_bf16_bits(q32) if in_dtype == "bf16" else q32
    pages_per_seq = (seq_lens + PAGE_SIZE - 1) // PAGE_SIZE
    num_pages = int(pages_per_seq.sum())
    perm = rng.permutation(num_pages).astype(np.int64)
    max_pages = int(max(1, pages_per_seq.max() if batch else 1))
    page_table = np.zeros((batch, max_pages), dtype=np.int32)
    slot = np.empty(T, dtype=np.int32)
    base = 0
    for b in range(batch):
        n = int(pages_per_seq[b])
        page_table[b, :n] = perm[base:base + n]
        base += n
        pos = np.arange(seq_lens[b])
        slot[tok_offsets[b]:tok_offsets[b + 1]] = page_table[b, pos // PAGE_SIZE] * PAGE_SIZE + pos % PAGE_SIZE
    return Workload(name=name, batch=batch, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                    head_dim=head_dim, in_dtype=in_dtype, seq_lens=seq_lens.astype(np.int32),
                    new_lens=new_lens.astype(np.int32), k=k, v=v, q=q, tok_offsets=tok_offsets,
                    page_table=page_table, slot_mapping=slot, num_pages=max(num_pages, 1),
                    meta=dict(seed=seed, n_outliers=n_outliers, outlier_factor=outlier_factor,
                              outlier_channels_k=[o.tolist() for o in out_k],
                              outlier_channels_v=[o.tolist() for o in out_v]))


def _ragged_lengths(batch, lo, hi, chunk):
    def draw(rng):
        u = rng.uniform(np.log(lo), np.log(hi), size=batch)
        ctx = np.floor(np.exp(u)).astype(np.int64)
        return ctx + chunk, np.full(batch, chunk)
    return draw


# The five named workloads (full sizes); tests build smaller ones of the same
# structure with make_workload.
def tiny(seed=1001):
    """1 sequence, 1 query head / 1 KV head, head_dim 64, context 256, fp32 inputs,
    2 outlier channels x20 on K and V."""
    return make_workload("tiny", 1, 1, 1, 64, [256], [256], in_dtype="f32", n_outliers=2,
                         outlier_factor=20.0, seed=seed)


def append_only(seed=1002, tokens=65536, heads=8):
    """One sequence of 65,536 tokens x 8 KV heads x head_dim 128, bf16, 4 outlier
    channels per head x15, appended from length 0 into 4,096 permuted pages."""
    return make_workload("append_65536x8x128", 1, heads, heads, 128, [tokens], [tokens], seed=seed)


def decode_gqa(seed=1003, batch=64, ctx=8192, new=1):
    """64 sequences x 8,192 context, 64 query heads / 8 KV heads, head_dim 128."""
    return make_workload(f"decode_gqa_{batch}x{ctx}", batch, 64, 8, 128, [ctx] * batch, [new] * batch,
                         seed=seed)


def long_context(seed=1004, batch=8, ctx=65536, new=1):
    """8 sequences x 65,536 context, 64 query heads / 8 KV heads, head_dim 128."""
    return make_workload(f"long_{batch}x{ctx}", batch, 64, 8, 128, [ctx] * batch, [new] * batch,
                         seed=seed)


def ragged(seed=1005, batch=128, lo=1024, hi=131072, chunk=256):
    """128 sequences, context log-uniform in [1,024, 131,072], 32 query / 4 KV heads,
    head_dim 128, plus a 256-token chunk appended per sequence before each decode."""
    return make_workload(f"ragged_{batch}", batch, 32, 4, 128, [0] * batch, [0] * batch, seed=seed,
                         draw_lengths=_ragged_lengths(batch, lo, hi, chunk))


def prefill_queries(wl: Workload, seed: int = 2001):
    """Query rows for chunked prefill over the workload's cache: one row per new
    token of every sequence (its new_lens[b] last positions), [T_q][H_q][d] in the
    workload's input dtype, drawn N(0, 1) from their own stream, and the row
    offsets cu_seqlens_q [B + 1] (int32)."""
    q_lens = np.asarray(wl.new_lens, dtype=np.int64)
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    rng = np.random.Generator(np.random.PCG64([seed, 7]))
    q32 = rng.standard_normal((int(cu[-1]), wl.num_q_heads, wl.head_dim), dtype=np.float32)
    return (_to_bf16_bits(q32) if wl.in_dtype == "bf16" else q32), cu


def rotation_signs(head_dim: int, seed: int = 3001) -> np.ndarray:
    """A sign vector for a randomized-sign Hadamard cache: head_dim values of +1.0
    or -1.0, each -1 with probability 1/2, from their own seeded stream."""
    rng = np.random.Generator(np.random.PCG64([seed, 11]))
    return np.where(rng.integers(0, 2, size=head_dim) == 1, -1.0, 1.0)
