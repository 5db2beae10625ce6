"""Helpers for the GPU parity tests: upload a workload, run libuq through its C ABI,
and build the oracle's expected values from the same seeded inputs (never from
anything the GPU produced)."""
from __future__ import annotations

import sys

import numpy as np

import oracle as O

TOL_REL_L2 = 1e-3      # attention output, relative L2 over the whole tensor
TOL_MAX_ABS = 5e-3     # attention output, max absolute error

FORMATS = ("fp4", "fp8", "bf16")
FMT_ID = {"fp4": O.FMT_FP4, "fp8": O.FMT_FP8, "bf16": O.FMT_BF16}


def announce(msg: str) -> None:
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def torch_mod():
    import torch
    return torch


def dev(arr: np.ndarray, in_dtype: str | None = None):
    """numpy -> CUDA tensor; uint16 arrays holding bf16 bits become bfloat16."""
    torch = torch_mod()
    if in_dtype == "bf16" or (in_dtype is None and arr.dtype == np.uint16):
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def uq():
    import bit_kv_cache_wht_amd as m
    return m


def append_fn(fmt):
    m = uq()
    return {"fp4": m.uq_quantize_append, "fp8": m.uq_append_fp8, "bf16": m.uq_append_bf16}[fmt]


def decode_fn(fmt):
    m = uq()
    return {"fp4": m.uq_decode_attention, "fp8": m.uq_decode_attention_fp8, "bf16": m.uq_decode_attention_bf16}[fmt]


def gpu_cache(fmt, wl, pools=None, k_only=False, signs=None):
    """A zeroed GPU cache for the workload, or one holding the given numpy pools;
    ``k_only`` / ``signs`` select the FP4 rotation variant."""
    m = uq()
    c = m.KvCache.allocate(FMT_ID[fmt], wl.num_pages, wl.num_kv_heads, wl.head_dim, k_only=k_only, signs=signs)
    if pools is not None:
        c.blocks(c.k_pool).copy_(dev(pools[0]))
        c.blocks(c.v_pool).copy_(dev(pools[1]))
    return c


def gpu_append(fmt, wl, cache=None, idx=None, slots=None, flags=0):
    """Writes tokens ``idx`` (default all) with their slots through the C ABI."""
    torch = torch_mod()
    cache = cache if cache is not None else gpu_cache(fmt, wl)
    idx = np.arange(wl.total_tokens) if idx is None else np.asarray(idx)
    sl = wl.slot_mapping[idx] if slots is None else np.asarray(slots, np.int32)
    k, v = dev(wl.k[idx], wl.in_dtype), dev(wl.v[idx], wl.in_dtype)
    append_fn(fmt)(cache, k, v, dev(np.ascontiguousarray(sl, dtype=np.int32)), flags)
    torch.cuda.synchronize()
    return cache


def oracle_append(fmt, wl, idx=None, slots=None, scale_mode="absmax", k_only=False, signs=None):
    kp, vp = O.new_pool(FMT_ID[fmt], wl.num_pages, wl.num_kv_heads, wl.head_dim), \
        O.new_pool(FMT_ID[fmt], wl.num_pages, wl.num_kv_heads, wl.head_dim)
    idx = np.arange(wl.total_tokens) if idx is None else np.asarray(idx)
    sl = wl.slot_mapping[idx] if slots is None else np.asarray(slots, np.int32)
    O.append(FMT_ID[fmt], kp, vp, wl.k[idx], wl.v[idx], sl, in_dtype=wl.in_dtype, scale_mode=scale_mode,
             k_only=k_only, signs=signs)
    return kp, vp


def oracle_threads() -> int:
    """Host threads for the oracle: the cores this process may run on, at most 16
    (a one-GPU share of a GPU host)."""
    import os
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _threaded(fn, items):
    """fn over items on oracle_threads() threads with BLAS held to one thread
    each (numpy releases the interpreter lock inside its array loops)."""
    from concurrent.futures import ThreadPoolExecutor
    import threadpoolctl
    with threadpoolctl.threadpool_limits(1):
        with ThreadPoolExecutor(oracle_threads()) as ex:
            return list(ex.map(fn, items))


def oracle_append_all(fmt, wl, chunk=4096):
    """The oracle's pools holding every token of the workload, from its raw
    inputs.  Chunks of tokens are appended by separate threads into the same
    pools: every byte of a pool belongs to one (slot, head), so the chunks
    write disjoint bytes."""
    kp, vp = O.new_pool(FMT_ID[fmt], wl.num_pages, wl.num_kv_heads, wl.head_dim), \
        O.new_pool(FMT_ID[fmt], wl.num_pages, wl.num_kv_heads, wl.head_dim)

    def one(t0):
        sl = slice(t0, min(t0 + chunk, wl.total_tokens))
        O.append(FMT_ID[fmt], kp, vp, wl.k[sl], wl.v[sl], wl.slot_mapping[sl], in_dtype=wl.in_dtype)

    _threaded(one, range(0, wl.total_tokens, chunk))
    return kp, vp


def oracle_decode_all(fmt, wl, pools, pv_scaled=False):
    """Every output row [B][H_q][d] of the oracle's decode over its pools, the
    (sequence, KV head) pairs on separate threads (``pv_scaled``: the oracle's
    scaled-MFMA PV decode)."""
    B, Hq, d = wl.batch, wl.num_q_heads, wl.head_dim
    G = Hq // wl.num_kv_heads
    out = np.zeros((B, Hq, d))

    def one(pair):
        b, hk = divmod(pair, wl.num_kv_heads)
        rows = [(b, hk * G + g) for g in range(G)]
        out[b, hk * G:(hk + 1) * G] = O.decode_attention_rows(
            FMT_ID[fmt], pools[0], pools[1], wl.num_kv_heads, d, wl.q, wl.page_table, wl.seq_lens, sm_scale(d),
            rows, in_dtype=wl.in_dtype, pv_scaled=pv_scaled)

    _threaded(one, range(B * wl.num_kv_heads))
    return out


def page_blocks_np(cache, pool, idx=None):
    """Pages `idx` (default all) of a device pool as numpy [n][H][block], after
    checking that the bytes past the head blocks of each page (the FP4 page
    padding) are still zero."""
    torch = torch_mod()
    rows = pool if idx is None else pool.index_select(0, torch.from_numpy(np.asarray(idx, np.int64)).cuda())
    a = rows.cpu().numpy()
    blk = uq().uq_head_block_bytes(cache.format, cache.head_dim)
    used = cache.num_kv_heads * blk
    assert not a[:, used:].any(), "bytes past the head blocks of a page were written"
    return np.ascontiguousarray(a[:, :used]).reshape(a.shape[0], cache.num_kv_heads, blk)


def pools_np(cache):
    return page_blocks_np(cache, cache.k_pool), page_blocks_np(cache, cache.v_pool)


def gpu_decode(fmt, wl, cache, flags=0, seq_lens=None, q=None):
    torch = torch_mod()
    m = uq()
    B, Hq, d = wl.batch, wl.num_q_heads, wl.head_dim
    ql = dev(wl.q if q is None else q, wl.in_dtype)
    pt = dev(np.ascontiguousarray(wl.page_table, dtype=np.int32))
    sl = dev(np.ascontiguousarray(wl.seq_lens if seq_lens is None else seq_lens, dtype=np.int32))
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.zeros(m.uq_decode_workspace_bytes(cache, B, Hq, wl.page_table.shape[1]), dtype=torch.uint8,
                     device="cuda")
    decode_fn(fmt)(cache, ql, pt, sl, 1.0 / np.sqrt(d), out, ws, flags=flags)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def sm_scale(d):
    return float(np.float32(1.0 / np.sqrt(d)))


def oracle_decode(fmt, wl, pools, rows=None, seq_lens=None, k_only=False, signs=None, pv_scaled=False, q=None):
    lens = wl.seq_lens if seq_lens is None else seq_lens
    q = wl.q if q is None else q
    if rows is None:
        return O.decode_attention(FMT_ID[fmt], pools[0], pools[1], wl.num_kv_heads, wl.head_dim, q,
                                  wl.page_table, lens, sm_scale(wl.head_dim), in_dtype=wl.in_dtype,
                                  k_only=k_only, signs=signs, pv_scaled=pv_scaled)
    return O.decode_attention_rows(FMT_ID[fmt], pools[0], pools[1], wl.num_kv_heads, wl.head_dim, q,
                                   wl.page_table, lens, sm_scale(wl.head_dim), rows, in_dtype=wl.in_dtype,
                                   k_only=k_only, signs=signs, pv_scaled=pv_scaled)


def oracle_decode_rows_from_inputs(fmt, wl, rows):
    """Expected rows for sampled (b, h) pairs, each built from the raw inputs of
    sequence b and its KV head alone (a private one-head oracle cache)."""
    out = np.zeros((len(rows), wl.head_dim))
    G = wl.num_q_heads // wl.num_kv_heads
    d = wl.head_dim
    cache = {}
    for n, (b, h) in enumerate(rows):
        hk = h // G
        L = int(wl.seq_lens[b])
        if L == 0:
            continue
        if (b, hk) not in cache:
            npg = (L + 15) // 16
            t0 = wl.tok_offsets[b]
            kp, vp = O.new_pool(FMT_ID[fmt], npg, 1, d), O.new_pool(FMT_ID[fmt], npg, 1, d)
            slots = np.arange(L, dtype=np.int32)              # private pages 0..npg-1 in order
            O.append(FMT_ID[fmt], kp, vp, wl.k[t0:t0 + L, hk:hk + 1], wl.v[t0:t0 + L, hk:hk + 1], slots,
                     in_dtype=wl.in_dtype)
            cache = {(b, hk): (kp, vp)}
        kp, vp = cache[(b, hk)]
        qrow = wl.q[b:b + 1, h:h + 1]
        out[n] = O.decode_attention_rows(FMT_ID[fmt], kp, vp, 1, d, qrow, np.arange((L + 15) // 16)[None, :],
                                         np.array([L]), sm_scale(d), [(0, 0)], in_dtype=wl.in_dtype)[0]
    return out


def assert_close(got, want, what=""):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = got - want
    rel = np.linalg.norm(err) / max(np.linalg.norm(want), 1e-30)
    mab = np.abs(err).max() if err.size else 0.0
    announce(f"{what}: rel-L2 {rel:.3e} max-abs {mab:.3e}")
    assert rel <= TOL_REL_L2 and mab <= TOL_MAX_ABS, f"{what}: rel-L2 {rel:.3e} max-abs {mab:.3e}"
    return rel, mab
