"""ctypes binding of libuq (include/uq.h).  Argument marshalling only."""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

UQ_OK, UQ_ERR_INVALID_ARG, UQ_ERR_UNSUPPORTED, UQ_ERR_WORKSPACE, UQ_ERR_HIP = 0, -1, -2, -3, -4
UQ_KV_FP4, UQ_KV_FP8, UQ_KV_BF16 = 0, 1, 2
UQ_IN_BF16, UQ_IN_F32 = 0, 1
UQ_PAGE_SIZE = 16
UQ_FLAG_OUT_ROTATED = 1
UQ_FLAG_SCALE_CONSTOPT = 2
UQ_FLAG_CHECK = 4
UQ_FLAG_PV_SCALED = 8
UQ_CHECK_BAD_LEN, UQ_CHECK_BAD_PAGE = 1, 2
UQ_ROT_K_ONLY = 1
UQ_ROT_SIGNS = 2

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libuq.so")


class UqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        detail = ""
        if status == UQ_ERR_HIP:
            detail = f" (hipError {uq_last_hip_error()})"
        super().__init__(f"{fn} failed: {uq_status_string(status)} [{status}]{detail}")
        self.status = status


class _Cache(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("num_pages", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
                ("rotation", ctypes.c_uint32), ("rotation_signs", ctypes.c_uint32 * 4)]


_P = ctypes.c_void_p
_I = ctypes.c_int32
_U = ctypes.c_uint32
_SZ = ctypes.c_size_t
_CP = ctypes.POINTER(_Cache)

_SIGS = {
    "uq_head_block_bytes": (_SZ, [_I, _I]),
    "uq_page_bytes": (_SZ, [_CP]),
    "uq_quantize_append": (ctypes.c_int, [_CP, _P, _P, _I, _P, _I, _U, _P]),
    "uq_append_fp8": (ctypes.c_int, [_CP, _P, _P, _I, _P, _I, _U, _P]),
    "uq_append_bf16": (ctypes.c_int, [_CP, _P, _P, _I, _P, _I, _U, _P]),
    "uq_rotate_quantize_query": (ctypes.c_int, [_P, _I, _P, _I, _I, _P]),
    "uq_rotate_quantize_query_cache": (ctypes.c_int, [_CP, _P, _I, _P, _I, _P]),
    "uq_decode_workspace_bytes": (_SZ, [_CP, _I, _I, _I]),
    "uq_decode_attention": (ctypes.c_int, [_CP, _P, _I, _P, _I, _P, _I, _I, ctypes.c_float, _P, _P, _SZ, _U, _P]),
    "uq_decode_attention_noalloc": (ctypes.c_int, [_CP, _P, _I, _P, _I, _P, _I, _I, ctypes.c_float, _P, _U, _P]),
    "uq_append_decode_attention": (ctypes.c_int, [_CP, _P, _P, _P, _I, _P, _I, _P, _I, _I, ctypes.c_float, _P, _P, _SZ,
                                                  _U, _P]),
    "uq_decode_attention_fp8": (ctypes.c_int, [_CP, _P, _I, _P, _I, _P, _I, _I, ctypes.c_float, _P, _P, _SZ, _U, _P]),
    "uq_decode_attention_bf16": (ctypes.c_int, [_CP, _P, _I, _P, _I, _P, _I, _I, ctypes.c_float, _P, _P, _SZ, _U, _P]),
    "uq_profile_next_decode": (ctypes.c_int, [_P, _P]),
    "uq_profile_next_decode_clock": (ctypes.c_int, [_P, _P]),
    "uq_stream_read": (ctypes.c_int, [_P, _SZ, _P, _P]),
    "uq_prefill_attention": (ctypes.c_int, [_CP, _P, _I, _P, _I, _P, _I, _P, _I, _I, ctypes.c_float, _P, _U, _P]),
    "uq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "uq_last_hip_error": (ctypes.c_int, []),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libuq.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m bit_kv_cache_wht_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(h, name)
            f.restype, f.argtypes = res, args
        _lib = h
    return _lib


@dataclass
class KvCache:
    """Descriptor of a paged K/V cache; pools are caller-owned uint8 device tensors
    of shape [num_pages][uq_page_bytes], a page being its head blocks back to back
    (``blocks`` views them as [num_pages][block position][block]; FP4 pages hold
    KV head h at position (h + 2 page) mod num_kv_heads, see include/uq.h)."""
    format: int
    num_pages: int
    num_kv_heads: int
    head_dim: int
    k_pool: object
    v_pool: object
    rotation: int = 0                        # UQ_ROT_* bits
    rotation_signs: tuple = (0, 0, 0, 0)     # sign bits of s (UQ_ROT_SIGNS)

    @classmethod
    def allocate(cls, fmt: int, num_pages: int, num_kv_heads: int, head_dim: int, device="cuda", zero=True,
                 k_only=False, signs=None):
        """Zeroed pools for a new cache.  FP4 only: ``k_only`` leaves V unrotated
        (UQ_ROT_K_ONLY); ``signs`` (head_dim values of +1 / -1) makes the rotation
        c_d H diag(signs) (UQ_ROT_SIGNS)."""
        import torch
        blk = uq_head_block_bytes(fmt, head_dim)
        if blk == 0:
            raise UqError("uq_head_block_bytes", UQ_ERR_UNSUPPORTED)
        pb = lib().uq_page_bytes(ctypes.byref(_Cache(fmt, num_pages, UQ_PAGE_SIZE, num_kv_heads, head_dim,
                                                      None, None)))
        alloc = torch.zeros if zero else torch.empty
        k = alloc((num_pages, pb), dtype=torch.uint8, device=device)
        v = alloc((num_pages, pb), dtype=torch.uint8, device=device)
        rot, words = (UQ_ROT_K_ONLY if k_only else 0), (0, 0, 0, 0)
        if signs is not None:
            rot |= UQ_ROT_SIGNS
            words = sign_words(signs, head_dim)
        return cls(fmt, num_pages, num_kv_heads, head_dim, k, v, rot, words)

    def blocks(self, pool):
        """[num_pages][num_kv_heads][head block bytes] view of a pool (no copy)."""
        blk = uq_head_block_bytes(self.format, self.head_dim)
        return pool.as_strided((self.num_pages, self.num_kv_heads, blk), (pool.stride(0), blk, 1))

    def c(self) -> _Cache:
        return _Cache(self.format, self.num_pages, UQ_PAGE_SIZE, self.num_kv_heads, self.head_dim,
                      _ptr(self.k_pool), _ptr(self.v_pool), self.rotation, (ctypes.c_uint32 * 4)(*self.rotation_signs))


def sign_words(signs, head_dim: int) -> tuple:
    """The four rotation_signs words for a vector of head_dim signs (+1 / -1):
    bit i % 32 of word i / 32 set where signs[i] is -1."""
    import numpy as np
    s = np.asarray(signs)
    if s.shape != (head_dim,) or not np.all(np.abs(s) == 1):
        raise ValueError("signs must hold head_dim values of +1 or -1")
    words = [0, 0, 0, 0]
    for i in np.nonzero(s < 0)[0]:
        words[int(i) // 32] |= 1 << (int(i) % 32)
    return tuple(words)


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return UQ_IN_BF16
    if t.dtype == torch.float32:
        return UQ_IN_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or float32)")


# Argument checks: every tensor the library reads or writes must have the shape
# and dtype the C call assumes, since a mismatch there becomes an out-of-bounds
# device access.  Shapes and dtypes are checked first and device placement last.
def _need(cond: bool, msg: str, exc=ValueError) -> None:
    if not cond:
        raise exc(msg)


def _shape(t, shape, name: str) -> None:
    _need(tuple(t.shape) == tuple(shape), f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")


def _int32(t, shape, name: str) -> None:
    import torch
    _need(t.dtype == torch.int32, f"{name}: dtype {t.dtype}, expected torch.int32", TypeError)
    _shape(t, shape, name)


def _float32(t, shape, name: str) -> None:
    import torch
    _need(t.dtype == torch.float32, f"{name}: dtype {t.dtype}, expected torch.float32", TypeError)
    _shape(t, shape, name)


def _contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors passed to libuq must be contiguous")


def _on_device(**named) -> None:
    for name, t in named.items():
        if t is not None and not isinstance(t, int) and t.device.type != "cuda":
            raise ValueError(f"{name} must be a GPU tensor (got device {t.device})")


def _cache_ok(cache) -> None:
    """The pools of a cache hold num_pages pages of uq_page_bytes each."""
    need = cache.num_pages * uq_page_bytes(cache)
    _need(need > 0, "invalid cache descriptor")
    pools = {name: getattr(cache, name) for name in ("k_pool", "v_pool")}
    for name, t in pools.items():
        if t is not None and not isinstance(t, int):
            _need(t.numel() * t.element_size() >= need, f"{name}: {t.numel() * t.element_size()} bytes, "
                  f"expected at least {need} (num_pages x uq_page_bytes)")
    _on_device(**pools)


def _check(fn: str, status: int) -> None:
    if status != UQ_OK:
        raise UqError(fn, status)


def uq_status_string(status: int) -> str:
    return lib().uq_status_string(status).decode()


def uq_last_hip_error() -> int:
    return lib().uq_last_hip_error()


def uq_head_block_bytes(fmt: int, head_dim: int) -> int:
    return lib().uq_head_block_bytes(fmt, head_dim)


def uq_page_bytes(cache: KvCache) -> int:
    c = cache.c()
    return lib().uq_page_bytes(ctypes.byref(c))


def _append(name, cache, k_new, v_new, slot_mapping, flags, stream):
    _contig(k_new, v_new, slot_mapping)
    n = int(k_new.shape[0])
    code = _dtype_code(k_new)
    _need(v_new.dtype == k_new.dtype, f"{name}: k_new is {k_new.dtype} but v_new is {v_new.dtype}", TypeError)
    _shape(k_new, (n, cache.num_kv_heads, cache.head_dim), "k_new")
    _shape(v_new, (n, cache.num_kv_heads, cache.head_dim), "v_new")
    _int32(slot_mapping, (n,), "slot_mapping")
    _cache_ok(cache)
    _on_device(k_new=k_new, v_new=v_new, slot_mapping=slot_mapping)
    c = cache.c()
    st = getattr(lib(), name)(ctypes.byref(c), _ptr(k_new), _ptr(v_new), code, _ptr(slot_mapping), n,
                              flags, _stream(stream))
    _check(name, st)


def uq_quantize_append(cache: KvCache, k_new, v_new, slot_mapping, flags: int = 0, stream=None) -> None:
    """FP4 write path; k_new, v_new [T][H_kv][d] bf16/f32, slot_mapping int32 [T]."""
    _append("uq_quantize_append", cache, k_new, v_new, slot_mapping, flags, stream)


def uq_append_fp8(cache: KvCache, k_new, v_new, slot_mapping, flags: int = 0, stream=None) -> None:
    _append("uq_append_fp8", cache, k_new, v_new, slot_mapping, flags, stream)


def uq_append_bf16(cache: KvCache, k_new, v_new, slot_mapping, flags: int = 0, stream=None) -> None:
    _append("uq_append_bf16", cache, k_new, v_new, slot_mapping, flags, stream)


def uq_rotate_quantize_query_cache(cache, q, q_fp8, stream=None) -> None:
    """The query rotation of FP4 cache `cache`, with its rotation variant:
    q [rows][head_dim] bf16/f32 -> q_fp8 uint8 [rows][head_dim]."""
    import torch
    _contig(q, q_fp8)
    code = _dtype_code(q)
    _need(q.dim() == 2 and int(q.shape[1]) == cache.head_dim,
          f"q: shape {tuple(q.shape)}, expected [rows][{cache.head_dim}]")
    rows = int(q.shape[0])
    _need(q_fp8.dtype == torch.uint8, f"q_fp8: dtype {q_fp8.dtype}, expected torch.uint8", TypeError)
    _shape(q_fp8, (rows, cache.head_dim), "q_fp8")
    _on_device(q=q, q_fp8=q_fp8)
    c = cache.c()
    st = lib().uq_rotate_quantize_query_cache(ctypes.byref(c), _ptr(q), code, _ptr(q_fp8), rows, _stream(stream))
    _check("uq_rotate_quantize_query_cache", st)


def uq_rotate_quantize_query(q, q_fp8, stream=None) -> None:
    """q [rows][d] bf16/f32 -> q_fp8 uint8 [rows][d] (E4M3 of the rotated query)."""
    import torch
    _contig(q, q_fp8)
    code = _dtype_code(q)
    _need(q.dim() == 2, f"q: {q.dim()} dimensions, expected [rows][head_dim]")
    rows, d = int(q.shape[0]), int(q.shape[-1])
    _need(q_fp8.dtype == torch.uint8, f"q_fp8: dtype {q_fp8.dtype}, expected torch.uint8", TypeError)
    _shape(q_fp8, (rows, d), "q_fp8")
    _on_device(q=q, q_fp8=q_fp8)
    st = lib().uq_rotate_quantize_query(_ptr(q), code, _ptr(q_fp8), rows, d, _stream(stream))
    _check("uq_rotate_quantize_query", st)


def uq_decode_workspace_bytes(cache: KvCache, num_seqs: int, num_q_heads: int, max_pages_per_seq: int) -> int:
    c = cache.c()
    return lib().uq_decode_workspace_bytes(ctypes.byref(c), num_seqs, num_q_heads, max_pages_per_seq)


def _decode_checks(name, cache, q, page_table, seq_lens, out, workspace, k_new=None, v_new=None):
    """Shapes and dtypes of a decode call's tensors; returns (B, H_q)."""
    _contig(q, page_table, seq_lens, out, workspace, k_new, v_new)
    code = _dtype_code(q)
    _need(q.dim() == 3 and int(q.shape[2]) == cache.head_dim,
          f"{name}: q shape {tuple(q.shape)}, expected [num_seqs][num_q_heads][{cache.head_dim}]")
    B, Hq = int(q.shape[0]), int(q.shape[1])
    _need(page_table.dim() == 2, f"page_table: {page_table.dim()} dimensions, expected [num_seqs][max_pages]")
    _int32(page_table, (B, int(page_table.shape[1])), "page_table")
    _int32(seq_lens, (B,), "seq_lens")
    _float32(out, (B, Hq, cache.head_dim), "out")
    for nm, t in (("k_new", k_new), ("v_new", v_new)):
        if t is not None:
            _need(t.dtype == q.dtype, f"{name}: {nm} is {t.dtype} but q is {q.dtype}", TypeError)
            _shape(t, (B, cache.num_kv_heads, cache.head_dim), nm)
    _cache_ok(cache)
    _on_device(q=q, page_table=page_table, seq_lens=seq_lens, out=out, workspace=workspace, k_new=k_new,
               v_new=v_new)
    return code, B, Hq


def _decode(name, cache, q, page_table, seq_lens, sm_scale, out, workspace, flags, stream):
    code, B, Hq = _decode_checks(name, cache, q, page_table, seq_lens, out, workspace)
    c = cache.c()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = getattr(lib(), name)(ctypes.byref(c), _ptr(q), code, _ptr(page_table), int(page_table.shape[1]),
                              _ptr(seq_lens), B, Hq, float(sm_scale), _ptr(out), _ptr(workspace), ws_bytes, flags,
                              _stream(stream))
    _check(name, st)


def uq_decode_attention(cache, q, page_table, seq_lens, sm_scale, out, workspace, flags=0, stream=None) -> None:
    """FP4 decode: q [B][H_q][d], page_table int32 [B][max_pages], seq_lens int32 [B],
    out float32 [B][H_q][d], workspace uint8 >= uq_decode_workspace_bytes."""
    _decode("uq_decode_attention", cache, q, page_table, seq_lens, sm_scale, out, workspace, flags, stream)


def uq_decode_attention_noalloc(cache, q, page_table, seq_lens, sm_scale, out, flags=0, stream=None) -> None:
    """FP4 decode as uq_decode_attention, with the library's static scratch array as
    its workspace (allocates nothing; calls overlapping in time on one GPU race)."""
    code, B, Hq = _decode_checks("uq_decode_attention_noalloc", cache, q, page_table, seq_lens, out, None)
    c = cache.c()
    st = lib().uq_decode_attention_noalloc(ctypes.byref(c), _ptr(q), code, _ptr(page_table),
                                           int(page_table.shape[1]), _ptr(seq_lens), B, Hq, float(sm_scale),
                                           _ptr(out), flags, _stream(stream))
    _check("uq_decode_attention_noalloc", st)


def uq_append_decode_attention(cache, k_new, v_new, q, page_table, seq_lens, sm_scale, out, workspace, flags=0,
                               stream=None) -> None:
    """Fused FP4 step: writes k_new / v_new [B][H_kv][d] (the dtype of q) at position
    seq_lens[b] - 1 of each sequence, then decodes as uq_decode_attention."""
    code, B, Hq = _decode_checks("uq_append_decode_attention", cache, q, page_table, seq_lens, out, workspace,
                                 k_new, v_new)
    c = cache.c()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().uq_append_decode_attention(ctypes.byref(c), _ptr(k_new), _ptr(v_new), _ptr(q), code,
                                          _ptr(page_table), int(page_table.shape[1]), _ptr(seq_lens), B, Hq,
                                          float(sm_scale), _ptr(out), _ptr(workspace), ws_bytes, flags,
                                          _stream(stream))
    _check("uq_append_decode_attention", st)


def decode_check_word(workspace) -> int:
    """The UQ_FLAG_CHECK error word (UQ_CHECK_* bits) held in the first 4 bytes of a
    decode workspace (synchronizes with the device)."""
    import torch
    return int(workspace[:4].view(torch.int32).item()) & 0xFFFFFFFF


def uq_decode_attention_fp8(cache, q, page_table, seq_lens, sm_scale, out, workspace, flags=0, stream=None) -> None:
    _decode("uq_decode_attention_fp8", cache, q, page_table, seq_lens, sm_scale, out, workspace, flags, stream)


def uq_decode_attention_bf16(cache, q, page_table, seq_lens, sm_scale, out, workspace, flags=0, stream=None) -> None:
    _decode("uq_decode_attention_bf16", cache, q, page_table, seq_lens, sm_scale, out, workspace, flags, stream)


def uq_profile_next_decode(start_event, stop_event) -> None:
    """Record two hipEvent_t handles (ints) around the next decode call's main kernel."""
    _check("uq_profile_next_decode", lib().uq_profile_next_decode(start_event, stop_event))


def uq_profile_next_decode_clock(clocks) -> int:
    """Arm the wall-clock span of the next decode call's main kernel: `clocks` is a
    device tensor of two int64 set to (-1, 0) (the unsigned maximum and zero);
    the kernel leaves (earliest workgroup start, latest workgroup end) there.
    Returns the clock's rate in kHz."""
    _need(clocks is not None and clocks.numel() == 2 and clocks.element_size() == 8, "clocks: two 64-bit integers")
    _on_device(clocks=clocks)
    khz = ctypes.c_int32(0)
    _check("uq_profile_next_decode_clock", lib().uq_profile_next_decode_clock(_ptr(clocks), ctypes.byref(khz)))
    return khz.value


def uq_stream_read(src, sink, stream=None) -> None:
    """Streaming read of the whole tensor `src` (bandwidth reference); XORs the XOR
    of its 32-bit words into the int32 tensor `sink` (one element)."""
    _contig(src, sink)
    _need(sink.numel() * sink.element_size() >= 4, "sink: at least one 32-bit word")
    _on_device(src=src, sink=sink)
    nbytes = src.numel() * src.element_size()
    _check("uq_stream_read", lib().uq_stream_read(_ptr(src), nbytes, _ptr(sink), _stream(stream)))


def uq_prefill_attention(cache, q, cu_seqlens_q, page_table, seq_lens, sm_scale, out, flags=0, stream=None) -> None:
    """Chunked-prefill attention: q [T_q][H_q][d] (bf16/f32), cu_seqlens_q int32
    [B + 1], out float32 [T_q][H_q][d]; each sequence's chunk is its last tokens."""
    _contig(q, cu_seqlens_q, page_table, seq_lens, out)
    code = _dtype_code(q)
    _need(q.dim() == 3 and int(q.shape[2]) == cache.head_dim,
          f"uq_prefill_attention: q shape {tuple(q.shape)}, expected [total_q][num_q_heads][{cache.head_dim}]")
    Tq, Hq = int(q.shape[0]), int(q.shape[1])
    _need(seq_lens.dim() == 1, "seq_lens: expected [num_seqs]")
    B = int(seq_lens.shape[0])
    _int32(seq_lens, (B,), "seq_lens")
    _int32(cu_seqlens_q, (B + 1,), "cu_seqlens_q")
    _need(page_table.dim() == 2, "page_table: expected [num_seqs][max_pages]")
    _int32(page_table, (B, int(page_table.shape[1])), "page_table")
    _float32(out, (Tq, Hq, cache.head_dim), "out")
    _cache_ok(cache)
    _on_device(q=q, cu_seqlens_q=cu_seqlens_q, page_table=page_table, seq_lens=seq_lens, out=out)
    c = cache.c()
    st = lib().uq_prefill_attention(ctypes.byref(c), _ptr(q), code, _ptr(cu_seqlens_q), Tq,
                                    _ptr(page_table), int(page_table.shape[1]), _ptr(seq_lens), B, Hq,
                                    float(sm_scale), _ptr(out), flags, _stream(stream))
    _check("uq_prefill_attention", st)
