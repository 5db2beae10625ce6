"""CPU checks of the Python binding's argument checks: every tensor the library
would read or write must have the shape and dtype the C call assumes (a
mismatch there would turn into an out-of-bounds device access), and must live
on the GPU.  The tensors here are CPU tensors, so every call stops in the
binding before the library is called."""
import pytest
import torch

import bit_kv_cache_wht_amd as uq

H, D = 2, 128


def cache(fmt=uq.UQ_KV_FP4, pages=8):
    c = uq.KvCache(fmt, pages, H, D, None, None)
    pb = uq.uq_page_bytes(c)
    c.k_pool = torch.zeros((pages, pb), dtype=torch.uint8)
    c.v_pool = torch.zeros((pages, pb), dtype=torch.uint8)
    return c


def kv(T=5, dtype=torch.bfloat16, h=H, d=D):
    return torch.zeros((T, h, d), dtype=dtype)


def slots(T=5, dtype=torch.int32):
    return torch.zeros(T, dtype=dtype)


def on_gpu_error():
    return pytest.raises(ValueError, match="must be a GPU tensor")


def test_append_checks():
    c = cache()
    with pytest.raises(TypeError, match="v_new is"):
        uq.uq_quantize_append(c, kv(), kv(dtype=torch.float32), slots())
    with pytest.raises(TypeError, match="v_new is"):
        uq.uq_quantize_append(c, kv(dtype=torch.float32), kv(), slots())
    with pytest.raises(TypeError):
        uq.uq_quantize_append(c, kv(dtype=torch.float16), kv(dtype=torch.float16), slots())
    with pytest.raises(ValueError, match="k_new: shape"):
        uq.uq_quantize_append(c, kv(h=3), kv(h=3), slots())
    with pytest.raises(ValueError, match="k_new: shape"):
        uq.uq_quantize_append(c, kv(d=64), kv(d=64), slots())
    with pytest.raises(ValueError, match="v_new: shape"):
        uq.uq_quantize_append(c, kv(T=5), kv(T=4), slots())
    with pytest.raises(ValueError, match="slot_mapping: shape"):
        uq.uq_quantize_append(c, kv(), kv(), slots(T=4))
    with pytest.raises(TypeError, match="slot_mapping: dtype"):
        uq.uq_quantize_append(c, kv(), kv(), slots(dtype=torch.int64))
    small = cache()
    small.v_pool = small.v_pool[:4]
    with pytest.raises(ValueError, match="v_pool"):
        uq.uq_append_fp8(small, kv(), kv(), slots())
    with on_gpu_error():
        uq.uq_append_bf16(cache(uq.UQ_KV_BF16), kv(), kv(), slots())


def test_query_checks():
    q = torch.zeros((7, D), dtype=torch.bfloat16)
    with pytest.raises(TypeError, match="q_fp8: dtype"):
        uq.uq_rotate_quantize_query(q, torch.zeros((7, D), dtype=torch.int8))
    with pytest.raises(ValueError, match="q_fp8: shape"):
        uq.uq_rotate_quantize_query(q, torch.zeros((6, D), dtype=torch.uint8))
    with pytest.raises(ValueError, match="dimensions"):
        uq.uq_rotate_quantize_query(q.reshape(7, 2, 64), torch.zeros((7, D), dtype=torch.uint8))
    with on_gpu_error():
        uq.uq_rotate_quantize_query(q, torch.zeros((7, D), dtype=torch.uint8))


def decode_args(B=3, Hq=8, P=4, qdt=torch.bfloat16):
    return dict(q=torch.zeros((B, Hq, D), dtype=qdt), page_table=torch.zeros((B, P), dtype=torch.int32),
                seq_lens=torch.zeros(B, dtype=torch.int32), sm_scale=0.1,
                out=torch.zeros((B, Hq, D), dtype=torch.float32), workspace=torch.zeros(1 << 20, dtype=torch.uint8))


@pytest.mark.parametrize("fn,fmt", [(uq.uq_decode_attention, uq.UQ_KV_FP4),
                                    (uq.uq_decode_attention_fp8, uq.UQ_KV_FP8),
                                    (uq.uq_decode_attention_bf16, uq.UQ_KV_BF16)])
def test_decode_checks(fn, fmt):
    c = cache(fmt)

    def bad(**kw):
        a = decode_args()
        a.update(kw)
        return a

    with pytest.raises(TypeError, match="page_table: dtype"):
        fn(c, **bad(page_table=torch.zeros((3, 4), dtype=torch.int64)))
    with pytest.raises(ValueError, match="page_table: shape"):
        fn(c, **bad(page_table=torch.zeros((2, 4), dtype=torch.int32)))
    with pytest.raises(TypeError, match="seq_lens: dtype"):
        fn(c, **bad(seq_lens=torch.zeros(3, dtype=torch.int64)))
    with pytest.raises(ValueError, match="seq_lens: shape"):
        fn(c, **bad(seq_lens=torch.zeros(4, dtype=torch.int32)))
    with pytest.raises(ValueError, match="q shape"):
        fn(c, **bad(q=torch.zeros((3, 8, 64), dtype=torch.bfloat16)))
    with pytest.raises(TypeError, match="out: dtype"):
        fn(c, **bad(out=torch.zeros((3, 8, D), dtype=torch.float16)))
    with pytest.raises(ValueError, match="out: shape"):
        fn(c, **bad(out=torch.zeros((3, 7, D), dtype=torch.float32)))
    with on_gpu_error():
        fn(c, **decode_args())


def test_fused_step_checks():
    c = cache()
    a = decode_args()
    with pytest.raises(TypeError, match="k_new is"):
        uq.uq_append_decode_attention(c, kv(T=3, dtype=torch.float32), kv(T=3), **a)
    with pytest.raises(ValueError, match="v_new: shape"):
        uq.uq_append_decode_attention(c, kv(T=3), kv(T=2), **a)
    with on_gpu_error():
        uq.uq_append_decode_attention(c, kv(T=3), kv(T=3), **a)


def test_prefill_checks():
    c = cache()
    B, Tq, Hq = 3, 10, 8
    ok = dict(q=torch.zeros((Tq, Hq, D), dtype=torch.bfloat16), cu_seqlens_q=torch.zeros(B + 1, dtype=torch.int32),
              page_table=torch.zeros((B, 4), dtype=torch.int32), seq_lens=torch.zeros(B, dtype=torch.int32),
              sm_scale=0.1, out=torch.zeros((Tq, Hq, D), dtype=torch.float32))

    def bad(**kw):
        a = dict(ok)
        a.update(kw)
        return a

    with pytest.raises(ValueError, match="cu_seqlens_q: shape"):
        uq.uq_prefill_attention(c, **bad(cu_seqlens_q=torch.zeros(B, dtype=torch.int32)))
    with pytest.raises(TypeError, match="cu_seqlens_q: dtype"):
        uq.uq_prefill_attention(c, **bad(cu_seqlens_q=torch.zeros(B + 1, dtype=torch.int64)))
    with pytest.raises(ValueError, match="page_table: shape"):
        uq.uq_prefill_attention(c, **bad(page_table=torch.zeros((B + 1, 4), dtype=torch.int32)))
    with pytest.raises(ValueError, match="out: shape"):
        uq.uq_prefill_attention(c, **bad(out=torch.zeros((Tq - 1, Hq, D), dtype=torch.float32)))
    with on_gpu_error():
        uq.uq_prefill_attention(c, **ok)


def test_stream_read_checks():
    with on_gpu_error():
        uq.uq_stream_read(torch.zeros(64, dtype=torch.int32), torch.zeros(1, dtype=torch.int32))
    with pytest.raises(ValueError, match="sink"):
        uq.uq_stream_read(torch.zeros(64, dtype=torch.int32), torch.zeros(0, dtype=torch.int32))
