"""HIP-graph capture of the serving step: the fused FP4 append + decode and the
plain decode are captured once (torch.cuda.CUDAGraph on the capture stream the
binding passes to the library) and replayed with new query contents written in
place between replays.  Every replay must agree with an eager call on the same
inputs (relative L2 1e-6: the split merge order may differ between launches)
and with the oracle.  The decode needs no clearing between launches: its split
counters return to zero by themselves, so the graph holds kernels only."""
import dataclasses

import numpy as np
import pytest

from bit_kv_cache_wht_amd import workloads as W

from gpu_util import announce, assert_close, dev, gpu_append, gpu_cache, oracle_append, oracle_decode, torch_mod, uq
from test_gpu_fused import _new_rows, _split

pytestmark = pytest.mark.gpu


def _rel_l2(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


@pytest.mark.parametrize("fused", [True, False])
def test_graph_replays_match_eager(fused):
    torch = torch_mod()
    m = uq()
    wl = W.make_workload("graph", 6, 32, 4, 128, [3000, 1500, 700, 64, 2500, 17], [3000, 1500, 700, 64, 2500, 17],
                         seed=321)
    pre, new, has = _split(wl)
    announce(f"graph capture fused={fused} lens={list(wl.seq_lens)}")
    cache = gpu_cache("fp4", wl)
    gpu_append("fp4", wl, cache, idx=pre if fused else None)
    k_new, v_new = _new_rows(wl, new, has)
    kd, vd = dev(k_new, wl.in_dtype), dev(v_new, wl.in_dtype)
    B, Hq, d = wl.batch, wl.num_q_heads, wl.head_dim
    qs = [wl.q] + [W.make_workload("graph_q", B, Hq, 4, d, [1] * B, [1] * B, seed=400 + i).q for i in range(3)]
    q = dev(qs[0], wl.in_dtype)
    pt = dev(np.ascontiguousarray(wl.page_table, dtype=np.int32))
    sl = dev(np.ascontiguousarray(wl.seq_lens, dtype=np.int32))
    out = torch.zeros((B, Hq, d), dtype=torch.float32, device="cuda")
    ws = torch.zeros(m.uq_decode_workspace_bytes(cache, B, Hq, wl.page_table.shape[1]), dtype=torch.uint8,
                     device="cuda")
    scale = float(np.float32(1.0 / np.sqrt(d)))

    def step():
        if fused:
            m.uq_append_decode_attention(cache, kd, vd, q, pt, sl, scale, out, ws)
        else:
            m.uq_decode_attention(cache, q, pt, sl, scale, out, ws)

    step()                                            # warm-up outside the capture (loads the code object)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    pools = oracle_append("fp4", wl)
    for i, qi in enumerate(qs):
        q.copy_(dev(qi, wl.in_dtype))
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        step()                                        # eager on the same inputs
        torch.cuda.synchronize()
        eager = out.cpu().numpy().astype(np.float64)
        assert np.isfinite(got).all(), f"replay {i}"
        assert _rel_l2(got, eager) < 1e-6, f"replay {i}: {_rel_l2(got, eager)}"
        assert_close(got, oracle_decode("fp4", dataclasses.replace(wl, q=qi), pools), f"graph replay {i}")
