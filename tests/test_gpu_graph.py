"""Stream capture of the hot path into a HIP graph.

The quantize, decode and dequantize calls allocate nothing, wait for nothing
and record no memset, so one stream capture of (quantize K, quantize V,
decode, dequantize K and V) must replay to the same bytes as the same calls
made eagerly.  Each replay runs after eager work on the same buffers (the
outputs are cleared and a differently seeded decode runs in between), and
every replay is compared with the eager results: packed caches and norms byte
for byte, the attention output and the reconstructed rows exactly (the kernels
are deterministic).
"""
import numpy as np
import pytest
import torch

import workloads
from compressed_attention_turboquant_amd import binding as B
from tests import harness as H

pytestmark = pytest.mark.gpu

CASES = {
    "haar d128 keys with QJL": workloads.CONFIGS["C3"].with_(B=1, N=777),
    "hadamard d256": workloads.CONFIGS["C5"].with_(B=1, N=515),
    "haar d128 causal 16 query tokens": workloads.CONFIGS["C4"].with_(B=1, N=600),
}


def _snapshot(cache):
    return {k: v.clone() for k, v in cache.arrays.items() if v is not None}


def _clear(cache):
    for v in cache.arrays.values():
        if v is not None:
            v.zero_()


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replays_match_eager(name):
    cfg = CASES[name]
    dev = torch.device("cuda:0")
    S, cap, d, N = cfg.B * cfg.Hkv, cfg.cap, cfg.d, cfg.N
    H.log(f"[graph] {name}")
    xk = workloads.kv_torch(cfg, 3, "K", dev).view(S, cap, d)[:, :N].contiguous()
    xv = workloads.kv_torch(cfg, 3, "V", dev).view(S, cap, d)[:, :N].contiguous()
    q = workloads.q_torch(cfg, 3, dev)
    q_other = workloads.q_torch(cfg, 4, dev)
    layer = H.gpu_layer(cfg)
    K = B.Cache(layer, B.TQ_KEYS, S, cap)
    V = B.Cache(layer, B.TQ_VALUES, S, cap)
    out = torch.empty((cfg.B, cfg.Hq, cfg.Tq, d), dtype=torch.float32, device=dev)
    ws = torch.zeros(max(B.decode_workspace_bytes(layer, cfg.B, cfg.Hq, cfg.Hkv, cfg.Tq, N), 1),
                     dtype=torch.uint8, device=dev)
    xk_hat = torch.empty((S, N, d), dtype=torch.float32, device=dev)
    xv_hat = torch.empty((S, N, d), dtype=torch.float16, device=dev)

    def step():
        B.quantize_kv(layer, B.TQ_KEYS, xk, K)
        B.quantize_kv(layer, B.TQ_VALUES, xv, V)
        B.attn_decode(layer, q, K, V, N, cfg.Hkv, cfg.causal, out=out, workspace=ws)
        B.dequantize(layer, B.TQ_KEYS, K, N, out=xk_hat)
        B.dequantize(layer, B.TQ_VALUES, V, N, out=xv_hat)

    step()
    torch.cuda.synchronize()
    ref_k, ref_v, ref_out = _snapshot(K), _snapshot(V), out.clone()
    ref_xk, ref_xv = xk_hat.clone(), xv_hat.clone()

    # Capture on a side stream (torch's graph capture requires one).
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for replay in range(3):
        # Eager work on the same buffers between replays.
        _clear(K)
        _clear(V)
        out.fill_(float("nan"))
        B.quantize_kv(layer, B.TQ_KEYS, xk, K)
        B.quantize_kv(layer, B.TQ_VALUES, xv, V)
        B.attn_decode(layer, q_other, K, V, N, cfg.Hkv, cfg.causal, out=out, workspace=ws)
        _clear(K)
        _clear(V)
        out.zero_()
        xk_hat.zero_()
        xv_hat.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for key, t in ref_k.items():
            assert torch.equal(K.arrays[key], t), f"{name}: replay {replay}: K {key} differs"
        for key, t in ref_v.items():
            assert torch.equal(V.arrays[key], t), f"{name}: replay {replay}: V {key} differs"
        assert torch.equal(out, ref_out), (
            f"{name}: replay {replay}: output differs by "
            f"{float((out - ref_out).abs().max()):.3e}")
        assert torch.equal(xk_hat, ref_xk), f"{name}: replay {replay}: dequantized keys differ"
        assert torch.equal(xv_hat, ref_xv), f"{name}: replay {replay}: dequantized values differ"
        H.log(f"  replay {replay}: caches, output and dequantized rows identical to the eager calls")
    assert np.isfinite(ref_out.cpu().numpy()).all()
