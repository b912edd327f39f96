"""tq_attn_decode_static (the decode entry point whose split partials live in
the library's fixed device scratch) against tq_attn_decode with a caller
workspace: two calls in a row through the C ABI, the second on a smaller
input, each compared element by element with the workspace call (same
kernels and split plan, so the results are identical)."""
import numpy as np
import pytest
import torch

import workloads
from compressed_attention_turboquant_amd import binding as B
from tests import harness as H

pytestmark = pytest.mark.gpu

CALLS = [
    ("haar d128 QJL, 4 x 8 KV heads x 5000 keys", workloads.CONFIGS["C3"].with_(B=4, N=5000, dist="normal"), True),
    ("haar d128 QJL, 1 x 8 KV heads x 777 keys", workloads.CONFIGS["C3"].with_(B=1, N=777, dist="normal"), False),
]


def test_static_scratch_decode_matches_workspace_decode():
    for i, (name, cfg, want_scores) in enumerate(CALLS):
        H.log(f"[static scratch decode] call {i}: {name}")
        cap = (cfg.N + 7) // 8 * 8
        S = cfg.B * cfg.Hkv
        packed = workloads.random_packed_numpy(cfg, S, cap, seed=30 + i)
        layer = H.gpu_layer(cfg)
        K, V = H.upload_packed(layer, cfg, packed, S, cap)
        q = torch.from_numpy(workloads.q_numpy(cfg, seed=30 + i)).cuda()
        need = B.decode_workspace_bytes(layer, cfg.B, cfg.Hq, cfg.Hkv, cfg.Tq, cfg.N)
        assert 0 < need <= B.DECODE_STATIC_SCRATCH_BYTES
        ref_out, ref_scores = B.attn_decode(layer, q, K, V, cfg.N, cfg.Hkv, cfg.causal, want_scores=want_scores)
        out = torch.full_like(ref_out, float("nan"))
        scores = torch.full_like(ref_scores, float("nan")) if want_scores else None
        B.attn_decode_static(layer, q, K, V, cfg.N, cfg.Hkv, cfg.causal, out=out, scores=scores)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"call {i}: output differs by {float((out - ref_out).abs().max()):.3e}"
        if want_scores:
            assert torch.equal(scores, ref_scores), f"call {i}: scores differ"
        assert np.isfinite(out.cpu().numpy()).all()
        H.log(f"  identical to the workspace call ({need} bytes of scratch used)")
