"""GPU parity at the five layer configurations' full sizes, sampled.

Each test builds the whole layer on the device exactly as bench.py does (same
generator, same calls, same launch configuration: quantize all keys, quantize
all values, decode without scores), then checks sampled (batch, KV head)
sequences one by one against the fp64 oracle, which encodes the same raw
inputs itself and decodes from its own codes:
  * codes bit-exact outside the 1e-5 boundary band, for every token of the
    sampled sequences, keys and values;
  * sign bits, norms and residual norms of those keys (rows whose codes
    differ inside the band against the residual recomputed from the GPU's
    codes);
  * the attention output of every query row reading those sequences, within
    2e-3, and the scores of those rows, from a second decode call with the
    scores output on -- both against the oracle's decode of the cache the GPU
    wrote (validated codes and signs, the oracle's norms and gammas), every
    key included;
  * the dequantized rows of those sequences, keys and values, into the
    input's dtype (as the bench step writes them), and for keys with QJL the
    two-stage reconstruction: against the oracle's reconstruction of the same
    fields, to 2e-6 of the norm for fp32 rows and to the fp16 rounding plus
    1.1e-4 (MSE) or 2e-4 (two-stage) of the norm for fp16 rows.
"""
import numpy as np
import pytest
import torch

import workloads
from compressed_attention_turboquant_amd import binding as B
from oracle import attention, codec
from tests import harness as H

pytestmark = pytest.mark.gpu


def _sampled_sequences(cfg):
    S = cfg.B * cfg.Hkv
    picks = {0, S - 1, (S * 5) // 11}
    return sorted(picks)


def _seq_key_codes(cache, s, cap, N, d, bits):
    rb = d * bits // 8
    raw = cache["idx"][s * cap * rb:(s * cap + N) * rb].cpu().numpy().reshape(N, rb)
    return codec.unpack_key_codes(raw, bits, d)


def _seq_signs(cache, s, cap, N, d):
    rb = d // 8
    raw = cache["sign"][s * cap * rb:(s * cap + N) * rb].cpu().numpy().reshape(N, rb)
    return codec.unpack_key_codes(raw, 1, d) == 1


def _seq_value_codes(cache, s, cap, N, d, bits):
    tb = d * bits                                  # bytes per 8-token tile
    raw = cache["idx"][s * (cap // 8) * tb:(s + 1) * (cap // 8) * tb].cpu().numpy()
    return codec.unpack_value_codes(raw, bits, 1, cap, d)[0, :N]


def _check_rows(got, ref, norm, half, extra, what):
    """Largest error of dequantized rows against the oracle's, as a fraction
    of the norm beyond what the output dtype allows."""
    scale = np.maximum(norm[:, None], 1e-30)
    if half:
        over = (np.abs(got - ref) - 2.0 ** -11 * np.abs(ref) - 2.0 ** -25) / scale
        assert over.max() <= extra, f"{what}: fp16 rows off by {over.max():.2e} of the norm beyond rounding"
        return over.max()
    err = np.abs(got - ref) / scale
    assert err.max() < 2e-6, f"{what}: error {err.max():.2e} of the norm"
    return err.max()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["C1", "C2", "C3", "C4", "C5"])
def test_full_size_sampled(name):
    cfg = workloads.CONFIGS[name]
    dev = torch.device("cuda:0")
    S, cap, d, N, G = cfg.B * cfg.Hkv, cfg.cap, cfg.d, cfg.N, cfg.G
    H.log(f"[full size] {name}: {S} sequences x {N} tokens, d={d}")
    Kx = workloads.kv_torch(cfg, 0, "K", dev)
    Vx = workloads.kv_torch(cfg, 0, "V", dev)
    q = workloads.q_torch(cfg, 0, dev)
    layer = H.gpu_layer(cfg)
    ol = H.OracleLayer(cfg)
    Kc = B.Cache(layer, B.TQ_KEYS, S, cap)
    Vc = B.Cache(layer, B.TQ_VALUES, S, cap)
    B.quantize_kv(layer, B.TQ_KEYS, Kx.view(S, cap, d), Kc)
    B.quantize_kv(layer, B.TQ_VALUES, Vx.view(S, cap, d), Vc)
    out, _ = B.attn_decode(layer, q, Kc, Vc, N, cfg.Hkv, cfg.causal)
    _, scores = B.attn_decode(layer, q, Kc, Vc, N, cfg.Hkv, cfg.causal, want_scores=True)
    torch.cuda.synchronize()
    Sk = ol.S if cfg.k_qjl else None
    worst_rel, worst_out = 0.0, 0.0
    fields = {}
    for s in _sampled_sequences(cfg):
        b, h = divmod(s, cfg.Hkv)
        H.log(f"  sequence {s} (batch {b}, KV head {h})")
        xk = Kx[b, h, :N].double().cpu().numpy()
        xv = Vx[b, h, :N].double().cpu().numpy()
        ek = codec.encode_rows(xk, ol.R, ol.ck, ol.bk, Sk)
        ev = codec.encode_rows(xv, ol.R, ol.cv, ol.bv)

        if cfg.k_qjl:
            kf, st = H.check_keys(_seq_key_codes(Kc, s, cap, N, d, cfg.k_bits), Kc["norm"][s * cap:s * cap + N].cpu().numpy(),
                                  ek, ol, f"{name} K s={s}", _seq_signs(Kc, s, cap, N, d),
                                  Kc["rnorm"][s * cap:s * cap + N].cpu().numpy())
        else:
            kf, st = H.check_keys(_seq_key_codes(Kc, s, cap, N, d, cfg.k_bits), Kc["norm"][s * cap:s * cap + N].cpu().numpy(),
                                  ek, ol, f"{name} K s={s}")
        vf, vflips = H.check_values(_seq_value_codes(Vc, s, cap, N, d, cfg.v_bits),
                                    Vc["norm"][s * cap:s * cap + N].cpu().numpy(), ev, ol, f"{name} V s={s}")
        assert st["code_rows"] < 0.01 * N and vflips < 0.01 * N
        cache = H.oracle_cache(kf, vf, 1, 1, N, d)
        qs = q[b:b + 1, h * G:(h + 1) * G].cpu().numpy()            # the G query heads of KV head h
        ref_out, ref_scores = attention.decode(qs, ol.R, ol.S, ol.ck, ol.cv, cache, N, bool(cfg.causal))
        worst_out = max(worst_out, H.compare_out(out[b:b + 1, h * G:(h + 1) * G].cpu().numpy(), ref_out,
                                                 f"{name} out s={s}"))
        scale = H.score_scale(qs, ol.R, ol.S, ol.ck, cache, N, G, cfg.k_qjl)
        gs = scores[b:b + 1, h * G:(h + 1) * G].cpu().numpy()
        worst_rel = max(worst_rel, H.compare_scores(gs, ref_scores, scale, f"{name} scores s={s}"))
        H.log(f"    keys with a band code difference {st['code_rows']}, with a band sign difference "
              f"{st['sign_rows']}; values with a band code difference {vflips}")
        fields[s] = (kf, vf)
    H.log(f"  worst score rel {worst_rel:.2e}, worst out abs {worst_out:.2e}")

    half = cfg.dtype == "f16"
    xhat = torch.empty((S, N, d), dtype=torch.float16 if half else torch.float32, device=dev)
    runs = [("K", B.TQ_KEYS, Kc, False), ("V", B.TQ_VALUES, Vc, False)]
    if cfg.k_qjl:
        runs.append(("K two-stage", B.TQ_KEYS, Kc, True))
    for what, which, cache, prod in runs:
        B.dequantize(layer, which, cache, N, out=xhat, prod=prod)
        torch.cuda.synchronize()
        worst = 0.0
        for s, (kf, vf) in fields.items():
            f = kf if which == B.TQ_KEYS else vf
            c = ol.ck if which == B.TQ_KEYS else ol.cv
            ref = (codec.reconstruct_prod(f["idx"], f["norm"], f["sign"], f["rnorm"], ol.R, c, ol.S) if prod
                   else codec.reconstruct_mse(f["idx"], f["norm"], ol.R, c, dither=f.get("dither")))
            got = xhat[s].double().cpu().numpy()
            worst = max(worst, _check_rows(got, ref, f["norm"], half, 2e-4 if prod else 1.1e-4,
                                           f"{name} dequantize {what} s={s}"))
        H.log(f"  dequantize {what}: worst {worst:.2e} of the norm" + (" beyond fp16 rounding" if half else ""))
