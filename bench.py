"""Benchmark of the TurboQuant KV-cache path on one MI355X.

One step = quantize the layer's keys, quantize its values, run decode
attention over the compressed cache, and dequantize both caches (into the
input's dtype), on synthetic inputs already resident in HBM.  The default workload is the Llama-3-8B-shaped layer (batch 16, 32 query
/ 8 KV heads, d=128, 131072 keys, fp16 inputs with per-channel LogNormal(0,
0.5) scales, keys 3-bit MSE + 1-bit QJL, values 3-bit, Haar rotation).

Printed (one JSON line on stdout):
  value              packed-KV bytes read by tq_attn_decode / its duration (GB/s)
  quantize_vectors_per_s   (K rows + V rows) / duration of the two quantize calls
  roofline           decode kernel vs the 8 TB/s HBM peak
  roofline_quantize  quantize kernel vs its bound
  roofline_dequantize  dequantize kernel vs its bound
  cpu_baseline       the fp64 oracle on a bounded sample of the same workload
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tq_attn_decode packed-KV GB/s (% HBM peak) + tq_quantize_kv vectors/sec"
HBM_PEAK_GBS = 8000.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def packed_bytes_per_token(cfg):
    k = cfg.d * cfg.k_bits // 8 + 4 + (cfg.d // 8 + 4 if cfg.k_qjl else 0)
    v = cfg.d * cfg.v_bits // 8 + 4
    return k, v


def traffic_from_profile(kernel_tag, workload, digest, per_launch_units):
    """HBM bytes per launch from committed rocprofv3 counter summaries, or None
    if there are none or the kernels changed since they were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel_tag}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("sources_digest") != digest:
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(cfg, K_dev, V_dev, q_dev, budget_s=8.0):
    """Time the fp64 oracle (as it stands) on a bounded sample of the workload.

    Decode: whole (batch 0, KV head h) sequences, decoded from packed bytes for
    the G query heads that share them, one after another until `budget_s` has
    passed.  Quantize: chunks of 8192 K rows and 8192 V rows taken from the
    sequences in order, until `budget_s` has passed.  Rates are scaled to the
    metric's units (packed-KV GB/s, vectors/s)."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    from oracle import attention, codebook, codec, transforms

    d, N, G = cfg.d, cfg.N, cfg.G
    R = transforms.rotation(d, cfg.rot, cfg.layer_seed)
    S = transforms.gaussian_projection(d, cfg.layer_seed)
    ck, bk = codebook.codebook(cfg.k_bits, d)
    cv, bv = codebook.codebook(cfg.v_bits, d)
    Sk = S if cfg.k_qjl else None
    seqs = [(b, h) for b in range(cfg.B) for h in range(cfg.Hkv)]

    # quantize: 8192-row chunks until the budget is spent
    chunk, nq = 8192, 0
    t_quant = 0.0
    for b, h in seqs:
        for t0 in range(0, N, chunk):
            xk = K_dev[b, h, t0:t0 + chunk].double().cpu().numpy()
            xv = V_dev[b, h, t0:t0 + chunk].double().cpu().numpy()
            t = time.perf_counter()
            codec.encode_rows(xk, R, ck, bk, Sk)
            codec.encode_rows(xv, R, cv, bv)
            t_quant += time.perf_counter() - t
            nq += xk.shape[0]
            if t_quant >= budget_s:
                break
        if t_quant >= budget_s:
            break

    # decode: whole sequences (packed untimed, unpack + decode timed)
    t_dec, nseq = 0.0, 0
    for b, h in seqs:
        xk = K_dev[b, h, :N].double().cpu().numpy()
        xv = V_dev[b, h, :N].double().cpu().numpy()
        q = q_dev[b:b + 1, h * G:(h + 1) * G].double().cpu().numpy()
        ek = codec.encode_rows(xk, R, ck, bk, Sk)
        ev = codec.encode_rows(xv, R, cv, bv)
        packed = {"k_idx": codec.pack_key_codes(ek["idx"], cfg.k_bits), "k_norm": ek["norm"].astype(np.float32),
                  "v_idx": codec.pack_value_codes(ev["idx"].reshape(1, N, d), cfg.v_bits),
                  "v_norm": ev["norm"].astype(np.float32)}
        if cfg.k_qjl:
            packed["k_sign"] = codec.pack_key_codes(ek["sign"].astype(np.int64), 1)
            packed["k_rnorm"] = ek["rnorm"].astype(np.float32)
        t = time.perf_counter()
        cache = attention.unpack_cache(packed, 1, 1, N, d, cfg.k_bits, cfg.v_bits, cfg.k_qjl)
        attention.decode(q, R, S, ck, cv, cache, N, bool(cfg.causal))
        t_dec += time.perf_counter() - t
        nseq += 1
        if t_dec >= budget_s:
            break
    kb, vb = packed_bytes_per_token(cfg)
    return {
        "value": round((kb + vb) * N * nseq / t_dec / 1e9, 4),
        "unit": "GB/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": f"decode of {nseq} of {len(seqs)} (batch, KV head) sequences ({G * cfg.Tq} query rows x "
                  f"{N} keys each, unpacked from packed bytes) in {t_dec:.2f} s; quantize of {nq} K + "
                  f"{nq} V rows in {t_quant:.2f} s",
        "quantize_vectors_per_s": round(2 * nq / t_quant, 1),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="C3")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, run a plain 1 GiB device copy (reference for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported (the path is "
              "measured on one GPU's share of the sequences)", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads
    from compressed_attention_turboquant_amd import binding as B
    from compressed_attention_turboquant_amd.profsummary import kernel_sources_digest

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    cfg = workloads.CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    S, cap, d = cfg.B * cfg.Hkv, cfg.cap, cfg.d
    log(f"workload {cfg.name}: generating K, V ({2 * S * cap * d * (2 if cfg.dtype == 'f16' else 4) / 1e9:.1f} GB)")
    Kx = workloads.kv_torch(cfg, 0, "K", dev)
    Vx = workloads.kv_torch(cfg, 0, "V", dev)
    q = workloads.q_torch(cfg, 0, dev)
    rot = B.TQ_ROT_HAAR if cfg.rot == "haar" else B.TQ_ROT_HADAMARD
    layer = B.make_rotation(d, rot, cfg.layer_seed, cfg.k_bits, cfg.k_qjl, cfg.v_bits)
    Kc = B.Cache(layer, B.TQ_KEYS, S, cap)
    Vc = B.Cache(layer, B.TQ_VALUES, S, cap)
    xk = Kx.view(S, cap, d)[:, : cfg.N] if cap == cfg.N else Kx.view(S, cap, d)[:, : cfg.N].contiguous()
    xv = Vx.view(S, cap, d)[:, : cfg.N] if cap == cfg.N else Vx.view(S, cap, d)[:, : cfg.N].contiguous()
    out = torch.empty((cfg.B, cfg.Hq, cfg.Tq, d), dtype=torch.float32, device=dev)
    ws = torch.empty(max(B.decode_workspace_bytes(layer, cfg.B, cfg.Hq, cfg.Hkv, cfg.Tq, cfg.N), 1),
                     dtype=torch.uint8, device=dev)
    xhat = torch.empty((S, cfg.N, d), dtype=torch.float16 if cfg.dtype == "f16" else torch.float32, device=dev)

    def step(ev=None):
        if ev: ev[0].record(stream)
        B.quantize_kv(layer, B.TQ_KEYS, xk, Kc)
        if ev: ev[1].record(stream)
        B.quantize_kv(layer, B.TQ_VALUES, xv, Vc)
        if ev: ev[2].record(stream)
        B.attn_decode(layer, q, Kc, Vc, cfg.N, cfg.Hkv, cfg.causal, out=out, workspace=ws)
        if ev: ev[3].record(stream)
        B.dequantize(layer, B.TQ_KEYS, Kc, cfg.N, out=xhat)
        B.dequantize(layer, B.TQ_VALUES, Vc, cfg.N, out=xhat)
        if ev: ev[4].record(stream)

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    qk_ms = sum(e[0].elapsed_time(e[1]) for e in events) / args.steps
    qv_ms = sum(e[1].elapsed_time(e[2]) for e in events) / args.steps
    dec_ms = sum(e[2].elapsed_time(e[3]) for e in events) / args.steps
    dq_ms = sum(e[3].elapsed_time(e[4]) for e in events) / args.steps
    kb, vb = packed_bytes_per_token(cfg)
    rows = cfg.B * cfg.Hkv * cfg.N
    packed = (kb + vb) * rows
    dec_gbs = packed / (dec_ms * 1e-3) / 1e9
    vec_s = 2 * rows / ((qk_ms + qv_ms) * 1e-3)
    in_bytes = 2 if cfg.dtype == "f16" else 4
    q_bytes = rows * (d * in_bytes * 2) + packed            # fp16 K and V in, packed cache out
    q_gbs = q_bytes / ((qk_ms + qv_ms) * 1e-3) / 1e9
    # dequantize: codes and norm in, rows of the input's dtype out, for K and V
    dq_bytes = rows * (d * (cfg.k_bits + cfg.v_bits) // 8 + 8 + 2 * d * in_bytes)
    dq_gbs = dq_bytes / (dq_ms * 1e-3) / 1e9
    digest = kernel_sources_digest()
    log(f"decode {dec_ms:.3f} ms ({dec_gbs:.0f} GB/s), quantize K {qk_ms:.3f} ms, V {qv_ms:.3f} ms, "
        f"dequantize K + V {dq_ms:.3f} ms ({dq_gbs:.0f} GB/s)")

    res = {
        "metric": METRIC,
        "value": round(dec_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {workloads.WORKLOAD_TEXT[cfg.name]}", "batch": cfg.B,
                   "q_heads": cfg.Hq, "kv_heads": cfg.Hkv, "head_dim": d, "seq_k": cfg.N,
                   "seq_q": cfg.Tq, "k_bits": cfg.k_bits, "k_qjl": cfg.k_qjl, "v_bits": cfg.v_bits,
                   "rotation": cfg.rot, "input_dtype": cfg.dtype},
        "hbm_peak_frac": round(dec_gbs / HBM_PEAK_GBS, 4),
        "decode_ms": round(dec_ms, 4),
        "quantize_k_ms": round(qk_ms, 4),
        "quantize_v_ms": round(qv_ms, 4),
        "quantize_vectors_per_s": round(vec_s, 1),
        "dequantize_ms": round(dq_ms, 4),
        "packed_kv_bytes": packed,
        "roofline": {"kernel": "tq_attn_decode (all launches of one call)", "bound": "hbm",
                     "achieved": round(dec_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic_from_profile("decode", cfg.name, digest, 1)},
        "roofline_quantize": {"kernel": "tq_quantize_kv (K and V calls)", "bound": "hbm",
                              "achieved": round(q_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                              "frac": round(q_gbs / HBM_PEAK_GBS, 4),
                              "traffic": traffic_from_profile("quantize", cfg.name, digest, 1)},
        "roofline_dequantize": {"kernel": "tq_dequantize (K and V calls)", "bound": "hbm",
                                "achieved": round(dq_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": round(dq_gbs / HBM_PEAK_GBS, 4),
                                "traffic": traffic_from_profile("dequantize", cfg.name, digest, 1)},
        "sources_digest": digest,
    }
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 1 GiB device-to-device copy kernel done")
        del src, dst
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle on a sample)")
        res["cpu_baseline"] = cpu_baseline(cfg, Kx, Vx, q)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
