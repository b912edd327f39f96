"""Benchmark of the TurboQuant KV-cache path on one MI355X.

One step = quantize the layer's keys, quantize its values, flush the
last-level cache, run decode attention over the compressed cache, then
dequantize both caches (into the input's dtype), on synthetic inputs already
resident in HBM.  The flush (plain reads of 2 GiB of unrelated data by the
probe kernel, outside the decode's timing events) leaves the 256 MB
last-level cache with none of the packed cache and no dirty lines: the decode
reads its whole cache from HBM and pays for no earlier kernel's write-back.
(Decode runs 5-15% slower for about a millisecond after heavy kernels, most
after the dequantize's 8.6 GB of writes; the workloads section times it
alone, back to back and after writes as well.)  The default workload is the Llama-3-8B-shaped layer (batch
16, 32 query / 8 KV heads, d=128, 131072 keys, fp16 inputs with per-channel
LogNormal(0, 0.5) scales, keys 3-bit MSE + 1-bit QJL, values 3-bit, Haar
rotation).

Printed (one JSON line on stdout):
  value              packed-KV bytes read by tq_attn_decode / its duration (GB/s)
  quantize_vectors_per_s   (K rows + V rows) / duration of the two quantize calls
  roofline           decode kernels vs the 8 TB/s HBM peak
  roofline_quantize, roofline_dequantize   the other two calls vs the same peak
  stream_read_gbs    the best rate of a streaming-read kernel on this GPU
                     (grid-stride and one contiguous chunk per workgroup)
  stream_rw_probe    the best rates of plain kernels that read 4 bytes per
                     byte written and 1 per 4 written (the mixes of quantize and
                     dequantize), with *_frac_of_stream_rw against them
  workloads          all five layer configurations: decode after the flush
                     and back to back, each against its own bound
                     (C1 launch latency, C4 matrix cores, the others HBM);
                     C2 also replayed from a HIP graph; quantize and dequantize
  cpu_baseline       the fp64 oracle on a bounded sample of the same workload
"""
import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tq_attn_decode packed-KV GB/s (% HBM peak) + tq_quantize_kv vectors/sec"
HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
FLUSH_BYTES = 2 << 30


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def packed_bytes_per_token(cfg):
    k = cfg.d * cfg.k_bits // 8 + 4 + (cfg.d // 8 + 4 if cfg.k_qjl else 0)
    v = cfg.d * cfg.v_bits // 8 + 4
    return k, v


def decode_flop(cfg):
    """Algorithmic flop of one decode call: per token-head and query row, d
    multiply-adds for the centroid term, d for the QJL term and d for P.V."""
    terms = 3 if cfg.k_qjl else 2
    return 2 * terms * cfg.d * cfg.G * cfg.Tq * cfg.rows


def traffic_from_profile(kernel_tag, workload, digest):
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


def host_cpu():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return model, n


def cpu_baseline(cfg, K_dev, V_dev, q_dev, budget_s=8.0):
    """Time the fp64 oracle (as it stands) on a bounded sample of the workload.

    Decode: whole (batch, KV head) sequences, decoded from packed bytes for
    the G query heads that share them, one after another until `budget_s` has
    passed.  Quantize: chunks of 8192 K rows and 8192 V rows taken from the
    sequences in order, until `budget_s` has passed.  Rates are scaled to the
    metric's units (packed-KV GB/s, vectors/s).  Run twice: with the BLAS
    thread pool as it is (the matrix products are its only multi-threaded
    part) and limited to one thread."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import attention, codebook, codec, transforms

    d, N, G = cfg.d, cfg.N, cfg.G
    R = transforms.rotation(d, cfg.rot, cfg.layer_seed)
    S = transforms.gaussian_projection(d, cfg.layer_seed)
    ck, bk = codebook.codebook(cfg.k_bits, d)
    cv, bv = codebook.codebook(cfg.v_bits, d)
    Sk = S if cfg.k_qjl else None
    seqs = [(b, h) for b in range(cfg.B) for h in range(cfg.Hkv)]

    def run(budget):
        chunk, nq, t_quant = 8192, 0, 0.0
        for b, h in seqs:
            for t0 in range(0, N, chunk):
                xk = K_dev[b, h, t0:t0 + chunk].double().cpu().numpy()
                xv = V_dev[b, h, t0:t0 + chunk].double().cpu().numpy()
                t = time.perf_counter()
                codec.encode_rows(xk, R, ck, bk, Sk)
                codec.encode_rows(xv, R, cv, bv)
                t_quant += time.perf_counter() - t
                nq += xk.shape[0]
                if t_quant >= budget:
                    break
            if t_quant >= budget:
                break
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
            if t_dec >= budget:
                break
        return nq, t_quant, nseq, t_dec

    kb, vb = packed_bytes_per_token(cfg)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    nq, tq_, nseq, td = run(budget_s)
    with threadpool_limits(limits=1):
        nq1, tq1, nseq1, td1 = run(budget_s / 2)
    model, ncpu = host_cpu()
    return {
        "value": round((kb + vb) * N * nseq / td / 1e9, 4),
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"decode of {nseq} of {len(seqs)} (batch, KV head) sequences ({G * cfg.Tq} query rows x "
                  f"{N} keys each, unpacked from packed bytes) in {td:.2f} s; quantize of {nq} K + "
                  f"{nq} V rows in {tq_:.2f} s; numpy fp64 with {threads} BLAS threads",
        "quantize_vectors_per_s": round(2 * nq / tq_, 1),
        "one_thread": {"value": round((kb + vb) * N * nseq1 / td1 / 1e9, 4), "unit": "GB/s",
                       "quantize_vectors_per_s": round(2 * nq1 / tq1, 1),
                       "sample": f"decode of {nseq1} sequences in {td1:.2f} s; quantize of {nq1} K + {nq1} V "
                                 f"rows in {tq1:.2f} s; BLAS limited to 1 thread"},
        "host_cpus": ncpu,
        "cpu_model": model,
    }


class Probe:
    """The streaming-read probe kernel (libtqprobe.so, built with the library)."""

    def __init__(self, dev):
        import torch
        path = os.path.join(ROOT, "compressed_attention_turboquant_amd", "libtqprobe.so")
        if not os.path.exists(path):
            raise ImportError(f"{path} is not built; run python -m compressed_attention_turboquant_amd.build")
        self.lib = ctypes.CDLL(path)
        self.lib.tq_probe_stream_threads.restype = ctypes.c_int64
        self.lib.tq_probe_stream_read.restype = ctypes.c_int
        self.lib.tq_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                                  ctypes.c_void_p]
        self.lib.tq_probe_stream_rw.restype = ctypes.c_int
        self.lib.tq_probe_stream_rw.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                                ctypes.c_void_p]
        self.lib.tq_probe_chunk_read.restype = ctypes.c_int
        self.lib.tq_probe_chunk_read.argtypes = self.lib.tq_probe_stream_read.argtypes
        self.lib.tq_probe_chunk_rw.restype = ctypes.c_int
        self.lib.tq_probe_chunk_rw.argtypes = self.lib.tq_probe_stream_rw.argtypes
        self.sink = torch.empty(self.lib.tq_probe_stream_threads() * 16, dtype=torch.uint8, device=dev)
        self.flush_buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.int32, device=dev)

    def read(self, buf, nontemporal, stream):
        rc = self.lib.tq_probe_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(), self.sink.data_ptr(),
                                           int(nontemporal), stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"stream probe launch failed: {rc}")

    def flush(self, stream):
        """Plain reads of 2 GiB of unrelated data: afterwards the 256 MB
        last-level cache holds none of a workload's cache and no dirty lines
        (a preceding write's lines are written back here, not in the next call)."""
        self.read(self.flush_buf, False, stream)

    def peak(self, dev, stream, nbytes=4 << 30, reps=6):
        """Best read rate over a 4 GiB buffer (16x the last-level cache), GB/s,
        for non-temporal and for plain loads, in a grid-stride pattern and one
        contiguous chunk per workgroup at a time (the faster one here)."""
        import torch
        buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
        out = {}
        for chunked in (False, True):
            fn = self.lib.tq_probe_chunk_read if chunked else self.lib.tq_probe_stream_read
            for nt in (True, False):
                best = 0.0
                for i in range(reps):
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    rc = fn(buf.data_ptr(), nbytes, self.sink.data_ptr(), int(nt), stream.cuda_stream)
                    e1.record(stream)
                    if rc != 0:
                        raise RuntimeError(f"stream probe launch failed: {rc}")
                    torch.cuda.synchronize()
                    if i > 0:
                        best = max(best, nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
                tag = ("chunked_" if chunked else "grid_stride_") + ("nontemporal" if nt else "plain")
                out[tag] = round(best, 1)
        del buf
        return out

    def peak_rw(self, dev, stream, small_bytes=2 << 30, reps=5):
        """Best rate (bytes read + written per second, GB/s) of plain kernels
        that read 4 bytes per byte written (a quantize call's mix) and read 1
        byte per 4 written (a dequantize call's), 2 GiB on the small side."""
        import torch
        words = small_bytes // 16
        small = torch.ones(small_bytes // 4, dtype=torch.int32, device=dev)
        large = torch.ones(4 * small_bytes // 4, dtype=torch.int32, device=dev)
        out = {}
        for read4, tag in ((1, "read4_write1"), (0, "read1_write4")):
            src, dst = (large, small) if read4 else (small, large)
            best = 0.0
            for fn in (self.lib.tq_probe_stream_rw, self.lib.tq_probe_chunk_rw):  # both patterns, the best counts
                for i in range(reps):
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    rc = fn(src.data_ptr(), dst.data_ptr(), words, read4, stream.cuda_stream)
                    e1.record(stream)
                    if rc != 0:
                        raise RuntimeError(f"stream probe launch failed: {rc}")
                    torch.cuda.synchronize()
                    if i > 0:
                        best = max(best, 5 * small_bytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
            out[tag] = round(best, 1)
        del small, large
        return out


class Layer:
    """One workload's inputs, layer tables and caches on the device."""

    def __init__(self, cfg, dev, Kx=None, Vx=None, q=None):
        import torch
        import workloads
        from compressed_attention_turboquant_amd import binding as B
        self.cfg, self.B = cfg, B
        S, cap, d = cfg.B * cfg.Hkv, cfg.cap, cfg.d
        self.Kx = Kx if Kx is not None else workloads.kv_torch(cfg, 0, "K", dev)
        self.Vx = Vx if Vx is not None else workloads.kv_torch(cfg, 0, "V", dev)
        self.q = q if q is not None else workloads.q_torch(cfg, 0, dev)
        rot = B.TQ_ROT_HAAR if cfg.rot == "haar" else B.TQ_ROT_HADAMARD
        flags = ((B.TQ_LAYER_BETA_CODEBOOK if cfg.codebook == "beta" else 0) | (B.TQ_LAYER_DITHER if cfg.dither else 0)
                 | (B.TQ_LAYER_VALUE_QJL if cfg.v_qjl else 0))
        t = time.perf_counter()
        self.layer = B.make_rotation(d, rot, cfg.layer_seed, cfg.k_bits, cfg.k_qjl, cfg.v_bits, flags=flags)
        torch.cuda.synchronize()
        self.layer_ms = (time.perf_counter() - t) * 1e3  # host tables and codebooks, and their upload
        self.Kc = B.Cache(self.layer, B.TQ_KEYS, S, cap)
        self.Vc = B.Cache(self.layer, B.TQ_VALUES, S, cap)
        view = lambda x: x.view(S, cap, d)[:, : cfg.N] if cap == cfg.N else x.view(S, cap, d)[:, : cfg.N].contiguous()
        self.xk, self.xv = view(self.Kx), view(self.Vx)
        self.out = torch.empty((cfg.B, cfg.Hq, cfg.Tq, d), dtype=torch.float32, device=dev)
        self.ws = torch.empty(max(B.decode_workspace_bytes(self.layer, cfg.B, cfg.Hq, cfg.Hkv, cfg.Tq, cfg.N), 1),
                              dtype=torch.uint8, device=dev)
        self.xhat = torch.empty((S, cfg.N, d), dtype=torch.float16 if cfg.dtype == "f16" else torch.float32,
                                device=dev)

    def quantize_k(self):
        self.B.quantize_kv(self.layer, self.B.TQ_KEYS, self.xk, self.Kc)

    def quantize_v(self):
        self.B.quantize_kv(self.layer, self.B.TQ_VALUES, self.xv, self.Vc)

    def dequantize(self):
        self.B.dequantize(self.layer, self.B.TQ_KEYS, self.Kc, self.cfg.N, out=self.xhat)
        self.B.dequantize(self.layer, self.B.TQ_VALUES, self.Vc, self.cfg.N, out=self.xhat)

    def dequantize_prod(self, which):
        cache = self.Kc if which == self.B.TQ_KEYS else self.Vc
        self.B.dequantize(self.layer, which, cache, self.cfg.N, out=self.xhat, prod=True)

    def decode(self):
        self.B.attn_decode(self.layer, self.q, self.Kc, self.Vc, self.cfg.N, self.cfg.Hkv, self.cfg.causal,
                           out=self.out, workspace=self.ws)


def timed(stream, fn, iters, before=None):
    """Mean duration (ms) of fn() over iters calls, each bracketed by HIP events
    on `stream`; before() (untimed) runs ahead of each call.  One untimed call
    first: the first launch of a kernel in a process also loads its code."""
    import torch
    if before:
        before()
    fn()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for e0, e1 in ev:
        if before:
            before()
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    return sum(e0.elapsed_time(e1) for e0, e1 in ev) / iters


def measure_workload(L, stream, probe, iters, stream_gbs, rw=None):
    """Decode (after a cache flush, and back to back), quantize and dequantize
    of one workload, each against its bound."""
    import torch
    import workloads
    cfg = L.cfg
    L.quantize_k()
    L.quantize_v()
    L.decode()
    torch.cuda.synchronize()
    q_k = timed(stream, L.quantize_k, iters)
    q_v = timed(stream, L.quantize_v, iters)
    deq = timed(stream, L.dequantize, iters)
    cold = timed(stream, L.decode, iters, before=lambda: probe.flush(stream))
    warm = timed(stream, L.decode, iters)
    # For comparison: right after 2 GiB of writes the last-level cache is full
    # of dirty lines, and writing them back shares HBM with the decode.
    after_write = timed(stream, L.decode, iters, before=lambda: probe.flush_buf.fill_(1))
    kb, vb = packed_bytes_per_token(cfg)
    packed = (kb + vb) * cfg.rows
    in_b = 2 if cfg.dtype == "f16" else 4
    gbs = packed / (cold * 1e-3) / 1e9
    rec = {
        "workload": f"{cfg.name}: {workloads.WORKLOAD_TEXT[cfg.name]}",
        "packed_kv_bytes": packed,
        "decode_ms": round(cold, 4),
        "decode_ms_back_to_back": round(warm, 4),
        "decode_ms_after_write": round(after_write, 4),
        "decode_gbs": round(gbs, 1),
        "decode_hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "decode_frac_of_stream": round(gbs / stream_gbs, 4) if stream_gbs else None,
        "quantize_k_ms": round(q_k, 4),
        "quantize_v_ms": round(q_v, 4),
        "quantize_vectors_per_s": round(2 * cfg.rows / ((q_k + q_v) * 1e-3), 1),
        "quantize_gbs": round((cfg.rows * 2 * cfg.d * in_b + packed) / ((q_k + q_v) * 1e-3) / 1e9, 1),
        "dequantize_ms": round(deq, 4),
        "dequantize_gbs": round(cfg.rows * (cfg.d * (cfg.k_bits + cfg.v_bits) // 8 + 8 + 2 * cfg.d * in_b)
                                / (deq * 1e-3) / 1e9, 1),
    }
    if rw:
        # against plain kernels with the same read/write mix (4:1 in, 1:4 out)
        rec["quantize_frac_of_stream_rw"] = round(rec["quantize_gbs"] / rw["read4_write1"], 4)
        rec["dequantize_frac_of_stream_rw"] = round(rec["dequantize_gbs"] / rw["read1_write4"], 4)
    if cfg.name == "C1":
        rec["roofline"] = {"bound": "latency", "achieved": round(cold * 1e3, 2), "unit": "us per call",
                           "peak": None, "frac": None,
                           "note": "92 KiB of packed KV: the call is launch and set-up latency"}
    elif cfg.name == "C4":
        fl = decode_flop(cfg)
        ach = fl / (cold * 1e-3) / 1e12
        rec["roofline"] = {"bound": "mfma", "achieved": round(ach, 2), "peak": MFMA_F16_PEAK_TFLOPS,
                           "unit": "TFLOP/s", "frac": round(ach / MFMA_F16_PEAK_TFLOPS, 4), "flop": fl,
                           "note": "128 query rows per KV head: 49,152 multiply-adds per 92 packed bytes"}
    else:
        rec["roofline"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(gbs / HBM_PEAK_GBS, 4)}
    if cfg.name == "C2":
        rec["decode_ms_graph"] = round(graph_decode_ms(L, 20), 4)
    return rec


def measure_next_rows(stage, W, stream, probe, iters, dev):
    """The rows past the hot path, each on the workload it extends: NEXT-2
    (reconstruction with the QJL term) and NEXT-3 (exact-law codebooks) at C3,
    NEXT-4 (dithered Hadamard) at C5, NEXT-1 (append one token per step, then
    decode) and NEXT-2 on values at C2's shape."""
    import torch
    import workloads
    B = W.B if W is not None else None
    out = {}
    if stage == "C3":
        cfg = W.cfg
        in_b = 2 if cfg.dtype == "f16" else 4
        kb, _ = packed_bytes_per_token(cfg)
        plain = timed(stream, lambda: B.dequantize(W.layer, B.TQ_KEYS, W.Kc, cfg.N, out=W.xhat), iters)
        prod = timed(stream, lambda: W.dequantize_prod(B.TQ_KEYS), iters)
        out["NEXT-2 keys"] = {
            "what": "tq_dequantize_prod of C3's keys (3-bit codes + QJL signs) into fp16 rows",
            "ms": round(prod, 4), "mse_only_ms": round(plain, 4),
            "gbs": round(cfg.rows * (kb + 2 * cfg.d * in_b) / (prod * 1e-3) / 1e9, 1)}
        Lb = Layer(cfg.with_(codebook="beta"), dev, Kx=W.Kx, Vx=W.Vx, q=W.q)
        Lb.quantize_k()
        Lb.quantize_v()
        qk = timed(stream, Lb.quantize_k, iters)
        qv = timed(stream, Lb.quantize_v, iters)
        dec = timed(stream, Lb.decode, iters, before=lambda: probe.flush(stream))
        kb, vb = packed_bytes_per_token(cfg)
        out["NEXT-3 exact-law codebook"] = {
            "what": "C3 with codebooks for the exact coordinate law (host Lloyd-Max solver at layer creation)",
            "layer_build_ms": round(Lb.layer_ms, 1), "quantize_k_ms": round(qk, 4), "quantize_v_ms": round(qv, 4),
            "decode_ms": round(dec, 4), "decode_gbs": round((kb + vb) * cfg.rows / (dec * 1e-3) / 1e9, 1)}
        del Lb
    elif stage == "C5":
        cfg = W.cfg.with_(dither=1)
        Ld = Layer(cfg, dev, Kx=W.Kx, Vx=W.Vx, q=W.q)
        Ld.quantize_k()
        Ld.quantize_v()
        qk = timed(stream, Ld.quantize_k, iters)
        qv = timed(stream, Ld.quantize_v, iters)
        dec = timed(stream, Ld.decode, iters, before=lambda: probe.flush(stream))
        deq = timed(stream, Ld.dequantize, iters)
        kb, vb = packed_bytes_per_token(cfg)
        out["NEXT-4 dithered Hadamard"] = {
            "what": "C5 with the dithered randomized Hadamard (per-token offset before quantizing)",
            "quantize_k_ms": round(qk, 4), "quantize_v_ms": round(qv, 4), "decode_ms": round(dec, 4),
            "decode_gbs": round((kb + vb) * cfg.rows / (dec * 1e-3) / 1e9, 1), "dequantize_ms": round(deq, 4)}
        del Ld
    else:  # after the workloads: C2's shape
        from compressed_attention_turboquant_amd import binding as B
        base = workloads.CONFIGS["C2"]
        # values with QJL (TurboQuant_prod on V; quantize and decode on the reference kernels)
        Lv = Layer(base.with_(v_qjl=1), dev)
        Lv.quantize_k()
        Lv.quantize_v()
        qv = timed(stream, Lv.quantize_v, iters)
        dec = timed(stream, Lv.decode, iters, before=lambda: probe.flush(stream))
        prod = timed(stream, lambda: Lv.dequantize_prod(B.TQ_VALUES), iters)
        out["NEXT-2 values"] = {
            "what": "C2's shape with QJL on values: quantize V, decode, tq_dequantize_prod of V",
            "quantize_v_ms": round(qv, 4), "decode_ms": round(dec, 4), "dequantize_prod_ms": round(prod, 4)}
        del Lv
        # append one token per step into caches with room for 64 more, then decode
        steps = 16
        cfg = base.with_(N=base.N + 64)
        S, d, N0 = cfg.B * cfg.Hkv, cfg.d, base.N
        Kx = workloads.kv_torch(cfg, 0, "K", dev).view(S, cfg.cap, d)
        Vx = workloads.kv_torch(cfg, 0, "V", dev).view(S, cfg.cap, d)
        q = workloads.q_torch(base, 0, dev)
        rot = B.TQ_ROT_HAAR if cfg.rot == "haar" else B.TQ_ROT_HADAMARD
        layer = B.make_rotation(d, rot, cfg.layer_seed, cfg.k_bits, cfg.k_qjl, cfg.v_bits)
        Kc, Vc = B.Cache(layer, B.TQ_KEYS, S, cfg.cap), B.Cache(layer, B.TQ_VALUES, S, cfg.cap)
        B.quantize_kv(layer, B.TQ_KEYS, Kx[:, :N0].contiguous(), Kc)
        B.quantize_kv(layer, B.TQ_VALUES, Vx[:, :N0].contiguous(), Vc)
        toks_k = [Kx[:, N0 + i:N0 + i + 1].contiguous() for i in range(steps)]
        toks_v = [Vx[:, N0 + i:N0 + i + 1].contiguous() for i in range(steps)]
        o = torch.empty((cfg.B, cfg.Hq, cfg.Tq, d), dtype=torch.float32, device=dev)
        ws = torch.empty(max(B.decode_workspace_bytes(layer, cfg.B, cfg.Hq, cfg.Hkv, cfg.Tq, N0 + i + 1)
                             for i in range(steps)), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        for i in range(steps):
            ev[i][0].record(stream)
            B.quantize_kv(layer, B.TQ_KEYS, toks_k[i], Kc, t0=N0 + i)
            ev[i][1].record(stream)
            B.quantize_kv(layer, B.TQ_VALUES, toks_v[i], Vc, t0=N0 + i)
            ev[i][2].record(stream)
            B.attn_decode(layer, q, Kc, Vc, N0 + i + 1, cfg.Hkv, 0, out=o, workspace=ws)
            ev[i][3].record(stream)
        torch.cuda.synchronize()
        mean = lambda a, b: sum(e[a].elapsed_time(e[b]) for e in ev[1:]) / (steps - 1) * 1e3
        out["NEXT-1 append and decode"] = {
            "what": f"C2's shape, {steps} steps: append one token per (batch, KV head) to K and V at t0 = N, "
                    "N + 1, ..., then decode over the cache so far",
            "append_k_us": round(mean(0, 1), 1), "append_v_us": round(mean(1, 2), 1),
            "decode_us": round(mean(2, 3), 1), "step_us": round(mean(0, 3), 1)}
        del Kx, Vx, Kc, Vc, ws
    return out


def graph_decode_ms(L, calls):
    """Per-call time of `calls` decode calls captured in one HIP graph and
    replayed (no host launch overhead between calls)."""
    import torch
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        L.decode()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for _ in range(calls):
            L.decode()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    best = None
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / calls
        best = t if best is None else min(best, t)
    del g
    return best


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="C3")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-workloads", action="store_true", help="skip the five-workload section")
    ap.add_argument("--workload-iters", type=int, default=10)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, run a plain 1 GiB device copy (reference for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported (the path is "
              "measured on one GPU's share of the sequences)", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads
    from compressed_attention_turboquant_amd.profsummary import kernel_sources_digest

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    cfg = workloads.CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    S, d = cfg.B * cfg.Hkv, cfg.d
    log(f"workload {cfg.name}: generating K, V ({2 * S * cfg.cap * d * (2 if cfg.dtype == 'f16' else 4) / 1e9:.1f} GB)")
    L = Layer(cfg, dev)
    probe = Probe(dev)

    def step(ev=None):
        if ev: ev[0].record(stream)
        L.quantize_k()
        if ev: ev[1].record(stream)
        L.quantize_v()
        if ev: ev[2].record(stream)
        probe.flush(stream)
        if ev: ev[3].record(stream)
        L.decode()
        if ev: ev[4].record(stream)
        L.dequantize()
        if ev: ev[5].record(stream)

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    qk_ms = sum(e[0].elapsed_time(e[1]) for e in events) / args.steps
    qv_ms = sum(e[1].elapsed_time(e[2]) for e in events) / args.steps
    dec_ms = sum(e[3].elapsed_time(e[4]) for e in events) / args.steps
    dq_ms = sum(e[4].elapsed_time(e[5]) for e in events) / args.steps
    kb, vb = packed_bytes_per_token(cfg)
    rows = cfg.rows
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
                     "traffic": traffic_from_profile("decode", cfg.name, digest)},
        "roofline_quantize": {"kernel": "tq_quantize_kv (K and V calls)", "bound": "hbm",
                              "achieved": round(q_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                              "frac": round(q_gbs / HBM_PEAK_GBS, 4),
                              "traffic": traffic_from_profile("quantize", cfg.name, digest)},
        "roofline_dequantize": {"kernel": "tq_dequantize (K and V calls)", "bound": "hbm",
                                "achieved": round(dq_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": round(dq_gbs / HBM_PEAK_GBS, 4),
                                "traffic": traffic_from_profile("dequantize", cfg.name, digest)},
        "sources_digest": digest,
    }
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 1 GiB device-to-device copy kernel done")
        del src, dst

    if not args.no_workloads:
        peaks = probe.peak(dev, stream)
        sgbs = max(peaks.values())
        res["stream_read_gbs"] = sgbs
        res["stream_read_probe"] = peaks
        res["decode_frac_of_stream"] = round(dec_gbs / sgbs, 4)
        log(f"streaming-read probe: {peaks} GB/s")
        rw = probe.peak_rw(dev, stream)
        res["stream_rw_probe"] = rw
        res["quantize_frac_of_stream_rw"] = round(q_gbs / rw["read4_write1"], 4)
        res["dequantize_frac_of_stream_rw"] = round(dq_gbs / rw["read1_write4"], 4)
        log(f"read/write streaming probe: {rw} GB/s")
        wl, nxt = {}, {}
        for name in ("C1", "C2", "C3", "C4", "C5"):
            c = workloads.CONFIGS[name]
            if name == cfg.name:
                W = L
            else:
                log(f"workload {name}: generating and quantizing")
                W = Layer(c, dev)
            wl[name] = measure_workload(W, stream, probe, args.workload_iters, sgbs, rw)
            if name in ("C3", "C5"):
                nxt.update(measure_next_rows(name, W, stream, probe, 3, dev))
            r = wl[name]
            log(f"  {name}: decode {r['decode_ms']:.4f} ms after a cache flush ({r['decode_gbs']:.0f} GB/s), "
                f"{r['decode_ms_back_to_back']:.4f} ms back to back; quantize {r['quantize_k_ms']:.3f} + "
                f"{r['quantize_v_ms']:.3f} ms; dequantize {r['dequantize_ms']:.3f} ms"
                + (f"; graph-replayed decode {r['decode_ms_graph']:.4f} ms" if "decode_ms_graph" in r else ""))
            if W is not L:
                del W
                torch.cuda.empty_cache()
        res["workloads"] = wl
        nxt.update(measure_next_rows("C2", None, stream, probe, 3, dev))
        res["next_rows"] = nxt
        log(f"next rows: {json.dumps(nxt)}")
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle on a sample)")
        res["cpu_baseline"] = cpu_baseline(cfg, L.Kx, L.Vx, L.q)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
