"""Seeded synthetic workloads for the TurboQuant KV-cache path.

This module only draws inputs: shapes, dtypes and value distributions of the
five synthetic layer configurations, plus random packed caches for exercising
the decode step on its own.  It holds none of the method's arithmetic (no
rotation, codebook, estimator or softmax), so both the fp64 oracle and the HIP
path can be fed from it without sharing any of the method's code.

Value recipes (the pages name model shapes, never data):
  C1  q, K, V ~ N(0,1), fp32.
  C2  q, K, V ~ N(0,1), fp16.
  C3  Llama-3-8B-shaped layer: K, V ~ N(0,1) times a per-(KV head, channel)
      scale drawn once from LogNormal(0, 0.5) (separate draws for K and V,
      fixed across tokens); q ~ N(0,1); fp16.
  C4  Qwen2.5-3B-shaped layer: K ~ N(0,1) with 4 seeded channels per KV head
      multiplied by 10; V ~ N(0,1); q ~ N(0,1); fp16; 16 query tokens with a
      causal mask over the last 16 keys.
  C5  K, V ~ Student-t(nu=5) (a normal over sqrt(chi2_5/5)); q ~ N(0,1); fp16.
Values are drawn in float64 (numpy) or float32 (torch), scaled, then rounded
to the storage dtype with round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

# Tags separate independent streams drawn from one seed.
TAG_Q, TAG_K, TAG_V, TAG_KSCALE, TAG_VSCALE, TAG_OUTLIER, TAG_PACKED = 1, 2, 3, 4, 5, 6, 7


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    Tq: int
    N: int
    dtype: str          # "f32" or "f16" for q, K and V
    k_bits: int         # MSE bits of the key codes
    k_qjl: int          # 1: keys also carry QJL sign bits and the residual norm
    v_bits: int         # MSE bits of the value codes
    rot: str            # "haar" or "hadamard"
    causal: int
    dist: str           # "normal", "lognormal_channels", "outlier_channels", "student_t5"
    layer_seed: int = 0
    codebook: str = "gaussian"   # codebook law: "gaussian" (N(0, 1/d)) or "beta" (exact coordinate law)
    dither: int = 0              # 1: dithered randomized Hadamard (per-token offset before quantizing)
    v_qjl: int = 0               # 1: values also carry QJL sign bits and the residual norm

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def rows(self) -> int:
        """Token-heads per tensor (rows of K, or of V)."""
        return self.B * self.Hkv * self.N

    @property
    def cap(self) -> int:
        """Token capacity per (batch, KV head): N rounded up to a multiple of 8."""
        return (self.N + 7) // 8 * 8

    def with_(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    "C1": LayerConfig("C1", B=1, Hq=1, Hkv=1, d=128, Tq=1, N=1024, dtype="f32",
                      k_bits=2, k_qjl=1, v_bits=2, rot="haar", causal=0, dist="normal"),
    "C2": LayerConfig("C2", B=1, Hq=32, Hkv=8, d=128, Tq=1, N=32768, dtype="f16",
                      k_bits=2, k_qjl=1, v_bits=3, rot="haar", causal=0, dist="normal"),
    "C3": LayerConfig("C3", B=16, Hq=32, Hkv=8, d=128, Tq=1, N=131072, dtype="f16",
                      k_bits=3, k_qjl=1, v_bits=3, rot="haar", causal=0,
                      dist="lognormal_channels"),
    "C4": LayerConfig("C4", B=64, Hq=16, Hkv=2, d=128, Tq=16, N=32768, dtype="f16",
                      k_bits=2, k_qjl=1, v_bits=2, rot="haar", causal=1,
                      dist="outlier_channels"),
    "C5": LayerConfig("C5", B=32, Hq=32, Hkv=8, d=256, Tq=1, N=65536, dtype="f16",
                      k_bits=4, k_qjl=0, v_bits=4, rot="hadamard", causal=0,
                      dist="student_t5"),
}

WORKLOAD_TEXT = {
    "C1": "1 head, d=128, seq_k=1024, fp32, K 2-bit MSE + 1-bit QJL, V 2-bit, Haar",
    "C2": "GQA 32/8 heads, d=128, seq_k=32768, fp16, K 2+1 QJL, V 3-bit, Haar",
    "C3": "Llama-3-8B-shaped layer: batch 16, 32/8 heads, d=128, seq_k=131072, fp16, "
          "per-channel LogNormal(0,0.5) scales, K 3+1 QJL, V 3-bit, Haar",
    "C4": "Qwen2.5-3B-shaped layer: batch 64, 16/2 heads, d=128, seq_k=32768, 16 causal "
          "query tokens, fp16, 4 outlier K channels x10, K 2+1 QJL, V 2-bit, Haar",
    "C5": "batch 32, 32/8 heads, d=256, seq_k=65536, fp16 Student-t(5), K 4-bit, V 4-bit, "
          "randomized Hadamard",
}


def _rng(seed: int, tag: int, *more: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tag, *more])))


def _np_dtype(dtype: str):
    return {"f32": np.float32, "f16": np.float16}[dtype]


def _kv_scale_numpy(cfg: LayerConfig, seed: int, which: str) -> np.ndarray:
    """Per-(KV head, channel) multiplier of the value distribution, float64 [Hkv, d]."""
    scale = np.ones((cfg.Hkv, cfg.d))
    if cfg.dist == "lognormal_channels":
        tag = TAG_KSCALE if which == "K" else TAG_VSCALE
        scale = np.exp(0.5 * _rng(seed, tag).standard_normal((cfg.Hkv, cfg.d)))
    elif cfg.dist == "outlier_channels" and which == "K":
        r = _rng(seed, TAG_OUTLIER)
        for h in range(cfg.Hkv):
            scale[h, r.choice(cfg.d, size=4, replace=False)] = 10.0
    return scale


def kv_numpy(cfg: LayerConfig, seed: int = 0, which: str = "K",
             B: Optional[int] = None, N: Optional[int] = None) -> np.ndarray:
    """K or V for the whole layer, [B, Hkv, N, d] in the storage dtype.

    Each (b, h) slice has its own stream, so slices can be regenerated alone.
    """
    B = cfg.B if B is None else B
    N = cfg.N if N is None else N
    tag = TAG_K if which == "K" else TAG_V
    scale = _kv_scale_numpy(cfg, seed, which)
    out = np.empty((B, cfg.Hkv, N, cfg.d), dtype=_np_dtype(cfg.dtype))
    for b in range(B):
        for h in range(cfg.Hkv):
            r = _rng(seed, tag, b, h)
            if cfg.dist == "student_t5":
                z = r.standard_normal((N, cfg.d))
                chi2 = (r.standard_normal((5, N, cfg.d)) ** 2).sum(axis=0)
                x = z / np.sqrt(chi2 / 5.0)
            else:
                x = r.standard_normal((N, cfg.d))
            out[b, h] = (x * scale[h]).astype(out.dtype)
    return out


def q_numpy(cfg: LayerConfig, seed: int = 0, B: Optional[int] = None) -> np.ndarray:
    """Queries [B, Hq, Tq, d] ~ N(0,1) in the storage dtype."""
    B = cfg.B if B is None else B
    x = _rng(seed, TAG_Q).standard_normal((B, cfg.Hq, cfg.Tq, cfg.d))
    return x.astype(_np_dtype(cfg.dtype))


def random_packed_numpy(cfg: LayerConfig, S: int, cap: int, seed: int = 0) -> dict:
    """A random compressed cache: any byte pattern is a valid set of codes.

    Returns uint8 code/sign arrays and float32 norms laid out for S sequences
    of capacity `cap`; norms are drawn as |N(0,1)|*sqrt(d) (key/value norms)
    and |N(0,0.3)| (residual norms), which is the scale real caches have.
    """
    r = _rng(seed, TAG_PACKED)
    d = cfg.d
    out = {
        "k_idx": r.integers(0, 256, size=S * cap * d * cfg.k_bits // 8, dtype=np.uint8),
        "v_idx": r.integers(0, 256, size=S * cap * d * cfg.v_bits // 8, dtype=np.uint8),
        "k_norm": (np.abs(r.standard_normal(S * cap)) * np.sqrt(d)).astype(np.float32),
        "v_norm": (np.abs(r.standard_normal(S * cap)) * np.sqrt(d)).astype(np.float32),
    }
    if cfg.k_qjl:
        out["k_sign"] = r.integers(0, 256, size=S * cap * d // 8, dtype=np.uint8)
        out["k_rnorm"] = np.abs(0.3 * r.standard_normal(S * cap)).astype(np.float32)
    if cfg.v_qjl:
        out["v_sign"] = r.integers(0, 256, size=S * cap * d // 8, dtype=np.uint8)
        out["v_rnorm"] = np.abs(0.3 * r.standard_normal(S * cap)).astype(np.float32)
    return out


# ----------------------------------------------------------------------------
# Device-side generation for the full-size layers (tens of GB; numpy on the
# host would take minutes).  Same recipes, drawn with torch's generator.
# ----------------------------------------------------------------------------

def kv_torch(cfg: LayerConfig, seed: int, which: str, device, B: Optional[int] = None,
             N: Optional[int] = None, out=None):
    """K or V [B, Hkv, cap, d] on `device` (tokens >= N are zero)."""
    import torch
    B = cfg.B if B is None else B
    N = cfg.N if N is None else N
    cap = (N + 7) // 8 * 8
    dt = {"f32": torch.float32, "f16": torch.float16}[cfg.dtype]
    if out is None:
        out = torch.zeros((B, cfg.Hkv, cap, cfg.d), dtype=dt, device=device)
    scale = torch.from_numpy(_kv_scale_numpy(cfg, seed, which)).to(device=device,
                                                                     dtype=torch.float32)
    g = torch.Generator(device=device)
    tag = TAG_K if which == "K" else TAG_V
    for b in range(B):
        g.manual_seed((seed * 1_000_003 + tag * 10_007 + b) & 0x7FFFFFFFFFFFFFFF)
        x = torch.randn((cfg.Hkv, N, cfg.d), generator=g, device=device, dtype=torch.float32)
        if cfg.dist == "student_t5":
            chi2 = torch.zeros_like(x)
            for _ in range(5):
                chi2 += torch.randn(x.shape, generator=g, device=device,
                                    dtype=torch.float32) ** 2
            x = x / torch.sqrt(chi2 / 5.0)
        x *= scale[:, None, :]
        out[b, :, :N].copy_(x.to(dt))
        del x
    return out


def q_torch(cfg: LayerConfig, seed: int, device, B: Optional[int] = None):
    import torch
    B = cfg.B if B is None else B
    return torch.from_numpy(q_numpy(cfg, seed, B)).to(device)
