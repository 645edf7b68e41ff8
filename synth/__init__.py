"""Seeded synthetic inputs for the Hymba hybrid-head mixer.

This module is data only: workload shapes, value distributions and seeded
draws. It holds none of the mixer's arithmetic (no conv, scan, rotary,
attention or normalisation), so both the CPU oracle and the GPU path can take
their inputs from it without sharing any computation.

Shapes follow the Hymba-1.5B description (51cto release article, section 2
"model architecture": hidden 1600, 25 attention heads, 16 SSM states, GQA,
RoPE, sliding-window attention in most layers, a few global layers) and the
meta-token prefix of the Hymba guide (section "2. Learnable Meta-Tokens").

Draws: every tensor has its own PCG64 stream seeded by
``SeedSequence([config_seed, layer, tensor_id])`` so that a tensor's values do
not depend on which other tensors were drawn. Values are drawn in float32;
for bf16 workloads each value is then rounded to the nearest bf16
(round-to-nearest-even) and kept as a float32 array holding that exact value.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Dict, Optional

import numpy as np

__all__ = [
    "MixerConfig",
    "CONFIGS",
    "config",
    "round_bf16",
    "make_prefill_inputs",
    "make_decode_inputs",
    "key_affine",
    "POISON",
]

# Value written into KV-cache rows a decode step must never read. It is large
# so that a kernel which reads a wrong row produces a visibly wrong result.
POISON = 8.0

# Stable per-tensor stream ids.
_TID = {
    "x": 1, "z": 2, "dt": 3, "B": 4, "C": 5, "q": 6, "k": 7, "v": 8,
    "A": 9, "conv_w": 10, "ssm_state": 11, "conv_state": 12,
    "k_cache": 13, "v_cache": 14, "k_affine": 15,
}


@dataclass(frozen=True)
class MixerConfig:
    """Geometry and input distribution of one mixer workload."""

    name: str
    batch: int
    n_meta: int
    n_tokens: int          # prompt rows per sequence (prefill); 1 for decode
    d_inner: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    window: int            # > 0 sliding window; <= 0 global causal
    act: str               # "f32" or "bf16"
    seed: int
    d_state: int = 16
    d_conv: int = 4
    rope_base: float = 10000.0
    norm_eps: float = 1e-6
    dt_mu: float = -4.0    # dt = softplus(N(dt_mu, dt_sigma))
    dt_sigma: float = 1.0
    conv_sigma: float = 0.1
    decode: bool = False
    cache_len: int = 0     # decode: rows already in the cache (new token's position)
    cache_capacity: int = 0
    n_layers: int = 1      # decode: layers sharing one KV cache
    ssm_heads: int = 0     # > 0: Mamba-2 form, A a scalar per head, dt per head (head width d_inner / ssm_heads)
    key_affine: bool = False   # decode: layers after the first read the shared keys through
                               # their own affine (k_scale, k_bias); prefill: the layer does
    workload: str = ""

    @property
    def head_dim_v(self) -> int:
        # value head width: attention output width equals d_inner so the two
        # branch outputs can be averaged channel by channel
        return self.d_inner // self.n_q_heads

    @property
    def seq_rows(self) -> int:
        return self.n_meta + self.n_tokens

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def with_(self, **kw) -> "MixerConfig":
        return replace(self, **kw)


CONFIGS: Dict[str, MixerConfig] = {
    "tiny_f32": MixerConfig(
        name="tiny_f32", batch=1, n_meta=8, n_tokens=64, d_inner=128,
        n_q_heads=2, n_kv_heads=1, head_dim=64, window=32, act="f32", seed=0,
        workload="tiny fp32 mixer, B=1, T=64+8 meta, 2q/1kv x 64, window 32, d_inner 128"),
    "swa_layer": MixerConfig(
        name="swa_layer", batch=1, n_meta=128, n_tokens=2048, d_inner=3200,
        n_q_heads=25, n_kv_heads=5, head_dim=64, window=1024, act="bf16", seed=1,
        workload="Hymba-1.5B-shaped SWA layer prefill, B=1, T=2048+128 meta, "
                 "25q/5kv x 64, window 1024, d_inner 3200, d_state 16"),
    "global_layer": MixerConfig(
        name="global_layer", batch=1, n_meta=128, n_tokens=8192, d_inner=3200,
        n_q_heads=25, n_kv_heads=5, head_dim=64, window=0, act="bf16", seed=2,
        workload="Hymba-1.5B-shaped global layer prefill, B=1, T=8192+128 meta, "
                 "full causal 25q/5kv x 64, d_inner 3200"),
    "batched_prefill": MixerConfig(
        name="batched_prefill", batch=16, n_meta=128, n_tokens=4096, d_inner=3200,
        n_q_heads=25, n_kv_heads=5, head_dim=64, window=1024, act="bf16", seed=3,
        dt_mu=-3.0, dt_sigma=2.0,
        workload="batched prefill, B=16, T=4096+128 meta, 25q/5kv x 64, window 1024"),
    "decode": MixerConfig(
        name="decode", batch=64, n_meta=128, n_tokens=1, d_inner=3200,
        n_q_heads=25, n_kv_heads=5, head_dim=64, window=1024, act="bf16", seed=4,
        decode=True, cache_len=8192, cache_capacity=8192, n_layers=2,
        workload="decode step, batch 64, cache 8192 rows (window 1024 + 128 meta), "
                 "25q/5kv x 64, KV cache shared read-only by two consecutive layers"),
    # the same step where the second layer reads the shared keys through its
    # own per-head affine (the cross-layer sharing variant of the Hymba guide)
    "decode_affine": MixerConfig(
        name="decode_affine", batch=64, n_meta=128, n_tokens=1, d_inner=3200,
        n_q_heads=25, n_kv_heads=5, head_dim=64, window=1024, act="bf16", seed=4,
        decode=True, cache_len=8192, cache_capacity=8192, n_layers=2, key_affine=True,
        workload="decode step, batch 64, cache 8192 rows (window 1024 + 128 meta), "
                 "25q/5kv x 64, KV cache shared read-only by two layers, the second "
                 "reading its keys through a per-head affine"),
}

CONFIG_ORDER = ["tiny_f32", "swa_layer", "global_layer", "batched_prefill", "decode"]


def config(name: str, **overrides) -> MixerConfig:
    cfg = CONFIGS[name]
    return cfg.with_(**overrides) if overrides else cfg


# ---------------------------------------------------------------------------
# value handling


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32.

    Finite inputs only (the draws here are always finite)."""
    a = np.array(a, dtype=np.float32, copy=True, order="C")
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    u += np.uint32(0x7FFF)
    u += lsb
    u &= np.uint32(0xFFFF0000)
    return a

def _rng(cfg: MixerConfig, layer: int, name: str) -> np.random.Generator:
    ss = np.random.SeedSequence([cfg.seed, layer, _TID[name]])
    return np.random.Generator(np.random.PCG64(ss))


def _normal(cfg, layer, name, shape, mu=0.0, sigma=1.0) -> np.ndarray:
    g = _rng(cfg, layer, name)
    a = g.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        a *= np.float32(sigma)
    if mu != 0.0:
        a += np.float32(mu)
    return a


def _softplus32(a: np.ndarray) -> np.ndarray:
    # part of the dt distribution: dt = softplus(N(mu, sigma)) drawn positive
    return np.logaddexp(np.float32(0.0), a).astype(np.float32)


def _act(cfg: MixerConfig, a: np.ndarray) -> np.ndarray:
    return round_bf16(a) if cfg.act == "bf16" else np.ascontiguousarray(a, np.float32)


def _params(cfg: MixerConfig, layer: int) -> Dict[str, np.ndarray]:
    D, N, K = cfg.d_inner, cfg.d_state, cfg.d_conv
    g = _rng(cfg, layer, "A")
    a_shape = (cfg.ssm_heads,) if cfg.ssm_heads > 0 else (D, N)   # per head, or per (channel, state)
    A = -np.exp(g.uniform(np.log(1.0), np.log(16.0), size=a_shape)).astype(np.float32)
    conv_w = _normal(cfg, layer, "conv_w", (D, K), sigma=cfg.conv_sigma)
    return {
        "A": A,
        "conv_w": conv_w,
        "D": np.ones(D, np.float32),
        "beta_attn": np.ones(D, np.float32),
        "beta_ssm": np.ones(D, np.float32),
    }


def key_affine(cfg: MixerConfig, layer: int) -> Dict[str, np.ndarray]:
    """Head-specific affine of a layer that reads another layer's keys:
    k_scale U[0.5, 1.5) and k_bias N(0, 1), each [Hkv, hd] fp32."""
    g = _rng(cfg, layer, "k_affine")
    shape = (cfg.n_kv_heads, cfg.head_dim)
    return {"k_scale": (np.float32(0.5) + g.random(size=shape, dtype=np.float32)).astype(np.float32),
            "k_bias": g.standard_normal(size=shape, dtype=np.float32)}


def make_prefill_inputs(cfg: MixerConfig, layer: int = 0) -> Dict[str, np.ndarray]:
    """x, z, dt [B,L,D]; B, C [B,L,N]; q [B,L,Hq,hd]; k [B,L,Hkv,hd]; v [B,L,Hkv,dv]
    in the activation dtype's values, plus fp32 parameters. With ssm_heads > 0
    dt is [B,L,ssm_heads] and A [ssm_heads]."""
    Bsz, L, D, N = cfg.batch, cfg.seq_rows, cfg.d_inner, cfg.d_state
    Ddt = cfg.ssm_heads if cfg.ssm_heads > 0 else D
    Hq, Hkv, hd, dv = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.head_dim_v
    out = {
        "x": _act(cfg, _normal(cfg, layer, "x", (Bsz, L, D))),
        "z": _act(cfg, _normal(cfg, layer, "z", (Bsz, L, D))),
        "dt": _act(cfg, _softplus32(_normal(cfg, layer, "dt", (Bsz, L, Ddt), cfg.dt_mu, cfg.dt_sigma))),
        "B": _act(cfg, _normal(cfg, layer, "B", (Bsz, L, N))),
        "C": _act(cfg, _normal(cfg, layer, "C", (Bsz, L, N))),
        "q": _act(cfg, _normal(cfg, layer, "q", (Bsz, L, Hq, hd))),
        "k": _act(cfg, _normal(cfg, layer, "k", (Bsz, L, Hkv, hd))),
        "v": _act(cfg, _normal(cfg, layer, "v", (Bsz, L, Hkv, dv))),
    }
    out.update(_params(cfg, layer))
    if cfg.key_affine:
        out.update(key_affine(cfg, layer))
    return out


def make_decode_inputs(cfg: MixerConfig, cache_len: Optional[np.ndarray] = None) -> Dict[str, object]:
    """One decode step for ``cfg.n_layers`` layers sharing one read-only KV cache.

    Shared: k_cache [B,cap,Hkv,hd], v_cache [B,cap,Hkv,dv] (rows treated as already
    rotated), k_new [B,Hkv,hd], v_new [B,Hkv,dv], cache_len [B] int32.
    Per layer l (dict ``layers[l]``): x, z, dt [B,D]; B, C [B,N]; q [B,Hq,hd];
    ssm_state [B,D,N] fp32; conv_state [B,D,d_conv-1] (act); parameters; with
    ``cfg.key_affine``, layers after the first also k_scale, k_bias [Hkv,hd].

    Rows [0, cache_len[b]) of sequence b hold N(0,1) draws; rows at or beyond
    cache_len[b] have not been written by any earlier step and hold POISON.
    """
    Bsz, D, N = cfg.batch, cfg.d_inner, cfg.d_state
    Hq, Hkv, hd, dv = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.head_dim_v
    cap = cfg.cache_capacity
    if cache_len is None:
        cache_len = np.full(Bsz, cfg.cache_len, np.int32)
    cache_len = np.asarray(cache_len, np.int32)
    assert cache_len.shape == (Bsz,) and int(cache_len.max()) <= cap

    kc = np.full((Bsz, cap, Hkv, hd), POISON, np.float32)
    vc = np.full((Bsz, cap, Hkv, dv), POISON, np.float32)
    gk = _rng(cfg, 0, "k_cache")
    gv = _rng(cfg, 0, "v_cache")
    for b in range(Bsz):
        p = int(cache_len[b])
        kc[b, :p] = gk.standard_normal(size=(p, Hkv, hd), dtype=np.float32)
        vc[b, :p] = gv.standard_normal(size=(p, Hkv, dv), dtype=np.float32)
    shared = {
        "k_cache": _act(cfg, kc),
        "v_cache": _act(cfg, vc),
        "k_new": _act(cfg, _normal(cfg, 0, "k", (Bsz, Hkv, hd))),
        "v_new": _act(cfg, _normal(cfg, 0, "v", (Bsz, Hkv, dv))),
        "cache_len": cache_len,
    }
    layers = []
    Ddt = cfg.ssm_heads if cfg.ssm_heads > 0 else D
    for l in range(cfg.n_layers):
        d = {
            "x": _act(cfg, _normal(cfg, l, "x", (Bsz, D))),
            "z": _act(cfg, _normal(cfg, l, "z", (Bsz, D))),
            "dt": _act(cfg, _softplus32(_normal(cfg, l, "dt", (Bsz, Ddt), cfg.dt_mu, cfg.dt_sigma))),
            "B": _act(cfg, _normal(cfg, l, "B", (Bsz, N))),
            "C": _act(cfg, _normal(cfg, l, "C", (Bsz, N))),
            "q": _act(cfg, _normal(cfg, l, "q", (Bsz, Hq, hd))),
            "ssm_state": _normal(cfg, l, "ssm_state", (Bsz, D, N)),
            "conv_state": _act(cfg, _normal(cfg, l, "conv_state", (Bsz, D, cfg.d_conv - 1))),
        }
        d.update(_params(cfg, l))
        if cfg.key_affine and l > 0:
            d.update(key_affine(cfg, l))
        layers.append(d)
    shared["layers"] = layers
    return shared
