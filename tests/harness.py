"""Shared helpers for the GPU tests and the benchmark: move seeded inputs to the
GPU, call the library through its C ABI, bring results back as float64."""
from __future__ import annotations

import numpy as np
import torch

import attention_lm_amd as H

TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}
TOL = {"f32": 1e-5, "bf16": 5e-3}   # relative L2 bounds (fp32 / bf16 with fp32 accumulation)


def rel_l2(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref.ravel())
    return float(np.linalg.norm((got - ref).ravel()) / (den if den > 0 else 1.0))


def slice_errors(got, ref, width):
    """Relative L2 error of each slice: the last axis cut into pieces of
    ``width`` elements (the whole axis if it does not divide), every other axis
    kept, so a slice is one (row, head) of the attention output, one block of
    channels of a row, or one channel's states. A slice whose reference norm is
    below a tenth of the RMS slice norm is measured against that floor (a
    decayed state or a near-zero block is not blown up by its own small norm)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    w = ref.shape[-1]
    sw = width if (width <= w and w % width == 0) else w
    g = got.reshape(-1, sw)
    r = ref.reshape(-1, sw)
    num = np.linalg.norm(g - r, axis=1)
    den = np.linalg.norm(r, axis=1)
    floor = 0.1 * np.sqrt(np.mean(den * den)) if den.size else 0.0
    return num / np.maximum(den, max(floor, 1e-30)), sw


def check(name, got, ref, tol, slice_width=128, slice_factor=4.0, say=print):
    """Relative L2 over the whole tensor <= tol, and over every slice (see
    slice_errors) <= slice_factor * tol, so that an error confined to one row,
    head, tile or channel block cannot hide in a large tensor's norm."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), name
    e = rel_l2(got, ref)
    se, sw = slice_errors(got, ref, slice_width)
    worst = int(np.argmax(se)) if se.size else 0
    ws = float(se[worst]) if se.size else 0.0
    where = np.unravel_index(worst, ref.shape[:-1] + (ref.shape[-1] // sw,)) if se.size else ()
    say(f"  {name:14s} rel_l2={e:.3e} (tol {tol:.0e}); worst {sw}-wide slice {ws:.3e} at {tuple(int(i) for i in where)}"
        f" (tol {slice_factor * tol:.0e})")
    assert e <= tol, (name, e, tol)
    assert ws <= slice_factor * tol, (name, "slice", where, ws)


def dev(a, act=None, device="cuda"):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if act is not None:
        t = t.to(TORCH_DT[act])
    return t.to(device)


def host(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def desc_for(cfg, **kw):
    d = dict(batch=cfg.batch, n_meta=cfg.n_meta, n_tokens=cfg.n_tokens, d_inner=cfg.d_inner,
             n_q_heads=cfg.n_q_heads, n_kv_heads=cfg.n_kv_heads, window=cfg.window, act=cfg.act,
             head_dim=cfg.head_dim, d_state=cfg.d_state, d_conv=cfg.d_conv,
             cache_capacity=cfg.cache_capacity, rope_base=cfg.rope_base, norm_eps=cfg.norm_eps,
             ssm_heads=cfg.ssm_heads)
    d.update(kw)
    return H.make_desc(**d)


class Prefill:
    """Device tensors and a bound call for one prefill workload."""

    def __init__(self, cfg, inp, with_outputs=True, with_cache=True, cache_capacity=None):
        self.cfg = cfg
        act = cfg.act
        L = cfg.seq_rows
        self.t = {k: dev(inp[k], act) for k in ("x", "z", "dt", "B", "C", "q", "k", "v")}
        self.p = {k: dev(inp[k]) for k in ("A", "D", "conv_w", "beta_attn", "beta_ssm")}
        Bsz, D = cfg.batch, cfg.d_inner
        dt_ = TORCH_DT[act]
        self.out = torch.empty((Bsz, L, D), dtype=dt_, device="cuda")
        self.cap = cache_capacity if cache_capacity is not None else L
        self.o = {}
        if with_outputs:
            self.o["ssm_state_out"] = torch.empty((Bsz, D, cfg.d_state), dtype=torch.float32, device="cuda")
            self.o["conv_state_out"] = torch.empty((Bsz, D, cfg.d_conv - 1), dtype=dt_, device="cuda")
            self.o["y_attn_out"] = torch.empty((Bsz, L, D), dtype=dt_, device="cuda")
            self.o["y_ssm_out"] = torch.empty((Bsz, L, D), dtype=dt_, device="cuda")
        if with_cache:
            self.o["k_cache"] = torch.full((Bsz, self.cap, cfg.n_kv_heads, cfg.head_dim), 7.0, dtype=dt_, device="cuda")
            self.o["v_cache"] = torch.full((Bsz, self.cap, cfg.n_kv_heads, cfg.head_dim_v), 7.0, dtype=dt_, device="cuda")
        self.desc = desc_for(cfg, cache_capacity=self.cap)
        for k in ("k_scale", "k_bias"):
            if inp.get(k) is not None:
                self.p[k] = dev(inp[k])
        self.params = H.make_params(self.p["A"], self.p["D"], self.p["conv_w"], self.p["beta_attn"], self.p["beta_ssm"],
                                    self.p.get("k_scale"), self.p.get("k_bias"))
        self.ws = torch.empty(max(H.hymba_mixer_prefill_workspace_bytes(self.desc), 256), dtype=torch.uint8,
                              device="cuda")

    def __call__(self, stream=None):
        t = self.t
        H.hymba_mixer_prefill(self.desc, self.params, t["x"], t["z"], t["dt"], t["B"], t["C"], t["q"], t["k"],
                              t["v"], self.out, workspace=self.ws, stream=stream, **self.o)

    def results(self):
        r = {"out": host(self.out)}
        for k, v in self.o.items():
            r[k] = host(v)
        return r


class Decode:
    """Device tensors for one decode step of several layers sharing one KV cache."""

    def __init__(self, cfg, inp):
        self.cfg = cfg
        act = cfg.act
        dt_ = TORCH_DT[act]
        self.k_cache = dev(inp["k_cache"], act)
        self.v_cache = dev(inp["v_cache"], act)
        self.k_new = dev(inp["k_new"], act)
        self.v_new = dev(inp["v_new"], act)
        self.cache_len = dev(inp["cache_len"])
        self.layers = []
        Bsz, D = cfg.batch, cfg.d_inner
        for li in inp["layers"]:
            L = {k: dev(li[k], act) for k in ("x", "z", "dt", "B", "C", "q", "conv_state")}
            L["ssm_state"] = dev(li["ssm_state"])
            L["params_t"] = {k: dev(li[k]) for k in ("A", "D", "conv_w", "beta_attn", "beta_ssm", "k_scale", "k_bias")
                             if li.get(k) is not None}
            pt = L["params_t"]
            L["params"] = H.make_params(pt["A"], pt["D"], pt["conv_w"], pt["beta_attn"], pt["beta_ssm"],
                                        pt.get("k_scale"), pt.get("k_bias"))
            L["out"] = torch.empty((Bsz, D), dtype=dt_, device="cuda")
            L["y_attn_out"] = torch.empty((Bsz, D), dtype=dt_, device="cuda")
            L["y_ssm_out"] = torch.empty((Bsz, D), dtype=dt_, device="cuda")
            self.layers.append(L)
        self.desc = desc_for(cfg)
        self.ws = torch.empty(max(H.hymba_mixer_decode_workspace_bytes(self.desc), 256), dtype=torch.uint8,
                              device="cuda")

    def call(self, l, stream=None, with_branches=True):
        L = self.layers[l]
        H.hymba_mixer_decode(self.desc, L["params"], L["x"], L["z"], L["dt"], L["B"], L["C"], L["q"], self.k_new,
                             self.v_new, self.k_cache, self.v_cache, self.cache_len, L["ssm_state"],
                             L["conv_state"], L["out"], y_attn_out=L["y_attn_out"] if with_branches else None,
                             y_ssm_out=L["y_ssm_out"] if with_branches else None, workspace=self.ws, stream=stream)
