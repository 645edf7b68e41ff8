"""Pins of the CPU oracle to things other than itself: closed forms, brute
force on tiny inputs, invariants, library routines and the pages' printed
worked examples. CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng(seed=0):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------
# conv


def test_conv_matches_torch_conv1d():
    g = rng(1)
    Bsz, L, D, K = 2, 11, 5, 4
    x = g.standard_normal((Bsz, L, D))
    w = g.standard_normal((D, K))
    u = O.causal_conv1d(x, w)
    xt = torch.from_numpy(x).permute(0, 2, 1)                      # [B, D, L]
    wt = torch.from_numpy(w)[:, None, :]                           # [D, 1, K]
    ref = torch.nn.functional.conv1d(xt, wt, groups=D, padding=K - 1)[..., :L]
    np.testing.assert_allclose(u, ref.permute(0, 2, 1).numpy(), rtol=1e-13, atol=1e-13)


def test_conv_tap_orientation():
    g = rng(2)
    x = g.standard_normal((1, 9, 3))
    e3 = np.zeros((3, 4)); e3[:, 3] = 1.0
    e0 = np.zeros((3, 4)); e0[:, 0] = 1.0
    np.testing.assert_array_equal(O.causal_conv1d(x, e3), x)       # last tap = current row
    u0 = O.causal_conv1d(x, e0)
    np.testing.assert_array_equal(u0[:, 3:], x[:, :-3])            # first tap = row t-3
    np.testing.assert_array_equal(u0[:, :3], 0.0)                  # zero history


def test_conv_history_split():
    g = rng(3)
    x = g.standard_normal((2, 12, 4))
    w = g.standard_normal((4, 4))
    full = O.causal_conv1d(x, w)
    part = O.causal_conv1d(x[:, 7:], w, history=x[:, 4:7])
    np.testing.assert_allclose(part, full[:, 7:], rtol=1e-14, atol=1e-14)


# ---------------------------------------------------------------------------
# selective scan


def _scan_inputs(seed, Bsz=2, L=9, D=3, N=4):
    g = rng(seed)
    u = g.standard_normal((Bsz, L, D))
    dt = np.log1p(np.exp(g.normal(-1.0, 1.0, (Bsz, L, D))))
    A = -np.exp(g.uniform(0.0, np.log(16.0), (D, N)))
    Bm = g.standard_normal((Bsz, L, N))
    Cm = g.standard_normal((Bsz, L, N))
    Dv = g.standard_normal(D)
    return u, dt, A, Bm, Cm, Dv


def test_scan_brute_force_quadratic_form():
    """y_t = sum_{s<=t} sum_n C_t[n] exp(A[c,n] sum_{r=s+1..t} dt_r) dt_s B_s[n] u_s + D u_t,
    materialised for every (t, s) pair independently of the recurrence."""
    u, dt, A, Bm, Cm, Dv = _scan_inputs(4)
    y, h = O.selective_scan(u, dt, A, Bm, Cm, Dv)
    Bsz, L, D = u.shape
    N = A.shape[1]
    ref = np.zeros_like(y)
    href = np.zeros((Bsz, D, N))
    for b in range(Bsz):
        for c in range(D):
            for t in range(L):
                acc = Dv[c] * u[b, t, c]
                for s in range(t + 1):
                    decay = np.exp(A[c] * dt[b, s + 1:t + 1, c].sum())
                    acc += np.sum(Cm[b, t] * decay * dt[b, s, c] * Bm[b, s] * u[b, s, c])
                ref[b, t, c] = acc
            for s in range(L):
                href[b, c] += np.exp(A[c] * dt[b, s + 1:, c].sum()) * dt[b, s, c] * Bm[b, s] * u[b, s, c]
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(h, href, rtol=1e-12, atol=1e-12)


def test_scan_constant_inputs_geometric_closed_form():
    delta, a, bval, xi, cval, dval = 0.07, -3.0, 0.8, 1.3, -0.6, 0.4
    L = 40
    u = np.full((1, L, 1), xi)
    dt = np.full((1, L, 1), delta)
    A = np.array([[a]])
    Bm = np.full((1, L, 1), bval)
    Cm = np.full((1, L, 1), cval)
    y, h = O.selective_scan(u, dt, A, Bm, Cm, np.array([dval]))
    r = math.exp(delta * a)
    t = np.arange(L)
    h_t = delta * bval * xi * (1 - r ** (t + 1)) / (1 - r)
    np.testing.assert_allclose(y[0, :, 0], cval * h_t + dval * xi, rtol=1e-12)
    np.testing.assert_allclose(h[0, 0, 0], h_t[-1], rtol=1e-12)


def test_scan_impulse_decays_geometrically():
    delta, a, bval = 0.3, -0.5, 2.0
    L = 25
    u = np.zeros((1, L, 1)); u[0, 0, 0] = 1.0
    dt = np.full((1, L, 1), delta)
    Bm = np.full((1, L, 1), bval)
    Cm = np.ones((1, L, 1))
    y, _ = O.selective_scan(u, dt, np.array([[a]]), Bm, Cm, np.array([0.0]))
    r = math.exp(delta * a)
    np.testing.assert_allclose(y[0, :, 0], delta * bval * r ** np.arange(L), rtol=1e-12)


def test_scan_step_size_limits():
    """Lecture 04, section 2: dt -> 0 leaves the state unchanged (token ignored);
    large dt resets the state to the current token's contribution."""
    g = rng(5)
    Bsz, L, D, N = 1, 6, 2, 3
    h0 = g.standard_normal((Bsz, D, N))
    u = g.standard_normal((Bsz, L, D))
    A = -np.exp(g.uniform(0.0, 2.0, (D, N)))
    Bm = g.standard_normal((Bsz, L, N))
    Cm = g.standard_normal((Bsz, L, N))
    _, h = O.selective_scan(u, np.full((Bsz, L, D), 1e-14), A, Bm, Cm, np.zeros(D), h0=h0)
    np.testing.assert_allclose(h, h0, rtol=1e-11, atol=1e-12)
    big = 1e3
    y, h = O.selective_scan(u, np.full((Bsz, L, D), big), A, Bm, Cm, np.zeros(D), h0=h0)
    np.testing.assert_allclose(h, big * Bm[:, -1, None, :] * u[:, -1, :, None], rtol=1e-12)
    np.testing.assert_allclose(y[:, -1], np.einsum("bdn,bn->bd", h, Cm[:, -1]), rtol=1e-12)


def test_scan_split_invariance():
    """Running the scan over [0, L1) and then [L1, L) from the carried state equals
    one run over [0, L) (how a prefix such as the meta rows fills the state)."""
    u, dt, A, Bm, Cm, Dv = _scan_inputs(6, L=15)
    y, h = O.selective_scan(u, dt, A, Bm, Cm, Dv)
    L1 = 6
    y1, h1 = O.selective_scan(u[:, :L1], dt[:, :L1], A, Bm[:, :L1], Cm[:, :L1], Dv)
    y2, h2 = O.selective_scan(u[:, L1:], dt[:, L1:], A, Bm[:, L1:], Cm[:, L1:], Dv, h0=h1)
    np.testing.assert_allclose(np.concatenate([y1, y2], 1), y, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(h2, h, rtol=1e-13, atol=1e-13)


def test_gate_special_cases():
    g = rng(7)
    y = g.standard_normal((2, 5, 3))
    z = g.standard_normal((2, 5, 3))
    np.testing.assert_array_equal(O.silu_gate(y, np.zeros_like(z)), 0.0)
    ref = y * torch.nn.functional.silu(torch.from_numpy(z)).numpy()
    np.testing.assert_allclose(O.silu_gate(y, z), ref, rtol=1e-14)
    # B = 0: the state stays zero and the branch output is D * u * silu(z)
    u, dt, A, Bm, Cm, Dv = _scan_inputs(8)
    ys, h = O.selective_scan(u, dt, A, np.zeros_like(Bm), Cm, Dv)
    np.testing.assert_array_equal(h, 0.0)
    zz = g.standard_normal(u.shape)
    np.testing.assert_allclose(O.silu_gate(ys, zz), Dv * u * zz / (1 + np.exp(-zz)), rtol=1e-14)


# ---------------------------------------------------------------------------
# rotary embedding


def test_rope_complex_formulation():
    g = rng(9)
    P, H, d, base = 13, 3, 64, 10000.0
    x = g.standard_normal((P, H, d))
    pos = np.arange(100, 100 + P)
    out = O.rope(x, pos, base)
    half = d // 2
    zc = x[..., :half] + 1j * x[..., half:]
    theta = base ** (-np.arange(half) * 2.0 / d)
    rot = zc * np.exp(1j * pos[:, None, None] * theta[None, None, :])
    np.testing.assert_allclose(out[..., :half], rot.real, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out[..., half:], rot.imag, rtol=1e-12, atol=1e-12)


def test_rope_identity_norm_and_relative_position():
    g = rng(10)
    d = 64
    q = g.standard_normal((1, 1, d))
    k = g.standard_normal((1, 1, d))
    np.testing.assert_array_equal(O.rope(q, np.array([0]), 1e4), q)
    qi = O.rope(q, np.array([37]), 1e4)
    np.testing.assert_allclose(np.linalg.norm(qi), np.linalg.norm(q), rtol=1e-14)
    dots = []
    for i, j in [(5, 2), (103, 100), (4003, 4000)]:
        dots.append(np.sum(O.rope(q, np.array([i]), 1e4) * O.rope(k, np.array([j]), 1e4)))
    np.testing.assert_allclose(dots, dots[0], rtol=1e-10)


# ---------------------------------------------------------------------------
# mask


@pytest.mark.parametrize("L,M,W", [(72, 8, 32), (40, 0, 7), (50, 5, 1), (33, 10, 0), (20, 25, 4), (64, 8, 100)])
def test_mask_ranges_closed_form(L, M, W):
    r = O.mask_ranges(L, M, W)
    i = np.arange(L)
    meta_end = np.minimum(M, i + 1)
    wb = np.maximum(M, i - W + 1) if W > 0 else np.full(L, M)
    we = i + 1
    empty = we <= wb
    wb = np.where(empty, M, wb)
    we = np.where(empty, M, we)
    cnt = np.minimum(i + 1, M + W) if W > 0 else i + 1
    np.testing.assert_array_equal(r[:, 0], meta_end)
    np.testing.assert_array_equal(r[:, 1], wb)
    np.testing.assert_array_equal(r[:, 2], we)
    np.testing.assert_array_equal(r[:, 3], cnt)
    np.testing.assert_array_equal(r[:, 3], r[:, 0] + r[:, 2] - r[:, 1])


def test_mask_window_covering_sequence_equals_global():
    L, M = 45, 6
    i, j = np.meshgrid(np.arange(L), np.arange(L), indexing="ij")
    glob = O.visible(i, j, M, 0)
    for W in (L - M, L, L + 17):
        np.testing.assert_array_equal(O.visible(i, j, M, W), glob)
    np.testing.assert_array_equal(glob, j <= i)


def test_mask_meta_always_visible():
    L, M = 60, 9
    i, j = np.meshgrid(np.arange(L), np.arange(L), indexing="ij")
    for W in (1, 2, 5, 30):
        vis = O.visible(i, j, M, W)
        np.testing.assert_array_equal(vis[:, :M], (j <= i)[:, :M])
    vis1 = O.visible(i, j, M, 1)
    np.testing.assert_array_equal(vis1, (j <= i) & ((j < M) | (j == i)))


# ---------------------------------------------------------------------------
# attention


def _attn_case(seed, Bsz=2, L=37, Hq=4, Hkv=2, d=16, dv=8):
    g = rng(seed)
    q = g.standard_normal((Bsz, L, Hq, d))
    k = g.standard_normal((Bsz, L, Hkv, d))
    v = g.standard_normal((Bsz, L, Hkv, dv))
    return q, k, v


@pytest.mark.parametrize("M,W", [(5, 8), (0, 0), (3, 1), (7, 100)])
def test_attention_matches_torch_sdpa(M, W):
    q, k, v = _attn_case(11)
    Bsz, L, Hq, d = q.shape
    Hkv = k.shape[2]
    out = O.attention(q, k, v, M, W)
    i, j = np.meshgrid(np.arange(L), np.arange(L), indexing="ij")
    mask = torch.from_numpy(O.visible(i, j, M, W))
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)
    kt = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, dim=1)
    vt = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
    np.testing.assert_allclose(out, ref.permute(0, 2, 1, 3).numpy(), rtol=1e-11, atol=1e-12)


def test_attention_zero_query_is_mean_of_visible_values():
    q, k, v = _attn_case(12)
    M, W = 4, 6
    out = O.attention(np.zeros_like(q), k, v, M, W)
    L = q.shape[1]
    for i in range(L):
        js = [j for j in range(L) if O.visible(i, j, M, W)]
        np.testing.assert_allclose(out[:, i, 0], v[:, js, 0].mean(axis=1), rtol=1e-12)
        np.testing.assert_allclose(out[:, i, 3], v[:, js, 1].mean(axis=1), rtol=1e-12)


def test_attention_window_one_no_meta_returns_own_value():
    q, k, v = _attn_case(13)
    out = O.attention(q, k, v, 0, 1)
    group = q.shape[2] // k.shape[2]
    for h in range(q.shape[2]):
        np.testing.assert_allclose(out[:, :, h], v[:, :, h // group], rtol=1e-14)


# ---------------------------------------------------------------------------
# fusion


def test_fuse_closed_forms():
    g = rng(14)
    R, W, eps = 6, 40, 1e-6
    ya = g.standard_normal((R, W)) * 3.0
    ys = g.standard_normal((R, W)) * 0.2
    one, zero = np.ones(W), np.zeros(W)
    oa = O.rms_fuse(ya, ys, one, zero, eps)
    os_ = O.rms_fuse(ya, ys, zero, one, eps)
    ms_a = np.mean(ya ** 2, axis=1)
    np.testing.assert_allclose(np.mean((2 * oa) ** 2, axis=1), ms_a / (ms_a + eps), rtol=1e-13)
    np.testing.assert_allclose(2 * oa, ya / np.sqrt(ms_a + eps)[:, None], rtol=1e-14)
    ba, bs = g.standard_normal(W), g.standard_normal(W)
    # linear in each beta
    np.testing.assert_allclose(O.rms_fuse(ya, ys, ba, bs, eps), ba * oa + bs * os_, rtol=1e-13, atol=1e-15)
    # mean of the two normalised branches
    np.testing.assert_allclose(O.rms_fuse(ya, ys, one, one, eps), oa + os_, rtol=1e-14)


# ---------------------------------------------------------------------------
# whole mixer: prefill / decode consistency


def _tiny_cfg(**kw):
    base = dict(batch=2, n_meta=3, n_tokens=10, d_inner=8, n_q_heads=4, n_kv_heads=2, head_dim=8,
                window=4, act="f32", seed=21)
    base.update(kw)
    return synth.config("tiny_f32").with_(**base)


@pytest.mark.parametrize("window", [4, 0, 1])
def test_decode_equals_prefill_of_one_more_row(window):
    cfg = _tiny_cfg(window=window)
    L = cfg.seq_rows
    full = synth.make_prefill_inputs(cfg)
    ref = O.mixer_prefill(cfg, full)
    # prefill on the first L-1 rows, then decode row L-1 from its caches and states
    short_cfg = cfg.with_(n_tokens=cfg.n_tokens - 1)
    short = {k: (v[:, :L - 1] if k in ("x", "z", "dt", "B", "C", "q", "k", "v") else v) for k, v in full.items()}
    pre = O.mixer_prefill(short_cfg, short)
    layer = {
        "x": full["x"][:, L - 1], "z": full["z"][:, L - 1], "dt": full["dt"][:, L - 1],
        "B": full["B"][:, L - 1], "C": full["C"][:, L - 1], "q": full["q"][:, L - 1],
        "ssm_state": pre["ssm_state"], "conv_state": pre["conv_state"],
        "A": full["A"], "conv_w": full["conv_w"], "D": full["D"],
        "beta_attn": full["beta_attn"], "beta_ssm": full["beta_ssm"],
    }
    k_cache = pre["k_rot"]
    v_cache = full["v"][:, :L - 1]
    cache_len = np.full(cfg.batch, L - 1)
    dec = O.mixer_decode(cfg, layer, k_cache, v_cache, full["k"][:, L - 1], full["v"][:, L - 1], cache_len)
    np.testing.assert_allclose(dec["y_ssm"], ref["y_ssm"][:, L - 1], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dec["y_attn"], ref["y_attn"][:, L - 1], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dec["out"], ref["out"][:, L - 1], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dec["ssm_state"], ref["ssm_state"], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dec["conv_state"], ref["conv_state"], rtol=0, atol=0)


def test_decode_shared_cache_is_read_only_and_layer_independent():
    cfg = synth.config("decode").with_(batch=3, d_inner=16, n_q_heads=4, n_kv_heads=2, head_dim=8,
                                       n_meta=4, window=6, cache_len=20, cache_capacity=24, act="f32")
    inp = synth.make_decode_inputs(cfg, cache_len=np.array([20, 9, 4], np.int32))
    kc, vc = inp["k_cache"].copy(), inp["v_cache"].copy()
    outs = [O.mixer_decode(cfg, inp["layers"][l], inp["k_cache"], inp["v_cache"], inp["k_new"], inp["v_new"],
                           inp["cache_len"]) for l in range(2)]
    np.testing.assert_array_equal(inp["k_cache"], kc)
    np.testing.assert_array_equal(inp["v_cache"], vc)
    # a private copy of the cache gives the same result as the shared buffer
    again = O.mixer_decode(cfg, inp["layers"][1], kc.copy(), vc.copy(), inp["k_new"], inp["v_new"], inp["cache_len"])
    np.testing.assert_array_equal(again["out"], outs[1]["out"])
    # rows at or beyond cache_len hold poison and must not influence the result
    kc2, vc2 = kc.copy(), vc.copy()
    for b, p in enumerate(inp["cache_len"]):
        kc2[b, p:] = -123.0
        vc2[b, p:] = 55.0
    again = O.mixer_decode(cfg, inp["layers"][0], kc2, vc2, inp["k_new"], inp["v_new"], inp["cache_len"])
    np.testing.assert_array_equal(again["out"], outs[0]["out"])


def test_tiny_config_runs_and_meta_rows_fill_state():
    cfg = synth.config("tiny_f32")
    inp = synth.make_prefill_inputs(cfg)
    res = O.mixer_prefill(cfg, inp)
    L, D = cfg.seq_rows, cfg.d_inner
    assert res["out"].shape == (1, L, D) and np.all(np.isfinite(res["out"]))
    # the state after the meta prefix differs from zero and changes the prompt rows' outputs
    M = cfg.n_meta
    cold = O.mixer_prefill(cfg.with_(n_meta=0), {**inp, **{k: inp[k][:, M:] for k in ("x", "z", "dt", "B", "C", "q", "k", "v")}})
    assert not np.allclose(cold["y_ssm"][0], res["y_ssm"][0, M:])


# ---------------------------------------------------------------------------
# cache sizes: the pages' worked examples


def test_kv_cache_worked_examples():
    with open(os.path.join(GOLDEN, "kv_cache_worked_examples.json")) as f:
        gold = json.load(f)["entries"]
    prev = None
    for e in gold:
        fn = getattr(O, e["fn"])
        b = fn(**e["args"])
        if "bytes" in e:
            assert b == e["bytes"], e["cite"]
            assert round(b / 2 ** 30, 2) == e["gib_printed"], e["cite"]
        if "gib_printed_2dp" in e:
            assert f"{b / 2 ** 30:.2f}" == e["gib_printed_2dp"], e["cite"]
        if "ratio_to_previous_1dp" in e:
            assert f"{prev / b:.1f}" == e["ratio_to_previous_1dp"], e["cite"]
        if "gb_approx" in e:
            assert abs(b / 1e9 - e["gb_approx"]) <= e["gb_tolerance"], (e["cite"], b / 1e9)
        if "ratio_to_previous_approx" in e:
            assert abs(b / prev - e["ratio_to_previous_approx"]) <= e["ratio_tolerance"], e["cite"]
        prev = b


# ---------------------------------------------------------------------------
# shared-KV key affine of a secondary layer (Hymba guide, "Systems Mechanics:
# Cross-Layer KV Cache Sharing")


def _affine(cfg, g, scale=True, bias=True):
    Hkv, d = cfg.n_kv_heads, cfg.head_dim
    ks = (0.5 + g.random((Hkv, d))) if scale else None
    kb = g.standard_normal((Hkv, d)) if bias else None
    return ks, kb


def test_key_affine_identity_and_bias_shift_invariance():
    """Unit scale and zero bias change nothing; a bias adds q . b to every
    score of a query row, a constant over its keys, which softmax removes."""
    cfg = _tiny_cfg(window=4)
    inp = synth.make_prefill_inputs(cfg)
    g = np.random.default_rng(5)
    plain = O.mixer_prefill(cfg, inp)
    unit = O.mixer_prefill(cfg, {**inp, "k_scale": np.ones((cfg.n_kv_heads, cfg.head_dim)),
                                 "k_bias": np.zeros((cfg.n_kv_heads, cfg.head_dim))})
    np.testing.assert_array_equal(unit["y_attn"], plain["y_attn"])
    ks, kb = _affine(cfg, g)
    scaled = O.mixer_prefill(cfg, {**inp, "k_scale": ks})
    both = O.mixer_prefill(cfg, {**inp, "k_scale": ks, "k_bias": kb})
    np.testing.assert_allclose(both["y_attn"], scaled["y_attn"], rtol=1e-11, atol=1e-13)
    # and the scale does change the result (it reshapes every head's scores)
    assert np.max(np.abs(scaled["y_attn"] - plain["y_attn"])) > 1e-3
    # the cache content a prefill returns is the plain rotated keys
    np.testing.assert_array_equal(both["k_rot"], plain["k_rot"])


def test_key_affine_scale_equals_query_scale_of_its_group():
    """(q . (k (.) w)) = ((q (.) w) . k): scaling every query head of kv group
    g by w[g] instead of the keys gives the same attention, which pins the
    head-to-group mapping of the per-kv-head vectors."""
    cfg = _tiny_cfg(window=0, n_q_heads=4, n_kv_heads=2)
    inp = synth.make_prefill_inputs(cfg)
    g = np.random.default_rng(6)
    ks, _ = _affine(cfg, g, bias=False)
    L = cfg.seq_rows
    pos = np.arange(L)
    q_rot = O.rope(inp["q"], pos, cfg.rope_base)
    k_rot = O.rope(inp["k"], pos, cfg.rope_base)
    group = cfg.n_q_heads // cfg.n_kv_heads
    q_scaled = q_rot * np.repeat(ks, group, axis=0)[None, None]     # query head h uses w[h // group]
    via_q = O.attention(q_scaled, k_rot, inp["v"], cfg.n_meta, cfg.window)
    via_k = O.attention(q_rot, O.shared_key_affine(k_rot, ks), inp["v"], cfg.n_meta, cfg.window)
    np.testing.assert_allclose(via_k, via_q, rtol=1e-12, atol=1e-13)
    ref = O.mixer_prefill(cfg, {**inp, "k_scale": ks})
    np.testing.assert_allclose(ref["y_attn"], via_k.reshape(cfg.batch, L, -1), rtol=1e-13, atol=1e-14)


def test_key_affine_decode_equals_prefill_of_one_more_row():
    """A secondary layer's decode step (affine over the shared cache and the
    new key) equals its prefill of one more row."""
    cfg = _tiny_cfg(window=4)
    L = cfg.seq_rows
    full = synth.make_prefill_inputs(cfg)
    ks, kb = _affine(cfg, np.random.default_rng(7))
    ref = O.mixer_prefill(cfg, {**full, "k_scale": ks, "k_bias": kb})
    short_cfg = cfg.with_(n_tokens=cfg.n_tokens - 1)
    short = {k: (v[:, :L - 1] if k in ("x", "z", "dt", "B", "C", "q", "k", "v") else v) for k, v in full.items()}
    pre = O.mixer_prefill(short_cfg, short)
    layer = {k: full[k][:, L - 1] for k in ("x", "z", "dt", "B", "C", "q")}
    layer.update(ssm_state=pre["ssm_state"], conv_state=pre["conv_state"], k_scale=ks, k_bias=kb,
                 **{k: full[k] for k in ("A", "conv_w", "D", "beta_attn", "beta_ssm")})
    dec = O.mixer_decode(cfg, layer, pre["k_rot"], full["v"][:, :L - 1], full["k"][:, L - 1], full["v"][:, L - 1],
                         np.full(cfg.batch, L - 1))
    np.testing.assert_allclose(dec["y_attn"], ref["y_attn"][:, L - 1], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dec["out"], ref["out"][:, L - 1], rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# continuing a prefill from its state, and the compact sliding-window cache
# (Hymba-1.5B article, section 1; Lecture 04, sections 1 and 2)

_PER_ROW = ("x", "z", "dt", "B", "C", "q", "k", "v")


def _rows(full, a, b):
    return {k: (v[:, a:b] if k in _PER_ROW else v) for k, v in full.items()}


def _chain(cfg, full, cuts, ring):
    """Prefill of rows [0, cuts[0]) then one continuation per later cut; the
    cache is one row per position or the compact ring. Returns the
    concatenated outputs, the final states and the cache."""
    L, M, W = cfg.seq_rows, cfg.n_meta, cfg.window
    Hkv, d, dv = cfg.n_kv_heads, cfg.head_dim, cfg.head_dim_v
    cap = M + W if ring else L
    pre = O.mixer_prefill(cfg.with_(n_tokens=cuts[0] - M), _rows(full, 0, cuts[0]))
    first = np.arange(cuts[0])
    kc = O.cache_store(np.zeros((cfg.batch, cap, Hkv, d)), pre["k_rot"], first, M, W, ring)
    vc = O.cache_store(np.zeros((cfg.batch, cap, Hkv, dv)), full["v"][:, :cuts[0]], first, M, W, ring)
    outs = {k: [pre[k]] for k in ("y_ssm", "y_attn", "out")}
    state, conv = pre["ssm_state"], pre["conv_state"]
    for a, b in zip(cuts, list(cuts[1:]) + [L]):
        r = O.mixer_prefill_continue(cfg.with_(n_tokens=b - a), _rows(full, a, b), a, state, conv, kc, vc,
                                     ring=ring)
        for k in outs:
            outs[k].append(r[k])
        state, conv, kc, vc = r["ssm_state"], r["conv_state"], r["k_cache"], r["v_cache"]
    res = {k: np.concatenate(v, axis=1) for k, v in outs.items()}
    res.update(ssm_state=state, conv_state=conv, k_cache=kc, v_cache=vc)
    return res


@pytest.mark.parametrize("ring", [False, True])
@pytest.mark.parametrize("cuts", [[3], [3, 4, 5], [5, 6, 11], [8, 12]])
def test_continuation_equals_one_prefill(ring, cuts):
    """Cutting a prefill anywhere after the meta rows and continuing from the
    carried state (SSM state, conv history, cache) gives the rows of one
    prefill: chunks of one row (conv history from the state) and chunks
    longer than the window (ring rows replaced within a chunk) included."""
    cfg = _tiny_cfg(n_meta=3, n_tokens=11, window=4)
    full = synth.make_prefill_inputs(cfg)
    ref = O.mixer_prefill(cfg, full)
    got = _chain(cfg, full, cuts, ring)
    for k in ("y_ssm", "y_attn", "out"):
        np.testing.assert_allclose(got[k], ref[k], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(got["ssm_state"], ref["ssm_state"], rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(got["conv_state"], ref["conv_state"])
    L, M, W = cfg.seq_rows, cfg.n_meta, cfg.window
    if ring:   # the meta rows and the last W positions, each in its ring row
        keep = np.concatenate([np.arange(M), np.arange(L - W, L)])
        rows = O.ring_slot(keep, M, W)
        np.testing.assert_array_equal(np.sort(rows), np.arange(M + W))
        np.testing.assert_allclose(got["k_cache"][:, rows], ref["k_rot"][:, keep], rtol=0, atol=1e-14)
        np.testing.assert_array_equal(got["v_cache"][:, rows], full["v"][:, keep])
    else:
        np.testing.assert_allclose(got["k_cache"], ref["k_rot"], rtol=0, atol=1e-14)
        np.testing.assert_array_equal(got["v_cache"], full["v"])


def test_continuation_global_layer_and_sequences_independent():
    cfg = _tiny_cfg(n_meta=2, n_tokens=9, window=0, batch=3)
    full = synth.make_prefill_inputs(cfg)
    ref = O.mixer_prefill(cfg, full)
    got = _chain(cfg, full, [4, 9], ring=False)
    np.testing.assert_allclose(got["out"], ref["out"], rtol=1e-12, atol=1e-12)
    with pytest.raises(ValueError):
        O.ring_slot([5], 2, 0)   # a global layer has no compact form


def test_ring_slot_closed_form_and_no_visible_row_lost():
    M, W = 3, 4
    p = np.arange(40)
    s = O.ring_slot(p, M, W)
    np.testing.assert_array_equal(s[:M + W], np.arange(M + W))          # first pass fills the rows in order
    np.testing.assert_array_equal(s[M:], M + (p[M:] - M) % W)
    assert s.max() == M + W - 1                                        # capacity n_meta + window
    for q in range(M, 40 - W):                                         # W consecutive positions: W distinct rows
        assert len(set(s[q:q + W])) == W
    # storing positions 0 .. p - 1 in order leaves every position that a query
    # at p can see in its row (no later position below p took that row)
    for pq in range(M, 40):
        owner = {}
        for q in range(pq):
            owner[int(s[q])] = q
        for q in O.visible_history(pq, M, W):
            assert owner[int(s[q])] == q, (pq, q)
        assert len(O.visible_history(pq, M, W)) == min(pq, M + W - 1)


@pytest.mark.parametrize("window", [4, 1])
def test_decode_on_the_ring_equals_decode_on_the_full_cache(window):
    """A decode step reads the same keys from the compact ring as from one row
    per position, also far past the ring's capacity."""
    cfg = _tiny_cfg(n_meta=3, window=window).with_(decode=True, cache_capacity=64, n_layers=1)
    for p in (3, 5, 3 + window, 29, 63):
        inp = synth.make_decode_inputs(cfg, cache_len=np.full(cfg.batch, p, np.int32))
        ring_k = O.cache_store(np.zeros((cfg.batch, cfg.n_meta + window, cfg.n_kv_heads, cfg.head_dim)),
                               inp["k_cache"][:, :p], np.arange(p), cfg.n_meta, window, True)
        ring_v = O.cache_store(np.zeros((cfg.batch, cfg.n_meta + window, cfg.n_kv_heads, cfg.head_dim_v)),
                               inp["v_cache"][:, :p], np.arange(p), cfg.n_meta, window, True)
        lay = inp["layers"][0]
        a = O.mixer_decode(cfg, lay, inp["k_cache"], inp["v_cache"], inp["k_new"], inp["v_new"], inp["cache_len"])
        b = O.mixer_decode(cfg, lay, ring_k, ring_v, inp["k_new"], inp["v_new"], inp["cache_len"], ring=True)
        np.testing.assert_allclose(b["out"], a["out"], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(b["y_attn"], a["y_attn"], rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------------------
# the Mamba-2 form: one decay rate and one step size per head (Lecture 04,
# section 3: scalar-times-identity state matrix, recurrence and matmul forms)


def _ssd_case(seed, Bsz=2, L=13, H=3, P=4, N=5):
    g = np.random.default_rng(seed)
    return dict(u=g.standard_normal((Bsz, L, H * P)), dt=g.uniform(0.01, 0.6, (Bsz, L, H)),
                A=-g.uniform(0.3, 4.0, H), Bm=g.standard_normal((Bsz, L, N)), Cm=g.standard_normal((Bsz, L, N)),
                D=g.standard_normal(H * P), h0=g.standard_normal((Bsz, H * P, N)), P=P)


def test_ssd_is_the_selective_scan_with_one_rate_per_head():
    c = _ssd_case(31)
    P, N = c["P"], c["Bm"].shape[2]
    A_exp = np.repeat(c["A"], P)[:, None] * np.ones((1, N))          # A[c, n] = A[c // P]
    dt_exp = np.repeat(c["dt"], P, axis=2)                            # dt[b, t, c] = dt[b, t, c // P]
    for h0 in (None, c["h0"]):
        y1, s1 = O.ssd_scan(c["u"], c["dt"], c["A"], c["Bm"], c["Cm"], c["D"], h0=h0)
        y2, s2 = O.selective_scan(c["u"], dt_exp, A_exp, c["Bm"], c["Cm"], c["D"], h0=h0)
        np.testing.assert_allclose(y1, y2, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(s1, s2, rtol=1e-12, atol=1e-12)


def test_ssd_dual_form_is_a_masked_product():
    """Zero initial state: per head, Y = (Lmask . (C B^T)) (dt x) + D x with
    Lmask[i, j] = exp(A (s_i - s_j)) for j <= i and 0 above the diagonal,
    s the running sum of dt: the quadratic, attention-like way to compute
    the same layer."""
    c = _ssd_case(32)
    u, dt, A, Bm, Cm, D, P = c["u"], c["dt"], c["A"], c["Bm"], c["Cm"], c["D"], c["P"]
    Bsz, L, Dch = u.shape
    y_ref, _ = O.ssd_scan(u, dt, A, Bm, Cm, D)
    y = np.zeros_like(u)
    for b in range(Bsz):
        for h in range(len(A)):
            s = np.cumsum(dt[b, :, h])
            i, j = np.meshgrid(np.arange(L), np.arange(L), indexing="ij")
            Lm = np.where(j <= i, np.exp(A[h] * (s[i] - s[j])), 0.0)
            X = u[b, :, h * P:(h + 1) * P]
            y[b, :, h * P:(h + 1) * P] = (Lm * (Cm[b] @ Bm[b].T)) @ (dt[b, :, h, None] * X) + D[h * P:(h + 1) * P] * X
    np.testing.assert_allclose(y, y_ref, rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("Q", [1, 4, 5, 13])
def test_ssd_block_decomposition(Q):
    """The chunked form: within a chunk the masked product, plus the carried
    state decayed to each row; chunk end states chained by the chunk's total
    decay. Equal to the recurrence for any chunk length."""
    c = _ssd_case(33)
    u, dt, A, Bm, Cm, D, P, h0 = c["u"], c["dt"], c["A"], c["Bm"], c["Cm"], c["D"], c["P"], c["h0"]
    Bsz, L, Dch = u.shape
    H, N = len(A), Bm.shape[2]
    y_ref, s_ref = O.ssd_scan(u, dt, A, Bm, Cm, D, h0=h0)
    y = np.zeros_like(u)
    state = h0.reshape(Bsz, H, P, N).copy()
    for t0 in range(0, L, Q):
        t1 = min(t0 + Q, L)
        for b in range(Bsz):
            for h in range(H):
                S = A[h] * np.cumsum(dt[b, t0:t1, h])                  # inclusive, from the chunk start
                X = u[b, t0:t1, h * P:(h + 1) * P] * dt[b, t0:t1, h, None]
                i, j = np.meshgrid(np.arange(t1 - t0), np.arange(t1 - t0), indexing="ij")
                M = np.where(j <= i, np.exp(S[i] - S[j]), 0.0) * (Cm[b, t0:t1] @ Bm[b, t0:t1].T)
                Hs = state[b, h]                                       # [P, N], entering the chunk
                y[b, t0:t1, h * P:(h + 1) * P] = (M @ X + np.exp(S)[:, None] * (Cm[b, t0:t1] @ Hs.T)
                                                  + D[h * P:(h + 1) * P] * u[b, t0:t1, h * P:(h + 1) * P])
                w = np.exp(S[-1] - S)                                  # decay of each row to the chunk end
                state[b, h] = np.exp(S[-1]) * Hs + (X * w[:, None]).T @ Bm[b, t0:t1]
    np.testing.assert_allclose(y, y_ref, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(state.reshape(Bsz, Dch, N), s_ref, rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("ring", [False, True])
def test_ssd_mixer_continuation_and_decode(ring):
    """The mixer with the Mamba-2 form: a continued prefill equals one prefill,
    and a decode step equals the prefill of one more row."""
    cfg = _tiny_cfg(n_meta=3, n_tokens=11, window=4, ssm_heads=2)
    full = synth.make_prefill_inputs(cfg)
    assert full["A"].shape == (2,) and full["dt"].shape == (cfg.batch, cfg.seq_rows, 2)
    ref = O.mixer_prefill(cfg, full)
    got = _chain(cfg, full, [5, 6, 11], ring)
    for k in ("y_ssm", "y_attn", "out"):
        np.testing.assert_allclose(got[k], ref[k], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(got["ssm_state"], ref["ssm_state"], rtol=1e-12, atol=1e-13)
    L = cfg.seq_rows
    short = {k: (v[:, :L - 1] if k in _PER_ROW else v) for k, v in full.items()}
    pre = O.mixer_prefill(cfg.with_(n_tokens=cfg.n_tokens - 1), short)
    layer = {k: full[k][:, L - 1] for k in ("x", "z", "dt", "B", "C", "q")}
    layer.update(ssm_state=pre["ssm_state"], conv_state=pre["conv_state"],
                 **{k: full[k] for k in ("A", "conv_w", "D", "beta_attn", "beta_ssm")})
    dec = O.mixer_decode(cfg, layer, pre["k_rot"], full["v"][:, :L - 1], full["k"][:, L - 1], full["v"][:, L - 1],
                         np.full(cfg.batch, L - 1))
    np.testing.assert_allclose(dec["out"], ref["out"][:, L - 1], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dec["ssm_state"], ref["ssm_state"], rtol=1e-12, atol=1e-13)
