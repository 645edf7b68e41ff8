"""GPU parity of a prefill continued from its state (chunked prefill) and of the
compact sliding-window cache, through the C ABI, against the float64 oracle.

A chain of calls (a fresh prefill, then continuations) must give the rows of
one prefill of the whole sequence: the oracle's pins establish that
equivalence, so the reference here is the oracle's one-call prefill. The
compact cache is checked row by row against the oracle's ring layout, and a
decode step over it against the oracle's decode on that layout."""
import numpy as np
import pytest
import torch

import oracle as O
import synth

pytestmark = pytest.mark.gpu

H = pytest.importorskip("attention_lm_amd")
from harness import TOL, TORCH_DT, Decode, desc_for, dev, host, rel_l2  # noqa: E402
from harness import check as _check  # noqa: E402

PER_ROW = ("x", "z", "dt", "B", "C", "q", "k", "v")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    H.load_library()


def say(*a):
    print(*a, flush=True)


def check(name, got, ref, tol, slice_width=128):
    if tol == 0.0:   # copies of stored values: bitwise
        np.testing.assert_array_equal(np.asarray(got), np.asarray(ref), err_msg=name)
        say(f"  {name:14s} bit-exact")
        return
    _check(name, got, ref, tol, slice_width=slice_width, say=say)


def run_chain(cfg, full, cuts, ring):
    """Fresh prefill of rows [0, cuts[0]), then one continuation per later cut.
    Returns the concatenated outputs and the final states and caches (host)."""
    act, dt_ = cfg.act, TORCH_DT[cfg.act]
    L, M, W = cfg.seq_rows, cfg.n_meta, cfg.window
    Bsz, D, Hkv = cfg.batch, cfg.d_inner, cfg.n_kv_heads
    cap = M + W if ring else L
    par = {k: dev(full[k]) for k in ("A", "D", "conv_w", "beta_attn", "beta_ssm")}
    params = H.make_params(par["A"], par["D"], par["conv_w"], par["beta_attn"], par["beta_ssm"])
    kc = torch.full((Bsz, cap, Hkv, cfg.head_dim), 7.0, dtype=dt_, device="cuda")
    vc = torch.full((Bsz, cap, Hkv, cfg.head_dim_v), 7.0, dtype=dt_, device="cuda")
    state = torch.empty((Bsz, D, cfg.d_state), dtype=torch.float32, device="cuda")
    conv = torch.empty((Bsz, D, cfg.d_conv - 1), dtype=dt_, device="cuda")
    outs = {"out": [], "y_attn": [], "y_ssm": []}
    bounds = [0] + list(cuts) + [L]
    for i, (a, b) in enumerate(zip(bounds[:-1], bounds[1:])):
        if b <= a:
            continue
        t = {k: dev(full[k][:, a:b], act) for k in PER_ROW}
        o = {k: torch.empty((Bsz, b - a, D), dtype=dt_, device="cuda") for k in outs}
        if i == 0:
            say(f" prefill rows [0, {b})")
            desc = desc_for(cfg.with_(n_tokens=b - M), cache_capacity=cap, cache_ring=ring)
            H.hymba_mixer_prefill(desc, params, *[t[k] for k in PER_ROW], o["out"], ssm_state_out=state,
                                  conv_state_out=conv, k_cache=kc, v_cache=vc, y_attn_out=o["y_attn"],
                                  y_ssm_out=o["y_ssm"])
        else:
            say(f" continue rows [{a}, {b})")
            desc = desc_for(cfg.with_(n_tokens=b - a), cache_capacity=cap, cache_ring=ring)
            H.hymba_mixer_prefill_continue(desc, params, a, *[t[k] for k in PER_ROW], o["out"], state, conv, kc,
                                           vc, y_attn_out=o["y_attn"], y_ssm_out=o["y_ssm"])
        torch.cuda.synchronize()
        for k in outs:
            outs[k].append(host(o[k]))
    res = {k: np.concatenate(v, axis=1) for k, v in outs.items()}
    res.update(ssm_state=host(state), conv_state=host(conv), k_cache=host(kc), v_cache=host(vc))
    return res


def check_chain(cfg, cuts, ring, rows=None):
    say(f"chain {cfg.name}: B={cfg.batch} L={cfg.seq_rows} M={cfg.n_meta} W={cfg.window} act={cfg.act} "
        f"cuts={cuts} ring={ring}")
    full = synth.make_prefill_inputs(cfg)
    got = run_chain(cfg, full, cuts, ring)
    ref = O.mixer_prefill(cfg, full, rows=rows)
    rsel = ref["rows"]
    tol = TOL[cfg.act]
    check("y_ssm", got["y_ssm"], ref["y_ssm"], tol)
    check("y_attn", got["y_attn"][:, rsel], ref["y_attn"], tol, slice_width=cfg.head_dim_v)
    check("out", got["out"][:, rsel], ref["out"], tol)
    check("ssm_state", got["ssm_state"], ref["ssm_state"], tol, slice_width=cfg.d_state)
    check("conv_state", got["conv_state"], ref["conv_state"], 0.0)
    L, M, W = cfg.seq_rows, cfg.n_meta, cfg.window
    keep = np.concatenate([np.arange(M), np.arange(max(M, L - W), L)]) if ring else np.arange(L)
    crow = O.cache_rows(keep, M, W, ring)
    check("k_cache", got["k_cache"][:, crow], ref["k_rot"][:, keep], tol, slice_width=cfg.head_dim)
    np.testing.assert_array_equal(got["v_cache"][:, crow], full["v"][:, keep])
    return full, got


CHAINS = [
    # bf16 window 40: a 2-row chunk (conv history from the state), a chunk longer than the window
    (dict(batch=2, n_meta=5, n_tokens=150, d_inner=320, n_q_heads=5, n_kv_heads=1, window=40, act="bf16",
          seed=51), [55, 57, 140]),
    # fp32, first call holds only the meta rows, then a single row, then the rest
    (dict(batch=1, n_meta=8, n_tokens=100, d_inner=256, n_q_heads=4, n_kv_heads=2, window=16, act="f32",
          seed=52), [8, 9, 60]),
    # GQA group 8, dv 32, window 1 (each row sees the meta rows and itself)
    (dict(batch=2, n_meta=3, n_tokens=70, d_inner=256, n_q_heads=8, n_kv_heads=1, window=1, act="bf16",
          seed=53), [10, 11, 45]),
    # a batch that takes the single-pass scan: the carried state and conv history
    # enter its registers and its first block's history rows
    (dict(batch=32, n_meta=4, n_tokens=40, d_inner=1024, n_q_heads=8, n_kv_heads=2, window=12, act="bf16",
          seed=55), [4, 6, 29]),
]


@pytest.mark.parametrize("ring", [False, True], ids=["rows", "ring"])
@pytest.mark.parametrize("kw,cuts", CHAINS, ids=[f"chain{i}" for i in range(len(CHAINS))])
def test_continuation_chain(kw, cuts, ring):
    cfg = synth.config("tiny_f32").with_(**kw, name="chain")
    check_chain(cfg, cuts, ring)


def test_continuation_global_layer():
    cfg = synth.config("tiny_f32").with_(batch=2, n_meta=6, n_tokens=120, d_inner=320, n_q_heads=5, n_kv_heads=1,
                                         window=0, act="bf16", seed=54, name="chain_global")
    check_chain(cfg, [40, 41, 100], ring=False)


@pytest.mark.parametrize("ring", [False, True], ids=["rows", "ring"])
def test_continuation_swa_layer_sampled(ring):
    """The 1.5B-shaped window-1024 layer prefilled in three calls (chunks of
    1024 and 1000 rows continue a 152-row start): sampled rows of every chunk."""
    cfg = synth.config("swa_layer")
    rows = np.unique(np.concatenate([np.arange(0, 2176, 17), [151, 152, 153, 1175, 1176, 1177, 2175]]))
    check_chain(cfg, [152, 1176], ring, rows=rows)


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_decode_on_the_compact_cache(act):
    """Decode over the ring, positions at, inside and far past its capacity,
    two layers (the second through its key affine) against the oracle's
    decode on the same ring."""
    M, W = 8, 50
    lens = np.array([8, 20, 58, 300, 5000], np.int32)
    base = synth.config("decode_affine").with_(batch=len(lens), d_inner=320, n_q_heads=5, n_kv_heads=1, n_meta=M, window=W,
                                        cache_capacity=int(lens.max()), act=act, name="dring")
    inp = synth.make_decode_inputs(base, cache_len=lens)
    ring_k = np.zeros((base.batch, M + W, 1, 64), np.float32)
    ring_v = np.zeros((base.batch, M + W, 1, base.head_dim_v), np.float32)
    for b, p in enumerate(lens):   # each sequence's rows below p, in position order, into the ring
        ring_k[b] = O.cache_store(ring_k[b:b + 1], inp["k_cache"][b:b + 1, :p], np.arange(p), M, W, True)[0]
        ring_v[b] = O.cache_store(ring_v[b:b + 1], inp["v_cache"][b:b + 1, :p], np.arange(p), M, W, True)[0]
    cfg = base.with_(cache_capacity=M + W)
    rinp = dict(inp, k_cache=ring_k, v_cache=ring_v)
    run = Decode(cfg, rinp)
    run.desc = desc_for(cfg, cache_ring=True)
    run.ws = torch.empty(max(H.hymba_mixer_decode_workspace_bytes(run.desc), 256), dtype=torch.uint8, device="cuda")
    kc0 = run.k_cache.clone()
    for l in range(cfg.n_layers):
        run.call(l)
    torch.cuda.synchronize()
    assert torch.equal(run.k_cache, kc0)
    tol = TOL[act]
    for l in range(cfg.n_layers):
        ref = O.mixer_decode(cfg, rinp["layers"][l], host(run.k_cache), host(run.v_cache), inp["k_new"],
                             inp["v_new"], lens, ring=True)
        L_ = run.layers[l]
        say(f" layer {l}")
        check("y_attn", host(L_["y_attn_out"]), ref["y_attn"], tol)
        check("out", host(L_["out"]), ref["out"], tol)
        check("ssm_state", host(L_["ssm_state"]), ref["ssm_state"], tol)


def test_ring_prefill_then_decode():
    """Prefill into the compact cache (a fresh call and a continuation), then
    a decode step at the next position: the oracle's prefill of one more row."""
    cfg = synth.config("tiny_f32").with_(batch=2, n_meta=6, n_tokens=91, d_inner=320, n_q_heads=5, n_kv_heads=1,
                                         window=33, act="bf16", seed=55, name="ring_dec")
    full = synth.make_prefill_inputs(cfg)
    L = cfg.seq_rows
    short_cfg = cfg.with_(n_tokens=cfg.n_tokens - 1)
    short = {k: (v[:, :L - 1] if k in PER_ROW else v) for k, v in full.items()}
    got = run_chain(short_cfg, short, [40], ring=True)
    M, W = cfg.n_meta, cfg.window
    dcfg = cfg.with_(decode=True, cache_capacity=M + W, n_layers=1)
    layer = {k: full[k][:, L - 1] for k in ("x", "z", "dt", "B", "C", "q")}
    layer.update(ssm_state=got["ssm_state"].astype(np.float32), conv_state=got["conv_state"],
                 **{k: full[k] for k in ("A", "D", "conv_w", "beta_attn", "beta_ssm")})
    inp = {"k_cache": got["k_cache"], "v_cache": got["v_cache"], "k_new": full["k"][:, L - 1],
           "v_new": full["v"][:, L - 1], "cache_len": np.full(cfg.batch, L - 1, np.int32), "layers": [layer]}
    run = Decode(dcfg, inp)
    run.desc = desc_for(dcfg, cache_ring=True)
    run.ws = torch.empty(max(H.hymba_mixer_decode_workspace_bytes(run.desc), 256), dtype=torch.uint8, device="cuda")
    run.call(0)
    torch.cuda.synchronize()
    ref = O.mixer_prefill(cfg, full, rows=np.array([L - 1]))
    check("y_ssm", host(run.layers[0]["y_ssm_out"]), ref["y_ssm"][:, L - 1], 5e-3)
    check("y_attn", host(run.layers[0]["y_attn_out"]), ref["y_attn"][:, 0], 5e-3)
    check("out", host(run.layers[0]["out"]), ref["out"][:, 0], 5e-3)


SSD_CHAINS = [
    # bf16, head width 64
    (dict(batch=2, n_meta=5, n_tokens=200, d_inner=256, n_q_heads=2, n_kv_heads=1, window=40, act="bf16", seed=65,
          ssm_heads=4), [55, 57, 140]),
    # fp32, head width 32 (four waves share each channel tile); a first call of the meta rows alone
    (dict(batch=2, n_meta=5, n_tokens=150, d_inner=128, n_q_heads=2, n_kv_heads=1, window=20, act="f32", seed=66,
          ssm_heads=4), [5, 70, 100]),
    # bf16, head width 128 (two channel tiles per wave); a call of exactly one chunk
    (dict(batch=1, n_meta=8, n_tokens=180, d_inner=256, n_q_heads=4, n_kv_heads=2, window=50, act="bf16", seed=67,
          ssm_heads=2), [64, 65, 130]),
]


@pytest.mark.parametrize("ring", [False, True], ids=["rows", "ring"])
@pytest.mark.parametrize("kw,cuts", SSD_CHAINS, ids=[f"ssdchain{i}" for i in range(len(SSD_CHAINS))])
def test_continuation_chain_ssd(kw, cuts, ring):
    """A chain of calls with the Mamba-2 form: the carried state enters the
    block form's chain, the conv history its first chunk."""
    cfg = synth.config("tiny_f32").with_(**kw, name="chain_ssd")
    check_chain(cfg, cuts, ring)
