"""The C ABI's calls captured into HIP graphs (torch.cuda.graph on the calling
stream; one branch of the prefill forks onto the library's second stream and
joins back inside the capture). Every replay must equal the eager call bit for
bit, with the program's own eager work and synchronizations between replays:
outputs cleared, and for the calls that update state in place (continuation,
decode) the state restored to what the eager call started from."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

H = pytest.importorskip("attention_lm_amd")
from harness import TORCH_DT, Decode, Prefill, desc_for, dev  # noqa: E402

PER_ROW_INPUTS = ("x", "z", "dt", "B", "C", "q", "k", "v")

REPLAYS = 3


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    H.load_library()


def snap(ts):
    return {k: v.clone() for k, v in ts.items()}


def capture(fn):
    """One eager call on a side stream (first-use set-up stays out of the
    capture), then the call captured into a graph."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def replay_and_check(g, outs, ref, before=None, start=None):
    for i in range(REPLAYS):
        for t in outs.values():
            t.zero_()
        if start is not None:
            for k, v in start.items():
                before[k].copy_(v)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in ref.items():
            assert torch.equal(outs[k], v), f"replay {i}: {k} differs from the eager call"


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_prefill_graph(act):
    cfg = synth.config("tiny_f32").with_(batch=2, n_meta=5, n_tokens=150, d_inner=320, n_q_heads=5, n_kv_heads=1,
                                          window=40, act=act, seed=91, name="graph_prefill")
    run = Prefill(cfg, synth.make_prefill_inputs(cfg))
    outs = dict(run.o, out=run.out)
    run()
    torch.cuda.synchronize()
    ref = snap(outs)
    replay_and_check(capture(run), outs, ref)


def test_prefill_graph_attention_branch_first():
    """A geometry whose attention branch is the longer one: the Mamba branch
    forks onto the second stream after the RoPE pass, inside the capture."""
    from test_gpu_parity import LATE_FORK, attention_outweighs_scan
    cfg = synth.config("tiny_f32").with_(**LATE_FORK, name="graph_late_fork")
    assert attention_outweighs_scan(cfg)
    run = Prefill(cfg, synth.make_prefill_inputs(cfg))
    outs = dict(run.o, out=run.out)
    run()
    torch.cuda.synchronize()
    ref = snap(outs)
    replay_and_check(capture(run), outs, ref)


def test_prefill_continue_graph():
    """A continuation on the compact cache: its carried conv history is staged
    by a device copy inside the call, and state, conv history and cache are
    updated in place."""
    cfg = synth.config("tiny_f32").with_(batch=2, n_meta=6, n_tokens=120, d_inner=320, n_q_heads=5, n_kv_heads=1,
                                          window=24, act="bf16", seed=92, name="graph_cont")
    full = synth.make_prefill_inputs(cfg)
    dt_ = TORCH_DT[cfg.act]
    M, W, L = cfg.n_meta, cfg.window, cfg.seq_rows
    Bsz, D = cfg.batch, cfg.d_inner
    cap, a = M + W, 70
    par = {k: dev(full[k]) for k in ("A", "D", "conv_w", "beta_attn", "beta_ssm")}
    params = H.make_params(par["A"], par["D"], par["conv_w"], par["beta_attn"], par["beta_ssm"])
    st = {"kc": torch.full((Bsz, cap, cfg.n_kv_heads, cfg.head_dim), 7.0, dtype=dt_, device="cuda"),
          "vc": torch.full((Bsz, cap, cfg.n_kv_heads, cfg.head_dim_v), 7.0, dtype=dt_, device="cuda"),
          "state": torch.empty((Bsz, D, cfg.d_state), dtype=torch.float32, device="cuda"),
          "conv": torch.empty((Bsz, D, cfg.d_conv - 1), dtype=dt_, device="cuda")}
    first = {k: dev(full[k][:, :a], cfg.act) for k in PER_ROW_INPUTS}
    out0 = torch.empty((Bsz, a, D), dtype=dt_, device="cuda")
    H.hymba_mixer_prefill(desc_for(cfg.with_(n_tokens=a - M), cache_capacity=cap, cache_ring=True), params,
                          *[first[k] for k in PER_ROW_INPUTS], out0, ssm_state_out=st["state"],
                          conv_state_out=st["conv"], k_cache=st["kc"], v_cache=st["vc"])
    torch.cuda.synchronize()
    start = snap(st)
    rest = {k: dev(full[k][:, a:], cfg.act) for k in PER_ROW_INPUTS}
    outs = {k: torch.empty((Bsz, L - a, D), dtype=dt_, device="cuda") for k in ("out", "y_attn", "y_ssm")}
    desc = desc_for(cfg.with_(n_tokens=L - a), cache_capacity=cap, cache_ring=True)
    ws = torch.empty(max(H.hymba_mixer_prefill_workspace_bytes(desc), 256), dtype=torch.uint8, device="cuda")

    def cont():
        H.hymba_mixer_prefill_continue(desc, params, a, *[rest[k] for k in PER_ROW_INPUTS], outs["out"],
                                       st["state"], st["conv"], st["kc"], st["vc"], y_attn_out=outs["y_attn"],
                                       y_ssm_out=outs["y_ssm"], workspace=ws)

    cont()
    torch.cuda.synchronize()
    ref = snap(dict(outs, **st))
    for k, v in start.items():
        st[k].copy_(v)
    g = capture(cont)   # (its eager warm-up call moved the state on again)
    replay_and_check(g, dict(outs, **st), ref, before=st, start=start)


def test_decode_graph():
    """A two-layer decode step over one shared cache; each layer updates its
    SSM state and conv history in place."""
    cfg = synth.config("decode_affine").with_(batch=5, d_inner=320, n_q_heads=5, n_kv_heads=1, n_meta=8, window=50,
                                               cache_capacity=300, name="graph_dec")
    dec = Decode(cfg, synth.make_decode_inputs(cfg, cache_len=np.array([300, 8, 9, 57, 120], np.int32)))
    st, outs = {}, {}
    for i, L in enumerate(dec.layers):
        st[f"ssm{i}"], st[f"conv{i}"] = L["ssm_state"], L["conv_state"]
        for k in ("out", "y_attn_out", "y_ssm_out"):
            outs[f"{k}{i}"] = L[k]
    start = snap(st)

    def step():
        for layer in range(len(dec.layers)):
            dec.call(layer)

    step()
    torch.cuda.synchronize()
    ref = snap(dict(outs, **st))
    for k, v in start.items():
        st[k].copy_(v)
    g = capture(step)
    replay_and_check(g, dict(outs, **st), ref, before=st, start=start)
