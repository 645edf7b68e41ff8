"""The allocation-free decode entry point (library-owned static scratch)
against hymba_mixer_decode with a caller workspace, through the C ABI: the
same inputs give the same outputs and in-place state updates, on two calls in
a row (the second smaller), and a geometry whose scratch does not fit is
refused before anything runs."""
import ctypes

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

H = pytest.importorskip("attention_lm_amd")
from attention_lm_amd import _lib  # noqa: E402
from harness import TOL, Decode, host  # noqa: E402
from harness import check as _check  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    H.load_library()


def say(*a):
    print(*a, flush=True)


def run_both(cfg, cache_len=None):
    """One decode step per layer through each entry point, on separate copies
    of the states; returns (with workspace, allocation-free) host results."""
    inp = synth.make_decode_inputs(cfg, cache_len=cache_len)
    res = []
    for noalloc in (False, True):
        run = Decode(cfg, inp)   # fresh device copies of every input and state
        out = []
        for l in range(cfg.n_layers):
            L = run.layers[l]
            args = (run.desc, L["params"], L["x"], L["z"], L["dt"], L["B"], L["C"], L["q"], run.k_new, run.v_new,
                    run.k_cache, run.v_cache, run.cache_len, L["ssm_state"], L["conv_state"], L["out"])
            if noalloc:
                H.hymba_mixer_decode_noalloc(*args, y_attn_out=L["y_attn_out"], y_ssm_out=L["y_ssm_out"])
            else:
                H.hymba_mixer_decode(*args, y_attn_out=L["y_attn_out"], y_ssm_out=L["y_ssm_out"], workspace=run.ws)
        torch.cuda.synchronize()
        for l in range(cfg.n_layers):
            L = run.layers[l]
            out.append({k: host(L[k]) for k in ("out", "y_attn_out", "y_ssm_out", "ssm_state", "conv_state")})
        res.append(out)
        del run
    return res


def compare(cfg, cache_len=None):
    say(f"decode {cfg.name}: B={cfg.batch} D={cfg.d_inner} cap={cfg.cache_capacity} act={cfg.act}")
    ws_res, na_res = run_both(cfg, cache_len)
    tol = TOL[cfg.act]
    for l, (a, b) in enumerate(zip(ws_res, na_res)):
        for k in a:
            if k == "conv_state":
                np.testing.assert_array_equal(b[k], a[k])
                continue
            _check(f"l{l} {k}", b[k], a[k], tol, slice_width=cfg.d_state if k == "ssm_state" else 128, say=say)
            # the same kernels with the same split count: bit for bit
            np.testing.assert_array_equal(b[k], a[k], err_msg=f"layer {l} {k}")


def test_noalloc_matches_workspace_entry_on_two_calls():
    # the decode workload (64 sequences over an 8192-row cache shared by two layers) ...
    compare(synth.config("decode"))
    # ... then a smaller call: fewer sequences, a narrower layer, ragged cache lengths
    small = synth.config("decode_affine").with_(batch=5, d_inner=320, n_q_heads=5, n_kv_heads=1, n_meta=8,
                                                window=50, cache_capacity=300, name="dsmall")
    compare(small, cache_len=np.array([300, 8, 9, 57, 120], np.int32))
    # and an fp32 call (the fp32 kernels and their rotated q / k in the scratch)
    f32 = synth.config("decode").with_(batch=3, d_inner=128, n_q_heads=2, n_kv_heads=1, n_meta=4, window=0,
                                       cache_capacity=200, act="f32", n_layers=1, name="df32")
    compare(f32, cache_len=np.array([199, 4, 130], np.int32))


def test_noalloc_refuses_scratch_beyond_its_size():
    lib = H.load_library()
    big = H.make_desc(batch=4096, n_meta=128, n_tokens=1, d_inner=3200, n_q_heads=25, n_kv_heads=5, window=1024,
                      act="bf16", cache_capacity=8192)
    buf = torch.zeros(1024, dtype=torch.float32, device="cuda")   # never touched: the call returns first
    p = buf.data_ptr()
    params = _lib.MixerParams(p, p, p, None, p, p)
    st = lib.hymba_mixer_decode_noalloc(ctypes.byref(big), ctypes.byref(params), *([p] * 16), None)
    assert st == -5, st   # HYMBA_EWORKSPACE: the static scratch is too small for this geometry
    torch.cuda.synchronize()
