"""GPU parity: the HIP library (through its C ABI) against the float64 CPU
oracle on seeded synthetic inputs. Relative L2 bounds: 1e-5 for fp32
workloads, 5e-3 for bf16 (fp32 accumulation); bit-exact for the mask ranges.
Each branch is checked before the fusion too, since the row RMS norm would hide
a per-row scale error."""
import numpy as np
import pytest
import torch

import oracle as O
import synth

pytestmark = pytest.mark.gpu

H = pytest.importorskip("attention_lm_amd")
from harness import TOL, Decode, Prefill, dev, host, rel_l2  # noqa: E402
from harness import check as _check  # noqa: E402


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


# ---------------------------------------------------------------------------
# mask ranges: bit exact


@pytest.mark.parametrize("L,M,W", [(72, 8, 32), (2176, 128, 1024), (8320, 128, 0), (100, 0, 1), (50, 60, 7),
                                   (300, 5, 1000), (33, 3, 2)])
def test_mask_ranges_bit_exact(L, M, W):
    desc = H.make_desc(batch=1, n_meta=M, n_tokens=L - M if L >= M else 0, d_inner=64, n_q_heads=1,
                       n_kv_heads=1, window=W, act="f32")
    Lr = desc.n_meta + desc.n_tokens
    r = torch.empty((Lr, 4), dtype=torch.int32, device="cuda")
    H.hymba_debug_mask_ranges(desc, r)
    torch.cuda.synchronize()
    ref = O.mask_ranges(Lr, M, W)
    np.testing.assert_array_equal(r.cpu().numpy(), ref)


# ---------------------------------------------------------------------------
# the prefill attention's own visibility decisions: bit exact


VIS_SHAPES = [
    # (batch, n_meta, n_tokens, Hq, Hkv, window, pos0)
    (1, 8, 64, 2, 1, 32, 0),            # the tiny workload
    (2, 5, 150, 5, 1, 40, 0),           # ragged tail, window across tiles
    (3, 33, 70, 2, 2, 17, 0),           # MHA, meta not a multiple of 32
    (1, 0, 97, 4, 2, 0, 0),             # no meta rows, global
    (1, 128, 300, 5, 1, 64, 0),         # meta longer than the window
    (2, 70, 0, 5, 5, 4, 0),             # meta rows only
    (1, 60, 50, 8, 1, 7, 0),            # G = 8, n_meta > n_tokens
    (1, 128, 2048, 25, 5, 1024, 0),     # the SWA layer
    (1, 128, 8192, 25, 5, 0, 0),        # the global layer
    (16, 128, 4096, 25, 5, 1024, 0),    # the batched workload
    (2, 6, 40, 5, 1, 33, 50),           # a continuation: rows at positions 50 .. 89
    (1, 128, 1024, 25, 5, 1024, 1152),  # a continuation of the SWA layer
]


@pytest.mark.parametrize("shape", VIS_SHAPES, ids=[f"vis{i}" for i in range(len(VIS_SHAPES))])
def test_prefill_visibility_bit_exact(shape):
    B, M, T, Hq, Hkv, W, pos0 = shape
    dv = 128 if Hq == 25 else 64
    desc = H.make_desc(batch=B, n_meta=M, n_tokens=T, d_inner=Hq * dv, n_q_heads=Hq, n_kv_heads=Hkv, window=W,
                       act="bf16")
    Lq = T if pos0 > 0 else M + T
    say(f"visibility B={B} M={M} Lq={Lq} pos0={pos0} Hq={Hq} Hkv={Hkv} W={W}")
    out = torch.full((B, Lq, Hq, 4), -7, dtype=torch.int32, device="cuda")
    H.hymba_debug_prefill_visibility(desc, pos0, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = O.mask_ranges(pos0 + Lq, M, W)[pos0:]
    np.testing.assert_array_equal(got, np.broadcast_to(ref[None, :, None, :], got.shape))
    # the kept keys are exactly the two ranges
    np.testing.assert_array_equal(ref[:, 3], ref[:, 0] + ref[:, 2] - ref[:, 1])


# ---------------------------------------------------------------------------
# fusion alone


# (the last two take the streaming form on a 256-CU device: at least four rows
# per wave of its resident grid, the row count ragged against that grid, and
# rows that fill the last 16-byte pieces of a lane only in part)
@pytest.mark.parametrize("act,rows,width", [("f32", 37, 128), ("bf16", 100, 3200), ("bf16", 5, 77), ("f32", 3, 13),
                                            ("bf16", 0, 64), ("bf16", 8200, 3200), ("f32", 12300, 1000)])
def test_fuse_heads(act, rows, width):
    g = np.random.default_rng(rows * 1000 + width)
    ya = g.standard_normal((rows, width)).astype(np.float32) * 3
    ys = g.standard_normal((rows, width)).astype(np.float32) * 0.1
    ba = g.standard_normal(width).astype(np.float32)
    bs = g.standard_normal(width).astype(np.float32)
    if act == "bf16":
        ya, ys = synth.round_bf16(ya), synth.round_bf16(ys)
    tya, tys = dev(ya, act), dev(ys, act)
    out = torch.empty((rows, width), dtype=tya.dtype, device="cuda")
    H.hymba_fuse_heads(tya, tys, dev(ba), dev(bs), rows, width, 1e-6, act, out)
    torch.cuda.synchronize()
    if rows == 0:
        return
    ref = O.rms_fuse(ya, ys, ba, bs, 1e-6)
    check("fuse", host(out), ref, TOL[act])


# ---------------------------------------------------------------------------
# prefill


def run_prefill_parity(cfg, rows=None, batches=None, state_tol=None):
    say(f"prefill {cfg.name}: B={cfg.batch} L={cfg.seq_rows} D={cfg.d_inner} Hq={cfg.n_q_heads} "
        f"Hkv={cfg.n_kv_heads} W={cfg.window} act={cfg.act}")
    inp = synth.make_prefill_inputs(cfg)
    run = Prefill(cfg, inp)
    run()
    torch.cuda.synchronize()
    got = run.results()
    bsel = np.arange(cfg.batch) if batches is None else np.asarray(batches)
    ref = O.mixer_prefill(cfg, inp, batches=bsel, rows=rows)
    rsel = ref["rows"]
    tol = TOL[cfg.act]
    dv = cfg.head_dim_v
    check("y_ssm", got["y_ssm_out"][bsel], ref["y_ssm"], tol)
    check("y_attn", got["y_attn_out"][bsel][:, rsel], ref["y_attn"], tol, slice_width=dv)   # per (row, head)
    check("out", got["out"][bsel][:, rsel], ref["out"], tol)
    check("ssm_state", got["ssm_state_out"][bsel], ref["ssm_state"], state_tol or tol, slice_width=cfg.d_state)
    check("conv_state", got["conv_state_out"][bsel], ref["conv_state"], 0.0)
    L = cfg.seq_rows
    check("k_cache", got["k_cache"][bsel][:, :L], ref["k_rot"], tol, slice_width=cfg.head_dim)
    np.testing.assert_array_equal(got["v_cache"][bsel][:, :L], inp["v"][bsel])
    return run, inp, got


def test_prefill_tiny_f32():
    run_prefill_parity(synth.config("tiny_f32"))


SMALL = [
    # several tiles and ragged tails: L not a multiple of 32/64, windows crossing tiles
    dict(batch=2, n_meta=5, n_tokens=150, d_inner=320, n_q_heads=5, n_kv_heads=1, window=40, act="bf16", seed=11),
    dict(batch=1, n_meta=0, n_tokens=97, d_inner=128, n_q_heads=4, n_kv_heads=2, window=0, act="bf16", seed=12),
    dict(batch=3, n_meta=33, n_tokens=70, d_inner=256, n_q_heads=2, n_kv_heads=2, window=17, act="f32", seed=13),
    dict(batch=1, n_meta=128, n_tokens=300, d_inner=640, n_q_heads=5, n_kv_heads=1, window=64, act="bf16", seed=14),
    dict(batch=2, n_meta=8, n_tokens=1, d_inner=64, n_q_heads=1, n_kv_heads=1, window=1, act="f32", seed=15),
    dict(batch=1, n_meta=70, n_tokens=0, d_inner=160, n_q_heads=5, n_kv_heads=5, window=4, act="bf16", seed=16),
]


@pytest.mark.parametrize("kw", SMALL, ids=[f"small{i}" for i in range(len(SMALL))])
def test_prefill_small_shapes(kw):
    cfg = synth.config("tiny_f32").with_(**kw, name="small")
    run_prefill_parity(cfg)


# batches whose (sequence, channel) count fills the chip take the single-pass scan
SINGLE_PASS = [
    dict(batch=32, n_meta=5, n_tokens=60, d_inner=1024, n_q_heads=8, n_kv_heads=2, window=16, act="bf16", seed=71),
    dict(batch=40, n_meta=3, n_tokens=27, d_inner=1024, n_q_heads=16, n_kv_heads=4, window=0, act="f32", seed=72),
    dict(batch=12, n_meta=8, n_tokens=1, d_inner=3200, n_q_heads=25, n_kv_heads=5, window=4, act="bf16", seed=73),
    # just over the batch threshold (6 x 100 channel pairs of 32: about one wave per SIMD)
    dict(batch=6, n_meta=4, n_tokens=40, d_inner=3200, n_q_heads=25, n_kv_heads=5, window=16, act="bf16", seed=76),
    # 800 channels: the last 64-channel block of a row holds 32 channels
    dict(batch=42, n_meta=4, n_tokens=13, d_inner=800, n_q_heads=25, n_kv_heads=5, window=8, act="bf16", seed=74),
]


@pytest.mark.parametrize("kw", SINGLE_PASS, ids=[f"single{i}" for i in range(len(SINGLE_PASS))])
def test_prefill_single_pass_scan(kw):
    cfg = synth.config("tiny_f32").with_(**kw, name="single")
    run = run_prefill_parity(cfg)[0]
    assert H.hymba_mixer_prefill_chunk_rows(run.desc) == cfg.seq_rows   # one chunk: the single-pass form ran


AFFINE_PREFILL = [
    # two kv heads with two query heads each: a head must take its own group's w
    dict(batch=2, n_meta=5, n_tokens=130, d_inner=256, n_q_heads=4, n_kv_heads=2, window=40, act="bf16", seed=41),
    dict(batch=1, n_meta=8, n_tokens=75, d_inner=256, n_q_heads=4, n_kv_heads=2, window=0, act="f32", seed=42),
]


@pytest.mark.parametrize("kw", AFFINE_PREFILL, ids=["bf16_swa", "f32_global"])
def test_prefill_shared_key_affine(kw):
    """A layer reading shared keys through its affine K w + b: attention as the
    oracle computes it (bias included), cache rows without the affine."""
    cfg = synth.config("tiny_f32").with_(**kw, key_affine=True, name="affine")
    run, inp, got = run_prefill_parity(cfg)
    plain = {k: v for k, v in inp.items() if k not in ("k_scale", "k_bias")}
    ref_plain = O.mixer_prefill(cfg, plain)
    assert rel_l2(got["y_attn_out"], ref_plain["y_attn"]) > 20 * TOL[cfg.act]   # the affine is not a no-op


def test_prefill_swa_layer_full():
    run_prefill_parity(synth.config("swa_layer"))


def block_rows(cfg, head=0, tail=0):
    """One query row from every position block of the prefill attention's work
    items (a block is 128 // G consecutive positions of one kv group; a row
    checks every head, so every (sequence, kv group, block) item is covered),
    at an offset that moves from block to block, plus the first ``head`` and
    the last ``tail`` rows."""
    L = cfg.seq_rows
    P = 128 // cfg.group
    starts = np.arange(0, L, P)
    rows = np.minimum(starts + (np.arange(len(starts)) * 7) % P, L - 1)
    return np.unique(np.concatenate([rows, np.arange(0, min(head, L)), np.arange(max(0, L - tail), L)]))


@pytest.mark.slow
def test_prefill_global_layer_every_block():
    """The global layer: the scan over every row; attention and the fused
    output on one row of every work item's position block."""
    cfg = synth.config("global_layer")
    run_prefill_parity(cfg, rows=block_rows(cfg, head=130, tail=40))


@pytest.mark.slow
def test_prefill_batched_every_sequence():
    """The batched workload (single-pass scan): the Mamba branch, final state
    and conv state of all 16 sequences over every row; attention and the
    fused output on one row of every position block of every sequence."""
    cfg = synth.config("batched_prefill")
    run_prefill_parity(cfg, rows=block_rows(cfg, head=20, tail=10))


@pytest.mark.slow
def test_prefill_ssd_batched_sequences():
    """The batched workload with its Mamba branch in the Mamba-2 form (50
    heads of 64 channels: 67 chunks x 50 heads x 16 sequences = 53,600
    chunk-head items, many rounds of both passes): the Mamba branch and the
    final states of all 16 sequences on every row; attention and the fused
    output on one row of every position block of every sequence."""
    cfg = synth.config("batched_prefill").with_(ssm_heads=50, name="batched_ssd")
    run_prefill_parity(cfg, rows=block_rows(cfg, head=20, tail=10))


# A global layer whose attention branch outweighs its scan: the library runs
# attention on the calling stream and forks the Mamba branch after the RoPE
# pass (the estimate below is the library's rule: attention flops over the
# visible pairs at 1e15 flop/s against scan elements at 2e12 per second).
LATE_FORK = dict(batch=1, n_meta=16, n_tokens=3984, d_inner=512, n_q_heads=16, n_kv_heads=2, window=0, act="bf16",
                 seed=75)


def attention_outweighs_scan(cfg):
    L = cfg.seq_rows
    cap = cfg.n_meta + cfg.window if cfg.window > 0 else L
    pairs = sum(min(i + 1, cap) for i in range(L)) * cfg.batch
    attn_s = pairs * cfg.n_q_heads * (2 * cfg.head_dim + 2 * cfg.head_dim_v) / 1e15
    scan_s = cfg.batch * L * cfg.d_inner * cfg.d_state / 2e12
    return attn_s > scan_s


def test_prefill_attention_branch_first():
    """The concurrent prefill with the Mamba branch forked after the RoPE
    pass: every row of every output against the oracle."""
    cfg = synth.config("tiny_f32").with_(**LATE_FORK, name="late_fork")
    assert attention_outweighs_scan(cfg)
    run_prefill_parity(cfg)


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_prefill_xcd_order_g8(act):
    """The attention's XCD-major work order (many rounds of workgroups) at
    another group shape: 8 sequences, 16 query heads over 2 kv heads (16
    positions per workgroup), head width 32; 69 position blocks x 16 streams.
    Every row of every output against the oracle."""
    cfg = synth.config("tiny_f32").with_(batch=8, n_meta=12, n_tokens=1088, d_inner=512, n_q_heads=16, n_kv_heads=2,
                                          window=100, act=act, seed=71, name="split")
    run_prefill_parity(cfg)


def test_prefill_deterministic_and_branch_isolation():
    cfg = synth.config("tiny_f32").with_(**SMALL[0], name="det")
    inp = synth.make_prefill_inputs(cfg)
    run = Prefill(cfg, inp)
    run()
    a = run.results()
    run()
    b = run.results()
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
    # beta = (1, 0): out is half the normalised attention branch
    inp2 = dict(inp, beta_ssm=np.zeros_like(inp["beta_ssm"]))
    run2 = Prefill(cfg, inp2)
    run2()
    got = run2.results()
    ya = got["y_attn_out"]
    ref = O.rms_fuse(ya, np.ones_like(ya), np.ones(cfg.d_inner), np.zeros(cfg.d_inner), cfg.norm_eps)
    check("beta=(1,0)", got["out"], ref, TOL[cfg.act])


# ---------------------------------------------------------------------------
# decode


def run_decode_parity(cfg, cache_len=None):
    say(f"decode {cfg.name}: B={cfg.batch} cap={cfg.cache_capacity} D={cfg.d_inner} W={cfg.window} act={cfg.act}")
    inp = synth.make_decode_inputs(cfg, cache_len=cache_len)
    run = Decode(cfg, inp)
    kc0 = run.k_cache.clone()
    vc0 = run.v_cache.clone()
    for l in range(cfg.n_layers):
        run.call(l)
    torch.cuda.synchronize()
    tol = TOL[cfg.act]
    assert torch.equal(run.k_cache, kc0) and torch.equal(run.v_cache, vc0)   # read-only, shared by both layers
    for l in range(cfg.n_layers):
        ref = O.mixer_decode(cfg, inp["layers"][l], inp["k_cache"], inp["v_cache"], inp["k_new"], inp["v_new"],
                             inp["cache_len"])
        L = run.layers[l]
        say(f" layer {l}")
        check("y_ssm", host(L["y_ssm_out"]), ref["y_ssm"], tol)
        check("y_attn", host(L["y_attn_out"]), ref["y_attn"], tol, slice_width=cfg.head_dim_v)   # per (row, head)
        check("out", host(L["out"]), ref["out"], tol)
        check("ssm_state", host(L["ssm_state"]), ref["ssm_state"], tol, slice_width=cfg.d_state)
        check("conv_state", host(L["conv_state"]), ref["conv_state"], 0.0)
        if inp["layers"][l].get("k_scale") is not None:   # a secondary layer: its affine matters
            plain = {k: v for k, v in inp["layers"][l].items() if k not in ("k_scale", "k_bias")}
            ref_plain = O.mixer_decode(cfg, plain, inp["k_cache"], inp["v_cache"], inp["k_new"], inp["v_new"],
                                       inp["cache_len"])
            assert rel_l2(host(L["y_attn_out"]), ref_plain["y_attn"]) > 20 * tol
    return run


def test_decode_small_ragged_cache_lengths():
    cfg = synth.config("decode_affine").with_(batch=5, d_inner=320, n_q_heads=5, n_kv_heads=1, n_meta=8, window=50,
                                       cache_capacity=300, cache_len=0, name="dsmall")
    run_decode_parity(cfg, cache_len=np.array([300, 8, 9, 57, 120], np.int32))


def test_decode_small_global_f32():
    cfg = synth.config("decode_affine").with_(batch=3, d_inner=128, n_q_heads=2, n_kv_heads=1, n_meta=4, window=0,
                                       cache_capacity=200, act="f32", name="dglob")
    run_decode_parity(cfg, cache_len=np.array([199, 4, 130], np.int32))


DECODE_EDGE = [
    # dv 32 (64-key tiles), a global layer, one sequence: many one-tile splits
    dict(batch=1, d_inner=64, n_q_heads=2, n_kv_heads=1, n_meta=3, window=0, cache_capacity=500, cache=[437]),
    # no GQA (G = 1), dv 128, no meta rows; an empty cache, one row, a full cache (p = capacity)
    dict(batch=4, d_inner=256, n_q_heads=2, n_kv_heads=2, n_meta=0, window=7, cache_capacity=64,
         cache=[0, 1, 63, 64]),
    # the largest group (8 query heads per kv head), dv 32, window wider than the cache
    dict(batch=2, d_inner=256, n_q_heads=8, n_kv_heads=1, n_meta=16, window=4096, cache_capacity=100,
         cache=[17, 100]),
]


@pytest.mark.parametrize("kw", DECODE_EDGE, ids=[f"edge{i}" for i in range(len(DECODE_EDGE))])
def test_decode_bf16_edge_shapes(kw):
    kw = dict(kw)
    cache = np.array(kw.pop("cache"), np.int32)
    cfg = synth.config("decode_affine").with_(**kw, name="dedge")
    run_decode_parity(cfg, cache_len=cache)


def test_decode_full_config():
    run_decode_parity(synth.config("decode"))


def test_decode_deterministic():
    """Two identical decode steps of the full workload (fresh copies of the
    states) give the same bits: no result depends on timing."""
    cfg = synth.config("decode")
    inp = synth.make_decode_inputs(cfg)
    outs = []
    for _ in range(3):
        run = Decode(cfg, inp)
        for l in range(cfg.n_layers):
            run.call(l)
        torch.cuda.synchronize()
        outs.append([{k: host(run.layers[l][k]) for k in ("out", "y_attn_out", "y_ssm_out", "ssm_state")}
                     for l in range(cfg.n_layers)])
        del run
    for other in outs[1:]:
        for l in range(cfg.n_layers):
            for k in outs[0][l]:
                np.testing.assert_array_equal(other[l][k], outs[0][l][k], err_msg=f"layer {l} {k}")


def test_prefill_swa_layer_deterministic():
    cfg = synth.config("swa_layer")
    inp = synth.make_prefill_inputs(cfg)
    run = Prefill(cfg, inp)
    run()
    a = run.results()
    run()
    b = run.results()
    for k in a:
        np.testing.assert_array_equal(b[k], a[k], err_msg=k)


def test_decode_full_config_key_affine():
    """The same step with the second layer reading the shared keys through its
    per-head affine."""
    run_decode_parity(synth.config("decode_affine"))


@pytest.mark.parametrize("ssm_heads", [0, 5], ids=["mamba1", "mamba2"])
def test_decode_continues_prefill(ssm_heads):
    """decode(prefill of L-1 rows) on the GPU equals the oracle's prefill of L rows, last row
    (the scan in either form: the Mamba-2 prefill's final state enters the Mamba-2 decode step)."""
    cfg = synth.config("tiny_f32").with_(batch=2, n_meta=6, n_tokens=90, d_inner=320, n_q_heads=5, n_kv_heads=1,
                                         window=33, act="bf16", seed=31, ssm_heads=ssm_heads, name="cont")
    full = synth.make_prefill_inputs(cfg)
    L = cfg.seq_rows
    short_cfg = cfg.with_(n_tokens=cfg.n_tokens - 1)
    short = {k: (v[:, :L - 1] if k in ("x", "z", "dt", "B", "C", "q", "k", "v") else v) for k, v in full.items()}
    pre = Prefill(short_cfg, short, cache_capacity=L + 3)
    pre()
    torch.cuda.synchronize()
    dcfg = cfg.with_(decode=True, cache_capacity=L + 3, n_layers=1)
    layer = {"x": full["x"][:, L - 1], "z": full["z"][:, L - 1], "dt": full["dt"][:, L - 1],
             "B": full["B"][:, L - 1], "C": full["C"][:, L - 1], "q": full["q"][:, L - 1],
             "ssm_state": np.zeros((2, 320, 16), np.float32), "conv_state": np.zeros((2, 320, 3), np.float32),
             **{k: full[k] for k in ("A", "D", "conv_w", "beta_attn", "beta_ssm")}}
    inp = {"k_cache": np.zeros((2, L + 3, 1, 64), np.float32), "v_cache": np.zeros((2, L + 3, 1, 64), np.float32),
           "k_new": full["k"][:, L - 1], "v_new": full["v"][:, L - 1],
           "cache_len": np.full(2, L - 1, np.int32), "layers": [layer]}
    run = Decode(dcfg, inp)
    run.k_cache.copy_(pre.o["k_cache"])
    run.v_cache.copy_(pre.o["v_cache"])
    run.layers[0]["ssm_state"].copy_(pre.o["ssm_state_out"])
    run.layers[0]["conv_state"].copy_(pre.o["conv_state_out"])
    run.call(0)
    torch.cuda.synchronize()
    ref = O.mixer_prefill(cfg, full, rows=np.array([L - 1]))
    check("y_ssm", host(run.layers[0]["y_ssm_out"]), ref["y_ssm"][:, L - 1], 5e-3)
    check("y_attn", host(run.layers[0]["y_attn_out"]), ref["y_attn"][:, 0], 5e-3)
    check("out", host(run.layers[0]["out"]), ref["out"][:, 0], 5e-3)


# ---------------------------------------------------------------------------
# the Mamba-2 form of the scan (one decay rate and step size per head)

SSD_SMALL = [
    # head width 64, several 64-row chunks and a ragged tail
    dict(batch=2, n_meta=5, n_tokens=150, d_inner=256, n_q_heads=2, n_kv_heads=1, window=40, act="bf16", seed=61,
         ssm_heads=4),
    # fp32, head width 32, one partial chunk
    dict(batch=1, n_meta=8, n_tokens=40, d_inner=128, n_q_heads=2, n_kv_heads=1, window=16, act="f32", seed=62,
         ssm_heads=4),
    # fp32, head width 128, chunks of 64 with a 1-row tail
    dict(batch=2, n_meta=3, n_tokens=126, d_inner=256, n_q_heads=4, n_kv_heads=2, window=0, act="f32", seed=63,
         ssm_heads=2),
    # bf16, head width 32, 8 heads
    dict(batch=1, n_meta=16, n_tokens=300, d_inner=256, n_q_heads=8, n_kv_heads=2, window=64, act="bf16", seed=64,
         ssm_heads=8),
    # bf16, head width 128, three heads, a ragged last chunk
    dict(batch=2, n_meta=2, n_tokens=190, d_inner=384, n_q_heads=3, n_kv_heads=1, window=50, act="bf16", seed=68,
         ssm_heads=3),
]


@pytest.mark.parametrize("kw", SSD_SMALL, ids=[f"ssd{i}" for i in range(len(SSD_SMALL))])
def test_prefill_ssd_small_shapes(kw):
    cfg = synth.config("tiny_f32").with_(**kw, name="ssd")
    run_prefill_parity(cfg)


def test_prefill_ssd_many_items_per_workgroup():
    """fp32, head width 32: 19 chunks x 32 heads x 3 sequences = 1824
    (chunk, head, sequence) items, more than one round of workgroups of
    either pass, with a ragged last chunk in every sequence."""
    cfg = synth.config("tiny_f32").with_(batch=3, n_meta=8, n_tokens=1200, d_inner=1024, n_q_heads=8, n_kv_heads=2,
                                          window=100, act="f32", seed=65, ssm_heads=32, name="ssd_many")
    run_prefill_parity(cfg)


def test_prefill_ssd_swa_layer_full():
    """The 1.5B-shaped window-1024 layer with its Mamba branch in the Mamba-2
    form: 50 heads of 64 channels."""
    run_prefill_parity(synth.config("swa_layer").with_(ssm_heads=50, name="swa_ssd"))


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_decode_ssd(act):
    cfg = synth.config("decode_affine").with_(batch=5, d_inner=320, n_q_heads=5, n_kv_heads=1, n_meta=8, window=50,
                                       cache_capacity=300, act=act, ssm_heads=5, name="dssd")
    run_decode_parity(cfg, cache_len=np.array([300, 8, 9, 57, 120], np.int32))
