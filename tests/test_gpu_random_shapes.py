"""GPU parity on seeded random geometries, against the float64 oracle.

The hand-picked shapes elsewhere target known edges; these draw the geometry
itself from a fixed-seed generator, over everything the descriptor allows:
batch, meta rows (including none), prompt rows (including none), window
(global, one row, shorter or longer than a tile or the sequence), GQA group
(1 to 8 query heads per kv head), value width (32, 64, 128), the Mamba-1 or
Mamba-2 form (head widths 32, 64, 128), the shared-key affine, and the
activation dtype; decode draws ragged cache lengths between the meta rows
and the capacity; chains of continued prefills draw their cut points and the
cache layout (one row per position, or the compact ring). Each case prints
its geometry before it runs."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

H = pytest.importorskip("attention_lm_amd")
from test_gpu_continue import check_chain  # noqa: E402
from test_gpu_parity import run_decode_parity, run_prefill_parity  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    H.load_library()


def _prefill_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        hkv = int(rng.choice([1, 2, 3]))
        g = int(rng.choice([1, 2, 3, 4, 5, 8]))
        dv = int(rng.choice([32, 64, 128]))
        hq = g * hkv
        d_inner = hq * dv
        n_meta = int(rng.choice([0, 1, 5, 16, 31, 64, 129]))
        n_tokens = int(rng.integers(0, 400))
        if n_meta + n_tokens < 1:
            continue
        window = int(rng.choice([0, 1, 3, 16, 33, 100, 500]))
        widths = [p for p in (32, 64, 128) if d_inner % p == 0]
        ssm_heads = d_inner // int(rng.choice(widths)) if rng.random() < 0.3 else 0
        cases.append(dict(batch=int(rng.integers(1, 4)), n_meta=n_meta, n_tokens=n_tokens, d_inner=d_inner,
                          n_q_heads=hq, n_kv_heads=hkv, window=window, act=str(rng.choice(["bf16", "f32"])),
                          seed=int(rng.integers(1000, 9999)), ssm_heads=ssm_heads,
                          key_affine=bool(rng.random() < 0.25)))
    return cases


def _decode_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        hkv = int(rng.choice([1, 2]))
        g = int(rng.choice([1, 2, 4, 5, 8]))
        dv = int(rng.choice([32, 64, 128]))
        hq = g * hkv
        d_inner = hq * dv
        n_meta = int(rng.choice([0, 3, 8, 40]))
        cap = int(rng.integers(max(n_meta, 1), 600))
        batch = int(rng.integers(1, 7))
        cache = rng.integers(n_meta, cap + 1, size=batch).astype(np.int32)
        widths = [p for p in (32, 64, 128) if d_inner % p == 0]
        ssm_heads = d_inner // int(rng.choice(widths)) if rng.random() < 0.3 else 0
        cases.append(dict(batch=batch, d_inner=d_inner, n_q_heads=hq, n_kv_heads=hkv, n_meta=n_meta,
                          window=int(rng.choice([0, 1, 9, 64, 700])), cache_capacity=cap,
                          act=str(rng.choice(["bf16", "f32"])), seed=int(rng.integers(1000, 9999)),
                          ssm_heads=ssm_heads, cache=cache.tolist()))
    return cases


def _chain_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        hkv = int(rng.choice([1, 2]))
        g = int(rng.choice([1, 2, 4, 5]))
        dv = int(rng.choice([32, 64, 128]))
        hq = g * hkv
        d_inner = hq * dv
        n_meta = int(rng.choice([1, 5, 16, 40]))
        n_tokens = int(rng.integers(20, 300))
        L = n_meta + n_tokens
        window = int(rng.choice([0, 1, 9, 33, 100]))
        ring = bool(window > 0 and rng.random() < 0.5)
        widths = [p for p in (32, 64, 128) if d_inner % p == 0]
        ssm_heads = d_inner // int(rng.choice(widths)) if rng.random() < 0.5 else 0
        first = n_meta + int(rng.integers(0, min(70, n_tokens)))
        later = sorted(set(int(c) for c in rng.integers(first + 1, L, size=int(rng.integers(1, 4)))))
        cases.append((dict(batch=int(rng.integers(1, 3)), n_meta=n_meta, n_tokens=n_tokens, d_inner=d_inner,
                           n_q_heads=hq, n_kv_heads=hkv, window=window, act=str(rng.choice(["bf16", "f32"])),
                           seed=int(rng.integers(1000, 9999)), ssm_heads=ssm_heads), [first] + later, ring))
    return cases


PREFILL_CASES = _prefill_cases(12, seed=20241204)
DECODE_CASES = _decode_cases(8, seed=20241205)
CHAIN_CASES = _chain_cases(10, seed=20241206)


@pytest.mark.parametrize("kw", PREFILL_CASES, ids=[f"prefill{i}" for i in range(len(PREFILL_CASES))])
def test_prefill_random_geometry(kw):
    print(f"geometry {kw}", flush=True)
    cfg = synth.config("tiny_f32").with_(**kw, name="rand")
    run_prefill_parity(cfg)


@pytest.mark.parametrize("kw", DECODE_CASES, ids=[f"decode{i}" for i in range(len(DECODE_CASES))])
def test_decode_random_geometry(kw):
    print(f"geometry {kw}", flush=True)
    kw = dict(kw)
    cache = np.array(kw.pop("cache"), np.int32)
    cfg = synth.config("decode_affine").with_(**kw, name="drand")
    run_decode_parity(cfg, cache_len=cache)


@pytest.mark.parametrize("case", CHAIN_CASES, ids=[f"chain{i}" for i in range(len(CHAIN_CASES))])
def test_chain_random_geometry(case):
    kw, cuts, ring = case
    print(f"geometry {kw} cuts={cuts} ring={ring}", flush=True)
    check_chain(synth.config("tiny_f32").with_(**kw, name="crand"), cuts, ring)
