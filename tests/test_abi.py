"""The C ABI library loads, exports every function the header declares, and
rejects bad arguments on the host before enqueuing anything. No GPU needed:
every call here returns from host-side validation (pointers are never
dereferenced)."""
import ctypes
import os
import re

import pytest

import attention_lm_amd as H
from attention_lm_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hymba_mixer.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?(?:int|size_t|char\s*\*|const char\s*\*)\s*\**\s*(hymba_\w+)\s*\(", text, re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        import attention_lm_amd.build as b
        b.build()
    return H.load_library()


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("hymba_mixer_prefill", "hymba_mixer_decode", "hymba_fuse_heads", "hymba_debug_mask_ranges"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert names
    for n in names:
        assert hasattr(lib, n), n
    # the binding wraps each one under the same name
    for n in names:
        assert hasattr(H, n) or n in ("hymba_abi_version",), n


def test_abi_version_and_status_strings(lib):
    assert H.hymba_abi_version() == 2
    assert H.hymba_status_string(0) == "ok"
    for s in (-1, -2, -3, -4, -5):
        assert H.hymba_status_string(s) != "unknown status"
    assert H.hymba_last_hip_error() == 0


def c1_desc(**kw):
    d = dict(batch=1, n_meta=128, n_tokens=2048, d_inner=3200, n_q_heads=25, n_kv_heads=5, window=1024,
             act="bf16", cache_capacity=8192)
    d.update(kw)
    return H.make_desc(**d)


def test_workspace_sizes(lib):
    d = c1_desc()
    L = 2176
    # rotated q and k, both branch outputs (bf16), then the scan's per-chunk
    # end states, summed dt and carried-in states (fp32): 25 channel blocks of
    # 128 -> ~2048/25 = 82 chunks wanted -> 26.5 rows, rounded down to whole
    # 8-row staging blocks: 24 rows -> 91 chunks (one slot more than chunks:
    # the Mamba-2 form's chain also yields the final state), then a copy of a
    # carried conv history, 3 rows, for a continuation
    n_chunk = (L + 23) // 24 + 1
    expect = (L * 25 * 64 + L * 5 * 64 + 2 * L * 3200) * 2 + n_chunk * 3200 * (16 + 1 + 16) * 4 + 3200 * 3 * 2
    got = H.hymba_mixer_prefill_workspace_bytes(d)
    assert expect <= got <= expect + 10 * 256
    # the compact cache adds the rows a continuation's attention reads: the
    # meta rows, up to window - 1 earlier rows and the new rows, K and V
    ring = H.hymba_mixer_prefill_workspace_bytes(c1_desc(cache_capacity=128 + 1024, cache_ring=True))
    assert ring - got == pytest.approx((128 + 1023 + 2048) * 5 * (64 + 128) * 2, abs=2 * 256)
    dd = c1_desc(batch=64)
    # room for a partial (o, m, l) per query head and 32-key tile of the 128 + 1024 visible keys
    n_split = (128 + 1024 + 31) // 32
    expect = 64 * 25 * n_split * 130 * 4 + 2 * 64 * 3200 * 2 + 64 * (25 + 5) * 64 * 4
    got = H.hymba_mixer_decode_workspace_bytes(dd)
    assert expect <= got <= expect + 5 * 256
    assert H.hymba_mixer_prefill_workspace_bytes(c1_desc(n_q_heads=24)) == 0     # invalid -> 0
    assert H.hymba_mixer_prefill_chunk_rows(d) == 24
    # never below one staging block; a larger batch gives longer chunks
    assert H.hymba_mixer_prefill_chunk_rows(c1_desc(n_tokens=64, n_meta=0)) == 8
    assert H.hymba_mixer_prefill_chunk_rows(c1_desc(batch=4)) == 96   # 21 chunks wanted -> 103.6 -> 96
    assert H.hymba_mixer_prefill_chunk_rows(c1_desc(n_q_heads=24)) == 0
    assert H.hymba_mixer_prefill_chunk_rows(c1_desc(ssm_heads=50)) == 64   # Mamba-2 form: 64-row chunks


@pytest.mark.parametrize("kw,status", [
    (dict(n_q_heads=24), -1),          # Hq * dv != d_inner
    (dict(n_kv_heads=4), -1),          # Hq % Hkv != 0
    (dict(batch=0), -1),
    (dict(n_meta=0, n_tokens=0), -1),
    (dict(d_state=8), -2),
    (dict(head_dim=128), -2),
    (dict(act=7), -1),
    (dict(ssm_heads=-1), -1),
    (dict(ssm_heads=3), -1),           # d_inner % ssm_heads != 0
    (dict(ssm_heads=128), -2),         # head width 25: no kernel
])
def test_prefill_rejects_bad_geometry(lib, kw, status):
    d = c1_desc(**kw)
    fake = 0x100000  # aligned, never dereferenced: validation fails first
    p = _lib.MixerParams(fake, fake, fake, None, fake, fake)
    st = lib.hymba_mixer_prefill(ctypes.byref(d), ctypes.byref(p), *([fake] * 9), None, None, None, None, None,
                                 None, fake, 1 << 40, None, None)
    assert st == status


def test_prefill_rejects_pointers_and_workspace(lib):
    d = c1_desc()
    fake = 0x100000
    p = _lib.MixerParams(fake, fake, fake, None, fake, fake)
    call = lambda args, ws=fake, wsb=1 << 40, params=p: lib.hymba_mixer_prefill(
        ctypes.byref(d), ctypes.byref(params), *args, None, None, None, None, None, None, ws, wsb, None, None)
    ok = [fake] * 9
    assert call([None] + ok[1:]) == -1                       # null input
    assert call(ok[:3] + [fake + 2] + ok[4:]) == -3          # misaligned input
    assert call(ok, ws=None) == -5                           # no workspace
    assert call(ok, wsb=16) == -5                            # workspace too small
    assert call(ok, ws=fake + 16) == -3                      # workspace not 256-byte aligned
    bad = _lib.MixerParams(fake, fake, fake, fake, fake, fake)
    assert call(ok, params=bad) == -2                        # conv bias unsupported
    nullp = _lib.MixerParams(None, fake, fake, None, fake, fake)
    assert call(ok, params=nullp) == -1
    skew = _lib.MixerParams(fake, fake, fake, None, fake, fake, fake + 4, None)
    assert call(ok, params=skew) == -3                       # misaligned k_scale
    # k_cache without v_cache, and a cache too short for L rows
    st = lib.hymba_mixer_prefill(ctypes.byref(d), ctypes.byref(p), *ok, None, None, fake, None, None, None, fake,
                                 1 << 40, None, None)
    assert st == -1
    d2 = c1_desc(cache_capacity=100)
    st = lib.hymba_mixer_prefill(ctypes.byref(d2), ctypes.byref(p), *ok, None, None, fake, fake, None, None, fake,
                                 1 << 40, None, None)
    assert st == -1


def test_decode_rejects_bad_arguments(lib):
    d = c1_desc(batch=64)
    fake = 0x100000
    p = _lib.MixerParams(fake, fake, fake, None, fake, fake)
    args = [fake] * 14
    call = lambda a, desc=d: lib.hymba_mixer_decode(ctypes.byref(desc), ctypes.byref(p), *a[:13], a[13], None,
                                                    None, fake, 1 << 40, None, None)
    assert call(args[:10] + [None] + args[11:]) == -1        # null cache_len
    assert call(args[:8] + [fake + 4] + args[9:]) == -3      # misaligned k_cache
    assert call(args, desc=c1_desc(batch=64, cache_capacity=0)) == -1
    st = lib.hymba_mixer_decode(ctypes.byref(d), ctypes.byref(p), *args, None, None, fake, 8, None, None)
    assert st == -5


def test_fuse_and_mask_validation(lib):
    fake = 0x100000
    assert lib.hymba_fuse_heads(fake, fake, fake, fake, 4, 0, 1e-6, 1, fake, None) == -1
    assert lib.hymba_fuse_heads(fake, fake, fake, fake, -1, 8, 1e-6, 1, fake, None) == -1
    assert lib.hymba_fuse_heads(fake, None, fake, fake, 4, 8, 1e-6, 1, fake, None) == -1
    assert lib.hymba_fuse_heads(fake, fake, fake, fake, 4, 8, 1e-6, 9, fake, None) == -1
    assert lib.hymba_fuse_heads(fake + 8, fake, fake, fake, 4, 8, 1e-6, 1, fake, None) == -3
    d = c1_desc()
    assert lib.hymba_debug_mask_ranges(ctypes.byref(d), None, None) == -1
    assert lib.hymba_debug_mask_ranges(ctypes.byref(d), fake + 4, None) == -3
    # the allocation-free decode validates its arguments before anything else
    dd = c1_desc(n_tokens=1)
    pp = _lib.MixerParams(fake, fake, fake, None, fake, fake)
    na = lib.hymba_mixer_decode_noalloc
    assert na(ctypes.byref(dd), ctypes.byref(pp), *([fake] * 13), None, None, None, None) == -1   # out missing
    assert na(ctypes.byref(dd), ctypes.byref(pp), *([fake] * 13), fake + 4, fake, None, None, None) == -3
    assert na(None, ctypes.byref(pp), *([fake] * 16), None) == -1
    # the prefill visibility export validates like a prefill call, then its own arguments
    assert lib.hymba_debug_prefill_visibility(ctypes.byref(d), 0, None, None) == -1
    assert lib.hymba_debug_prefill_visibility(ctypes.byref(d), 0, fake + 4, None) == -3
    assert lib.hymba_debug_prefill_visibility(ctypes.byref(d), -1, fake, None) == -1
    assert lib.hymba_debug_prefill_visibility(ctypes.byref(d), 100, fake, None) == -1   # pos0 below n_meta
    bad = c1_desc(n_kv_heads=3)
    assert lib.hymba_debug_prefill_visibility(ctypes.byref(bad), 0, fake, None) == -1


def test_continue_and_compact_cache_validation(lib):
    fake = 0x100000
    p = _lib.MixerParams(fake, fake, fake, None, fake, fake)

    def cont(desc, pos0, ptrs=None, ws=fake, wsb=1 << 40):
        ptrs = ptrs or [fake] * 13   # x z dt B C q k v out ssm_state conv_state k_cache v_cache
        return lib.hymba_mixer_prefill_continue(ctypes.byref(desc), ctypes.byref(p), pos0, *ptrs, None, None, ws,
                                                wsb, None)

    d = c1_desc(n_tokens=512)
    assert cont(d, 127) == -1                       # starts inside the meta rows
    assert cont(d, 8192 - 511) == -1                # one row per position: needs pos0 + n_tokens rows
    assert cont(d, 8192 - 512, ws=None) == -5       # valid up to the workspace
    for i in (9, 10, 11, 12):                       # states and cache are required
        ptrs = [fake] * 13
        ptrs[i] = None
        assert cont(d, 1000, ptrs) == -1
    ptrs = [fake] * 13
    ptrs[10] = fake + 2
    assert cont(d, 1000, ptrs) == -3
    assert cont(c1_desc(n_tokens=0), 1000) == -1
    # the compact cache: sliding-window layers only, at least n_meta + window rows
    assert cont(c1_desc(window=0, cache_ring=True), 1000) == -1
    assert cont(c1_desc(cache_capacity=1151, cache_ring=True), 1000) == -1
    ring = c1_desc(n_tokens=512, cache_capacity=1152, cache_ring=True)
    assert cont(ring, 100000, ws=None) == -5        # any position past the meta rows
    bad = c1_desc()
    bad.cache_ring = 2
    assert cont(bad, 1000) == -1
    # a fresh prefill into the compact cache needs n_meta + window rows, not L
    st = lib.hymba_mixer_prefill(ctypes.byref(c1_desc(cache_capacity=1152, cache_ring=True)), ctypes.byref(p),
                                 *([fake] * 9), None, None, fake, fake, None, None, None, 1 << 40, None, None)
    assert st == -5
    # decode reads it the same way
    dd = c1_desc(batch=64, cache_capacity=1152, cache_ring=True)
    st = lib.hymba_mixer_decode(ctypes.byref(dd), ctypes.byref(p), *([fake] * 14), None, None, None, 1 << 40,
                                None, None)
    assert st == -5
    dd.cache_capacity = 1151
    st = lib.hymba_mixer_decode(ctypes.byref(dd), ctypes.byref(p), *([fake] * 14), None, None, fake, 1 << 40,
                                None, None)
    assert st == -1
