"""ctypes binding of libhymba_mixer.so: argument marshalling only.

Every entry point of include/hymba_mixer.h has a Python function of the same
name. Tensors are torch tensors on the GPU (torch is used for device memory and
streams only); the work itself runs in the library's HIP kernels. Nothing here
falls back to another implementation: if the library cannot be loaded, or a
call returns an error status, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libhymba_mixer.so")

HYMBA_F32, HYMBA_BF16 = 0, 1
STATUS = {0: "HYMBA_OK", -1: "HYMBA_EINVAL", -2: "HYMBA_EUNSUPPORTED", -3: "HYMBA_EALIGN",
          -4: "HYMBA_EHIP", -5: "HYMBA_EWORKSPACE"}

_EXPORTS = [
    "hymba_mixer_prefill_workspace_bytes",
    "hymba_mixer_decode_workspace_bytes",
    "hymba_mixer_prefill",
    "hymba_mixer_prefill_continue",
    "hymba_mixer_decode",
    "hymba_mixer_decode_noalloc",
    "hymba_fuse_heads",
    "hymba_debug_mask_ranges",
    "hymba_debug_prefill_visibility",
    "hymba_status_string",
    "hymba_last_hip_error",
    "hymba_abi_version",
]


class MixerDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_meta", ctypes.c_int32), ("n_tokens", ctypes.c_int32),
        ("d_inner", ctypes.c_int32), ("d_state", ctypes.c_int32), ("d_conv", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("head_dim_v", ctypes.c_int32), ("window", ctypes.c_int32), ("cache_capacity", ctypes.c_int32),
        ("rope_base", ctypes.c_float), ("norm_eps", ctypes.c_float), ("act", ctypes.c_int),
        ("cache_ring", ctypes.c_int32), ("ssm_heads", ctypes.c_int32),
    ]


class MixerParams(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p)
                for n in ("A", "D", "conv_w", "conv_b", "beta_attn", "beta_ssm", "k_scale", "k_bias")]


class HymbaError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str = ""):
        self.status = status
        super().__init__(f"{fn} returned {status} ({STATUS.get(status, '?')}){': ' + detail if detail else ''}")


_lib = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the HIP library (once). Raises if it has not been built.

    HYMBA_MIXER_LIB names another build of the same library to load instead
    (the host-sanitizer build that the CPU tests drive)."""
    global _lib
    if _lib is not None:
        return _lib
    if path is None:
        path = os.environ.get("HYMBA_MIXER_LIB") or LIB_PATH
    if not os.path.exists(path):
        raise ImportError(f"{path} not found: build it first (python -m attention_lm_amd.build)")
    lib = ctypes.CDLL(path)
    vp, sz, i32, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64
    pdesc, pparams = ctypes.POINTER(MixerDesc), ctypes.POINTER(MixerParams)
    lib.hymba_mixer_prefill_workspace_bytes.argtypes = [pdesc]
    lib.hymba_mixer_prefill_workspace_bytes.restype = sz
    lib.hymba_mixer_prefill_chunk_rows.argtypes = [pdesc]
    lib.hymba_mixer_prefill_chunk_rows.restype = ctypes.c_int
    lib.hymba_mixer_decode_workspace_bytes.argtypes = [pdesc]
    lib.hymba_mixer_decode_workspace_bytes.restype = sz
    lib.hymba_mixer_prefill.argtypes = [pdesc, pparams] + [vp] * 8 + [vp] + [vp] * 6 + [vp, sz, vp, vp]
    lib.hymba_mixer_prefill.restype = ctypes.c_int
    lib.hymba_mixer_prefill_continue.argtypes = [pdesc, pparams, i32] + [vp] * 8 + [vp] + [vp] * 6 + [vp, sz, vp]
    lib.hymba_mixer_prefill_continue.restype = ctypes.c_int
    lib.hymba_mixer_decode.argtypes = [pdesc, pparams] + [vp] * 8 + [vp, vp, vp] + [vp, vp] + [vp, vp, vp] + [vp, sz, vp, vp]
    lib.hymba_mixer_decode.restype = ctypes.c_int
    lib.hymba_mixer_decode_noalloc.argtypes = [pdesc, pparams] + [vp] * 8 + [vp, vp, vp] + [vp, vp] + [vp, vp, vp] + [vp]
    lib.hymba_mixer_decode_noalloc.restype = ctypes.c_int
    lib.hymba_fuse_heads.argtypes = [vp, vp, vp, vp, i64, i32, ctypes.c_float, ctypes.c_int, vp, vp]
    lib.hymba_fuse_heads.restype = ctypes.c_int
    lib.hymba_debug_mask_ranges.argtypes = [pdesc, vp, vp]
    lib.hymba_debug_mask_ranges.restype = ctypes.c_int
    lib.hymba_debug_prefill_visibility.argtypes = [pdesc, i32, vp, vp]
    lib.hymba_debug_prefill_visibility.restype = ctypes.c_int
    lib.hymba_status_string.argtypes = [ctypes.c_int]
    lib.hymba_status_string.restype = ctypes.c_char_p
    lib.hymba_last_hip_error.argtypes = []
    lib.hymba_last_hip_error.restype = ctypes.c_int
    lib.hymba_abi_version.argtypes = []
    lib.hymba_abi_version.restype = ctypes.c_int
    _lib = lib
    return lib


PREFILL_STAGES = ("ssm_chunk_end", "ssm_chunk_carry", "ssm_chunk_out", "rope_prefill", "attn_prefill", "fuse")
DECODE_STAGES = ("ssm_decode", "attn_decode", "decode_merge_fuse")


def make_desc(batch, n_meta, n_tokens, d_inner, n_q_heads, n_kv_heads, window, act, head_dim=64,
              head_dim_v=None, d_state=16, d_conv=4, cache_capacity=0, rope_base=10000.0,
              norm_eps=1e-6, cache_ring=False, ssm_heads=0) -> MixerDesc:
    if head_dim_v is None:
        head_dim_v = d_inner // n_q_heads
    act_code = {"f32": HYMBA_F32, "bf16": HYMBA_BF16}.get(act, act)
    return MixerDesc(batch, n_meta, n_tokens, d_inner, d_state, d_conv, n_q_heads, n_kv_heads, head_dim,
                     head_dim_v, window, cache_capacity, rope_base, norm_eps, act_code, int(bool(cache_ring)),
                     int(ssm_heads))


def make_params(A, D, conv_w, beta_attn, beta_ssm, k_scale=None, k_bias=None) -> MixerParams:
    """k_scale / k_bias: [n_kv_heads, head_dim] fp32 affine on shared keys, or None."""
    return MixerParams(_ptr(A), _ptr(D), _ptr(conv_w), None, _ptr(beta_attn), _ptr(beta_ssm), _ptr(k_scale),
                       _ptr(k_bias))


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, status: int):
    if status != 0:
        lib = load_library()
        detail = ""
        if status == -4:
            detail = f"hipError {lib.hymba_last_hip_error()}"
        raise HymbaError(fn, status, detail)


def _workspace(nbytes: int, device):
    import torch
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def hymba_mixer_prefill_workspace_bytes(desc: MixerDesc) -> int:
    return int(load_library().hymba_mixer_prefill_workspace_bytes(ctypes.byref(desc)))


def hymba_mixer_prefill_chunk_rows(desc: MixerDesc) -> int:
    return int(load_library().hymba_mixer_prefill_chunk_rows(ctypes.byref(desc)))


def hymba_mixer_decode_workspace_bytes(desc: MixerDesc) -> int:
    return int(load_library().hymba_mixer_decode_workspace_bytes(ctypes.byref(desc)))


def hymba_mixer_prefill(desc: MixerDesc, params: MixerParams, x, z, dt, B, C, q, k, v, out,
                        ssm_state_out=None, conv_state_out=None, k_cache=None, v_cache=None,
                        y_attn_out=None, y_ssm_out=None, workspace=None, stage_events=None, stream=None):
    lib = load_library()
    if workspace is None:
        workspace = _workspace(hymba_mixer_prefill_workspace_bytes(desc), out.device)
    st = lib.hymba_mixer_prefill(
        ctypes.byref(desc), ctypes.byref(params), _ptr(x), _ptr(z), _ptr(dt), _ptr(B), _ptr(C), _ptr(q),
        _ptr(k), _ptr(v), _ptr(out), _ptr(ssm_state_out), _ptr(conv_state_out), _ptr(k_cache), _ptr(v_cache),
        _ptr(y_attn_out), _ptr(y_ssm_out), _ptr(workspace), workspace.numel() * workspace.element_size(),
        stage_events, _stream(stream))
    _check("hymba_mixer_prefill", st)


def hymba_mixer_prefill_continue(desc: MixerDesc, params: MixerParams, pos0: int, x, z, dt, B, C, q, k, v, out,
                                 ssm_state, conv_state, k_cache, v_cache, y_attn_out=None, y_ssm_out=None,
                                 workspace=None, stream=None):
    lib = load_library()
    if workspace is None:
        workspace = _workspace(hymba_mixer_prefill_workspace_bytes(desc), out.device)
    st = lib.hymba_mixer_prefill_continue(
        ctypes.byref(desc), ctypes.byref(params), int(pos0), _ptr(x), _ptr(z), _ptr(dt), _ptr(B), _ptr(C),
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(ssm_state), _ptr(conv_state), _ptr(k_cache), _ptr(v_cache),
        _ptr(y_attn_out), _ptr(y_ssm_out), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream))
    _check("hymba_mixer_prefill_continue", st)


def hymba_mixer_decode(desc: MixerDesc, params: MixerParams, x, z, dt, B, C, q, k_new, v_new, k_cache,
                       v_cache, cache_len, ssm_state, conv_state, out, y_attn_out=None, y_ssm_out=None,
                       workspace=None, stage_events=None, stream=None):
    lib = load_library()
    if workspace is None:
        workspace = _workspace(hymba_mixer_decode_workspace_bytes(desc), out.device)
    st = lib.hymba_mixer_decode(
        ctypes.byref(desc), ctypes.byref(params), _ptr(x), _ptr(z), _ptr(dt), _ptr(B), _ptr(C), _ptr(q),
        _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(cache_len), _ptr(ssm_state),
        _ptr(conv_state), _ptr(out), _ptr(y_attn_out), _ptr(y_ssm_out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), stage_events, _stream(stream))
    _check("hymba_mixer_decode", st)


def hymba_mixer_decode_noalloc(desc: MixerDesc, params: MixerParams, x, z, dt, B, C, q, k_new, v_new, k_cache,
                               v_cache, cache_len, ssm_state, conv_state, out, y_attn_out=None, y_ssm_out=None,
                               stream=None):
    """hymba_mixer_decode with the library's own static scratch (no workspace)."""
    st = load_library().hymba_mixer_decode_noalloc(
        ctypes.byref(desc), ctypes.byref(params), _ptr(x), _ptr(z), _ptr(dt), _ptr(B), _ptr(C), _ptr(q),
        _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(cache_len), _ptr(ssm_state),
        _ptr(conv_state), _ptr(out), _ptr(y_attn_out), _ptr(y_ssm_out), _stream(stream))
    _check("hymba_mixer_decode_noalloc", st)


def hymba_fuse_heads(y_attn, y_ssm, beta_attn, beta_ssm, n_rows: int, width: int, eps: float, act,
                     out, stream=None):
    act_code = {"f32": HYMBA_F32, "bf16": HYMBA_BF16}.get(act, act)
    st = load_library().hymba_fuse_heads(_ptr(y_attn), _ptr(y_ssm), _ptr(beta_attn), _ptr(beta_ssm),
                                         int(n_rows), int(width), float(eps), act_code, _ptr(out),
                                         _stream(stream))
    _check("hymba_fuse_heads", st)


def hymba_debug_mask_ranges(desc: MixerDesc, ranges, stream=None):
    st = load_library().hymba_debug_mask_ranges(ctypes.byref(desc), _ptr(ranges), _stream(stream))
    _check("hymba_debug_mask_ranges", st)


def hymba_debug_prefill_visibility(desc: MixerDesc, pos0: int, out, stream=None):
    st = load_library().hymba_debug_prefill_visibility(ctypes.byref(desc), int(pos0), _ptr(out), _stream(stream))
    _check("hymba_debug_prefill_visibility", st)


def hymba_status_string(status: int) -> str:
    return load_library().hymba_status_string(int(status)).decode()


def hymba_last_hip_error() -> int:
    return int(load_library().hymba_last_hip_error())


def hymba_abi_version() -> int:
    return int(load_library().hymba_abi_version())
