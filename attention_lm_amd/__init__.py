"""Hymba hybrid-head token mixer for MI355X (gfx950).

The compute lives in libhymba_mixer.so (hand-written HIP kernels behind a C
ABI, declared in include/hymba_mixer.h); this package only builds it and binds
it with ctypes. See ``attention_lm_amd.build`` and ``attention_lm_amd._lib``.
"""
from ._lib import (  # noqa: F401
    HYMBA_BF16,
    HYMBA_F32,
    HymbaError,
    LIB_PATH,
    MixerDesc,
    MixerParams,
    hymba_abi_version,
    hymba_debug_mask_ranges,
    hymba_debug_prefill_visibility,
    hymba_fuse_heads,
    hymba_last_hip_error,
    hymba_mixer_decode,
    hymba_mixer_decode_noalloc,
    hymba_mixer_decode_workspace_bytes,
    hymba_mixer_prefill,
    hymba_mixer_prefill_chunk_rows,
    hymba_mixer_prefill_continue,
    hymba_mixer_prefill_workspace_bytes,
    hymba_status_string,
    load_library,
    make_desc,
    make_params,
)
