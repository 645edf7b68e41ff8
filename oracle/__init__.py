"""CPU oracle for the Hymba hybrid-head mixer (test infrastructure only).

Plain, slow, float64 NumPy definitions of what the mixer computes. Only the
tests, the package smoke check and the benchmark's CPU-baseline leg may import
this package; the GPU library never calls it. It shares no code with the HIP
path (the two meet only in the seeded input generator in ``synth``, which
holds no arithmetic of the method).
"""
from .hymba_oracle import (  # noqa: F401
    causal_conv1d,
    selective_scan,
    ssd_scan,
    silu_gate,
    rope,
    rope_angles,
    visible,
    mask_ranges,
    attention,
    shared_key_affine,
    rms_fuse,
    mixer_prefill,
    mixer_prefill_continue,
    mixer_decode,
    ring_slot,
    cache_rows,
    cache_store,
    visible_history,
    kv_cache_bytes,
    ssm_state_bytes,
)
