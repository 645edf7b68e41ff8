"""Float64 CPU oracle of the Hymba hybrid-head mixer (test infrastructure only).

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
use this module. Everything here is the plain definition, evaluated the slow
and obvious way in NumPy float64 from the exact stored input values:

* the Mamba branch: causal depthwise conv, the selective SSM recurrence run as
  a sequential loop over time, the D skip and the silu(z) gate;
* the attention branch: rotary embedding, grouped-query softmax attention over
  a full score matrix with an explicit visibility mask (meta prefix, sliding
  window or global causal);
* the fusion: per-row RMS normalisation of each branch, per-channel beta, mean.

Sources (web pages, cited by title and section):

* [Hymba guide] "Hymba Guide: NVIDIA Hybrid-Head Mamba & Attention SLM":
  "1. Parallel Hybrid-Head Layer Formulation", "2. Learnable Meta-Tokens",
  "Systems Mechanics: Cross-Layer KV Cache Sharing".
* [Jamba] "Jamba: Hybrid SSM-Transformer": "How It Actually Works",
  "1. Layer Interleaving Ratio" (selective SSM update, scaled dot-product
  attention), "2. KV Cache Memory Economics", "Worked Example", "Code".
* [Lecture 04] "Lecture 04 - Beyond the Dense Transformer: Mamba, SSMs, and
  the Hybrid Wave": section 1 (the KV cache loop), section 2 (SSM loop,
  discretisation and the two limits of the step size), section 8 (sizes).
* [Hymba-1.5B article] 51cto release article on Hymba-1.5B-Base: section 1
  (meta tokens, cross-layer KV sharing, sliding-window attention), section 2
  (model shapes: GQA, RoPE, 16 SSM states, 3 full-attention layers).

Where the pages leave a step open, the plainest reading is taken; each such
reading is named in the docstring of the function that applies it. The pages
print no mixer output, so the numerics of the readings themselves (conv taps,
RoPE pairing, value-head width, norm type) are fixed only by those readings;
every function below is pinned by the CPU tests to closed forms, brute force,
invariants or library routines.
"""
from __future__ import annotations

from typing import Dict, Iterable, Optional

import numpy as np

F64 = np.float64


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=F64)


# ---------------------------------------------------------------------------
# Mamba branch


def causal_conv1d(x, w, history=None) -> np.ndarray:
    """Causal depthwise conv along time, per channel.

    u[b,t,c] = sum_j w[c,j] * x[b, t-(K-1)+j, c]; the last tap multiplies the
    current row. Rows before the start come from ``history`` ([B, K-1, D],
    oldest first) or are zero. No bias and no activation after the conv.
    The pages do not describe this conv; this is the plain reading of a causal
    depthwise conv1d placed before the selective scan.

    x: [B, L, D]; w: [D, K] -> u: [B, L, D]
    """
    x = _f64(x)
    w = _f64(w)
    Bsz, L, D = x.shape
    K = w.shape[1]
    if history is None:
        pad = np.zeros((Bsz, K - 1, D), F64)
    else:
        pad = _f64(history)
    xp = np.concatenate([pad, x], axis=1)  # row t of x is row t+K-1 of xp
    u = np.zeros((Bsz, L, D), F64)
    for j in range(K):
        u += w[None, None, :, j] * xp[:, j:j + L, :]
    return u


def selective_scan(u, dt, A, Bm, Cm, D, h0=None):
    """Selective SSM recurrence, one time step after another.

    Jamba, "1. Layer Interleaving Ratio": h_t = exp(dt_t A) h_{t-1} + (dt_t B_t) x_t,
    y_t = C_t h_t. Lecture 04, section 2: A is discretised as exp(dt A) and B as
    dt B; section 2's loop carries a fixed-size state through time. Here A is
    per (channel, state) and diagonal, so the update is element-wise per
    state; B_t and C_t are shared by all channels; D adds the skip D*u_t.

    u, dt: [B, L, D]; A: [D, N]; Bm, Cm: [B, L, N]; D: [D]; h0: [B, D, N] or None.
    Returns y [B, L, D] (before the gate) and the final state [B, D, N].
    """
    u, dt, A, Bm, Cm, D = map(_f64, (u, dt, A, Bm, Cm, D))
    Bsz, L, Dch = u.shape
    N = A.shape[1]
    h = np.zeros((Bsz, Dch, N), F64) if h0 is None else _f64(h0).copy()
    y = np.zeros((Bsz, L, Dch), F64)
    for t in range(L):
        dA = np.exp(dt[:, t, :, None] * A[None, :, :])                 # exp(dt A)
        dBx = (dt[:, t, :, None] * Bm[:, t, None, :]) * u[:, t, :, None]  # (dt B) x
        h = dA * h + dBx
        y[:, t, :] = np.einsum("bdn,bn->bd", h, Cm[:, t, :]) + D[None, :] * u[:, t, :]
    return y, h


def ssd_scan(u, dt, A, Bm, Cm, D, h0=None):
    """The Mamba-2 form of the selective SSM, one time step after another
    (Lecture 04, section 3: the state matrix is a scalar times the identity,
    with heads as in attention; the recurrence is one of the two ways to
    compute the layer, the block-matmul form the other).

    Channels are grouped into H heads of P = D / H consecutive channels; head
    h has one decay rate A[h] and one step size dt[:, t, h], so a step decays
    the head's whole P x N state by the scalar exp(dt A):
      h_t = exp(dt_t A) h_{t-1} + dt_t x_t B_t^T,  y_t = h_t C_t + D x_t.
    B and C are shared by all heads.

    u: [B, L, D]; dt: [B, L, H]; A: [H]; Bm, Cm: [B, L, N]; D: [D];
    h0: [B, D, N] or None (row c of the state belongs to head c // P).
    Returns y [B, L, D] (before the gate) and the final state [B, D, N].
    """
    u, dt, A, Bm, Cm, D = map(_f64, (u, dt, A, Bm, Cm, D))
    Bsz, L, Dch = u.shape
    H = A.shape[0]
    P = Dch // H
    N = Bm.shape[2]
    h = np.zeros((Bsz, H, P, N), F64) if h0 is None else _f64(h0).reshape(Bsz, H, P, N).copy()
    y = np.zeros((Bsz, L, Dch), F64)
    for t in range(L):
        decay = np.exp(dt[:, t, :] * A[None, :])                              # [B, H]: one scalar per head
        xt = u[:, t, :].reshape(Bsz, H, P)
        h = decay[:, :, None, None] * h + (dt[:, t, :, None, None] * xt[..., None]) * Bm[:, t, None, None, :]
        y[:, t, :] = np.einsum("bhpn,bn->bhp", h, Cm[:, t, :]).reshape(Bsz, Dch) + D[None, :] * u[:, t, :]
    return y, h.reshape(Bsz, Dch, N)


def _scan(cfg, u, dt, A, Bm, Cm, D, h0=None):
    """The Mamba branch's scan for this workload: the Mamba-2 form when the
    configuration has SSM heads, else the selective scan per (channel, state)."""
    if getattr(cfg, "ssm_heads", 0) > 0:
        return ssd_scan(u, dt, A, Bm, Cm, D, h0=h0)
    return selective_scan(u, dt, A, Bm, Cm, D, h0=h0)


def silu_gate(y, z) -> np.ndarray:
    """Output gate of the Mamba branch: y * silu(z), silu(z) = z / (1 + exp(-z)).
    Not described on the pages; the plain reading of a silu(z) gate."""
    y, z = _f64(y), _f64(z)
    return y * (z / (1.0 + np.exp(-z)))


# ---------------------------------------------------------------------------
# Attention branch


def rope_angles(positions, head_dim: int, base: float) -> np.ndarray:
    """angle[p, i] = pos_p * base**(-2i/d) for i < d/2 (float64)."""
    pos = _f64(positions)
    i = np.arange(head_dim // 2, dtype=F64)
    theta = base ** (-2.0 * i / head_dim)
    return pos[:, None] * theta[None, :]


def rope(x, positions, base: float) -> np.ndarray:
    """Rotary position embedding (named in the Hymba-1.5B article, section 2).

    Reading: rotate-half pairing, element i with element i + d/2, by the angle
    pos * base**(-2i/d); absolute positions count the meta rows.
    x: [..., P, H, d] with positions [P] -> same shape.
    """
    x = _f64(x)
    d = x.shape[-1]
    ang = rope_angles(positions, d, base)          # [P, d/2]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1, x2 = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def visible(i, j, n_meta: int, window: int):
    """May query row i attend to key row j?

    Causal (j <= i). Meta rows (j < n_meta) are visible to every later row
    under any window (Hymba guide, "2. Learnable Meta-Tokens"; Hymba-1.5B
    article, section 2: meta tokens interact with all later tokens). Other
    rows need i - j < window when the layer uses a sliding window (window > 0);
    window <= 0 is a global (full causal) layer.
    Works element-wise on integer arrays.
    """
    i = np.asarray(i)
    j = np.asarray(j)
    ok = j <= i
    if window > 0:
        ok = ok & ((j < n_meta) | (i - j < window))
    return ok


def mask_ranges(n_rows: int, n_meta: int, window: int) -> np.ndarray:
    """Per query row: [meta_end, win_begin, win_end, count] (int32).

    Found by enumerating ``visible`` over every key j: the visible meta keys
    are [0, meta_end); the visible non-meta keys are [win_begin, win_end)
    (both equal to n_meta when there are none); count is the number of
    visible keys.
    """
    out = np.zeros((n_rows, 4), np.int32)
    j = np.arange(n_rows)
    for i in range(n_rows):
        vis = visible(i, j, n_meta, window)
        meta_vis = np.nonzero(vis & (j < n_meta))[0]
        win_vis = np.nonzero(vis & (j >= n_meta))[0]
        meta_end = int(meta_vis.max()) + 1 if meta_vis.size else 0
        if win_vis.size:
            wb, we = int(win_vis.min()), int(win_vis.max()) + 1
        else:
            wb = we = n_meta
        out[i] = (meta_end, wb, we, int(vis.sum()))
    return out


def attention(q_rot, k_rot, v, n_meta: int, window: int, rows: Optional[np.ndarray] = None,
              key_positions: Optional[np.ndarray] = None, query_positions: Optional[np.ndarray] = None,
              block: int = 512) -> np.ndarray:
    """Grouped-query scaled dot-product attention over a visibility mask.

    Jamba, "1. Layer Interleaving Ratio": softmax(Q K^T / sqrt(d_k)) V. Each
    group of Hq/Hkv consecutive query heads reads one key/value head
    (GQA, Hymba-1.5B article, section 2). A full score block is formed per
    (sequence, head), invisible entries are removed, and the softmax subtracts
    the row maximum before exponentiating.

    q_rot: [B, Lq, Hq, d]; k_rot: [B, Lk, Hkv, d]; v: [B, Lk, Hkv, dv]
    rows: query rows to evaluate (default all); returns [B, len(rows), Hq, dv].
    Positions default to the row indices (prefill).
    """
    q_rot, k_rot, v = _f64(q_rot), _f64(k_rot), _f64(v)
    Bsz, Lq, Hq, d = q_rot.shape
    Lk, Hkv, dv = k_rot.shape[1], k_rot.shape[2], v.shape[3]
    group = Hq // Hkv
    if rows is None:
        rows = np.arange(Lq)
    rows = np.asarray(rows)
    qpos = np.arange(Lq) if query_positions is None else np.asarray(query_positions)
    kpos = np.arange(Lk) if key_positions is None else np.asarray(key_positions)
    scale = 1.0 / np.sqrt(d)
    out = np.zeros((Bsz, len(rows), Hq, dv), F64)
    for b in range(Bsz):
        for h in range(Hq):
            g = h // group
            K = k_rot[b, :, g, :]
            V = v[b, :, g, :]
            for r0 in range(0, len(rows), block):
                rr = rows[r0:r0 + block]
                s = (q_rot[b, rr, h, :] @ K.T) * scale              # [nr, Lk]
                m = visible(qpos[rr][:, None], kpos[None, :], n_meta, window)
                s = np.where(m, s, -np.inf)
                s = s - s.max(axis=1, keepdims=True)
                p = np.exp(s)
                p /= p.sum(axis=1, keepdims=True)
                out[b, r0:r0 + len(rr), h, :] = p @ V
    return out


def shared_key_affine(k_rot, k_scale=None, k_bias=None) -> np.ndarray:
    """Keys as a secondary layer sees a primary layer's shared cache: the
    head-specific affine K~ = K (.) w_scale + b_bias (Hymba guide, "Systems
    Mechanics: Cross-Layer KV Cache Sharing", "1. The KV Sharing Mechanism").

    Reading: w_scale and b_bias are per kv head vectors over the key
    dimension, [Hkv, d], applied element-wise to the keys as the cache holds
    them (rotated); the values are shared unchanged (the pages' formula names
    the keys only). None = identity. k_rot: [..., Hkv, d].
    """
    k = _f64(k_rot)
    if k_scale is not None:
        k = k * _f64(k_scale)
    if k_bias is not None:
        k = k + _f64(k_bias)
    return k


# ---------------------------------------------------------------------------
# Fusion of the two branches


def rms_fuse(y_attn, y_ssm, beta_attn, beta_ssm, eps: float) -> np.ndarray:
    """out = (beta_attn * n(y_attn) + beta_ssm * n(y_ssm)) / 2 per row, with
    n(y) = y / sqrt(mean(y^2) + eps) over the row's channels.

    The pages combine the two head families (Hymba guide, "1. Parallel
    Hybrid-Head Layer Formulation", concatenation then an output projection
    outside this mixer); the normalise-scale-average combination is the
    reading used here: RMS norm without a separate gain, per-channel beta.
    y_attn, y_ssm: [..., W]; beta_*: [W].
    """
    ya, ys = _f64(y_attn), _f64(y_ssm)
    na = ya / np.sqrt(np.mean(ya * ya, axis=-1, keepdims=True) + eps)
    ns = ys / np.sqrt(np.mean(ys * ys, axis=-1, keepdims=True) + eps)
    return 0.5 * (_f64(beta_attn) * na + _f64(beta_ssm) * ns)


# ---------------------------------------------------------------------------
# Whole mixer


def mixer_prefill(cfg, inp: Dict[str, np.ndarray], batches: Optional[Iterable[int]] = None,
                  rows: Optional[np.ndarray] = None, with_attention: bool = True) -> Dict[str, np.ndarray]:
    """Prefill of L = n_meta + n_tokens rows per sequence, meta rows first
    (Hymba guide, "2. Learnable Meta-Tokens": meta tokens are prepended; they
    pre-populate the SSM state and stay visible to attention).

    Both branches read the same rows (Hymba guide, "1. Parallel Hybrid-Head
    Layer Formulation"). The conv history and SSM state start at zero.

    ``batches`` restricts to some sequences; ``rows`` restricts the attention
    and fused outputs to some query rows (the scan always runs over all rows).
    Optional inp["k_scale"], inp["k_bias"] ([Hkv, d]): the attention reads the
    keys through shared_key_affine (a secondary layer); k_rot, the keys a
    cache would store, are returned without it.
    Returns float64 arrays: y_ssm [b, L, D], ssm_state [b, D, N],
    conv_state [b, D, K-1] (last K-1 raw x rows, oldest first),
    k_rot [b, L, Hkv, d], and for the selected rows y_attn [b, R, D] and
    out [b, R, D].
    """
    bsel = np.arange(cfg.batch) if batches is None else np.asarray(list(batches))
    L = cfg.seq_rows
    rsel = np.arange(L) if rows is None else np.asarray(rows)
    x = _f64(inp["x"])[bsel]
    u = causal_conv1d(x, inp["conv_w"])
    y, h = _scan(cfg, u, _f64(inp["dt"])[bsel], inp["A"], _f64(inp["B"])[bsel], _f64(inp["C"])[bsel], inp["D"])
    y_ssm = silu_gate(y, _f64(inp["z"])[bsel])
    K = cfg.d_conv
    conv_state = np.zeros((len(bsel), cfg.d_inner, K - 1), F64)
    for j in range(K - 1):                       # oldest first
        t = L - (K - 1) + j
        if t >= 0:
            conv_state[:, :, j] = x[:, t, :]
    res = {"y_ssm": y_ssm, "ssm_state": h, "conv_state": conv_state, "rows": rsel}
    pos = np.arange(L)
    k_rot = rope(_f64(inp["k"])[bsel], pos, cfg.rope_base)
    res["k_rot"] = k_rot
    if with_attention:
        q_rot = rope(_f64(inp["q"])[bsel], pos, cfg.rope_base)
        k_att = shared_key_affine(k_rot, inp.get("k_scale"), inp.get("k_bias"))
        ya = attention(q_rot, k_att, _f64(inp["v"])[bsel], cfg.n_meta, cfg.window, rows=rsel)
        y_attn = ya.reshape(len(bsel), len(rsel), cfg.n_q_heads * cfg.head_dim_v)  # head-major concat
        res["y_attn"] = y_attn
        res["out"] = rms_fuse(y_attn, y_ssm[:, rsel, :], inp["beta_attn"], inp["beta_ssm"], cfg.norm_eps)
    return res


# ---------------------------------------------------------------------------
# KV cache layouts: one row per position, or the compact sliding-window form


def ring_slot(positions, n_meta: int, window: int) -> np.ndarray:
    """Cache row of absolute position p in the compact cache of a sliding-window
    layer (Hymba-1.5B article, section 1: SWA layers keep a compact cache).

    Reading: a query at position i sees the meta rows and the positions
    i - window + 1 .. i, so a cache of n_meta + window rows suffices: meta
    rows keep their own row, later positions share a ring of ``window`` rows,
    p -> n_meta + (p - n_meta) mod window. Positions ``window`` apart share a
    row and the later one replaces the earlier, which no query can still see.
    """
    if window <= 0:
        raise ValueError("a compact cache needs a sliding window (window > 0)")
    p = np.asarray(positions, np.int64)
    return np.where(p < n_meta, p, n_meta + (p - n_meta) % window)


def cache_rows(positions, n_meta: int, window: int, ring: bool) -> np.ndarray:
    """Cache row of each position: the position itself, or its ring_slot."""
    p = np.asarray(positions, np.int64)
    return ring_slot(p, n_meta, window) if ring else p


def cache_store(cache, rows, positions, n_meta: int, window: int, ring: bool) -> np.ndarray:
    """A copy of ``cache`` [B, cap, H, d] with rows[:, i] stored at the row of
    positions[i], in increasing position order (so a later position replaces
    an earlier one that shares its ring row)."""
    out = _f64(cache).copy()
    pos = np.asarray(positions, np.int64)
    order = np.argsort(pos, kind="stable")
    dst = cache_rows(pos, n_meta, window, ring)
    for i in order:
        out[:, dst[i]] = _f64(rows)[:, i]
    return out


def visible_history(p: int, n_meta: int, window: int) -> np.ndarray:
    """Positions below p that a query at position p (>= n_meta) can see: the
    meta rows and, under a window, p - window + 1 .. p - 1 (``visible``)."""
    j = np.arange(p)
    return j[visible(p, j, n_meta, window)]


def mixer_prefill_continue(cfg, inp: Dict[str, np.ndarray], pos0: int, ssm_state, conv_state, k_cache, v_cache,
                           ring: bool = False) -> Dict[str, np.ndarray]:
    """Prefill of T further rows per sequence at positions pos0 .. pos0 + T - 1
    (T = inp["x"].shape[1]), continuing an earlier prefill (or decode steps)
    from its state.

    The Mamba branch resumes from the carried state: conv history and SSM state
    after row pos0 - 1 (Hymba guide, "2. Learnable Meta-Tokens": the state
    carries what came before; Lecture 04, section 2: a fixed-size state is all
    the scan needs). Attention sees the cached rotated keys and values of
    earlier positions and the new rows under the usual visibility rule
    (Lecture 04, section 1: the cache grows per token). Reading: pos0 is the
    same for every sequence and pos0 >= n_meta (the meta rows were in the
    first call). The cache is one row per position, or the ring of
    ``ring_slot`` when ``ring``.

    inp: x, z, dt [B,T,D]; B, C [B,T,N]; q [B,T,Hq,d]; k [B,T,Hkv,d];
    v [B,T,Hkv,dv]; parameters; optional k_scale, k_bias (shared_key_affine).
    ssm_state [B,D,N]; conv_state [B,D,K-1] (oldest first); k_cache, v_cache
    [B,cap,Hkv,d(v)] with the rows of positions < pos0.
    Returns y_ssm, y_attn, out [B,T,D]; ssm_state, conv_state after the last
    row; k_rot [B,T,Hkv,d] of the new rows; k_cache, v_cache with the new rows
    stored (copies).
    """
    n_meta, window = cfg.n_meta, cfg.window
    if pos0 < n_meta:
        raise ValueError("a continuation starts at or after the meta rows")
    x = _f64(inp["x"])
    Bsz, T, D = x.shape
    K = cfg.d_conv
    hist = np.transpose(_f64(conv_state), (0, 2, 1))                      # [B,K-1,D]
    u = causal_conv1d(x, inp["conv_w"], history=hist)
    y, h = _scan(cfg, u, _f64(inp["dt"]), inp["A"], _f64(inp["B"]), _f64(inp["C"]), inp["D"], h0=ssm_state)
    y_ssm = silu_gate(y, _f64(inp["z"]))
    xh = np.concatenate([hist, x], axis=1)                                # rows pos0-K+1 .. pos0+T-1
    new_conv = np.transpose(xh[:, -(K - 1):, :], (0, 2, 1))
    pos = pos0 + np.arange(T)
    q_rot = rope(_f64(inp["q"]), pos, cfg.rope_base)
    k_rot = rope(_f64(inp["k"]), pos, cfg.rope_base)
    old = visible_history(pos0, n_meta, window)                           # what any new row may still see
    src = cache_rows(old, n_meta, window, ring)
    keys = np.concatenate([_f64(k_cache)[:, src], k_rot], axis=1)
    vals = np.concatenate([_f64(v_cache)[:, src], _f64(inp["v"])], axis=1)
    keys = shared_key_affine(keys, inp.get("k_scale"), inp.get("k_bias"))
    ya = attention(q_rot, keys, vals, n_meta, window, key_positions=np.concatenate([old, pos]),
                   query_positions=pos)
    y_attn = ya.reshape(Bsz, T, cfg.n_q_heads * cfg.head_dim_v)
    out = rms_fuse(y_attn, y_ssm, inp["beta_attn"], inp["beta_ssm"], cfg.norm_eps)
    return {"y_ssm": y_ssm, "y_attn": y_attn, "out": out, "ssm_state": h, "conv_state": new_conv,
            "k_rot": k_rot,
            "k_cache": cache_store(k_cache, k_rot, pos, n_meta, window, ring),
            "v_cache": cache_store(v_cache, inp["v"], pos, n_meta, window, ring)}


def mixer_decode(cfg, layer_inp: Dict[str, np.ndarray], k_cache, v_cache, k_new, v_new,
                 cache_len, ring: bool = False) -> Dict[str, np.ndarray]:
    """One new row per sequence at position p = cache_len[b].

    Lecture 04, section 1: the new token attends over the cached keys and
    values of earlier rows plus its own; section 2: the SSM carries a fixed
    size state, updated once. The cache holds rotated keys and values for
    rows < p and is only read (Hymba guide, "1. The KV Sharing Mechanism":
    layers that share a cache read the same key/value tensors). Visibility is
    the prefill rule at query row p. Conv state holds the last K-1 raw x rows,
    oldest first, and both states are advanced by one row.

    Optional layer_inp["k_scale"], ["k_bias"] ([Hkv, d]): this layer is a
    secondary one and reads the shared keys (the new row's included) through
    shared_key_affine. With ``ring`` the cache is the compact form of
    ``ring_slot`` and only the positions the new row can see are read from it.

    Returns out, y_attn, y_ssm [B, D] and the new ssm_state [B, D, N],
    conv_state [B, D, K-1] (float64).
    """
    li = layer_inp
    Bsz, D = li["x"].shape
    K = cfg.d_conv
    x = _f64(li["x"])[:, None, :]                                   # [B,1,D]
    hist = np.transpose(_f64(li["conv_state"]), (0, 2, 1))          # [B,K-1,D]
    u = causal_conv1d(x, li["conv_w"], history=hist)
    y, h = _scan(cfg, u, _f64(li["dt"])[:, None, :], li["A"], _f64(li["B"])[:, None, :],
                 _f64(li["C"])[:, None, :], li["D"], h0=li["ssm_state"])
    y_ssm = silu_gate(y, _f64(li["z"])[:, None, :])[:, 0, :]
    new_conv = np.concatenate([_f64(li["conv_state"])[:, :, 1:], _f64(li["x"])[:, :, None]], axis=2)

    Hq, dv = cfg.n_q_heads, cfg.head_dim_v
    y_attn = np.zeros((Bsz, Hq * dv), F64)
    for b in range(Bsz):
        p = int(cache_len[b])
        pos = np.array([p])
        q_rot = rope(_f64(li["q"])[b][None, None], pos, cfg.rope_base)          # [1,1,Hq,d]
        kn = rope(_f64(k_new)[b][None, None], pos, cfg.rope_base)[0]             # [1,Hkv,d]
        old = visible_history(p, cfg.n_meta, cfg.window) if ring else np.arange(p)
        src = cache_rows(old, cfg.n_meta, cfg.window, ring)
        keys = np.concatenate([_f64(k_cache[b])[src], kn], axis=0)[None]         # [1,n+1,Hkv,d]
        keys = shared_key_affine(keys, li.get("k_scale"), li.get("k_bias"))
        vals = np.concatenate([_f64(v_cache[b])[src], _f64(v_new)[b][None]], axis=0)[None]
        ya = attention(q_rot, keys, vals, cfg.n_meta, cfg.window, rows=np.array([0]),
                       key_positions=np.append(old, p), query_positions=pos)
        y_attn[b] = ya.reshape(Hq * dv)
    out = rms_fuse(y_attn, y_ssm, li["beta_attn"], li["beta_ssm"], cfg.norm_eps)
    return {"out": out, "y_attn": y_attn, "y_ssm": y_ssm, "ssm_state": h, "conv_state": new_conv}


# ---------------------------------------------------------------------------
# Cache sizes


def kv_cache_bytes(batch: int, seq_len: int, n_attn_layers: int, kv_heads: int, head_dim: int,
                   dtype_bytes: int = 2) -> int:
    """Jamba, "2. KV Cache Memory Economics": keys and values (factor 2), each
    element dtype_bytes wide, for every token, attention layer, KV head and
    head dimension. Lecture 04, section 1 states the same product."""
    return 2 * dtype_bytes * batch * seq_len * n_attn_layers * kv_heads * head_dim


def ssm_state_bytes(layers: int, heads: int, head_dim: int, d_state: int, batch: int,
                    dtype_bytes: int = 2) -> int:
    """Lecture 04, section 8: the fixed SSM state, independent of context."""
    return layers * heads * head_dim * d_state * batch * dtype_bytes
