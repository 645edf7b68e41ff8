/*
 * hymba_mixer.h -- C ABI of the Hymba hybrid-head token mixer for MI355X (gfx950).
 *
 * The mixer of one Hymba layer, taking the already-projected tensors. The same
 * rows feed two parallel branches ("Hymba Guide: NVIDIA Hybrid-Head Mamba &
 * Attention SLM", section "1. Parallel Hybrid-Head Layer Formulation"):
 *
 *   Mamba branch     u = causal depthwise conv1d(x);
 *                    h_t = exp(dt_t * A) (.) h_{t-1} + (dt_t * B_t) * u_t,
 *                    y_t = C_t . h_t + D * u_t;  y_ssm = y * silu(z)
 *                    ("Jamba: Hybrid SSM-Transformer", "1. Layer Interleaving
 *                    Ratio"; "Lecture 04 - Beyond the Dense Transformer",
 *                    section 2, discretisation exp(dt A), dt B).
 *   Attention branch GQA softmax(q k^T / sqrt(64)) v with RoPE on q and k, over
 *                    meta-token rows that every later row sees plus a sliding
 *                    window (or all earlier rows in a global layer)
 *                    (Hymba guide, "2. Learnable Meta-Tokens"; 51cto Hymba-1.5B
 *                    article, sections 1-2: GQA, RoPE, sliding-window attention
 *                    in most layers, three full-attention layers).
 *   Fusion           out = (beta_attn * rmsnorm(y_attn) + beta_ssm * rmsnorm(y_ssm)) / 2
 *                    per row (RMS norm over the row's d_inner channels, no gain).
 *
 * Conventions shared by every entry point:
 *  - Tensor pointers are DEVICE pointers, caller-owned, contiguous row-major,
 *    16-byte aligned. The library never allocates or frees device memory and
 *    never synchronises the host; scratch space comes from the caller's
 *    `workspace` argument (size from the *_workspace_bytes queries).
 *  - All argument checks run on the host first; on any error nothing is
 *    enqueued and a negative hymba_status is returned.
 *  - Work is enqueued asynchronously on `stream` (NULL = the null stream).
 *    Results are deterministic run to run: reductions use no atomics.
 *  - Inputs are read-only. No output may alias an input or another output.
 *  - Activation tensors (x, z, dt, B, C, q, k, v, out, y_*, conv state, KV
 *    cache) share one dtype, `act`. Parameters and the SSM state are fp32.
 *    Arithmetic is fp32 throughout; bf16 products on the matrix cores
 *    accumulate in fp32; each output is rounded once to its storage type.
 *  - Return value: HYMBA_OK, or a negative hymba_status. HYMBA_EHIP means a
 *    HIP call failed; hymba_last_hip_error() gives its hipError_t (per thread).
 *  - State kept by the library: the last HIP error (per thread); per calling
 *    thread and device, a second stream (non-blocking, default priority) and
 *    two events, created on the first prefill call, on which one branch of a
 *    prefill runs beside the other (joined on `stream` before the fusion);
 *    the compute-unit count of each device, read once; and the
 *    static scratch of hymba_mixer_decode_noalloc on each device. Nothing else
 *    persists between calls.
 *  - Beyond the minimal interface (tensors, sizes, stream), prefill and decode
 *    take a caller workspace (the library never allocates) and an optional
 *    array of events that time each stage.
 */
#ifndef HYMBA_MIXER_H_
#define HYMBA_MIXER_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HYMBA_ABI_VERSION 2
#define HYMBA_PREFILL_STAGES 6
#define HYMBA_DECODE_STAGES 3
/* Bytes of the library-owned device scratch of hymba_mixer_decode_noalloc,
 * one copy per device that the library runs on. */
#define HYMBA_DECODE_SCRATCH_BYTES (16u << 20)

/* Activation dtype. C++ sees the same 32-bit enum with a fixed underlying
 * type, so that checking a caller's out-of-range value is well defined. */
#ifdef __cplusplus
typedef enum : int32_t { HYMBA_F32 = 0, HYMBA_BF16 = 1 } hymba_dtype;
#else
typedef enum { HYMBA_F32 = 0, HYMBA_BF16 = 1 } hymba_dtype;
#endif

typedef enum {
  HYMBA_OK = 0,
  HYMBA_EINVAL = -1,        /* null pointer, bad size or inconsistent geometry */
  HYMBA_EUNSUPPORTED = -2,  /* valid geometry this build has no kernel for     */
  HYMBA_EALIGN = -3,        /* a tensor pointer is not 16-byte aligned          */
  HYMBA_EHIP = -4,          /* a HIP runtime call or kernel launch failed       */
  HYMBA_EWORKSPACE = -5     /* workspace missing or smaller than required       */
} hymba_status;

/* Geometry of one mixer call.
 *  batch       sequences (prefill) or sequences with one new row each (decode)
 *  n_meta      meta-token rows at the start of every sequence (Hymba guide,
 *              "2. Learnable Meta-Tokens": prepended to the prompt)
 *  n_tokens    prompt rows after the meta rows (prefill); L = n_meta + n_tokens
 *              rows per sequence. A continuation call processes n_tokens rows.
 *              Decode ignores it.
 *  d_inner     Mamba channels; also the attention output width (n_q_heads * head_dim_v)
 *  d_state     SSM state size per channel: 16 (Hymba-1.5B article, section 2)
 *  d_conv      conv taps: 4
 *  n_q_heads, n_kv_heads   GQA: query head h reads kv head h / (n_q_heads / n_kv_heads);
 *              this build supports groups of up to 8 query heads per kv head
 *  head_dim    query/key width: 64
 *  head_dim_v  value width: d_inner / n_q_heads, one of 32, 64, 128
 *  window      > 0: query row i sees non-meta key rows j with i - j < window;
 *              <= 0: global causal layer. Meta rows are always visible.
 *  cache_capacity  rows per sequence in k_cache / v_cache
 *  rope_base   rotary base (10000); rotation pairs element i with i + head_dim/2
 *  norm_eps    added to the mean square in the RMS norm (1e-6)
 *  act         dtype of every activation tensor and of the KV cache
 *  cache_ring  0: cache row p holds position p. 1: the compact cache of a
 *              sliding-window layer (Hymba-1.5B article, section 1): position
 *              p < n_meta at row p, later positions in a ring of `window` rows,
 *              row n_meta + (p - n_meta) % window. A query at position p needs
 *              no older row, so the cache holds n_meta + window rows whatever
 *              the context length. Needs window > 0 and
 *              cache_capacity >= n_meta + window.
 *  ssm_heads   0: the selective scan with A [d_inner, d_state] and dt per
 *              channel. > 0: the Mamba-2 form ("Lecture 04 - Beyond the Dense
 *              Transformer", section 3): ssm_heads heads of P = d_inner /
 *              ssm_heads consecutive channels, each with one decay rate and
 *              one step size, so A is [ssm_heads] and dt [.., ssm_heads]
 *              (prefill [batch, L, ssm_heads], decode [batch, ssm_heads]);
 *              states keep their [batch, d_inner, d_state] layout. This build
 *              has kernels for P = 32, 64, 128.
 */
typedef struct {
  int32_t batch, n_meta, n_tokens;
  int32_t d_inner, d_state, d_conv;
  int32_t n_q_heads, n_kv_heads, head_dim, head_dim_v;
  int32_t window;
  int32_t cache_capacity;
  float rope_base, norm_eps;
  hymba_dtype act;
  int32_t cache_ring;
  int32_t ssm_heads;
} hymba_mixer_desc;

/* Per-layer fp32 parameters, device pointers.
 *  A          [d_inner, d_state], negative entries (continuous-time decay)
 *  D          [d_inner] skip weight
 *  conv_w     [d_inner, d_conv]; tap d_conv-1 multiplies the current row
 *  conv_b     must be NULL (the conv has no bias)
 *  beta_attn, beta_ssm   [d_inner] per-channel scales of the fusion
 *  k_scale, k_bias       [n_kv_heads, head_dim] or NULL: the head-specific
 *      affine a layer applies to keys it reads from another layer's shared
 *      cache, K' = K * k_scale + k_bias on the rotated keys (Hymba guide,
 *      "Systems Mechanics: Cross-Layer KV Cache Sharing", section 1). Values
 *      are shared unchanged. NULL k_scale = all ones. The library scales the
 *      rotated queries by k_scale of their kv head instead of touching the
 *      keys; k_bias adds q . k_bias to every score of a query, which the
 *      softmax removes, so it is accepted and never read. The cache and
 *      k_rot outputs always hold the keys without the affine.             */
typedef struct {
  const float *A, *D, *conv_w, *conv_b;
  const float *beta_attn, *beta_ssm;
  const float *k_scale, *k_bias;
} hymba_mixer_params;

/* Bytes of caller-provided device workspace the call needs for this geometry
 * (0 if none). Returns 0 as well for an invalid descriptor; the call itself
 * then reports the error. */
size_t hymba_mixer_prefill_workspace_bytes(const hymba_mixer_desc* desc);
size_t hymba_mixer_decode_workspace_bytes(const hymba_mixer_desc* desc);

/* Rows per chunk of the prefill selective scan: the sequence is cut into
 * chunks of this many rows that are scanned in parallel (the first pass
 * computes the end state of every chunk but the last, a carry pass chains
 * them, the output pass rescans every chunk from its carried-in state; in the
 * Mamba-2 form the first pass covers every chunk and the output pass is block
 * matrix products).
 * Host-side query for sizing and work accounting; 0 if desc is invalid. */
int hymba_mixer_prefill_chunk_rows(const hymba_mixer_desc* desc);

/* Prefill of L = n_meta + n_tokens rows per sequence, meta rows first; conv
 * history and SSM state start at zero (the meta rows fill them: Hymba guide,
 * "2. Learnable Meta-Tokens").
 *  x, z, dt   [batch, L, d_inner]   dt already positive (no softplus inside)
 *  B, C       [batch, L, d_state]   shared by all channels
 *  q          [batch, L, n_q_heads, head_dim]    not rotated
 *  k          [batch, L, n_kv_heads, head_dim]   not rotated
 *  v          [batch, L, n_kv_heads, head_dim_v]
 *  out        [batch, L, d_inner]   fused output
 * Optional outputs (NULL = not written):
 *  ssm_state_out   [batch, d_inner, d_state] fp32 state after row L-1
 *  conv_state_out  [batch, d_inner, d_conv-1] raw x of rows L-3..L-1, oldest
 *                  first (zeros where the row index is negative)
 *  k_cache, v_cache  [batch, cache_capacity, n_kv_heads, head_dim(_v)]: the
 *                  rotated keys and the values of rows 0..L-1 are stored, at
 *                  rows 0..L-1 (needs cache_capacity >= L) or, with
 *                  cache_ring, the meta rows and the last `window` rows in
 *                  their ring rows. Pass both or neither.
 *  y_attn_out      [batch, L, d_inner] attention branch before the fusion,
 *                  head-major (channel c = head c / head_dim_v, dim c % head_dim_v)
 *  y_ssm_out       [batch, L, d_inner] Mamba branch before the fusion
 *  workspace       device scratch of hymba_mixer_prefill_workspace_bytes(desc)
 *                  bytes, 256-byte aligned; contents are not preserved.
 *  stage_events    NULL, or 2 * HYMBA_PREFILL_STAGES caller-created events:
 *                  events 2i and 2i+1 are recorded when stage i's kernel starts
 *                  and when it ends (stages: scan chunk end states, chunk
 *                  carries, scan output, rotary, attention, fusion; one kernel
 *                  each; a stage with nothing to do records both back to back).
 *                  For per-kernel timing; the caller owns the events.
 * Without stage events the two branches run concurrently: the one the
 * library estimates to be longer on `stream`, the other on a second stream of
 * the calling thread that waits for the work enqueued on `stream` before the
 * call (the Mamba branch may instead wait for the RoPE pass too); both join
 * on `stream` before the fusion, so ordering on `stream` is as if serial.
 * With stage events every stage runs on `stream`, one after the other.       */
int hymba_mixer_prefill(const hymba_mixer_desc* desc, const hymba_mixer_params* params,
                        const void* x, const void* z, const void* dt, const void* B, const void* C,
                        const void* q, const void* k, const void* v,
                        void* out,
                        float* ssm_state_out, void* conv_state_out,
                        void* k_cache, void* v_cache,
                        void* y_attn_out, void* y_ssm_out,
                        void* workspace, size_t workspace_bytes,
                        hipEvent_t* stage_events, hipStream_t stream);

/* Prefill continued from an earlier call's state: n_tokens further rows per
 * sequence at positions pos0 .. pos0 + n_tokens - 1, the same pos0 for every
 * sequence (chunked prefill). The Mamba branch resumes from the carried SSM
 * state and conv history ("Lecture 04 - Beyond the Dense Transformer",
 * section 2: the fixed-size state is all the scan carries); attention sees the
 * cached rotated keys and values of earlier positions and the new rows under
 * the prefill visibility rule (section 1: the cache grows per token).
 *  pos0        rows already processed per sequence; n_meta <= pos0 (the meta
 *              rows belong to the first call)
 *  x .. v, out as hymba_mixer_prefill, with n_tokens rows (no meta rows)
 *  ssm_state   IN/OUT [batch, d_inner, d_state] fp32: the state after row
 *              pos0 - 1 on entry, after the last new row on return
 *  conv_state  IN/OUT [batch, d_inner, d_conv-1] raw x of the 3 rows before
 *              pos0, oldest first; the last 3 rows on return
 *  k_cache, v_cache  IN/OUT: rotated keys and values of the positions below
 *              pos0 that a new row can see (rows as cache_ring says); the new
 *              rows are stored the same way. Without cache_ring needs
 *              cache_capacity >= pos0 + n_tokens.
 *  y_attn_out, y_ssm_out  optional, [batch, n_tokens, d_inner]
 *  workspace   hymba_mixer_prefill_workspace_bytes(desc) bytes, 256-byte aligned
 * The two branches run concurrently as in hymba_mixer_prefill.               */
int hymba_mixer_prefill_continue(const hymba_mixer_desc* desc, const hymba_mixer_params* params, int32_t pos0,
                                 const void* x, const void* z, const void* dt, const void* B, const void* C,
                                 const void* q, const void* k, const void* v,
                                 void* out,
                                 float* ssm_state, void* conv_state,
                                 void* k_cache, void* v_cache,
                                 void* y_attn_out, void* y_ssm_out,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* One decode step: one new row per sequence at position p_b = cache_len[b]
 * ("Lecture 04 - Beyond the Dense Transformer", section 1: the new token
 * attends over the cached rows and itself; section 2: the SSM state is updated
 * once and does not grow).
 *  x, z, dt   [batch, d_inner];  B, C [batch, d_state]
 *  q          [batch, n_q_heads, head_dim]; k_new [batch, n_kv_heads, head_dim];
 *  v_new      [batch, n_kv_heads, head_dim_v]   (q, k_new not rotated: both are
 *             rotated to position p_b inside)
 *  k_cache, v_cache  READ-ONLY [batch, cache_capacity, n_kv_heads, head_dim(_v)]
 *             holding rotated keys and values of rows < p_b (with cache_ring:
 *             of the positions p_b can see, in their ring rows). Several layers may
 *             pass the same buffers (Hymba guide, "Systems Mechanics: Cross-Layer
 *             KV Cache Sharing"); the library never writes them. Appending the
 *             new row is the caller's job.
 *  cache_len  [batch] int32 on the device; n_meta <= p_b <= cache_capacity is the
 *             caller's contract (with cache_ring, any p_b >= n_meta). Values
 *             that break it are clamped to [0, cache_capacity] (ring: to
 *             p_b >= 0) so that no access leaves the buffers.
 *  ssm_state  IN/OUT [batch, d_inner, d_state] fp32, updated in place
 *  conv_state IN/OUT [batch, d_inner, d_conv-1] raw x, oldest first, shifted in place
 *  out        [batch, d_inner]; y_attn_out, y_ssm_out optional [batch, d_inner]
 *  workspace  hymba_mixer_decode_workspace_bytes(desc) bytes, 256-byte aligned.
 *  stage_events NULL, or 2 * HYMBA_DECODE_STAGES caller-created events: start
 *             and end of each stage as for prefill (stages: SSM step, query/key
 *             rotation + attention partials, merge + fusion; the start event
 *             is taken by the stage's first kernel, the end by its last). In
 *             bf16 the SSM step runs inside the attention stage's launch, as
 *             workgroups of its own, and its stage records both events back
 *             to back. */
int hymba_mixer_decode(const hymba_mixer_desc* desc, const hymba_mixer_params* params,
                       const void* x, const void* z, const void* dt, const void* B, const void* C,
                       const void* q, const void* k_new, const void* v_new,
                       const void* k_cache, const void* v_cache, const int32_t* cache_len,
                       float* ssm_state, void* conv_state,
                       void* out, void* y_attn_out, void* y_ssm_out,
                       void* workspace, size_t workspace_bytes,
                       hipEvent_t* stage_events, hipStream_t stream);

/* hymba_mixer_decode without a workspace argument and without any device
 * allocation, for callers that cannot allocate: code under HIP graph capture,
 * serving loops that forbid hipMalloc, harnesses that manage all memory.
 * Same arguments, results and in-place updates as hymba_mixer_decode (minus
 * workspace and stage events); the kernels are the same. Its scratch (split
 * partials [batch, n_q_heads, n_split, head_dim_v + 2] fp32 for the n_split
 * splits the launch uses, and the branch outputs the caller does not ask for)
 * lives in a static device array of HYMBA_DECODE_SCRATCH_BYTES bytes that the
 * library holds on each device until the process ends. A geometry whose
 * scratch does not fit returns HYMBA_EWORKSPACE before anything is enqueued
 * (the decode workload of 64 sequences, 25 query heads of 128 values and a
 * 1152-key window needs about 5.8 MB). No part of the scratch has to start
 * at zero: every call writes all of it that it reads. All calls on one device
 * share the array, so calls that overlap on one device (concurrent streams or
 * threads) race and give undefined results; calls in one stream order are
 * safe. The caller still provides every input and output.                */
int hymba_mixer_decode_noalloc(const hymba_mixer_desc* desc, const hymba_mixer_params* params,
                               const void* x, const void* z, const void* dt, const void* B, const void* C,
                               const void* q, const void* k_new, const void* v_new,
                               const void* k_cache, const void* v_cache, const int32_t* cache_len,
                               float* ssm_state, void* conv_state,
                               void* out, void* y_attn_out, void* y_ssm_out, hipStream_t stream);

/* The fusion on its own: for each of n_rows rows of `width` channels,
 *   out = (beta_attn * y_attn / sqrt(mean(y_attn^2) + eps)
 *        + beta_ssm  * y_ssm  / sqrt(mean(y_ssm^2)  + eps)) / 2.
 * y_attn, y_ssm, out: [n_rows, width] of dtype act; beta_*: [width] fp32.
 * n_rows may be 0 (nothing enqueued). width >= 1.                            */
int hymba_fuse_heads(const void* y_attn, const void* y_ssm,
                     const float* beta_attn, const float* beta_ssm,
                     int64_t n_rows, int32_t width, float eps, hymba_dtype act,
                     void* out, hipStream_t stream);

/* The visibility rule as the decode attention applies it (one query row at a
 * position p sees the meta rows [0, min(n_meta, p+1)) and the window rows),
 * exported for exact tests ("Hymba Guide: NVIDIA Hybrid-Head Mamba &
 * Attention SLM", "2. Learnable Meta-Tokens": meta rows stay visible to every
 * later row under any window).
 * For each query row i < L = n_meta + n_tokens writes 4 int32 to ranges[4*i]:
 *   meta_end   visible meta keys are [0, meta_end)         = min(n_meta, i+1)
 *   win_begin, win_end   visible non-meta keys are [win_begin, win_end); both
 *              equal n_meta when there are none
 *   count      number of visible keys
 * ranges: device int32 [L, 4].                                               */
int hymba_debug_mask_ranges(const hymba_mixer_desc* desc, int32_t* ranges, hipStream_t stream);

/* The prefill attention's own visibility decisions, exported for exact tests:
 * the kernel's work order, key-tile walk, per-wave decisions to skip a 32-key
 * sub-tile or take it unmasked, and per-lane masking, run on zero scores.
 * For each sequence b, query row r and query head h writes 4 int32 at
 * out[((b * Lq + r) * n_q_heads + h) * 4] in the format of
 * hymba_debug_mask_ranges: [meta_end, win_begin, win_end, count], where count
 * is the number of keys whose score the kernel keeps (so the kept keys are
 * exactly the two ranges when count = meta_end + win_end - win_begin).
 *  pos0   0: a fresh prefill of Lq = n_meta + n_tokens rows at positions
 *         0 .. Lq-1; > 0: a continuation of Lq = n_tokens rows at positions
 *         pos0 .. pos0+Lq-1 over a cache of one row per position (n_meta <=
 *         pos0).
 *  out    device int32 [batch, Lq, n_q_heads, 4]; entries are written once
 *         each; rows of a column without a query are not written.
 * Errors as hymba_mixer_prefill (geometry), HYMBA_EINVAL for a bad pos0.    */
int hymba_debug_prefill_visibility(const hymba_mixer_desc* desc, int32_t pos0, int32_t* out, hipStream_t stream);

/* Static text for a hymba_status value. */
const char* hymba_status_string(int status);

/* hipError_t of the last failed HIP call made by this library on the calling
 * thread (hipSuccess if none). */
int hymba_last_hip_error(void);

/* HYMBA_ABI_VERSION of the built library. */
int hymba_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HYMBA_MIXER_H_ */
