// Internal launchers shared by the C-ABI layer (api.hip) and the kernel files.
// All arguments have been validated by the caller; launchers only enqueue.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/hymba_mixer.h"
#include "ssm_step.hpp"

namespace hymba {

// Optional timing events of one launch, recorded by the dispatch itself
// (start when the kernel begins, stop when it ends).
struct Timing {
  hipEvent_t start = nullptr, stop = nullptr;
};
#define HYMBA_LAUNCH(kernel, grid, block, shmem, stream, tm, ...) \
  hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, (tm).start, (tm).stop, 0, __VA_ARGS__)
// a stage that has nothing to launch still records its events (zero length)
inline hipError_t no_kernel(hipStream_t stream, Timing tm) {
  if (tm.start) {
    hipError_t e = hipEventRecord(tm.start, stream);
    if (e != hipSuccess) return e;
  }
  return tm.stop ? hipEventRecord(tm.stop, stream) : hipSuccess;
}

// fuse.hip ------------------------------------------------------------------
hipError_t launch_fuse(const void* y_attn, const void* y_ssm, const float* beta_attn,
                       const float* beta_ssm, int64_t n_rows, int width, float eps,
                       hymba_dtype act, void* out, hipStream_t stream, Timing tm = {}, int n_cu = 0);
hipError_t launch_mask_ranges(int n_rows, int n_meta, int window, int32_t* ranges,
                              hipStream_t stream);

// ssm.hip -------------------------------------------------------------------
struct SsmPrefillArgs {
  const void *x, *z, *dt, *B, *C;
  const float *A, *D, *conv_w;
  void* y;                 // [batch, L, d_inner] act
  float* state_out;        // optional [batch, d_inner, 16]
  void* conv_state_out;    // optional [batch, d_inner, 3]
  const float* state_in;   // optional [batch, d_inner, 16] state before row 0 (else zero)
  const void* conv_in;     // optional [batch, d_inner, 3] raw x of rows -3..-1 (else zero); not conv_state_out
  float* agg;              // workspace [n_chunks, batch, d_inner, 16]
  float* sdt;              // workspace [n_chunks, batch, d_inner]
  float* carry;            // workspace [n_chunks, batch, d_inner, 16]
  int chunk_rows;          // from ssm_prefill_chunk_rows()
  int batch, L, d_inner;
  int head_width;          // 0: A [d_inner, 16], dt per channel; > 0: Mamba-2 heads of this many channels,
                           // A [d_inner / head_width], dt [batch, L, d_inner / head_width]
  hymba_dtype act;
};
int ssm_prefill_chunk_rows(int batch, int L, int d_inner);
// true when the batch alone fills the chip: the prefill scan is then one pass
// over whole sequences (chunk rows = L, no end-state pass and no carry chain)
bool ssm_single_pass(int batch, int d_inner);
// The three kernels of the chunked prefill scan, in this order: chunk end
// states (nothing to do for a single chunk), carries between chunks, output.
hipError_t launch_ssm_chunk_end(const SsmPrefillArgs& a, hipStream_t stream, Timing tm = {});
hipError_t launch_ssm_chunk_carry(const SsmPrefillArgs& a, hipStream_t stream, Timing tm = {});
hipError_t launch_ssm_chunk_out(const SsmPrefillArgs& a, hipStream_t stream, Timing tm = {});
// The chunk carry chain alone: carry[0] = state_in (or 0), carry[k + 1] =
// exp(a sdt[k]) carry[k] + agg[k] for k < n_slots - 1, per (sequence, channel,
// state); a = A[c, n], or A[c / head_width] when head_width > 0.
hipError_t launch_ssm_carry_chain(const float* A, const float* agg, const float* sdt, const float* state_in,
                                  float* carry, int n_slots, int batch, int d_inner, int head_width,
                                  hipStream_t stream, Timing tm = {});
// Mamba-2 form (ssd.hip): chunk states, carry chain, outputs; rows per chunk
int ssd_chunk_rows();
hipError_t launch_ssd_prefill(const SsmPrefillArgs& a, hipStream_t stream, Timing tm_state = {}, Timing tm_carry = {},
                              Timing tm_out = {});

struct SsmDecodeArgs {
  const void *x, *z, *dt, *B, *C;
  const float *A, *D, *conv_w;
  float* state;            // in/out [batch, d_inner, 16]
  void* conv_state;        // in/out [batch, d_inner, 3] act
  void* y;                 // [batch, d_inner] act
  int batch, d_inner;
  int head_width;          // > 0: Mamba-2 heads (A and dt per head)
  hymba_dtype act;
};
hipError_t launch_ssm_decode(const SsmDecodeArgs& a, hipStream_t stream, Timing tm = {});
template <typename T>
inline ssm_step::Ptrs<T> ssm_step_ptrs(const SsmDecodeArgs& a) {
  ssm_step::Ptrs<T> p;
  p.x = (const T*)a.x; p.z = (const T*)a.z; p.dt = (const T*)a.dt; p.B = (const T*)a.B; p.C = (const T*)a.C;
  p.A = a.A; p.D = a.D; p.conv_w = a.conv_w; p.state = a.state; p.conv_state = (T*)a.conv_state; p.y = (T*)a.y;
  p.d_inner = a.d_inner;
  p.head_width = a.head_width;
  return p;
}

// attn.hip ------------------------------------------------------------------
struct RopeArgs {
  const void *q, *k, *v;   // inputs [batch, L, H, d]
  void* q_rot;             // [batch, L, Hq, hd] act
  void* k_rot;             // rows with stride k_rows per sequence
  void* v_copy;            // optional, rows with stride v_rows per sequence
  int64_t k_rows, v_rows;  // rows per sequence of k_rot / v_copy
  int64_t k_row0, v_row0;  // rows of k_rot / v_copy that receive input row 0
  const float* k_scale;    // [Hkv, 64] or null: query heads of kv head g are scaled by row g
  int batch, L, n_q_heads, n_kv_heads, head_dim, head_dim_v;
  int pos0;                // position of input row 0 (rotation angle)
  float rope_base;
  hymba_dtype act;
};
hipError_t launch_rope_prefill(const RopeArgs& a, hipStream_t stream, Timing tm = {});

struct AttnPrefillArgs {
  const void* q_rot;       // [batch, L, Hq, 64]: query row r is at position q_pos0 + r
  const void* k_rot;       // [batch, k_rows, Hkv, 64]: key row j is at position j
  const void* v;           // [batch, v_rows, Hkv, dv]
  int64_t k_rows, v_rows;
  void* y;                 // [batch, L, Hq*dv] act
  int batch, L, n_meta, window, n_q_heads, n_kv_heads, head_dim_v;
  int q_pos0;
  int n_cu;                // compute units of the device (work ordering)
  hymba_dtype act;
};
hipError_t launch_attn_prefill(const AttnPrefillArgs& a, hipStream_t stream, Timing tm = {});
// the prefill attention's visibility decisions per query column, [batch, Lq, Hq, 4]
// (see prefill_visibility_kernel)
hipError_t launch_prefill_visibility(int batch, int Lq, int q_pos0, int n_meta, int window, int Hq, int Hkv, int n_cu,
                                     int32_t* out, hipStream_t stream);

struct AttnDecodeArgs {
  const void *q, *k_new, *v_new;       // [batch, H, d] not rotated
  const void *k_cache, *v_cache;       // [batch, cap, Hkv, d]
  const int32_t* cache_len;
  float* q_rot;                        // workspace [batch, Hq, 64]
  float* k_rot;                        // workspace [batch, Hkv, 64]
  float* partial;                      // [batch, Hq, n_split, dv + 2]
  const float* k_scale;                // [Hkv, 64] or null (query scale of the shared-key affine)
  int n_split, keys_per_split;         // n_split: splits of this launch (decode_active_splits)
  int n_cu;                            // compute units of the device (split count)
  int batch, cap, n_meta, window, n_q_heads, n_kv_heads, head_dim_v;
  int ring;                            // cache is the compact ring of n_meta + window rows
  float rope_base;
  hymba_dtype act;
  // bf16: the Mamba branch's step of the same call, run by workgroups of its
  // own inside the attention launch (null: none)
  const SsmDecodeArgs* ssm = nullptr;
};
hipError_t launch_attn_decode(const AttnDecodeArgs& a, hipStream_t stream, Timing tm = {});
// partial slots per (sequence, query head) the workspace holds: enough for any launch
void decode_split_plan(int n_meta, int window, int cap, int* n_split, int* keys_per_split);
// splits (partials per head) one launch uses, at most the plan's slot count
int decode_active_splits(const AttnDecodeArgs& a);
// waves of the bf16 decode attention kernel that one compute unit holds
int decode_wave_slots_per_cu(int dv);

// Whole K and V rows (all kv heads) of n positions per sequence, from one
// buffer to another. The positions are [pa, pa + na) then [pb, pb + n - na).
// Each side locates position P of copy index i as kIndex (row i), kLinear
// (row P - base) or kRing (cache row of P in the compact ring).
struct KvSide {
  enum Mode { kIndex = 0, kLinear = 1, kRing = 2 };
  const void* k;
  const void* v;
  int64_t k_rows, v_rows;  // rows per sequence
  int mode, base;
};
struct KvCopyArgs {
  KvSide src, dst;         // (dst.k, dst.v are written)
  int n, na, pa, pb;
  int n_meta, window, batch, n_kv_heads, head_dim_v;
  hymba_dtype act;
};
hipError_t launch_kv_copy(const KvCopyArgs& a, hipStream_t stream);

// decode epilogue: merge of the split partials + fusion with the Mamba output
struct DecodeCombineArgs {
  const float* partial;    // [batch, Hq, n_split, dv + 2]
  const void* y_ssm;       // [batch, Hq * dv] act
  const float *beta_attn, *beta_ssm;
  float eps;
  void* y_attn;            // out [batch, Hq * dv] act
  void* out;               // out [batch, Hq * dv] act
  int n_split, batch, n_q_heads, head_dim_v;
  hymba_dtype act;
};
hipError_t launch_decode_combine(const DecodeCombineArgs& a, hipStream_t stream, Timing tm = {});

}  // namespace hymba
