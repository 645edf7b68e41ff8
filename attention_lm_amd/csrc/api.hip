// C ABI of the Hymba mixer library: argument validation, workspace layout and
// the order of kernel launches. Every check runs before anything is enqueued.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <unordered_map>

#include "../../include/hymba_mixer.h"
#include "launch.hpp"

namespace {

thread_local int g_last_hip_error = 0;

// Per calling thread and device: a second stream (default priority) and two
// events, used to run one prefill branch concurrently with the other.
// Per-thread so that calls from different host threads never share them.
struct ForkCtx {
  hipStream_t aux = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  ~ForkCtx() {
    if (fork) (void)hipEventDestroy(fork);
    if (join) (void)hipEventDestroy(join);
    if (aux) (void)hipStreamDestroy(aux);
  }
};
thread_local std::unordered_map<int, ForkCtx> g_fork;

hipError_t fork_ctx(ForkCtx** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  ForkCtx& c = g_fork[dev];
  if (!c.aux) {
    if ((e = hipStreamCreateWithFlags(&c.aux, hipStreamNonBlocking)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&c.fork, hipEventDisableTiming)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&c.join, hipEventDisableTiming)) != hipSuccess) return e;
  }
  *out = &c;
  return hipSuccess;
}

// Compute units of the current device (cached per device).
hipError_t device_cus(int* n_cu) {
  static std::atomic<int> cache[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *n_cu = c;
      return hipSuccess;
    }
  }
  int v = 0;
  e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (v < 1) v = 1;
  if (dev >= 0 && dev < 64) cache[dev].store(v, std::memory_order_relaxed);
  *n_cu = v;
  return hipSuccess;
}

int hip_status(hipError_t e) {
  if (e == hipSuccess) return HYMBA_OK;
  g_last_hip_error = (int)e;
  return HYMBA_EHIP;
}

#define HYMBA_TRY(expr)                         \
  do {                                          \
    hipError_t e_ = (expr);                     \
    if (e_ != hipSuccess) return hip_status(e_); \
  } while (0)

// inside a function returning hipError_t
#define TRY_E(expr)                  \
  do {                               \
    hipError_t e_ = (expr);          \
    if (e_ != hipSuccess) return e_; \
  } while (0)

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
size_t act_bytes(hymba_dtype t) { return t == HYMBA_BF16 ? 2 : 4; }
size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }

// Geometry checks shared by prefill and decode.
int check_desc(const hymba_mixer_desc* d, bool decode) {
  if (!d) return HYMBA_EINVAL;
  if (d->act != HYMBA_F32 && d->act != HYMBA_BF16) return HYMBA_EINVAL;
  if (d->batch < 1 || d->n_meta < 0 || d->d_inner < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1 ||
      d->head_dim < 1 || d->head_dim_v < 1 || d->d_state < 1 || d->d_conv < 1)
    return HYMBA_EINVAL;
  if (!decode && (d->n_tokens < 0 || (int64_t)d->n_meta + d->n_tokens < 1)) return HYMBA_EINVAL;
  if ((int64_t)d->n_meta + d->n_tokens > INT32_MAX / 2) return HYMBA_EINVAL;
  if (d->n_q_heads % d->n_kv_heads != 0) return HYMBA_EINVAL;
  if ((int64_t)d->n_q_heads * d->head_dim_v != d->d_inner) return HYMBA_EINVAL;
  if (!(d->rope_base > 0.f) || !(d->norm_eps >= 0.f)) return HYMBA_EINVAL;
  if (d->cache_capacity < 0) return HYMBA_EINVAL;
  if (decode && d->cache_capacity < 1) return HYMBA_EINVAL;
  if (d->cache_ring != 0 && d->cache_ring != 1) return HYMBA_EINVAL;
  if (d->ssm_heads < 0 || (d->ssm_heads > 0 && d->d_inner % d->ssm_heads != 0)) return HYMBA_EINVAL;
  if (d->ssm_heads > 0) {   // Mamba-2 heads: widths with a kernel
    const int P = d->d_inner / d->ssm_heads;
    if (P != 32 && P != 64 && P != 128) return HYMBA_EUNSUPPORTED;
  }
  // the compact cache exists for sliding-window layers and holds n_meta + window rows
  if (d->cache_ring && (d->window <= 0 || (int64_t)d->cache_capacity < (int64_t)d->n_meta + d->window))
    return HYMBA_EINVAL;
  // what this build has kernels for
  if (d->d_state != 16 || d->d_conv != 4 || d->head_dim != 64) return HYMBA_EUNSUPPORTED;
  if (d->head_dim_v != 32 && d->head_dim_v != 64 && d->head_dim_v != 128) return HYMBA_EUNSUPPORTED;
  if (d->n_q_heads / d->n_kv_heads > 8) return HYMBA_EUNSUPPORTED;
  if (d->d_inner % 8 != 0) return HYMBA_EUNSUPPORTED;
  // prefill attention addresses one sequence's K and V rows of one kv head
  // with 32-bit byte offsets
  const int64_t row_bytes = (int64_t)d->n_kv_heads * (d->head_dim > d->head_dim_v ? d->head_dim : d->head_dim_v) *
                            (int64_t)act_bytes(d->act);
  if (!decode && ((int64_t)d->n_meta + d->n_tokens) * row_bytes > INT32_MAX) return HYMBA_EUNSUPPORTED;
  // the decode epilogue keeps one sequence's row in the registers of one workgroup
  if (decode && d->d_inner > 16384) return HYMBA_EUNSUPPORTED;
  // decode attention likewise addresses one sequence's cache rows
  if (decode && (int64_t)d->cache_capacity * row_bytes > INT32_MAX) return HYMBA_EUNSUPPORTED;
  // and the scan stores one sequence's y the same way
  if (!decode && ((int64_t)d->n_meta + d->n_tokens) * d->d_inner * (int64_t)act_bytes(d->act) > INT32_MAX)
    return HYMBA_EUNSUPPORTED;
  return HYMBA_OK;
}

int check_params(const hymba_mixer_params* p) {
  if (!p || !p->A || !p->D || !p->conv_w || !p->beta_attn || !p->beta_ssm) return HYMBA_EINVAL;
  if (p->conv_b) return HYMBA_EUNSUPPORTED;
  if (!aligned16(p->A) || !aligned16(p->D) || !aligned16(p->conv_w) || !aligned16(p->beta_attn) ||
      !aligned16(p->beta_ssm) || !aligned16(p->k_scale))
    return HYMBA_EALIGN;
  return HYMBA_OK;
}

// Workspace of both prefill entry points: a fresh prefill has L = n_meta +
// n_tokens rows, a continuation n_tokens rows (and, with the compact cache,
// an assembly of the meta rows, up to window - 1 earlier rows and the new rows
// that its attention reads).
struct PrefillWs {
  size_t q_rot, k_rot, y_attn, y_ssm, agg, sdt, carry, conv_in, asm_k, asm_v, total;
  int chunk_rows;        // fresh prefill
  int chunk_rows_cont;   // continuation
  int asm_rows;          // rows per sequence of the assembly (0 without the compact cache)
  bool carry_ok;
};
PrefillWs prefill_ws(const hymba_mixer_desc* d) {
  const size_t es = act_bytes(d->act);
  const size_t rows = (size_t)d->batch * ((size_t)d->n_meta + d->n_tokens);
  PrefillWs w;
  w.q_rot = 0;
  w.k_rot = w.q_rot + round256(rows * d->n_q_heads * d->head_dim * es);
  w.y_attn = w.k_rot + round256(rows * d->n_kv_heads * d->head_dim * es);
  w.y_ssm = w.y_attn + round256(rows * d->d_inner * es);
  w.agg = w.y_ssm + round256(rows * d->d_inner * es);
  const int L = d->n_meta + d->n_tokens;
  if (d->ssm_heads > 0) {   // Mamba-2 form: fixed chunks
    w.chunk_rows = w.chunk_rows_cont = hymba::ssd_chunk_rows();
  } else {
    w.chunk_rows = hymba::ssm_prefill_chunk_rows(d->batch, L, d->d_inner);
    w.chunk_rows_cont = hymba::ssm_prefill_chunk_rows(d->batch, d->n_tokens > 0 ? d->n_tokens : 1, d->d_inner);
  }
  // (one slot more than chunks: the Mamba-2 form's carry chain also yields the final state)
  const size_t nchunk = 1 + std::max((size_t)((L + w.chunk_rows - 1) / w.chunk_rows),
                                     (size_t)((d->n_tokens + w.chunk_rows_cont - 1) / w.chunk_rows_cont));
  const size_t chans = (size_t)d->batch * d->d_inner;
  w.sdt = w.agg + round256(nchunk * chans * 16 * sizeof(float));
  w.carry = w.sdt + round256(nchunk * chans * sizeof(float));
  w.conv_in = w.carry + round256(nchunk * chans * 16 * sizeof(float));
  w.asm_k = w.conv_in + round256(chans * (d->d_conv - 1) * es);
  w.asm_rows = d->cache_ring ? d->n_meta + d->window - 1 + d->n_tokens : 0;
  const size_t arows = (size_t)d->batch * w.asm_rows;
  w.asm_v = w.asm_k + round256(arows * d->n_kv_heads * d->head_dim * es);
  w.total = w.asm_v + round256(arows * d->n_kv_heads * d->head_dim_v * es);
  w.carry_ok = nchunk * chans * 16 * sizeof(float) <= (size_t)INT32_MAX;   // 32-bit offsets in the carry chain
  return w;
}

// bytes of one cache row (all kv heads) of the wider of K and V
int64_t kv_row_bytes(const hymba_mixer_desc* d) {
  return (int64_t)d->n_kv_heads * (d->head_dim > d->head_dim_v ? d->head_dim : d->head_dim_v) *
         (int64_t)act_bytes(d->act);
}

struct DecodeWs {
  size_t partial, y_ssm, y_attn, q_rot, k_rot, total;
  int n_split, keys_per_split;
};
// Scratch of one decode call: split partials for `slots` splits per (sequence,
// query head), the branch outputs the caller does not keep, and (fp32 path)
// the rotated queries and new keys. slots < 0: the plan's largest split count
// (room for any launch on any device).
DecodeWs decode_ws(const hymba_mixer_desc* d, int slots = -1) {
  DecodeWs w;
  hymba::decode_split_plan(d->n_meta, d->window, d->cache_capacity, &w.n_split, &w.keys_per_split);
  if (slots >= 0) w.n_split = slots;
  const size_t B = (size_t)d->batch;
  w.partial = 0;
  w.y_ssm = round256(B * d->n_q_heads * w.n_split * (d->head_dim_v + 2) * sizeof(float));
  w.y_attn = w.y_ssm + round256(B * d->d_inner * act_bytes(d->act));
  w.q_rot = w.y_attn + round256(B * d->d_inner * act_bytes(d->act));
  w.k_rot = w.q_rot + round256(B * d->n_q_heads * d->head_dim * sizeof(float));
  w.total = w.k_rot + round256(B * d->n_kv_heads * d->head_dim * sizeof(float));
  return w;
}

}  // namespace

extern "C" {

size_t hymba_mixer_prefill_workspace_bytes(const hymba_mixer_desc* desc) {
  if (check_desc(desc, false) != HYMBA_OK) return 0;
  const PrefillWs ws = prefill_ws(desc);
  return ws.carry_ok ? ws.total : 0;
}

int hymba_mixer_prefill_chunk_rows(const hymba_mixer_desc* desc) {
  if (check_desc(desc, false) != HYMBA_OK) return 0;
  return prefill_ws(desc).chunk_rows;
}

size_t hymba_mixer_decode_workspace_bytes(const hymba_mixer_desc* desc) {
  if (check_desc(desc, true) != HYMBA_OK) return 0;
  return decode_ws(desc).total;
}

}  // extern "C"

namespace {

// One prefill call, fresh (pos0 = 0, no carried state) or continuing.
struct PrefillCall {
  const void *x, *z, *dt, *B, *C, *q, *k, *v;
  void* out;
  int pos0;                       // position of the call's first row
  bool cont;                      // continuation: rows are n_tokens rows at pos0 ..
  const float* state_in;          // continuation: carried SSM state (may equal state_out)
  const void* conv_in;            // continuation: carried conv history (may equal conv_out)
  float* state_out;
  void* conv_out;
  void *k_cache, *v_cache;
  void *y_attn_out, *y_ssm_out;
  void* workspace;
  size_t workspace_bytes;
  hipEvent_t* stage_events;
};

// How a concurrent prefill forks. The longer branch should start first. If
// the attention branch is the longer one it runs on `stream` and the Mamba
// branch forks onto the second stream right after the RoPE pass (the
// attention workgroups then take the chip first and the scan's fill in beside
// them). Otherwise the Mamba branch runs on `stream`, its first kernel
// starting at once, and the attention branch (RoPE pass, then attention)
// forks onto the second stream, so that its workgroups arrive after the
// scan's first pass has been dispatched. The branch lengths are estimated from their work at rates
// measured on MI355X for these kernels: attention ~1.0e15 flop/s over the
// visible (query, key) pairs, the single-pass scan ~3.2e12 and the chunked
// scan ~2.0e12 (row, channel, state) elements per second. (Measured with the
// 25q/5kv layers: global layer 0.515 -> 0.486 ms forking late, SWA layer
// 0.116 -> 0.121 ms and the batched workload 1.90 -> 2.00 ms forking late;
// with the Mamba branch on `stream` and the attention branch forked, SWA
// layer 0.123 -> 0.110 ms against the attention branch on `stream`.) The
// Mamba-2 form never forks late.
bool fork_after_rope(const hymba_mixer_desc* d, int pos0, int n_rows) {
  if (d->ssm_heads > 0) return false;
  const double cap = d->window > 0 ? (double)d->n_meta + d->window : 1e300;
  auto vis = [&](double n) {   // sum over rows i < n of min(i + 1, cap)
    return n <= cap ? n * (n + 1) / 2 : cap * (cap + 1) / 2 + (n - cap) * cap;
  };
  const double pairs = (vis((double)pos0 + n_rows) - vis((double)pos0)) * d->batch;
  const double attn_s = pairs * d->n_q_heads * (2.0 * d->head_dim + 2.0 * d->head_dim_v) / 1.0e15;
  const double elems = (double)d->batch * n_rows * d->d_inner * d->d_state;
  const double scan_s = elems / (hymba::ssm_single_pass(d->batch, d->d_inner) ? 3.2e12 : 2.0e12);
  return attn_s > scan_s;
}

int prefill_impl(const hymba_mixer_desc* desc, const hymba_mixer_params* params, const PrefillCall& c,
                 hipStream_t stream) {
  const int M = desc->n_meta, W = desc->window;
  const bool ring = desc->cache_ring != 0;
  const int L = c.cont ? desc->n_tokens : M + desc->n_tokens;   // rows in this call
  const PrefillWs ws = prefill_ws(desc);
  if (!ws.carry_ok) return HYMBA_EUNSUPPORTED;
  if (!c.workspace || c.workspace_bytes < ws.total) return HYMBA_EWORKSPACE;
  if (((uintptr_t)c.workspace & 255u) != 0) return HYMBA_EALIGN;

  char* wsb = (char*)c.workspace;
  void* q_rot = wsb + ws.q_rot;
  void* y_attn = c.y_attn_out ? c.y_attn_out : (void*)(wsb + ws.y_attn);
  void* y_ssm = c.y_ssm_out ? c.y_ssm_out : (void*)(wsb + ws.y_ssm);

  // stage i's kernel records stage_events[2i] when it starts and [2i+1] when it ends
  auto tm = [&](int i) -> hymba::Timing {
    hymba::Timing t;
    if (c.stage_events) {
      t.start = c.stage_events[2 * i];
      t.stop = c.stage_events[2 * i + 1];
    }
    return t;
  };
  // The two branches are independent until the fusion: without stage events
  // they run concurrently, one of them on a second stream.
  ForkCtx* fc = nullptr;
  if (!c.stage_events) HYMBA_TRY(fork_ctx(&fc));
  // The longer branch runs on `stream`, the other on the second stream (see
  // fork_after_rope).
  const bool late = fc && fork_after_rope(desc, c.pos0, L);
  hipStream_t ssm_stream = stream, attn_stream = stream;
  if (fc) (late ? ssm_stream : attn_stream) = fc->aux;
  // Mamba branch (conv + scan), on ssm_stream
  auto mamba_branch = [&]() -> hipError_t {
    hymba::SsmPrefillArgs sa;
    sa.x = c.x; sa.z = c.z; sa.dt = c.dt; sa.B = c.B; sa.C = c.C;
    sa.A = params->A; sa.D = params->D; sa.conv_w = params->conv_w;
    sa.y = y_ssm; sa.state_out = c.state_out; sa.conv_state_out = c.conv_out;
    sa.state_in = c.state_in;
    sa.conv_in = nullptr;
    if (c.conv_in) {   // a private copy: the output pass writes the caller's buffer while it is still read
      void* staged = wsb + ws.conv_in;
      TRY_E(hipMemcpyAsync(staged, c.conv_in,
                           (size_t)desc->batch * desc->d_inner * (desc->d_conv - 1) * act_bytes(desc->act),
                           hipMemcpyDeviceToDevice, ssm_stream));
      sa.conv_in = staged;
    }
    sa.agg = (float*)(wsb + ws.agg); sa.sdt = (float*)(wsb + ws.sdt); sa.carry = (float*)(wsb + ws.carry);
    sa.chunk_rows = c.cont ? ws.chunk_rows_cont : ws.chunk_rows;
    sa.batch = desc->batch; sa.L = L; sa.d_inner = desc->d_inner; sa.act = desc->act;
    sa.head_width = desc->ssm_heads > 0 ? desc->d_inner / desc->ssm_heads : 0;
    if (sa.head_width > 0) {
      TRY_E(hymba::launch_ssd_prefill(sa, ssm_stream, tm(0), tm(1), tm(2)));
    } else {
      TRY_E(hymba::launch_ssm_chunk_end(sa, ssm_stream, tm(0)));
      TRY_E(hymba::launch_ssm_chunk_carry(sa, ssm_stream, tm(1)));
      TRY_E(hymba::launch_ssm_chunk_out(sa, ssm_stream, tm(2)));
    }
    return hipSuccess;
  };

  // The fork point of the branch that runs on the second stream: it waits
  // for what was enqueued on `stream` before the fork.
  auto fork_point = [&]() -> hipError_t {
    TRY_E(hipEventRecord(fc->fork, stream));
    return hipStreamWaitEvent(fc->aux, fc->fork, 0);
  };
  bool forked = false;
  auto after_rope = [&]() -> hipError_t {
    if (!late || forked) return hipSuccess;
    forked = true;
    TRY_E(fork_point());
    TRY_E(mamba_branch());
    return hipEventRecord(fc->join, fc->aux);
  };
  auto attention_branch = [&]() -> hipError_t {
    // Attention branch. Where the rotated keys and the values that attention
    // reads live (row j of k_src / v_src = position j - shift):
    //  * fresh, cache of one row per position: the cache itself (rope stores there);
    //  * fresh otherwise: the workspace keys and the input values;
    //  * continuation, one row per position: the cache (rope appends the new rows);
    //  * continuation, compact ring: an assembly of meta rows, the earlier rows
    //    the new ones can see, and the new rows.
    hymba::RopeArgs ra;
    ra.q = c.q; ra.k = c.k; ra.v = c.v; ra.q_rot = q_rot;
    ra.k_scale = params->k_scale;
    ra.batch = desc->batch; ra.L = L; ra.n_q_heads = desc->n_q_heads; ra.n_kv_heads = desc->n_kv_heads;
    ra.head_dim = desc->head_dim; ra.head_dim_v = desc->head_dim_v; ra.rope_base = desc->rope_base;
    ra.act = desc->act;
    ra.pos0 = c.pos0;
    hymba::AttnPrefillArgs aa;
    aa.q_rot = q_rot; aa.y = y_attn;
    aa.batch = desc->batch; aa.L = L; aa.n_meta = M; aa.window = W;
    aa.n_q_heads = desc->n_q_heads; aa.n_kv_heads = desc->n_kv_heads; aa.head_dim_v = desc->head_dim_v;
    aa.act = desc->act;
    TRY_E(device_cus(&aa.n_cu));
    hymba::KvCopyArgs kc;   // rows into the compact ring (fresh prefill, continuation)
    kc.n = 0;
    kc.n_meta = M; kc.window = W; kc.batch = desc->batch; kc.n_kv_heads = desc->n_kv_heads;
    kc.head_dim_v = desc->head_dim_v; kc.act = desc->act;
    kc.dst.k = c.k_cache; kc.dst.v = c.v_cache; kc.dst.k_rows = kc.dst.v_rows = desc->cache_capacity;
    kc.dst.mode = hymba::KvSide::kRing; kc.dst.base = 0;
    const int64_t cap = desc->cache_capacity;

    if (!c.cont) {
      if (c.k_cache && !ring) {
        ra.k_rot = c.k_cache; ra.k_rows = cap; ra.v_copy = c.v_cache; ra.v_rows = cap;
      } else {
        ra.k_rot = wsb + ws.k_rot; ra.k_rows = L; ra.v_copy = nullptr; ra.v_rows = L;
      }
      ra.k_row0 = ra.v_row0 = 0;
      aa.k_rot = ra.k_rot; aa.k_rows = ra.k_rows; aa.v = c.v; aa.v_rows = L; aa.q_pos0 = 0;
      if (c.k_cache && ring) {   // the meta rows and the last `window` rows survive in the ring
        kc.src.k = ra.k_rot; kc.src.v = c.v; kc.src.k_rows = L; kc.src.v_rows = L;
        kc.src.mode = hymba::KvSide::kLinear; kc.src.base = 0;
        kc.na = std::min(M, L); kc.pa = 0; kc.pb = std::max(M, L - W);
        kc.n = kc.na + (L - kc.pb);
      }
      TRY_E(hymba::launch_rope_prefill(ra, attn_stream, tm(3)));
      TRY_E(after_rope());
    } else if (!ring) {
      ra.k_rot = c.k_cache; ra.k_rows = cap; ra.v_copy = c.v_cache; ra.v_rows = cap;
      ra.k_row0 = ra.v_row0 = c.pos0;
      aa.k_rot = c.k_cache; aa.k_rows = cap; aa.v = c.v_cache; aa.v_rows = cap; aa.q_pos0 = c.pos0;
      TRY_E(hymba::launch_rope_prefill(ra, attn_stream, tm(3)));
      TRY_E(after_rope());
    } else {
      // assembly row r: position r below n_meta, then a0 + (r - n_meta); the
      // attention runs on assembly rows as positions (the window rule depends on
      // position differences only, and every key was rotated at its true position)
      const int a0 = std::max(M, c.pos0 - W + 1), nw = c.pos0 - a0;
      const int R = ws.asm_rows;
      void* asm_k = wsb + ws.asm_k;
      void* asm_v = wsb + ws.asm_v;
      hymba::KvCopyArgs g = kc;   // ring -> assembly: meta rows, then positions a0 .. pos0 - 1
      g.src = kc.dst;
      g.dst.k = asm_k; g.dst.v = asm_v; g.dst.k_rows = g.dst.v_rows = R; g.dst.mode = hymba::KvSide::kIndex;
      g.dst.base = 0;
      g.na = M; g.pa = 0; g.pb = a0; g.n = M + nw;
      TRY_E(hymba::launch_kv_copy(g, attn_stream));
      ra.k_rot = asm_k; ra.k_rows = R; ra.v_copy = asm_v; ra.v_rows = R;
      ra.k_row0 = ra.v_row0 = M + nw;
      aa.k_rot = asm_k; aa.k_rows = R; aa.v = asm_v; aa.v_rows = R; aa.q_pos0 = M + nw;
      TRY_E(hymba::launch_rope_prefill(ra, attn_stream, tm(3)));
      TRY_E(after_rope());
      // the new rows that stay: the last `window` positions (after the gather above)
      kc.src.k = asm_k; kc.src.v = asm_v; kc.src.k_rows = kc.src.v_rows = R;
      kc.src.mode = hymba::KvSide::kLinear; kc.src.base = c.pos0 - (M + nw);
      kc.pb = std::max(c.pos0, c.pos0 + L - W); kc.na = 0; kc.pa = 0;
      kc.n = c.pos0 + L - kc.pb;
    }
    TRY_E(hymba::launch_kv_copy(kc, attn_stream));
    TRY_E(hymba::launch_attn_prefill(aa, attn_stream, tm(4)));
    return hipSuccess;
  };
  // Concurrent branches: with a late fork the attention branch runs on
  // `stream` and forks the Mamba branch after its RoPE pass; otherwise the
  // Mamba branch runs on `stream`, starting at once, and the attention branch
  // forks onto the second stream. With stage events, the order of the stage
  // list on `stream`.
  if (fc && late) {
    HYMBA_TRY(attention_branch());
  } else if (fc) {
    HYMBA_TRY(fork_point());
    HYMBA_TRY(mamba_branch());
    HYMBA_TRY(attention_branch());
    HYMBA_TRY(hipEventRecord(fc->join, fc->aux));
  } else {
    HYMBA_TRY(mamba_branch());
    HYMBA_TRY(attention_branch());
  }
  if (fc) HYMBA_TRY(hipStreamWaitEvent(stream, fc->join, 0));

  int n_cu = 0;
  HYMBA_TRY(device_cus(&n_cu));
  HYMBA_TRY(hymba::launch_fuse(y_attn, y_ssm, params->beta_attn, params->beta_ssm, (int64_t)desc->batch * L,
                               desc->d_inner, desc->norm_eps, desc->act, c.out, stream, tm(5), n_cu));
  return HYMBA_OK;
}

int check_prefill_io(const void* const* req, int n_req, const void* const* opt, int n_opt) {
  for (int i = 0; i < n_req; ++i)
    if (!req[i]) return HYMBA_EINVAL;
  for (int i = 0; i < n_req; ++i)
    if (!aligned16(req[i])) return HYMBA_EALIGN;
  for (int i = 0; i < n_opt; ++i)
    if (opt[i] && !aligned16(opt[i])) return HYMBA_EALIGN;
  return HYMBA_OK;
}

}  // namespace

extern "C" {

int hymba_mixer_prefill(const hymba_mixer_desc* desc, const hymba_mixer_params* params, const void* x,
                        const void* z, const void* dt, const void* B, const void* C, const void* q, const void* k,
                        const void* v, void* out, float* ssm_state_out, void* conv_state_out, void* k_cache,
                        void* v_cache, void* y_attn_out, void* y_ssm_out, void* workspace,
                        size_t workspace_bytes, hipEvent_t* stage_events, hipStream_t stream) {
  int st = check_desc(desc, false);
  if (st != HYMBA_OK) return st;
  st = check_params(params);
  if (st != HYMBA_OK) return st;
  const void* req[] = {x, z, dt, B, C, q, k, v, out};
  const void* opt[] = {ssm_state_out, conv_state_out, k_cache, v_cache, y_attn_out, y_ssm_out};
  st = check_prefill_io(req, 9, opt, 6);
  if (st != HYMBA_OK) return st;
  if ((k_cache == nullptr) != (v_cache == nullptr)) return HYMBA_EINVAL;
  const int L = desc->n_meta + desc->n_tokens;
  if (k_cache && !desc->cache_ring && desc->cache_capacity < L) return HYMBA_EINVAL;
  PrefillCall c = {};
  c.x = x; c.z = z; c.dt = dt; c.B = B; c.C = C; c.q = q; c.k = k; c.v = v; c.out = out;
  c.pos0 = 0; c.cont = false;
  c.state_out = ssm_state_out; c.conv_out = conv_state_out;
  c.k_cache = k_cache; c.v_cache = v_cache;
  c.y_attn_out = y_attn_out; c.y_ssm_out = y_ssm_out;
  c.workspace = workspace; c.workspace_bytes = workspace_bytes; c.stage_events = stage_events;
  return prefill_impl(desc, params, c, stream);
}

int hymba_mixer_prefill_continue(const hymba_mixer_desc* desc, const hymba_mixer_params* params, int32_t pos0,
                                 const void* x, const void* z, const void* dt, const void* B, const void* C,
                                 const void* q, const void* k, const void* v, void* out, float* ssm_state,
                                 void* conv_state, void* k_cache, void* v_cache, void* y_attn_out, void* y_ssm_out,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_desc(desc, false);
  if (st != HYMBA_OK) return st;
  st = check_params(params);
  if (st != HYMBA_OK) return st;
  const void* req[] = {x, z, dt, B, C, q, k, v, out, ssm_state, conv_state, k_cache, v_cache};
  const void* opt[] = {y_attn_out, y_ssm_out};
  st = check_prefill_io(req, 13, opt, 2);
  if (st != HYMBA_OK) return st;
  const int T = desc->n_tokens;
  if (T < 1 || pos0 < desc->n_meta || (int64_t)pos0 + T > INT32_MAX / 2) return HYMBA_EINVAL;
  // rows the attention addresses with 32-bit byte offsets: positions below
  // pos0 + T in the cache, or the assembly of the compact form
  const int64_t key_rows = desc->cache_ring ? (int64_t)prefill_ws(desc).asm_rows : (int64_t)pos0 + T;
  if (!desc->cache_ring && desc->cache_capacity < (int64_t)pos0 + T) return HYMBA_EINVAL;
  if (key_rows * kv_row_bytes(desc) > INT32_MAX) return HYMBA_EUNSUPPORTED;
  PrefillCall c = {};
  c.x = x; c.z = z; c.dt = dt; c.B = B; c.C = C; c.q = q; c.k = k; c.v = v; c.out = out;
  c.pos0 = pos0; c.cont = true;
  c.state_in = ssm_state; c.conv_in = conv_state;
  c.state_out = ssm_state; c.conv_out = conv_state;
  c.k_cache = k_cache; c.v_cache = v_cache;
  c.y_attn_out = y_attn_out; c.y_ssm_out = y_ssm_out;
  c.workspace = workspace; c.workspace_bytes = workspace_bytes; c.stage_events = nullptr;
  return prefill_impl(desc, params, c, stream);
}

}  // extern "C"

namespace {

struct DecodeCall {
  const void *x, *z, *dt, *B, *C, *q, *k_new, *v_new, *k_cache, *v_cache;
  const int32_t* cache_len;
  float* ssm_state;
  void *conv_state, *out, *y_attn_out, *y_ssm_out;
};

int check_decode_io(const DecodeCall& c) {
  const void* req[] = {c.x, c.z, c.dt, c.B, c.C, c.q, c.k_new, c.v_new, c.k_cache, c.v_cache, c.cache_len,
                       c.ssm_state, c.conv_state, c.out};
  for (const void* p : req)
    if (!p) return HYMBA_EINVAL;
  for (const void* p : req)
    if (!aligned16(p)) return HYMBA_EALIGN;
  if ((c.y_attn_out && !aligned16(c.y_attn_out)) || (c.y_ssm_out && !aligned16(c.y_ssm_out))) return HYMBA_EALIGN;
  return HYMBA_OK;
}

// splits (partials per query head) a decode launch on this device uses
hipError_t decode_splits(const hymba_mixer_desc* d, int* n_split) {
  hymba::AttnDecodeArgs aa = {};
  aa.batch = d->batch; aa.cap = d->cache_capacity; aa.n_meta = d->n_meta; aa.window = d->window;
  aa.n_q_heads = d->n_q_heads; aa.n_kv_heads = d->n_kv_heads; aa.head_dim_v = d->head_dim_v; aa.act = d->act;
  hipError_t e = device_cus(&aa.n_cu);
  if (e != hipSuccess) return e;
  *n_split = hymba::decode_active_splits(aa);
  return hipSuccess;
}

// The decode step on validated arguments, with its scratch at wsb laid out as
// ws (room for at least n_split partial slots).
int decode_impl(const hymba_mixer_desc* desc, const hymba_mixer_params* params, const DecodeCall& c, char* wsb,
                const DecodeWs& ws, int n_split, hipEvent_t* stage_events, hipStream_t stream) {
  float* partial = (float*)(wsb + ws.partial);
  void* y_ssm = c.y_ssm_out ? c.y_ssm_out : (void*)(wsb + ws.y_ssm);
  void* y_attn = c.y_attn_out ? c.y_attn_out : (void*)(wsb + ws.y_attn);

  auto tm = [&](int i) -> hymba::Timing {
    hymba::Timing t;
    if (stage_events) {
      t.start = stage_events[2 * i];
      t.stop = stage_events[2 * i + 1];
    }
    return t;
  };
  // One stream. In bf16 the Mamba step runs inside the attention launch, as
  // workgroups of its own (its stage records its events back to back): the
  // step's state traffic then overlaps the cache stream, where a launch of
  // its own ran before the attention, and a fork/join across two streams
  // measured ~10 µs slower per call than running the kernels in order.
  hymba::SsmDecodeArgs sa;
  sa.x = c.x; sa.z = c.z; sa.dt = c.dt; sa.B = c.B; sa.C = c.C;
  sa.A = params->A; sa.D = params->D; sa.conv_w = params->conv_w;
  sa.state = c.ssm_state; sa.conv_state = c.conv_state; sa.y = y_ssm;
  sa.batch = desc->batch; sa.d_inner = desc->d_inner; sa.act = desc->act;
  sa.head_width = desc->ssm_heads > 0 ? desc->d_inner / desc->ssm_heads : 0;
  const bool fused = desc->act == HYMBA_BF16;
  if (fused)
    HYMBA_TRY(hymba::no_kernel(stream, tm(0)));
  else
    HYMBA_TRY(hymba::launch_ssm_decode(sa, stream, tm(0)));

  hymba::AttnDecodeArgs aa;
  aa.q = c.q; aa.k_new = c.k_new; aa.v_new = c.v_new; aa.k_cache = c.k_cache; aa.v_cache = c.v_cache;
  aa.cache_len = c.cache_len; aa.partial = partial; aa.k_scale = params->k_scale;
  aa.q_rot = (float*)(wsb + ws.q_rot); aa.k_rot = (float*)(wsb + ws.k_rot);
  aa.n_split = n_split; aa.keys_per_split = ws.keys_per_split;
  aa.batch = desc->batch; aa.cap = desc->cache_capacity; aa.n_meta = desc->n_meta; aa.window = desc->window;
  aa.n_q_heads = desc->n_q_heads; aa.n_kv_heads = desc->n_kv_heads; aa.head_dim_v = desc->head_dim_v;
  aa.rope_base = desc->rope_base; aa.act = desc->act; aa.ring = desc->cache_ring;
  aa.ssm = fused ? &sa : nullptr;
  HYMBA_TRY(device_cus(&aa.n_cu));
  HYMBA_TRY(hymba::launch_attn_decode(aa, stream, tm(1)));

  hymba::DecodeCombineArgs ca;
  ca.partial = partial; ca.y_ssm = y_ssm; ca.beta_attn = params->beta_attn; ca.beta_ssm = params->beta_ssm;
  ca.eps = desc->norm_eps; ca.y_attn = y_attn; ca.out = c.out;
  ca.n_split = n_split; ca.batch = desc->batch; ca.n_q_heads = desc->n_q_heads;
  ca.head_dim_v = desc->head_dim_v; ca.act = desc->act;
  HYMBA_TRY(hymba::launch_decode_combine(ca, stream, tm(2)));
  return HYMBA_OK;
}

// Library-owned scratch of the allocation-free decode entry point: one copy
// per device, held until the process ends. Host code never passes the
// array's name to a kernel (on the host it is only a stand-in); it uses the
// device address hipGetSymbolAddress gives for the current device.
constexpr size_t kDecodeScratchBytes = (size_t)HYMBA_DECODE_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// The device address of `scratch` on the current device, looked up with that
// device current the first time it is needed there.
hipError_t scratch_on_device(char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = (char*)p;
  return hipSuccess;
}

}  // namespace

extern "C" {

int hymba_mixer_decode(const hymba_mixer_desc* desc, const hymba_mixer_params* params, const void* x,
                       const void* z, const void* dt, const void* B, const void* C, const void* q,
                       const void* k_new, const void* v_new, const void* k_cache, const void* v_cache,
                       const int32_t* cache_len, float* ssm_state, void* conv_state, void* out, void* y_attn_out,
                       void* y_ssm_out, void* workspace, size_t workspace_bytes, hipEvent_t* stage_events,
                       hipStream_t stream) {
  int st = check_desc(desc, true);
  if (st != HYMBA_OK) return st;
  st = check_params(params);
  if (st != HYMBA_OK) return st;
  const DecodeCall c = {x, z, dt, B, C, q, k_new, v_new, k_cache, v_cache, cache_len, ssm_state, conv_state,
                        out, y_attn_out, y_ssm_out};
  st = check_decode_io(c);
  if (st != HYMBA_OK) return st;
  const DecodeWs ws = decode_ws(desc);
  if (!workspace || workspace_bytes < ws.total) return HYMBA_EWORKSPACE;
  if (((uintptr_t)workspace & 255u) != 0) return HYMBA_EALIGN;
  int n_split = 0;
  HYMBA_TRY(decode_splits(desc, &n_split));   // <= ws.n_split partial slots
  return decode_impl(desc, params, c, (char*)workspace, ws, n_split, stage_events, stream);
}

int hymba_mixer_decode_noalloc(const hymba_mixer_desc* desc, const hymba_mixer_params* params, const void* x,
                               const void* z, const void* dt, const void* B, const void* C, const void* q,
                               const void* k_new, const void* v_new, const void* k_cache, const void* v_cache,
                               const int32_t* cache_len, float* ssm_state, void* conv_state, void* out,
                               void* y_attn_out, void* y_ssm_out, hipStream_t stream) {
  int st = check_desc(desc, true);
  if (st != HYMBA_OK) return st;
  st = check_params(params);
  if (st != HYMBA_OK) return st;
  const DecodeCall c = {x, z, dt, B, C, q, k_new, v_new, k_cache, v_cache, cache_len, ssm_state, conv_state,
                        out, y_attn_out, y_ssm_out};
  st = check_decode_io(c);
  if (st != HYMBA_OK) return st;
  int n_split = 0;
  HYMBA_TRY(decode_splits(desc, &n_split));
  const DecodeWs ws = decode_ws(desc, n_split);   // exactly the splits this launch uses
  if (ws.total > kDecodeScratchBytes) return HYMBA_EWORKSPACE;
  char* wsb = nullptr;
  HYMBA_TRY(scratch_on_device(&wsb));
  return decode_impl(desc, params, c, wsb, ws, n_split, nullptr, stream);
}

int hymba_fuse_heads(const void* y_attn, const void* y_ssm, const float* beta_attn, const float* beta_ssm,
                     int64_t n_rows, int32_t width, float eps, hymba_dtype act, void* out, hipStream_t stream) {
  if (act != HYMBA_F32 && act != HYMBA_BF16) return HYMBA_EINVAL;
  if (n_rows < 0 || width < 1 || !(eps >= 0.f)) return HYMBA_EINVAL;
  if (n_rows == 0) return HYMBA_OK;  // nothing to do (empty tensors may carry null pointers)
  if (!y_attn || !y_ssm || !beta_attn || !beta_ssm || !out) return HYMBA_EINVAL;
  if (!aligned16(y_attn) || !aligned16(y_ssm) || !aligned16(beta_attn) || !aligned16(beta_ssm) || !aligned16(out))
    return HYMBA_EALIGN;
  int n_cu = 0;
  HYMBA_TRY(device_cus(&n_cu));
  return hip_status(hymba::launch_fuse(y_attn, y_ssm, beta_attn, beta_ssm, n_rows, width, eps, act, out, stream, {},
                                       n_cu));
}

int hymba_debug_mask_ranges(const hymba_mixer_desc* desc, int32_t* ranges, hipStream_t stream) {
  if (!desc || !ranges) return HYMBA_EINVAL;
  if (desc->n_meta < 0 || desc->n_tokens < 0 || (int64_t)desc->n_meta + desc->n_tokens > INT32_MAX / 2)
    return HYMBA_EINVAL;
  if (!aligned16(ranges)) return HYMBA_EALIGN;
  return hip_status(hymba::launch_mask_ranges(desc->n_meta + desc->n_tokens, desc->n_meta, desc->window, ranges,
                                              stream));
}

int hymba_debug_prefill_visibility(const hymba_mixer_desc* desc, int32_t pos0, int32_t* out, hipStream_t stream) {
  int st = check_desc(desc, false);
  if (st != HYMBA_OK) return st;
  if (!out) return HYMBA_EINVAL;
  if (!aligned16(out)) return HYMBA_EALIGN;
  if (pos0 < 0 || (pos0 > 0 && (desc->n_tokens < 1 || pos0 < desc->n_meta)) ||
      (int64_t)pos0 + desc->n_tokens > INT32_MAX / 2)
    return HYMBA_EINVAL;
  const int Lq = pos0 > 0 ? desc->n_tokens : desc->n_meta + desc->n_tokens;
  int n_cu = 0;
  HYMBA_TRY(device_cus(&n_cu));
  return hip_status(hymba::launch_prefill_visibility(desc->batch, Lq, pos0, desc->n_meta, desc->window, desc->n_q_heads,
                                                     desc->n_kv_heads, n_cu, out, stream));
}

const char* hymba_status_string(int status) {
  switch (status) {
    case HYMBA_OK: return "ok";
    case HYMBA_EINVAL: return "invalid argument";
    case HYMBA_EUNSUPPORTED: return "unsupported geometry";
    case HYMBA_EALIGN: return "pointer not 16-byte aligned (workspace: 256-byte)";
    case HYMBA_EHIP: return "HIP runtime error";
    case HYMBA_EWORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
  }
}

int hymba_last_hip_error(void) { return g_last_hip_error; }

int hymba_abi_version(void) { return HYMBA_ABI_VERSION; }

}  // extern "C"
