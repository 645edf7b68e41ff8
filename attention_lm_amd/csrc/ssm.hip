// Mamba branch: causal depthwise conv (4 taps) + selective scan (d_state 16)
// + D skip + silu(z) gate, for prefill (whole sequences) and decode (one row).
//
// Recurrence ("Jamba: Hybrid SSM-Transformer", "1. Layer Interleaving Ratio";
// "Lecture 04 - Beyond the Dense Transformer", section 2):
//   h_t = exp(dt_t A) (.) h_{t-1} + (dt_t B_t) u_t,   y_t = C_t . h_t + D u_t.
//
// Prefill design: the sequence is cut into chunks of CT rows and every
// (sequence, 128-channel block, chunk) is a workgroup, one lane per channel
// with its 16 states in registers, so even a single sequence fills the chip.
//   1. chunk_end:   each chunk (except the last) is scanned from a zero state;
//                   its end state a_k and the sum of its dt, S_k, go to the
//                   workspace.
//   2. chunk_carry: one thread per (sequence, channel, state) chains the chunks:
//                   H_{k+1} = exp(A S_k) H_k + a_k (the decay over a chunk is
//                   exp(A times its total dt)), giving every chunk's carry-in H_k.
//   3. chunk_out:   each chunk is scanned again from its carry-in, forming
//                   y_t = C_t . h_t + D u_t, gated by silu(z_t); the last chunk
//                   also writes the final state and the conv history.
// The conv history of a chunk is re-read from x (3 rows before it).
#include "common.hpp"
#include "launch.hpp"
#include "ssm_step.hpp"

namespace hymba {

namespace {

template <int N>
__device__ __forceinline__ void load_n(const bf16* p, float* o) {
  if constexpr (N % 8 == 0) {
#pragma unroll
    for (int k = 0; k < N / 8; ++k) load16(p + 8 * k, o + 8 * k);
  } else if constexpr (N == 4) {
    uint2 v = *reinterpret_cast<const uint2*>(p);
    o[0] = bf16_lo(v.x); o[1] = bf16_hi(v.x); o[2] = bf16_lo(v.y); o[3] = bf16_hi(v.y);
  } else if constexpr (N == 2) {
    uint32_t v = *reinterpret_cast<const uint32_t*>(p);
    o[0] = bf16_lo(v); o[1] = bf16_hi(v);
  } else {
#pragma unroll
    for (int k = 0; k < N; ++k) o[k] = to_f32(p[k]);
  }
}
template <int N>
__device__ __forceinline__ void load_n(const float* p, float* o) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int k = 0; k < N / 4; ++k) load16(p + 4 * k, o + 4 * k);
  } else if constexpr (N == 2) {
    float2 v = *reinterpret_cast<const float2*>(p);
    o[0] = v.x; o[1] = v.y;
  } else {
#pragma unroll
    for (int k = 0; k < N; ++k) o[k] = p[k];
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// silu(z) = z / (1 + e^{-z})
__device__ __forceinline__ float silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + fast_exp2(-z * kLog2e));
}

constexpr int kStates = 16;
constexpr int kConv = 4;

constexpr int kChanPerBlock = 128;   // one lane per channel
constexpr int kRowBlock = 8;         // rows staged in LDS per step

// Row t of B or C (16 values, the same for every channel) as raw 32-bit words:
// a uniform address, so the compiler reads it with scalar loads into SGPRs and
// the VALU takes the values as scalar operands (no LDS broadcast traffic).
template <typename T> struct RowWords { static constexpr int n = kStates * (int)sizeof(T) / 4; };
template <typename T>
__device__ __forceinline__ void load_words(const T* __restrict__ p, uint32_t* w) {
#pragma unroll
  for (int j = 0; j < RowWords<T>::n; ++j) w[j] = reinterpret_cast<const uint32_t*>(p)[j];
}
__device__ __forceinline__ float word_val(const uint32_t* w, int n, bf16*) {
  return (n & 1) ? bf16_hi(w[n >> 1]) : bf16_lo(w[n >> 1]);
}
__device__ __forceinline__ float word_val(const uint32_t* w, int n, float*) { return __uint_as_float(w[n]); }

// One pass of the chunked scan over rows [t0, t1) of 128 channels.
//  OUT = false: start from zero, write the chunk's end state and dt sum.
//  OUT = true:  start from the chunk's carry-in, write gated y (and, for the
//               last chunk, the final SSM state and conv history).
// The per-channel inputs (x with its conv history, dt, z) are staged through
// LDS in blocks of kRowBlock rows, double-buffered: the global loads of block
// i+1 are in flight while block i is scanned.
template <typename T, bool OUT>
__global__ __launch_bounds__(kChanPerBlock) void ssm_chunk_kernel(
    const T* __restrict__ x, const T* __restrict__ z, const T* __restrict__ dt, const T* __restrict__ Bm,
    const T* __restrict__ Cm, const float* __restrict__ A, const float* __restrict__ Dp,
    const float* __restrict__ conv_w, const T* __restrict__ conv_in, const float* __restrict__ carry,
    float* __restrict__ agg, float* __restrict__ sdt, T* __restrict__ y, float* __restrict__ state_out,
    T* __restrict__ conv_state_out, int L, int Dch, int CT) {
  constexpr int E = Vec16<T>::n;                  // elements per 16-byte vector
  constexpr int RV = kChanPerBlock / E;           // vectors per 128-channel row
  constexpr int XR = kRowBlock + kConv - 1;       // x rows per block (with conv history)
  constexpr int NX = (XR * RV + kChanPerBlock - 1) / kChanPerBlock;
  constexpr int XRP = NX * kChanPerBlock / RV;    // x rows staged: XR, padded so every thread has NX items
  constexpr int NR = kRowBlock * RV / kChanPerBlock;
  static_assert(NX * kChanPerBlock % RV == 0 && kRowBlock * RV % kChanPerBlock == 0, "staging shape");
  // one stage: a block is copied to registers before the next one is loaded
  __shared__ __attribute__((aligned(16))) T xs[XRP][kChanPerBlock];
  __shared__ __attribute__((aligned(16))) T ds[kRowBlock][kChanPerBlock];
  __shared__ __attribute__((aligned(16))) T zs[OUT ? kRowBlock : 1][kChanPerBlock];

  const int tid = threadIdx.x;
  const int c0 = blockIdx.x * kChanPerBlock;
  const int c = c0 + tid;
  const int k = blockIdx.y;
  const int b = blockIdx.z;
  const int batch = gridDim.z;
  const int nchunk = gridDim.y;
  const bool cv = c < Dch;
  const int cc = cv ? c : Dch - 1;
  const int64_t seq = (int64_t)b * L;
  const int t0 = k * CT, t1 = min(t0 + CT, L);

  // Block staging: buffer loads that write LDS directly (16 bytes per lane,
  // lanes contiguous), so no staging registers. x rows outside [0, L) and
  // dt/z rows outside [0, t1) read as zeros (dt = 0 leaves the state as is).
  // Item it = (row it / RV, 16-byte vector it % RV) lands at byte 16 it of the
  // stage, which is exactly the [row][channel] layout.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t row_b = (uint32_t)(Dch * sizeof(T));
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(x + seq * Dch, (uint32_t)L * row_b);
  const __amdgpu_buffer_rsrc_t drs = make_rsrc(dt + seq * Dch, (uint32_t)t1 * row_b);
  const __amdgpu_buffer_rsrc_t zrs = make_rsrc(z + seq * Dch, (uint32_t)t1 * row_b);
  auto fetch = [&](int tb) {
#pragma unroll
    for (int r = 0; r < NX; ++r) {
      const int it = tid + r * kChanPerBlock, row = it / RV, v = it % RV, t = tb - (kConv - 1) + row;
      const int it0 = 64 * wave + r * kChanPerBlock;   // first item of this wave's load
      buf_load16_lds(xrs, (uint32_t)t * row_b + (uint32_t)((c0 + v * E) * sizeof(T)), &xs[0][0] + it0 * E);
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int it = tid + r * kChanPerBlock, row = it / RV, v = it % RV, t = tb + row;
      const int it0 = 64 * wave + r * kChanPerBlock;
      const uint32_t off = (uint32_t)t * row_b + (uint32_t)((c0 + v * E) * sizeof(T));
      buf_load16_lds(drs, off, &ds[0][0] + it0 * E);
      if constexpr (OUT) buf_load16_lds(zrs, off, &zs[0][0] + it0 * E);
    }
  };

  float A2[kStates], w[kConv], h[kStates];
#pragma unroll
  for (int n = 0; n < kStates; ++n) A2[n] = A[(int64_t)cc * kStates + n] * kLog2e;
#pragma unroll
  for (int j = 0; j < kConv; ++j) w[j] = conv_w[(int64_t)cc * kConv + j];
  float Dc = 0.f;
  if constexpr (OUT) {
    Dc = Dp[cc];
    const float4* cp = reinterpret_cast<const float4*>(carry + (((int64_t)k * batch + b) * Dch + cc) * kStates);
#pragma unroll
    for (int q = 0; q < kStates / 4; ++q) {
      const float4 v4 = cp[q];
      h[4 * q] = v4.x; h[4 * q + 1] = v4.y; h[4 * q + 2] = v4.z; h[4 * q + 3] = v4.w;
    }
  } else {
#pragma unroll
    for (int n = 0; n < kStates; ++n) h[n] = 0.f;
  }
  float S = 0.f;
  const T* Bseq = Bm + seq * kStates;
  const T* Cseq = Cm + seq * kStates;
  // y of this sequence through a buffer descriptor that ends at row t1: stores
  // of rows past the chunk and of lanes without a channel are dropped, so the
  // row loop has no branches
  const __amdgpu_buffer_rsrc_t yrs = make_rsrc(y + seq * Dch, (uint32_t)((int64_t)t1 * Dch * sizeof(T)));
  const uint32_t ylane = cv ? (uint32_t)(c * sizeof(T)) : kBufferNowhere;
  constexpr int RW = RowWords<T>::n;

  const int nblk = (t1 - t0 + kRowBlock - 1) / kRowBlock;
  fetch(t0);
  __syncthreads();
  if (conv_in && t0 == 0) {   // rows -3 .. -1: the carried conv history (oldest first)
#pragma unroll
    for (int r = 0; r < kConv - 1; ++r) xs[r][tid] = conv_in[((int64_t)b * Dch + cc) * (kConv - 1) + r];
    __syncthreads();
  }
  for (int ib = 0; ib < nblk; ++ib) {
    const int tb = t0 + ib * kRowBlock;
    // this block's per-channel inputs, LDS -> registers, before any scalar
    // load is in flight (scalar loads return out of order, so a wait for an
    // LDS read behind one would also wait for it)
    float xr[XR], dr[kRowBlock], zr[OUT ? kRowBlock : 1];
#pragma unroll
    for (int i = 0; i < XR; ++i) xr[i] = to_f32(xs[i][tid]);
#pragma unroll
    for (int i = 0; i < kRowBlock; ++i) {
      dr[i] = to_f32(ds[i][tid]);
      if constexpr (OUT) zr[i] = to_f32(zs[i][tid]);
    }
    __syncthreads();   // every wave has its copy: the stage is free
    // the next block (past the chunk on the last one: then all dt are zero and
    // it is never used), loading while this one is scanned; no branches
    fetch(tb + kRowBlock);
    // B/C rows one ahead of their use; staged rows at or past t1 hold dt = 0
    // (state unchanged, y not stored) and read the B/C row t1 - 1
    uint32_t bw[RW], cw[OUT ? RW : 1];
    load_words(Bseq + (int64_t)min(tb, t1 - 1) * kStates, bw);
    if constexpr (OUT) load_words(Cseq + (int64_t)min(tb, t1 - 1) * kStates, cw);
#pragma unroll
    for (int i = 0; i < kRowBlock; ++i) {
      // keep the scalar prefetch exactly one row ahead (SGPR pressure)
      __builtin_amdgcn_sched_barrier(0);
      uint32_t bn[RW], cn[OUT ? RW : 1];
      if (i + 1 < kRowBlock) {
        const int tn = min(tb + i + 1, t1 - 1);
        load_words(Bseq + (int64_t)tn * kStates, bn);
        if constexpr (OUT) load_words(Cseq + (int64_t)tn * kStates, cn);
      }
      const float u = fmaf(w[0], xr[i], fmaf(w[1], xr[i + 1], fmaf(w[2], xr[i + 2], w[3] * xr[i + 3])));
      const float d = dr[i];
      const float du = d * u;
      if constexpr (OUT) {
        float acc = Dc * u;
#pragma unroll
        for (int n = 0; n < kStates; ++n) {
          h[n] = fmaf(fast_exp2(d * A2[n]), h[n], du * word_val(bw, n, (T*)nullptr));
          acc = fmaf(word_val(cw, n, (T*)nullptr), h[n], acc);
        }
        buf_store(yrs, (uint32_t)((tb + i) * Dch * (int)sizeof(T)) + ylane, from_f32<T>(acc * silu(zr[i])));
      } else {
#pragma unroll
        for (int n = 0; n < kStates; ++n) h[n] = fmaf(fast_exp2(d * A2[n]), h[n], du * word_val(bw, n, (T*)nullptr));
        S += d;
      }
      if (i + 1 < kRowBlock) {
#pragma unroll
        for (int j = 0; j < RW; ++j) {
          bw[j] = bn[j];
          if constexpr (OUT) cw[j] = cn[j];
        }
      }
    }
    __syncthreads();   // (waits for the stage loads first)
  }

  if (!cv) return;
  if constexpr (!OUT) {
    const int64_t o = (((int64_t)k * batch + b) * Dch + c);
    float4* ap = reinterpret_cast<float4*>(agg + o * kStates);
#pragma unroll
    for (int q = 0; q < kStates / 4; ++q) ap[q] = make_float4(h[4 * q], h[4 * q + 1], h[4 * q + 2], h[4 * q + 3]);
    sdt[o] = S;
  } else if (k == nchunk - 1) {
    if (state_out) {
      float4* sp = reinterpret_cast<float4*>(state_out + ((int64_t)b * Dch + c) * kStates);
#pragma unroll
      for (int q = 0; q < kStates / 4; ++q) sp[q] = make_float4(h[4 * q], h[4 * q + 1], h[4 * q + 2], h[4 * q + 3]);
    }
    if (conv_state_out) {   // raw x of rows L-3, L-2, L-1 (before row 0: the carried history, or zero)
      T* csp = conv_state_out + ((int64_t)b * Dch + c) * (kConv - 1);
#pragma unroll
      for (int j = 0; j < kConv - 1; ++j) {
        const int t = L - (kConv - 1) + j;
        csp[j] = t >= 0  ? x[(seq + t) * Dch + c]
                 : conv_in ? conv_in[((int64_t)b * Dch + c) * (kConv - 1) + (kConv - 1) + t]
                           : from_f32<T>(0.f);
      }
    }
  }
}

// carry[k] = state entering chunk k, from the chunk end states agg[k] (zero
// start) and the chunk dt sums sdt[k]: carry[0] = 0 and
// carry[k+1] = exp(A sdt[k]) carry[k] + agg[k]. These affine steps compose
// associatively, so each (sequence, channel, state) chain is cut into
// kCarrySegs segments, one per wave of a workgroup of 64 chains. Each wave
// composes its segment from a zero start (end state and summed dt), the waves
// swap those through LDS, and each wave walks its segment again from its true
// start, storing every carry. That is eight times the waves of one walk per
// chain (the chain is latency-bound: few dependent steps, all memory); the
// second walk reuses the loaded values when a segment fits in one batch.
// Eight segments of up to 12 steps measured faster than four of 24 (SWA
// layer 10.4 -> 9.6 us, batched Mamba-2 workload 104 -> 89 us) and than
// sixteen of 6 (10.3 / 122 us).
constexpr int kCarrySegs = 8;
constexpr int kCarryBatch = 12;
__global__ __launch_bounds__(64 * kCarrySegs) void ssm_chunk_carry_kernel(const float* __restrict__ A,
                                                                         const float* __restrict__ agg,
                                                                         const float* __restrict__ sdt,
                                                                         const float* __restrict__ state_in,
                                                                         float* __restrict__ carry, int nchunk,
                                                                         int batch, int Dch, int head_width) {
  constexpr int KB = kCarryBatch;
  __shared__ float seg_h[kCarrySegs][64], seg_s[kCarrySegs][64];
  const int lane = threadIdx.x & 63;
  const int seg = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t per = (int64_t)batch * Dch * kStates;
  const int64_t idx = (int64_t)blockIdx.x * 64 + lane;   // chain (b, c, n)
  const bool valid = idx < per;
  const int64_t ci = valid ? idx : per - 1;
  const int n = (int)(ci % kStates);
  const int64_t bc = ci / kStates;
  const int c = (int)(bc % Dch);
  const float a2 = (head_width > 0 ? A[c / head_width] : A[(int64_t)c * kStates + n]) * kLog2e;
  const int steps = nchunk - 1;   // chunks 0 .. nchunk-2 feed a later chunk
  const int seg_len = (steps + kCarrySegs - 1) / kCarrySegs;
  const int k0 = min(steps, seg * seg_len), k1 = min(steps, k0 + seg_len);
  const int nb = (k1 - k0 + KB - 1) / KB;
  // Views of this segment's chunks (agg, sdt from chunk k0, carry from k0 + 1)
  // sized to end with the segment: a step past it reads (agg 0, sdt 0), the
  // identity step, and stores nothing.
  const int64_t nseg = k1 - k0;
  const __amdgpu_buffer_rsrc_t ars = make_rsrc(agg + k0 * per, (uint32_t)(nseg * per * sizeof(float)));
  const __amdgpu_buffer_rsrc_t srs =
      make_rsrc(sdt + k0 * (per / kStates), (uint32_t)(nseg * (per / kStates) * sizeof(float)));
  const __amdgpu_buffer_rsrc_t crs = make_rsrc(carry + (k0 + 1) * per, (uint32_t)(nseg * per * sizeof(float)));
  const float h_in = state_in ? state_in[ci] : 0.f;   // the state entering chunk 0
  if (seg == 0 && valid) carry[idx] = h_in;
  auto load = [&](int kb, float* av, float* sv) {   // steps kb .. kb + KB - 1 of the segment
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      const int64_t k = kb + i;
      av[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ars, (uint32_t)((k * per + ci) * 4), 0, 0));
      sv[i] = __uint_as_float(
          __builtin_amdgcn_raw_buffer_load_b32(srs, (uint32_t)((k * (per / kStates) + bc) * 4), 0, 0));
    }
  };
  float av[KB], sv[KB], an[KB], sn[KB];
  // first walk: the segment's own end state H and dt sum S
  float H = 0.f, S = 0.f;
  load(0, av, sv);
  for (int j = 0; j < nb; ++j) {
    if (j + 1 < nb) load((j + 1) * KB, an, sn);
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      H = fmaf(fast_exp2(a2 * sv[i]), H, av[i]);
      S += sv[i];
    }
    if (j + 1 < nb) {
#pragma unroll
      for (int i = 0; i < KB; ++i) {
        av[i] = an[i];
        sv[i] = sn[i];
      }
    }
  }
  seg_h[seg][lane] = H;
  seg_s[seg][lane] = S;
  __syncthreads();
  // the state entering this segment: the earlier segments, in order
  float H0 = h_in;
  for (int s = 0; s < seg; ++s) H0 = fmaf(fast_exp2(a2 * seg_s[s][lane]), H0, seg_h[s][lane]);
  // second walk from the true start, storing carry[k + 1]
  H = H0;
  for (int j = 0; j < nb; ++j) {
    const int kb = j * KB;
    if (nb > 1) load(kb, av, sv);   // one batch: still in registers
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      H = fmaf(fast_exp2(a2 * sv[i]), H, av[i]);
      const int64_t k = kb + i;
      buf_store(crs, valid ? (uint32_t)((k * per + idx) * sizeof(float)) : kBufferNowhere, H);
    }
  }
}

// Wait until at most n of this wave's vector memory operations are
// outstanding (0 <= n; counts of 63 and more wait for nothing). s_waitcnt
// takes an immediate, so the count is dispatched to constant waits.
__device__ __forceinline__ void vm_wait_at_most(int n) {
#define HYMBA_VMW(k) \
  case k: __builtin_amdgcn_s_waitcnt(((k) & 15) | (((k) >> 4) << 14) | 0x0F70); break;
  switch (n) {
    HYMBA_VMW(0) HYMBA_VMW(1) HYMBA_VMW(2) HYMBA_VMW(3) HYMBA_VMW(4) HYMBA_VMW(5) HYMBA_VMW(6) HYMBA_VMW(7)
    HYMBA_VMW(8) HYMBA_VMW(9) HYMBA_VMW(10) HYMBA_VMW(11) HYMBA_VMW(12) HYMBA_VMW(13) HYMBA_VMW(14) HYMBA_VMW(15)
    default: break;
  }
#undef HYMBA_VMW
}

// ---------------------------------------------------------------------------
// Single-pass scan, for batches whose (sequence, channel) count alone fills
// the chip: one exp(dt A) per element instead of two, and no carry chain.
// Workgroup = 64 channels of one sequence x 16 states, 256 lanes: wave w holds
// the states 4w .. 4w + 3 and lane l the channel c0 + l, in registers for the
// whole sequence. Per block of kScanRows rows:
//   A. two (row, channel) items per lane (rows w and w + 4, channel l): the
//      conv output u, dt and dt u as fp32 in LDS (D u stays in the lane's
//      registers); the block's B and C rows as fp32, grouped by state quad;
//   B. every lane advances its four states over the block's rows and leaves
//      its part of C . h for each row in LDS;
//   C. the same two items per lane: y = the four parts + D u, times silu(z).
// Work that is per (row, channel) (conv, dt u, gate) is done once, not once
// per state, and each exp(dt A) is formed once. The next blocks' raw inputs
// load straight into LDS meanwhile. Four states per lane keep the register
// footprint per SIMD small enough (3 to 4 waves of 56 VGPRs on the batched
// workload) that a workgroup of the attention branch fits beside the scan's
// on every compute unit.
constexpr int kScanChan = 64;
constexpr int kScanRows = 8;
constexpr int kScanQuads = kStates / 4;   // one wave per state quad
constexpr int kScanStages = 3;            // staging ring: two blocks in flight ahead of the one in use
constexpr int kScanRowsLoaded = 1;        // rows of phase B whose LDS values are in registers at once
constexpr int kScanItems = kScanRows * kScanChan / 256;   // (row, channel) items per lane in phases A and C
static_assert(kScanQuads * 64 == 256 && kScanChan == 64 && kScanItems * kScanQuads == kScanRows,
              "wave = state quad = row offset, lane = channel");

template <typename T>
struct Scan1Stage {   // one block's inputs as loaded (16-byte pieces, row-major)
  T x[kScanRows + kConv - 1][kScanChan];   // rows tb - 3 .. tb + kScanRows - 1
  T dt[kScanRows][kScanChan];
  T z[kScanRows][kScanChan];
  T b[kScanRows][kStates];
  T c[kScanRows][kStates];
};

template <typename T>
__global__ __launch_bounds__(256) void ssm_scan1_kernel(
    const T* __restrict__ x, const T* __restrict__ z, const T* __restrict__ dt, const T* __restrict__ Bm,
    const T* __restrict__ Cm, const float* __restrict__ A, const float* __restrict__ Dp,
    const float* __restrict__ conv_w, const T* __restrict__ conv_in, const float* __restrict__ state_in,
    T* __restrict__ y, float* __restrict__ state_out, T* __restrict__ conv_state_out, int L, int Dch) {
  constexpr int E = Vec16<T>::n;                // elements per 16-byte piece
  constexpr int CP = kScanChan / E;             // pieces per 64-channel row
  constexpr int SP = kStates / E;               // pieces per B or C row
  constexpr int R = kScanRows;
  __shared__ __attribute__((aligned(16))) Scan1Stage<T> stage[kScanStages];
  __shared__ __attribute__((aligned(16))) float2 dd[R][kScanChan];             // (dt, dt u)
  __shared__ __attribute__((aligned(16))) float4 bcq[R][kScanQuads][2];        // B, then C, of a state quad
  __shared__ float part[R][kScanQuads][kScanChan];                             // each quad's share of C . h

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // B: state quad; A, C: rows wave, wave + 4
  // One 64-channel block of a bf16 row is one 128-byte line, so no two
  // workgroups share a line of x, dt, z or y.
  const int nblk_c = (Dch + kScanChan - 1) / kScanChan;
  const int id = (int)blockIdx.x;
  const int c0 = (id % nblk_c) * kScanChan;
  const int c = c0 + lane;
  const bool cv = c < Dch;
  const int cc = cv ? c : Dch - 1;
  const int64_t b = id / nblk_c;
  const int64_t seq = b * L;
  const uint32_t row_b = (uint32_t)(Dch * sizeof(T));
  // x over rows [0, L): a row index below 0 wraps past the end and reads zero
  // (zero conv history); dt and z past L read zero (dt = 0 leaves the state
  // as it is); y stores past L are dropped.
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(x + seq * Dch, (uint32_t)L * row_b);
  const __amdgpu_buffer_rsrc_t drs = make_rsrc(dt + seq * Dch, (uint32_t)L * row_b);
  const __amdgpu_buffer_rsrc_t zrs = make_rsrc(z + seq * Dch, (uint32_t)L * row_b);
  const __amdgpu_buffer_rsrc_t brs = make_rsrc(Bm + seq * kStates, (uint32_t)(L * kStates * sizeof(T)));
  const __amdgpu_buffer_rsrc_t crs = make_rsrc(Cm + seq * kStates, (uint32_t)(L * kStates * sizeof(T)));
  const __amdgpu_buffer_rsrc_t yrs = make_rsrc(y + seq * Dch, (uint32_t)L * row_b);
  const uint32_t col_b = (uint32_t)(c0 * sizeof(T));

  // One array of a block: n 16-byte pieces, piece i at LDS dst + 16 i, loaded
  // by one wave (lane i of each instruction writes dst + 16 (i0 + i)). A
  // piece's byte offset is its block-independent part (row within the block,
  // column), computed once per lane, plus the block's first row times the row
  // stride, one scalar per block; uint32 arithmetic, so the rows before 0 wrap
  // past the end of the descriptor and read zero.
  constexpr int NXP = (R + kConv - 1) * CP, NDP = R * CP, NBP = R * SP;
  constexpr int NXI = (NXP + 63) / 64;   // load instructions for x
  constexpr int NDI = (NDP + 63) / 64;   // ... for dt, and for z
  static_assert(NBP <= 64, "B and C pieces fit one instruction each");
  uint32_t xo[NXI], dzo[NDI];
#pragma unroll
  for (int k = 0; k < NXI; ++k) {
    const int it = 64 * k + lane;
    xo[k] = (uint32_t)(it / CP) * row_b + col_b + (uint32_t)(16 * (it % CP));
  }
#pragma unroll
  for (int k = 0; k < NDI; ++k) {
    const int it = 64 * k + lane;
    dzo[k] = (uint32_t)(it / CP) * row_b + col_b + (uint32_t)(16 * (it % CP));
  }
  const uint32_t bco = (uint32_t)(16 * lane);
  auto fetch = [&](int tb, Scan1Stage<T>& s) {
    if (wave == 0) {
      const uint32_t base = (uint32_t)(tb - (kConv - 1)) * row_b;
#pragma unroll
      for (int k = 0; k < NXI; ++k)
        if (64 * k + lane < NXP) buf_load16_lds(xrs, xo[k] + base, (char*)&s.x[0][0] + 16 * 64 * k);
    } else if (wave < 3) {
      const uint32_t base = (uint32_t)tb * row_b;
#pragma unroll
      for (int k = 0; k < NDI; ++k)
        if (64 * k + lane < NDP)
          buf_load16_lds(wave == 1 ? drs : zrs, dzo[k] + base,
                         (wave == 1 ? (char*)&s.dt[0][0] : (char*)&s.z[0][0]) + 16 * 64 * k);
    } else {
      const uint32_t base = (uint32_t)(tb * kStates * (int)sizeof(T));
      if (lane < NBP) {
        buf_load16_lds(brs, bco + base, (char*)&s.b[0][0]);
        buf_load16_lds(crs, bco + base, (char*)&s.c[0][0]);
      }
    }
  };
  const uint32_t yo = (uint32_t)(c * sizeof(T));   // phase C: this lane's channel

  const float4 a4 = *reinterpret_cast<const float4*>(A + (int64_t)cc * kStates + 4 * wave);
  const float a0 = a4.x * kLog2e, a1 = a4.y * kLog2e, a2 = a4.z * kLog2e, a3 = a4.w * kLog2e;
  float w[kConv];
#pragma unroll
  for (int j = 0; j < kConv; ++j) w[j] = conv_w[(int64_t)cc * kConv + j];
  const float Dc = Dp[cc];
  float h0 = 0.f, h1 = 0.f, h2 = 0.f, h3 = 0.f;
  if (state_in) {
    const float4 s4 = *reinterpret_cast<const float4*>(state_in + (b * Dch + cc) * kStates + 4 * wave);
    h0 = s4.x;
    h1 = s4.y;
    h2 = s4.z;
    h3 = s4.w;
  }

  // Staging ring of kScanStages blocks: block ib + kScanStages - 1 is fetched
  // when block ib starts. Fetches past the sequence read zeros into stages
  // that are never used, so every wave issues the same loads per block and a
  // wait can count them. Before block ib, this wave's memory operations issued
  // after block ib's loads are: the loads of the blocks fetched since (n_ld
  // instructions per block) and kScanItems y stores per finished block, for at
  // most kScanStages - 1 blocks; vmcnt drains in issue order, so waiting until
  // that many remain means block ib's loads have landed.
  const int n_ld = wave == 0 ? NXI : wave < 3 ? NDI : 2;   // load instructions of this wave per block
  const int nblk = (L + R - 1) / R;
#pragma unroll
  for (int k = 0; k < kScanStages - 1; ++k) fetch(k * R, stage[k]);
  for (int ib = 0; ib < nblk; ++ib) {
    Scan1Stage<T>& s = stage[ib % kScanStages];
    vm_wait_at_most((kScanStages - 2) * n_ld + min(ib, kScanStages - 1) * kScanItems);
    lds_barrier();   // block ib has landed (every wave waited for its loads); block ib - 1 is done
    if (ib == 0 && conv_in) {   // rows -3 .. -1: the carried conv history (oldest first)
      if (tid < (kConv - 1) * kScanChan) s.x[wave][lane] = conv_in[(b * Dch + cc) * (kConv - 1) + wave];
      lds_barrier();
    }
    fetch((ib + kScanStages - 1) * R, stage[(ib + kScanStages - 1) % kScanStages]);
    // A: lane = (rows wave + 4 k, channel lane)
    float du[kScanItems];   // D u of this lane's items, used again in phase C
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) {
      const int r = wave + kScanQuads * k;
      float xv[kConv];
#pragma unroll
      for (int j = 0; j < kConv; ++j) xv[j] = to_f32(s.x[r + j][lane]);
      const float u = fmaf(w[0], xv[0], fmaf(w[1], xv[1], fmaf(w[2], xv[2], w[3] * xv[3])));
      const float d = to_f32(s.dt[r][lane]);
      dd[r][lane] = make_float2(d, d * u);
      du[k] = Dc * u;
    }
    if (tid < R * kScanQuads) {
      const int t = tid / kScanQuads, qd = tid % kScanQuads;
      bcq[t][qd][0] = make_float4(to_f32(s.b[t][4 * qd]), to_f32(s.b[t][4 * qd + 1]), to_f32(s.b[t][4 * qd + 2]),
                                  to_f32(s.b[t][4 * qd + 3]));
      bcq[t][qd][1] = make_float4(to_f32(s.c[t][4 * qd]), to_f32(s.c[t][4 * qd + 1]), to_f32(s.c[t][4 * qd + 2]),
                                  to_f32(s.c[t][4 * qd + 3]));
    }
    lds_barrier();
    // B: lane = (state quad wave, channel lane); the values of kScanRowsLoaded
    // rows are read from LDS together, so that the row loop waits once per group
#pragma unroll
    for (int t0 = 0; t0 < R; t0 += kScanRowsLoaded) {
      float2 q[kScanRowsLoaded];
      float4 gb[kScanRowsLoaded], gc[kScanRowsLoaded];
#pragma unroll
      for (int t = 0; t < kScanRowsLoaded; ++t) {
        q[t] = dd[t0 + t][lane];
        gb[t] = bcq[t0 + t][wave][0];
        gc[t] = bcq[t0 + t][wave][1];
      }
#pragma unroll
      for (int t = 0; t < kScanRowsLoaded; ++t) {
        h0 = fmaf(fast_exp2(q[t].x * a0), h0, q[t].y * gb[t].x);
        h1 = fmaf(fast_exp2(q[t].x * a1), h1, q[t].y * gb[t].y);
        h2 = fmaf(fast_exp2(q[t].x * a2), h2, q[t].y * gb[t].z);
        h3 = fmaf(fast_exp2(q[t].x * a3), h3, q[t].y * gb[t].w);
        part[t0 + t][wave][lane] = fmaf(gc[t].x, h0, fmaf(gc[t].y, h1, fmaf(gc[t].z, h2, gc[t].w * h3)));
      }
    }
    lds_barrier();
    // C: lane = (rows wave + 4 k, channel lane)
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) {
      const int r = wave + kScanQuads * k;
      float acc = du[k];
#pragma unroll
      for (int p = 0; p < kScanQuads; ++p) acc += part[r][p][lane];
      const float g = acc * silu(to_f32(s.z[r][lane]));
      buf_store(yrs, cv ? yo + (uint32_t)(ib * R + r) * row_b : kBufferNowhere, from_f32<T>(g));
    }
  }
  // the prefetches past the sequence land before the workgroup's LDS is released
  vm_wait_at_most(0);

  if (!cv) return;
  if (state_out)
    *reinterpret_cast<float4*>(state_out + (b * Dch + c) * kStates + 4 * wave) = make_float4(h0, h1, h2, h3);
  if (conv_state_out && wave == 0) {   // raw x of rows L-3, L-2, L-1 (before row 0: the carried history, or zero)
    T* csp = conv_state_out + (b * Dch + c) * (kConv - 1);
#pragma unroll
    for (int j = 0; j < kConv - 1; ++j) {
      const int t = L - (kConv - 1) + j;
      csp[j] = t >= 0    ? x[(seq + t) * Dch + c]
               : conv_in ? conv_in[(b * Dch + c) * (kConv - 1) + (kConv - 1) + t]
                         : from_f32<T>(0.f);
    }
  }
}

// Decode step (ssm_step.hpp): a lane quad per (sequence, channel), 4 states
// per lane, and two channels per quad (c and c + d_inner / 2), so that the
// whole step is one round of workgroups; every load of a lane is issued
// before its first use. Grid: (channel-pair blocks, sequences).
template <typename T>
__global__ __launch_bounds__(256) void ssm_decode_kernel(ssm_step::Ptrs<T> p) {
  const int q = threadIdx.x & 3;
  const int qi = blockIdx.x * 64 + (threadIdx.x >> 2);   // channel pair within the sequence
  const int64_t b = blockIdx.y;
  const int half = p.d_inner / 2;                          // (d_inner is a multiple of 8)
  const bool ok = qi < half;                               // the same for the whole quad
  ssm_step::Item<T> it[2];
  ssm_step::load(p, it[0], b, ok ? qi : 0, q, ok);
  ssm_step::load(p, it[1], b, ok ? qi + half : 0, q, ok);
  ssm_step::finish(p, it[0], q);
  ssm_step::finish(p, it[1], q);
}

template <typename T>
hipError_t chunk_end_t(const SsmPrefillArgs& a, hipStream_t stream, Timing tm) {
  const int CT = a.chunk_rows;
  const int nchunk = (a.L + CT - 1) / CT;
  if (nchunk < 2) return no_kernel(stream, tm);
  const int cblocks = (a.d_inner + kChanPerBlock - 1) / kChanPerBlock;
  HYMBA_LAUNCH((ssm_chunk_kernel<T, false>), dim3(cblocks, nchunk - 1, a.batch), dim3(kChanPerBlock), 0, stream, tm,
                     (const T*)a.x, (const T*)a.z, (const T*)a.dt, (const T*)a.B, (const T*)a.C, a.A, a.D, a.conv_w,
                     (const T*)a.conv_in, (const float*)nullptr, a.agg, a.sdt, (T*)nullptr, (float*)nullptr,
                     (T*)nullptr, a.L, a.d_inner, CT);
  return hipGetLastError();
}

template <typename T>
hipError_t chunk_out_t(const SsmPrefillArgs& a, hipStream_t stream, Timing tm) {
  const int CT = a.chunk_rows;
  const int nchunk = (a.L + CT - 1) / CT;
  const int cblocks = (a.d_inner + kChanPerBlock - 1) / kChanPerBlock;
  // the output pass covers every chunk (the grid's y extent is nchunk)
  HYMBA_LAUNCH((ssm_chunk_kernel<T, true>), dim3(cblocks, nchunk, a.batch), dim3(kChanPerBlock), 0, stream, tm,
                     (const T*)a.x, (const T*)a.z, (const T*)a.dt, (const T*)a.B, (const T*)a.C, a.A, a.D, a.conv_w,
                     (const T*)a.conv_in, a.carry, (float*)nullptr, (float*)nullptr, (T*)a.y, a.state_out,
                     (T*)a.conv_state_out, a.L, a.d_inner, CT);
  return hipGetLastError();
}

template <typename T>
hipError_t scan1_t(const SsmPrefillArgs& a, hipStream_t stream, Timing tm) {
  const dim3 grid((unsigned)((a.d_inner + kScanChan - 1) / kScanChan * a.batch));   // (channel block, sequence)
  HYMBA_LAUNCH(ssm_scan1_kernel<T>, grid, dim3(256), 0, stream, tm, (const T*)a.x, (const T*)a.z, (const T*)a.dt,
               (const T*)a.B, (const T*)a.C, a.A, a.D, a.conv_w, (const T*)a.conv_in, a.state_in, (T*)a.y,
               a.state_out, (T*)a.conv_state_out, a.L, a.d_inner);
  return hipGetLastError();
}

}  // namespace

bool ssm_single_pass(int batch, int d_inner) {
  // the single-pass form's waves (64 channels x 4 states of one sequence
  // each) fill the chip on their own: about one per SIMD of a 256-CU device
  // or more. Measured on 4224-row sequences of 3200 channels (prefill step):
  // the chunked form is faster at batch 2 and 4 (0.38 / 0.73 ms against
  // 0.70 / 0.78), the single pass from batch 6 on (0.97 / 1.15 / 1.38 ms
  // against 1.01 / 1.25 / 1.59 at batch 6 / 8 / 10)
  return (int64_t)batch * ((d_inner + 31) / 32) >= 512;
}

int ssm_prefill_chunk_rows(int batch, int L, int d_inner) {
  if (ssm_single_pass(batch, d_inner)) return L;   // one chunk: the whole sequence
  // Every (sequence, channel block, chunk) workgroup is two waves and all of
  // them are resident at once, so a SIMD's time is its number of waves times
  // the rows per chunk. Ask for at least 2048 workgroups (four waves on each
  // of the 1024 SIMDs of a 256-CU chip: enough to hide the scan's latency),
  // then round the rows per chunk down to whole staging blocks: rounding up
  // would drop below four waves per SIMD, where the busiest SIMDs hold a
  // whole wave more than the average (2176 rows, 25 channel blocks: 24-row
  // chunks give 4.4 waves per SIMD, 32-row chunks 3.3).
  const int64_t per_chunk = (int64_t)batch * ((d_inner + kChanPerBlock - 1) / kChanPerBlock);
  const int64_t want = (2048 + per_chunk - 1) / per_chunk;   // chunks per sequence
  int64_t ct = L / want / kRowBlock * kRowBlock;
  if (ct < kRowBlock) ct = kRowBlock;
  // the carry chain keeps a whole segment in registers up to kCarryBatch
  // steps per segment; past that it reads every end state twice
  const int64_t max_chunks = (int64_t)kCarrySegs * kCarryBatch + 1;
  const int64_t ct_chain = ((L + max_chunks - 1) / max_chunks + kRowBlock - 1) / kRowBlock * kRowBlock;
  return (int)std::max(ct, ct_chain);
}

hipError_t launch_ssm_chunk_end(const SsmPrefillArgs& a, hipStream_t stream, Timing tm) {
  if (a.act == HYMBA_BF16) return chunk_end_t<bf16>(a, stream, tm);
  return chunk_end_t<float>(a, stream, tm);
}

hipError_t launch_ssm_carry_chain(const float* A, const float* agg, const float* sdt, const float* state_in,
                                  float* carry, int n_slots, int batch, int d_inner, int head_width,
                                  hipStream_t stream, Timing tm) {
  const int64_t per = (int64_t)batch * d_inner * kStates;
  HYMBA_LAUNCH(ssm_chunk_carry_kernel, dim3((unsigned)((per + 63) / 64)), dim3(64 * kCarrySegs), 0, stream, tm, A,
               agg, sdt, state_in, carry, n_slots, batch, d_inner, head_width);
  return hipGetLastError();
}

hipError_t launch_ssm_chunk_carry(const SsmPrefillArgs& a, hipStream_t stream, Timing tm) {
  if (ssm_single_pass(a.batch, a.d_inner)) return no_kernel(stream, tm);   // the state starts in registers
  const int nchunk = (a.L + a.chunk_rows - 1) / a.chunk_rows;
  return launch_ssm_carry_chain(a.A, a.agg, a.sdt, a.state_in, a.carry, nchunk, a.batch, a.d_inner, 0, stream, tm);
}

hipError_t launch_ssm_chunk_out(const SsmPrefillArgs& a, hipStream_t stream, Timing tm) {
  if (ssm_single_pass(a.batch, a.d_inner)) {
    if (a.act == HYMBA_BF16) return scan1_t<bf16>(a, stream, tm);
    return scan1_t<float>(a, stream, tm);
  }
  if (a.act == HYMBA_BF16) return chunk_out_t<bf16>(a, stream, tm);
  return chunk_out_t<float>(a, stream, tm);
}

hipError_t launch_ssm_decode(const SsmDecodeArgs& a, hipStream_t stream, Timing tm) {
  const dim3 grid((unsigned)((a.d_inner / 2 + 63) / 64), (unsigned)a.batch), block(256);
  if (a.act == HYMBA_BF16)
    HYMBA_LAUNCH(ssm_decode_kernel<bf16>, grid, block, 0, stream, tm, ssm_step_ptrs<bf16>(a));
  else
    HYMBA_LAUNCH(ssm_decode_kernel<float>, grid, block, 0, stream, tm, ssm_step_ptrs<float>(a));
  return hipGetLastError();
}

}  // namespace hymba
