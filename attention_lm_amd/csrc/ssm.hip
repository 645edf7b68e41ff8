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

// 16 wave-uniform values of one row of B or C (shared by all channels)
template <typename T>
__device__ __forceinline__ void load_row16(const T* p, float* o) {
  load_n<kStates>(p, o);
}

template <typename T>
__global__ __launch_bounds__(kChanPerBlock) void ssm_chunk_end_kernel(
    const T* __restrict__ x, const T* __restrict__ dt, const T* __restrict__ Bm, const float* __restrict__ A,
    const float* __restrict__ conv_w, float* __restrict__ agg, float* __restrict__ sdt, int L, int Dch, int CT) {
  const int c = blockIdx.x * kChanPerBlock + threadIdx.x;
  const int k = blockIdx.y;
  const int b = blockIdx.z;
  const int batch = gridDim.z;
  const bool cv = c < Dch;
  const int cc = cv ? c : Dch - 1;   // clamped channel for loads; results of invalid lanes are dropped
  const int64_t seq = (int64_t)b * L;
  const int t0 = k * CT, t1 = min(t0 + CT, L);

  float A2[kStates], w[kConv], h[kStates];
#pragma unroll
  for (int n = 0; n < kStates; ++n) {
    A2[n] = A[(int64_t)cc * kStates + n] * kLog2e;
    h[n] = 0.f;
  }
#pragma unroll
  for (int j = 0; j < kConv; ++j) w[j] = conv_w[(int64_t)cc * kConv + j];
  float xm3 = t0 >= 3 ? to_f32(x[(seq + t0 - 3) * Dch + cc]) : 0.f;
  float xm2 = t0 >= 2 ? to_f32(x[(seq + t0 - 2) * Dch + cc]) : 0.f;
  float xm1 = t0 >= 1 ? to_f32(x[(seq + t0 - 1) * Dch + cc]) : 0.f;
  float S = 0.f;
  // next row's x and dt are loaded one iteration ahead
  T xn = x[(seq + t0) * Dch + cc], dn = dt[(seq + t0) * Dch + cc];
#pragma unroll 2
  for (int t = t0; t < t1; ++t) {
    const float xt = to_f32(xn), d = to_f32(dn);
    const int tn = min(t + 1, t1 - 1);
    xn = x[(seq + tn) * Dch + cc];
    dn = dt[(seq + tn) * Dch + cc];
    const float u = fmaf(w[0], xm3, fmaf(w[1], xm2, fmaf(w[2], xm1, w[3] * xt)));
    xm3 = xm2; xm2 = xm1; xm1 = xt;
    const float du = d * u;
    float Bv[kStates];
    load_row16(Bm + (seq + t) * kStates, Bv);
#pragma unroll
    for (int n = 0; n < kStates; ++n) h[n] = fmaf(fast_exp2(d * A2[n]), h[n], du * Bv[n]);
    S += d;
  }
  if (!cv) return;
  const int64_t o = (((int64_t)k * batch + b) * Dch + c);
  float4* ap = reinterpret_cast<float4*>(agg + o * kStates);
#pragma unroll
  for (int q = 0; q < kStates / 4; ++q) ap[q] = make_float4(h[4 * q], h[4 * q + 1], h[4 * q + 2], h[4 * q + 3]);
  sdt[o] = S;
}

// carry[k] = state entering chunk k, from the chunk end states agg[k] (zero start)
// and the chunk dt sums sdt[k].
__global__ __launch_bounds__(256) void ssm_chunk_carry_kernel(const float* __restrict__ A,
                                                              const float* __restrict__ agg,
                                                              const float* __restrict__ sdt,
                                                              float* __restrict__ carry, int nchunk, int batch,
                                                              int Dch) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // (b, c, n)
  const int64_t per = (int64_t)batch * Dch * kStates;
  if (idx >= per) return;
  const int n = (int)(idx % kStates);
  const int64_t bc = idx / kStates;
  const int c = (int)(bc % Dch);
  const float a2 = A[(int64_t)c * kStates + n] * kLog2e;
  float H = 0.f;
  carry[idx] = 0.f;
#pragma unroll 4
  for (int k = 0; k + 1 < nchunk; ++k) {
    const float a = agg[k * per + idx];
    const float s = sdt[k * (per / kStates) + bc];
    H = fmaf(fast_exp2(a2 * s), H, a);
    carry[(k + 1) * per + idx] = H;
  }
}

template <typename T>
__global__ __launch_bounds__(kChanPerBlock) void ssm_chunk_out_kernel(
    const T* __restrict__ x, const T* __restrict__ z, const T* __restrict__ dt, const T* __restrict__ Bm,
    const T* __restrict__ Cm, const float* __restrict__ A, const float* __restrict__ Dp,
    const float* __restrict__ conv_w, const float* __restrict__ carry, T* __restrict__ y,
    float* __restrict__ state_out, T* __restrict__ conv_state_out, int L, int Dch, int CT) {
  const int c = blockIdx.x * kChanPerBlock + threadIdx.x;
  const int k = blockIdx.y;
  const int b = blockIdx.z;
  const int batch = gridDim.z;
  const int nchunk = gridDim.y;
  const bool cv = c < Dch;
  const int cc = cv ? c : Dch - 1;
  const int64_t seq = (int64_t)b * L;
  const int t0 = k * CT, t1 = min(t0 + CT, L);

  float A2[kStates], w[kConv], h[kStates];
  const float4* cp = reinterpret_cast<const float4*>(carry + (((int64_t)k * batch + b) * Dch + cc) * kStates);
#pragma unroll
  for (int q = 0; q < kStates / 4; ++q) {
    const float4 v = cp[q];
    h[4 * q] = v.x; h[4 * q + 1] = v.y; h[4 * q + 2] = v.z; h[4 * q + 3] = v.w;
  }
#pragma unroll
  for (int n = 0; n < kStates; ++n) A2[n] = A[(int64_t)cc * kStates + n] * kLog2e;
#pragma unroll
  for (int j = 0; j < kConv; ++j) w[j] = conv_w[(int64_t)cc * kConv + j];
  const float Dc = Dp[cc];
  float xm3 = t0 >= 3 ? to_f32(x[(seq + t0 - 3) * Dch + cc]) : 0.f;
  float xm2 = t0 >= 2 ? to_f32(x[(seq + t0 - 2) * Dch + cc]) : 0.f;
  float xm1 = t0 >= 1 ? to_f32(x[(seq + t0 - 1) * Dch + cc]) : 0.f;
  T xn = x[(seq + t0) * Dch + cc], dn = dt[(seq + t0) * Dch + cc], zn = z[(seq + t0) * Dch + cc];
#pragma unroll 2
  for (int t = t0; t < t1; ++t) {
    const float xt = to_f32(xn), d = to_f32(dn), zt = to_f32(zn);
    const int tn = min(t + 1, t1 - 1);
    xn = x[(seq + tn) * Dch + cc];
    dn = dt[(seq + tn) * Dch + cc];
    zn = z[(seq + tn) * Dch + cc];
    const float u = fmaf(w[0], xm3, fmaf(w[1], xm2, fmaf(w[2], xm1, w[3] * xt)));
    xm3 = xm2; xm2 = xm1; xm1 = xt;
    const float du = d * u;
    float Bv[kStates], Cv[kStates];
    load_row16(Bm + (seq + t) * kStates, Bv);
    load_row16(Cm + (seq + t) * kStates, Cv);
    float acc = Dc * u;
#pragma unroll
    for (int n = 0; n < kStates; ++n) {
      h[n] = fmaf(fast_exp2(d * A2[n]), h[n], du * Bv[n]);
      acc = fmaf(Cv[n], h[n], acc);
    }
    if (cv) y[(seq + t) * Dch + c] = from_f32<T>(acc * silu(zt));
  }
  if (k == nchunk - 1 && cv) {
    if (state_out) {
      float4* sp = reinterpret_cast<float4*>(state_out + ((int64_t)b * Dch + c) * kStates);
#pragma unroll
      for (int q = 0; q < kStates / 4; ++q) sp[q] = make_float4(h[4 * q], h[4 * q + 1], h[4 * q + 2], h[4 * q + 3]);
    }
    if (conv_state_out) {   // raw x of rows L-3, L-2, L-1 (zero before row 0)
      T* cs = conv_state_out + ((int64_t)b * Dch + c) * (kConv - 1);
      cs[0] = from_f32<T>(xm3);
      cs[1] = from_f32<T>(xm2);
      cs[2] = from_f32<T>(xm1);
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void ssm_decode_kernel(
    const T* __restrict__ x, const T* __restrict__ z, const T* __restrict__ dt,
    const T* __restrict__ Bm, const T* __restrict__ Cm, const float* __restrict__ A,
    const float* __restrict__ Dp, const float* __restrict__ conv_w, float* __restrict__ state,
    T* __restrict__ conv_state, T* __restrict__ y, int batch, int Dch) {
  // lane quad (4 lanes) per (sequence, channel); 4 states per lane
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int q = (int)(gid & 3);
  const int64_t bc = gid >> 2;
  if (bc >= (int64_t)batch * Dch) return;  // uniform over each quad
  const int c = (int)(bc % Dch);
  const int64_t b = bc / Dch;

  float cs[kConv - 1];
#pragma unroll
  for (int j = 0; j < kConv - 1; ++j) cs[j] = to_f32(conv_state[bc * (kConv - 1) + j]);
  const T xr = x[bc];
  const float xn = to_f32(xr);
  float u = conv_w[(int64_t)c * kConv + kConv - 1] * xn;
#pragma unroll
  for (int j = 0; j < kConv - 1; ++j) u = fmaf(conv_w[(int64_t)c * kConv + j], cs[j], u);
  const float d = to_f32(dt[bc]);
  const float du = d * u;

  float4 h4 = *reinterpret_cast<const float4*>(state + bc * kStates + 4 * q);
  float4 a4 = *reinterpret_cast<const float4*>(A + (int64_t)c * kStates + 4 * q);
  float Bv[4], Cv[4];
  load_n<4>(Bm + b * kStates + 4 * q, Bv);
  load_n<4>(Cm + b * kStates + 4 * q, Cv);
  float h[4] = {h4.x, h4.y, h4.z, h4.w};
  const float a[4] = {a4.x, a4.y, a4.z, a4.w};
  float part = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    h[j] = fmaf(fast_exp2(d * a[j] * kLog2e), h[j], du * Bv[j]);
    part = fmaf(Cv[j], h[j], part);
  }
  part += __shfl_xor(part, 1, 64);
  part += __shfl_xor(part, 2, 64);
  *reinterpret_cast<float4*>(state + bc * kStates + 4 * q) = make_float4(h[0], h[1], h[2], h[3]);
  if (q == 0) {
    const float yv = fmaf(Dp[c], u, part) * silu(to_f32(z[bc]));
    y[bc] = from_f32<T>(yv);
#pragma unroll
    for (int j = 0; j < kConv - 2; ++j) conv_state[bc * (kConv - 1) + j] = conv_state[bc * (kConv - 1) + j + 1];
    conv_state[bc * (kConv - 1) + kConv - 2] = xr;
  }
}

template <typename T>
hipError_t prefill_t(const SsmPrefillArgs& a, hipStream_t stream) {
  const int CT = a.chunk_rows;
  const int nchunk = (a.L + CT - 1) / CT;
  const dim3 block(kChanPerBlock);
  const int cblocks = (a.d_inner + kChanPerBlock - 1) / kChanPerBlock;
  if (nchunk > 1) {
    hipLaunchKernelGGL(ssm_chunk_end_kernel<T>, dim3(cblocks, nchunk - 1, a.batch), block, 0, stream, (const T*)a.x,
                       (const T*)a.dt, (const T*)a.B, a.A, a.conv_w, a.agg, a.sdt, a.L, a.d_inner, CT);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t per = (int64_t)a.batch * a.d_inner * kStates;
  hipLaunchKernelGGL(ssm_chunk_carry_kernel, dim3((unsigned)((per + 255) / 256)), dim3(256), 0, stream, a.A, a.agg,
                     a.sdt, a.carry, nchunk, a.batch, a.d_inner);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ssm_chunk_out_kernel<T>, dim3(cblocks, nchunk, a.batch), block, 0, stream, (const T*)a.x,
                     (const T*)a.z, (const T*)a.dt, (const T*)a.B, (const T*)a.C, a.A, a.D, a.conv_w, a.carry,
                     (T*)a.y, a.state_out, (T*)a.conv_state_out, a.L, a.d_inner, CT);
  return hipGetLastError();
}

}  // namespace

int ssm_prefill_chunk_rows(int batch, int L, int d_inner) {
  // enough (sequence, channel block, chunk) workgroups to fill the chip
  // several times over, without making the carry chain long
  const int64_t per_chunk = (int64_t)batch * ((d_inner + kChanPerBlock - 1) / kChanPerBlock);
  const int64_t want = (2048 + per_chunk - 1) / per_chunk;   // chunks per sequence
  int64_t ct = (L + want - 1) / want;
  ct = (ct + 15) / 16 * 16;
  if (ct < 16) ct = 16;
  return (int)ct;
}

hipError_t launch_ssm_prefill(const SsmPrefillArgs& a, hipStream_t stream) {
  if (a.act == HYMBA_BF16) return prefill_t<bf16>(a, stream);
  return prefill_t<float>(a, stream);
}

hipError_t launch_ssm_decode(const SsmDecodeArgs& a, hipStream_t stream) {
  const int64_t threads = (int64_t)a.batch * a.d_inner * 4;
  if (threads == 0) return hipSuccess;
  dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  if (a.act == HYMBA_BF16)
    hipLaunchKernelGGL(ssm_decode_kernel<bf16>, grid, block, 0, stream, (const bf16*)a.x, (const bf16*)a.z,
                       (const bf16*)a.dt, (const bf16*)a.B, (const bf16*)a.C, a.A, a.D, a.conv_w, a.state,
                       (bf16*)a.conv_state, (bf16*)a.y, a.batch, a.d_inner);
  else
    hipLaunchKernelGGL(ssm_decode_kernel<float>, grid, block, 0, stream, (const float*)a.x, (const float*)a.z,
                       (const float*)a.dt, (const float*)a.B, (const float*)a.C, a.A, a.D, a.conv_w, a.state,
                       (float*)a.conv_state, (float*)a.y, a.batch, a.d_inner);
  return hipGetLastError();
}

}  // namespace hymba
