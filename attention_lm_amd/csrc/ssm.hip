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
constexpr int kRowBlock = 16;        // rows staged in LDS per step

// One pass of the chunked scan over rows [t0, t1) of 128 channels.
//  OUT = false: start from zero, write the chunk's end state and dt sum.
//  OUT = true:  start from the chunk's carry-in, write gated y (and, for the
//               last chunk, the final SSM state and conv history).
// Inputs are staged through LDS in blocks of kRowBlock rows, double-buffered:
// the global loads of block i+1 are in flight while block i is scanned.
template <typename T, bool OUT>
__global__ __launch_bounds__(kChanPerBlock) void ssm_chunk_kernel(
    const T* __restrict__ x, const T* __restrict__ z, const T* __restrict__ dt, const T* __restrict__ Bm,
    const T* __restrict__ Cm, const float* __restrict__ A, const float* __restrict__ Dp,
    const float* __restrict__ conv_w, const float* __restrict__ carry, float* __restrict__ agg,
    float* __restrict__ sdt, T* __restrict__ y, float* __restrict__ state_out, T* __restrict__ conv_state_out,
    int L, int Dch, int CT) {
  constexpr int E = Vec16<T>::n;                  // elements per 16-byte vector
  constexpr int RV = kChanPerBlock / E;           // vectors per 128-channel row
  constexpr int XR = kRowBlock + kConv - 1;       // x rows per block (with conv history)
  constexpr int NX = (XR * RV + kChanPerBlock - 1) / kChanPerBlock;
  constexpr int NR = (kRowBlock * RV + kChanPerBlock - 1) / kChanPerBlock;
  constexpr int NBC = (kRowBlock * kStates / E + kChanPerBlock - 1) / kChanPerBlock;
  __shared__ __attribute__((aligned(16))) T xs[2][XR][kChanPerBlock];
  __shared__ __attribute__((aligned(16))) T ds[2][kRowBlock][kChanPerBlock];
  __shared__ __attribute__((aligned(16))) T zs[OUT ? 2 : 1][OUT ? kRowBlock : 1][kChanPerBlock];
  __shared__ __attribute__((aligned(16))) float bs[2][kRowBlock][kStates];
  __shared__ __attribute__((aligned(16))) float cs[OUT ? 2 : 1][OUT ? kRowBlock : 1][kStates];

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

  // staging registers
  uint4 rx[NX], rd[NR], rz[OUT ? NR : 1], rb[NBC], rc[OUT ? NBC : 1];
  auto vec_ok = [&](int t, int v) { return t >= 0 && t < L && c0 + (v + 1) * E <= Dch; };
  auto fetch = [&](int tb) {
#pragma unroll
    for (int r = 0; r < NX; ++r) {
      const int it = tid + r * kChanPerBlock, row = it / RV, v = it % RV, t = tb - (kConv - 1) + row;
      rx[r] = make_uint4(0, 0, 0, 0);
      if (it < XR * RV && vec_ok(t, v)) rx[r] = *reinterpret_cast<const uint4*>(x + (seq + t) * Dch + c0 + v * E);
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int it = tid + r * kChanPerBlock, row = it / RV, v = it % RV, t = tb + row;
      rd[r] = make_uint4(0, 0, 0, 0);
      if (it < kRowBlock * RV && t < t1 && vec_ok(t, v))
        rd[r] = *reinterpret_cast<const uint4*>(dt + (seq + t) * Dch + c0 + v * E);
      if constexpr (OUT) {
        rz[r] = make_uint4(0, 0, 0, 0);
        if (it < kRowBlock * RV && t < t1 && vec_ok(t, v))
          rz[r] = *reinterpret_cast<const uint4*>(z + (seq + t) * Dch + c0 + v * E);
      }
    }
#pragma unroll
    for (int r = 0; r < NBC; ++r) {
      const int it = tid + r * kChanPerBlock;          // 16-byte vector of the block's B (or C) rows
      const int t = tb + (it * E) / kStates;
      rb[r] = make_uint4(0, 0, 0, 0);
      if (it * E < kRowBlock * kStates && t < t1) rb[r] = *reinterpret_cast<const uint4*>(Bm + seq * kStates + (int64_t)tb * kStates + it * E);
      if constexpr (OUT) {
        rc[r] = make_uint4(0, 0, 0, 0);
        if (it * E < kRowBlock * kStates && t < t1) rc[r] = *reinterpret_cast<const uint4*>(Cm + seq * kStates + (int64_t)tb * kStates + it * E);
      }
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int r = 0; r < NX; ++r) {
      const int it = tid + r * kChanPerBlock;
      if (it < XR * RV) *reinterpret_cast<uint4*>(&xs[buf][it / RV][(it % RV) * E]) = rx[r];
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int it = tid + r * kChanPerBlock;
      if (it < kRowBlock * RV) {
        *reinterpret_cast<uint4*>(&ds[buf][it / RV][(it % RV) * E]) = rd[r];
        if constexpr (OUT) *reinterpret_cast<uint4*>(&zs[buf][it / RV][(it % RV) * E]) = rz[r];
      }
    }
#pragma unroll
    for (int r = 0; r < NBC; ++r) {
      const int it = tid + r * kChanPerBlock;
      if (it * E < kRowBlock * kStates) {
        float f[E];
        load16(reinterpret_cast<const T*>(&rb[r]), f);
        float* dst = &bs[buf][0][0] + it * E;
#pragma unroll
        for (int e = 0; e < E; ++e) dst[e] = f[e];
        if constexpr (OUT) {
          load16(reinterpret_cast<const T*>(&rc[r]), f);
          float* dc = &cs[buf][0][0] + it * E;
#pragma unroll
          for (int e = 0; e < E; ++e) dc[e] = f[e];
        }
      }
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
  float xm3 = 0.f, xm2 = 0.f, xm1 = 0.f;

  const int nblk = (t1 - t0 + kRowBlock - 1) / kRowBlock;
  fetch(t0);
  stash(0);
  __syncthreads();
  for (int ib = 0; ib < nblk; ++ib) {
    const int buf = ib & 1;
    const int tb = t0 + ib * kRowBlock;
    if (ib + 1 < nblk) fetch(tb + kRowBlock);
    xm3 = to_f32(xs[buf][0][tid]);
    xm2 = to_f32(xs[buf][1][tid]);
    xm1 = to_f32(xs[buf][2][tid]);
    // staged rows at or past t1 hold dt = 0 (state unchanged) and are not stored
#pragma unroll 4
    for (int i = 0; i < kRowBlock; ++i) {
      const float xt = to_f32(xs[buf][i + kConv - 1][tid]);
      const float d = to_f32(ds[buf][i][tid]);
      const float u = fmaf(w[0], xm3, fmaf(w[1], xm2, fmaf(w[2], xm1, w[3] * xt)));
      if (tb + i < t1) { xm3 = xm2; xm2 = xm1; xm1 = xt; }
      const float du = d * u;
      float Bv[kStates];
#pragma unroll
      for (int q = 0; q < kStates / 4; ++q) {
        const float4 v4 = *reinterpret_cast<const float4*>(&bs[buf][i][4 * q]);
        Bv[4 * q] = v4.x; Bv[4 * q + 1] = v4.y; Bv[4 * q + 2] = v4.z; Bv[4 * q + 3] = v4.w;
      }
      if constexpr (OUT) {
        float Cv[kStates];
#pragma unroll
        for (int q = 0; q < kStates / 4; ++q) {
          const float4 v4 = *reinterpret_cast<const float4*>(&cs[buf][i][4 * q]);
          Cv[4 * q] = v4.x; Cv[4 * q + 1] = v4.y; Cv[4 * q + 2] = v4.z; Cv[4 * q + 3] = v4.w;
        }
        float acc = Dc * u;
#pragma unroll
        for (int n = 0; n < kStates; ++n) {
          h[n] = fmaf(fast_exp2(d * A2[n]), h[n], du * Bv[n]);
          acc = fmaf(Cv[n], h[n], acc);
        }
        const float zt = to_f32(zs[buf][i][tid]);
        if (cv && tb + i < t1) y[(seq + tb + i) * Dch + c] = from_f32<T>(acc * silu(zt));
      } else {
#pragma unroll
        for (int n = 0; n < kStates; ++n) h[n] = fmaf(fast_exp2(d * A2[n]), h[n], du * Bv[n]);
        S += d;
      }
    }
    if (ib + 1 < nblk) stash(buf ^ 1);
    __syncthreads();
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
    if (conv_state_out) {   // raw x of rows L-3, L-2, L-1 (zero before row 0)
      T* csp = conv_state_out + ((int64_t)b * Dch + c) * (kConv - 1);
      csp[0] = from_f32<T>(xm3);
      csp[1] = from_f32<T>(xm2);
      csp[2] = from_f32<T>(xm1);
    }
  }
}

// carry[k] = state entering chunk k, from the chunk end states agg[k] (zero start)
// and the chunk dt sums sdt[k]; loads are issued in batches ahead of the chain.
__global__ __launch_bounds__(256) void ssm_chunk_carry_kernel(const float* __restrict__ A,
                                                              const float* __restrict__ agg,
                                                              const float* __restrict__ sdt,
                                                              float* __restrict__ carry, int nchunk, int batch,
                                                              int Dch) {
  constexpr int KB = 16;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // (b, c, n)
  const int64_t per = (int64_t)batch * Dch * kStates;
  if (idx >= per) return;
  const int n = (int)(idx % kStates);
  const int64_t bc = idx / kStates;
  const int c = (int)(bc % Dch);
  const float a2 = A[(int64_t)c * kStates + n] * kLog2e;
  float H = 0.f;
  carry[idx] = 0.f;
  for (int k0 = 0; k0 + 1 < nchunk; k0 += KB) {
    float av[KB], sv[KB];
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      const int kk = min(k0 + i, nchunk - 2);
      av[i] = agg[kk * per + idx];
      sv[i] = sdt[kk * (per / kStates) + bc];
    }
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      if (k0 + i + 1 < nchunk) {
        H = fmaf(fast_exp2(a2 * sv[i]), H, av[i]);
        carry[(k0 + i + 1) * per + idx] = H;
      }
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
    hipLaunchKernelGGL((ssm_chunk_kernel<T, false>), dim3(cblocks, nchunk - 1, a.batch), block, 0, stream,
                       (const T*)a.x, (const T*)a.z, (const T*)a.dt, (const T*)a.B, (const T*)a.C, a.A, a.D,
                       a.conv_w, (const float*)nullptr, a.agg, a.sdt, (T*)nullptr, (float*)nullptr, (T*)nullptr,
                       a.L, a.d_inner, CT);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t per = (int64_t)a.batch * a.d_inner * kStates;
  hipLaunchKernelGGL(ssm_chunk_carry_kernel, dim3((unsigned)((per + 255) / 256)), dim3(256), 0, stream, a.A, a.agg,
                     a.sdt, a.carry, nchunk, a.batch, a.d_inner);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the output pass covers every chunk (the grid's y extent is nchunk)
  hipLaunchKernelGGL((ssm_chunk_kernel<T, true>), dim3(cblocks, nchunk, a.batch), block, 0, stream, (const T*)a.x,
                     (const T*)a.z, (const T*)a.dt, (const T*)a.B, (const T*)a.C, a.A, a.D, a.conv_w, a.carry,
                     (float*)nullptr, (float*)nullptr, (T*)a.y, a.state_out, (T*)a.conv_state_out, a.L, a.d_inner,
                     CT);
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
