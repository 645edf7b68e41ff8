// Mamba branch: causal depthwise conv (4 taps) + selective scan (d_state 16)
// + D skip + silu(z) gate, for prefill (whole sequences) and decode (one row).
//
// Recurrence ("Jamba: Hybrid SSM-Transformer", "1. Layer Interleaving Ratio";
// "Lecture 04 - Beyond the Dense Transformer", section 2):
//   h_t = exp(dt_t A) (.) h_{t-1} + (dt_t B_t) u_t,   y_t = C_t . h_t + D u_t.
//
// Prefill design. A workgroup owns CPB channels of one sequence and walks the
// sequence in blocks of NW*TC rows; wave w takes rows [w*TC, (w+1)*TC) of each
// block. Lane (channel c, slice s) holds SPL of the 16 states of c in
// registers. Per block:
//   pass 1  each wave scans its TC rows from a zero state, keeping every
//           exp(dt A) factor in registers, and leaves its end state and the
//           sum of its dt in LDS;
//   combine one thread per (channel, state) chains the NW wave results with
//           the block's carried state: the decay over a wave's rows is
//           exp(A * sum(dt)), so a wave's carry-in is a short linear chain;
//   pass 2  each wave re-runs its rows from its true carry-in using the cached
//           factors (no further exp), forms y_t, gates it and stores it.
// So every (row, channel, state) costs one exp. Rows past the end of the
// sequence use dt = 0, which leaves the state unchanged.
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

template <typename T, int SPL, int TC, int NW>
__global__ __launch_bounds__(64 * NW) void ssm_prefill_kernel(
    const T* __restrict__ x, const T* __restrict__ z, const T* __restrict__ dt,
    const T* __restrict__ Bm, const T* __restrict__ Cm, const float* __restrict__ A,
    const float* __restrict__ Dp, const float* __restrict__ conv_w, T* __restrict__ y,
    float* __restrict__ state_out, T* __restrict__ conv_state_out, int L, int Dch) {
  constexpr int LPC = kStates / SPL;  // lanes per channel
  constexpr int CPB = 64 / LPC;       // channels per workgroup
  constexpr int NT = 64 * NW;

  __shared__ float aggH[NW][kStates][CPB];
  __shared__ float aggS[NW][CPB];
  __shared__ float carryH[kStates][CPB];
  __shared__ float A2s[kStates][CPB];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int cl = lane / LPC;
  const int qs = lane % LPC;
  const int c0 = blockIdx.x * CPB;
  const int c = c0 + cl;
  const bool cvalid = c < Dch;
  const int n0 = qs * SPL;
  const int64_t seq = (int64_t)blockIdx.y * L;

  for (int k = threadIdx.x; k < kStates * CPB; k += NT) {
    const int n = k / CPB, cc = k % CPB;
    const int cg = c0 + cc;
    A2s[n][cc] = cg < Dch ? A[(int64_t)cg * kStates + n] * kLog2e : 0.f;
    carryH[n][cc] = 0.f;
  }
  float A2[SPL];
#pragma unroll
  for (int j = 0; j < SPL; ++j) A2[j] = cvalid ? A[(int64_t)c * kStates + n0 + j] * kLog2e : 0.f;
  float w[kConv];
#pragma unroll
  for (int j = 0; j < kConv; ++j) w[j] = cvalid ? conv_w[(int64_t)c * kConv + j] : 0.f;
  const float Dc = cvalid ? Dp[c] : 0.f;
  __syncthreads();

  constexpr int ROWS = NW * TC;
  const int nblk = (L + ROWS - 1) / ROWS;
  for (int blk = 0; blk < nblk; ++blk) {
    const int r0 = blk * ROWS + wave * TC;
    // conv over rows r0-3 .. r0+TC-1 (zero history before row 0)
    float xv[TC + kConv - 1];
#pragma unroll
    for (int k = 0; k < TC + kConv - 1; ++k) {
      const int t = r0 - (kConv - 1) + k;
      xv[k] = (cvalid && t >= 0 && t < L) ? to_f32(x[(seq + t) * Dch + c]) : 0.f;
    }
    float u[TC], dtv[TC], dtu[TC], zv[TC];
#pragma unroll
    for (int i = 0; i < TC; ++i) {
      const int t = r0 + i;
      const bool ok = cvalid && t < L;
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < kConv; ++j) acc = fmaf(w[j], xv[i + j], acc);
      u[i] = acc;
      dtv[i] = ok ? to_f32(dt[(seq + t) * Dch + c]) : 0.f;
      zv[i] = ok ? to_f32(z[(seq + t) * Dch + c]) : 0.f;
      dtu[i] = dtv[i] * acc;
    }

    // pass 1: scan from zero, cache exp(dt A)
    float dA[TC][SPL];
    float h[SPL];
#pragma unroll
    for (int j = 0; j < SPL; ++j) h[j] = 0.f;
    float S = 0.f;
#pragma unroll
    for (int i = 0; i < TC; ++i) {
      const int t = min(r0 + i, L - 1);
      float Bv[SPL];
      load_n<SPL>(Bm + (seq + t) * kStates + n0, Bv);
#pragma unroll
      for (int j = 0; j < SPL; ++j) {
        const float a = fast_exp2(dtv[i] * A2[j]);
        dA[i][j] = a;
        h[j] = fmaf(a, h[j], dtu[i] * Bv[j]);
      }
      S += dtv[i];
    }
#pragma unroll
    for (int j = 0; j < SPL; ++j) aggH[wave][n0 + j][cl] = h[j];
    if (qs == 0) aggS[wave][cl] = S;
    __syncthreads();

    // combine: carry-in of each wave, then the block's end state
    for (int k = threadIdx.x; k < kStates * CPB; k += NT) {
      const int n = k / CPB, cc = k % CPB;
      float carry = carryH[n][cc];
      const float a2 = A2s[n][cc];
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) {
        const float hw = aggH[ww][n][cc];
        const float P = fast_exp2(a2 * aggS[ww][cc]);
        aggH[ww][n][cc] = carry;
        carry = fmaf(P, carry, hw);
      }
      carryH[n][cc] = carry;
    }
    __syncthreads();

    // pass 2: rerun from the true carry-in, output gated y
#pragma unroll
    for (int j = 0; j < SPL; ++j) h[j] = aggH[wave][n0 + j][cl];
#pragma unroll
    for (int i = 0; i < TC; ++i) {
      const int t = r0 + i;
      const int tc = min(t, L - 1);
      float Bv[SPL], Cv[SPL];
      load_n<SPL>(Bm + (seq + tc) * kStates + n0, Bv);
      load_n<SPL>(Cm + (seq + tc) * kStates + n0, Cv);
      float part = 0.f;
#pragma unroll
      for (int j = 0; j < SPL; ++j) {
        h[j] = fmaf(dA[i][j], h[j], dtu[i] * Bv[j]);
        part = fmaf(Cv[j], h[j], part);
      }
#pragma unroll
      for (int o = 1; o < LPC; o <<= 1) part += __shfl_xor(part, o, 64);
      const float yv = fmaf(Dc, u[i], part) * silu(zv[i]);
      if (qs == 0 && cvalid && t < L) y[(seq + t) * Dch + c] = from_f32<T>(yv);
    }
    // the next block's pass 1 writes aggH/aggS only after every wave passed the
    // barrier above; its combine runs after the next barrier
  }

  const int b = blockIdx.y;
  if (state_out) {
    for (int k = threadIdx.x; k < kStates * CPB; k += NT) {
      const int cc = k / kStates, n = k % kStates;
      const int cg = c0 + cc;
      if (cg < Dch) state_out[((int64_t)b * Dch + cg) * kStates + n] = carryH[n][cc];
    }
  }
  if (conv_state_out) {
    for (int k = threadIdx.x; k < (kConv - 1) * CPB; k += NT) {
      const int cc = k / (kConv - 1), j = k % (kConv - 1);
      const int cg = c0 + cc;
      const int t = L - (kConv - 1) + j;
      if (cg < Dch)
        conv_state_out[((int64_t)b * Dch + cg) * (kConv - 1) + j] =
            t >= 0 ? x[(seq + t) * Dch + cg] : from_f32<T>(0.f);
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

template <typename T, int SPL, int TC, int NW>
hipError_t prefill_t(const SsmPrefillArgs& a, hipStream_t stream) {
  constexpr int CPB = 64 / (kStates / SPL);
  dim3 grid((a.d_inner + CPB - 1) / CPB, a.batch);
  hipLaunchKernelGGL((ssm_prefill_kernel<T, SPL, TC, NW>), grid, dim3(64 * NW), 0, stream, (const T*)a.x,
                     (const T*)a.z, (const T*)a.dt, (const T*)a.B, (const T*)a.C, a.A, a.D, a.conv_w, (T*)a.y,
                     a.state_out, (T*)a.conv_state_out, a.L, a.d_inner);
  return hipGetLastError();
}

template <typename T>
hipError_t prefill_pick(const SsmPrefillArgs& a, hipStream_t stream) {
  // Enough workgroups to cover the 256 compute units: fewer states per lane
  // (more lanes per channel) when the batch has few channels.
  const int64_t chans = (int64_t)a.batch * a.d_inner;
  if (chans >= 64 * 256) return prefill_t<T, 16, 4, 8>(a, stream);
  if (chans >= 32 * 256) return prefill_t<T, 8, 8, 8>(a, stream);
  return prefill_t<T, 4, 8, 8>(a, stream);
}

}  // namespace

hipError_t launch_ssm_prefill(const SsmPrefillArgs& a, hipStream_t stream) {
  if (a.act == HYMBA_BF16) return prefill_pick<bf16>(a, stream);
  return prefill_pick<float>(a, stream);
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
