// Mamba branch in the Mamba-2 form ("Lecture 04 - Beyond the Dense
// Transformer", section 3): the state matrix is a scalar per head, so a head's
// whole P x 16 state decays by one factor per row, and the scan can be done as
// block matrix products on the matrix cores.
//
// Head h owns channels h P .. h P + P - 1, decay rate A[h] and step size
// dt[b, t, h]; B_t and C_t are shared by all heads. With S_i = A (dt_0 + ..
// + dt_i) running from a chunk's first row and H the state entering the chunk,
//   y_i = exp(S_i) C_i . H + sum_{j <= i} exp(S_i - S_j) (C_i . B_j) dt_j u_j + D u_i
// and the chunk leaves the state exp(S_last) H + sum_j exp(S_last - S_j) dt_j u_j B_j^T.
//
// Prefill, sequences cut into chunks of 64 rows:
//   1. ssd_state_kernel: per (chunk, head, sequence), the state a chunk
//      leaves from a zero start (P x 16, fp32 VALU) and its dt sum;
//   2. the chunk carry chain of the selective scan (ssm.hip), with one decay
//      rate per head, gives every chunk's entering state and the final state;
//   3. ssd_out_kernel: per (chunk, head, sequence), Y = [M | C exp(S)] x
//      [U ; H^T] on the matrix cores, M[i][j] = (C_i . B_j) exp(S_i - S_j) dt_j
//      below the diagonal (fp32 VALU into LDS), then D u and the silu(z) gate.
// The conv (4 taps, causal, per channel) is recomputed in both passes from x
// (and the carried history before row 0).
#include <utility>

#include "common.hpp"
#include "launch.hpp"
#include "mma.hpp"

namespace hymba {

namespace {

constexpr int kQ = 64;         // rows per chunk
constexpr int kSt = 16;        // states
constexpr int kTaps = 4;       // conv taps
constexpr int kSsdThreads = 256;
constexpr int kRowPad = 4;     // LDS row padding (floats), keeps 16-byte alignment

__device__ __forceinline__ float ssd_silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * kLog2e));
}

// inclusive running sum over the 64 lanes of a wave
__device__ __forceinline__ float wave_scan(float v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const float o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  return v;
}

// What both passes stage for chunk k of head h of sequence b: per row, dt and
// S (in log2 units, A log2(e) times the running dt sum); the conv input rows
// t0 - 3 .. t0 + 63 of the head's channels; the conv taps.
template <typename T, int P>
struct ChunkIn {
  T xs[kQ + kTaps - 1][P];
  float s2[kQ], dts[kQ];
  float cw[P][kTaps];
  float total;   // dt sum over the chunk
};

template <typename T, int P>
__device__ __forceinline__ void stage_chunk(ChunkIn<T, P>& ci, const T* __restrict__ x, const T* __restrict__ dt,
                                            const float* __restrict__ A, const float* __restrict__ conv_w,
                                            const T* __restrict__ conv_in, int64_t b, int h, int t0, int nr, int L,
                                            int D, int H) {
  const int tid = threadIdx.x;
  const int c0 = h * P;
  if (tid < 64) {
    const float d = tid < nr ? to_f32(dt[((b * L) + t0 + tid) * H + h]) : 0.f;
    const float cum = wave_scan(d, tid);
    ci.dts[tid] = d;
    ci.s2[tid] = A[h] * kLog2e * cum;
    if (tid == 63) ci.total = cum;
  }
  for (int e = tid; e < (kQ + kTaps - 1) * P; e += kSsdThreads) {
    const int r = e / P, p = e % P, t = t0 - (kTaps - 1) + r;
    T v = from_f32<T>(0.f);
    if (t >= 0 && t < L)
      v = x[(b * L + t) * D + c0 + p];
    else if (t < 0 && conv_in)
      v = conv_in[(b * D + c0 + p) * (kTaps - 1) + (kTaps - 1) + t];
    ci.xs[r][p] = v;
  }
  for (int e = tid; e < P * kTaps; e += kSsdThreads) ci.cw[e / kTaps][e % kTaps] = conv_w[(int64_t)c0 * kTaps + e];
}

template <typename T, int P>
__device__ __forceinline__ float conv_at(const ChunkIn<T, P>& ci, int j, int p) {
  float u = 0.f;
#pragma unroll
  for (int k = 0; k < kTaps; ++k) u = fmaf(ci.cw[p][k], to_f32(ci.xs[j + k][p]), u);
  return u;
}

// Pass 1: agg[k][b][c][n] = sum_j exp(S_last - S_j) dt_j u_j[c] B_j[n] for the
// head's channels c, and sdt[k][b][c] = the chunk's dt sum.
template <typename T, int P>
__global__ __launch_bounds__(kSsdThreads) void ssd_state_kernel(
    const T* __restrict__ x, const T* __restrict__ dt, const T* __restrict__ Bm, const float* __restrict__ A,
    const float* __restrict__ conv_w, const T* __restrict__ conv_in, float* __restrict__ agg,
    float* __restrict__ sdt, int L, int D, int H, int batch) {
  __shared__ ChunkIn<T, P> ci;
  __shared__ __attribute__((aligned(16))) float us[kQ][P + kRowPad];   // u_j dt_j exp(S_last - S_j)
  __shared__ __attribute__((aligned(16))) float bs[kQ][kSt];
  const int k = blockIdx.x, h = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int tid = threadIdx.x;
  const int t0 = k * kQ, nr = min(kQ, L - t0);
  stage_chunk(ci, x, dt, A, conv_w, conv_in, b, h, t0, nr, L, D, H);
  for (int e = tid; e < kQ * kSt; e += kSsdThreads) {
    const int j = e / kSt;
    bs[j][e % kSt] = j < nr ? to_f32(Bm[(b * L + t0 + j) * kSt + e % kSt]) : 0.f;
  }
  __syncthreads();
  const float s2_last = ci.s2[kQ - 1];
  for (int e = tid; e < kQ * P; e += kSsdThreads) {
    const int j = e / P, p = e % P;
    us[j][p] = conv_at(ci, j, p) * ci.dts[j] * __builtin_amdgcn_exp2f(s2_last - ci.s2[j]);
  }
  __syncthreads();
  const int c0 = h * P;
  const int64_t row0 = ((int64_t)k * batch + b) * D + c0;   // (chunk, sequence, first channel of the head)
  for (int o = tid; o < P * (kSt / 4); o += kSsdThreads) {
    const int p = o / (kSt / 4), n0 = 4 * (o % (kSt / 4));
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll 8
    for (int j = 0; j < kQ; ++j) {
      const float u = us[j][p];
      const float4 bv = *reinterpret_cast<const float4*>(&bs[j][n0]);
      a0 = fmaf(u, bv.x, a0); a1 = fmaf(u, bv.y, a1); a2 = fmaf(u, bv.z, a2); a3 = fmaf(u, bv.w, a3);
    }
    *reinterpret_cast<float4*>(agg + (row0 + p) * kSt + n0) = make_float4(a0, a1, a2, a3);
  }
  for (int p = tid; p < P; p += kSsdThreads) sdt[row0 + p] = ci.total;
}

// Pass 3: the chunk's outputs from its entering state carry[k] (see above).
template <typename T, int P>
__global__ __launch_bounds__(kSsdThreads) void ssd_out_kernel(
    const T* __restrict__ x, const T* __restrict__ z, const T* __restrict__ dt, const T* __restrict__ Bm,
    const T* __restrict__ Cm, const float* __restrict__ A, const float* __restrict__ Dp,
    const float* __restrict__ conv_w, const T* __restrict__ conv_in, const float* __restrict__ carry,
    T* __restrict__ y, float* __restrict__ state_out, T* __restrict__ conv_state_out, int L, int D, int H,
    int batch, int nchunk) {
  typedef Mma<T> M;
  __shared__ ChunkIn<T, P> ci;
  __shared__ __attribute__((aligned(16))) float ut[P][kQ + kRowPad];   // u, [channel][row]
  __shared__ __attribute__((aligned(16))) float ms[kQ][kQ + kRowPad];  // M[i][j]
  __shared__ __attribute__((aligned(16))) float bs[kQ][kSt];
  __shared__ __attribute__((aligned(16))) float cs[kQ][kSt];
  __shared__ __attribute__((aligned(16))) float hs[P][kSt];            // entering state
  const int k = blockIdx.x, h = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int tid = threadIdx.x;
  const int t0 = k * kQ, nr = min(kQ, L - t0);
  const int c0 = h * P;
  stage_chunk(ci, x, dt, A, conv_w, conv_in, b, h, t0, nr, L, D, H);
  for (int e = tid; e < kQ * kSt; e += kSsdThreads) {
    const int j = e / kSt, n = e % kSt;
    const bool in = j < nr;
    bs[j][n] = in ? to_f32(Bm[(b * L + t0 + j) * kSt + n]) : 0.f;
    cs[j][n] = in ? to_f32(Cm[(b * L + t0 + j) * kSt + n]) : 0.f;
  }
  const float* hin = carry + (((int64_t)k * batch + b) * D + c0) * kSt;
  for (int e = tid; e < P * kSt; e += kSsdThreads) hs[e / kSt][e % kSt] = hin[e];
  __syncthreads();
  // u (transposed) and the masked, decayed C B^T block: each thread a 4 x 4
  // block of (i, j)
  for (int e = tid; e < kQ * P; e += kSsdThreads) {
    const int j = e / P, p = e % P;
    ut[p][j] = conv_at(ci, j, p);
  }
  {
    const int i0 = 4 * (tid / 16), j0 = 4 * (tid % 16);
    float g[4][4] = {};
#pragma unroll
    for (int q = 0; q < kSt / 4; ++q) {
      float4 cr[4], br[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        cr[a] = *reinterpret_cast<const float4*>(&cs[i0 + a][4 * q]);
        br[a] = *reinterpret_cast<const float4*>(&bs[j0 + a][4 * q]);
      }
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          g[a][c] = fmaf(cr[a].x, br[c].x, fmaf(cr[a].y, br[c].y, fmaf(cr[a].z, br[c].z, fmaf(cr[a].w, br[c].w, g[a][c]))));
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int i = i0 + a;
      float m4[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int j = j0 + c;
        m4[c] = j <= i ? g[a][c] * __builtin_amdgcn_exp2f(ci.s2[i] - ci.s2[j]) * ci.dts[j] : 0.f;
      }
      *reinterpret_cast<float4*>(&ms[i][j0]) = make_float4(m4[0], m4[1], m4[2], m4[3]);
    }
  }
  __syncthreads();
  // Y tiles of 32 rows x 32 channels, one per wave in turn
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lq = lane & 31, hh = lane >> 5;
  constexpr int NTP = P / 32;
  for (int tile = wave; tile < 2 * NTP; tile += kSsdThreads / 64) {
    const int ti = tile / NTP, tp = tile % NTP;
    const int ia = 32 * ti + lq, pb = 32 * tp + lq;   // this lane's A row and B column
    f32x16_t acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
    for (int kb = 0; kb < kQ / 16; ++kb) {
      const typename M::Frag fa = M::from_f32(&ms[ia][16 * kb + 8 * hh]);
      const typename M::Frag fb = M::from_f32(&ut[pb][16 * kb + 8 * hh]);
      acc = M::mma(fa, fb, acc);
    }
    {   // the entering state: rows of C scaled by exp(S_i), against H^T
      const float es = __builtin_amdgcn_exp2f(ci.s2[ia]);
      float cv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) cv[e] = cs[ia][8 * hh + e] * es;
      acc = M::mma(M::from_f32(cv), M::from_f32(&hs[pb][8 * hh]), acc);
    }
    const int c = c0 + pb;
    const float Dc = Dp[c];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = 32 * ti + 8 * (r >> 2) + 4 * hh + (r & 3);
      if (i < nr) {
        const int64_t o = (b * L + t0 + i) * D + c;
        y[o] = from_f32<T>(fmaf(Dc, ut[pb][i], acc[r]) * ssd_silu(to_f32(z[o])));
      }
    }
  }
  if (k == nchunk - 1) {
    // the state after the last row (the carry chain's last entry) and the conv
    // history (raw x of rows L-3 .. L-1; before row 0 the carried history)
    if (state_out) {
      const float* hl = carry + (((int64_t)nchunk * batch + b) * D + c0) * kSt;
      for (int e = tid; e < P * kSt; e += kSsdThreads) state_out[(b * D + c0) * kSt + e] = hl[e];
    }
    if (conv_state_out) {
      for (int e = tid; e < P * (kTaps - 1); e += kSsdThreads) {
        const int p = e / (kTaps - 1), j = e % (kTaps - 1);
        const int t = L - (kTaps - 1) + j;
        T v = from_f32<T>(0.f);
        if (t >= 0)
          v = x[(b * L + t) * D + c0 + p];
        else if (conv_in)
          v = conv_in[(b * D + c0 + p) * (kTaps - 1) + (kTaps - 1) + t];
        conv_state_out[(b * D + c0 + p) * (kTaps - 1) + j] = v;
      }
    }
  }
}

template <typename T, int P>
hipError_t ssd_t(const SsmPrefillArgs& a, hipStream_t stream, Timing tm_state, Timing tm_carry, Timing tm_out) {
  const int nchunk = (a.L + kQ - 1) / kQ;
  const int H = a.d_inner / P;
  const dim3 grid((unsigned)nchunk, (unsigned)H, (unsigned)a.batch);
  HYMBA_LAUNCH((ssd_state_kernel<T, P>), grid, dim3(kSsdThreads), 0, stream, tm_state, (const T*)a.x, (const T*)a.dt,
               (const T*)a.B, a.A, a.conv_w, (const T*)a.conv_in, a.agg, a.sdt, a.L, a.d_inner, H, a.batch);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the carry chain over every chunk: carry[nchunk] is the final state
  e = launch_ssm_carry_chain(a.A, a.agg, a.sdt, a.state_in, a.carry, nchunk + 1, a.batch, a.d_inner, P, stream,
                             tm_carry);
  if (e != hipSuccess) return e;
  HYMBA_LAUNCH((ssd_out_kernel<T, P>), grid, dim3(kSsdThreads), 0, stream, tm_out, (const T*)a.x, (const T*)a.z,
               (const T*)a.dt, (const T*)a.B, (const T*)a.C, a.A, a.D, a.conv_w, (const T*)a.conv_in, a.carry,
               (T*)a.y, a.state_out, (T*)a.conv_state_out, a.L, a.d_inner, H, a.batch, nchunk);
  return hipGetLastError();
}

template <typename T>
hipError_t ssd_dispatch(const SsmPrefillArgs& a, hipStream_t stream, Timing t0, Timing t1, Timing t2) {
  switch (a.head_width) {
    case 32: return ssd_t<T, 32>(a, stream, t0, t1, t2);
    case 64: return ssd_t<T, 64>(a, stream, t0, t1, t2);
    case 128: return ssd_t<T, 128>(a, stream, t0, t1, t2);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int ssd_chunk_rows() { return kQ; }

hipError_t launch_ssd_prefill(const SsmPrefillArgs& a, hipStream_t stream, Timing tm_state, Timing tm_carry,
                              Timing tm_out) {
  if (a.act == HYMBA_BF16) return ssd_dispatch<bf16>(a, stream, tm_state, tm_carry, tm_out);
  return ssd_dispatch<float>(a, stream, tm_state, tm_carry, tm_out);
}

}  // namespace hymba
