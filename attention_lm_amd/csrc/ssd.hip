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
//      In bf16 each fp32 operand enters as a bf16 value plus its bf16
//      rounding error (three products): Y and D u can nearly cancel when dt
//      is large, and one bf16 rounding of M and U would then show in y.
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

// What both passes stage for chunk k of head h of sequence b, in LDS: per
// row, dt and S (log2 units: A log2(e) times the running dt sum); the conv
// input rows t0 - 3 .. t0 + 63 of the head's channels (fp32); the conv taps;
// the chunk's B rows (and, for the output pass, C rows).
template <typename T, int P>
struct ChunkIn {
  // (rows enough for the output pass to place its 64 x 68 M block, and the
  // state pass its P x 68 transposed conv output, here once the x rows are dead)
  static constexpr int kDead = (kQ > P ? kQ : P) * (kQ + kRowPad);
  static constexpr int kXRows = (kQ + kTaps - 1) > (kDead + P - 1) / P ? (kQ + kTaps - 1) : (kDead + P - 1) / P;
  float xs[kXRows][P];
  float bs[kQ][kSt];
  float s2[kQ], dts[kQ];
  float cw[P][kTaps];
  float total;   // dt sum over the chunk
};

// Global loads of a chunk, issued together into registers (buffer loads: rows
// at or past L read zeros), then written to LDS by commit().
template <typename T, int P>
struct ChunkLoads {
  static constexpr int E = Vec16<T>::n;                          // elements per 16-byte load
  static constexpr int XV = P / E;                                // 16-byte pieces per x row
  static constexpr int NX = ((kQ + kTaps - 1) * XV + kSsdThreads - 1) / kSsdThreads;
  static constexpr int BV = kSt / E;                              // pieces per B/C row
  static constexpr int NB = (kQ * BV + kSsdThreads - 1) / kSsdThreads;
  u32x4_t xv[NX], bv[NB], cv[NB];
  float dt;

  __device__ __forceinline__ void issue(const T* x, const T* dtp, const T* Bm, const T* Cm, int64_t b, int h,
                                        int t0, int L, int D, int H, bool with_c) {
    const int tid = threadIdx.x;
    const int c0 = h * P;
    const __amdgpu_buffer_rsrc_t xrs = make_rsrc(x + b * L * D, (uint32_t)((int64_t)L * D * sizeof(T)));
#pragma unroll
    for (int q = 0; q < NX; ++q) {
      const int it = tid + q * kSsdThreads, r = it / XV, v = it % XV, t = t0 - (kTaps - 1) + r;
      const bool ok = it < (kQ + kTaps - 1) * XV && t >= 0;
      xv[q] = buf_load16(xrs, ok ? (uint32_t)(((int64_t)t * D + c0 + v * E) * sizeof(T)) : kBufferNowhere);
    }
    const uint32_t rowb = kSt * sizeof(T);
    const __amdgpu_buffer_rsrc_t brs = make_rsrc(Bm + b * L * kSt, (uint32_t)L * rowb);
    const __amdgpu_buffer_rsrc_t crs = make_rsrc(Cm + b * L * kSt, (uint32_t)L * rowb);
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      const int it = tid + q * kSsdThreads, j = it / BV, v = it % BV;
      const uint32_t off = it < kQ * BV ? (uint32_t)(t0 + j) * rowb + 16u * v : kBufferNowhere;
      bv[q] = buf_load16(brs, off);
      if (with_c) cv[q] = buf_load16(crs, off);
    }
    const __amdgpu_buffer_rsrc_t drs = make_rsrc(dtp + b * L * H, (uint32_t)((int64_t)L * H * sizeof(T)));
    dt = 0.f;
    if (tid < 64) {
      const uint32_t off = (uint32_t)(((int64_t)(t0 + tid) * H + h) * sizeof(T));
      if constexpr (sizeof(T) == 2)
        dt = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(drs, off, 0, 0) << 16);
      else
        dt = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(drs, off, 0, 0));
    }
  }

  __device__ __forceinline__ static void unpack(u32x4_t w, float* o) {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) { o[2 * e] = bf16_lo(w[e]); o[2 * e + 1] = bf16_hi(w[e]); }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = __uint_as_float(w[e]);
    }
  }

  // LDS writes; rows before row 0 come from the carried history when given
  __device__ __forceinline__ void commit(ChunkIn<T, P>& ci, float (*cs)[kSt], const float* A, const float* conv_w,
                                         const T* conv_in, int64_t b, int h, int t0, int D) {
    const int tid = threadIdx.x;
    const int c0 = h * P;
#pragma unroll
    for (int q = 0; q < NX; ++q) {
      const int it = tid + q * kSsdThreads, r = it / XV, v = it % XV, t = t0 - (kTaps - 1) + r;
      if (it < (kQ + kTaps - 1) * XV) {
        float f[E];
        unpack(xv[q], f);
        if (t < 0 && conv_in) {
#pragma unroll
          for (int e = 0; e < E; ++e)
            f[e] = to_f32(conv_in[(b * D + c0 + v * E + e) * (kTaps - 1) + (kTaps - 1) + t]);
        }
#pragma unroll
        for (int e = 0; e < E; ++e) ci.xs[r][v * E + e] = f[e];
      }
    }
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      const int it = tid + q * kSsdThreads, j = it / BV, v = it % BV;
      if (it < kQ * BV) {
        float f[E];
        unpack(bv[q], f);
#pragma unroll
        for (int e = 0; e < E; ++e) ci.bs[j][v * E + e] = f[e];
        if (cs) {
          unpack(cv[q], f);
#pragma unroll
          for (int e = 0; e < E; ++e) cs[j][v * E + e] = f[e];
        }
      }
    }
    if (tid < 64) {
      const float cum = wave_scan(dt, tid);
      ci.dts[tid] = dt;
      ci.s2[tid] = A[h] * kLog2e * cum;
      if (tid == 63) ci.total = cum;
    }
    for (int e = tid; e < P * kTaps; e += kSsdThreads) ci.cw[e / kTaps][e % kTaps] = conv_w[(int64_t)c0 * kTaps + e];
  }
};

// An fp32 operand fragment (8 values) as two bf16 fragments: the values
// rounded, then their rounding errors rounded. A product from the three
// parts hi.hi + hi.lo + lo.hi keeps about 16 mantissa bits of each operand.
__device__ __forceinline__ void split_bf16(const float* v, bf16x8_t& hi, bf16x8_t& lo) {
  float h[8], l[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    h[t] = __uint_as_float((uint32_t)f32_to_bf16_bits(v[t]) << 16);
    l[t] = v[t] - h[t];
  }
  hi = Mma<bf16>::from_f32(h);
  lo = Mma<bf16>::from_f32(l);
}
// acc += A B^T for fp32 operand fragments a, b: in bf16, from their split
// parts (three products); in fp32, one fp32 product.
template <typename T>
__device__ __forceinline__ f32x16_t mma_split(const float* a, const float* b, f32x16_t acc) {
  if constexpr (sizeof(T) == 2) {
    bf16x8_t ah, al, bh, bl;
    split_bf16(a, ah, al);
    split_bf16(b, bh, bl);
    acc = Mma<bf16>::mma(ah, bh, acc);
    acc = Mma<bf16>::mma(ah, bl, acc);
    return Mma<bf16>::mma(al, bh, acc);
  } else {
    return Mma<float>::mma(Mma<float>::from_f32(a), Mma<float>::from_f32(b), acc);
  }
}

template <typename T, int P>
__device__ __forceinline__ float conv_at(const ChunkIn<T, P>& ci, int j, int p) {
  float u = 0.f;
#pragma unroll
  for (int k = 0; k < kTaps; ++k) u = fmaf(ci.cw[p][k], ci.xs[j + k][p], u);
  return u;
}

// Pass 1: agg[k][b][c][n] = sum_j exp(S_last - S_j) dt_j u_j[c] B_j[n] for the
// head's channels c, and sdt[k][b][c] = the chunk's dt sum. The conv output of
// each (row, channel), times its row weight, is formed once (into LDS, where
// the staged x rows were, transposed to [channel][row]); the sum over rows is
// a P x 16 product on the matrix cores, one 32-channel tile per wave. In bf16
// the weighted conv outputs enter as a bf16 pair (the value rounded, then the
// rounding error rounded), so the state keeps ~16 mantissa bits; B is exact
// in bf16. fp32 uses fp32 products.
template <typename T, int P>
__global__ __launch_bounds__(kSsdThreads) void ssd_state_kernel(
    const T* __restrict__ x, const T* __restrict__ dt, const T* __restrict__ Bm, const float* __restrict__ A,
    const float* __restrict__ conv_w, const T* __restrict__ conv_in, float* __restrict__ agg,
    float* __restrict__ sdt, int L, int D, int H, int batch) {
  typedef Mma<T> M;
  constexpr int NU = kQ * P / kSsdThreads;   // conv outputs per thread
  static_assert(kQ * P % kSsdThreads == 0 && P / 32 <= kSsdThreads / 64, "one 32-channel tile per wave");
  __shared__ ChunkIn<T, P> ci;
  __shared__ float wj[kQ];   // dt_j exp(S_last - S_j)
  const int k = blockIdx.x, h = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lq = lane & 31, hh = lane >> 5;
  const int t0 = k * kQ;
  {
    ChunkLoads<T, P> ld;
    ld.issue(x, dt, Bm, nullptr, b, h, t0, L, D, H, false);
    ld.commit(ci, nullptr, A, conv_w, conv_in, b, h, t0, D);
  }
  __syncthreads();
  if (tid < kQ) wj[tid] = ci.dts[tid] * __builtin_amdgcn_exp2f(ci.s2[kQ - 1] - ci.s2[tid]);
  __syncthreads();
  float u[NU];
#pragma unroll
  for (int i = 0; i < NU; ++i) {
    const int e = tid + i * kSsdThreads, j = e / P, p = e % P;
    u[i] = conv_at(ci, j, p) * wj[j];
  }
  __syncthreads();   // the staged x rows are dead: U^T takes their place
  typedef float URow[kQ + kRowPad];
  URow* const ut = reinterpret_cast<URow*>(&ci.xs[0][0]);
#pragma unroll
  for (int i = 0; i < NU; ++i) {
    const int e = tid + i * kSsdThreads, j = e / P, p = e % P;
    ut[p][j] = u[i];
  }
  __syncthreads();
  const int c0 = h * P;
  const int64_t row0 = ((int64_t)k * batch + b) * D + c0;   // (chunk, sequence, first channel of the head)
  if (wave < P / 32) {
    // rows of the product: channels 32 wave + lq; columns: states lq (< 16)
    f32x16_t acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < kQ / 16; ++ks) {
      const int j0 = 16 * ks + 8 * hh;
      float bv[8], av[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) bv[t] = lq < kSt ? ci.bs[j0 + t][lq] : 0.f;
#pragma unroll
      for (int t = 0; t < 8; ++t) av[t] = ut[32 * wave + lq][j0 + t];
      const typename M::Frag fb = M::from_f32(bv);
      if constexpr (sizeof(T) == 2) {
        float hi[8], lo[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          hi[t] = __uint_as_float((uint32_t)f32_to_bf16_bits(av[t]) << 16);
          lo[t] = av[t] - hi[t];
        }
        acc = M::mma(M::from_f32(hi), fb, acc);
        acc = M::mma(M::from_f32(lo), fb, acc);
      } else {
        acc = M::mma(M::from_f32(av), fb, acc);
      }
    }
    if (lq < kSt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int p = 32 * wave + 8 * (r >> 2) + 4 * hh + (r & 3);
        agg[(row0 + p) * kSt + lq] = acc[r];
      }
    }
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
  constexpr int NTP = P / 32;
  __shared__ ChunkIn<T, P> ci;
  __shared__ __attribute__((aligned(16))) float ut[P][kQ + kRowPad];   // u, [channel][row]
  __shared__ __attribute__((aligned(16))) float cs[kQ][kSt];
  __shared__ __attribute__((aligned(16))) float hs[P][kSt];            // entering state
  const int k = blockIdx.x, h = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lq = lane & 31, hh = lane >> 5;
  const int t0 = k * kQ, nr = min(kQ, L - t0);
  const int c0 = h * P;
  {
    ChunkLoads<T, P> ld;
    ld.issue(x, dt, Bm, Cm, b, h, t0, L, D, H, true);
    const float4* hin = reinterpret_cast<const float4*>(carry + (((int64_t)k * batch + b) * D + c0) * kSt);
    float4 hv[(P * kSt / 4 + kSsdThreads - 1) / kSsdThreads];
#pragma unroll
    for (int q = 0; q < (int)(sizeof(hv) / sizeof(hv[0])); ++q) {
      const int it = tid + q * kSsdThreads;
      if (it < P * kSt / 4) hv[q] = hin[it];
    }
    ld.commit(ci, cs, A, conv_w, conv_in, b, h, t0, D);
#pragma unroll
    for (int q = 0; q < (int)(sizeof(hv) / sizeof(hv[0])); ++q) {
      const int it = tid + q * kSsdThreads;
      if (it < P * kSt / 4) reinterpret_cast<float4*>(&hs[0][0])[it] = hv[q];
    }
  }
  __syncthreads();
  // u, transposed to [channel][row]
  for (int e = tid; e < kQ * P; e += kSsdThreads) {
    const int j = e / P, p = e % P;
    ut[p][j] = conv_at(ci, j, p);
  }
  __syncthreads();   // the staged x rows are dead: M takes their place
  typedef float MRow[kQ + kRowPad];
  static_assert(sizeof(ci.xs) >= sizeof(float) * kQ * (kQ + kRowPad), "M fits where x was staged");
  MRow* const ms = reinterpret_cast<MRow*>(&ci.xs[0][0]);
  // M = C B^T on the matrix cores (one 32 x 32 tile per wave), masked below
  // the diagonal and decayed: M[i][j] = (C_i . B_j) exp(S_i - S_j) dt_j
  {
    const int ti = wave >> 1, tj = wave & 1;
    f32x16_t g;
#pragma unroll
    for (int r = 0; r < 16; ++r) g[r] = 0.f;
    if (tj <= ti) g = M::mma(M::from_f32(&cs[32 * ti + lq][8 * hh]), M::from_f32(&ci.bs[32 * tj + lq][8 * hh]), g);
    const int j = 32 * tj + lq;
    const float s2j = ci.s2[j], dtj = ci.dts[j];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = 32 * ti + 8 * (r >> 2) + 4 * hh + (r & 3);
      ms[i][j] = j <= i ? g[r] * __builtin_amdgcn_exp2f(ci.s2[i] - s2j) * dtj : 0.f;
    }
  }
  // this lane's gate inputs, loaded while the block products run
  const uint32_t rowb = (uint32_t)(D * sizeof(T));
  const __amdgpu_buffer_rsrc_t zrs = make_rsrc(z + (b * L + t0) * D, (uint32_t)nr * rowb);
  const __amdgpu_buffer_rsrc_t yrs = make_rsrc(y + (b * L + t0) * D, (uint32_t)nr * rowb);
  __syncthreads();
  // Y tiles of 32 rows x 32 channels, one per wave in turn
  for (int tile = wave; tile < 2 * NTP; tile += kSsdThreads / 64) {
    const int ti = tile / NTP, tp = tile % NTP;
    const int ia = 32 * ti + lq, pb = 32 * tp + lq;   // this lane's A row and B column
    const uint32_t col = (uint32_t)((c0 + pb) * sizeof(T));
    float zv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = 32 * ti + 8 * (r >> 2) + 4 * hh + (r & 3);
      const uint32_t off = (uint32_t)i * rowb + col;
      if constexpr (sizeof(T) == 2)
        zv[r] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(zrs, off, 0, 0) << 16);
      else
        zv[r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(zrs, off, 0, 0));
    }
    f32x16_t acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
    for (int kb = 0; kb < kQ / 16; ++kb) {
      if (kb <= (2 * ti + 1))   // key blocks past this tile's last row are all zero
        acc = mma_split<T>(&ms[ia][16 * kb + 8 * hh], &ut[pb][16 * kb + 8 * hh], acc);
    }
    {   // the entering state: rows of C scaled by exp(S_i), against H^T
      const float es = __builtin_amdgcn_exp2f(ci.s2[ia]);
      float cv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) cv[e] = cs[ia][8 * hh + e] * es;
      acc = mma_split<T>(cv, &hs[pb][8 * hh], acc);
    }
    const float Dc = Dp[c0 + pb];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = 32 * ti + 8 * (r >> 2) + 4 * hh + (r & 3);
      buf_store(yrs, (uint32_t)i * rowb + col, from_f32<T>(fmaf(Dc, ut[pb][i], acc[r]) * ssd_silu(zv[r])));
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
