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
//      leaves from a zero start (P x 16, a product over the chunk's rows on
//      the matrix cores) and its dt sum;
//   2. the chunk carry chain of the selective scan (ssm.hip), with one decay
//      rate per head, gives every chunk's entering state and the final state;
//   3. ssd_out_kernel: per (chunk, head, sequence), Y = [M | C exp(S)] x
//      [U ; H^T] on the matrix cores, M[i][j] = (C_i . B_j) exp(S_i - S_j) dt_j
//      on and below the diagonal (C B^T on the matrix cores, the decay on the
//      VALU, kept in registers), then D u and the silu(z) gate. In bf16 each
//      fp32 operand enters as a bf16 value plus its bf16 rounding error
//      (three products): Y and D u can nearly cancel when dt is large, and
//      one bf16 rounding of M and U would then show in y.
// The conv (4 taps, causal, per channel) is recomputed in both passes from x
// (and the carried history before row 0).
#include "common.hpp"
#include "launch.hpp"
#include "mma.hpp"

namespace hymba {

namespace {

constexpr int kQ = 64;         // rows per chunk
constexpr int kSt = 16;        // states
constexpr int kTaps = 4;       // conv taps
constexpr int kSsdThreads = 256;

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

// n 16-byte pieces straight into LDS, piece q at dst + 16 q, read from byte
// offset off(q) of descriptor r (an offset out of range reads zeros); the
// workgroup's waves take 64 pieces per load instruction in turn.
template <typename F>
__device__ __forceinline__ void stage_pieces(__amdgpu_buffer_rsrc_t r, char* dst, int n, int wave, int lane, F off) {
  for (int q0 = 64 * wave; q0 < n; q0 += kSsdThreads) {
    const int q = q0 + lane;
    if (q < n) buf_load16_lds(r, off(q), dst + 16 * q0);
  }
}

// The chunk's x rows t0 - 3 .. t0 + 63 of channels c0 .. c0 + P - 1, raw and
// row-major ([67][P]), into LDS at dst; rows before 0 and at or past L read
// zeros (rows before 0 are replaced by the carried history later, if any).
template <typename T, int P>
__device__ __forceinline__ void stage_x(const T* x, char* dst, int64_t b, int t0, int L, int D, int c0, int wave,
                                        int lane) {
  constexpr int E = Vec16<T>::n;
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(x + b * L * D, (uint32_t)((int64_t)L * D * sizeof(T)));
  stage_pieces(xrs, dst, (kQ + kTaps - 1) * (P / E), wave, lane, [&](int q) {
    const int t = t0 - (kTaps - 1) + q / (P / E);
    return t >= 0 ? (uint32_t)(((int64_t)t * D + c0 + (q % (P / E)) * E) * sizeof(T)) : kBufferNowhere;
  });
}

// Rows -3 .. -1 of chunk 0 from the carried history (raw x of those rows,
// oldest first); called once every wave's loads into LDS have landed, and
// followed by a barrier.
template <typename T, int P>
__device__ __forceinline__ void put_history(T (*xr)[P], const T* conv_in, int64_t b, int D, int c0, int tid) {
  for (int e = tid; e < (kTaps - 1) * P; e += kSsdThreads) {
    const int r = e / P, p = e % P;
    xr[r][p] = conv_in[(b * D + c0 + p) * (kTaps - 1) + r];
  }
}

// dt of row t0 + lane for head h (zero at or past L)
template <typename T>
__device__ __forceinline__ float load_dt(const T* dt, int64_t b, int t0, int L, int H, int h, int lane) {
  const __amdgpu_buffer_rsrc_t drs = make_rsrc(dt + b * L * H, (uint32_t)((int64_t)L * H * sizeof(T)));
  const uint32_t off = (uint32_t)(((int64_t)(t0 + lane) * H + h) * sizeof(T));
  if constexpr (sizeof(T) == 2)
    return __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(drs, off, 0, 0) << 16);
  else
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(drs, off, 0, 0));
}

// LDS of the state pass: the raw x rows (later the partial sums of the waves
// that share a channel tile), B transposed to [state][row], the row weights.
template <typename T, int P>
struct StateStage {
  static constexpr int kNT = P / 32;                 // 32-channel tiles
  static constexpr int kNK = 4 / kNT;                // waves per tile, each a share of the rows
  static constexpr int kBPitch = kQ + 8;             // B^T row pitch (elements)
  static constexpr int kXBytes = (kQ + kTaps - 1) * P * (int)sizeof(T);
  static constexpr int kRedBytes = (kNK - 1) * kNT * 64 * 8 * (int)sizeof(float);
  __attribute__((aligned(16))) char area[kXBytes > kRedBytes ? kXBytes : kRedBytes];
  __attribute__((aligned(16))) T bt[kSt][kBPitch];
  __attribute__((aligned(16))) float wj[kQ];        // dt_j exp(S_last - S_j)
  __device__ __forceinline__ T (*xr())[P] { return reinterpret_cast<T (*)[P]>(area); }
  __device__ __forceinline__ float (*red())[64][8] { return reinterpret_cast<float (*)[64][8]>(area); }
};

// Pass 1: agg[k][b][c][n] = sum_j exp(S_last - S_j) dt_j u_j[c] B_j[n] for the
// head's channels c, and sdt[k][b][c] = the chunk's dt sum. The sum over the
// chunk's rows is a product on the matrix cores with the states as rows (16
// of 32 used) and the channels as columns: a lane owns one channel and forms
// that channel's conv outputs for its operand rows itself, from registers,
// times the row weights; B^T is the other operand. In bf16 the weighted conv
// outputs enter as a bf16 pair (the value rounded, then the rounding error
// rounded), so the state keeps ~16 mantissa bits; B is exact in bf16. fp32
// uses fp32 products. With fewer than four 32-channel tiles the waves of a
// tile each take a share of the rows and their sums are added in LDS.
template <typename T, int P>
__global__ __launch_bounds__(kSsdThreads) void ssd_state_kernel(
    const T* __restrict__ x, const T* __restrict__ dt, const T* __restrict__ Bm, const float* __restrict__ A,
    const float* __restrict__ conv_w, const T* __restrict__ conv_in, float* __restrict__ agg,
    float* __restrict__ sdt, int L, int D, int H, int batch) {
  typedef Mma<T> M;
  typedef StateStage<T, P> S;
  constexpr int E = Vec16<T>::n;
  constexpr int NT = S::kNT, NK = S::kNK, KBW = 4 / NK;   // tiles, waves per tile, 16-row blocks per wave
  static_assert(kQ == 64 && NT * NK == 4, "four waves over the channel tiles and row shares");
  __shared__ S st;
  const int k = blockIdx.x, h = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lq = lane & 31, hh = lane >> 5;
  const int t0 = k * kQ;
  const int c0 = h * P;

  stage_x<T, P>(x, st.area, b, t0, L, D, c0, wave, lane);
  // B rows, 16 bytes per thread, written transposed
  const uint32_t rowb = kSt * sizeof(T);
  const __amdgpu_buffer_rsrc_t brs = make_rsrc(Bm + b * L * kSt, (uint32_t)L * rowb);
  constexpr int NBP = kQ * kSt / E;
  u32x4_t bv = {0u, 0u, 0u, 0u};
  if (tid < NBP) bv = buf_load16(brs, (uint32_t)t0 * rowb + 16u * tid);
  const float dtv = wave == 0 ? load_dt(dt, b, t0, L, H, h, lane) : 0.f;
  const int tp = wave % NT, ks = wave / NT;   // channel tile, share of the rows
  const int c = 32 * tp + lq;                 // this lane's channel (operand column)
  float w[kTaps];
#pragma unroll
  for (int j = 0; j < kTaps; ++j) w[j] = conv_w[(int64_t)(c0 + c) * kTaps + j];
  wait_loads();
  if (tid < NBP) {
    const int j = tid / (kSt / E), n0 = (tid % (kSt / E)) * E;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        st.bt[n0 + 2 * e][j] = bf16{(uint16_t)(bv[e] & 0xffffu)};
        st.bt[n0 + 2 * e + 1][j] = bf16{(uint16_t)(bv[e] >> 16)};
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) st.bt[n0 + e][j] = __uint_as_float(bv[e]);
    }
  }
  float total = 0.f;
  if (wave == 0) {
    const float cum = wave_scan(dtv, lane);
    const float s2 = A[h] * kLog2e * cum;
    st.wj[lane] = dtv * __builtin_amdgcn_exp2f(__shfl(s2, 63, 64) - s2);
    total = __shfl(cum, 63, 64);
  }
  lds_barrier();   // every wave's loads have landed
  if (t0 == 0 && conv_in) {
    put_history<T, P>(st.xr(), conv_in, b, D, c0, tid);
    lds_barrier();
  }

  // the product over this wave's 16-row blocks
  f32x16_t acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
  for (int kk = 0; kk < KBW; ++kk) {
    const int j0 = 16 * (ks * KBW + kk) + 8 * hh;   // operand rows j0 .. j0 + 7
    float xv[8 + kTaps - 1];
#pragma unroll
    for (int m = 0; m < 8 + kTaps - 1; ++m) xv[m] = to_f32(st.xr()[j0 + m][c]);
    const float4 wa = *reinterpret_cast<const float4*>(&st.wj[j0]);
    const float4 wb = *reinterpret_cast<const float4*>(&st.wj[j0 + 4]);
    const float wr[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
    float uv[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      float v = w[0] * xv[m];
#pragma unroll
      for (int j = 1; j < kTaps; ++j) v = fmaf(w[j], xv[m + j], v);
      uv[m] = v * wr[m];
    }
    typename M::Frag fb = M::frag_at(&st.bt[lq & (kSt - 1)][j0]);
    if (lq >= kSt) fb = M::zero();
    if constexpr (sizeof(T) == 2) {
      bf16x8_t uh, ul;
      split_bf16(uv, uh, ul);
      acc = M::mma(fb, uh, acc);
      acc = M::mma(fb, ul, acc);
    } else {
      acc = M::mma(fb, M::from_f32(uv), acc);
    }
  }
  // acc[r] for r < 8: state 8 (r / 4) + 4 hh + r % 4 of channel c
  const int64_t row0 = ((int64_t)k * batch + b) * D + c0;   // (chunk, sequence, first channel of the head)
  if constexpr (NK > 1) {
    lds_barrier();   // every x read is done: the partial sums take the area
    if (ks > 0) {
#pragma unroll
      for (int r = 0; r < 8; ++r) st.red()[(ks - 1) * NT + tp][lane][r] = acc[r];
    }
    lds_barrier();
    if (ks == 0) {
#pragma unroll
      for (int q = 1; q < NK; ++q)
#pragma unroll
        for (int r = 0; r < 8; ++r) acc[r] += st.red()[(q - 1) * NT + tp][lane][r];
    }
  }
  if (ks == 0) {
    float4* dst = reinterpret_cast<float4*>(agg + (row0 + c) * kSt + 4 * hh);
    dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    dst[2] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
  if (wave == 0) {
    for (int p = lane; p < P; p += 64) sdt[row0 + p] = total;
  }
}

// LDS of the output pass. The raw x rows and, once the conv has consumed
// them, its output u share one area; u is stored transposed, [channel][row],
// in bf16 as the value rounded and its rounding error rounded.
template <typename T, int P>
struct OutStage {
  static constexpr int kUPitch = kQ + 4;                   // u row pitch (elements)
  static constexpr int kParts = sizeof(T) == 2 ? 2 : 1;
  static constexpr int kXBytes = (kQ + kTaps - 1) * P * (int)sizeof(T);
  static constexpr int kUBytes = kParts * P * kUPitch * (int)sizeof(T);
  __attribute__((aligned(16))) char area[kXBytes > kUBytes ? kXBytes : kUBytes];
  __attribute__((aligned(16))) T bs[kQ][kSt];   // B rows of the chunk, as loaded
  __attribute__((aligned(16))) T cs[kQ][kSt];   // C rows
  __attribute__((aligned(16))) float hs[P][kSt];   // entering state
  __attribute__((aligned(16))) float s2[kQ];    // A log2(e) (dt_0 + .. + dt_j)
  __attribute__((aligned(16))) float dts[kQ];   // dt_j
  __device__ __forceinline__ T (*xr())[P] { return reinterpret_cast<T (*)[P]>(area); }
  __device__ __forceinline__ T (*u(int part))[kUPitch] {
    return reinterpret_cast<T (*)[kUPitch]>(area + part * P * kUPitch * (int)sizeof(T));
  }
};

// 8 operand values of row `row` of u at rows j0 .. j0 + 3 and j0 + 8 .. j0 + 11
template <typename T, int P>
__device__ __forceinline__ typename Mma<T>::Frag u_frag(OutStage<T, P>& st, int part, int row, int j0) {
  if constexpr (sizeof(T) == 2) {
    const u32x2_t a = *reinterpret_cast<const u32x2_t*>(&st.u(part)[row][j0]);
    const u32x2_t b = *reinterpret_cast<const u32x2_t*>(&st.u(part)[row][j0 + 8]);
    return __builtin_bit_cast(bf16x8_t, u32x4_t{a.x, a.y, b.x, b.y});
  } else {
    const float4 a = *reinterpret_cast<const float4*>(&st.u(part)[row][j0]);
    const float4 b = *reinterpret_cast<const float4*>(&st.u(part)[row][j0 + 8]);
    F32x8 f;
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
    return f;
  }
}

// Pass 3: the chunk's outputs from its entering state carry[k] (see above).
// The chunk's x rows (with three rows of history), B and C rows and entering
// state load straight into LDS. Each thread forms the conv output of one
// channel over a run of consecutive rows from registers. Each wave owns a
// 32-row block of Y (rows i) and one or two 32-channel tiles: it forms the
// decayed C B^T blocks that row block needs on the matrix cores with the
// operands swapped, so that a lane holds row i of M and the result is already
// the next product's A operand; the U operand takes the rows j in the same
// order. The gate inputs z load while the products run.
template <typename T, int P>
__global__ __launch_bounds__(kSsdThreads) void ssd_out_kernel(
    const T* __restrict__ x, const T* __restrict__ z, const T* __restrict__ dt, const T* __restrict__ Bm,
    const T* __restrict__ Cm, const float* __restrict__ A, const float* __restrict__ Dp,
    const float* __restrict__ conv_w, const T* __restrict__ conv_in, const float* __restrict__ carry,
    T* __restrict__ y, float* __restrict__ state_out, T* __restrict__ conv_state_out, int L, int D, int H,
    int batch, int nchunk) {
  typedef Mma<T> M;
  typedef OutStage<T, P> S;
  constexpr int E = Vec16<T>::n;                 // elements per 16-byte piece
  constexpr int NTP = P / 32;                    // 32-channel tiles
  constexpr int TPW = NTP > 1 ? NTP / 2 : 1;     // tiles per wave
  constexpr int RB = kQ * P / kSsdThreads;       // conv rows per thread
  static_assert(kQ == 64 && NTP >= 1 && NTP <= 4 && RB % 4 == 0, "two 32-row blocks; whole row runs per thread");
  __shared__ S st;
  const int k = blockIdx.x, h = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lq = lane & 31, hh = lane >> 5;
  const int t0 = k * kQ, nr = min(kQ, L - t0);
  const int c0 = h * P;

  // --- staging: x, B, C and the entering state into LDS; dt and the taps into registers
  {
    stage_x<T, P>(x, st.area, b, t0, L, D, c0, wave, lane);
    const uint32_t rowb = kSt * sizeof(T);
    const __amdgpu_buffer_rsrc_t brs = make_rsrc(Bm + b * L * kSt, (uint32_t)L * rowb);
    const __amdgpu_buffer_rsrc_t crs = make_rsrc(Cm + b * L * kSt, (uint32_t)L * rowb);
    auto bc_off = [&](int q) { return (uint32_t)t0 * rowb + 16u * q; };
    stage_pieces(brs, reinterpret_cast<char*>(&st.bs[0][0]), kQ * kSt / E, wave, lane, bc_off);
    stage_pieces(crs, reinterpret_cast<char*>(&st.cs[0][0]), kQ * kSt / E, wave, lane, bc_off);
    const __amdgpu_buffer_rsrc_t hrs =
        make_rsrc(carry + (((int64_t)k * batch + b) * D + c0) * kSt, (uint32_t)(P * kSt * sizeof(float)));
    stage_pieces(hrs, reinterpret_cast<char*>(&st.hs[0][0]), P * kSt / 4, wave, lane,
                 [](int q) { return 16u * q; });
  }
  const float dtv = wave == 0 ? load_dt(dt, b, t0, L, H, h, lane) : 0.f;
  const int cp = tid % P, rb = tid / P;          // conv: channel, run of rows
  float w[kTaps];
#pragma unroll
  for (int j = 0; j < kTaps; ++j) w[j] = conv_w[(int64_t)(c0 + cp) * kTaps + j];
  wait_loads();
  if (wave == 0) {
    const float cum = wave_scan(dtv, lane);
    st.dts[lane] = dtv;
    st.s2[lane] = A[h] * kLog2e * cum;
  }
  lds_barrier();   // every wave's loads have landed
  if (t0 == 0 && conv_in) {
    put_history<T, P>(st.xr(), conv_in, b, D, c0, tid);
    lds_barrier();
  }

  // --- the wave's tiles and their gate inputs (in flight from here to the epilogue)
  const bool active = NTP > 1 || wave < 2;
  const int ti = NTP > 1 ? wave >> 1 : wave & 1;
  const int tp0 = NTP > 1 ? (wave & 1) * TPW : 0;
  const int ia = 32 * ti + lq;                   // this lane's row of M (A operand)
  const uint32_t rowb = (uint32_t)(D * sizeof(T));
  const __amdgpu_buffer_rsrc_t zrs = make_rsrc(z + (b * L + t0) * D, (uint32_t)nr * rowb);
  float zv[TPW][16];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    const uint32_t col = (uint32_t)((c0 + 32 * (tp0 + tt) + lq) * sizeof(T));
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = 32 * ti + 8 * (r >> 2) + 4 * hh + (r & 3);
      const uint32_t off = active ? (uint32_t)i * rowb + col : kBufferNowhere;
      if constexpr (sizeof(T) == 2)
        zv[tt][r] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(zrs, off, 0, 0) << 16);
      else
        zv[tt][r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(zrs, off, 0, 0));
    }
  }

  // --- conv: channel cp, rows rb RB .. rb RB + RB - 1, from registers
  float uv[RB];
  {
    float xv[RB + kTaps - 1];
#pragma unroll
    for (int m = 0; m < RB + kTaps - 1; ++m) xv[m] = to_f32(st.xr()[rb * RB + m][cp]);
#pragma unroll
    for (int m = 0; m < RB; ++m) {
      float v = w[0] * xv[m];
#pragma unroll
      for (int j = 1; j < kTaps; ++j) v = fmaf(w[j], xv[m + j], v);
      uv[m] = v;
    }
  }
  lds_barrier();   // every x read is done: u takes the area
#pragma unroll
  for (int m = 0; m < RB; m += 4) {
    if constexpr (sizeof(T) == 2) {
      float hi[4], lo[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        hi[e] = __uint_as_float((uint32_t)f32_to_bf16_bits(uv[m + e]) << 16);
        lo[e] = uv[m + e] - hi[e];
      }
      *reinterpret_cast<u32x2_t*>(&st.u(0)[cp][rb * RB + m]) = u32x2_t{pack_bf16x2(hi[0], hi[1]), pack_bf16x2(hi[2], hi[3])};
      *reinterpret_cast<u32x2_t*>(&st.u(1)[cp][rb * RB + m]) = u32x2_t{pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3])};
    } else {
      *reinterpret_cast<float4*>(&st.u(0)[cp][rb * RB + m]) = make_float4(uv[m], uv[m + 1], uv[m + 2], uv[m + 3]);
    }
  }
  lds_barrier();

  if (active) {
    f32x16_t acc[TPW];
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[tt][r] = 0.f;
    const float s2i = st.s2[ia];
    for (int tj = 0; tj <= ti; ++tj) {
      // M^T block (rows j of block tj, columns i of block ti): B_j . C_i
      f32x16_t g;
#pragma unroll
      for (int r = 0; r < 16; ++r) g[r] = 0.f;
      g = M::mma(M::frag_at(&st.bs[32 * tj + lq][8 * hh]), M::frag_at(&st.cs[ia][8 * hh]), g);
      float mv[16];   // M[i][j] for this lane's i and j = 32 tj + 8 (r / 4) + 4 hh + r % 4
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j4 = 32 * tj + 8 * q + 4 * hh;
        const float4 s2j = *reinterpret_cast<const float4*>(&st.s2[j4]);
        const float4 dj = *reinterpret_cast<const float4*>(&st.dts[j4]);
        const float sj[4] = {s2j.x, s2j.y, s2j.z, s2j.w}, djv[4] = {dj.x, dj.y, dj.z, dj.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          mv[4 * q + e] = (tj < ti || j4 + e <= ia) ? g[4 * q + e] * __builtin_amdgcn_exp2f(s2i - sj[e]) * djv[e] : 0.f;
      }
      // Y += M U over the block's rows j, 16 at a time
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2) {
        const int j0 = 32 * tj + 16 * q2 + 4 * hh;
        if constexpr (sizeof(T) == 2) {
          bf16x8_t ah, al;
          split_bf16(&mv[8 * q2], ah, al);
#pragma unroll
          for (int tt = 0; tt < TPW; ++tt) {
            const int pb = 32 * (tp0 + tt) + lq;
            const bf16x8_t uh = u_frag(st, 0, pb, j0), ul = u_frag(st, 1, pb, j0);
            acc[tt] = M::mma(ah, uh, acc[tt]);
            acc[tt] = M::mma(ah, ul, acc[tt]);
            acc[tt] = M::mma(al, uh, acc[tt]);
          }
        } else {
          const typename M::Frag a = M::from_f32(&mv[8 * q2]);
#pragma unroll
          for (int tt = 0; tt < TPW; ++tt) acc[tt] = M::mma(a, u_frag(st, 0, 32 * (tp0 + tt) + lq, j0), acc[tt]);
        }
      }
    }
    // the entering state: rows of C scaled by exp(S_i), against H^T
    const float es = __builtin_amdgcn_exp2f(s2i);
    float cv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) cv[e] = to_f32(st.cs[ia][8 * hh + e]) * es;
    const __amdgpu_buffer_rsrc_t yrs = make_rsrc(y + (b * L + t0) * D, (uint32_t)nr * rowb);
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
      const int pb = 32 * (tp0 + tt) + lq;
      acc[tt] = mma_split<T>(cv, &st.hs[pb][8 * hh], acc[tt]);
      const float Dc = Dp[c0 + pb];
      const uint32_t col = (uint32_t)((c0 + pb) * sizeof(T));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i4 = 32 * ti + 8 * q + 4 * hh;
        float u4[4];
        if constexpr (sizeof(T) == 2) {
          const u32x2_t a = *reinterpret_cast<const u32x2_t*>(&st.u(0)[pb][i4]);
          const u32x2_t l = *reinterpret_cast<const u32x2_t*>(&st.u(1)[pb][i4]);
          u4[0] = bf16_lo(a.x) + bf16_lo(l.x); u4[1] = bf16_hi(a.x) + bf16_hi(l.x);
          u4[2] = bf16_lo(a.y) + bf16_lo(l.y); u4[3] = bf16_hi(a.y) + bf16_hi(l.y);
        } else {
          const float4 a = *reinterpret_cast<const float4*>(&st.u(0)[pb][i4]);
          u4[0] = a.x; u4[1] = a.y; u4[2] = a.z; u4[3] = a.w;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * q + e;
          buf_store(yrs, (uint32_t)(i4 + e) * rowb + col, from_f32<T>(fmaf(Dc, u4[e], acc[tt][r]) * ssd_silu(zv[tt][r])));
        }
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
