// Attention branch: rotary embedding, prefill flash attention on the matrix
// cores, and split-key decode attention over a read-only (shareable) KV cache.
//
// Attention is softmax(q k^T / sqrt(d_k)) v ("Jamba: Hybrid SSM-Transformer",
// "1. Layer Interleaving Ratio"), grouped-query (GQA) with RoPE (51cto
// Hymba-1.5B article, section 2), over the visibility rule in common.hpp:
// meta-token rows visible to all later rows, plus a sliding window or, in a
// global layer, every earlier row.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace hymba {

namespace {

constexpr int kHd = 64;                 // query/key head width
constexpr float kScaleLog2e = 0.125f * kLog2e;  // 1/sqrt(64) folded with log2(e)

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 8 consecutive elements <-> fp32
__device__ __forceinline__ void load8(const bf16* p, float* o) { load16(p, o); }
__device__ __forceinline__ void load8(const float* p, float* o) { load16(p, o); load16(p + 4, o + 4); }
__device__ __forceinline__ void store8(bf16* p, const float* o) { store16(p, o); }
__device__ __forceinline__ void store8(float* p, const float* o) { store16(p, o); store16(p + 4, o + 4); }
__device__ __forceinline__ void copy8(const bf16* s, bf16* d) {
  *reinterpret_cast<uint4*>(d) = *reinterpret_cast<const uint4*>(s);
}
__device__ __forceinline__ void copy8(const float* s, float* d) {
  *reinterpret_cast<float4*>(d) = *reinterpret_cast<const float4*>(s);
  *reinterpret_cast<float4*>(d + 4) = *reinterpret_cast<const float4*>(s + 4);
}

// cos/sin of pos * base^(-2i/64), angle formed and reduced in fp64.
__device__ __forceinline__ void rope_cs(int pos, int i, float base, float* c, float* s) {
  const double inv_freq = pow((double)base, -2.0 * (double)i / (double)kHd);
  const double ang = (double)pos * inv_freq;
  double sd, cd;
  sincos(ang, &sd, &cd);
  *c = (float)cd;
  *s = (float)sd;
}

// ---------------------------------------------------------------------------
// RoPE prologue (prefill): q -> q_rot, k -> k_rot (e.g. straight into the KV
// cache), optionally v -> v_copy. Rotate-half pairs (i, i+32).

constexpr int kRopeRows = 8;

template <typename T>
__global__ __launch_bounds__(256) void rope_prefill_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, T* __restrict__ q_rot,
    T* __restrict__ k_rot, T* __restrict__ v_copy, int64_t k_rows, int64_t v_rows, int L, int Hq, int Hkv,
    int dv, float base) {
  __shared__ float cs[kRopeRows][kHd / 2];
  __shared__ float sn[kRopeRows][kHd / 2];
  const int r0 = blockIdx.x * kRopeRows;
  const int64_t b = blockIdx.y;
  for (int t = threadIdx.x; t < kRopeRows * (kHd / 2); t += blockDim.x) {
    const int r = t / (kHd / 2), i = t % (kHd / 2);
    rope_cs(r0 + r, i, base, &cs[r][i], &sn[r][i]);
  }
  __syncthreads();
  const int nrows = min(kRopeRows, L - r0);
  // rotation work items: (row, head, group of 8 pairs); heads 0..Hq-1 are q, then k
  const int H = Hq + Hkv;
  const int items = nrows * H * 4;
  for (int it = threadIdx.x; it < items; it += blockDim.x) {
    const int g8 = it & 3;
    const int hr = it >> 2;
    const int hd = hr % H;
    const int r = hr / H;
    const int row = r0 + r;
    const T* src;
    T* dst;
    if (hd < Hq) {
      src = q + ((b * L + row) * Hq + hd) * kHd;
      dst = q_rot + ((b * L + row) * Hq + hd) * kHd;
    } else {
      src = k + ((b * L + row) * Hkv + (hd - Hq)) * kHd;
      dst = k_rot + ((b * k_rows + row) * Hkv + (hd - Hq)) * kHd;
    }
    float lo[8], hi[8], olo[8], ohi[8];
    load8(src + 8 * g8, lo);
    load8(src + 32 + 8 * g8, hi);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float c = cs[r][8 * g8 + e], s = sn[r][8 * g8 + e];
      olo[e] = lo[e] * c - hi[e] * s;
      ohi[e] = hi[e] * c + lo[e] * s;
    }
    store8(dst + 8 * g8, olo);
    store8(dst + 32 + 8 * g8, ohi);
  }
  if (v_copy) {
    const int per_row = Hkv * dv / 8;
    for (int it = threadIdx.x; it < nrows * per_row; it += blockDim.x) {
      const int r = it / per_row, e = it % per_row;
      copy8(v + (b * L + r0 + r) * (int64_t)(Hkv * dv) + 8 * e, v_copy + (b * v_rows + r0 + r) * (int64_t)(Hkv * dv) + 8 * e);
    }
  }
}

// ---------------------------------------------------------------------------
// Prefill attention on the matrix cores.
//
// Workgroup = one (sequence, kv head, block of 32*PB query rows); one wave per
// (query head of the group, 32-row block). All its waves read the same key and
// value tiles, staged in LDS once per workgroup (GQA reuse).
//
// Per 32-key sub-tile each wave computes S^T = K Q^T with 32x32x16 bf16 MFMA
// (fp32 inputs: 32x32x2). In that layout each lane owns one query column and
// 16 keys, so softmax statistics need only one cross-lane step (lanes l and
// l+32) and the exp'd scores, converted in registers, are directly the B
// operand of O^T = V^T P^T: no LDS round trip for P. V is stored transposed in
// LDS with keys permuted inside each 16-key chunk to match that operand.
// Online softmax keeps running max m and per-lane partial sums l.

constexpr int BK = 64;                     // keys per LDS stage (two 32-key sub-tiles)
template <typename T> struct AttnTile {
  static constexpr int kpad = kHd + 16 / (int)sizeof(T);   // padded K row (elements)
  static constexpr int vpad = BK + 16 / (int)sizeof(T);    // padded V^T row (elements)
};

// slot s of a 16-key chunk holds key kperm(s); an involution
__device__ __forceinline__ int kperm(int s) { return (s & 3) | ((s & 4) << 1) | ((s & 8) >> 1); }

template <typename T>
struct Mma;
template <>
struct Mma<bf16> {
  typedef bf16x8_t Frag;   // 8 bf16 per lane
  static __device__ __forceinline__ Frag lds_frag(const bf16* p) {
    return __builtin_bit_cast(Frag, *reinterpret_cast<const uint4*>(p));
  }
  static __device__ __forceinline__ Frag from_f32(const float* v) {
    uint4 u;
    u.x = pack_bf16x2(v[0], v[1]); u.y = pack_bf16x2(v[2], v[3]);
    u.z = pack_bf16x2(v[4], v[5]); u.w = pack_bf16x2(v[6], v[7]);
    return __builtin_bit_cast(Frag, u);
  }
  static __device__ __forceinline__ f32x16_t mma(const Frag& a, const Frag& b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
struct F32x8 { float v[8]; };
template <>
struct Mma<float> {
  typedef F32x8 Frag;      // 8 fp32 per lane; slot t of lane half h is k = 8h + t
  static __device__ __forceinline__ Frag lds_frag(const float* p) {
    Frag f;
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = *reinterpret_cast<const float4*>(p + 4);
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
    return f;
  }
  static __device__ __forceinline__ Frag from_f32(const float* v) {
    Frag f;
#pragma unroll
    for (int t = 0; t < 8; ++t) f.v[t] = v[t];
    return f;
  }
  static __device__ __forceinline__ f32x16_t mma(const Frag& a, const Frag& b, f32x16_t c) {
#pragma unroll
    for (int t = 0; t < 8; ++t) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.v[t], b.v[t], c, 0, 0, 0);
    return c;
  }
};

template <typename T, int DV>
__global__ __launch_bounds__(640) void attn_prefill_kernel(
    const T* __restrict__ q_rot, const T* __restrict__ k_rot, const T* __restrict__ v, T* __restrict__ y,
    int64_t k_rows, int64_t v_rows, int L, int n_meta, int window, int Hq, int Hkv, int pb) {
  typedef Mma<T> M;
  typedef typename M::Frag Frag;
  constexpr int KP = AttnTile<T>::kpad;
  constexpr int VP = AttnTile<T>::vpad;
  constexpr int NDB = DV / 32;
  __shared__ __attribute__((aligned(16))) T Ks[2][BK][KP];
  __shared__ __attribute__((aligned(16))) T Vt[2][DV][VP];

  const int group = Hq / Hkv;
  const int nthreads = blockDim.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lq = lane & 31;   // query column / operand row of this lane
  const int hh = lane >> 5;   // lane half
  const int g = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int p0 = blockIdx.x * 32 * pb;
  const int p1 = min(p0 + 32 * pb, L);
  const int h = g * group + (wave % group);
  const int q0 = p0 + 32 * (wave / group);
  const int qa = q0, qb = min(q0 + 32, L);
  const int my_q = q0 + lq;

  // Q^T operand: lane holds Q[my_q][16 kc + 8 hh .. +7]
  Frag qf[4];
  {
    float tmp[8];
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      if (my_q < L) {
        load8(q_rot + ((b * L + my_q) * Hq + h) * kHd + 16 * kc + 8 * hh, tmp);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) tmp[e] = 0.f;
      }
      qf[kc] = M::from_f32(tmp);
    }
  }

  f32x16_t acc[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[d][r] = 0.f;
  float m_run = -INFINITY;  // running max of scaled scores (log2 units)
  float l_run = 0.f;        // this lane's partial sum

  // key tiles: meta part then window part
  const int meta_end = min(n_meta, p1);
  const int wb = window > 0 ? max(n_meta, p0 - window + 1) : n_meta;
  const int n1 = (meta_end + BK - 1) / BK;
  int k2s = wb / BK;
  const int k2e = (p1 + BK - 1) / BK;
  if (k2s < n1) k2s = n1;
  const int ntiles = n1 + max(0, k2e - k2s);

  const T* kbase = k_rot + (b * k_rows) * Hkv * kHd + g * kHd;
  const T* vbase = v + (b * v_rows) * Hkv * DV + g * DV;
  constexpr int KCH = kHd * (int)sizeof(T) / 16;  // 16-byte chunks per K row
  constexpr int E16 = 16 / (int)sizeof(T);

  auto load_tile = [&](int idx, int buf) {
    const int kt = idx < n1 ? idx : k2s + (idx - n1);
    const int j0 = kt * BK;
    for (int it = tid; it < BK * KCH; it += nthreads) {
      const int kk = it / KCH, ch = it % KCH;
      const int j = j0 + kk;
      uint4 val = make_uint4(0, 0, 0, 0);
      if (j < L) val = *reinterpret_cast<const uint4*>(kbase + (int64_t)j * Hkv * kHd + ch * E16);
      *reinterpret_cast<uint4*>(&Ks[buf][kk][ch * E16]) = val;
    }
    // V: item = (4-key quad, 8-wide dv chunk); written transposed, keys permuted
    constexpr int NQ = BK / 4, NC = DV / 8;
    for (int it = tid; it < NQ * NC; it += nthreads) {
      const int kq = it / NC, dc = it % NC;
      float vv[4][8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = j0 + 4 * kq + e;
        if (j < L) {
          load8(vbase + (int64_t)j * Hkv * DV + 8 * dc, vv[e]);
        } else {
#pragma unroll
          for (int t = 0; t < 8; ++t) vv[e][t] = 0.f;
        }
      }
      const int kk0 = 4 * kq;                       // first key of the quad within the stage
      const int col = (kk0 & ~15) + kperm(kk0 & 15);  // 4 contiguous slots
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        T* dst = &Vt[buf][8 * dc + t][col];
        if constexpr (sizeof(T) == 2) {
          uint2 w2;
          w2.x = pack_bf16x2(vv[0][t], vv[1][t]);
          w2.y = pack_bf16x2(vv[2][t], vv[3][t]);
          *reinterpret_cast<uint2*>(dst) = w2;
        } else {
          *reinterpret_cast<float4*>(dst) = make_float4(vv[0][t], vv[1][t], vv[2][t], vv[3][t]);
        }
      }
    }
  };

  if (ntiles > 0) load_tile(0, 0);
  __syncthreads();

  for (int idx = 0; idx < ntiles; ++idx) {
    const int buf = idx & 1;
    if (idx + 1 < ntiles) load_tile(idx + 1, buf ^ 1);
    const int kt = idx < n1 ? idx : k2s + (idx - n1);

#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int j0 = kt * BK + sub * 32;
      const int j1 = j0 + 32;
      // classify this 32x32 block for this wave
      if (qa >= qb) continue;
      const bool none = (j0 > qb - 1) ||
                        (window > 0 && j0 >= n_meta && qa - (j1 - 1) >= window);
      if (none) continue;
      const bool full = (j1 - 1 <= qa) &&
                        (window <= 0 || j1 <= n_meta || (qb - 1) - max(j0, n_meta) < window);

      f32x16_t s;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const Frag a = M::lds_frag(&Ks[buf][sub * 32 + lq][16 * kc + 8 * hh]);
        s = M::mma(a, qf[kc], s);
      }
      // scores of keys j0 + 8(r/4) + 4hh + (r%4), query my_q
      float mt = -INFINITY;
      if (full) {
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[r]);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = j0 + 8 * (r >> 2) + 4 * hh + (r & 3);
          const bool vis = my_q < L && key_visible(my_q, j, n_meta, window);
          s[r] = vis ? s[r] : -INFINITY;
          mt = fmaxf(mt, s[r]);
        }
      }
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      const float m_new = fmaxf(m_run, mt * kScaleLog2e);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      m_run = m_new;
      float p[16];
      float psum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = fast_exp2(fmaf(s[r], kScaleLog2e, -m_use));
        psum += p[r];
      }
      l_run = fmaf(l_run, alpha, psum);
#pragma unroll
      for (int d = 0; d < NDB; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[d][r] *= alpha;
      const Frag pf0 = M::from_f32(&p[0]);
      const Frag pf1 = M::from_f32(&p[8]);
#pragma unroll
      for (int d = 0; d < NDB; ++d) {
        const Frag va0 = M::lds_frag(&Vt[buf][32 * d + lq][sub * 32 + 0 + 8 * hh]);
        acc[d] = M::mma(va0, pf0, acc[d]);
        const Frag va1 = M::lds_frag(&Vt[buf][32 * d + lq][sub * 32 + 16 + 8 * hh]);
        acc[d] = M::mma(va1, pf1, acc[d]);
      }
    }
    __syncthreads();
  }

  // normalise and store: lane holds O[my_q][32 d + 8 jj + 4 hh + (0..3)]
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (my_q < L) {
    const float inv = 1.0f / l_tot;
    T* yrow = y + ((b * L + my_q) * Hq + h) * DV;
#pragma unroll
    for (int d = 0; d < NDB; ++d) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int col = 32 * d + 8 * jj + 4 * hh;
        const float o0 = acc[d][4 * jj + 0] * inv, o1 = acc[d][4 * jj + 1] * inv;
        const float o2 = acc[d][4 * jj + 2] * inv, o3 = acc[d][4 * jj + 3] * inv;
        if constexpr (sizeof(T) == 2) {
          uint2 w2;
          w2.x = pack_bf16x2(o0, o1);
          w2.y = pack_bf16x2(o2, o3);
          *reinterpret_cast<uint2*>(yrow + col) = w2;
        } else {
          *reinterpret_cast<float4*>(yrow + col) = make_float4(o0, o1, o2, o3);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Decode attention: one workgroup per (split of the visible keys, kv head,
// sequence). The visible keys of position p are the meta rows and the window
// rows of the cache plus the new row p itself; they are numbered meta first,
// then window, and split into chunks of kKeysPerSplit. Each workgroup writes
// (o, m, l) per query head of the group; the combine kernel merges them.

constexpr int kKeysPerSplit = 64;
constexpr int kMaxGroup = 16;

template <typename T, int DV>
__global__ __launch_bounds__(256) void attn_decode_kernel(
    const T* __restrict__ q, const T* __restrict__ k_new, const T* __restrict__ v_new,
    const T* __restrict__ k_cache, const T* __restrict__ v_cache, const int32_t* __restrict__ cache_len,
    float* __restrict__ partial, int n_split, int cap, int n_meta, int window, int Hq, int Hkv, float base) {
  constexpr int KS = kKeysPerSplit;
  __shared__ float qs[kMaxGroup][kHd];
  __shared__ float kn[kHd];
  __shared__ float Ks[KS][kHd + 1];
  __shared__ float Vs[KS][DV];
  __shared__ float ps[kMaxGroup][KS];

  const int s = blockIdx.x, g = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int group = Hq / Hkv;
  const int tid = threadIdx.x;
  int p = cache_len[b];
  p = p < 0 ? 0 : (p > cap ? cap : p);
  const MaskRange mr = mask_range(p, n_meta, window);
  const int n_vis = mr.meta_end + (mr.win_end - mr.win_begin);
  const int i0 = s * KS;
  const int nk = max(0, min(KS, n_vis - i0));
  float* outp = partial + (((b * Hq) + g * group) * n_split + s) * (DV + 2);
  const int64_t pstride = (int64_t)n_split * (DV + 2);  // between heads

  if (nk == 0) {
    for (int t = tid; t < group * (DV + 2); t += blockDim.x) {
      const int hq = t / (DV + 2), e = t % (DV + 2);
      outp[hq * pstride + e] = e == DV ? -INFINITY : 0.f;
    }
    return;
  }

  // rotate the group's queries and the new key to position p
  for (int t = tid; t < (group + 1) * (kHd / 2); t += blockDim.x) {
    const int hq = t / (kHd / 2), i = t % (kHd / 2);
    float c, sn;
    rope_cs(p, i, base, &c, &sn);
    const T* src = hq < group ? q + (b * Hq + g * group + hq) * kHd : k_new + (b * Hkv + g) * kHd;
    const float lo = to_f32(src[i]), hi = to_f32(src[i + 32]);
    float* dst = hq < group ? qs[hq] : kn;
    dst[i] = lo * c - hi * sn;
    dst[i + 32] = hi * c + lo * sn;
  }
  __syncthreads();

  // stage K and V rows of the chunk (new row from k_new / v_new)
  constexpr int E = Vec16<T>::n;
  for (int it = tid; it < nk * (kHd / E); it += blockDim.x) {
    const int kk = it / (kHd / E), ch = it % (kHd / E);
    const int vi = i0 + kk;
    const int j = vi < mr.meta_end ? vi : mr.win_begin + (vi - mr.meta_end);
    float tmp[E];
    if (j == p) {
#pragma unroll
      for (int e = 0; e < E; ++e) tmp[e] = kn[ch * E + e];
    } else {
      load16(k_cache + ((b * cap + j) * Hkv + g) * kHd + ch * E, tmp);
    }
#pragma unroll
    for (int e = 0; e < E; ++e) Ks[kk][ch * E + e] = tmp[e];
  }
  for (int it = tid; it < nk * (DV / E); it += blockDim.x) {
    const int kk = it / (DV / E), ch = it % (DV / E);
    const int vi = i0 + kk;
    const int j = vi < mr.meta_end ? vi : mr.win_begin + (vi - mr.meta_end);
    const T* src = j == p ? v_new + (b * Hkv + g) * DV + ch * E : v_cache + ((b * cap + j) * Hkv + g) * DV + ch * E;
    float tmp[E];
    load16(src, tmp);
#pragma unroll
    for (int e = 0; e < E; ++e) Vs[kk][ch * E + e] = tmp[e];
  }
  __syncthreads();

  // scores (log2 units)
  for (int t = tid; t < group * KS; t += blockDim.x) {
    const int hq = t / KS, kk = t % KS;
    float sc = -INFINITY;
    if (kk < nk) {
      float a = 0.f;
#pragma unroll 16
      for (int d = 0; d < kHd; ++d) a = fmaf(qs[hq][d], Ks[kk][d], a);
      sc = a * kScaleLog2e;
    }
    ps[hq][kk] = sc;
  }
  __syncthreads();
  // softmax pieces per head: one wave per head (KS == 64 == wave size)
  const int lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  for (int hq = wave; hq < group; hq += nw) {
    const float sc = ps[hq][lane];
    float m = sc;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    const float pv = lane < nk ? fast_exp2(sc - m) : 0.f;
    const float l = wave_sum(pv);
    ps[hq][lane] = pv;
    if (lane == 0) {
      outp[hq * pstride + DV] = m;
      outp[hq * pstride + DV + 1] = l;
    }
  }
  __syncthreads();
  // o = sum_k p_k v_k
  for (int t = tid; t < group * DV; t += blockDim.x) {
    const int hq = t / DV, d = t % DV;
    float a = 0.f;
    for (int kk = 0; kk < nk; ++kk) a = fmaf(ps[hq][kk], Vs[kk][d], a);
    outp[hq * pstride + d] = a;
  }
}

// Merge the split partials of every head, then fuse with the Mamba branch:
// one workgroup per sequence.
template <typename T, int DV>
__global__ __launch_bounds__(256) void decode_combine_kernel(
    const float* __restrict__ partial, const T* __restrict__ y_ssm, const float* __restrict__ ba,
    const float* __restrict__ bs, T* __restrict__ out, T* __restrict__ y_attn_out, int n_split, int Hq,
    float eps) {
  extern __shared__ float ya[];   // [Hq * DV]
  __shared__ float red[2][4];
  const int64_t b = blockIdx.x;
  const int W = Hq * DV;
  const int tid = threadIdx.x;
  const float* pb = partial + b * Hq * (int64_t)n_split * (DV + 2);
  float sa = 0.f, ss = 0.f;
  for (int t = tid; t < W; t += blockDim.x) {
    const int h = t / DV, d = t % DV;
    const float* ph = pb + (int64_t)h * n_split * (DV + 2);
    float m = -INFINITY;
    for (int s = 0; s < n_split; ++s) m = fmaxf(m, ph[s * (DV + 2) + DV]);
    float l = 0.f, o = 0.f;
    for (int s = 0; s < n_split; ++s) {
      const float ms = ph[s * (DV + 2) + DV];
      if (ms == -INFINITY) continue;
      const float f = fast_exp2(ms - m);
      l = fmaf(ph[s * (DV + 2) + DV + 1], f, l);
      o = fmaf(ph[s * (DV + 2) + d], f, o);
    }
    const float v = o / l;
    ya[t] = v;
    sa = fmaf(v, v, sa);
    const float vs = to_f32(y_ssm[b * W + t]);
    ss = fmaf(vs, vs, ss);
  }
  sa = wave_sum(sa);
  ss = wave_sum(ss);
  const int lane = tid & 63, wave = tid >> 6;
  if (lane == 0) { red[0][wave] = sa; red[1][wave] = ss; }
  __syncthreads();
  sa = 0.f; ss = 0.f;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) { sa += red[0][w]; ss += red[1][w]; }
  const float inv_w = 1.0f / (float)W;
  const float ra = 0.5f / sqrtf(sa * inv_w + eps);
  const float rs = 0.5f / sqrtf(ss * inv_w + eps);
  for (int t = tid; t < W; t += blockDim.x) {
    const float v = ya[t];
    const float vs = to_f32(y_ssm[b * W + t]);
    out[b * W + t] = from_f32<T>(fmaf(ba[t] * ra, v, bs[t] * rs * vs));
    if (y_attn_out) y_attn_out[b * W + t] = from_f32<T>(v);
  }
}

template <typename T>
hipError_t rope_t(const RopeArgs& a, hipStream_t stream) {
  dim3 grid((a.L + kRopeRows - 1) / kRopeRows, a.batch);
  hipLaunchKernelGGL(rope_prefill_kernel<T>, grid, dim3(256), 0, stream, (const T*)a.q, (const T*)a.k,
                     (const T*)a.v, (T*)a.q_rot, (T*)a.k_rot, (T*)a.v_copy, a.k_rows, a.v_rows, a.L, a.n_q_heads,
                     a.n_kv_heads, a.head_dim_v, a.rope_base);
  return hipGetLastError();
}

template <typename T, int DV>
hipError_t attn_prefill_t(const AttnPrefillArgs& a, hipStream_t stream) {
  // 32-row query blocks per workgroup: two (more K/V reuse per LDS stage) when
  // that still leaves several workgroups per compute unit; at most 10 waves.
  const int group = a.n_q_heads / a.n_kv_heads;
  const int64_t blocks1 = (int64_t)((a.L + 31) / 32) * a.n_kv_heads * a.batch;
  const int pb = (group <= 5 && blocks1 >= 1024) ? 2 : 1;
  dim3 grid((a.L + 32 * pb - 1) / (32 * pb), a.n_kv_heads, a.batch);
  dim3 block(64 * group * pb);
  hipLaunchKernelGGL((attn_prefill_kernel<T, DV>), grid, block, 0, stream, (const T*)a.q_rot, (const T*)a.k_rot,
                     (const T*)a.v, (T*)a.y, a.k_rows, a.v_rows, a.L, a.n_meta, a.window, a.n_q_heads, a.n_kv_heads,
                     pb);
  return hipGetLastError();
}

template <typename T, int DV>
hipError_t attn_decode_t(const AttnDecodeArgs& a, hipStream_t stream) {
  dim3 grid(a.n_split, a.n_kv_heads, a.batch);
  hipLaunchKernelGGL((attn_decode_kernel<T, DV>), grid, dim3(256), 0, stream, (const T*)a.q, (const T*)a.k_new,
                     (const T*)a.v_new, (const T*)a.k_cache, (const T*)a.v_cache, a.cache_len, a.partial,
                     a.n_split, a.cap, a.n_meta, a.window, a.n_q_heads, a.n_kv_heads, a.rope_base);
  return hipGetLastError();
}

template <typename T, int DV>
hipError_t combine_t(const DecodeCombineArgs& a, hipStream_t stream) {
  const size_t shm = (size_t)a.n_q_heads * DV * sizeof(float);
  hipLaunchKernelGGL((decode_combine_kernel<T, DV>), dim3(a.batch), dim3(256), shm, stream, a.partial,
                     (const T*)a.y_ssm, a.beta_attn, a.beta_ssm, (T*)a.out, (T*)a.y_attn_out, a.n_split,
                     a.n_q_heads, a.eps);
  return hipGetLastError();
}

#define HYMBA_DISPATCH_DV(DVV, FN, T, ...)                      \
  switch (DVV) {                                                \
    case 32: return FN<T, 32>(__VA_ARGS__);                     \
    case 64: return FN<T, 64>(__VA_ARGS__);                     \
    case 128: return FN<T, 128>(__VA_ARGS__);                   \
    default: return hipErrorInvalidValue;                       \
  }

}  // namespace

hipError_t launch_rope_prefill(const RopeArgs& a, hipStream_t stream) {
  if (a.act == HYMBA_BF16) return rope_t<bf16>(a, stream);
  return rope_t<float>(a, stream);
}

hipError_t launch_attn_prefill(const AttnPrefillArgs& a, hipStream_t stream) {
  if (a.act == HYMBA_BF16) { HYMBA_DISPATCH_DV(a.head_dim_v, attn_prefill_t, bf16, a, stream) }
  HYMBA_DISPATCH_DV(a.head_dim_v, attn_prefill_t, float, a, stream)
}

void decode_split_plan(int n_meta, int window, int cap, int* n_split, int* keys_per_split) {
  // most keys a decode row can see: meta + window (SWA), or the whole cache + itself
  int64_t max_vis = (int64_t)cap + 1;
  if (window > 0 && (int64_t)n_meta + window < max_vis) max_vis = (int64_t)n_meta + window;
  *keys_per_split = kKeysPerSplit;
  *n_split = (int)((max_vis + kKeysPerSplit - 1) / kKeysPerSplit);
}

hipError_t launch_attn_decode(const AttnDecodeArgs& a, hipStream_t stream) {
  if (a.act == HYMBA_BF16) { HYMBA_DISPATCH_DV(a.head_dim_v, attn_decode_t, bf16, a, stream) }
  HYMBA_DISPATCH_DV(a.head_dim_v, attn_decode_t, float, a, stream)
}

hipError_t launch_decode_combine(const DecodeCombineArgs& a, hipStream_t stream) {
  if (a.act == HYMBA_BF16) { HYMBA_DISPATCH_DV(a.head_dim_v, combine_t, bf16, a, stream) }
  HYMBA_DISPATCH_DV(a.head_dim_v, combine_t, float, a, stream)
}

}  // namespace hymba
