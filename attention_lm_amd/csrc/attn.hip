// Attention branch: rotary embedding, prefill flash attention on the matrix
// cores, and split-key decode attention over a read-only (shareable) KV cache.
//
// Attention is softmax(q k^T / sqrt(d_k)) v ("Jamba: Hybrid SSM-Transformer",
// "1. Layer Interleaving Ratio"), grouped-query (GQA) with RoPE (51cto
// Hymba-1.5B article, section 2), over the visibility rule in common.hpp:
// meta-token rows visible to all later rows, plus a sliding window or, in a
// global layer, every earlier row.
#include <math.h>

#include <algorithm>
#include <atomic>

#include "common.hpp"
#include "launch.hpp"
#include "mma.hpp"

namespace hymba {

namespace {

constexpr int kHd = 64;                 // query/key head width
constexpr float kScaleLog2e = 0.125f * kLog2e;  // 1/sqrt(64) folded with log2(e)

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// max of three scores without the NaN-quieting copies the compiler puts in front
// of fmaxf on values it cannot prove canonical (scores are never NaN)
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
// A VALU instruction may read a matrix-core result only some wait states
// after the MFMA issues (gfx950: 12 for v_mfma_f32_32x32x16_bf16, 18 for
// v_mfma_f32_32x32x2_f32). The compiler pads its own instructions, but not
// the operands of inline asm such as max3f: before max3f reads score
// registers that an MFMA has just written, this wait (18 states) is placed,
// and since it takes the registers as in/out operands every later read of them
// is ordered after it.
__device__ __forceinline__ void mfma_result_wait(f32x16_t& a) { asm volatile("s_nop 15\n\ts_nop 1" : "+v"(a)); }
__device__ __forceinline__ void mfma_result_wait(f32x16_t& a, f32x16_t& b) {
  asm volatile("s_nop 15\n\ts_nop 1" : "+v"(a), "+v"(b));
}

// 8 consecutive elements <-> fp32
__device__ __forceinline__ void load8(const bf16* p, float* o) { load16(p, o); }
__device__ __forceinline__ void load8(const float* p, float* o) { load16(p, o); load16(p + 4, o + 4); }
__device__ __forceinline__ void store8(bf16* p, const float* o) { store16(p, o); }
__device__ __forceinline__ void store8(float* p, const float* o) { store16(p, o); store16(p + 4, o + 4); }

// cos/sin of pos * base^(-2i/64), angle formed and reduced in fp64.
__device__ __forceinline__ void rope_cs(int pos, int i, float base, float* c, float* s) {
  const double inv_freq = pow((double)base, -2.0 * (double)i / (double)kHd);
  const double ang = (double)pos * inv_freq;
  double sd, cd;
  sincos(ang, &sd, &cd);
  *c = (float)cd;
  *s = (float)sd;
}

// The same cos/sin from the frequency step r = base^(-2/64) (formed on the
// host in fp64): the frequency r^i by repeated squaring, the angle in fp64,
// reduced by 2 pi in fp64 (two-part constant), then sin/cos of the reduced
// angle in fp32 (the fp64 angle carries the same error as in rope_cs).
__device__ __forceinline__ void rope_cs_step(int pos, int i, double r, float* c, float* s) {
  double f = 1.0, x = r;
#pragma unroll
  for (int bit = 0; bit < 5; ++bit) {   // i < 32
    if (i & (1 << bit)) f *= x;
    x *= x;
  }
  const double ang = (double)pos * f;
  constexpr double kInv2Pi = 0.15915494309189533577, k2PiHi = 6.283185307179586232, k2PiLo = 2.4492935982947064e-16;
  const double n = rint(ang * kInv2Pi);
  const double red = fma(-n, k2PiLo, fma(-n, k2PiHi, ang));
  sincosf((float)red, s, c);
}

// ---------------------------------------------------------------------------
// RoPE prologue (prefill): q -> q_rot, k -> k_rot (e.g. straight into the KV
// cache), optionally v -> v_copy. Rotate-half pairs (i, i+32). The rotated
// queries are also scaled by log2(e)/sqrt(64), so that q.k comes out as the
// softmax exponent in base 2.

// Two rows per workgroup: for the usual head counts a thread then has one
// rotation item and at most one value-copy item. A thread issues the loads of
// its first items before the workgroup forms the rows' cos/sin (the angles do
// not depend on them), so the loads' latency overlaps that arithmetic; beside
// a scan that keeps the VALU busy, a pass that formed its angles first and
// loaded afterwards spent most of its time waiting on one after the other.
constexpr int kRopeRows = 2;
constexpr int kRopeThreads = 256;

template <typename T>
__global__ __launch_bounds__(kRopeThreads) void rope_prefill_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, T* __restrict__ q_rot,
    T* __restrict__ k_rot, T* __restrict__ v_copy, int64_t k_rows, int64_t v_rows, int64_t k_row0, int64_t v_row0,
    const float* __restrict__ k_scale, int L, int pos0, int Hq, int Hkv, int dv, double freq_step, float q_scale) {
  __shared__ float cs[kRopeRows][kHd / 2];
  __shared__ float sn[kRopeRows][kHd / 2];
  const int r0 = blockIdx.x * kRopeRows;
  const int64_t b = blockIdx.y;
  const int tid = threadIdx.x;
  const int nrows = min(kRopeRows, L - r0);
  const int H = Hq + Hkv;
  const int rot_items = nrows * H * 4;                      // (row, head, group of 8 pairs)
  const int per_row = Hkv * dv / 8;
  const int v_items = v_copy ? nrows * per_row : 0;         // (row, 8-element chunk)
  const int n_items = max(rot_items, v_items);

  // one (rotation, value-copy) item pair: loads, then rotation and stores
  struct Item {
    bool has_v, has_r;
    int g8, rr;
    float vf[8], lo[8], hi[8], slo[8], shi[8];   // slo, shi: per-dim output scale of the pair's halves
    int64_t v_dst;
    T* dst;
  };
  auto load = [&](int it, Item& m) {
    m.has_v = it < v_items;
    m.v_dst = 0;
    if (m.has_v) {
      const int r = it / per_row, e = it % per_row;
      load8(v + (b * L + r0 + r) * (int64_t)(Hkv * dv) + 8 * e, m.vf);
      m.v_dst = (b * v_rows + v_row0 + r0 + r) * (int64_t)(Hkv * dv) + 8 * e;
    }
    m.has_r = it < rot_items;
    m.g8 = it & 3;
    const int hr = it >> 2, hd = hr % H;
    m.rr = hr / H;
    m.dst = nullptr;
#pragma unroll
    for (int e = 0; e < 8; ++e) m.slo[e] = m.shi[e] = 1.f;
    if (m.has_r) {
      const int row = r0 + m.rr;
      const T* src;
      if (hd < Hq) {
        src = q + ((b * L + row) * Hq + hd) * kHd;
        m.dst = q_rot + ((b * L + row) * Hq + hd) * kHd;
        if (k_scale) {   // shared-key affine: q (.) w of the head's kv group
          const float* w = k_scale + (hd / (Hq / Hkv)) * kHd;
          load8(w + 8 * m.g8, m.slo);
          load8(w + 32 + 8 * m.g8, m.shi);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) { m.slo[e] *= q_scale; m.shi[e] *= q_scale; }
      } else {
        src = k + ((b * L + row) * Hkv + (hd - Hq)) * kHd;
        m.dst = k_rot + ((b * k_rows + k_row0 + row) * Hkv + (hd - Hq)) * kHd;
      }
      load8(src + 8 * m.g8, m.lo);
      load8(src + 32 + 8 * m.g8, m.hi);
    }
  };
  auto finish = [&](Item& m) {
    if (m.has_r) {
      float olo[8], ohi[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float c = cs[m.rr][8 * m.g8 + e], s = sn[m.rr][8 * m.g8 + e];
        olo[e] = (m.lo[e] * c - m.hi[e] * s) * m.slo[e];
        ohi[e] = (m.hi[e] * c + m.lo[e] * s) * m.shi[e];
      }
      store8(m.dst + 8 * m.g8, olo);
      store8(m.dst + 32 + 8 * m.g8, ohi);
    }
    if (m.has_v) store8(v_copy + m.v_dst, m.vf);
  };

  Item m;
  if (tid < n_items) load(tid, m);
  for (int t = tid; t < kRopeRows * (kHd / 2); t += blockDim.x) {
    const int r = t / (kHd / 2), i = t % (kHd / 2);
    rope_cs_step(pos0 + r0 + r, i, freq_step, &cs[r][i], &sn[r][i]);
  }
  __syncthreads();
  if (tid < n_items) finish(m);
  for (int it = tid + (int)blockDim.x; it < n_items; it += blockDim.x) {   // heads past one round of threads
    load(it, m);
    finish(m);
  }
}

// ---------------------------------------------------------------------------
// Prefill attention on the matrix cores.
//
// Workgroup = 4 waves = 128 query columns of one (sequence, kv head): P
// consecutive positions times the G query heads of the GQA group (column c is
// position p0 + c / G, head c % G; P = floor(128 / G)). All columns read the
// same key/value tiles, staged in LDS once per workgroup, so a K/V byte is
// fetched once for every query head that uses it.
//
// Per 32-key sub-tile each wave computes S^T = K Q^T with 32x32x16 bf16 MFMA
// (fp32 inputs: 32x32x2). In that layout each lane owns one query column and
// 16 keys, so softmax statistics need only one cross-lane step (lanes l and
// l+32) and the exp'd scores, converted in registers, are directly the B
// operand of O^T = V^T P^T: no LDS round trip for P. V is stored transposed in
// LDS with keys permuted inside each 16-key chunk to match that operand.
//
// Scores come out of the MFMA already in log2 units and already shifted by the
// column's reference max: Q is pre-scaled by log2(e)/sqrt(64) in the RoPE
// prologue and the score accumulator starts at -m. Each score then costs one
// exp2. The reference moves (and the running sums are rescaled) only when a
// score exceeds it by more than 2^8; numerator and denominator always share
// it, so the result is exact up to rounding. Both sub-tiles' score products are
// issued before the first softmax so that the exp work of one overlaps the
// matrix work of the other.

constexpr int BK = 64;                     // keys per LDS stage (two 32-key sub-tiles)
constexpr int kAttnWaves = 4;
constexpr int kAttnCols = 32 * kAttnWaves;
constexpr float kRescaleSlack = 8.0f;
// slot s of a 16-key chunk holds key kperm(s); an involution
__device__ __forceinline__ int kperm(int s) { return (s & 3) | ((s & 4) << 1) | ((s & 8) >> 1); }

// Staging of one 64-key K/V tile in LDS (two stages, double-buffered).
//
// bf16: buffer loads write LDS directly (16 bytes per lane, lanes contiguous),
// so no staging registers and no stash. K rows (128 B) and V rows (2 dv B)
// keep their natural layout; the 16-byte chunks of a row are XOR-swizzled by
// the row index so that the operand reads below are bank-conflict free (the
// swizzle is applied on the global side: each lane loads the chunk that
// belongs at its LDS position). K operands are plain 16-byte reads (8
// consecutive dims of one key). V operands need 8 keys of one dv: two
// transposing reads (ds_read_b64_tr_b16), each giving a 16-lane group 4 keys x
// 16 dvs, so V is never transposed in memory.
// fp32: registers -> padded LDS, with V stored transposed (tests use fp32).
// Rows at or past L read as zeros; their keys are masked out of every score.
typedef __attribute__((address_space(3))) char lds_char;
typedef short v4i16_t __attribute__((ext_vector_type(4)));

template <typename T, int DV, int NT>
struct TileStage;

template <int DV, int NT>
struct TileStage<bf16, DV, NT> {
  typedef bf16x8_t Frag;
  static constexpr int KROWB = kHd * 2, VROWB = DV * 2;          // bytes per K / V row
  static constexpr int KCH = KROWB / 16, VCH = VROWB / 16;       // 16-byte chunks per row
  static constexpr int KSTAGE = BK * KROWB, VSTAGE = BK * VROWB;
  static constexpr int kStageBytes = KSTAGE + VSTAGE;
  static constexpr int KN = BK * KCH / NT, VN = BK * VCH / NT;   // loads per thread per tile
  static_assert(BK * KCH % NT == 0 && BK * VCH % NT == 0, "tile shape");
  // K: 16 consecutive rows at one chunk hit 16 distinct 16-byte bank slots.
  static __device__ __forceinline__ int ksw(int row) { return (row >> 1) & (KCH - 1); }
  // V: the 4 rows x 2 halves of 32 bytes that one 32-lane half of a
  // transposing read touches land in 8 distinct 32-byte bank slots.
  static constexpr int VRPB = VROWB >= 256 ? 1 : 256 / VROWB;   // V rows per 256-byte bank sweep
  static __device__ __forceinline__ int vsw(int row) { return (4 * ((row & 3) / VRPB)) & (VCH - 1); }
  __amdgpu_buffer_rsrc_t krs, vrs;
  uint32_t kstride_b, vstride_b;
  uint32_t koff[KN], voff[VN];   // per-lane global byte offsets of a tile starting at row 0
  int kro[4], vro[DV / 32];      // per-lane LDS byte offsets of the operand reads (see kfrag, vfrag)
  int wave, lane;
  __device__ __forceinline__ void init(int tid, const bf16* kbase, const bf16* vbase, int64_t kstride,
                                       int64_t vstride, int L) {
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    lane = tid & 63;
    kstride_b = (uint32_t)(kstride * 2);
    vstride_b = (uint32_t)(vstride * 2);
    krs = make_rsrc(kbase, (uint32_t)(((int64_t)(L - 1) * kstride + kHd) * 2));
    vrs = make_rsrc(vbase, (uint32_t)(((int64_t)(L - 1) * vstride + DV) * 2));
#pragma unroll
    for (int r = 0; r < KN; ++r) {
      const int pos = r * NT + 64 * wave + lane, row = pos / KCH, cp = pos % KCH;
      koff[r] = (uint32_t)row * kstride_b + 16u * (uint32_t)(cp ^ ksw(row));
    }
#pragma unroll
    for (int r = 0; r < VN; ++r) {
      const int pos = r * NT + 64 * wave + lane, row = pos / VCH, cp = pos % VCH;
      voff[r] = (uint32_t)row * vstride_b + 16u * (uint32_t)(cp ^ vsw(row));
    }
    // The swizzles of the rows read below depend on the lane only (rows
    // 32 i + lq for K; 4 (g / 2) + j / 4 plus a multiple of 4 for V), so each
    // read is a per-lane offset plus a constant.
    const int lq = lane & 31, hh = lane >> 5, g = lane >> 4, j = lane & 15;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) kro[cc] = lq * KROWB + 16 * ((2 * cc + hh) ^ ksw(lq));
    const int vrow = 4 * (g >> 1) + (j >> 2);
#pragma unroll
    for (int d = 0; d < DV / 32; ++d) {
      const int dv = 32 * d + 16 * (g & 1) + 4 * (j & 3);
      vro[d] = KSTAGE + vrow * VROWB + 16 * ((dv >> 3) ^ vsw(vrow)) + 8 * ((dv >> 2) & 1);
    }
  }
  // tile rows [j0, j0 + BK) into the stage at dst
  __device__ __forceinline__ void fetch(int j0, lds_char* dst) {
    const uint32_t kt = (uint32_t)j0 * kstride_b, vt = (uint32_t)j0 * vstride_b;
    lds_char* kd = dst;
    lds_char* vd = dst + KSTAGE;
#pragma unroll
    for (int r = 0; r < KN; ++r) buf_load16_lds(krs, koff[r] + kt, kd + (r * NT + 64 * wave) * 16);
#pragma unroll
    for (int r = 0; r < VN; ++r) buf_load16_lds(vrs, voff[r] + vt, vd + (r * NT + 64 * wave) * 16);
  }
  __device__ __forceinline__ void stash(lds_char*) {}
  // The B operand of S^T = K Q^T for the 16 dims of chunk c % 4 and the 32
  // keys of half c / 4: lane l holds K[32 (c / 4) + l % 32][16 (c % 4) + 8 (l / 32) + t].
  // Addresses are formed as the stage base plus one offset, so that the
  // compiler sees which stage every read is in.
  __device__ __forceinline__ Frag kfrag(const lds_char* src, int c) const {
    const lds_char* p = src + kro[c & 3] + (c >> 2) * 32 * KROWB;
    return __builtin_bit_cast(Frag, *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>(p));
  }
  // The A operand of O^T = V^T P^T for dv block d and the 16 keys from key0:
  // lane l holds V[key0 + 8(t/4) + 4(l/32) + t%4][32 d + l%32] in slot t.
  // (key0 a multiple of 16.) In a 16-lane group g, lane j = 4 k + m points at
  // V[key0 + 4 (g / 2) + k][32 d + 16 (g % 2) + 4 m .. + 3]; the transposing
  // read hands lane j the 4 keys of dv 32 d + 16 (g % 2) + j.
  __device__ __forceinline__ Frag vfrag(const lds_char* src, int d, int key0) const {
    typedef __attribute__((address_space(3))) v4i16_t lds_v4;
    const lds_char* p = src + vro[d] + key0 * VROWB;
    const v4i16_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)p);
    const v4i16_t c = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(p + 8 * VROWB));
    typedef short v8i16_t __attribute__((ext_vector_type(8)));
    const v8i16_t v = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
    return __builtin_bit_cast(Frag, v);
  }
};

template <int DV, int NT>
struct TileStage<float, DV, NT> {
  typedef F32x8 Frag;
  static constexpr int KP = kHd + 4;     // padded K row (floats)
  static constexpr int VP = BK + 4;      // padded V^T row (floats)
  static constexpr int KSTAGE = BK * KP * 4, VSTAGE = DV * VP * 4;
  static constexpr int kStageBytes = KSTAGE + VSTAGE;
  static constexpr int KCH = kHd / 4;
  static constexpr int KMAX = (BK * KCH + NT - 1) / NT;
  static constexpr int NQ = BK / 4, NC = DV / 8;
  static constexpr int VMAX = (NQ * NC + NT - 1) / NT;
  float4 kreg[KMAX];
  float vreg[VMAX][4][8];
  int tid_, L_, lane;
  const float *kbase_, *vbase_;
  int64_t kstride_, vstride_;
  typedef __attribute__((address_space(3))) float lds_float;
  static __device__ __forceinline__ lds_float* Ks(lds_char* p) { return (lds_float*)p; }
  static __device__ __forceinline__ lds_float* Vt(lds_char* p) { return (lds_float*)(p + KSTAGE); }
  static __device__ __forceinline__ const lds_float* Ks(const lds_char* p) { return (const lds_float*)p; }
  static __device__ __forceinline__ const lds_float* Vt(const lds_char* p) { return (const lds_float*)(p + KSTAGE); }
  static __device__ __forceinline__ Frag frag_at(const lds_float* p) {
    Frag f;
#pragma unroll
    for (int t = 0; t < 8; ++t) f.v[t] = p[t];
    return f;
  }
  __device__ __forceinline__ void init(int tid, const float* kbase, const float* vbase, int64_t kstride,
                                       int64_t vstride, int L) {
    tid_ = tid;
    lane = tid & 63;
    L_ = L;
    kbase_ = kbase;
    vbase_ = vbase;
    kstride_ = kstride;
    vstride_ = vstride;
  }
  __device__ __forceinline__ void fetch(int j0, lds_char*) {
#pragma unroll
    for (int r = 0; r < KMAX; ++r) {
      const int it = tid_ + r * NT;
      kreg[r] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (it < BK * KCH) {
        const int j = j0 + it / KCH;
        if (j < L_) kreg[r] = *reinterpret_cast<const float4*>(kbase_ + (int64_t)j * kstride_ + (it % KCH) * 4);
      }
    }
#pragma unroll
    for (int r = 0; r < VMAX; ++r) {
      const int it = tid_ + r * NT;
      if (it < NQ * NC) {
        const int kq = it % NQ, dc = it / NQ;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = j0 + 4 * kq + e;
          if (key < L_) {
            load8(vbase_ + (int64_t)key * vstride_ + 8 * dc, vreg[r][e]);
          } else {
#pragma unroll
            for (int t = 0; t < 8; ++t) vreg[r][e][t] = 0.f;
          }
        }
      }
    }
  }
  // V stored transposed, keys permuted inside each 16-key chunk (slot s holds key kperm(s))
  __device__ __forceinline__ void stash(lds_char* dst) {
    lds_float* ks = Ks(dst);
    lds_float* vt = Vt(dst);
#pragma unroll
    for (int r = 0; r < KMAX; ++r) {
      const int it = tid_ + r * NT;
      if (it < BK * KCH) {
        lds_float* d = &ks[(it / KCH) * KP + (it % KCH) * 4];
        d[0] = kreg[r].x; d[1] = kreg[r].y; d[2] = kreg[r].z; d[3] = kreg[r].w;
      }
    }
#pragma unroll
    for (int r = 0; r < VMAX; ++r) {
      const int it = tid_ + r * NT;
      if (it < NQ * NC) {
        const int kq = it % NQ, dc = it / NQ;
        const int kk0 = 4 * kq;
        const int col = (kk0 & ~15) + kperm(kk0 & 15);  // 4 contiguous slots
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          lds_float* d = &vt[(8 * dc + t) * VP + col];
          d[0] = vreg[r][0][t]; d[1] = vreg[r][1][t]; d[2] = vreg[r][2][t]; d[3] = vreg[r][3][t];
        }
      }
    }
  }
  __device__ __forceinline__ Frag kfrag(const lds_char* src, int c) const {
    return frag_at(Ks(src) + ((c >> 2) * 32 + (lane & 31)) * KP + 8 * (2 * (c & 3) + (lane >> 5)));
  }
  __device__ __forceinline__ Frag vfrag(const lds_char* src, int d, int key0) const {
    return frag_at(Vt(src) + (32 * d + (lane & 31)) * VP + key0 + 8 * (lane >> 5));
  }
};

// Per-lane state of the online softmax of one query column (shared by lanes l
// and l+32, which hold 16 keys each of every 32-key sub-tile).
template <int NDB>
struct SoftmaxState {
  f32x16_t acc[NDB];   // O^T block d: this lane's column, dv 32d + 8(r/4) + 4hh + r%4
  f32x16_t negm;       // every entry -mref: the initial score accumulator
  float mref;          // reference max (log2 units) subtracted from the scores
  float thr;           // rescale when a shifted score exceeds this (-inf until a score was seen)
  float l;             // this lane's part of the sum of 2^(s - mref)

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int d = 0; d < NDB; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[d][r] = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) negm[r] = 0.f;
    mref = 0.f;
    thr = -INFINITY;
    l = 0.f;
  }
  // A shifted score of this column (t: this lane's max) passed the threshold:
  // agree on the column max with the partner lane, move the reference to it and
  // rescale the sums. s (and s_next, scored against the same reference) are
  // re-shifted.
  __device__ __forceinline__ void rescale(float t, f32x16_t& s, f32x16_t* s_next) {
    const float mt = fmaxf(t, __shfl_xor(t, 32, 64));
    const bool need = mt > thr;                 // the same in both lanes of the column
    const float delta = need ? mt : 0.f;
    // nothing has been accumulated before the first reference: scale by 0
    const float alpha = need ? (thr == -INFINITY ? 0.f : fast_exp2(-delta)) : 1.f;
    if (need) thr = kRescaleSlack;
    mref += delta;
    l *= alpha;
#pragma unroll
    for (int d = 0; d < NDB; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[d][r] *= alpha;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      negm[r] -= delta;
      s[r] -= delta;
    }
    if (s_next) {
#pragma unroll
      for (int r = 0; r < 16; ++r) (*s_next)[r] -= delta;
    }
  }
};

// Visible keys of this lane's query, as intervals: meta keys [0, meta_hi) and
// window keys [win_lo, win_hi) (both empty for a column without a query).
struct LaneKeys {
  int meta_hi, win_lo, win_hi;
};

// s[r] (key j0 + 4hh + 8(r/4) + r%4) := -inf where the key is not visible.
// A sub-tile entirely below n_meta or entirely at or above it needs one
// interval test per score; one that straddles n_meta (n_meta not a multiple
// of 32) tests both.
__device__ __forceinline__ void mask_scores(f32x16_t& s, const LaneKeys& lk, int j0, int hh, int n_meta) {
  const int base = j0 + 4 * hh;
  if (j0 + 32 <= n_meta || j0 >= n_meta) {
    const bool meta = j0 < n_meta;
    const int lo = meta ? 0 : lk.win_lo, hi = meta ? lk.meta_hi : lk.win_hi;
    const int rel = base - lo;
    const uint32_t len = (uint32_t)max(hi - lo, 0);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const uint32_t u = (uint32_t)(rel + 8 * (r >> 2) + (r & 3));
      s[r] = u < len ? s[r] : -INFINITY;
    }
  } else {
    const uint32_t wlen = (uint32_t)max(lk.win_hi - lk.win_lo, 0);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = base + 8 * (r >> 2) + (r & 3);
      const bool vis = j < lk.meta_hi || (uint32_t)(j - lk.win_lo) < wlen;
      s[r] = vis ? s[r] : -INFINITY;
    }
  }
}

// The index logic of the prefill attention, shared by the kernel and by the
// debug export that checks it exactly: the workgroup's item (sequence, kv
// head, block of P positions) from its launch index, the key tiles it visits
// (the meta tiles, then the window tiles), each wave's decision per 32-key
// sub-tile (skip it, or take it without a mask) and each lane's visible key
// intervals, which mask the remaining sub-tiles in mask_scores.
//
// Workgroup = 4 waves = 128 query columns: P = floor(128 / G) consecutive
// positions times the G query heads of one kv head (column c is position
// p0 + c / G, head c % G). Query row r is at position q_pos0 + r; key row j
// is at position j; positions below L = q_pos0 + Lq exist.
//
// Work order: a workgroup's cost grows with its position block (more keys in
// the causal window, up to the full window); two workgroups fit on a CU. Items
// are handed out heaviest first (largest-first scheduling). When all of them
// fit at once (between one and two per CU), n_items - n_cu CUs get a second
// workgroup (workgroup n_cu + j lands beside workgroup j): the CUs that keep
// one workgroup take the heaviest items, and each other CU pairs one of the
// next heaviest with one of the lightest.
struct PrefillIndex {
  int L, n_meta, window;
  int64_t b;      // sequence
  int g;          // kv head
  int p0, p1;     // the workgroup's positions [p0, p1)
  int qa, qb;     // positions spanned by this wave's valid columns
  int my_q;       // this lane's query position (L: the column has no query)
  int h;          // this lane's query head
  int n1, k2s, ntiles;   // tiles: [0, n1) of meta keys, then k2s, k2s + 1, .. (64 keys each)
  LaneKeys lk;

  __device__ __forceinline__ void init(int wg, int n_cu, int Lq, int q_pos0, int n_meta_, int window_, int Hq,
                                       int Hkv, int batch, int wave, int lane) {
    n_meta = n_meta_;
    window = window_;
    L = q_pos0 + Lq;
    const int G = Hq / Hkv;                 // query heads per kv head
    const int P = kAttnCols / G;            // positions per workgroup
    const int nxb = (Lq + P - 1) / P;
    const int hb_n = Hkv * batch;
    const int n_items = nxb * hb_n;
    int pb, hb;
    const int n_xcd = n_cu / 32;   // 32 CUs per XCD
    if (n_items > 2 * n_cu && n_xcd > 1 && hb_n % n_xcd == 0) {
      // Many rounds of workgroups: launch index wg runs on XCD wg % n_xcd (each
      // XCD has its own L2). XCD x takes the (sequence, kv head) streams
      // x, x + n_xcd, .. one after another, each from its last position block
      // down, so the workgroups it holds at once are neighbouring blocks of one
      // or two streams and share their keys and values in its L2.
      const int x = wg % n_xcd, k = wg / n_xcd;
      hb = x + n_xcd * (k / nxb);
      pb = nxb - 1 - k % nxb;
    } else {
      int rank = wg;
      if (n_items > n_cu && n_items <= 2 * n_cu) {
        const int n_pair = n_items - n_cu, n_single = n_cu - n_pair;
        if (wg < n_cu) rank = wg < n_pair ? n_single + wg : wg - n_pair;
        else rank = n_items - 1 - (wg - n_cu);
      }
      pb = nxb - 1 - rank / hb_n;
      hb = rank % hb_n;
    }
    g = hb % Hkv;
    b = hb / Hkv;
    p0 = q_pos0 + pb * P;
    p1 = min(p0 + P, L);
    const int col = 32 * wave + (lane & 31);
    const bool col_ok = col < P * G;
    my_q = col_ok ? p0 + col / G : L;
    h = g * G + (col_ok ? col % G : 0);
    const int c_lo = 32 * wave, c_hi = min(32 * wave + 31, P * G - 1);
    qa = p0 + c_lo / G;
    qb = c_lo <= c_hi ? min(p0 + c_hi / G + 1, L) : qa;
    lk.meta_hi = my_q < L ? min(my_q + 1, n_meta) : 0;
    lk.win_hi = my_q < L ? my_q + 1 : 0;
    lk.win_lo = window > 0 ? max(my_q - window + 1, n_meta) : n_meta;
    // key tiles: meta part then window part
    const int meta_end = min(n_meta, p1);
    const int wb = window > 0 ? max(n_meta, p0 - window + 1) : n_meta;
    n1 = (meta_end + BK - 1) / BK;
    k2s = wb / BK;
    const int k2e = (p1 + BK - 1) / BK;
    if (k2s < n1) k2s = n1;
    ntiles = n1 + max(0, k2e - k2s);
  }
  __device__ __forceinline__ int tile_j0(int idx) const { return (idx < n1 ? idx : k2s + (idx - n1)) * BK; }
  // sub-tile [j0, j0 + 32) against this wave's positions [qa, qb): no key
  // visible to any column
  __device__ __forceinline__ bool none_for(int j0) const {
    const int j1 = j0 + 32;
    return qa >= qb || (j0 > qb - 1) || (window > 0 && j0 >= n_meta && qa - (j1 - 1) >= window);
  }
  // ... or every key visible to every column
  __device__ __forceinline__ bool full_for(int j0) const {
    const int j1 = j0 + 32;
    return qa < qb && (j1 - 1 <= qa) && (window <= 0 || j1 <= n_meta || (qb - 1) - max(j0, n_meta) < window);
  }
};

// OCC: waves per SIMD the register allocation aims for. Three (bf16) when
// there are many rounds of workgroups (the latency of one wave's tile chain is
// hidden better), else two: the work order for one or two rounds places two
// workgroups per CU.
template <typename T, int DV, int OCC>
__global__ __launch_bounds__(64 * kAttnWaves) __attribute__((amdgpu_waves_per_eu(OCC))) void attn_prefill_kernel(
    const T* __restrict__ q_rot, const T* __restrict__ k_rot, const T* __restrict__ v, T* __restrict__ y,
    int64_t k_rows, int64_t v_rows, int Lq, int q_pos0, int n_meta, int window, int Hq, int Hkv, int batch,
    int n_cu) {
  typedef Mma<T> M;
  typedef typename M::Frag Frag;
  constexpr int NDB = DV / 32;
  constexpr int NT = 64 * kAttnWaves;
  typedef TileStage<T, DV, NT> Stage;
  // the two stages are separate objects, so that the compiler can tell reads
  // of one from the loads into the other and need not wait for those
  __shared__ __attribute__((aligned(16))) char lds_stage0[Stage::kStageBytes];
  __shared__ __attribute__((aligned(16))) char lds_stage1[Stage::kStageBytes];
  lds_char* const stage0 = (lds_char*)lds_stage0;
  lds_char* const stage1 = (lds_char*)lds_stage1;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: tile decisions are scalar
  const int hh = lane >> 5;   // lane half
  const int L = q_pos0 + Lq;
  PrefillIndex ix;
  ix.init((int)blockIdx.x, n_cu, Lq, q_pos0, n_meta, window, Hq, Hkv, batch, wave, lane);
  const int64_t b = ix.b;
  const int g = ix.g;
  const int my_q = ix.my_q, h = ix.h;
  const LaneKeys lk = ix.lk;

  // Q^T operand: lane holds Q[my_q][16 kc + 8 hh .. +7] (pre-scaled)
  Frag qf[4];
#pragma unroll
  for (int kc = 0; kc < 4; ++kc)
    qf[kc] = my_q < L ? M::frag_at(q_rot + ((b * Lq + my_q - q_pos0) * Hq + h) * kHd + 16 * kc + 8 * hh)
                      : M::zero();

  SoftmaxState<NDB> st;
  st.init();

  const int ntiles = ix.ntiles;
  const int64_t kstride = (int64_t)Hkv * kHd, vstride = (int64_t)Hkv * DV;
  Stage stage;
  stage.init(tid, k_rot + (b * k_rows) * kstride + g * kHd, v + (b * v_rows) * vstride + g * DV, kstride, vstride,
             L);
  auto tile_j0 = [&](int idx) { return ix.tile_j0(idx); };

  // every workgroup has at least the tile of its own first position (ntiles >= 1)
  stage.fetch(tile_j0(0), stage0);
  stage.stash(stage0);
  wait_loads();
  __syncthreads();

  auto none_for = [&](int j0) { return ix.none_for(j0); };
  auto full_for = [&](int j0) { return ix.full_for(j0); };
  // 2^s of 16 shifted scores -> two B operands; l += their sum
  auto probs = [&](const f32x16_t& s, Frag& pa, Frag& pb) {
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) p[r] = fast_exp2(s[r]);
    pa = M::from_f32(&p[0]);
    pb = M::from_f32(&p[8]);
    float a[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) a[r] = p[r] + p[r + 8];
#pragma unroll
    for (int r = 0; r < 4; ++r) a[r] += a[r + 4];
    st.l += (a[0] + a[1]) + (a[2] + a[3]);
  };

  // one tile: scores from stage cur while the next tile loads into nxt
  auto tile = [&](int idx, lds_char* cur, lds_char* nxt) __attribute__((always_inline)) {
    const int jt = tile_j0(idx);
    // the next tile (after the last tile: rows that are staged but never
    // read), so that the loop body has no data-dependent branches
    stage.fetch(tile_j0(idx + 1), nxt);
    if (!(none_for(jt) && none_for(jt + 32))) {
      // K operands of both sub-tiles, then both score products
      // (the K operands of one sub-tile at a time: fewer live registers)
      f32x16_t s0 = st.negm, s1 = st.negm;
      {
        Frag kf[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) kf[c] = stage.kfrag(cur, c);
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) s0 = M::mma(kf[kc], qf[kc], s0);
      }
      {
        Frag kf[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) kf[c] = stage.kfrag(cur, 4 + c);
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) s1 = M::mma(kf[kc], qf[kc], s1);
      }
      // a sub-tile that some column sees only in part is masked (one that no
      // column of the wave sees ends up all -inf and adds nothing)
      if (!full_for(jt)) mask_scores(s0, lk, jt, hh, n_meta);
      if (!full_for(jt + 32)) mask_scores(s1, lk, jt + 32, hh, n_meta);
      mfma_result_wait(s0, s1);
      // this lane's max of both sub-tiles: four independent max3 chains
      float tm[4] = {s0[0], s0[1], s0[2], s0[3]};
#pragma unroll
      for (int r = 0; r < 4; ++r) tm[r] = max3f(tm[r], s1[r], s0[4 + r]);
#pragma unroll
      for (int r = 0; r < 4; ++r) tm[r] = max3f(tm[r], s1[4 + r], s0[8 + r]);
#pragma unroll
      for (int r = 0; r < 4; ++r) tm[r] = max3f(tm[r], s1[8 + r], s0[12 + r]);
#pragma unroll
      for (int r = 0; r < 4; ++r) tm[r] = max3f(tm[r], s1[12 + r], s1[12 + r]);
      const float t = max3f(tm[0], tm[1], max3f(tm[2], tm[3], tm[3]));
      if (__any(t > st.thr)) st.rescale(t, s0, &s1);
      // P of the first sub-tile and its V product, which runs while the second
      // sub-tile's P is formed
      // (the V operands of one dv block at a time)
      Frag pa, pb;
      probs(s0, pa, pb);
#pragma unroll
      for (int d = 0; d < NDB; ++d) {
        const Frag v0 = stage.vfrag(cur, d, 0), v1 = stage.vfrag(cur, d, 16);
        st.acc[d] = M::mma(v0, pa, st.acc[d]);
        st.acc[d] = M::mma(v1, pb, st.acc[d]);
      }
      probs(s1, pa, pb);
#pragma unroll
      for (int d = 0; d < NDB; ++d) {
        const Frag v0 = stage.vfrag(cur, d, 32), v1 = stage.vfrag(cur, d, 48);
        st.acc[d] = M::mma(v0, pa, st.acc[d]);
        st.acc[d] = M::mma(v1, pb, st.acc[d]);
      }
    }
    stage.stash(nxt);
    wait_loads();
    __syncthreads();
  };
  // two tiles per trip, so that each stage is a fixed object in each half
  for (int idx = 0;;) {
    tile(idx, stage0, stage1);
    if (++idx >= ntiles) break;
    tile(idx, stage1, stage0);
    if (++idx >= ntiles) break;
  }

  // normalise and store: lane holds O[column][32 d + 8 jj + 4 hh + (0..3)]
  const float l_tot = st.l + __shfl_xor(st.l, 32, 64);   // the column's sum over both lane halves
  if (my_q < L) {
    const float inv = 1.0f / l_tot;
    T* yrow = y + ((b * Lq + my_q - q_pos0) * Hq + h) * DV;
#pragma unroll
    for (int d = 0; d < NDB; ++d) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int c = 32 * d + 8 * jj + 4 * hh;
        const float o0 = st.acc[d][4 * jj + 0] * inv, o1 = st.acc[d][4 * jj + 1] * inv;
        const float o2 = st.acc[d][4 * jj + 2] * inv, o3 = st.acc[d][4 * jj + 3] * inv;
        if constexpr (sizeof(T) == 2) {
          uint2 w2;
          w2.x = pack_bf16x2(o0, o1);
          w2.y = pack_bf16x2(o2, o3);
          *reinterpret_cast<uint2*>(yrow + c) = w2;
        } else {
          *reinterpret_cast<float4*>(yrow + c) = make_float4(o0, o1, o2, o3);
        }
      }
    }
  }
}

// The prefill attention's visibility decisions, exported for exact tests:
// the same work order, tile walk, per-wave skip / unmasked decisions and
// per-lane masking as attn_prefill_kernel, applied to zero scores. For each
// query column the keys left finite are summarised as
// [meta_end, win_begin, win_end, count] (the ranges of the visible meta keys
// [0, meta_end) and window keys [win_begin, win_end), both n_meta when empty;
// count = keys taken). out: [batch, Lq, Hq, 4].
__global__ __launch_bounds__(64 * kAttnWaves) void prefill_visibility_kernel(int32_t* __restrict__ out, int Lq,
                                                                             int q_pos0, int n_meta, int window,
                                                                             int Hq, int Hkv, int batch, int n_cu) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5;
  PrefillIndex ix;
  ix.init((int)blockIdx.x, n_cu, Lq, q_pos0, n_meta, window, Hq, Hkv, batch, wave, lane);
  int count = 0, meta_end = 0, win_lo = INT32_MAX, win_hi = -1;
  for (int idx = 0; idx < ix.ntiles; ++idx) {
    const int jt = ix.tile_j0(idx);
    if (ix.none_for(jt) && ix.none_for(jt + 32)) continue;
    for (int half = 0; half < 2; ++half) {
      const int j0 = jt + 32 * half;
      f32x16_t sc;
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[r] = 0.f;
      if (!ix.full_for(j0)) mask_scores(sc, ix.lk, j0, hh, n_meta);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = j0 + 4 * hh + 8 * (r >> 2) + (r & 3);   // the key of score register r
        if (sc[r] != -INFINITY) {
          ++count;
          if (j < n_meta) {
            meta_end = max(meta_end, j + 1);
          } else {
            win_lo = min(win_lo, j);
            win_hi = max(win_hi, j + 1);
          }
        }
      }
    }
  }
  count += __shfl_xor(count, 32, 64);
  meta_end = max(meta_end, __shfl_xor(meta_end, 32, 64));
  win_lo = min(win_lo, __shfl_xor(win_lo, 32, 64));
  win_hi = max(win_hi, __shfl_xor(win_hi, 32, 64));
  if (ix.my_q < ix.L && hh == 0) {
    const bool any = win_hi >= 0;
    int32_t* o = out + ((ix.b * Lq + (ix.my_q - q_pos0)) * Hq + ix.h) * 4;
    o[0] = meta_end;
    o[1] = any ? win_lo : n_meta;
    o[2] = any ? win_hi : n_meta;
    o[3] = count;
  }
}

// ---------------------------------------------------------------------------
// Decode attention.
//
// decode_rope: rotates each sequence's queries and its new key to position
// p = cache_len[b] once (fp32, into the workspace).
// attn_decode: one workgroup per (chunk of the visible keys, kv head,
// sequence). The visible keys of row p are the meta rows, the window rows of
// the cache and the new row p itself, numbered meta first, then window. Each
// workgroup reads its chunk's K rows straight into registers (one key per
// thread), stages the V rows in LDS, and writes per query head of the group
// the partial (o, m, l) of an online softmax.
// decode_merge: one workgroup per (query head, sequence) merges the chunks'
// partials into the attention output of that head.

constexpr int kKeysPerSplit = 128;
constexpr int kMaxGroup = 10;

__device__ __forceinline__ int clamp_pos(int p, int cap) { return p < 0 ? 0 : (p > cap ? cap : p); }
// Position of a decode step's new row: cache_len, clamped so that no cache
// access leaves the buffer (a cache of one row per position holds rows < p;
// the compact ring holds any position, so only p >= 0 is needed there).
__device__ __forceinline__ int decode_pos(int cache_len, int cap, bool ring) {
  return ring ? max(cache_len, 0) : clamp_pos(cache_len, cap);
}
// Cache row of position j < p: the position itself, or, in the compact cache
// of a sliding-window layer, its row in the ring of `window` rows after the
// n_meta meta rows.
__device__ __forceinline__ int cache_row(int j, int n_meta, int window, bool ring) {
  return ring && j >= n_meta ? n_meta + (j - n_meta) % window : j;
}

template <typename T>
__global__ __launch_bounds__(256) void decode_rope_kernel(const T* __restrict__ q, const T* __restrict__ k_new,
                                                          const int32_t* __restrict__ cache_len,
                                                          float* __restrict__ q_rot, float* __restrict__ k_rot,
                                                          const float* __restrict__ k_scale, int batch, int Hq,
                                                          int Hkv, int cap, int ring, float base) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // (b, head, i)
  const int H = Hq + Hkv;
  if (idx >= (int64_t)batch * H * (kHd / 2)) return;
  const int i = (int)(idx % (kHd / 2));
  const int hd = (int)((idx / (kHd / 2)) % H);
  const int64_t b = idx / ((kHd / 2) * H);
  const int p = decode_pos(cache_len[b], cap, ring);
  float c, sn;
  rope_cs(p, i, base, &c, &sn);
  const T* src = hd < Hq ? q + (b * Hq + hd) * kHd : k_new + (b * Hkv + (hd - Hq)) * kHd;
  float* dst = hd < Hq ? q_rot + (b * Hq + hd) * kHd : k_rot + (b * Hkv + (hd - Hq)) * kHd;
  const float lo = to_f32(src[i]), hi = to_f32(src[i + 32]);
  float wlo = 1.f, whi = 1.f;   // shared-key affine on the query side: q (.) w of its kv group
  if (k_scale && hd < Hq) {
    const float* w = k_scale + (hd / (Hq / Hkv)) * kHd;
    wlo = w[i];
    whi = w[i + 32];
  }
  dst[i] = (lo * c - hi * sn) * wlo;
  dst[i + 32] = (hi * c + lo * sn) * whi;
}

template <typename T, int DV>
__global__ __launch_bounds__(256) void attn_decode_kernel(
    const float* __restrict__ q_rot, const float* __restrict__ k_rot, const T* __restrict__ v_new,
    const T* __restrict__ k_cache, const T* __restrict__ v_cache, const int32_t* __restrict__ cache_len,
    float* __restrict__ partial, int n_split, int cap, int n_meta, int window, int ring, int Hq, int Hkv) {
  constexpr int KS = kKeysPerSplit;
  constexpr int E = Vec16<T>::n;            // elements per 16-byte load
  __shared__ float qs[kMaxGroup][kHd];
  __shared__ float ps[kMaxGroup][KS];
  __shared__ __attribute__((aligned(16))) T Vs[KS][DV];

  const int s = blockIdx.x, g = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int group = Hq / Hkv;
  const int tid = threadIdx.x;
  const int p = decode_pos(cache_len[b], cap, ring);
  const MaskRange mr = mask_range(p, n_meta, window);
  const int n_vis = mr.meta_end + (mr.win_end - mr.win_begin);
  const int i0 = s * KS;
  const int nk = max(0, min(KS, n_vis - i0));
  float* outp = partial + (((b * Hq) + g * group) * n_split + s) * (DV + 2);
  const int64_t pstride = (int64_t)n_split * (DV + 2);  // between query heads

  if (nk == 0) {
    for (int t = tid; t < group * (DV + 2); t += blockDim.x) {
      const int hq = t / (DV + 2), e = t % (DV + 2);
      outp[hq * pstride + e] = e == DV ? -INFINITY : 0.f;
    }
    return;
  }
  auto key_row = [&](int vi) { return vi < mr.meta_end ? vi : mr.win_begin + (vi - mr.meta_end); };

  // V rows of the chunk -> LDS (raw copy)
  constexpr int VCH = DV / E;
  for (int it = tid; it < nk * VCH; it += blockDim.x) {
    const int kk = it / VCH, ch = it % VCH;
    const int j = key_row(i0 + kk);
    const T* src = j == p ? v_new + (b * Hkv + g) * DV
                          : v_cache + ((b * cap + cache_row(j, n_meta, window, ring)) * Hkv + g) * DV;
    *reinterpret_cast<uint4*>(&Vs[kk][ch * E]) = *reinterpret_cast<const uint4*>(src + ch * E);
  }
  for (int t = tid; t < group * kHd; t += blockDim.x) qs[t / kHd][t % kHd] = q_rot[(b * Hq + g * group) * kHd + t];
  // this thread's key row -> registers
  float kr[kHd];
  const bool has_key = tid < nk;
  if (has_key) {
    const int j = key_row(i0 + tid);
    if (j == p) {
#pragma unroll
      for (int d = 0; d < kHd; ++d) kr[d] = k_rot[(b * Hkv + g) * kHd + d];
    } else {
      const T* src = k_cache + ((b * cap + cache_row(j, n_meta, window, ring)) * Hkv + g) * kHd;
#pragma unroll
      for (int ch = 0; ch < kHd / E; ++ch) load16(src + ch * E, kr + ch * E);
    }
  }
  __syncthreads();
  if (tid < KS) {
    for (int hq = 0; hq < group; ++hq) {
      float a = 0.f;
#pragma unroll
      for (int d = 0; d < kHd; ++d) a = fmaf(qs[hq][d], kr[d], a);
      ps[hq][tid] = has_key ? a * kScaleLog2e : -INFINITY;
    }
  }
  __syncthreads();
  // softmax pieces: one wave per query head, two keys per lane
  const int lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  for (int hq = wave; hq < group; hq += nw) {
    const float s0 = ps[hq][lane], s1 = ps[hq][lane + 64];
    float m = fmaxf(s0, s1);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    const float p0 = fast_exp2(s0 - m), p1 = fast_exp2(s1 - m);   // exp2(-inf) = 0 for absent keys
    const float l = wave_sum(p0 + p1);
    ps[hq][lane] = p0;
    ps[hq][lane + 64] = p1;
    if (lane == 0) {
      outp[hq * pstride + DV] = m;
      outp[hq * pstride + DV + 1] = l;
    }
  }
  __syncthreads();
  // o[h][d..d+3] = sum_k p[h][k] v[k][d..d+3]
  constexpr int NQ = DV / 4;
  for (int t = tid; t < group * NQ; t += blockDim.x) {
    const int hq = t / NQ, dq = t % NQ;
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    for (int kk = 0; kk < nk; ++kk) {
      const float pk = ps[hq][kk];
      float v4[4];
      if constexpr (sizeof(T) == 2) {
        const uint2 w2 = *reinterpret_cast<const uint2*>(&Vs[kk][4 * dq]);
        v4[0] = bf16_lo(w2.x); v4[1] = bf16_hi(w2.x); v4[2] = bf16_lo(w2.y); v4[3] = bf16_hi(w2.y);
      } else {
        const float4 w4 = *reinterpret_cast<const float4*>(&Vs[kk][4 * dq]);
        v4[0] = w4.x; v4[1] = w4.y; v4[2] = w4.z; v4[3] = w4.w;
      }
      a0 = fmaf(pk, v4[0], a0); a1 = fmaf(pk, v4[1], a1);
      a2 = fmaf(pk, v4[2], a2); a3 = fmaf(pk, v4[3], a3);
    }
    *reinterpret_cast<float4*>(outp + hq * pstride + 4 * dq) = make_float4(a0, a1, a2, a3);
  }
}

constexpr int kDecodeTile = 32;     // keys per partial slot in the workspace (the most splits a launch uses)
constexpr int kMaxGroupFlash = 8;   // query heads per kv head (larger groups are rejected up front)

// Flash-decoding, one wave per split: the wave of (split s, kv head g,
// sequence b) streams its own run of 32-key tiles and keeps every dv block, so
// no score or softmax work is repeated across waves (the heads of a group are
// the MFMA columns, padded to 32). K goes from the cache straight into the
// operand registers (a lane holds one key row, 16 bytes per 16 dims); V is
// staged in LDS, two 32-row stages per wave, for the transposing operand
// reads. The new row p, absent from the read-only cache, opens split 0's
// online softmax before its first tile. The running maximum is raised only
// when a tile's maximum exceeds it by more than kRescaleSlack (base-2 units),
// so most tiles skip rescaling the accumulators. Writes the same partials
// (o, m, l) per split as the other decode kernels.
constexpr int kWaveTile = 32;   // keys per tile

// The decode step of the Mamba branch (ssm_step.hpp) as done by the extra
// workgroups of the attention launch: wave r of R for sequence b takes the
// channels r * 16 + i * R * 16 .. + 15 (one lane quad each), kSsmRoleItems
// of them per lane quad with all their loads in flight together. The step
// reads and rewrites the fp32 state while the attention workgroups stream
// the cache, instead of in a launch of its own before them.
constexpr int kSsmRoleItems = 4;
constexpr int kDecodeSsmReserve = 2;   // wave slots per CU the split plan leaves to them
__device__ __forceinline__ void decode_ssm_role(const ssm_step::Ptrs<bf16>& p, int r, int R, int64_t b) {
  const int q = threadIdx.x & 3, quad = threadIdx.x >> 2;
  const int stride = R * 16;
  for (int c0 = r * 16; c0 < p.d_inner; c0 += kSsmRoleItems * stride) {   // wave-uniform
    ssm_step::Item<bf16> it[kSsmRoleItems];
#pragma unroll
    for (int k = 0; k < kSsmRoleItems; ++k) {
      const int c = c0 + k * stride + quad;
      const bool ok = c < p.d_inner;   // the same for the whole quad
      ssm_step::load(p, it[k], b, ok ? c : 0, q, ok);
    }
#pragma unroll
    for (int k = 0; k < kSsmRoleItems; ++k) ssm_step::finish(p, it[k], q);
  }
}

template <int DV, bool RING>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2)))
void attn_decode_wave_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k_new, const bf16* __restrict__ v_new,
    const bf16* __restrict__ k_cache, const bf16* __restrict__ v_cache, const int32_t* __restrict__ cache_len,
    float* __restrict__ partial, const float* __restrict__ k_scale, int n_split, int cap, int n_meta, int window,
    int Hq, int Hkv, double freq_step, ssm_step::Ptrs<bf16> ssm) {
  if ((int)blockIdx.x >= n_split) {   // a workgroup of the Mamba step (see decode_ssm_role)
    decode_ssm_role(ssm, ((int)blockIdx.x - n_split) * (int)gridDim.y + (int)blockIdx.y,
                    ((int)gridDim.x - n_split) * (int)gridDim.y, blockIdx.z);
    return;
  }
  typedef Mma<bf16> M;
  constexpr int KROWB = kHd * 2, VROWB = DV * 2;        // bytes per K / V row
  constexpr int VCH = VROWB / 16;                       // 16-byte chunks per V row
  constexpr int VN = kWaveTile * VCH / 64;              // V loads per lane per tile
  constexpr int VSTAGE = kWaveTile * VROWB;
  constexpr int NDB = DV / 32;                          // 32-wide dv blocks
  constexpr int VRPB = VROWB >= 256 ? 1 : 256 / VROWB;  // V rows per 256-byte bank sweep
  static_assert(kWaveTile * VCH % 64 == 0 && VN + 4 < 64, "tile shape");
  __shared__ __attribute__((aligned(16))) char lds_v0[VSTAGE];
  __shared__ __attribute__((aligned(16))) char lds_v1[VSTAGE];
  __shared__ float rope_c[kHd / 2], rope_s[kHd / 2];
  __shared__ __attribute__((aligned(16))) uint16_t q_lds[kMaxGroupFlash][kHd];   // bf16 bits
  lds_char* const vst0 = (lds_char*)lds_v0;
  lds_char* const vst1 = (lds_char*)lds_v1;
  auto vsw = [](int row) { return (4 * ((row & 3) / VRPB)) & (VCH - 1); };

  const int s = blockIdx.x, g = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int group = Hq / Hkv;
  const int lane = threadIdx.x;
  const int lq = lane & 31, hh = lane >> 5;
  const bool has_new = s == 0;
  const int len = cache_len[b];
  // The wave's small inputs are loaded first, all together and without
  // branches, ahead of the cache stream that the whole chip starts at once
  // (behind it they would wait as long as a tile): the group's query pairs
  // (dims i, i + 32 of head h for item 32 h + i; kQItems items per lane) with
  // their shared-key weights (a null k_scale reads as zeros from an empty
  // descriptor: weight 1), the new row's key (all 64 dims) and this lane's
  // values of v_new (used by split 0 only).
  constexpr int kQItems = kMaxGroupFlash * (kHd / 2) / 64;
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(q + (b * Hq + g * group) * kHd, (uint32_t)(group * kHd * 2));
  const __amdgpu_buffer_rsrc_t wrs = make_rsrc(k_scale ? k_scale + g * kHd : nullptr, k_scale ? kHd * 4 : 0);
  const float w_one = k_scale ? 0.f : 1.f;
  uint32_t qlo[kQItems], qhi[kQItems];
  float wpl[kQItems], wph[kQItems];
#pragma unroll
  for (int j = 0; j < kQItems; ++j) {
    const int it = lane + 64 * j, qh = it / (kHd / 2), qi = it % (kHd / 2);
    const uint32_t off = qh < group ? (uint32_t)(qh * kHd + qi) * 2 : kBufferNowhere;
    qlo[j] = __builtin_amdgcn_raw_buffer_load_b16(qrs, off, 0, 0);
    qhi[j] = __builtin_amdgcn_raw_buffer_load_b16(qrs, off + kHd, 0, 0);
    wpl[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(wrs, (uint32_t)qi * 4, 0, 0));
    wph[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(wrs, (uint32_t)(qi + kHd / 2) * 4, 0, 0));
  }
  const __amdgpu_buffer_rsrc_t knrs = make_rsrc(k_new + (b * Hkv + g) * kHd, kHd * 2);
  const __amdgpu_buffer_rsrc_t vnrs = make_rsrc(v_new + (b * Hkv + g) * DV, DV * 2);
  u32x4_t knew[kHd / 8];
#pragma unroll
  for (int c = 0; c < kHd / 8; ++c) knew[c] = buf_load16(knrs, 16 * c);
  u32x2_t vnew[DV / 32][4];
#pragma unroll
  for (int d = 0; d < DV / 32; ++d)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      vnew[d][rr] = __builtin_amdgcn_raw_buffer_load_b64(vnrs, (uint32_t)(32 * d + 8 * rr + 4 * hh) * 2, 0, 0);
  const int p = decode_pos(len, cap, RING);
  const MaskRange mr = mask_range(p, n_meta, window);
  // visible keys held in the cache: all but the last visible key, the new row p
  const int n_old = mr.meta_end + (mr.win_end - mr.win_begin) - 1;
  const int n_tiles = (n_old + kWaveTile - 1) / kWaveTile;
  const int per = (n_tiles + n_split - 1) / n_split;
  const int t0 = min(n_tiles, s * per), t1 = min(n_tiles, t0 + per);
  float* outp = partial + (((b * Hq) + g * group) * n_split + s) * (DV + 2);
  const int64_t pstride = (int64_t)n_split * (DV + 2);   // between query heads
  if (t0 >= t1 && !has_new) {
    for (int t = lane; t < group * (DV + 2); t += 64) {
      const int hq = t / (DV + 2), e = t % (DV + 2);
      outp[hq * pstride + e] = e == DV ? -INFINITY : 0.f;
    }
    return;
  }
  // cache row of visible key vi (meta keys first, then the window in order);
  // in the ring, window key o is at ring row w0 + o folded once into [0, window)
  const int w0 = RING ? (mr.win_begin - n_meta) % window : 0;
  auto key_row = [&](int vi) {
    if constexpr (RING) {
      const int r = w0 + (vi - mr.meta_end);
      return vi < mr.meta_end ? vi : n_meta + (r >= window ? r - window : r);
    } else {
      return vi < mr.meta_end ? vi : mr.win_begin + (vi - mr.meta_end);
    }
  };
  // tile t: row r is visible key 32 t + r; rows at or past n_old read zeros
  const uint32_t kv_row = (uint32_t)Hkv * KROWB, vv_row = (uint32_t)Hkv * VROWB;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(k_cache + b * cap * Hkv * kHd, (uint32_t)cap * kv_row);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(v_cache + b * cap * Hkv * DV, (uint32_t)cap * vv_row);
  // V rows into LDS with the 16-byte chunks of row r XOR-swizzled by vsw(r)
  auto fetch_v = [&](int t, lds_char* dst) {
#pragma unroll
    for (int r = 0; r < VN; ++r) {
      const int it = r * 64 + lane, row = it / VCH, cp = it % VCH, vi = kWaveTile * t + row;
      const uint32_t off = vi < n_old ? (uint32_t)key_row(vi) * vv_row + (uint32_t)(g * VROWB + 16 * (cp ^ vsw(row)))
                                      : kBufferNowhere;
      buf_load16_lds(vrs, off, dst + r * 64 * 16);
    }
  };
  // the K operand: lane (row lq, half hh) holds dims 16 kc + 8 hh .. + 7 of key 32 t + lq
  auto fetch_k = [&](int t, M::Frag* kf) {
    const int vi = kWaveTile * t + lq;
    const uint32_t off = vi < n_old ? (uint32_t)key_row(vi) * kv_row + (uint32_t)(g * KROWB + 16 * hh) : kBufferNowhere;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) kf[kc] = __builtin_bit_cast(M::Frag, buf_load16(krs, off + 32 * kc));
  };
  // loads in a fixed order (V then K), so that a wait for the K operand of
  // tile t also covers tile t's V rows; the first two tiles go out before the
  // prologue's own work
  M::Frag kfa[4], kfb[4];
  if (t0 < t1) {
    fetch_v(t0, vst0);
    __builtin_amdgcn_sched_barrier(0);
    fetch_k(t0, kfa);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (t0 + 1 < t1) {
    fetch_v(t0 + 1, vst1);
    __builtin_amdgcn_sched_barrier(0);
    fetch_k(t0 + 1, kfb);
    __builtin_amdgcn_sched_barrier(0);
  }

  // the group's queries at position p, times the shared-key weights w[g] and
  // log2(e)/sqrt(64), as bf16 in LDS: item (head h, pair i) rotates dims i, i + 32
  if (lane < kHd / 2) rope_cs_step(p, lane, freq_step, &rope_c[lane], &rope_s[lane]);
  lds_barrier();   // (a __syncthreads() would also wait for the tile in flight)
#pragma unroll
  for (int j = 0; j < kQItems; ++j) {
    const int it = lane + 64 * j, qh = it / (kHd / 2), qi = it % (kHd / 2);
    if (qh < group) {
      const float lo = __uint_as_float(qlo[j] << 16), hi = __uint_as_float(qhi[j] << 16);
      const float c = rope_c[qi], sn = rope_s[qi];
      q_lds[qh][qi] = f32_to_bf16_bits((lo * c - hi * sn) * (wpl[j] + w_one) * kScaleLog2e);
      q_lds[qh][qi + kHd / 2] = f32_to_bf16_bits((hi * c + lo * sn) * (wph[j] + w_one) * kScaleLog2e);
    }
  }
  lds_barrier();
  // Q^T operand: column lq (query head of the group), dims 16 kc + 8 hh .. + 7;
  // columns past the group are zero
  const bool qv = lq < group;
  M::Frag qf[4];
#pragma unroll
  for (int kc = 0; kc < 4; ++kc) {
    const M::Frag f = *(const __attribute__((address_space(3))) M::Frag*)((lds_char*)q_lds + (qv ? lq : 0) * (kHd * 2) +
                                                                          32 * kc + 16 * hh);
    qf[kc] = qv ? f : M::zero();
  }

  // accumulators: O^T block d, register r holds dv 32 d + 8 (r / 4) + 4 hh + r % 4 of column lq
  f32x16_t acc[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[d][r] = 0.f;
  float m = -INFINITY, l = 0.f;
  if (has_new) {
    // score of the new key (rotated, rounded to bf16 like a cached key) against
    // this column's query, over this lane's 32 dims, then both lane halves
    auto kval = [&](int dim) {   // raw dim of the new key (lane-uniform register index after unrolling)
      const uint32_t w = knew[dim >> 3][(dim >> 1) & 3];
      return (dim & 1) ? bf16_hi(w) : bf16_lo(w);
    };
    float dot = 0.f;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int dim0 = 16 * kc + e;                 // this lane's dim is dim0 + 8 hh
        const int dim = dim0 + 8 * hh, i = dim & (kHd / 2 - 1);
        const float x = hh ? kval(dim0 + 8) : kval(dim0);
        const float xp = hh ? kval((dim0 + 8) ^ (kHd / 2)) : kval(dim0 ^ (kHd / 2));
        const float kr = dim < kHd / 2 ? x * rope_c[i] - xp * rope_s[i] : x * rope_c[i] + xp * rope_s[i];
        const float qd = __uint_as_float((uint32_t)q_lds[qv ? lq : 0][dim] << 16);
        dot = fmaf(qv ? qd : 0.f, __uint_as_float((uint32_t)f32_to_bf16_bits(kr) << 16), dot);
      }
    m = dot + __shfl_xor(dot, 32, 64);
    l = hh == 0 ? 1.f : 0.f;   // its weight 2^(s - m) = 1, counted once per column
#pragma unroll
    for (int d = 0; d < NDB; ++d)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const u32x2_t w2 = vnew[d][rr];
        acc[d][4 * rr] = bf16_lo(w2.x);
        acc[d][4 * rr + 1] = bf16_hi(w2.x);
        acc[d][4 * rr + 2] = bf16_lo(w2.y);
        acc[d][4 * rr + 3] = bf16_hi(w2.y);
      }
  }
  float thr = m + kRescaleSlack;   // -inf without the new key: the first tile sets the maximum

  // per-lane LDS offset of the V operand reads: in each 16-lane group gi, lane
  // j = 4 k + q reads V[4 (gi / 2) + k][16 (gi % 2) + 4 q .. + 3] (transposed)
  const int gi = lane >> 4, jj = lane & 15;
  const int vrow_l = 4 * (gi >> 1) + (jj >> 2);
  const int vdv = 16 * (gi & 1) + 4 * (jj & 3);
  const int vro = vrow_l * VROWB + 16 * ((vdv >> 3) ^ vsw(vrow_l)) + 8 * ((vdv >> 2) & 1);
  typedef __attribute__((address_space(3))) v4i16_t lds_v4;
  typedef short v8i16_t __attribute__((ext_vector_type(8)));

  // tile t from (cur, kf); tile t + 1 loads into (nxt, kn) (for the first
  // tile it is already on its way)
  auto tile = [&](int t, lds_char* cur, lds_char* nxt, const M::Frag* kf, M::Frag* kn) __attribute__((always_inline)) {
    if (t > t0 && t + 1 < t1) {
      fetch_v(t + 1, nxt);
      __builtin_amdgcn_sched_barrier(0);
      fetch_k(t + 1, kn);
      __builtin_amdgcn_sched_barrier(0);
    }
    // scores: lane holds keys 32 t + 8 (r / 4) + 4 hh + r % 4 of column lq
    f32x16_t sc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[r] = 0.f;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) sc = M::mma(kf[kc], qf[kc], sc);
    const int vbase = kWaveTile * t;
    if (vbase + kWaveTile > n_old) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = vbase + 8 * (r >> 2) + 4 * hh + (r & 3);
        sc[r] = key < n_old ? sc[r] : -INFINITY;
      }
    }
    mfma_result_wait(sc);
    float tm[4] = {sc[0], sc[1], sc[2], sc[3]};
#pragma unroll
    for (int r = 0; r < 4; ++r) tm[r] = max3f(tm[r], sc[4 + r], sc[8 + r]);
#pragma unroll
    for (int r = 0; r < 4; ++r) tm[r] = fmaxf(tm[r], sc[12 + r]);
    const float tmx = max3f(tm[0], tm[1], fmaxf(tm[2], tm[3]));
    if (__any(tmx > thr)) {
      const float mn = fmaxf(m, fmaxf(tmx, __shfl_xor(tmx, 32, 64)));   // the column's maximum
      const float alpha = fast_exp2(m - mn);                             // 0 while m = -inf
      m = mn;
      thr = mn + kRescaleSlack;
      l *= alpha;
#pragma unroll
      for (int d = 0; d < NDB; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[d][r] *= alpha;
    }
    float pv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) pv[r] = fast_exp2(sc[r] - m);
    float a8[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) a8[r] = pv[r] + pv[r + 8];
#pragma unroll
    for (int r = 0; r < 4; ++r) a8[r] += a8[r + 4];
    l += (a8[0] + a8[1]) + (a8[2] + a8[3]);
    const M::Frag pf0 = M::from_f32(&pv[0]), pf1 = M::from_f32(&pv[8]);
    // tile t's V rows have landed once at most this many loads are outstanding
    // (tile t + 1's V and K, issued after them)
    __builtin_amdgcn_s_waitcnt(((VN + 4) & 15) | (((VN + 4) >> 4) << 14) | 0x0F70);   // vmcnt(VN + 4)
    asm volatile("" ::: "memory");
#pragma unroll
    for (int d = 0; d < NDB; ++d) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const lds_char* vp = cur + ((vro ^ (d << 6)) + 16 * kk * VROWB);
        const v4i16_t va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)vp);
        const v4i16_t vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(vp + 8 * VROWB));
        const v8i16_t v8 = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
        acc[d] = M::mma(__builtin_bit_cast(M::Frag, v8), kk ? pf1 : pf0, acc[d]);
      }
    }
    // the V reads of this stage are done before a later tile loads into it
    __builtin_amdgcn_s_waitcnt(0xC07F);
    asm volatile("" ::: "memory");
  };
  for (int t = t0; t < t1;) {
    tile(t, vst0, vst1, kfa, kfb);
    if (++t >= t1) break;
    tile(t, vst1, vst0, kfb, kfa);
    ++t;
  }

  l += __shfl_xor(l, 32, 64);
  if (qv) {
    float* o = outp + lq * pstride;
#pragma unroll
    for (int d = 0; d < NDB; ++d)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<float4*>(o + 32 * d + 8 * q4 + 4 * hh) =
            make_float4(acc[d][4 * q4], acc[d][4 * q4 + 1], acc[d][4 * q4 + 2], acc[d][4 * q4 + 3]);
    if (hh == 0) {
      o[DV] = m;
      o[DV + 1] = l;
    }
  }
}

// Decode epilogue, one workgroup per sequence: merge the split partials of
// every query head, y = sum_s o_s 2^(m_s - m) / sum_s l_s 2^(m_s - m), write
// the attention output and fuse it with the Mamba output as the prefill fusion
// does (RMS-normalise each branch over the row, scale by the betas, average),
// from the merged values in registers.
constexpr int kCombineMaxThreads = 1024;
constexpr int kCombineItems = 4;   // (head, 4 dv) items per thread at most: up to 16384 channels
constexpr int kMergeBatch = 8;     // split partials loaded together

template <typename T, int DV, int KI>
__global__ __launch_bounds__(kCombineMaxThreads) void decode_combine_kernel(
    const float* __restrict__ partial, const T* __restrict__ ys, const float* __restrict__ ba,
    const float* __restrict__ bs, float eps, int n_split, int Hq, T* __restrict__ y_attn, T* __restrict__ out) {
  constexpr int NQ = DV / 4;
  __shared__ float red[2][kCombineMaxThreads / 64];
  const int64_t b = blockIdx.x;
  const int tid = threadIdx.x;
  const int nt = blockDim.x;   // whole waves
  const int width = Hq * DV;
  const int n_items = Hq * NQ;
  float ya[KI][4], yv[KI][4], bav[KI][4], bsv[KI][4];
  float sa = 0.f, ss = 0.f;
  // the Mamba output and the betas first: their loads overlap the merge's
#pragma unroll
  for (int k = 0; k < KI; ++k) {
    const int it = tid + k * nt;
    if (it < n_items) {
      const int c = (it / NQ) * DV + 4 * (it % NQ);
      if constexpr (sizeof(T) == 2) {
        const uint2 w2 = *reinterpret_cast<const uint2*>(ys + b * width + c);
        yv[k][0] = bf16_lo(w2.x); yv[k][1] = bf16_hi(w2.x); yv[k][2] = bf16_lo(w2.y); yv[k][3] = bf16_hi(w2.y);
      } else {
        load16(ys + b * width + c, yv[k]);
      }
      load16(ba + c, bav[k]);
      load16(bs + c, bsv[k]);
    }
  }
#pragma unroll
  for (int k = 0; k < KI; ++k) {
    const int it = tid + k * nt;
    if (it < n_items) {
      const int h = it / NQ, dq = it % NQ;
      const float* ph = partial + ((b * Hq) + h) * (int64_t)n_split * (DV + 2);
      // the splits in batches of kMergeBatch, every load of a batch issued
      // before the first use (past n_split: the last split again, weighted 0)
      float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
      for (int s0 = 0; s0 < n_split; s0 += kMergeBatch) {
        float ms[kMergeBatch], ls[kMergeBatch];
        float4 os[kMergeBatch];
#pragma unroll
        for (int j = 0; j < kMergeBatch; ++j) {
          const float* q = ph + min(s0 + j, n_split - 1) * (DV + 2);
          ms[j] = q[DV];
          ls[j] = q[DV + 1];
          os[j] = *reinterpret_cast<const float4*>(q + 4 * dq);
        }
        float mb = m;
#pragma unroll
        for (int j = 0; j < kMergeBatch; ++j) mb = fmaxf(mb, s0 + j < n_split ? ms[j] : -INFINITY);
        if (mb != -INFINITY) {   // (else every split so far is empty)
          const float fo = m == -INFINITY ? 0.f : fast_exp2(m - mb);
          l *= fo; o0 *= fo; o1 *= fo; o2 *= fo; o3 *= fo;
#pragma unroll
          for (int j = 0; j < kMergeBatch; ++j) {
            const float f = (s0 + j < n_split && ms[j] != -INFINITY) ? fast_exp2(ms[j] - mb) : 0.f;
            l = fmaf(ls[j], f, l);
            o0 = fmaf(os[j].x, f, o0); o1 = fmaf(os[j].y, f, o1); o2 = fmaf(os[j].z, f, o2); o3 = fmaf(os[j].w, f, o3);
          }
          m = mb;
        }
      }
      const float il = 1.0f / l;
      ya[k][0] = o0 * il; ya[k][1] = o1 * il; ya[k][2] = o2 * il; ya[k][3] = o3 * il;
      const int c = h * DV + 4 * dq;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sa = fmaf(ya[k][e], ya[k][e], sa);
        ss = fmaf(yv[k][e], yv[k][e], ss);
      }
      float w4[8] = {ya[k][0], ya[k][1], ya[k][2], ya[k][3], 0.f, 0.f, 0.f, 0.f};
      if constexpr (sizeof(T) == 2) {
        uint2 w2;
        w2.x = pack_bf16x2(w4[0], w4[1]);
        w2.y = pack_bf16x2(w4[2], w4[3]);
        *reinterpret_cast<uint2*>(y_attn + b * width + c) = w2;
      } else {
        store16(y_attn + b * width + c, w4);
      }
    }
  }
  sa = wave_sum(sa);
  ss = wave_sum(ss);
  if ((tid & 63) == 0) {
    red[0][tid >> 6] = sa;
    red[1][tid >> 6] = ss;
  }
  __syncthreads();
  sa = 0.f;
  ss = 0.f;
  for (int w = 0; w < nt / 64; ++w) {
    sa += red[0][w];
    ss += red[1][w];
  }
  const float inv_w = 1.0f / (float)width;
  const float ra = 0.5f / sqrtf(sa * inv_w + eps);
  const float rs = 0.5f / sqrtf(ss * inv_w + eps);
#pragma unroll
  for (int k = 0; k < KI; ++k) {
    const int it = tid + k * nt;
    if (it < n_items) {
      const int c = (it / NQ) * DV + 4 * (it % NQ);
      float r[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = fmaf(bav[k][e] * ra, ya[k][e], bsv[k][e] * rs * yv[k][e]);
      if constexpr (sizeof(T) == 2) {
        uint2 w2;
        w2.x = pack_bf16x2(r[0], r[1]);
        w2.y = pack_bf16x2(r[2], r[3]);
        *reinterpret_cast<uint2*>(out + b * width + c) = w2;
      } else {
        store16(out + b * width + c, r);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// KV row copies between a cache (one row per position, or the compact ring)
// and the rows the prefill attention reads. Workgroup = (copy index, sequence);
// 16-byte pieces of the K row, then of the V row.
__device__ __forceinline__ int64_t kv_side_row(int mode, int base, int i, int P, int n_meta, int window) {
  if (mode == KvSide::kIndex) return i;
  if (mode == KvSide::kLinear) return P - base;
  return cache_row(P, n_meta, window, true);
}

__global__ __launch_bounds__(64) void kv_copy_kernel(KvCopyArgs a, int k_row_bytes, int v_row_bytes) {
  const int i = blockIdx.x;
  const int64_t b = blockIdx.y;
  const int P = i < a.na ? a.pa + i : a.pb + (i - a.na);
  const int64_t sr = kv_side_row(a.src.mode, a.src.base, i, P, a.n_meta, a.window);
  const int64_t dr = kv_side_row(a.dst.mode, a.dst.base, i, P, a.n_meta, a.window);
  const char* sk = (const char*)a.src.k + (b * a.src.k_rows + sr) * k_row_bytes;
  const char* sv = (const char*)a.src.v + (b * a.src.v_rows + sr) * v_row_bytes;
  char* dk = (char*)a.dst.k + (b * a.dst.k_rows + dr) * k_row_bytes;
  char* dv = (char*)a.dst.v + (b * a.dst.v_rows + dr) * v_row_bytes;
  for (int o = 16 * (int)threadIdx.x; o < k_row_bytes; o += 16 * 64)
    *reinterpret_cast<uint4*>(dk + o) = *reinterpret_cast<const uint4*>(sk + o);
  for (int o = 16 * (int)threadIdx.x; o < v_row_bytes; o += 16 * 64)
    *reinterpret_cast<uint4*>(dv + o) = *reinterpret_cast<const uint4*>(sv + o);
}

}  // namespace

hipError_t launch_kv_copy(const KvCopyArgs& a, hipStream_t stream) {
  if (a.n <= 0 || a.batch <= 0) return hipSuccess;
  const int es = a.act == HYMBA_BF16 ? 2 : 4;
  const int k_row_bytes = a.n_kv_heads * kHd * es, v_row_bytes = a.n_kv_heads * a.head_dim_v * es;
  hipLaunchKernelGGL(kv_copy_kernel, dim3((unsigned)a.n, (unsigned)a.batch), dim3(64), 0, stream, a, k_row_bytes,
                     v_row_bytes);
  return hipGetLastError();
}

namespace {

template <typename T>
hipError_t rope_t(const RopeArgs& a, hipStream_t stream, Timing tm) {
  dim3 grid((a.L + kRopeRows - 1) / kRopeRows, a.batch);
  HYMBA_LAUNCH(rope_prefill_kernel<T>, grid, dim3(kRopeThreads), 0, stream, tm, (const T*)a.q, (const T*)a.k,
                     (const T*)a.v, (T*)a.q_rot, (T*)a.k_rot, (T*)a.v_copy, a.k_rows, a.v_rows, a.k_row0,
                     a.v_row0, a.k_scale, a.L, a.pos0, a.n_q_heads,
                     a.n_kv_heads, a.head_dim_v, std::pow((double)a.rope_base, -2.0 / kHd), kScaleLog2e);
  return hipGetLastError();
}

template <typename T, int DV>
hipError_t attn_prefill_t(const AttnPrefillArgs& a, hipStream_t stream, Timing tm) {
  const int G = a.n_q_heads / a.n_kv_heads;
  const int P = kAttnCols / G;   // positions per workgroup
  const int64_t hb_n = (int64_t)a.n_kv_heads * a.batch;
  const int64_t n_items = (int64_t)((a.L + P - 1) / P) * hb_n;
  const int n_xcd = a.n_cu / 32;
  // the XCD-major order of PrefillIndex (many rounds of workgroups)
  const bool many = n_items > 2 * (int64_t)a.n_cu && n_xcd > 1 && hb_n % n_xcd == 0;
#define HYMBA_ATTN_PREFILL(OCC)                                                                                   \
  HYMBA_LAUNCH((attn_prefill_kernel<T, DV, OCC>), dim3((unsigned)n_items), dim3(64 * kAttnWaves), 0, stream, tm, \
               (const T*)a.q_rot, (const T*)a.k_rot, (const T*)a.v, (T*)a.y, a.k_rows, a.v_rows, a.L, a.q_pos0,   \
               a.n_meta, a.window, a.n_q_heads, a.n_kv_heads, a.batch, a.n_cu)
  if constexpr (sizeof(T) == 2) {
    if (many)
      HYMBA_ATTN_PREFILL(3);
    else
      HYMBA_ATTN_PREFILL(2);
  } else {
    HYMBA_ATTN_PREFILL(1);
  }
#undef HYMBA_ATTN_PREFILL
  return hipGetLastError();
}

template <typename T, int DV>
hipError_t attn_decode_t(const AttnDecodeArgs& a, hipStream_t stream, Timing tm) {
  Timing t_first, t_last;   // the stage's start on its first kernel, its end on its last
  t_first.start = tm.start;
  t_last.stop = tm.stop;
  if constexpr (sizeof(T) == 2) {
    // rotation inside the attention kernel: one launch for the stage, with
    // the Mamba step's workgroups (if any) after each (kv head, sequence)'s
    // splits: as many per (kv head, sequence) as the wave slots the attention
    // leaves free hold (at least one), so that the whole grid is resident
    const double freq_step = std::pow((double)a.rope_base, -2.0 / kHd);
    int ssm_x = 0;
    ssm_step::Ptrs<bf16> sp = {};
    if (a.ssm) {
      sp = ssm_step_ptrs<bf16>(*a.ssm);
      const int64_t rows = (int64_t)a.batch * a.n_kv_heads;
      const int64_t slots = decode_wave_slots_per_cu(DV) * (int64_t)a.n_cu;
      ssm_x = (int)std::max<int64_t>(1, (slots - (int64_t)a.n_split * rows) / std::max<int64_t>(1, rows));
      // (no more waves per sequence than 16-channel groups)
      const int64_t groups = ((int64_t)a.ssm->d_inner + 15) / 16;
      ssm_x = (int)std::min<int64_t>(ssm_x, std::max<int64_t>(1, (groups + a.n_kv_heads - 1) / a.n_kv_heads));
    }
    const dim3 grid((unsigned)(a.n_split + ssm_x), (unsigned)a.n_kv_heads, (unsigned)a.batch);
    if (a.ring)
      HYMBA_LAUNCH((attn_decode_wave_kernel<DV, true>), grid, dim3(64), 0, stream, tm, (const bf16*)a.q,
                   (const bf16*)a.k_new, (const bf16*)a.v_new, (const bf16*)a.k_cache, (const bf16*)a.v_cache,
                   a.cache_len, a.partial, a.k_scale, a.n_split, a.cap, a.n_meta, a.window, a.n_q_heads,
                   a.n_kv_heads, freq_step, sp);
    else
      HYMBA_LAUNCH((attn_decode_wave_kernel<DV, false>), grid, dim3(64), 0, stream, tm, (const bf16*)a.q,
                   (const bf16*)a.k_new, (const bf16*)a.v_new, (const bf16*)a.k_cache, (const bf16*)a.v_cache,
                   a.cache_len, a.partial, a.k_scale, a.n_split, a.cap, a.n_meta, a.window, a.n_q_heads,
                   a.n_kv_heads, freq_step, sp);
    return hipGetLastError();
  }
  const int64_t n = (int64_t)a.batch * (a.n_q_heads + a.n_kv_heads) * (kHd / 2);
  HYMBA_LAUNCH(decode_rope_kernel<T>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, t_first, (const T*)a.q,
                     (const T*)a.k_new, a.cache_len, a.q_rot, a.k_rot, a.k_scale, a.batch, a.n_q_heads,
                     a.n_kv_heads, a.cap, a.ring,
                     a.rope_base);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  HYMBA_LAUNCH((attn_decode_kernel<T, DV>), dim3(a.n_split, a.n_kv_heads, a.batch), dim3(256), 0, stream, t_last,
                 a.q_rot, a.k_rot, (const T*)a.v_new, (const T*)a.k_cache, (const T*)a.v_cache, a.cache_len,
                 a.partial, a.n_split, a.cap, a.n_meta, a.window, a.ring, a.n_q_heads, a.n_kv_heads);
  return hipGetLastError();
}

template <typename T, int DV>
hipError_t combine_t(const DecodeCombineArgs& a, hipStream_t stream, Timing tm) {
  // whole waves, one (head, 4 dv) item per thread while that fits in one
  // workgroup, else up to kCombineItems each (the row stays in registers)
  const int n_items = a.n_q_heads * (DV / 4);
  const int per = (n_items + kCombineMaxThreads - 1) / kCombineMaxThreads;
  const int threads = std::max(64, (n_items + 64 * per - 1) / (64 * per) * 64);
  if (per > kCombineItems) return hipErrorInvalidValue;
  if (threads > kCombineMaxThreads) return hipErrorInvalidValue;
#define HYMBA_COMBINE(KI)                                                                                    \
  HYMBA_LAUNCH((decode_combine_kernel<T, DV, KI>), dim3(a.batch), dim3(threads), 0, stream, tm, a.partial,   \
               (const T*)a.y_ssm, a.beta_attn, a.beta_ssm, a.eps, a.n_split, a.n_q_heads, (T*)a.y_attn, (T*)a.out)
  if (per == 1)
    HYMBA_COMBINE(1);
  else if (per == 2)
    HYMBA_COMBINE(2);
  else
    HYMBA_COMBINE(4);
#undef HYMBA_COMBINE
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

hipError_t launch_prefill_visibility(int batch, int Lq, int q_pos0, int n_meta, int window, int Hq, int Hkv, int n_cu,
                                     int32_t* out, hipStream_t stream) {
  const int P = kAttnCols / (Hq / Hkv);
  const int64_t n_items = (int64_t)((Lq + P - 1) / P) * Hkv * batch;
  if (n_items <= 0) return hipSuccess;
  hipLaunchKernelGGL(prefill_visibility_kernel, dim3((unsigned)n_items), dim3(64 * kAttnWaves), 0, stream, out, Lq,
                     q_pos0, n_meta, window, Hq, Hkv, batch, n_cu);
  return hipGetLastError();
}

hipError_t launch_rope_prefill(const RopeArgs& a, hipStream_t stream, Timing tm) {
  if (a.act == HYMBA_BF16) return rope_t<bf16>(a, stream, tm);
  return rope_t<float>(a, stream, tm);
}

hipError_t launch_attn_prefill(const AttnPrefillArgs& a, hipStream_t stream, Timing tm) {
  if (a.act == HYMBA_BF16) { HYMBA_DISPATCH_DV(a.head_dim_v, attn_prefill_t, bf16, a, stream, tm) }
  HYMBA_DISPATCH_DV(a.head_dim_v, attn_prefill_t, float, a, stream, tm)
}

// most keys a decode row can see: meta + window (SWA), or the whole cache + itself
static int64_t decode_max_visible(int n_meta, int window, int cap) {
  int64_t max_vis = (int64_t)cap + 1;
  if (window > 0 && (int64_t)n_meta + window < max_vis) max_vis = (int64_t)n_meta + window;
  return max_vis;
}

// waves (one-wave workgroups) of the bf16 decode kernel that one CU holds,
// as the runtime's occupancy query gives them for its registers and LDS;
// asked once per value width (the same code object serves every device)
template <int DV>
int decode_wave_slots_t() {
  static std::atomic<int> cached{0};
  int n = cached.load(std::memory_order_relaxed);
  if (n > 0) return n;
  int per_cu_blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu_blocks, attn_decode_wave_kernel<DV, false>, 64, 0) !=
          hipSuccess ||
      per_cu_blocks < 1) {
    (void)hipGetLastError();   // fall back to the LDS bound
    const int stage = kWaveTile * DV * 2;
    per_cu_blocks = std::max(1, (160 * 1024) / (2 * stage + 1536));
  }
  cached.store(per_cu_blocks, std::memory_order_relaxed);
  return per_cu_blocks;
}

int decode_wave_slots_per_cu(int dv) {
  switch (dv) {
    case 32: return decode_wave_slots_t<32>();
    case 64: return decode_wave_slots_t<64>();
    default: return decode_wave_slots_t<128>();
  }
}

void decode_split_plan(int n_meta, int window, int cap, int* n_split, int* keys_per_split) {
  // room for one partial per 32-key tile: the most splits any launch uses
  const int64_t max_vis = decode_max_visible(n_meta, window, cap);
  *keys_per_split = kDecodeTile;
  *n_split = (int)((max_vis + kDecodeTile - 1) / kDecodeTile);
}

int decode_active_splits(const AttnDecodeArgs& a) {
  const int64_t max_vis = decode_max_visible(a.n_meta, a.window, a.cap);
  if (a.act != HYMBA_BF16)   // one split per kKeysPerSplit keys
    return (int)((max_vis + kKeysPerSplit - 1) / kKeysPerSplit);
  // one wave per split, all resident at once: eight waves per CU (more were
  // measured no faster: the step is bound by the memory system), fewer where
  // the two V stages of a wave run short of LDS
  // (less the slots left to the Mamba step's workgroups of the same launch)
  const int64_t per_cu =
      std::max<int64_t>(1, std::min<int64_t>(8, decode_wave_slots_per_cu(a.head_dim_v)) - kDecodeSsmReserve);
  const int64_t tiles = (max_vis + kWaveTile - 1) / kWaveTile;
  const int64_t rows = (int64_t)a.batch * a.n_kv_heads;
  const int64_t want = std::max<int64_t>(1, (per_cu * a.n_cu) / std::max<int64_t>(1, rows));
  return (int)std::min(tiles, want);
}

hipError_t launch_attn_decode(const AttnDecodeArgs& a, hipStream_t stream, Timing tm) {
  if (a.act == HYMBA_BF16) { HYMBA_DISPATCH_DV(a.head_dim_v, attn_decode_t, bf16, a, stream, tm) }
  HYMBA_DISPATCH_DV(a.head_dim_v, attn_decode_t, float, a, stream, tm)
}

hipError_t launch_decode_combine(const DecodeCombineArgs& a, hipStream_t stream, Timing tm) {
  if (a.act == HYMBA_BF16) { HYMBA_DISPATCH_DV(a.head_dim_v, combine_t, bf16, a, stream, tm) }
  HYMBA_DISPATCH_DV(a.head_dim_v, combine_t, float, a, stream, tm)
}

}  // namespace hymba
