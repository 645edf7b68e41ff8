// One decode step of the Mamba branch for one (sequence, channel), split over
// a quad of lanes (4 states each): conv over the 3-row history and x, the
// state update h = exp(dt A) h + dt B u, y = (C . h + D u) silu(z), and the
// shifted conv history ("Jamba: Hybrid SSM-Transformer", "1. Layer
// Interleaving Ratio"; "Lecture 04 - Beyond the Dense Transformer", section 2).
// Used by the fp32 decode kernel of the Mamba branch (ssm_decode_kernel) and,
// in bf16, by the Mamba-step workgroups inside the decode attention launch.
#pragma once

#include "common.hpp"

namespace hymba {
namespace ssm_step {

constexpr int kStates = 16;
constexpr int kConv = 4;

template <typename T>
struct Ptrs {
  const T *x, *z, *dt, *B, *C;   // [batch, d_inner] (dt: [batch, heads] with heads) / [batch, 16]
  const float *A, *D, *conv_w;   // [d_inner, 16] (or [heads]), [d_inner], [d_inner, 4]
  float* state;                  // in/out [batch, d_inner, 16]
  T* conv_state;                 // in/out [batch, d_inner, 3]
  T* y;                          // out [batch, d_inner]
  int d_inner;
  int head_width;                // > 0: Mamba-2 heads of this many channels, one A and dt per head
};

// Everything a lane needs for its item, loaded by load() and used by finish(),
// so that all of a lane's loads can be in flight together.
template <typename T>
struct Item {
  float cs[kConv - 1], w[kConv], B[4], C[4], d, z, Dc;
  float4 h4, a4;
  T x;
  int64_t bc;
  bool ok;
};

__device__ __forceinline__ void load4(const float* p, float* o) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
}
__device__ __forceinline__ void load4(const bf16* p, float* o) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  o[0] = bf16_lo(v.x); o[1] = bf16_hi(v.x); o[2] = bf16_lo(v.y); o[3] = bf16_hi(v.y);
}

// lane q (0..3) of the quad of channel c of sequence b; ok must be the same
// for the whole quad (finish() reduces over it); a quad that is not ok loads
// channel 0 of sequence 0 and stores nothing
template <typename T>
__device__ __forceinline__ void load(const Ptrs<T>& p, Item<T>& it, int64_t b, int c, int q, bool ok) {
  it.ok = ok;
  if (!ok) { b = 0; c = 0; }
  it.bc = b * p.d_inner + c;
#pragma unroll
  for (int j = 0; j < kConv - 1; ++j) it.cs[j] = to_f32(p.conv_state[it.bc * (kConv - 1) + j]);
  it.x = p.x[it.bc];
  const int hw = p.head_width;
  it.d = to_f32(hw > 0 ? p.dt[b * (p.d_inner / hw) + c / hw] : p.dt[it.bc]);
  it.z = to_f32(p.z[it.bc]);
  it.Dc = p.D[c];
  load4(p.conv_w + (int64_t)c * kConv, it.w);
  it.h4 = *reinterpret_cast<const float4*>(p.state + it.bc * kStates + 4 * q);
  if (hw > 0) {
    const float a = p.A[c / hw];
    it.a4 = make_float4(a, a, a, a);
  } else {
    it.a4 = *reinterpret_cast<const float4*>(p.A + (int64_t)c * kStates + 4 * q);
  }
  load4(p.B + b * kStates + 4 * q, it.B);
  load4(p.C + b * kStates + 4 * q, it.C);
}

template <typename T>
__device__ __forceinline__ void finish(const Ptrs<T>& p, const Item<T>& it, int q) {
  const float xn = to_f32(it.x);
  float u = it.w[kConv - 1] * xn;
#pragma unroll
  for (int j = 0; j < kConv - 1; ++j) u = fmaf(it.w[j], it.cs[j], u);
  const float du = it.d * u;
  float h[4] = {it.h4.x, it.h4.y, it.h4.z, it.h4.w};
  const float a[4] = {it.a4.x, it.a4.y, it.a4.z, it.a4.w};
  float part = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    h[j] = fmaf(__builtin_amdgcn_exp2f(it.d * a[j] * kLog2e), h[j], du * it.B[j]);
    part = fmaf(it.C[j], h[j], part);
  }
  part += __shfl_xor(part, 1, 64);
  part += __shfl_xor(part, 2, 64);
  if (!it.ok) return;
  *reinterpret_cast<float4*>(p.state + it.bc * kStates + 4 * q) = make_float4(h[0], h[1], h[2], h[3]);
  if (q == 0) {
    // silu(z) = z / (1 + e^-z)
    const float g = it.z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-it.z * kLog2e));
    p.y[it.bc] = from_f32<T>(fmaf(it.Dc, u, part) * g);
    T* cp = p.conv_state + it.bc * (kConv - 1);
#pragma unroll
    for (int j = 0; j < kConv - 2; ++j) cp[j] = from_f32<T>(it.cs[j + 1]);
    cp[kConv - 2] = it.x;
  }
}

}  // namespace ssm_step
}  // namespace hymba
