// Matrix-core operands shared by the attention and the Mamba-2 scan kernels:
// one 32 x 32 output tile accumulated over K = 16 per call. The A operand of
// lane l is row l % 32 of A at k = 8 (l / 32) .. + 7, the B operand column
// l % 32 of B at the same k; output register r of lane l is row
// 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32.
// bf16: one v_mfma_f32_32x32x16_bf16. fp32: eight v_mfma_f32_32x32x2f32, slot
// t of lane half h being k = 8 h + t.
#pragma once

#include "common.hpp"

namespace hymba {
namespace {

template <typename T>
struct Mma;
template <>
struct Mma<bf16> {
  typedef bf16x8_t Frag;   // 8 bf16 per lane
  static __device__ __forceinline__ Frag frag_at(const bf16* p) {
    return __builtin_bit_cast(Frag, *reinterpret_cast<const u32x4_t*>(p));
  }
  static __device__ __forceinline__ Frag zero() { return __builtin_bit_cast(Frag, u32x4_t{0u, 0u, 0u, 0u}); }
  static __device__ __forceinline__ Frag from_f32(const float* v) {
    u32x4_t u;
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
  static __device__ __forceinline__ Frag frag_at(const float* p) {
    Frag f;
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = *reinterpret_cast<const float4*>(p + 4);
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
    return f;
  }
  static __device__ __forceinline__ Frag zero() {
    Frag f;
#pragma unroll
    for (int t = 0; t < 8; ++t) f.v[t] = 0.f;
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

}  // namespace
}  // namespace hymba
