// Shared device helpers for the Hymba mixer kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hymba {

constexpr float kLog2e = 1.4426950408889634f;

// bf16 storage type (bit pattern). Arithmetic always happens in fp32.
struct bf16 {
  uint16_t u;
};

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));   // register-friendly 16 bytes
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return __uint_as_float((uint32_t)v.u << 16); }
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}
// two floats -> two bf16 in one word (lo in the low half); one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

template <typename T> __device__ __forceinline__ T from_f32(float f);
template <> __device__ __forceinline__ float from_f32<float>(float f) { return f; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float f) { return bf16{f32_to_bf16_bits(f)}; }

// Elements of T per 16-byte vector.
template <typename T> struct Vec16 { static constexpr int n = 16 / sizeof(T); };

// Load 16 bytes (Vec16<T>::n elements) as fp32.
__device__ __forceinline__ void load16(const float* p, float* o) {
  float4 v = *reinterpret_cast<const float4*>(p);
  o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
}
__device__ __forceinline__ void load16(const bf16* p, float* o) {
  uint4 v = *reinterpret_cast<const uint4*>(p);
  o[0] = bf16_lo(v.x); o[1] = bf16_hi(v.x); o[2] = bf16_lo(v.y); o[3] = bf16_hi(v.y);
  o[4] = bf16_lo(v.z); o[5] = bf16_hi(v.z); o[6] = bf16_lo(v.w); o[7] = bf16_hi(v.w);
}
__device__ __forceinline__ void store16(float* p, const float* o) {
  *reinterpret_cast<float4*>(p) = make_float4(o[0], o[1], o[2], o[3]);
}
__device__ __forceinline__ void store16(bf16* p, const float* o) {
  uint4 v;
  v.x = pack_bf16x2(o[0], o[1]); v.y = pack_bf16x2(o[2], o[3]);
  v.z = pack_bf16x2(o[4], o[5]); v.w = pack_bf16x2(o[6], o[7]);
  *reinterpret_cast<uint4*>(p) = v;
}

// Raw buffer access (gfx9 descriptor word 3: 32-bit data format; no stride,
// swizzle or index). A load whose byte offset is at or past the descriptor's
// size reads zeros and a store there is dropped; neither touches memory.
constexpr int kBufferWord3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferWord3);
}
__device__ __forceinline__ u32x4_t buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ void buf_store(__amdgpu_buffer_rsrc_t r, uint32_t off, bf16 v) {
  __builtin_amdgcn_raw_buffer_store_b16(v.u, r, off, 0, 0);
}
__device__ __forceinline__ void buf_store(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);
}
// 16 bytes per lane straight into LDS: lane i of the wave writes bytes
// [16 i, 16 i + 16) from lds_base (which must be the same for the whole wave);
// an out-of-range lane writes zeros.
__device__ __forceinline__ void buf_load16_lds(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                               __attribute__((address_space(3))) void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_base, 16, off, 0, 0, 0);
}
__device__ __forceinline__ void buf_load16_lds(__amdgpu_buffer_rsrc_t r, uint32_t off, void* lds_base) {
  buf_load16_lds(r, off, (__attribute__((address_space(3))) void*)lds_base);
}
// an offset that every descriptor above treats as out of range
constexpr uint32_t kBufferNowhere = 0x80000000u;

// Waits and barriers for kernels that keep global loads in flight across a
// barrier (a __syncthreads() waits for every outstanding load, loads into LDS
// included). gfx9 s_waitcnt fields: vmcnt bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8. The empty asm statements keep the compiler from moving memory
// accesses across the barrier.
//
// wait for all of this wave's outstanding global loads, including those that
// write LDS (vmcnt 0; expcnt and lgkmcnt at their maximum)
__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// workgroup barrier after LDS writes: lgkmcnt 0, vmcnt and expcnt untouched
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wave64 butterfly sum / max (deterministic order).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ---------------------------------------------------------------------------
// Visibility of key row j to query row i: the ranges a decode row sees.
//
// Causal: j <= i. The meta-token rows j < n_meta are visible to every later
// row under any window (Hymba guide, "2. Learnable Meta-Tokens"; the
// Hymba-1.5B article, section 2). Other rows need i - j < window in a
// sliding-window layer (window > 0); window <= 0 is a global causal layer.
struct MaskRange {
  int meta_end;   // visible meta keys: [0, meta_end)
  int win_begin;  // visible non-meta keys: [win_begin, win_end); both n_meta if none
  int win_end;
};

__host__ __device__ __forceinline__ MaskRange mask_range(int i, int n_meta, int window) {
  MaskRange r;
  r.meta_end = i + 1 < n_meta ? i + 1 : n_meta;
  int wb = n_meta;
  if (window > 0) {
    int lo = i - window + 1;
    wb = lo > n_meta ? lo : n_meta;
  }
  int we = i + 1;
  if (we <= wb) { wb = n_meta; we = n_meta; }
  r.win_begin = wb;
  r.win_end = we;
  return r;
}

}  // namespace hymba
