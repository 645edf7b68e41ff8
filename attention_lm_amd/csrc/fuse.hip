// Fusion of the two branch outputs: per row, RMS-normalise each branch over its
// channels, scale by the per-channel betas and average. HBM-bound: each row's
// two inputs are read once from HBM (the second pass over the row hits cache)
// and the output written once. One wave per row, four rows per workgroup, or
// (many rows) a resident grid whose waves walk rows with the next row's loads
// in flight.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace hymba {

namespace {

constexpr int kRowsPerBlock = 4;

// The fused row is the step's last write and nothing in the step reads it
// again: stream it out (non-temporal) instead of keeping it in the caches
// (10.9 -> 9.6 us on the 2176-row layer).
__device__ __forceinline__ void store16_stream(bf16* p, const float* r) {
  const u32x4_t w = {pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3]), pack_bf16x2(r[4], r[5]),
                     pack_bf16x2(r[6], r[7])};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(p));
}
__device__ __forceinline__ void store16_stream(float* p, const float* r) {
  const f32x4_t w = {r[0], r[1], r[2], r[3]};
  __builtin_nontemporal_store(w, reinterpret_cast<f32x4_t*>(p));
}


// VEC: 16-byte vectors; MAXV > 0: the row fits in MAXV vectors per lane and is
// kept in registers (all loads issued up front); MAXV == 0: two passes over
// the row (the second one hits cache).
template <typename T, bool VEC, int MAXV>
__global__ __launch_bounds__(64 * kRowsPerBlock) void fuse_rows_kernel(
    const T* __restrict__ ya, const T* __restrict__ ys, const float* __restrict__ ba,
    const float* __restrict__ bs, int64_t n_rows, int width, float eps, T* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  const bool live = row < n_rows;
  if (!live) {
    if constexpr (MAXV == 0) return;
    row = n_rows - 1;   // a past-the-end wave only helps stage the betas; it stores nothing
  }
  const T* a = ya + row * (int64_t)width;
  const T* s = ys + row * (int64_t)width;
  T* o = out + row * (int64_t)width;
  constexpr int V = VEC ? Vec16<T>::n : 1;
  const float inv_w = 1.0f / (float)width;

  if constexpr (MAXV > 0) {
    // the workgroup's copy of the betas (dynamic LDS: 2 x width floats), read
    // from L2 once per workgroup while the rows are loading
    extern __shared__ float sbeta[];
    float va[MAXV][V], vs[MAXV][V];
    float sa = 0.f, ss = 0.f;
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
      const int c = (lane + 64 * i) * V;
      if (c < width) {
        load16(a + c, va[i]);
        load16(s + c, vs[i]);
      }
    }
    for (int c4 = threadIdx.x * 4; c4 < width; c4 += blockDim.x * 4) {
      *reinterpret_cast<float4*>(sbeta + c4) = *reinterpret_cast<const float4*>(ba + c4);
      *reinterpret_cast<float4*>(sbeta + width + c4) = *reinterpret_cast<const float4*>(bs + c4);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
      const int c = (lane + 64 * i) * V;
      if (c < width) {
#pragma unroll
        for (int e = 0; e < V; ++e) {
          sa = fmaf(va[i][e], va[i][e], sa);
          ss = fmaf(vs[i][e], vs[i][e], ss);
        }
      }
    }
    sa = wave_sum(sa);
    ss = wave_sum(ss);
    const float ra = 0.5f / sqrtf(sa * inv_w + eps);
    const float rs = 0.5f / sqrtf(ss * inv_w + eps);
    if (!live) return;
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
      const int c = (lane + 64 * i) * V;
      if (c < width) {
        float bav[V], bsv[V], r[V];
        load16(sbeta + c, bav);
        if constexpr (V == 8) load16(sbeta + c + 4, bav + 4);
        load16(sbeta + width + c, bsv);
        if constexpr (V == 8) load16(sbeta + width + c + 4, bsv + 4);
#pragma unroll
        for (int e = 0; e < V; ++e) r[e] = fmaf(bav[e] * ra, va[i][e], bsv[e] * rs * vs[i][e]);
        store16_stream(o + c, r);
      }
    }
  } else {
    float sa = 0.f, ss = 0.f;
    for (int c = lane * V; c < width; c += 64 * V) {
      float va[V], vs[V];
      if constexpr (VEC) {
        load16(a + c, va);
        load16(s + c, vs);
      } else {
        va[0] = to_f32(a[c]);
        vs[0] = to_f32(s[c]);
      }
#pragma unroll
      for (int e = 0; e < V; ++e) {
        sa = fmaf(va[e], va[e], sa);
        ss = fmaf(vs[e], vs[e], ss);
      }
    }
    sa = wave_sum(sa);
    ss = wave_sum(ss);
    const float ra = 0.5f / sqrtf(sa * inv_w + eps);
    const float rs = 0.5f / sqrtf(ss * inv_w + eps);
    for (int c = lane * V; c < width; c += 64 * V) {
      float va[V], vs[V], r[V];
      if constexpr (VEC) {
        load16(a + c, va);
        load16(s + c, vs);
      } else {
        va[0] = to_f32(a[c]);
        vs[0] = to_f32(s[c]);
      }
#pragma unroll
      for (int e = 0; e < V; ++e) r[e] = fmaf(ba[c + e] * ra, va[e], bs[c + e] * rs * vs[e]);
      if constexpr (VEC) {
        store16_stream(o + c, r);
      } else {
        o[c] = from_f32<T>(r[0]);
      }
    }
  }
}

// One 16-byte piece of a row as loaded, and as floats.
__device__ __forceinline__ void unpack16(u32x4_t w, const bf16*, float* o) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    o[2 * e] = bf16_lo(w[e]);
    o[2 * e + 1] = bf16_hi(w[e]);
  }
}
__device__ __forceinline__ void unpack16(u32x4_t w, const float*, float* o) {
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = __uint_as_float(w[e]);
}

// Rows that fit in NV 16-byte pieces per lane (width a multiple of 8 bf16 /
// 4 fp32): a fixed grid of workgroups (as many as are resident at once),
// each staging the betas in LDS once and its waves walking rows
// wave, wave + waves of the grid, ...; the next row's loads are issued before
// the current row is reduced and written, so every wave keeps two rows of
// loads in flight. The fused rows go out with plain stores: non-temporal ones
// measured slower in this form (251 against 241 us on 67,584 rows).
template <typename T, int NV>
__global__ __launch_bounds__(64 * kRowsPerBlock) void fuse_rows_stream_kernel(
    const T* __restrict__ ya, const T* __restrict__ ys, const float* __restrict__ ba,
    const float* __restrict__ bs, int64_t n_rows, int width, float eps, T* __restrict__ out) {
  constexpr int V = Vec16<T>::n;
  extern __shared__ float sbeta[];   // 2 x width floats
  const int lane = threadIdx.x & 63;
  const int64_t stride = (int64_t)gridDim.x * kRowsPerBlock;
  int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  const float inv_w = 1.0f / (float)width;
  const uint32_t row_b = (uint32_t)width * sizeof(T);
  // rows at or past n_rows read zeros (the descriptors end there)
  u32x4_t ca[NV], cs[NV];
  auto issue = [&](int64_t r, u32x4_t* da, u32x4_t* ds) {
    const bool ok = r < n_rows;
    const T* a = ya + (ok ? r : 0) * (int64_t)width;
    const T* s = ys + (ok ? r : 0) * (int64_t)width;
    const __amdgpu_buffer_rsrc_t rsa = make_rsrc(a, ok ? row_b : 0u);
    const __amdgpu_buffer_rsrc_t rss = make_rsrc(s, ok ? row_b : 0u);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const uint32_t off = (uint32_t)((lane + 64 * i) * 16);
      da[i] = buf_load16(rsa, off);
      ds[i] = buf_load16(rss, off);
    }
  };
  issue(row, ca, cs);
  for (int c4 = threadIdx.x * 4; c4 < width; c4 += blockDim.x * 4) {
    *reinterpret_cast<float4*>(sbeta + c4) = *reinterpret_cast<const float4*>(ba + c4);
    *reinterpret_cast<float4*>(sbeta + width + c4) = *reinterpret_cast<const float4*>(bs + c4);
  }
  __syncthreads();
  while (row < n_rows) {   // wave-uniform
    u32x4_t na[NV], ns[NV];
    issue(row + stride, na, ns);
    float sa = 0.f, ss = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      float fa[V], fs[V];
      unpack16(ca[i], (const T*)nullptr, fa);
      unpack16(cs[i], (const T*)nullptr, fs);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        sa = fmaf(fa[e], fa[e], sa);
        ss = fmaf(fs[e], fs[e], ss);
      }
    }
    sa = wave_sum(sa);
    ss = wave_sum(ss);
    const float ra = 0.5f / sqrtf(sa * inv_w + eps);
    const float rs = 0.5f / sqrtf(ss * inv_w + eps);
    T* o = out + row * (int64_t)width;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c = (lane + 64 * i) * V;
      if (c < width) {
        float fa[V], fs[V], bav[V], bsv[V], r[V];
        unpack16(ca[i], (const T*)nullptr, fa);
        unpack16(cs[i], (const T*)nullptr, fs);
        load16(sbeta + c, bav);
        if constexpr (V == 8) load16(sbeta + c + 4, bav + 4);
        load16(sbeta + width + c, bsv);
        if constexpr (V == 8) load16(sbeta + width + c + 4, bsv + 4);
#pragma unroll
        for (int e = 0; e < V; ++e) r[e] = fmaf(bav[e] * ra, fa[e], bsv[e] * rs * fs[e]);
        store16(o + c, r);
      }
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      ca[i] = na[i];
      cs[i] = ns[i];
    }
    row += stride;
  }
}

__global__ void mask_ranges_kernel(int n_rows, int n_meta, int window, int32_t* __restrict__ ranges) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_rows) return;
  MaskRange r = mask_range(i, n_meta, window);
  int4 v = make_int4(r.meta_end, r.win_begin, r.win_end, r.meta_end + (r.win_end - r.win_begin));
  *reinterpret_cast<int4*>(ranges + 4 * (int64_t)i) = v;
}

constexpr int kStreamPieces = 7;        // 16-byte pieces per lane: rows up to 3584 bf16 / 1792 fp32
// resident workgroups per CU (registers: two rows of 16-byte pieces per lane)
template <typename T> constexpr int kStreamBlocksPerCu = sizeof(T) == 2 ? 2 : 3;

template <typename T>
hipError_t fuse_t(const void* ya, const void* ys, const float* ba, const float* bs, int64_t n_rows,
                  int width, float eps, void* out, hipStream_t stream, Timing tm, int n_cu) {
  if (n_rows == 0) return no_kernel(stream, tm);
  const int64_t blocks = (n_rows + kRowsPerBlock - 1) / kRowsPerBlock;
  constexpr int V = Vec16<T>::n;
  const bool vec = (width % V) == 0;
  dim3 grid((unsigned)blocks), block(64 * kRowsPerBlock);
  // streaming form where every wave of a resident grid walks at least four
  // rows (on the 2176-row layer, about one row per wave, the one-row-per-wave
  // form is 0.9 us faster; on 67,584 rows the streaming form 270 -> 241 us)
  const int64_t resident = (int64_t)kStreamBlocksPerCu<T> * n_cu;
  if (vec && width <= 64 * V * kStreamPieces && n_cu > 0 && n_rows >= 4 * kRowsPerBlock * resident) {
    const int64_t g = std::min<int64_t>(blocks, resident);
    HYMBA_LAUNCH((fuse_rows_stream_kernel<T, kStreamPieces>), dim3((unsigned)g), block, 2 * width * sizeof(float),
                 stream, tm, (const T*)ya, (const T*)ys, ba, bs, n_rows, width, eps, (T*)out);
  } else if (vec && width <= 64 * V * 8)
    HYMBA_LAUNCH((fuse_rows_kernel<T, true, 8>), grid, block, 2 * width * sizeof(float), stream, tm, (const T*)ya, (const T*)ys, ba,
                       bs, n_rows, width, eps, (T*)out);
  else if (vec)
    HYMBA_LAUNCH((fuse_rows_kernel<T, true, 0>), grid, block, 0, stream, tm, (const T*)ya, (const T*)ys, ba,
                       bs, n_rows, width, eps, (T*)out);
  else
    HYMBA_LAUNCH((fuse_rows_kernel<T, false, 0>), grid, block, 0, stream, tm, (const T*)ya, (const T*)ys, ba,
                       bs, n_rows, width, eps, (T*)out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fuse(const void* y_attn, const void* y_ssm, const float* beta_attn, const float* beta_ssm,
                       int64_t n_rows, int width, float eps, hymba_dtype act, void* out, hipStream_t stream,
                       Timing tm, int n_cu) {
  if (act == HYMBA_BF16)
    return fuse_t<bf16>(y_attn, y_ssm, beta_attn, beta_ssm, n_rows, width, eps, out, stream, tm, n_cu);
  return fuse_t<float>(y_attn, y_ssm, beta_attn, beta_ssm, n_rows, width, eps, out, stream, tm, n_cu);
}

hipError_t launch_mask_ranges(int n_rows, int n_meta, int window, int32_t* ranges, hipStream_t stream) {
  if (n_rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(mask_ranges_kernel, dim3((n_rows + 255) / 256), dim3(256), 0, stream, n_rows, n_meta,
                     window, ranges);
  return hipGetLastError();
}

}  // namespace hymba
