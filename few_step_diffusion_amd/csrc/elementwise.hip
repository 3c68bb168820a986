// Streaming kernels of the sampler (renoise, Euler) and the adapter merge.
//
// Source: "Open-H3-Regenerate-2K: High-Resolution Video Refinement with
// Few-Step Diffusion" (agientry.com), section "Three steps instead of dozens":
// renoise equation and the schedule / Euler update equation.  Merge:
// "Open-H3-Regenerate-2K：MiniMax H3 的开源 4K 精修方案" (comfyui-wiki.com),
// section "三个步如何完成工作".
//
// Renoise and Euler read two fp32 streams and write one (12 bytes per
// element): they are HBM-bound.  Each lane moves 16-byte vectors with
// non-temporal loads and stores (the streams are touched once; plain accesses
// measured at half the bandwidth), one vector per lane, over a grid that covers
// the array, in one-wave workgroups: cache-cold batches of launches measured
// 64 > 128 > 256 > 1024 threads per workgroup (at 2K 78% / 77% / 76% / 75.5% of
// 8 TB/s; at 4K 81.6% / 81.3% / 79.5% / 80.3%), the finer granularity keeping
// the CUs' wave slots full to the end of the grid.
#include "fsd_internal.h"

namespace fsd {

namespace {

constexpr int kThreads = 256;          // merge kernels
constexpr int kStreamThreads = 64;     // renoise / Euler: one wave per workgroup
constexpr int kUnroll = 1;

typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f4 ld_stream(const f4* p) {
  return __builtin_nontemporal_load(p);
}
__device__ __forceinline__ void st_stream(f4* p, f4 v) {
  __builtin_nontemporal_store(v, p);
}

// z = a·u + b·e with a = 1 - sigma, b = sigma; z may be u or e (same index).
__global__ __launch_bounds__(kStreamThreads) void renoise_kernel(const f4* u, const f4* e,
                                                           float a, float b, f4* z,
                                                           int64_t n4, const float* us,
                                                           const float* es, float* zs,
                                                           int64_t n) {
  const int64_t step = (int64_t)gridDim.x * kStreamThreads * kUnroll;
  for (int64_t base = (int64_t)blockIdx.x * kStreamThreads * kUnroll + threadIdx.x; base < n4;
       base += step) {
    f4 uu[kUnroll], ee[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
      const int64_t i = base + (int64_t)k * kStreamThreads;
      if (i < n4) {
        uu[k] = ld_stream(u + i);
        ee[k] = ld_stream(e + i);
      }
    }
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
      const int64_t i = base + (int64_t)k * kStreamThreads;
      if (i < n4) {
        f4 r;
        r.x = fmaf(b, ee[k].x, a * uu[k].x);
        r.y = fmaf(b, ee[k].y, a * uu[k].y);
        r.z = fmaf(b, ee[k].z, a * uu[k].z);
        r.w = fmaf(b, ee[k].w, a * uu[k].w);
        st_stream(z + i, r);
      }
    }
  }
  // the n % 4 trailing elements
  if (blockIdx.x == 0) {
    const int64_t i = 4 * n4 + threadIdx.x;
    if (i < n) zs[i] = fmaf(b, es[i], a * us[i]);
  }
}

// z = z + d·v (in place).
__global__ __launch_bounds__(kStreamThreads) void euler_kernel(f4* z, const f4* v, float d,
                                                         int64_t n4, float* zs, const float* vs,
                                                         int64_t n) {
  const int64_t step = (int64_t)gridDim.x * kStreamThreads * kUnroll;
  for (int64_t base = (int64_t)blockIdx.x * kStreamThreads * kUnroll + threadIdx.x; base < n4;
       base += step) {
    f4 zz[kUnroll], vv[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
      const int64_t i = base + (int64_t)k * kStreamThreads;
      if (i < n4) {
        zz[k] = ld_stream(z + i);
        vv[k] = ld_stream(v + i);
      }
    }
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
      const int64_t i = base + (int64_t)k * kStreamThreads;
      if (i < n4) {
        f4 r;
        r.x = fmaf(d, vv[k].x, zz[k].x);
        r.y = fmaf(d, vv[k].y, zz[k].y);
        r.z = fmaf(d, vv[k].z, zz[k].z);
        r.w = fmaf(d, vv[k].w, zz[k].w);
        st_stream(z + i, r);
      }
    }
  }
  if (blockIdx.x == 0) {
    const int64_t i = 4 * n4 + threadIdx.x;
    if (i < n) zs[i] = fmaf(d, vs[i], zs[i]);
  }
}

int stream_grid(int64_t n4) {
  // One 16-byte vector per lane per trip and a grid that covers the whole
  // array (no grid-stride trips unless the grid limit is reached): measured
  // faster than fewer blocks with several vectors per lane, because the
  // dispatcher keeps every CU's wave slots full up to the last block.
  const int64_t per_block = (int64_t)kStreamThreads * kUnroll;
  int64_t g = (n4 + per_block - 1) / per_block;
  const int64_t cap = 0x7fffffff;
  if (g > cap) g = cap;
  return (int)(g < 1 ? 1 : g);
}

__global__ __launch_bounds__(kThreads) void merge_rows_kernel(const float* src, int64_t rows,
                                                              int64_t cols, bf16_t* dst,
                                                              int64_t ld_dst) {
  const int64_t total = rows * cols;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * kThreads) {
    const int64_t r = i / cols, c = i - r * cols;
    const __bf16 h = (__bf16)src[i];
    dst[r * ld_dst + c] = __builtin_bit_cast(bf16_t, h);
  }
}

// B_i columns: dst[r, c] = bf16(fp32(scale · src[r, c])).
__global__ __launch_bounds__(kThreads) void merge_cols_kernel(const float* src, int64_t rows,
                                                              int64_t cols, float scale,
                                                              bf16_t* dst, int64_t ld_dst) {
  const int64_t total = rows * cols;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * kThreads) {
    const int64_t r = i / cols, c = i - r * cols;
    const float p = scale * src[i];
    const __bf16 h = (__bf16)p;
    dst[r * ld_dst + c] = __builtin_bit_cast(bf16_t, h);
  }
}

int flat_grid(int64_t total) {
  int64_t g = (total + kThreads - 1) / kThreads;
  if (g > 256 * 16) g = 256 * 16;
  return (int)(g < 1 ? 1 : g);
}

}  // namespace

hipError_t launch_renoise(const float* u, const float* eps, float sigma, float* z, int64_t n,
                          hipStream_t s) {
  const float a = 1.0f - sigma;
  const int64_t n4 = n / 4;
  hipLaunchKernelGGL(renoise_kernel, dim3(stream_grid(n4)), dim3(kStreamThreads), 0, s,
                     (const f4*)u, (const f4*)eps, a, sigma, (f4*)z, n4, u, eps, z, n);
  return hipGetLastError();
}

hipError_t launch_euler(float* z, const float* v, float dsigma, int64_t n, hipStream_t s) {
  const int64_t n4 = n / 4;
  hipLaunchKernelGGL(euler_kernel, dim3(stream_grid(n4)), dim3(kStreamThreads), 0, s, (f4*)z,
                     (const f4*)v, dsigma, n4, z, v, n);
  return hipGetLastError();
}

hipError_t launch_merge_rows(const float* src, int64_t rows, int64_t cols, bf16_t* dst,
                             int64_t ld_dst, hipStream_t s) {
  hipLaunchKernelGGL(merge_rows_kernel, dim3(flat_grid(rows * cols)), dim3(kThreads), 0, s, src,
                     rows, cols, dst, ld_dst);
  return hipGetLastError();
}

hipError_t launch_merge_cols(const float* src, int64_t rows, int64_t cols, float scale,
                             bf16_t* dst, int64_t ld_dst, hipStream_t s) {
  hipLaunchKernelGGL(merge_cols_kernel, dim3(flat_grid(rows * cols)), dim3(kThreads), 0, s, src,
                     rows, cols, scale, dst, ld_dst);
  return hipGetLastError();
}

}  // namespace fsd
