// Token embed (latent channels -> model width) and head (model width ->
// latent channels) of the synthetic velocity stand-in.  The pages give no
// widths for the transformer, so these projections belong to the stand-in;
// the 24-channel channel-last latent follows "Open-H3-Regenerate-2K:
// High-Resolution Video Refinement with Few-Step Diffusion" (agientry.com),
// section "Why upscaling happens in latent space", shape equation.
//
// embed: X[m, n] = bf16(sum_c z[m, c]·E[n, c]).  K = C is tiny (24), so this
//   is a write-bound outer product: each lane keeps two columns of E in
//   registers, a block stages 64 latent rows in LDS and streams out 64 rows of
//   X (1 KiB contiguous per row per block).  fp32 FMAs, no MFMA: z stays fp32.
// head:  v[m, c] = sum_n H[m, n]·P[c, n].  A read-bound GEMM with N = C <= 32:
//   each wave owns 128 rows and the 32 (zero-padded) columns, one
//   32x32x16 bf16 MFMA per (32-row block, 16 k).  Within every 64-wide slice of
//   k a lane walks 32 contiguous k (64 bytes) of its row; the MFMA's sum over k
//   does not depend on which k a lane supplies as long as H and P agree, so
//   both operands use the same assignment.
#include "fsd_internal.h"

namespace fsd {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kMaxC = 32;
constexpr int kEmbedRows = 64;
constexpr int kEmbedCols = 2 * kThreads;   // two output columns per lane
constexpr int kHeadRowsPerWave = 128;

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float((uint32_t)h << 16);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__global__ __launch_bounds__(kThreads) void embed_kernel(const float* z, const bf16_t* E,
                                                         bf16_t* X, int64_t ldx, int64_t M,
                                                         int C, int64_t D) {
  __shared__ float zs[kEmbedRows * kMaxC];
  const int64_t m0 = (int64_t)blockIdx.y * kEmbedRows;
  const int rows = (int)((M - m0) < kEmbedRows ? (M - m0) : kEmbedRows);
  for (int i = threadIdx.x; i < rows * C; i += kThreads) zs[i] = z[m0 * C + i];
  const int64_t n = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 2;
  float e0[kMaxC], e1[kMaxC];
#pragma unroll
  for (int c = 0; c < kMaxC; ++c) {
    e0[c] = (n < D && c < C) ? bf16_to_f32(E[n * C + c]) : 0.0f;
    e1[c] = (n < D && c < C) ? bf16_to_f32(E[(n + 1) * C + c]) : 0.0f;
  }
  __syncthreads();
  if (n >= D) return;
  for (int r = 0; r < rows; ++r) {
    const float* zr = zs + r * C;
    float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
    for (int c = 0; c < kMaxC; ++c) {
      if (c < C) {
        s0 = fmaf(zr[c], e0[c], s0);
        s1 = fmaf(zr[c], e1[c], s1);
      }
    }
    const uint32_t packed = (uint32_t)__builtin_bit_cast(bf16_t, (__bf16)s0) |
                            ((uint32_t)__builtin_bit_cast(bf16_t, (__bf16)s1) << 16);
    *(uint32_t*)(X + (m0 + r) * ldx + n) = packed;
  }
}

__global__ __launch_bounds__(kThreads) void head_kernel(const bf16_t* H, int64_t ldh,
                                                        const bf16_t* P, float* v, int64_t M,
                                                        int64_t D, int C) {
  const int lane = threadIdx.x & 63;
  const int64_t wave_id = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int64_t m0 = wave_id * kHeadRowsPerWave;
  if (m0 >= M) return;
  const int64_t rows_valid = (M - m0) < kHeadRowsPerWave ? (M - m0) : kHeadRowsPerWave;
  const __amdgpu_buffer_rsrc_t rH = make_rsrc(H + m0 * ldh, rows_valid * ldh * 2);
  const __amdgpu_buffer_rsrc_t rP = make_rsrc(P, (int64_t)C * D * 2);   // rows >= C read 0
  const int j = lane & 31;
  const int h = lane >> 5;
  f32x16 acc[4];
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[bi][e] = 0.0f;
  const uint32_t p_row = (uint32_t)(j * D * 2);
  uint32_t h_row[4];
#pragma unroll
  for (int bi = 0; bi < 4; ++bi) h_row[bi] = (uint32_t)((bi * 32 + j) * ldh * 2);
  for (int64_t k0 = 0; k0 < D; k0 += 64) {
    u32x4 pf[4], hf[4][4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint32_t koff = (uint32_t)((k0 + 32 * h + 8 * s) * 2);
      pf[s] = __builtin_amdgcn_raw_buffer_load_b128(rP, p_row + koff, 0, 0);
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
        hf[bi][s] = __builtin_amdgcn_raw_buffer_load_b128(rH, h_row[bi] + koff, 0, 0);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
        acc[bi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, hf[bi][s]),
                                                          __builtin_bit_cast(bf16x8, pf[s]),
                                                          acc[bi], 0, 0, 0);
  }
  if (j >= C) return;
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int i = bi * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
      if (i < rows_valid) v[(m0 + i) * C + j] = acc[bi][e];
    }
}

}  // namespace

hipError_t launch_embed(const float* z, const bf16_t* E, bf16_t* X, int64_t ldx, int64_t M,
                        int C, int64_t D, hipStream_t s) {
  if (M == 0) return hipSuccess;
  const dim3 grid((unsigned)((D + kEmbedCols - 1) / kEmbedCols),
                  (unsigned)((M + kEmbedRows - 1) / kEmbedRows));
  hipLaunchKernelGGL(embed_kernel, grid, dim3(kThreads), 0, s, z, E, X, ldx, M, C, D);
  return hipGetLastError();
}

hipError_t launch_head(const bf16_t* H, int64_t ldh, const bf16_t* P, float* v, int64_t M,
                       int64_t D, int C, hipStream_t s) {
  if (M == 0) return hipSuccess;
  const int64_t waves = (M + kHeadRowsPerWave - 1) / kHeadRowsPerWave;
  const int64_t blocks = (waves + 3) / 4;
  hipLaunchKernelGGL(head_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, H, ldh, P, v, M,
                     D, C);
  return hipGetLastError();
}

}  // namespace fsd
