// Token embed (latent channels -> model width) and head (model width ->
// latent channels) of the synthetic velocity stand-in.  The pages give no
// widths for the transformer, so these projections belong to the stand-in;
// the 24-channel channel-last latent follows "Open-H3-Regenerate-2K:
// High-Resolution Video Refinement with Few-Step Diffusion" (agientry.com),
// section "Why upscaling happens in latent space", shape equation.
//
// embed: X[m, n] = bf16(sum_c z[m, c]·E[n, c]).  K = C is tiny (<= 32), so
//   the kernel is bound by writing X.  The sums run on MFMA with fp32
//   accumulation: z (fp32) is split as z = zh + zl with zh = bf16(z) and
//   zl = bf16(z - zh), which leaves a relative error below 2^-16 in z, far
//   under the bf16 rounding of X itself, and X = zh·Eᵀ + zl·Eᵀ takes two
//   32x32x16 bf16 MFMAs per 16 channels.  E is the MFMA's first operand, so a
//   lane holds 4 consecutive columns of one token and writes them as one
//   8-byte store.  One wave owns 128 tokens x 512 columns: its z fragments
//   are loaded once, and each E fragment serves 4 blocks of 32 tokens.
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
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kMaxC = 32;
constexpr int kEmbedTokens = 128;          // tokens per wave (4 MFMA blocks)
constexpr int kEmbedCols = 512;            // output columns per wave
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kHeadRowsPerWave = 128;

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float((uint32_t)h << 16);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Physical 16-byte chunk of logical chunk c in staged row r: XOR with bits
// 1..3 of the row spreads 16 consecutive rows over the 16 chunk slots of a
// 256-byte bank line.
__device__ __forceinline__ int embed_swz(int r, int c) { return c ^ ((r >> 1) & 7); }

__global__ __launch_bounds__(kThreads) void embed_kernel(const float* z, const bf16_t* E,
                                                         bf16_t* X, int64_t ldx, int64_t M,
                                                         int C, int64_t D, int vec_e) {
  const int lane = threadIdx.x & 63;
  const int64_t wave_id = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int64_t nchunk = (D + kEmbedCols - 1) / kEmbedCols;
  const int64_t m0 = (wave_id / nchunk) * kEmbedTokens;
  const int64_t c0 = (wave_id % nchunk) * kEmbedCols;
  if (m0 >= M) return;
  const int j = lane & 31;
  const int h = lane >> 5;
  // z fragments (operand B): token m0 + 32·bi + j, channels 16·kb + 8·h + e
  bf16x8 zh[4][2], zl[4][2];
#pragma unroll
  for (int bi = 0; bi < 4; ++bi) {
    const int64_t t = m0 + 32 * bi + j;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = 16 * kb + 8 * h + e;
        const float v = (t < M && c < C) ? z[t * C + c] : 0.0f;
        const __bf16 hi = (__bf16)v;
        zh[bi][kb][e] = hi;
        zl[bi][kb][e] = (__bf16)(v - (float)hi);
      }
  }
  // E fragments (operand A): column n0 + j, channels 16·kb + 8·h + e.  Rows
  // past D fall outside the buffer and read as zeros; channels past C are
  // masked (they would read the next row).
  const __amdgpu_buffer_rsrc_t rE = make_rsrc(E, D * C * 2);
  // per-wave staging: 128 tokens x 64 columns (128 B per token row)
  __shared__ __attribute__((aligned(16))) char stage_all[(kThreads / 64) * kEmbedTokens * 128];
  char* stage = stage_all + (threadIdx.x >> 6) * kEmbedTokens * 128;
  const int64_t c_end = (c0 + kEmbedCols) < D ? (c0 + kEmbedCols) : D;
  for (int64_t n0 = c0; n0 < c_end; n0 += 32) {
    const int64_t n = n0 + j;
    bf16x8 ef[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int k0 = 16 * kb + 8 * h;
      if (vec_e) {
        const uint32_t off = k0 < C ? (uint32_t)((n * C + k0) * 2) : kOutOfRange;
        ef[kb] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rE, off, 0, 0));
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t off = (k0 + e) < C ? (uint32_t)((n * C + k0 + e) * 2) : kOutOfRange;
          const uint16_t bits = __builtin_amdgcn_raw_buffer_load_b16(rE, off, 0, 0);
          ef[kb][e] = __builtin_bit_cast(__bf16, bits);
        }
      }
    }
    f32x16 acc[4];
#pragma unroll
    for (int bi = 0; bi < 4; ++bi) {
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[bi][e] = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        acc[bi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ef[kb], zh[bi][kb], acc[bi], 0, 0, 0);
        acc[bi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ef[kb], zl[bi][kb], acc[bi], 0, 0, 0);
      }
    }
    // Stage: lane holds token 32·bi + j, columns n0 + 8·g + 4·h + 0..3, i.e.
    // 8 bytes of logical chunk (n0 % 64)/8 + g of its staged row.
    const int half = (int)((n0 - c0) >> 5) & 1;
#pragma unroll
    for (int bi = 0; bi < 4; ++bi) {
      const int r = 32 * bi + j;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 pk;
        pk.x = (uint32_t)__builtin_bit_cast(bf16_t, (__bf16)acc[bi][4 * g]) |
               ((uint32_t)__builtin_bit_cast(bf16_t, (__bf16)acc[bi][4 * g + 1]) << 16);
        pk.y = (uint32_t)__builtin_bit_cast(bf16_t, (__bf16)acc[bi][4 * g + 2]) |
               ((uint32_t)__builtin_bit_cast(bf16_t, (__bf16)acc[bi][4 * g + 3]) << 16);
        *(u32x2*)(stage + r * 128 + (embed_swz(r, 4 * half + g) << 4) + 8 * h) = pk;
      }
    }
    // every 64 columns (or at the end of the wave's range) write whole rows
    if (half == 1 || n0 + 32 >= c_end) {
      const int64_t col = n0 - 32 * half;            // first column of the staged slab
      __builtin_amdgcn_s_waitcnt(0xc07f);            // lgkmcnt(0): the wave's staging is done
#pragma unroll 4
      for (int it = 0; it < kEmbedTokens / 8; ++it) {
        const int r = 8 * it + (lane >> 3);
        const int pc = lane & 7;
        const int lc = embed_swz(r, pc);             // the swizzle is an involution
        const int64_t t = m0 + r;
        const int64_t nn = col + 8 * lc;
        const u32x4 v = *(const u32x4*)(stage + r * 128 + (pc << 4));
        if (t < M && nn < D) __builtin_nontemporal_store(v, (u32x4*)(X + t * ldx + nn));
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);            // reads done before the next slab's writes
    }
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
  const int64_t waves = ((M + kEmbedTokens - 1) / kEmbedTokens) *
                        ((D + kEmbedCols - 1) / kEmbedCols);
  const int64_t blocks = (waves + kThreads / 64 - 1) / (kThreads / 64);
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const int vec_e = (C % 8 == 0) && (((uintptr_t)E & 15u) == 0);
  hipLaunchKernelGGL(embed_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, z, E, X, ldx,
                     M, C, D, vec_e);
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
