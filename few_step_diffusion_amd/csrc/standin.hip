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
// head:  v[m, c] = sum_n H[m, n]·P[c, n].  A read-bound GEMM with N = C <= 32
//   (zero-padded to 32).  One wave per block owns 64 rows (two 32-row MFMA
//   blocks) and walks k in steps of 64 through a 4-stage LDS ring filled by
//   LDS-DMA (buffer_load ... lds): every load moves whole 128-byte lines of H
//   (8 rows x 128 B), which direct register loads in the MFMA's lane layout
//   (one row per lane) cannot.  Each stage also holds the 32 x 64 slab of P;
//   rows past M or C fall outside their buffers and read as zeros.  Rows are
//   stored with their 16-byte chunks XOR-swizzled by (row >> 1) & 7.
// head + Euler: the same kernel applies the sampler's Euler update
//   z <- z + (sigma_next - sigma)·v ("Open-H3-Regenerate-2K: High-Resolution
//   Video Refinement with Few-Step Diffusion" (agientry.com), section "Three
//   steps instead of dozens", Euler update equation) to the latent in place
//   as it produces v, so v never goes through HBM.
#include "fsd_internal.h"
#include "mx_codec.h"

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
constexpr int kHeadRows = 64;                // rows per (one-wave) block
constexpr int kHeadStages = 4;
constexpr int kHeadHBytes = kHeadRows * 128;  // 64 k of 64 rows
constexpr int kHeadStage = kHeadHBytes + 32 * 128;   // + 64 k of 32 (padded) P rows
constexpr int kHeadLoads = kHeadRows / 8 + 4;        // LDS-DMA loads per stage

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

// QX: X also leaves as MXFP8 (codes Xq with row stride ldxq, scales Xs for sMp
// rows in the quantizer's layout; D a multiple of 128, so every slab is 64
// whole columns): after a slab's bf16 rows are written, lane l quantizes the
// two 32-column blocks of staged rows l and l + 64, exactly as the quantizer
// would from the stored X, puts the codes over the row's first four chunks
// (already read) and the slab's codes leave as 64-byte row segments.
template <bool QX>
__global__ __launch_bounds__(kThreads) void embed_kernel(const float* z, const bf16_t* E,
                                                         bf16_t* X, int64_t ldx, int64_t M,
                                                         int C, int64_t D, int vec_e,
                                                         uint8_t* Xq, int64_t ldxq, uint8_t* Xs,
                                                         int64_t sMp) {
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
      if constexpr (QX) {
        // scale bytes of the slab: 2 blocks x 2 64-row groups x 16 dwords,
        // dword (2·blk + group)·16 + r holding rows 16i + r of the group
        __shared__ __attribute__((aligned(16))) uint8_t sc_all[(kThreads / 64) * 256];
        uint8_t* sl = sc_all + (threadIdx.x >> 6) * 256;
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
          const int r = lane + 64 * rr;
          const int64_t t = m0 + r;
#pragma unroll
          for (int blk = 0; blk < 2; ++blk) {
            uint32_t w[16];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const u32x4 v = *(const u32x4*)(stage + r * 128 + (embed_swz(r, 4 * blk + c) << 4));
              w[4 * c] = v.x; w[4 * c + 1] = v.y; w[4 * c + 2] = v.z; w[4 * c + 3] = v.w;
            }
            uint32_t q[8];
            const uint32_t sbyte = mx_block_bf16(w, q);
            {
              char* rowp = stage + r * 128;
              *(u32x4*)(rowp + (embed_swz(r, 2 * blk) << 4)) = (u32x4){q[0], q[1], q[2], q[3]};
              *(u32x4*)(rowp + (embed_swz(r, 2 * blk + 1) << 4)) = (u32x4){q[4], q[5], q[6], q[7]};
            }
            sl[((2 * blk + rr) * 16 + (r & 15)) * 4 + ((r & 63) >> 4)] =
                (uint8_t)(t < M ? sbyte : 127u);
          }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);
#pragma unroll
        for (int it = 0; it < kEmbedTokens / 16; ++it) {
          const int r = 16 * it + (lane >> 2), ch = lane & 3;
          const int64_t t = m0 + r;
          if (t < M) {
            const u32x4 v = *(const u32x4*)(stage + r * 128 + (embed_swz(r, ch) << 4));
            __builtin_nontemporal_store(v, (u32x4*)(Xq + t * ldxq + col + 16 * ch));
          }
        }
        // lane = 32·blk + 16·group + r
        const int blk = lane >> 5, grp = (lane >> 4) & 1, r16 = lane & 15;
        const int64_t B = (col >> 5) + blk;
        const int64_t base = (B >> 2) * (sMp >> 6);
        uint32_t* sdst = (uint32_t*)Xs + 16 * (B & 3) + r16;
        __builtin_nontemporal_store(*(const uint32_t*)(sl + lane * 4),
                                    sdst + (base + (m0 >> 6) + grp) * 64);
        // the last token wave also fills the padding groups up to sMp (rows
        // past M, never covered by a wave of 128 tokens): scale 127
        if (m0 + kEmbedTokens >= M && m0 + kEmbedTokens < sMp)
          __builtin_nontemporal_store(0x7f7f7f7fu, sdst + (base + (m0 >> 6) + 2 + grp) * 64);
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);            // reads done before the next slab's writes
    }
  }
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

template <int n>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(n >= 0 && n < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (0 << 8) | ((n >> 4) << 14));
}

// EULER: instead of writing v, apply the Euler update z += dsigma·v in place
// (v never leaves registers; same fp32 fma as the separate Euler kernel).
template <bool EULER>
__global__ __launch_bounds__(64) void head_kernel(const bf16_t* H, int64_t ldh, const bf16_t* P,
                                                  float* v, int64_t M, int64_t D, int C,
                                                  float dsigma) {
  __shared__ __attribute__((aligned(1024))) char lds[kHeadStages * kHeadStage];
  const int lane = threadIdx.x;
  const int64_t m0 = (int64_t)blockIdx.x * kHeadRows;
  const int64_t rows_valid = (M - m0) < kHeadRows ? (M - m0) : kHeadRows;
  const __amdgpu_buffer_rsrc_t rH = make_rsrc(H + m0 * ldh, rows_valid * ldh * 2);
  const __amdgpu_buffer_rsrc_t rP = make_rsrc(P, (int64_t)C * D * 2);   // rows >= C read 0
  const int nk = (int)(D / 64);
  // LDS-DMA: load i moves rows 8i .. 8i+7 of the stage's H slab (i < 8) or of
  // its P slab (i >= 8); lane l fills row 8i + l/8, physical chunk l%8 with
  // logical chunk swz(row, l%8).  The key ((8i + l/8) >> 1) & 7 only depends
  // on the lane and on the parity of i.
  const int lrow = lane >> 3;
  const uint32_t cx_even = (uint32_t)(((lane & 7) ^ ((lrow >> 1) & 7)) * 16);
  const uint32_t cx_odd = (uint32_t)(((lane & 7) ^ (((lrow >> 1) + 4) & 7)) * 16);
  auto issue = [&](int kt, int st) {
    const bool live = kt < nk;
    const uint32_t kb = (uint32_t)kt * 128;
    char* base = lds + st * kHeadStage;
#pragma unroll
    for (int i = 0; i < kHeadRows / 8; ++i) {
      const uint32_t cx = (i & 1) ? cx_odd : cx_even;
      const uint32_t off = live ? (uint32_t)((8 * i + lrow) * ldh * 2) + kb + cx : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rH, (lds_ptr_t)(base + i * 1024), 16, off, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t cx = (i & 1) ? cx_odd : cx_even;
      const uint32_t off = live ? (uint32_t)((8 * i + lrow) * D * 2) + kb + cx : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rP, (lds_ptr_t)(base + kHeadHBytes + i * 1024), 16,
                                               off, 0, 0, 0);
    }
  };
  // fragments: lane l reads row 32·bi + l%32 (P: row l%32), logical chunk
  // 2·ks + l/32; for such rows the key ((l%32) >> 1) & 7 is the lane's own
  const int j = lane & 31;
  const int h = lane >> 5;
  const int key = (j >> 1) & 7;
  f32x16 acc[2];
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[bi][e] = 0.0f;
#pragma unroll
  for (int st = 0; st < kHeadStages - 1; ++st) issue(st, st);
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt % kHeadStages;
    wait_vm_lgkm0<(kHeadStages - 2) * kHeadLoads>();   // step kt has landed
    // stage (kt - 1) % stages was read in the previous iteration (those reads
    // have retired: the wait above also drained lgkmcnt)
    issue(kt + kHeadStages - 1, (kt + kHeadStages - 1) % kHeadStages);
    const char* base = lds + st * kHeadStage;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int co = ((2 * ks + h) ^ key) * 16;
      const bf16x8 pf = *(const bf16x8*)(base + kHeadHBytes + j * 128 + co);
#pragma unroll
      for (int bi = 0; bi < 2; ++bi) {
        const bf16x8 hf = *(const bf16x8*)(base + (32 * bi + j) * 128 + co);
        acc[bi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hf, pf, acc[bi], 0, 0, 0);
      }
    }
  }
  wait_vm_lgkm0<0>();   // the out-of-range loads past the end have landed too
  if (j >= C) return;
  // lane holds channel j of rows 32·bi + 8·(e/4) + 4·h + e%4
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int i = 32 * bi + 8 * (e >> 2) + 4 * h + (e & 3);
      if (i < rows_valid) {
        float* out = v + (m0 + i) * C + j;
        if constexpr (EULER) *out = fmaf(dsigma, acc[bi][e], *out);
        else *out = acc[bi][e];
      }
    }
}

}  // namespace

hipError_t launch_embed(const float* z, const bf16_t* E, bf16_t* X, int64_t ldx, int64_t M,
                        int C, int64_t D, hipStream_t s) {
  if (C < 1 || C > kMaxC) return hipErrorInvalidValue;   // the kernels take at most 32 channels
  if (M == 0) return hipSuccess;
  const int64_t waves = ((M + kEmbedTokens - 1) / kEmbedTokens) *
                        ((D + kEmbedCols - 1) / kEmbedCols);
  const int64_t blocks = (waves + kThreads / 64 - 1) / (kThreads / 64);
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const int vec_e = (C % 8 == 0) && (((uintptr_t)E & 15u) == 0);
  hipLaunchKernelGGL(embed_kernel<false>, dim3((unsigned)blocks), dim3(kThreads), 0, s, z, E, X,
                     ldx, M, C, D, vec_e, nullptr, (int64_t)0, nullptr, (int64_t)0);
  return hipGetLastError();
}

hipError_t launch_embed_mx(const float* z, const bf16_t* E, bf16_t* X, int64_t ldx, int64_t M,
                           int C, int64_t D, uint8_t* Xq, int64_t ldxq, uint8_t* Xs,
                           hipStream_t s) {
  if (C < 1 || C > kMaxC) return hipErrorInvalidValue;   // the kernels take at most 32 channels
  if (M == 0) return hipSuccess;
  if (D % 128) return hipErrorInvalidValue;
  const int64_t waves = ((M + kEmbedTokens - 1) / kEmbedTokens) *
                        ((D + kEmbedCols - 1) / kEmbedCols);
  const int64_t blocks = (waves + kThreads / 64 - 1) / (kThreads / 64);
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const int vec_e = (C % 8 == 0) && (((uintptr_t)E & 15u) == 0);
  const int64_t sMp = (M + 255) / 256 * 256;
  hipLaunchKernelGGL(embed_kernel<true>, dim3((unsigned)blocks), dim3(kThreads), 0, s, z, E, X,
                     ldx, M, C, D, vec_e, Xq, ldxq, Xs, sMp);
  return hipGetLastError();
}

hipError_t launch_head(const bf16_t* H, int64_t ldh, const bf16_t* P, float* v, int64_t M,
                       int64_t D, int C, hipStream_t s) {
  if (C < 1 || C > kMaxC) return hipErrorInvalidValue;   // the kernels take at most 32 channels
  if (M == 0) return hipSuccess;
  const int64_t blocks = (M + kHeadRows - 1) / kHeadRows;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(head_kernel<false>, dim3((unsigned)blocks), dim3(64), 0, s, H, ldh, P, v, M,
                     D, C, 0.0f);
  return hipGetLastError();
}

hipError_t launch_head_euler(const bf16_t* H, int64_t ldh, const bf16_t* P, float* z,
                             float dsigma, int64_t M, int64_t D, int C, hipStream_t s) {
  if (C < 1 || C > kMaxC) return hipErrorInvalidValue;   // the kernels take at most 32 channels
  if (M == 0) return hipSuccess;
  const int64_t blocks = (M + kHeadRows - 1) / kHeadRows;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(head_kernel<true>, dim3((unsigned)blocks), dim3(64), 0, s, H, ldh, P, z, M,
                     D, C, dsigma);
  return hipGetLastError();
}

}  // namespace fsd
