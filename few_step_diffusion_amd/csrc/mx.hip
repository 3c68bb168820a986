// MXFP8 (E4M3 elements, E8M0 scales per 32 elements) for the linears of the
// refiner.
//
// The pages run the refiner's linears in MXFP8 (FP8 GEMMs whose operands are
// quantized again at every stage), with SwiGLU fused into a one-pass activation
// quantizer ("Open-H3-Regenerate-2K: High-Resolution Video Refinement with
// Few-Step Diffusion", agientry.com, section "Where the 3.9x speedup comes
// from", inference-configuration table).  They fix no block size, scale rule or
// rounding; this file follows the OCP Microscaling (MX) v1.0 format:
//   * blocks of 32 consecutive elements along K;
//   * shared scale 2^e, e = floor(log2(amax)) - 8 (8 = E4M3's top exponent),
//     clamped to E8M0's [-127, 127] and stored as e + 127;
//   * elements x·2^-e rounded to nearest-even in E4M3 (bias 7, 3 mantissa
//     bits, subnormals to 2^-9), magnitudes past 448 saturated to 448.
//
// Layout written here (and read by the MXFP8 GEMM): elements as bytes [M, Kp]
// with Kp = K rounded up to a multiple of 128 (one GEMM K step), the padding
// zero.  Scales are grouped by K step t (128 elements) and 64-row group g:
// dword (t·Mp/64 + g)·64 + 16·b + r holds in its byte i the scale of row
// 64g + 16i + r over block 4t + b, for t < Kp/128, g < Mp/64 with Mp = M
// rounded up to 256, and b, i < 4, r < 16 (padded rows and blocks hold 127, a
// scale of 1).  That is the order in which the GEMM's 64 lanes take a row
// block's scales, with one dword serving four 16-row blocks.
#include "fsd_internal.h"
#include "mx_codec.h"

namespace fsd {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void mx_quantize_kernel(const bf16_t* X, int64_t ldx,
                                                               int64_t M, int64_t K, uint8_t* Q,
                                                               int64_t ldq, uint8_t* S,
                                                               int64_t Mp, int64_t Kp) {
  const int64_t nb = Kp / 32;                          // blocks per row
  const int64_t id = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (id >= Mp * nb) return;
  const int64_t m = id / nb;
  const int64_t b = id - m * nb;
  uint8_t* s_out =
      S + (((b >> 2) * (Mp >> 6) + (m >> 6)) * 64 + (b & 3) * 16 + (m & 15)) * 4 + ((m >> 4) & 3);
  if (m >= M) {                                        // padded row: scale only
    *s_out = 127;
    return;
  }
  uint32_t out[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
  uint32_t sbyte = 127u;                               // a block past K: zeros, scale 1
  if (b * 32 < K) {
    uint32_t w[16];                                    // 32 bf16, two per word
    const u32x4* src = (const u32x4*)(X + m * ldx + b * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 v = src[i];
      w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
    }
    sbyte = mx_block_bf16(w, out);
  }
  u32x4* dst = (u32x4*)(Q + m * ldq + b * 32);
  dst[0] = (u32x4){out[0], out[1], out[2], out[3]};
  dst[1] = (u32x4){out[4], out[5], out[6], out[7]};
  *s_out = (uint8_t)sbyte;
}

}  // namespace

hipError_t launch_mx_quantize(const bf16_t* X, int64_t ldx, int64_t M, int64_t K, uint8_t* Q,
                              int64_t ldq, uint8_t* S, hipStream_t s) {
  const int64_t Kp = (K + 127) / 128 * 128;
  const int64_t Mp = (M + 255) / 256 * 256;
  const int64_t total = Mp * (Kp / 32);
  const int64_t blocks = (total + kThreads - 1) / kThreads;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mx_quantize_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, X, ldx,
                     M, K, Q, ldq, S, Mp, Kp);
  return hipGetLastError();
}

}  // namespace fsd
