// MXFP8 block codec shared by the quantizer kernel (mx.hip) and the GEMM's
// fused SwiGLU->MXFP8 epilogue (gemm.hip).  Format (OCP MX v1.0 reading):
// 32-element blocks, E8M0 scale 2^e with e = floor(log2 amax) - 8 clamped to
// [-127, 127], E4M3 elements rounded to nearest-even and saturated at 448.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fsd {

// E4M3 byte of y (finite fp32), nearest-even, saturated to 448.
__device__ __forceinline__ uint32_t to_e4m3(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a >= 0x43e00000u) return sign | 0x7eu;          // |y| >= 448
  if (a >= 0x3c800000u) {                              // |y| >= 2^-6: normal in E4M3
    uint32_t q = a >> 20;                              // fp32 exponent and top 3 mantissa bits
    const uint32_t rem = a & 0xfffffu;
    q += (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) ? 1u : 0u;
    q -= 120u << 3;                                    // rebias 127 -> 7
    return sign | (q > 0x7eu ? 0x7eu : q);
  }
  // subnormal in E4M3: k·2^-9 with k = nearest-even |y|·2^9 in 0..8 (8 = 2^-6)
  const uint32_t k = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  return sign | k;
}

// Quantizes one block of 32 bf16 values, packed two per word (element 2i in
// the low half of w[i]): writes the 32 E4M3 bytes to out[0..7] (element j in
// byte j % 4 of out[j / 4]) and returns the biased E8M0 scale byte.
__device__ __forceinline__ uint32_t mx_block_bf16(const uint32_t w[16], uint32_t out[8]) {
  // amax from the bf16 bit patterns (exact in fp32)
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t lo = (w[i] << 16) & 0x7fffffffu, hi = w[i] & 0x7fff0000u;
    amax = lo > amax ? lo : amax;
    amax = hi > amax ? hi : amax;
  }
  int e = -127;
  if (amax != 0) {
    e = (int)(amax >> 23) - 127 - 8;                   // floor(log2 amax) - 8
    if (e < -127) e = -127;                            // (a subnormal amax lands here too)
    if (e > 127) e = 127;
  }
  const float inv = __uint_as_float((uint32_t)(127 - e) << 23);   // 2^-e, exact
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int idx = 4 * i + j;
      const uint32_t bits = (idx & 1) ? (w[idx >> 1] & 0xffff0000u) : (w[idx >> 1] << 16);
      word |= to_e4m3(__uint_as_float(bits) * inv) << (8 * j);
    }
    out[i] = word;
  }
  return (uint32_t)(e + 127);
}

}  // namespace fsd
