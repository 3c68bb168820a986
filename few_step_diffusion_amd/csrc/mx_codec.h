// MXFP8 block codec shared by the quantizer kernel (mx.hip) and the GEMM's
// fused SwiGLU->MXFP8 epilogue (gemm.hip).  Format (OCP MX v1.0 reading):
// 32-element blocks, E8M0 scale 2^e with e = floor(log2 amax) - 8 clamped to
// [-127, 127], E4M3 elements rounded to nearest-even and saturated at 448.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fsd {

// Two E4M3 bytes of (y0, y1) into bits 0..15 (HI = false) or 16..31 (HI =
// true) of `old`: nearest-even, magnitudes past 448 saturated to 448, E4M3
// subnormals down to 2^-9.  gfx950's conversion (OCP E4M3) after a clamp to
// +-448; checked byte for byte against a bit-level nearest-even reference on a
// million values covering every binade from 2^-30 to 2^12, all rounding
// boundaries and ties, signed zeros and the 448..512 range.  (A NaN input
// gives the E4M3 NaN code.)
template <bool HI>
__device__ __forceinline__ uint32_t e4m3_pair(float y0, float y1, uint32_t old) {
  const float c0 = __builtin_amdgcn_fmed3f(y0, -448.0f, 448.0f);
  const float c1 = __builtin_amdgcn_fmed3f(y1, -448.0f, 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c0, c1, (int)old, HI);
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
  auto elem = [&](int idx) {                           // element idx of the block, scaled
    const uint32_t bits = (idx & 1) ? (w[idx >> 1] & 0xffff0000u) : (w[idx >> 1] << 16);
    return __uint_as_float(bits) * inv;
  };
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t lo = e4m3_pair<false>(elem(4 * i), elem(4 * i + 1), 0u);
    out[i] = e4m3_pair<true>(elem(4 * i + 2), elem(4 * i + 3), lo);
  }
  return (uint32_t)(e + 127);
}

}  // namespace fsd
