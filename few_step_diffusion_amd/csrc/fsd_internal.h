// Internal declarations shared by the HIP translation units of libfsd.so.
// Not part of the public ABI (include/fsd.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fsd {

typedef uint16_t bf16_t;   // bfloat16 storage word

// One MFMA GEMM launch: Y = epi(alpha · [A0 | A1]·[B0 | B1]ᵀ + bias) (+ res).
// Segment 0 runs over K0 columns of (A0, B0), segment 1 over K1 columns of
// (A1, B1); K1 == 0 disables segment 1.  A* are [M, K*] with row stride lda*,
// B* are [N, K*] with row stride ldb*.  With SwiGLU the N accumulator columns
// are [gate | up] halves and Y has N/2 columns.
// For the MXFP8 kinds the operands are E4M3 bytes (lengths K0, K1 and strides
// in elements = bytes, K a multiple of 128) and sA*, sB* their E8M0 scales in
// the layout mx.hip writes (per 128-k step and 64-row group, 64 dwords), for
// sMp (A) and sNp (B) rows: the operand's row count rounded up to 256.
struct GemmParams {
  const void* A0; int64_t lda0;
  const void* B0; int64_t ldb0;
  const void* A1; int64_t lda1;
  const void* B1; int64_t ldb1;
  int64_t M, N, K0, K1;
  float alpha;
  const float* bias;
  const bf16_t* res; int64_t ldr;
  bf16_t* Y; int64_t ldy;
  const uint8_t* sA0; const uint8_t* sB0;
  const uint8_t* sA1; const uint8_t* sB1;
  int64_t sMp, sNp;
  // MXFP8 output (GEMM_MX_UP_SWIGLU_MX: SwiGLU's H, [M, N/2]; GEMM_MX_DOWN_Q and
  // GEMM_MX_UP_Q: output columns [q0, q1), as a matrix [M, q1 - q0] padded to a
  // multiple of 128): E4M3 bytes with row stride ldyq and their scales for sYp
  // (M rounded up to 256) rows
  uint8_t* Yq; int64_t ldyq;
  uint8_t* Ys; int64_t sYp;
  int64_t q0, q1;
  // MXFP8 operands of one row chunk inside larger scale arrays: A0's rows start
  // at 64-row group sa_g0 of sA0 (sMp rows), the output's at group sy_g0 of Ys
  // (sYp rows); sA1 holds sMp1 rows (0: sMp)
  int64_t sa_g0, sy_g0, sMp1;
};

enum GemmKind {
  GEMM_DOWN = 0,        // phase A: T = bf16(alpha · X·Aᵀ), N = rank (tile 256 x 192)
  GEMM_UP = 1,          // phase B, plain / bias / residual epilogue (tile 256 x 256)
  GEMM_UP_SWIGLU = 2,   // phase B with the SwiGLU epilogue
  GEMM_MX_DOWN = 3,     // the same three with MXFP8 operands
  GEMM_MX_UP = 4,
  GEMM_MX_UP_SWIGLU = 5,
  GEMM_MX_UP_SWIGLU_MX = 6, // ... whose H leaves quantized to MXFP8 (N/2 % 128 == 0)
  GEMM_MX_DOWN_Q = 7,       // MX phase A whose T leaves as MXFP8 (Y may be null)
  GEMM_MX_UP_Q = 8          // MX phase B, bf16 Y plus MXFP8 of columns [q0, q1)
};

hipError_t launch_gemm(GemmKind kind, const GemmParams& p, hipStream_t s);
// Phase B of one chunk (pb: GEMM_UP, or GEMM_UP_SWIGLU when swiglu) and phase A
// of the next (pa: GEMM_DOWN) in one launch; either may have M == 0.
hipError_t launch_gemm_pair(bool swiglu, const GemmParams& pb, const GemmParams& pa,
                            hipStream_t s);
// The same on MXFP8 operands: phase B of one chunk (pb: GEMM_MX_UP, _UP_Q,
// _UP_SWIGLU or _UP_SWIGLU_MX by swiglu / qout) and phase A of the next, its T
// leaving as MXFP8 (pa: GEMM_MX_DOWN_Q).
hipError_t launch_gemm_pair_mx(bool swiglu, bool qout, const GemmParams& pb,
                               const GemmParams& pa, hipStream_t s);

hipError_t launch_renoise(const float* u, const float* eps, float sigma, float* z,
                          int64_t n, hipStream_t s);
hipError_t launch_euler(float* z, const float* v, float dsigma, int64_t n, hipStream_t s);
hipError_t launch_merge_rows(const float* src, int64_t rows, int64_t cols, bf16_t* dst,
                             int64_t ld_dst, hipStream_t s);
hipError_t launch_merge_cols(const float* src, int64_t rows, int64_t cols, float scale,
                             bf16_t* dst, int64_t ld_dst, hipStream_t s);
hipError_t launch_embed(const float* z, const bf16_t* E, bf16_t* X, int64_t ldx, int64_t M,
                        int C, int64_t D, hipStream_t s);
// embed whose X also leaves as MXFP8 (codes [M, D] with row stride ldxq, scales
// for M rounded up to 256 rows; D a multiple of 128)
hipError_t launch_embed_mx(const float* z, const bf16_t* E, bf16_t* X, int64_t ldx, int64_t M,
                           int C, int64_t D, uint8_t* Xq, int64_t ldxq, uint8_t* Xs,
                           hipStream_t s);
hipError_t launch_head(const bf16_t* H, int64_t ldh, const bf16_t* P, float* v, int64_t M,
                       int64_t D, int C, hipStream_t s);
hipError_t launch_head_euler(const bf16_t* H, int64_t ldh, const bf16_t* P, float* z,
                             float dsigma, int64_t M, int64_t D, int C, hipStream_t s);
// Dense attention over S tokens, H heads of 128: O = softmax(Q·Kᵀ·scale)·V per
// head; V is first transposed per head into Vt ([H·128][attention_padded_tokens(S)]).
int64_t attention_padded_tokens(int64_t S);
hipError_t launch_attention(const bf16_t* Q, const bf16_t* K, const bf16_t* V, int64_t ld,
                            bf16_t* O, int64_t ldo, int64_t S, int H, float scale,
                            bf16_t* Vt, hipStream_t s);
hipError_t launch_mx_quantize(const bf16_t* X, int64_t ldx, int64_t M, int64_t K, uint8_t* Q,
                              int64_t ldq, uint8_t* S, hipStream_t s);

}  // namespace fsd
