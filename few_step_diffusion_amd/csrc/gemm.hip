// bf16 MFMA GEMM for the two phases of the LoRA-fused linear on gfx950.
//
// Source of the operation: each adapted linear layer of the refiner's
// transformer computes X·W0ᵀ + s·(X·Aᵀ)·Bᵀ with the merged rank-576 LoRA
// ("Open-H3-Regenerate-2K：MiniMax H3 的开源 4K 精修方案", comfyui-wiki.com,
// section "三个步如何完成工作").  Phase A writes T = bf16(s·X·Aᵀ); phase B
// runs one K-loop over the concatenation [X | T]·[W0 | B]ᵀ, so the LoRA
// up-projection costs no extra pass over Y.  The SwiGLU epilogue follows
// Shazeer, "GLU Variants Improve Transformer" (2020).
//
// Kernel shape (one workgroup = 4 waves of 64 lanes, one output tile):
//   * tile BM x BN = 256 x (64·WN), K staged through LDS in steps of 64;
//     each wave owns a (32·WM) x (32·WN) sub-tile = WM x WN blocks of the
//     32x32x16 bf16 MFMA (v_mfma_f32_32x32x16_bf16), fp32 accumulators.
//   * operands are K-contiguous rows (X row-major, W0 in out x in layout), so
//     a lane's MFMA fragment (8 consecutive k of one row) is one 16-byte
//     chunk.  Global -> LDS moves 16-byte chunks with buffer loads whose
//     range check returns zeros for rows past M or N; a K tail is zeroed by
//     pushing the offset out of range.
//   * LDS holds two stages (double buffer, one barrier per K step).  Each
//     128-byte tile row stores its eight chunks XOR-swizzled by
//     (row ^ row>>3) & 7, so the 16-byte fragment reads of 8 or 16
//     consecutive rows hit distinct banks.
//   * workgroup ids are remapped so that each XCD (ids round-robin over 8)
//     gets a contiguous run of tiles, ordered in groups of 4 tile-rows: the
//     32 tiles an XCD runs at once share 4 X-tiles and 8 W-tiles in its L2.
#include "fsd_internal.h"

namespace fsd {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int BK = 64;
constexpr int kChunks = BK / 8;          // 16-byte chunks per tile row and stage
constexpr int kRowsPerPass = kThreads / kChunks;   // 32 tile rows per load pass
constexpr int kGroupM = 4;
constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ __forceinline__ int lds_slot(int r, int c) {
  return r * kChunks + (c ^ ((r ^ (r >> 3)) & 7));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float((uint32_t)h << 16);
}
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, (__bf16)f);
}

template <int WM, int WN, bool SWIGLU>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmParams p) {
  constexpr int BM = 64 * WM;
  constexpr int BN = 64 * WN;
  constexpr int A_LOADS = BM / kRowsPerPass;
  constexpr int B_LOADS = BN / kRowsPerPass;
  constexpr int STAGE = (BM + BN) * kChunks;
  static_assert(!SWIGLU || (WN % 2 == 0), "SwiGLU pairs gate and up blocks within a wave");
  __shared__ u32x4 lds[2 * STAGE];

  // ---- which tile ---------------------------------------------------------
  const int64_t M = p.M;
  const int64_t N = p.N;
  const int64_t F = N / 2;
  constexpr int TN = SWIGLU ? BN / 2 : BN;        // output columns per tile
  const int64_t Nout = SWIGLU ? F : N;
  const int tiles_m = (int)((M + BM - 1) / BM);
  const int tiles_n = (int)((Nout + TN - 1) / TN);
  const int total = tiles_m * tiles_n;
  const int wg = blockIdx.x;
  const int xcd = wg & 7, local = wg >> 3;
  const int per = total >> 3, rem = total & 7;
  const int L = xcd * per + (xcd < rem ? xcd : rem) + local;
  const int group_tiles = kGroupM * tiles_n;
  const int grp = L / group_tiles;
  const int first_m = grp * kGroupM;
  const int gm = (tiles_m - first_m) < kGroupM ? (tiles_m - first_m) : kGroupM;
  const int in_g = L - grp * group_tiles;
  const int tm = first_m + in_g % gm;
  const int tn = in_g / gm;

  const int64_t m0 = (int64_t)tm * BM;
  const int64_t rows_valid = (M - m0) < BM ? (M - m0) : BM;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int ld_row = t >> 3;
  const int ld_chunk = t & 7;

  // ---- buffer resources ------------------------------------------------------
  const __amdgpu_buffer_rsrc_t rA0 = make_rsrc(p.A0 + m0 * p.lda0, rows_valid * p.lda0 * 2);
  const __amdgpu_buffer_rsrc_t rB0 = make_rsrc(p.B0, N * p.ldb0 * 2);
  const bool has1 = p.K1 > 0;
  const __amdgpu_buffer_rsrc_t rA1 =
      has1 ? make_rsrc(p.A1 + m0 * p.lda1, rows_valid * p.lda1 * 2) : rA0;
  const __amdgpu_buffer_rsrc_t rB1 = has1 ? make_rsrc(p.B1, N * p.ldb1 * 2) : rB0;

  // global row (of B) held by tile row rt
  auto b_row = [&](int rt) -> int64_t {
    if constexpr (SWIGLU) {
      constexpr int WNC = WN * 32, HALFC = WNC / 2;
      const int wn_ = rt / WNC, within = rt % WNC;
      const int half = within / HALFC;
      const int64_t j = (int64_t)tn * TN + wn_ * HALFC + within % HALFC;
      return half * F + j;          // up rows past N read as zeros
    } else {
      return (int64_t)tn * TN + rt; // rows past N read as zeros
    }
  };
  uint32_t b_off0[B_LOADS], b_off1[B_LOADS];
#pragma unroll
  for (int i = 0; i < B_LOADS; ++i) {
    const int64_t n = b_row(ld_row + kRowsPerPass * i);
    b_off0[i] = (uint32_t)(n * p.ldb0 * 2);
    b_off1[i] = (uint32_t)(n * p.ldb1 * 2);
  }

  const int nk0 = (int)((p.K0 + BK - 1) / BK);
  const int nk1 = (int)((p.K1 + BK - 1) / BK);
  const int nk = nk0 + nk1;

  u32x4 ra[A_LOADS], rb[B_LOADS];
  auto gload = [&](int kt) {
    const bool seg1 = kt >= nk0;
    const int64_t kbase = (int64_t)(seg1 ? kt - nk0 : kt) * BK + ld_chunk * 8;
    const int64_t kseg = seg1 ? p.K1 : p.K0;
    const uint32_t koff = kbase < kseg ? (uint32_t)(kbase * 2) : kOutOfRange;
    const int64_t lda = seg1 ? p.lda1 : p.lda0;
    const __amdgpu_buffer_rsrc_t rA = seg1 ? rA1 : rA0;
    const __amdgpu_buffer_rsrc_t rB = seg1 ? rB1 : rB0;
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
      const uint32_t off = (uint32_t)((ld_row + kRowsPerPass * i) * lda * 2) + koff;
      ra[i] = __builtin_amdgcn_raw_buffer_load_b128(rA, off, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) {
      const uint32_t off = (seg1 ? b_off1[i] : b_off0[i]) + koff;
      rb[i] = __builtin_amdgcn_raw_buffer_load_b128(rB, off, 0, 0);
    }
  };
  auto lstore = [&](int stage) {
    u32x4* base = lds + stage * STAGE;
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) base[lds_slot(ld_row + kRowsPerPass * i, ld_chunk)] = ra[i];
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i)
      base[BM * kChunks + lds_slot(ld_row + kRowsPerPass * i, ld_chunk)] = rb[i];
  };

  f32x16 acc[WM][WN];
#pragma unroll
  for (int bi = 0; bi < WM; ++bi)
#pragma unroll
    for (int bj = 0; bj < WN; ++bj)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[bi][bj][v] = 0.0f;

  gload(0);
  lstore(0);
  __syncthreads();

  const int frag_row = lane & 31;
  const int frag_chunk = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const u32x4* As = lds + cur * STAGE;
    const u32x4* Bs = As + BM * kChunks;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 a[WM], b[WN];
#pragma unroll
      for (int bi = 0; bi < WM; ++bi) {
        const int r = wm * WM * 32 + bi * 32 + frag_row;
        a[bi] = __builtin_bit_cast(bf16x8, As[lds_slot(r, 2 * ks + frag_chunk)]);
      }
#pragma unroll
      for (int bj = 0; bj < WN; ++bj) {
        const int r = wn * WN * 32 + bj * 32 + frag_row;
        b[bj] = __builtin_bit_cast(bf16x8, Bs[lds_slot(r, 2 * ks + frag_chunk)]);
      }
#pragma unroll
      for (int bi = 0; bi < WM; ++bi)
#pragma unroll
        for (int bj = 0; bj < WN; ++bj)
          acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[bi], b[bj], acc[bi][bj], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue ---------------------------------------------------------------
  // Accumulator v of block (bi, bj) holds row 8·(v/4) + 4·(lane/32) + v%4 and
  // column lane%32 of that 32x32 block.
  const float alpha = p.alpha;
  const int col_in_block = lane & 31;
  const int row_in_block = 4 * (lane >> 5);
  if constexpr (SWIGLU) {
    constexpr int HALF = WN / 2;
#pragma unroll
    for (int bj = 0; bj < HALF; ++bj) {
      const int64_t j = (int64_t)tn * TN + wn * HALF * 32 + bj * 32 + col_in_block;
      const bool col_ok = j < F;
      const float bg = (p.bias && col_ok) ? p.bias[j] : 0.0f;
      const float bu = (p.bias && col_ok) ? p.bias[F + j] : 0.0f;
#pragma unroll
      for (int bi = 0; bi < WM; ++bi)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int i = wm * WM * 32 + bi * 32 + 8 * (v >> 2) + row_in_block + (v & 3);
          if (col_ok && i < rows_valid) {
            const float g = acc[bi][bj][v] * alpha + bg;
            const float u = acc[bi][bj + HALF][v] * alpha + bu;
            const float h = g / (1.0f + __expf(-g)) * u;
            p.Y[(m0 + i) * p.ldy + j] = f32_to_bf16(h);
          }
        }
    }
  } else {
#pragma unroll
    for (int bj = 0; bj < WN; ++bj) {
      const int64_t n = (int64_t)tn * TN + wn * WN * 32 + bj * 32 + col_in_block;
      const bool col_ok = n < N;
      const float bn = (p.bias && col_ok) ? p.bias[n] : 0.0f;
#pragma unroll
      for (int bi = 0; bi < WM; ++bi)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int i = wm * WM * 32 + bi * 32 + 8 * (v >> 2) + row_in_block + (v & 3);
          if (col_ok && i < rows_valid) {
            float y = acc[bi][bj][v] * alpha + bn;
            if (p.res) y += bf16_to_f32(p.res[(m0 + i) * p.ldr + n]);
            p.Y[(m0 + i) * p.ldy + n] = f32_to_bf16(y);
          }
        }
    }
  }
}

template <int WM, int WN, bool SWIGLU>
hipError_t launch(const GemmParams& p, hipStream_t s) {
  constexpr int BM = 64 * WM;
  constexpr int TN = SWIGLU ? 32 * WN : 64 * WN;
  const int64_t nout = SWIGLU ? p.N / 2 : p.N;
  const int64_t tiles = ((p.M + BM - 1) / BM) * ((nout + TN - 1) / TN);
  if (tiles <= 0) return hipSuccess;
  if (tiles > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_kernel<WM, WN, SWIGLU>), dim3((unsigned)tiles), dim3(kThreads), 0, s,
                     p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(GemmKind kind, const GemmParams& p, hipStream_t s) {
  switch (kind) {
    case GEMM_DOWN: return launch<4, 3, false>(p, s);
    case GEMM_UP: return launch<4, 4, false>(p, s);
    case GEMM_UP_SWIGLU: return launch<4, 4, true>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace fsd
