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
// Kernel shape (one workgroup = 8 waves of 64 lanes, two per SIMD, one
// output tile):
//   * tile BM x BN = 256 x (64·WN); the waves form a 4 x 2 grid, each owning
//     a (32·WM) x (32·WN) sub-tile = 2WM x 2WN blocks of
//     v_mfma_f32_16x16x32_bf16 with fp32 accumulators (128 per lane at
//     WM = 2, WN = 4).  The W fragment is the MFMA's first operand, so a lane
//     ends up owning 4 consecutive output columns of one token.
//   * operands are K-contiguous rows (X row-major, W0 in out x in layout): a
//     lane's MFMA fragment (8 consecutive k of one row) is one 16-byte chunk.
//   * K is staged in steps of BK = 64, so a tile row of one step is one
//     128-byte L2 line and every L2 request is a whole line (at BK = 32 the
//     64-byte half-line requests doubled the L2 request rate, which was the
//     limit).  Global -> LDS uses 16-byte LDS-DMA buffer loads
//     (buffer_load ... lds): no VGPR staging, and the buffer range check turns
//     rows past M or N (and, by pushing the offset out of range, a K tail)
//     into zeros.
//   * A sits in a ring of three LDS slots and B in a ring of two (160 KB of
//     LDS in all).
//   * ping-pong: the two waves on a SIMD (waves w and w + 4) belong to two
//     groups that alternate, each K step, between a compute phase (all
//     MFMAs of the step back to back from fragments already in registers)
//     and a memory phase (every fragment of the next step from LDS, plus its
//     share of the LDS-DMA loads: group 1 loads A, group 0 loads B).  Two
//     barriers per step switch the phases, so a SIMD's MFMA pipe always has
//     one wave streaming MFMAs while the other does its memory work, instead
//     of both interleaving reads, loads and MFMAs.
//   * each 128-byte tile row stores its eight chunks XOR-swizzled by
//     (row>>1) & 7: the fragment reads of 16 consecutive rows then cover all
//     16 chunk slots of a 256-byte bank line (no bank conflicts).
//   * workgroup ids are remapped so that each XCD (ids round-robin over 8)
//     gets a contiguous run of tiles, ordered in groups of 4 tile-rows: the
//     32 tiles an XCD runs at once share 4 X tiles and 8 W tiles in its L2.
//   * residual: the loads the last two K steps issue for the steps past the
//     end land in four slots that are no longer read, so for plain 256 x 256
//     tiles they carry the tile's residual into the epilogue's staging layout
//     instead of zeros (measured at M = 532,800, K = 3072 + 576, N = 3072: the
//     residual's cost fell from 0.75 to 0.23 ms of 9.2).
//   * epilogue: each wave stages its bf16 results (and the residual) through
//     LDS and writes whole row segments with 16-byte non-temporal stores: the
//     output is written once and not re-read by this kernel, so it should not
//     evict the X and W lines that other tiles are re-reading from L2 and the
//     Infinity Cache.
#include <type_traits>
#include <utility>

#include "fsd_internal.h"
#include "mx_codec.h"

namespace fsd {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kWaveRows = 4;        // waves along M
constexpr int kWaveCols = 2;        // waves along N
constexpr int kWaves = kWaveRows * kWaveCols;
constexpr int kThreads = 64 * kWaves;
constexpr int BK = 64;              // k per LDS stage
constexpr int ROWB = BK * 2;        // bytes per tile row per stage: one 128-byte L2 line
constexpr int CPR = ROWB / 16;      // 16-byte chunks per tile row (8)
constexpr int RPL = 64 / CPR;       // tile rows per 64-lane LDS-DMA load (8)
constexpr int KS = BK / 32;         // MFMA k-blocks per stage (2 x 32 k)
constexpr int NSLOT_A = 3;          // LDS slots of the A ring (loads spread over a step)
constexpr int NSLOT_B = 2;          // LDS slots of the B ring
constexpr int kGroupM = 4;
constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

// Physical 16-byte chunk of logical chunk c in tile row `row` (an involution).
// Rows are 128 bytes, so two rows share one 256-byte bank line; XOR-ing the
// chunk with bits 1..3 of the row spreads 16 consecutive rows over all 16
// chunk slots of the line.
__device__ __forceinline__ int swz(int row, int c) { return c ^ ((row >> 1) & (CPR - 1)); }

// s_waitcnt with vmcnt <= n (n < 64), lgkmcnt = 0, expcnt untouched.
template <int n>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(n >= 0 && n < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (0 << 8) | ((n >> 4) << 14));
}

template <typename Fn, int... Is>
__device__ __forceinline__ void static_for_seq(Fn&& fn, std::integer_sequence<int, Is...>) {
  (fn(std::integral_constant<int, Is>{}), ...);
}
// fn(std::integral_constant<int, 0>) ... fn(std::integral_constant<int, N - 1>)
template <int N, typename Fn>
__device__ __forceinline__ void static_for(Fn&& fn) {
  static_for_seq(fn, std::make_integer_sequence<int, N>{});
}

// MX: E4M3 operands with E8M0 block scales (v_mfma_scale_f32_16x16x128_f8f6f4):
// a K step is 128 elements, still one 128-byte line per tile row.
// QOUT with SWIGLU: H leaves as MXFP8 (E4M3 bytes and scales) instead of bf16.
// QOUT without SWIGLU: the bf16 output (when p.Y is set) plus the MXFP8 form of
// its columns [p.q0, p.q1), in the bytes the quantizer would write from it.
constexpr int kLdsBytes = 160 * 1024;      // gfx950's LDS per CU: every tile shape fits

// One output tile of one GEMM (workgroup `wg` of the launch's tiles of this
// GEMM), staged through `lds` (kLdsBytes).
template <int WM, int WN, bool SWIGLU, bool MX, bool QOUT>
__device__ __forceinline__ void gemm_tile(const GemmParams& p, const int wg, char* lds) {
  constexpr int ESZ = MX ? 1 : 2;           // bytes per element
  constexpr int KSTEP = ROWB / ESZ;         // elements per K step
  constexpr int BM = kWaveRows * WM * 32;
  constexpr int BN = kWaveCols * WN * 32;
  constexpr int A_TOT = BM / RPL;           // LDS-DMA loads per stage (A)
  constexpr int B_TOT = BN / RPL;           // ... (B)
  constexpr int A_STAGE = BM * ROWB;        // bytes of one A stage
  constexpr int B_STAGE = BN * ROWB;
  constexpr int B_BASE = NSLOT_A * A_STAGE; // LDS: [A slots | B slots]
  constexpr int LDS_BYTES = NSLOT_A * A_STAGE + NSLOT_B * B_STAGE;
  static_assert(LDS_BYTES <= kLdsBytes, "gfx950 has 160 KB of LDS per CU");
  static_assert(!SWIGLU || (WN % 2 == 0), "SwiGLU pairs gate and up blocks within a wave");

  // ---- which tile ---------------------------------------------------------
  const int64_t M = p.M;
  const int64_t N = p.N;
  const int64_t F = N / 2;
  constexpr int TN = SWIGLU ? BN / 2 : BN;        // output columns per tile
  const int64_t Nout = SWIGLU ? F : N;
  const int tiles_m = (int)((M + BM - 1) / BM);
  const int tiles_n = (int)((Nout + TN - 1) / TN);
  const int total = tiles_m * tiles_n;
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

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / kWaveCols, wn = wave % kWaveCols;

  // ---- buffer resources ------------------------------------------------------
  const char* A0 = (const char*)p.A0;
  const char* A1 = (const char*)p.A1;
  const __amdgpu_buffer_rsrc_t rA0 = make_rsrc(A0 + m0 * p.lda0 * ESZ, rows_valid * p.lda0 * ESZ);
  const __amdgpu_buffer_rsrc_t rB0 = make_rsrc(p.B0, N * p.ldb0 * ESZ);
  const bool has1 = p.K1 > 0;
  const __amdgpu_buffer_rsrc_t rA1 =
      has1 ? make_rsrc(A1 + m0 * p.lda1 * ESZ, rows_valid * p.lda1 * ESZ) : rA0;
  const __amdgpu_buffer_rsrc_t rB1 = has1 ? make_rsrc(p.B1, N * p.ldb1 * ESZ) : rB0;

  // ---- global -> LDS assignment ------------------------------------------------
  // The two waves on a SIMD are wave w and wave w + 4, so the waves form two
  // groups of four, one wave per SIMD each (see the main loop).  Group 1
  // (waves 4..7) loads A and group 0 (waves 0..3) loads B.  Loader wl =
  // wave & 3 issues loads q = 4·i + wl of its operand: lane l writes LDS row
  // 8q + l/8 = 32·i + my_row, physical chunk l%8, fetching logical chunk
  // swz(row, l%8), so the eight lanes of a row fetch one whole 128-byte line.
  // Since 32·i leaves (row >> 1) & 7 unchanged, the swizzle depends on the
  // lane and wl only, and every row offset is a per-lane base plus a scalar
  // that only depends on i.
  constexpr int A_PER = (A_TOT + 3) / 4;    // loads per loader wave per step
  constexpr int B_PER = (B_TOT + 3) / 4;
  const int wl = wave & 3;
  const int wgrp = wave >> 2;
  const int my_row = wl * RPL + lane / CPR;            // tile row of load i = 0
  const uint32_t cx = (uint32_t)(swz(my_row, lane % CPR) * 16);
  // A rows: m0 + 32·i + my_row
  const uint32_t a_lane0 = (uint32_t)(my_row * p.lda0 * ESZ) + cx;
  const uint32_t a_lane1 = (uint32_t)(my_row * p.lda1 * ESZ) + cx;
  const uint32_t a_i0 = (uint32_t)(32 * p.lda0 * ESZ);
  const uint32_t a_i1 = (uint32_t)(32 * p.lda1 * ESZ);
  // B rows: tile row rt = 32·i + my_row holds global row tn·TN + my_row +
  // piece(i), plus F for the up half of a SwiGLU tile (rows past N read 0)
  const uint32_t b_lane0 = (uint32_t)(((int64_t)tn * TN + my_row) * p.ldb0 * ESZ) + cx;
  const uint32_t b_lane1 = (uint32_t)(((int64_t)tn * TN + my_row) * p.ldb1 * ESZ) + cx;
  auto b_piece = [&](int i, int64_t ldb) -> uint32_t {
    if constexpr (SWIGLU) {
      // wave column (i / 4) of 64 outputs; gate rows for i % 4 < 2, up rows after
      return (uint32_t)((((i / 4) * 64 + (i % 2) * 32) + ((i % 4) / 2) * F) * ldb * ESZ);
    } else {
      return (uint32_t)(32 * i * ldb * ESZ);
    }
  };

  // per-segment scalars, read once (selected by value inside the loop)
  const int K0 = __builtin_amdgcn_readfirstlane((int)p.K0);
  const int K1 = __builtin_amdgcn_readfirstlane((int)p.K1);
  const int nk0 = (K0 + KSTEP - 1) / KSTEP;
  const int nk1 = (K1 + KSTEP - 1) / KSTEP;
  const int nk = nk0 + nk1;

  // Residual prefetch (plain 256 x 256 tiles with a residual).  The loads a
  // loader issues for the steps nk and nk + 1 past the end of the K loop land
  // in four 32 KB slots that nothing reads any more (A slots nk % 3 and
  // (nk + 1) % 3, B slots nk % 2 and (nk + 1) % 2); instead of zeros they
  // bring the tile's 256 x 256 bf16 residual straight into the epilogue's
  // staging layout, so its latency overlaps the last two K steps.  Part g of
  // the residual (tile rows 64g .. 64g + 63, i.e. wave row g) goes to step
  // nk + g of A for g < 2 and to step nk + g - 2 of B; each part is two 16 KB
  // wave regions (wave columns 0 and 1) of 64 rows x 256 bytes whose 16-byte
  // chunks are XOR-swizzled by the row's low 4 bits.  The same number of
  // loads is issued as for a K step, so the loaders' vmcnt waits are unchanged.
  constexpr bool RES_PF = !SWIGLU && WM == 2 && WN == 4 && A_STAGE == 32768 &&
                          B_STAGE == 32768 && A_PER == 8 && B_PER == 8;
  const bool res_pf = RES_PF && p.res != nullptr;
  const __amdgpu_buffer_rsrc_t rR =
      res_pf ? make_rsrc(p.res + m0 * p.ldr, rows_valid * p.ldr * 2) : rA0;
  auto issue_res = [&](int g, int slot_bytes) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = 4 * i + wl;                      // 1 KB piece of the 32 KB part
      const int hh = q >> 4;                          // wave column of the region
      const int r = ((q & 15) << 2) + (lane >> 4);    // row within the region
      const int lc = (lane & 15) ^ (r & 15);          // logical chunk of physical lane & 15
      const int64_t c = (int64_t)tn * 256 + 128 * hh + 8 * lc;
      const uint32_t off =
          c < N ? (uint32_t)((((int64_t)(64 * g + r)) * p.ldr + c) * 2) : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rR, (lds_ptr_t)(lds + slot_bytes + q * 1024), 16, off, 0, 0, 0);
    }
  };

  // This wave's LDS-DMA loads of its operand for K-step kt into slot `slot`.
  // Branch-free but for the wave-uniform check of a partial last round:
  // chunks past the segment's K (a partial last step) and every chunk of a
  // step past the end (kt >= nk) take an out-of-range offset and land as
  // zeros without touching memory.
  auto issue_a = [&](int kt, int slot) {
    const bool seg1 = kt >= nk0;
    const int kbase = (seg1 ? kt - nk0 : kt) * KSTEP;
    const int kseg = seg1 ? K1 : K0;
    const int kleft = kt < nk ? kseg - kbase : 0;
    const uint32_t climit = (uint32_t)(kleft >= KSTEP ? ROWB : kleft * ESZ);
    const bool in_k = cx < climit;
    const __amdgpu_buffer_rsrc_t r = seg1 ? rA1 : rA0;
    const uint32_t base = (seg1 ? a_lane1 : a_lane0) + (uint32_t)(kbase * ESZ);
    const uint32_t stp = seg1 ? a_i1 : a_i0;
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      const int q = 4 * i + wl;
      if (A_TOT % 4 != 0 && q >= A_TOT) continue;
      const uint32_t off = in_k ? base + i * stp : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (lds_ptr_t)(lds + slot * A_STAGE + q * 1024), 16, off, 0, 0, 0);
    }
  };
  auto issue_b = [&](int kt, int slot) {
    const bool seg1 = kt >= nk0;
    const int kbase = (seg1 ? kt - nk0 : kt) * KSTEP;
    const int kseg = seg1 ? K1 : K0;
    const int kleft = kt < nk ? kseg - kbase : 0;
    const uint32_t climit = (uint32_t)(kleft >= KSTEP ? ROWB : kleft * ESZ);
    const bool in_k = cx < climit;
    const __amdgpu_buffer_rsrc_t r = seg1 ? rB1 : rB0;
    const uint32_t base = (seg1 ? b_lane1 : b_lane0) + (uint32_t)(kbase * ESZ);
#pragma unroll
    for (int i = 0; i < B_PER; ++i) {
      const int q = 4 * i + wl;
      if (B_TOT % 4 != 0 && q >= B_TOT) continue;
      const uint32_t piece = seg1 ? b_piece(i, p.ldb1) : b_piece(i, p.ldb0);
      const uint32_t off = in_k ? base + piece : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (lds_ptr_t)(lds + B_BASE + slot * B_STAGE + q * 1024), 16, off, 0, 0, 0);
    }
  };

  // the loads of steps that may lie past the end (the prologue and the last two
  // iterations): the residual parts instead of zeros when it is prefetched
  auto issue_a_tail = [&](int kt, int slot) {
    if (RES_PF && res_pf && kt >= nk) issue_res(kt - nk, slot * A_STAGE);
    else issue_a(kt, slot);
  };
  auto issue_b_tail = [&](int kt, int slot) {
    if (RES_PF && res_pf && kt >= nk) issue_res(2 + kt - nk, B_BASE + slot * B_STAGE);
    else issue_b(kt, slot);
  };

  // ---- LDS -> MFMA fragments -----------------------------------------------------
  // v_mfma_f32_16x16x32_bf16: a lane holds 8 consecutive k of one row of each
  // operand, row l%16 and k-chunk l/16 of the 32-k block.  Fragment (16 rows x
  // 32 k) of block row base rb (a multiple of 16) in k-block kk: lane l reads
  // row rb + l%16, logical chunk 4·kk + l/16.  For such rows the swizzle key
  // ((l%16) >> 1) & 7 does not depend on rb, so one lane offset per k-block
  // serves every block.  (16x16x32 moves half the accumulator bytes per
  // multiply-add of 32x32x16 through the register file; with random operands
  // that lowers power enough to run the MFMAs at a measurably higher clock.)
  constexpr int RB = WM * 2;               // 16-row blocks per wave (tokens)
  constexpr int CB = WN * 2;               // 16-column blocks per wave (outputs)
  const int key_lane = ((lane & 15) >> 1) & (CPR - 1);
  // bf16: 8 consecutive k per lane; MX (probed on gfx950): 32 k per lane, bytes
  // 0..15 = k 16·(l/16) + 0..15 and bytes 16..31 = k 64 + 16·(l/16) + 0..15 of
  // the 128-k block, i.e. logical chunks l/16 and 4 + l/16 of the row.
  constexpr int NFL = MX ? 2 : KS;
  uint32_t frag_lane[NFL];
#pragma unroll
  for (int f = 0; f < NFL; ++f) {
    const int chunk = MX ? 4 * f + (lane >> 4) : 4 * f + (lane >> 4);
    frag_lane[f] = (uint32_t)((lane & 15) * ROWB + ((chunk ^ key_lane) * 16));
  }
  const uint32_t a_wave = (uint32_t)(wm * WM * 32 * ROWB);
  const uint32_t b_wave = (uint32_t)(B_BASE + wn * WN * 32 * ROWB);
  // every fragment of one K step (bf16: KS x (RB + CB) x 16 bytes per lane;
  // MX: (RB + CB) x 32 bytes per lane)
  bf16x8 fa[MX ? 1 : KS][MX ? 1 : RB], fb[MX ? 1 : KS][MX ? 1 : CB];
  i32x8 xa[MX ? RB : 1], xb[MX ? CB : 1];
  // MX block scales.  The scale array holds, for each 128-k step t and 64-row
  // group g, one dword per lane l = 16·b + r whose byte i is the E8M0 scale of
  // row 64g + 16i + r over 32-k block b of the step: the MFMA's byte select
  // then picks the scale of 16-row block i, so a wave keeps one dword per
  // four 16-row blocks.  A wave's A rows start on a 64-row boundary; its B
  // rows may start 16, 32 or 48 rows into a group (96-row waves), in which
  // case one dword more is loaded and consecutive dwords are re-aligned with
  // a funnel shift before the MFMAs.
  constexpr int NGA = (RB + 3) / 4;
  constexpr int NGB = (CB + 3) / 4;
  constexpr bool B_ALIGNED = SWIGLU || (TN % 64 == 0 && (WN * 32) % 64 == 0);
  constexpr int NLB = B_ALIGNED ? NGB : NGB + 1;
  static_assert(!MX || (WM * 32) % 64 == 0, "MX: a wave's A rows span whole 64-row groups");
  static_assert(!MX || !SWIGLU || (WN * 16) % 64 == 0, "MX: SwiGLU halves span whole groups");
  uint32_t sca[MX ? NGA : 1], scb[MX ? NLB : 1];
  auto read_step = [&](int sa, int sb) {
    if constexpr (MX) {
      const uint32_t ao = a_wave + sa * A_STAGE;
      const uint32_t bo = b_wave + sb * B_STAGE;
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const u32x4 lo = *(const u32x4*)(lds + ao + frag_lane[0] + i * 16 * ROWB);
        const u32x4 hi = *(const u32x4*)(lds + ao + frag_lane[1] + i * 16 * ROWB);
        xa[i] = (i32x8){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                        (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int j = 0; j < CB; ++j) {
        const u32x4 lo = *(const u32x4*)(lds + bo + frag_lane[0] + j * 16 * ROWB);
        const u32x4 hi = *(const u32x4*)(lds + bo + frag_lane[1] + j * 16 * ROWB);
        xb[j] = (i32x8){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                        (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const uint32_t ao = frag_lane[kk] + a_wave + sa * A_STAGE;
        const uint32_t bo = frag_lane[kk] + b_wave + sb * B_STAGE;
#pragma unroll
        for (int i = 0; i < RB; ++i) fa[kk][i] = *(const bf16x8*)(lds + ao + i * 16 * ROWB);
#pragma unroll
        for (int j = 0; j < CB; ++j) fb[kk][j] = *(const bf16x8*)(lds + bo + j * 16 * ROWB);
      }
    }
  };
  // MX scales of step kt (buffer loads: groups past the padded scale arrays
  // read as zeros)
  const __amdgpu_buffer_rsrc_t rsA0 =
      MX ? make_rsrc(p.sA0, (K0 / 128) * p.sMp * 4) : rA0;
  const __amdgpu_buffer_rsrc_t rsB0 =
      MX ? make_rsrc(p.sB0, (K0 / 128) * p.sNp * 4) : rB0;
  const int64_t sMp1 = p.sMp1 ? p.sMp1 : p.sMp;
  const __amdgpu_buffer_rsrc_t rsA1 =
      (MX && has1) ? make_rsrc(p.sA1, (K1 / 128) * sMp1 * 4) : rsA0;
  const __amdgpu_buffer_rsrc_t rsB1 =
      (MX && has1) ? make_rsrc(p.sB1, (K1 / 128) * p.sNp * 4) : rsB0;
  const int64_t ga = (m0 + wm * WM * 32) >> 6;          // A: first 64-row group
  // B: first group of each dword (SwiGLU: gate half, then up half) and the
  // funnel shift in bits for waves that start inside a group
  const int64_t nb0 = SWIGLU ? (int64_t)tn * TN + wn * (WN * 16)
                             : (int64_t)tn * TN + wn * WN * 32;
  const int64_t gb = nb0 >> 6;
  const int bsh = (int)(nb0 & 63) >> 1;
  constexpr int NSC = MX ? NGA + NLB : 0;   // scale loads per step
  auto load_scales = [&](int kt) {
    if constexpr (MX) {
      const bool seg1 = kt >= nk0;
      const int64_t t = seg1 ? kt - nk0 : kt;
      const __amdgpu_buffer_rsrc_t ra = seg1 ? rsA1 : rsA0;
      const __amdgpu_buffer_rsrc_t rb = seg1 ? rsB1 : rsB0;
      // (A0's rows start at group sa_g0 of its scale array; A1 is chunk-local)
      const int64_t ta = t * ((seg1 ? sMp1 : p.sMp) >> 6) + (seg1 ? 0 : p.sa_g0);
      const int64_t tb = t * (p.sNp >> 6);
#pragma unroll
      for (int q = 0; q < NGA; ++q)
        sca[q] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(
            ra, (uint32_t)(((ta + ga + q) * 64 + lane) * 4), 0, 0);
#pragma unroll
      for (int q = 0; q < NLB; ++q) {
        const int64_t g = SWIGLU ? q * (F >> 6) + gb : gb + q;
        scb[q] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(
            rb, (uint32_t)(((tb + g) * 64 + lane) * 4), 0, 0);
      }
    }
  };

  f32x4 acc[RB][CB];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < CB; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[i][j][v] = 0.0f;

  auto compute_step = [&]() {
    if constexpr (MX) {
      uint32_t sbv[NGB];
#pragma unroll
      for (int q = 0; q < NGB; ++q)
        sbv[q] = B_ALIGNED ? scb[q] : __builtin_amdgcn_alignbit(scb[q + 1], scb[q], bsh);
      // the byte selects are immediates: unroll over compile-time indexes
      static_for<RB>([&](auto I) {
        static_for<CB>([&](auto J) {
          constexpr int i = decltype(I)::value, j = decltype(J)::value;
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              xb[j], xa[i], acc[i][j], 0, 0, j & 3, (int)sbv[j >> 2], i & 3, (int)sca[i >> 2]);
        });
      });
    } else {
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
#pragma unroll
        for (int i = 0; i < RB; ++i)
#pragma unroll
          for (int j = 0; j < CB; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[kk][j], fa[kk][i], acc[i][j],
                                                                0, 0, 0);
    }
  };

  // ---- main loop: ping-pong ----------------------------------------------------------
  // A K step is two phases separated by barriers.  In phase 0 of step kt,
  // group 0 runs its RB·CB·KS MFMAs of step kt back to back from fragments
  // already in registers, while group 1 reads every fragment of step kt from
  // LDS and issues the A loads of step kt+2; in phase 1 the roles swap: group
  // 1 computes step kt while group 0 issues the B loads of step kt+2 and reads
  // the fragments of step kt+1.  Each SIMD holds one wave of each group, so
  // its MFMA pipe always has one wave streaming MFMAs while the other does
  // the memory work.
  //   A of step kt sits in slot kt % 3 (read in phase 1 of kt-1 and phase 0
  //   of kt); A(kt+2) refills slot (kt+2) % 3, free since phase 0 of kt-1,
  //   and has until phase 1 of kt+1.  B of step kt sits in slot kt % 2; B(kt+2)
  //   refills it in phase 1 of kt and has until phase 1 of kt+1.  Each loader
  //   waits for its own loads before the barrier that precedes their first
  //   reader (vector-memory loads retire in order).
  constexpr int A_WAIT = A_TOT / 4;        // A loads a group-1 wave issues per step
  static_assert(A_TOT % 4 == 0, "every loader issues the same number of A loads");
  // The last two iterations issue the loads of steps nk and nk + 1; they run
  // as a separate copy of the loop body so that the steady-state loop keeps
  // no residual test.
  if (wgrp == 1) {
    issue_a_tail(0, 0);
    issue_a_tail(1, 1);
    wait_vm_lgkm0<A_WAIT>();               // A(0) has landed
  } else {
    issue_b_tail(0, 0);
    issue_b_tail(1, 1);
    wait_vm_lgkm0<B_PER>();                // B(0) has landed (over-waits if partial)
  }
  __builtin_amdgcn_s_barrier();
  int sa = 0;                              // A slot of step kt (kt % 3)
  const int nk_main = nk - 2;              // iterations whose loads are all in range
  // MX scales: each group loads the next step's right after its last MFMA of
  // this one (the registers are free then), so the loads have the barrier and
  // the whole memory phase to land before that phase's final wait needs them.
  if (wgrp == 0) {
    load_scales(0);
    read_step(0, 0);
    if constexpr (MX) wait_vm_lgkm0<0>();    // the scales were issued after B(1)
    else wait_vm_lgkm0<B_PER>();
    __builtin_amdgcn_s_barrier();
    auto body0 = [&](int kt, auto tail) {
      const int sb = kt & 1;
      const int sa_next = sa == NSLOT_A - 1 ? 0 : sa + 1;
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(1);
      compute_step();
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
      // MX reads unconditionally (after the last step: stale LDS and scales that
      // are never used), which keeps the 8-register fragments out of phis
      load_scales(kt + 1);                 // (MX) retire before the B loads below
      wait_vm_lgkm0<NSC>();                // B(kt+1) has landed
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (decltype(tail)::value) issue_b_tail(kt + 2, sb);
      else issue_b(kt + 2, sb);
      if (MX || kt + 1 < nk) read_step(sa_next, sb ^ 1);
      wait_vm_lgkm0<B_PER>();              // fragments (and scales) in registers
      __builtin_amdgcn_s_barrier();
      sa = sa_next;
    };
    int kt = 0;
    for (; kt < nk_main; ++kt) body0(kt, std::false_type{});
    for (; kt < nk; ++kt) body0(kt, std::true_type{});
  } else {
    load_scales(0);
    __builtin_amdgcn_s_barrier();
    auto body1 = [&](int kt, auto tail) {
      const int sb = kt & 1;
      const int sa_next = sa == NSLOT_A - 1 ? 0 : sa + 1;
      const int sa_load = sa_next == NSLOT_A - 1 ? 0 : sa_next + 1;   // (kt + 2) % 3
      __builtin_amdgcn_sched_barrier(0);
      read_step(sa, sb);
      if constexpr (decltype(tail)::value) issue_a_tail(kt + 2, sa_load);
      else issue_a(kt + 2, sa_load);
      wait_vm_lgkm0<A_WAIT>();             // A(kt+1) has landed; fragments in registers
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(1);
      compute_step();
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
      load_scales(kt + 1);                 // (MX) retire before the A loads of the next step
      __builtin_amdgcn_s_barrier();
      sa = sa_next;
    };
    int kt = 0;
    for (; kt < nk_main; ++kt) body1(kt, std::false_type{});
    for (; kt < nk; ++kt) body1(kt, std::true_type{});
  }
  // all LDS-DMA writes (including the out-of-range loads past the end) have
  // landed and every wave is done with the rings before LDS is reused below
  wait_vm_lgkm0<0>();
  __builtin_amdgcn_s_barrier();

  // ---- epilogue ---------------------------------------------------------------
  // Block (i, j) holds the transposed 16x16 output: lane l owns token
  // 16·i + l%16 of the wave and the four consecutive output columns
  // 16·j + 4·(l/16) + 0..3 (accumulator elements 0..3).  Each
  // wave stages its (token x column) bf16 tile in its own LDS region, adding
  // the residual (loaded into the same place first) before the single
  // rounding, then writes whole row segments with 16-byte stores.  Staged rows
  // keep their 16-byte chunks XOR-swizzled (power-of-two chunk counts) or are
  // padded by 16 bytes, so the 8-byte writes of 16 consecutive tokens hit
  // distinct banks.
  constexpr int OC = SWIGLU ? WN * 16 : WN * 32;    // output columns per wave
  constexpr int ORB = OC * 2;                       // bytes of one staged row
  constexpr int OCH = ORB / 16;                     // 16-byte chunks per row
  constexpr bool POW2 = (OCH & (OCH - 1)) == 0;
  constexpr int PITCH = POW2 ? ORB : ORB + 16;
  constexpr int RP = POW2 ? (256 / ORB > 0 ? 256 / ORB : 1) : 1;   // staged rows per 256 B
  constexpr int OROWS = WM * 32;                    // tokens per wave
  static_assert(kWaves * OROWS * PITCH <= LDS_BYTES, "epilogue staging must fit in LDS");
  // (with the residual prefetch, wave row g's regions are the slots that
  // received residual part g)
  int ow_bytes = wave * OROWS * PITCH;
  if constexpr (RES_PF) {
    const int g = wm, n3 = nk % 3;
    const int a_slot = g == 0 ? n3 : (n3 == 2 ? 0 : n3 + 1);
    const int b_slot = (nk + (g - 2)) & 1;
    ow_bytes = (g < 2 ? a_slot * A_STAGE : B_BASE + b_slot * B_STAGE) + wn * (OROWS * PITCH);
  }
  char* ow = lds + ow_bytes;
  auto pchunk = [&](int row, int c) -> int {      // physical chunk of logical chunk c
    if constexpr (POW2) return c ^ ((row / RP) & (OCH - 1));
    else return c;
  };
  const int64_t col0 = (int64_t)tn * TN + wn * OC;     // first output column of the wave
  const int64_t tok0 = (int64_t)wm * OROWS;            // first tile row of the wave
  const float alpha = p.alpha;

  if (!RES_PF && p.res) {
    // residual tile -> LDS (same layout), one 16-byte chunk per lane
    for (int idx = lane; idx < OROWS * OCH; idx += 64) {
      const int row = idx / OCH, pc = idx % OCH;
      const int lc = pchunk(row, pc);               // pchunk is an involution
      const int64_t c = col0 + lc * 8;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (tok0 + row < rows_valid && c < Nout)
        v = __builtin_nontemporal_load((const u32x4*)(p.res + (m0 + tok0 + row) * p.ldr + c));
      *(u32x4*)(ow + row * PITCH + pc * 16) = v;
    }
    __builtin_amdgcn_s_waitcnt(0);
  }

  const int tok = lane & 15;
  const int c4 = 4 * (lane >> 4);
  auto slot = [&](int row, int oc) -> char* {
    return ow + row * PITCH + pchunk(row, oc >> 3) * 16 + (oc & 7) * 2;
  };
  auto bias4 = [&](int64_t n, bool ok) -> f32x4 {
    f32x4 b = {0.0f, 0.0f, 0.0f, 0.0f};
    if (p.bias && ok) {
#pragma unroll
      for (int k = 0; k < 4; ++k) b[k] = p.bias[n + k];
    }
    return b;
  };
  if constexpr (SWIGLU) {
    // gate columns are the wave's first CB/2 blocks, the matching up columns
    // the last CB/2
    constexpr int HALFB = CB / 2;
#pragma unroll
    for (int j = 0; j < HALFB; ++j) {
      const int oc = j * 16 + c4;
      const int64_t n = col0 + oc;
      const f32x4 bg = bias4(n, n < F);
      const f32x4 bu = bias4(F + n, n < F);
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        float h[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float gt = acc[i][j][k] * alpha + bg[k];
          const float up = acc[i][j + HALFB][k] * alpha + bu[k];
          // silu(g)·u with a hardware reciprocal (1 ulp) instead of an IEEE
          // divide (ten VALU ops of 4 cycles each per wave64): the product
          // is rounded to bf16 right after, and g -> -inf still gives -0
          h[k] = gt * __builtin_amdgcn_rcpf(1.0f + __expf(-gt)) * up;
        }
        u32x2 pk;
        pk.x = f32_to_bf16(h[0]) | (f32_to_bf16(h[1]) << 16);
        pk.y = f32_to_bf16(h[2]) | (f32_to_bf16(h[3]) << 16);
        *(u32x2*)slot(i * 16 + tok, oc) = pk;
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      const int oc = j * 16 + c4;
      const f32x4 bn = bias4(col0 + oc, col0 + oc < Nout);
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        char* s = slot(i * 16 + tok, oc);
        float y[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) y[k] = acc[i][j][k] * alpha + bn[k];
        if (p.res) {
          const u32x2 rv = *(const u32x2*)s;
          y[0] += __uint_as_float(rv.x << 16);
          y[1] += __uint_as_float(rv.x & 0xffff0000u);
          y[2] += __uint_as_float(rv.y << 16);
          y[3] += __uint_as_float(rv.y & 0xffff0000u);
        }
        u32x2 pk;
        pk.x = f32_to_bf16(y[0]) | (f32_to_bf16(y[1]) << 16);
        pk.y = f32_to_bf16(y[2]) | (f32_to_bf16(y[3]) << 16);
        *(u32x2*)s = pk;
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);   // the wave's staged tile is complete (its own region)
  if constexpr (QOUT && SWIGLU) {
    // SwiGLU -> MXFP8 in one pass: the wave's staged 64 x 64 bf16 tile of H is
    // two 32-column blocks per row.  Lane l quantizes block l >> 5 of rows
    // 16·i + l%16, i = 2·((l >> 4) & 1) + k for k = 0, 1, stores its 32 E4M3
    // bytes, and drops each scale byte into LDS at its place in the scale
    // layout (byte i of word 16·block + l%16).  The wave's 128 scale bytes are
    // words 32·wn .. 32·wn + 31 of one (step, 64-row group) region and leave
    // with one coalesced store.  Rows past M store no elements and scale 127.
    static_assert(SWIGLU && OC == 64 && OROWS == 64, "one 64-row group, two blocks per wave");
    uint8_t* sl = (uint8_t*)(lds + kWaves * OROWS * PITCH + wave * 128);
    static_assert(kWaves * (OROWS * PITCH + 128) <= LDS_BYTES, "scale staging must fit in LDS");
    const int qb = lane >> 5, qr = lane & 15, qi = (lane >> 4) & 1;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int i = 2 * qi + k;
      const int row = 16 * i + qr;
      uint32_t w[16];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const u32x4 v = *(const u32x4*)(ow + row * PITCH + pchunk(row, 4 * qb + c) * 16);
        w[4 * c] = v.x; w[4 * c + 1] = v.y; w[4 * c + 2] = v.z; w[4 * c + 3] = v.w;
      }
      uint32_t q[8];
      const uint32_t sbyte = mx_block_bf16(w, q);
      const bool valid = tok0 + row < rows_valid;
      if (valid) {
        u32x4* dst = (u32x4*)(p.Yq + (m0 + tok0 + row) * p.ldyq + col0 + 32 * qb);
        __builtin_nontemporal_store((u32x4){q[0], q[1], q[2], q[3]}, dst);
        __builtin_nontemporal_store((u32x4){q[4], q[5], q[6], q[7]}, dst + 1);
      }
      sl[(16 * qb + qr) * 4 + i] = (uint8_t)(valid ? sbyte : 127u);
    }
    __builtin_amdgcn_s_waitcnt(0);
    if (lane < 32) {
      const uint32_t word = *(const uint32_t*)(sl + lane * 4);
      const int64_t g = ((m0 + tok0) >> 6) + p.sy_g0;     // the wave's 64-row group
      uint32_t* dst = (uint32_t*)p.Ys + ((int64_t)tn * (p.sYp >> 6) + g) * 64 + 32 * wn + lane;
      __builtin_nontemporal_store(word, dst);
    }
    return;
  }
  if (!QOUT || p.Y) {
    for (int idx = lane; idx < OROWS * OCH; idx += 64) {
      const int row = idx / OCH, pc = idx % OCH;
      const int64_t c = col0 + pchunk(row, pc) * 8;
      if (tok0 + row < rows_valid && c < Nout) {
        const u32x4 v = *(const u32x4*)(ow + row * PITCH + pc * 16);
        __builtin_nontemporal_store(v, (u32x4*)(p.Y + (m0 + tok0 + row) * p.ldy + c));
      }
    }
  }
  if constexpr (QOUT) {
    // The staged bf16 tile -> MXFP8 of output columns [q0, q1), i.e. column
    // c - q0 of a matrix of qk = q1 - q0 columns padded to qkp (a multiple of
    // 128) with zero elements and scale 127.  Lane l quantizes row l of the
    // wave for each of its NBLK 32-column blocks (q0 and q1 are multiples of
    // 32, so a block is wholly inside, past q1 (padding), or outside).  The
    // 32 code bytes of block b overwrite logical chunks 2b, 2b + 1 of the
    // lane's own staged row, which hold bf16 of blocks it has already read;
    // the codes then leave as whole row segments, 16 bytes per lane over
    // consecutive addresses.  (Each lane storing its own row's 32 bytes
    // instead touched 64 lines per store and cost about 14 us per tile.)
    // The scale byte goes into LDS at its place in the scale layout: byte
    // (row >> 4) of dword 16·b + row % 16 of the (K step, 64-row group)
    // region, b = the block within its K step.  Rows past M store no elements
    // and scale 127.  The scale staging sits past the tiles' staging regions
    // (with the residual prefetch: in A slot (nk + 2) % 3, which neither the
    // residual nor the last K step's fragments occupy any more).
    constexpr int NBLK = OC / 32;
    static_assert(OC % 32 == 0 && OROWS == 64, "whole blocks, one 64-row group per wave");
    constexpr int SCB = NBLK * 64;                     // scale bytes per wave
    static_assert(RES_PF ? kWaves * SCB <= A_STAGE
                         : kWaves * (OROWS * PITCH + SCB) <= LDS_BYTES,
                  "scale staging must fit in LDS");
    const int sbase = RES_PF ? ((nk + 2) % 3) * A_STAGE : kWaves * OROWS * PITCH;
    uint8_t* sl = (uint8_t*)(lds + sbase + wave * SCB);
    const int64_t qk = p.q1 - p.q0;
    const int64_t qkp = (qk + 127) / 128 * 128;
    const int64_t g = ((m0 + tok0) >> 6) + p.sy_g0;    // the wave's 64-row group
    const int64_t sgrp = p.sYp >> 6;                   // 64-row groups per K step
    const int row = lane;
    const bool valid = tok0 + row < rows_valid;
    uint8_t* yq_row = p.Yq + (m0 + tok0 + row) * p.ldyq;
    int b_lo = NBLK, b_hi = 0;                         // the wave's blocks in [0, qkp)
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk) {
      const int64_t qc = col0 + 32 * blk - p.q0;       // wave-uniform
      if (qc < 0 || qc >= qkp) continue;
      uint32_t q[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
      uint32_t sbyte = 127u;
      if (qc < qk) {
        uint32_t w[16];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const u32x4 v = *(const u32x4*)(ow + row * PITCH + pchunk(row, 4 * blk + c) * 16);
          w[4 * c] = v.x; w[4 * c + 1] = v.y; w[4 * c + 2] = v.z; w[4 * c + 3] = v.w;
        }
        sbyte = mx_block_bf16(w, q);
      }
      {
        char* rowp = ow + row * PITCH;
        *(u32x4*)(rowp + pchunk(row, 2 * blk) * 16) = (u32x4){q[0], q[1], q[2], q[3]};
        *(u32x4*)(rowp + pchunk(row, 2 * blk + 1) * 16) = (u32x4){q[4], q[5], q[6], q[7]};
      }
      b_lo = blk < b_lo ? blk : b_lo;
      b_hi = blk + 1;
      sl[(16 * blk + (row & 15)) * 4 + (row >> 4)] = (uint8_t)(valid ? sbyte : 127u);
    }
    __builtin_amdgcn_s_waitcnt(0);
    for (int idx = lane; idx < OROWS * 2 * NBLK; idx += 64) {
      const int r = idx / (2 * NBLK), ch = idx % (2 * NBLK);
      const int bb = ch >> 1;
      if (bb >= b_lo && bb < b_hi && tok0 + r < rows_valid) {
        const u32x4 v = *(const u32x4*)(ow + r * PITCH + pchunk(r, ch) * 16);
        __builtin_nontemporal_store(
            v, (u32x4*)(p.Yq + (m0 + tok0 + r) * p.ldyq + (col0 - p.q0) + ch * 16));
      }
    }
    if (lane < NBLK * 16) {
      const int blk = lane >> 4, r = lane & 15;
      const int64_t qc = col0 + 32 * blk - p.q0;
      if (qc >= 0 && qc < qkp) {
        const int64_t B = qc >> 5;
        const uint32_t word = *(const uint32_t*)(sl + lane * 4);
        __builtin_nontemporal_store(
            word, (uint32_t*)p.Ys + ((B >> 2) * sgrp + g) * 64 + 16 * (B & 3) + r);
      }
    }
    // padding blocks that no tile covers (at most three, past the last tile
    // column): the last wave column of the last tile column writes them
    const int64_t covered = (int64_t)tiles_n * TN;     // output columns the tiles span
    if (tn == tiles_n - 1 && wn == kWaveCols - 1 && p.q0 + qkp > covered) {
      for (int64_t qc = (covered - p.q0 + 31) / 32 * 32; qc < qkp; qc += 32) {
        if (qc < 0) continue;
        if (valid) {
          u32x4* dst = (u32x4*)(yq_row + qc);
          __builtin_nontemporal_store((u32x4){0u, 0u, 0u, 0u}, dst);
          __builtin_nontemporal_store((u32x4){0u, 0u, 0u, 0u}, dst + 1);
        }
        if (lane < 16) {
          const int64_t B = qc >> 5;
          __builtin_nontemporal_store(
              0x7f7f7f7fu, (uint32_t*)p.Ys + ((B >> 2) * sgrp + g) * 64 + 16 * (B & 3) + lane);
        }
      }
    }
  }
}

template <int WM, int WN, bool SWIGLU, bool MX, bool QOUT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(1024))) char lds[kLdsBytes];
  gemm_tile<WM, WN, SWIGLU, MX, QOUT>(p, blockIdx.x, lds);
}

// Two independent GEMMs in one launch: workgroups [0, nb) are the tiles of
// phase B (pb: 256 x 256 tiles, plain or SwiGLU epilogue) of one chunk of rows,
// workgroups [nb, nb + na) the phase-A tiles (pa: 256 x 192) of the next
// chunk.  Workgroups start in id order, so the shorter phase-A tiles fill the
// CUs that phase B's last wave leaves idle, instead of a launch of their own
// ramping up and draining.  The two GEMMs share no buffer: phase B reads the T
// that the previous launch wrote, phase A writes the other half of the
// workspace.
template <bool SWIGLU>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_pair_kernel(GemmParams pb, GemmParams pa, int nb) {
  __shared__ __attribute__((aligned(1024))) char lds[kLdsBytes];
  const int wg = blockIdx.x;
  if (wg < nb) gemm_tile<2, 4, SWIGLU, false, false>(pb, wg, lds);
  else gemm_tile<2, 3, false, false, false>(pa, wg - nb, lds);
}

// The MXFP8 counterpart: phase B tiles (plain, SwiGLU, with or without the
// quantized output) then the phase-A tiles of the next chunk, T leaving as MXFP8.
template <bool SWIGLU, bool QOUT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_pair_mx_kernel(GemmParams pb, GemmParams pa, int nb) {
  __shared__ __attribute__((aligned(1024))) char lds[kLdsBytes];
  const int wg = blockIdx.x;
  if (wg < nb) gemm_tile<2, 4, SWIGLU, true, QOUT>(pb, wg, lds);
  else gemm_tile<2, 3, false, true, true>(pa, wg - nb, lds);
}

template <int WM, int WN, bool SWIGLU>
int64_t tile_count(const GemmParams& p) {
  constexpr int BM = kWaveRows * WM * 32;
  constexpr int TN = (SWIGLU ? 16 : 32) * kWaveCols * WN;
  const int64_t nout = SWIGLU ? p.N / 2 : p.N;
  return ((p.M + BM - 1) / BM) * ((nout + TN - 1) / TN);
}

template <int WM, int WN, bool SWIGLU, bool MX, bool QOUT = false>
hipError_t launch(const GemmParams& p, hipStream_t s) {
  constexpr int BM = kWaveRows * WM * 32;
  constexpr int TN = (SWIGLU ? 16 : 32) * kWaveCols * WN;
  const int64_t nout = SWIGLU ? p.N / 2 : p.N;
  const int64_t tiles = ((p.M + BM - 1) / BM) * ((nout + TN - 1) / TN);
  if (tiles <= 0) return hipSuccess;
  if (tiles > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_kernel<WM, WN, SWIGLU, MX, QOUT>), dim3((unsigned)tiles),
                     dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(GemmKind kind, const GemmParams& p, hipStream_t s) {
  switch (kind) {
    case GEMM_DOWN: return launch<2, 3, false, false>(p, s);
    case GEMM_UP: return launch<2, 4, false, false>(p, s);
    case GEMM_UP_SWIGLU: return launch<2, 4, true, false>(p, s);
    case GEMM_MX_DOWN: return launch<2, 3, false, true>(p, s);
    case GEMM_MX_UP: return launch<2, 4, false, true>(p, s);
    case GEMM_MX_UP_SWIGLU: return launch<2, 4, true, true>(p, s);
    case GEMM_MX_UP_SWIGLU_MX: return launch<2, 4, true, true, true>(p, s);
    case GEMM_MX_DOWN_Q: return launch<2, 3, false, true, true>(p, s);
    case GEMM_MX_UP_Q: return launch<2, 4, false, true, true>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_pair(bool swiglu, const GemmParams& pb, const GemmParams& pa,
                            hipStream_t s) {
  const int64_t nb = swiglu ? tile_count<2, 4, true>(pb) : tile_count<2, 4, false>(pb);
  const int64_t na = tile_count<2, 3, false>(pa);
  if (nb <= 0 && na <= 0) return hipSuccess;
  if (nb + na > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(nb + na));
  if (swiglu) hipLaunchKernelGGL(gemm_pair_kernel<true>, grid, dim3(kThreads), 0, s, pb, pa, (int)nb);
  else hipLaunchKernelGGL(gemm_pair_kernel<false>, grid, dim3(kThreads), 0, s, pb, pa, (int)nb);
  return hipGetLastError();
}

hipError_t launch_gemm_pair_mx(bool swiglu, bool qout, const GemmParams& pb,
                               const GemmParams& pa, hipStream_t s) {
  const int64_t nb = swiglu ? tile_count<2, 4, true>(pb) : tile_count<2, 4, false>(pb);
  const int64_t na = tile_count<2, 3, false>(pa);
  if (nb <= 0 && na <= 0) return hipSuccess;
  if (nb + na > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(nb + na)), block(kThreads);
  if (swiglu && qout) hipLaunchKernelGGL((gemm_pair_mx_kernel<true, true>), grid, block, 0, s, pb, pa, (int)nb);
  else if (swiglu) hipLaunchKernelGGL((gemm_pair_mx_kernel<true, false>), grid, block, 0, s, pb, pa, (int)nb);
  else if (qout) hipLaunchKernelGGL((gemm_pair_mx_kernel<false, true>), grid, block, 0, s, pb, pa, (int)nb);
  else hipLaunchKernelGGL((gemm_pair_mx_kernel<false, false>), grid, block, 0, s, pb, pa, (int)nb);
  return hipGetLastError();
}

}  // namespace fsd
