// Dense softmax attention of the refine path, O_h = softmax(Q_h·K_hᵀ·scale)·V_h
// per head, over the whole token sequence.
//
// The pages' baseline refine runs its attention densely in bf16 ("Open-H3-
// Regenerate-2K: High-Resolution Video Refinement with Few-Step Diffusion",
// agientry.com, section "Where the 3.9x speedup comes from", the dense-BF16
// baseline row); the operation itself is textbook scaled dot-product attention.
//
// Flash-style: one workgroup per (head, 256 queries), eight waves of 32 queries.
// Key blocks of 64 stream through a double-buffered LDS stage (K rows and the
// same keys of a pre-transposed Vᵀ) by LDS-DMA; per block each wave forms
// S = K·Qᵀ (16x16x32 bf16 MFMA, fp32), updates its running row maximum and sum
// in the exp2 domain, rescales its fp32 output and adds P·V with P rounded to
// bf16.  Lane l of a 16x16 block holds query l%16 and four consecutive keys (S)
// or head dims (O) 4·(l/16)..+3, so a query's row statistics reduce over the
// four lanes l%16 + 16c.  As the P·V operand a lane then holds keys 4c..4c+3 of
// two adjacent 16-key blocks; the transposed V stores each 32-key group in that
// order (4-key quarters of its two halves interleaved), so the matching V
// fragment is one 16-byte read.  The running maximum is kept until a block's
// maximum exceeds it by more than 2^8 (P stays <= 256, exact enough for bf16
// and fp32 sums), so the fp32 output is rescaled only in the rare blocks where
// some row of the wave needs it, and the exact row maximum (a reduction over
// four lanes) is formed only in those blocks.  The row sums of P come from the matrix pipe:
// a ninth 16-column output block is P times a block of ones, so the softmax
// denominator uses the same bf16 P as the numerator and costs no VALU adds.
#include <math.h>

#include <type_traits>

#include "fsd_internal.h"

namespace fsd {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kD = 128;                   // head dimension
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBQ = 32 * kWaves;          // queries per workgroup
constexpr int kBK = 64;                   // keys per block
constexpr int kKRow = kD * 2;             // K tile row: one key, 256 bytes
constexpr int kKTile = kBK * kKRow;       // 16 KB
constexpr int kVRow = kBK * 2;            // Vᵀ tile row: one head dim, 64 keys, 128 bytes
constexpr int kVTile = kD * kVRow;        // 16 KB
constexpr int kStage = kKTile + kVTile;   // one buffer of the double-buffered stage

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  // raw buffer: stride 0, num_records in bytes; offsets past it read as zero
  const uint32_t n = bytes <= 0 ? 0u : (bytes >= 0x7fffffffLL ? 0x7fffffffu : (uint32_t)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, 0x00020000);
}

struct AttnParams {
  const bf16_t* Q; const bf16_t* K; const bf16_t* Vt;
  bf16_t* O;
  int64_t ld, ldo;      // row strides of Q/K/V and O (elements)
  int64_t S, Sp;        // tokens; Vᵀ row length (S rounded up to kBK, zero padded)
  int H, nqb;           // heads; query blocks per head
  float scale_log2;     // scale · log2(e)
};

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attention_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(1024))) char lds[2 * kStage];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, c4 = lane >> 4;

  // workgroup -> (head, query block); ids go round-robin over the 8 XCDs, so
  // each XCD takes a contiguous run of the sequence and its concurrent
  // workgroups stream the same keys of one head through its L2
  const int total = p.H * p.nqb;
  const int wg = blockIdx.x, xcd = wg & 7, local = wg >> 3;
  const int per = total >> 3, rem = total & 7;
  const int L = xcd * per + (xcd < rem ? xcd : rem) + local;
  const int h = L / p.nqb, qb = L - h * p.nqb;
  const int64_t S = p.S;
  const int64_t q0 = (int64_t)qb * kBQ;
  const int64_t qrows = (S - q0) < kBQ ? (S - q0) : kBQ;

  // this wave's Q fragments for the whole loop: rows 32·wave + 16·qi + l%16,
  // head dims 32·kk + 8·(l/16) .. +7 (rows past S read as zeros)
  const __amdgpu_buffer_rsrc_t rQ =
      make_rsrc(p.Q + q0 * p.ld + (int64_t)h * kD, qrows * p.ld * 2 - (int64_t)h * kD * 2);
  bf16x8 qf[2][4];
#pragma unroll
  for (int qi = 0; qi < 2; ++qi)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int row = 32 * wave + 16 * qi + r16;
      const uint32_t off = (uint32_t)(((int64_t)row * p.ld + 32 * kk + 8 * c4) * 2);
      const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rQ, off, 0, 0));
      qf[qi][kk] = __builtin_bit_cast(bf16x8, v);
    }

  // LDS-DMA of key block j into buffer `buf`: the K tile is 64 rows of 256
  // bytes, 16-byte chunks XOR-swizzled by the row's low 4 bits; the Vᵀ tile is
  // 128 rows (head dims) of 64 keys, chunks swizzled by the row's low 3 bits.
  // Each wave issues two 1 KB loads of each tile.
  const __amdgpu_buffer_rsrc_t rV =
      make_rsrc(p.Vt + (int64_t)h * kD * p.Sp, (int64_t)kD * p.Sp * 2);
  uint32_t k_off[2], v_off[2];             // per-lane byte offsets within a block
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int i = 2 * wave + t;
    const int krow = 4 * i + c4;                                // key within the block
    k_off[t] = (uint32_t)(((int64_t)krow * p.ld + 8 * (r16 ^ (krow & 15))) * 2);
    const int vrow = 8 * i + (lane >> 3);                      // head dim
    v_off[t] = (uint32_t)(((int64_t)vrow * p.Sp + 8 * ((lane & 7) ^ (vrow & 7))) * 2);
  }
  auto issue_block = [&](int j, int buf) {
    const int64_t k0 = (int64_t)j * kBK;
    const int64_t krows = (S - k0) < kBK ? (S - k0) : kBK;
    const __amdgpu_buffer_rsrc_t rK =
        make_rsrc(p.K + k0 * p.ld + (int64_t)h * kD, krows * p.ld * 2 - (int64_t)h * kD * 2);
    char* st = lds + buf * kStage;
#pragma unroll
    for (int t = 0; t < 2; ++t)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rK, (lds_ptr_t)(st + (2 * wave + t) * 1024), 16,
                                               k_off[t], 0, 0, 0);
#pragma unroll
    for (int t = 0; t < 2; ++t)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rV, (lds_ptr_t)(st + kKTile + (2 * wave + t) * 1024),
                                               16, v_off[t] + (uint32_t)(k0 * 2), 0, 0, 0);
  };

  // o[qi][0..7]: the output's 128 head dims; o[qi][8]: every column holds the
  // running sum of P over the keys (P times a block of ones)
  f32x4 o[2][9];
#pragma unroll
  for (int qi = 0; qi < 2; ++qi)
#pragma unroll
    for (int dj = 0; dj < 9; ++dj) o[qi][dj] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
  float m_run[2] = {-INFINITY, -INFINITY};
  const bf16x8 ones = {(__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f,
                       (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f};

  const int nkb = (int)((S + kBK - 1) / kBK);
  issue_block(0, 0);
  // key block j in stage buffer BUF = j & 1 (a compile-time constant: the loop
  // below runs two blocks per trip, so every LDS address is a fixed per-lane
  // offset plus an immediate)
  auto block = [&](int j, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    // own loads of block j (and, once, the Q fragments) have landed; after the
    // barrier so have everyone's, and every wave is done with block j - 1
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    if (j + 1 < nkb) issue_block(j + 1, buf ^ 1);
    const char* kt = lds + buf * kStage;
    const char* vt = kt + kKTile;

    // S = K·Qᵀ for 64 keys x 32 queries
    f32x4 s[2][4];
#pragma unroll
    for (int qi = 0; qi < 2; ++qi)
#pragma unroll
      for (int kj = 0; kj < 4; ++kj) s[qi][kj] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int kj = 0; kj < 4; ++kj) {
        const int row = 16 * kj + r16;
        const int pc = (4 * kk + c4) ^ r16;                // row & 15 == l % 16
        const bf16x8 kf = *(const bf16x8*)(kt + row * kKRow + pc * 16);
#pragma unroll
        for (int qi = 0; qi < 2; ++qi)
          s[qi][kj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[qi][kk], s[qi][kj], 0, 0, 0);
      }
    // keys past S (last block only) take no weight
    if (j == nkb - 1) {
      const int kvalid = (int)(S - (int64_t)j * kBK);
#pragma unroll
      for (int kj = 0; kj < 4; ++kj)
#pragma unroll
        for (int t = 0; t < 4; ++t)
          if (16 * kj + 4 * c4 + t >= kvalid) { s[0][kj][t] = -INFINITY; s[1][kj][t] = -INFINITY; }
    }
    // online softmax in the exp2 domain: first the exponent arguments against the
    // running maximum; only when one of them exceeds 8 (some row's maximum grew
    // by more than a factor 2^8 — always so in the first block) is the exact row
    // maximum formed and the output rescaled, so the common block needs no
    // cross-lane reduction
    bf16x8 pf[2][2];
#pragma unroll
    for (int qi = 0; qi < 2; ++qi) {
      float tt[4][4];
      float tm = -INFINITY;
#pragma unroll
      for (int kj = 0; kj < 4; ++kj)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          tt[kj][t] = fmaf(s[qi][kj][t], p.scale_log2, -m_run[qi]);
          tm = fmaxf(tm, tt[kj][t]);
        }
      if (__builtin_amdgcn_ballot_w64(!(tm <= 8.0f)) != 0) {   // wave-uniform, rare
        float mx = -INFINITY;
#pragma unroll
        for (int kj = 0; kj < 4; ++kj)
#pragma unroll
          for (int t = 0; t < 4; ++t) mx = fmaxf(mx, s[qi][kj][t]);
        // row maximum over lanes l, l^16, l^32, l^48: gfx950's row swaps give
        // each lane the pair {x[l], x[l^16]} (then {x[l], x[l^32]}) without LDS
        const auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                          false, false);
        mx = fmaxf(__uint_as_float(p16[0]), __uint_as_float(p16[1]));
        const auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                          false, false);
        mx = fmaxf(__uint_as_float(p32[0]), __uint_as_float(p32[1]));
        const float m_blk = mx * p.scale_log2;
        const bool grow = m_blk > m_run[qi] + 8.0f;
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
          const float m_new = grow ? m_blk : m_run[qi];
          const float alpha = __builtin_amdgcn_exp2f(m_run[qi] - m_new);
#pragma unroll
          for (int dj = 0; dj < 9; ++dj) o[qi][dj] *= alpha;
          m_run[qi] = m_new;
#pragma unroll
          for (int kj = 0; kj < 4; ++kj)
#pragma unroll
            for (int t = 0; t < 4; ++t) tt[kj][t] = fmaf(s[qi][kj][t], p.scale_log2, -m_run[qi]);
        }
      }
      // P as the PV operand: slots 0..3 = keys 4c..4c+3 of key block 2·kk2,
      // slots 4..7 = the same of block 2·kk2 + 1 (the Vᵀ fragment matches)
#pragma unroll
      for (int kk2 = 0; kk2 < 2; ++kk2)
        pf[qi][kk2] = (bf16x8){(__bf16)__builtin_amdgcn_exp2f(tt[2 * kk2][0]),
                               (__bf16)__builtin_amdgcn_exp2f(tt[2 * kk2][1]),
                               (__bf16)__builtin_amdgcn_exp2f(tt[2 * kk2][2]),
                               (__bf16)__builtin_amdgcn_exp2f(tt[2 * kk2][3]),
                               (__bf16)__builtin_amdgcn_exp2f(tt[2 * kk2 + 1][0]),
                               (__bf16)__builtin_amdgcn_exp2f(tt[2 * kk2 + 1][1]),
                               (__bf16)__builtin_amdgcn_exp2f(tt[2 * kk2 + 1][2]),
                               (__bf16)__builtin_amdgcn_exp2f(tt[2 * kk2 + 1][3])};
    }
    // O += P·V: Vᵀ fragment of head dims 16·dj + l%16, keys 32·kk2 + 4c + 0..3
    // and 32·kk2 + 16 + 4c + 0..3: chunk 4·kk2 + c of the interleaved row
#pragma unroll
    for (int kk2 = 0; kk2 < 2; ++kk2)
#pragma unroll
      for (int dj = 0; dj < 8; ++dj) {
        const int row = 16 * dj + r16;
        const bf16x8 vf =
            *(const bf16x8*)(vt + row * kVRow + (((4 * kk2 + c4) ^ (row & 7)) << 4));
#pragma unroll
        for (int qi = 0; qi < 2; ++qi)
          o[qi][dj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[qi][kk2], o[qi][dj], 0, 0, 0);
      }
#pragma unroll
    for (int kk2 = 0; kk2 < 2; ++kk2)
#pragma unroll
      for (int qi = 0; qi < 2; ++qi)
        o[qi][8] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf[qi][kk2], o[qi][8], 0, 0, 0);
  };
  int j = 0;
  for (; j + 1 < nkb; j += 2) {
    block(j, std::integral_constant<int, 0>{});
    block(j + 1, std::integral_constant<int, 1>{});
  }
  if (j < nkb) block(j, std::integral_constant<int, 0>{});

  // O / l, rounded to bf16: lane l writes query 16·qi + l%16, head dims
  // 16·dj + 4c .. +3 (8 bytes)
#pragma unroll
  for (int qi = 0; qi < 2; ++qi) {
    const int64_t q = q0 + 32 * wave + 16 * qi + r16;
    if (q >= S) continue;
    const float inv = 1.0f / o[qi][8][0];
    bf16_t* dst = p.O + q * p.ldo + (int64_t)h * kD + 4 * c4;
#pragma unroll
    for (int dj = 0; dj < 8; ++dj) {
      u32x2 w;
      w.x = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(o[qi][dj][0] * inv)) |
            ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(o[qi][dj][1] * inv)) << 16);
      w.y = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(o[qi][dj][2] * inv)) |
            ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(o[qi][dj][3] * inv)) << 16);
      *(u32x2*)(dst + 16 * dj) = w;
    }
  }
}

// Vᵀ per head: Vt[(h·D + d)·Sp + perm(s)] = V[s·ld + h·D + d], zeros for
// s >= S, where perm interleaves the 4-key quarters of the two 16-key halves of
// each 32-key group: s = 32g + 16a + 4c + t  ->  32g + 8c + 4a + t.
// One 64-token x 64-dim tile per workgroup through LDS.
constexpr int kTT = 64;
__global__ __launch_bounds__(256) void transpose_v_kernel(const bf16_t* V, int64_t ld, int64_t S,
                                                         int64_t Sp, int H, bf16_t* Vt) {
  __shared__ uint16_t tile[kTT][kTT + 2];
  const int64_t s0 = (int64_t)blockIdx.x * kTT;
  const int d0 = blockIdx.y * kTT;
  const int h = blockIdx.z;
  // read 64 rows x 128 bytes: 512 chunks of 8 elements, two per thread
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int idx = threadIdx.x + 256 * t;
    const int r = idx >> 3, c = idx & 7;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (s0 + r < S) v = *(const u32x4*)(V + (s0 + r) * ld + (int64_t)h * kD + d0 + 8 * c);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    const int rp = (r & 32) | ((r & 12) << 1) | ((r & 16) >> 2) | (r & 3);   // perm within 64
#pragma unroll
    for (int e = 0; e < 8; ++e)
      tile[8 * c + e][rp] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
  }
  __syncthreads();
  // write 64 head-dim rows x 128 bytes
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int idx = threadIdx.x + 256 * t;
    const int r = idx >> 3, c = idx & 7;
    u32x4 v;
    v.x = (uint32_t)tile[r][8 * c + 0] | ((uint32_t)tile[r][8 * c + 1] << 16);
    v.y = (uint32_t)tile[r][8 * c + 2] | ((uint32_t)tile[r][8 * c + 3] << 16);
    v.z = (uint32_t)tile[r][8 * c + 4] | ((uint32_t)tile[r][8 * c + 5] << 16);
    v.w = (uint32_t)tile[r][8 * c + 6] | ((uint32_t)tile[r][8 * c + 7] << 16);
    *(u32x4*)(Vt + ((int64_t)h * kD + d0 + r) * Sp + s0 + 8 * c) = v;
  }
}

}  // namespace

int64_t attention_padded_tokens(int64_t S) { return (S + kBK - 1) / kBK * kBK; }

hipError_t launch_attention(const bf16_t* Q, const bf16_t* K, const bf16_t* V, int64_t ld,
                            bf16_t* O, int64_t ldo, int64_t S, int H, float scale,
                            bf16_t* Vt, hipStream_t s) {
  if (S <= 0 || H <= 0) return hipSuccess;
  const int64_t Sp = attention_padded_tokens(S);
  hipLaunchKernelGGL(transpose_v_kernel, dim3((unsigned)(Sp / kTT), kD / kTT, (unsigned)H),
                     dim3(256), 0, s, V, ld, S, Sp, H, Vt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  AttnParams p;
  p.Q = Q; p.K = K; p.Vt = Vt; p.O = O;
  p.ld = ld; p.ldo = ldo; p.S = S; p.Sp = Sp;
  p.H = H;
  p.nqb = (int)((S + kBQ - 1) / kBQ);
  p.scale_log2 = scale * 1.4426950408889634f;
  const int64_t blocks = (int64_t)H * p.nqb;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(attention_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace fsd
