// C ABI of libfsd.so (include/fsd.h): argument validation, M-chunking of the
// LoRA linear through the caller's workspace, and kernel launches.
//
// Every entry point validates all arguments before it makes any HIP call, so
// an invalid request returns its status without touching the device.  The
// library keeps no state and never allocates, frees or synchronises.
#include <math.h>
#include <string.h>

#include <mutex>

#include "../../include/fsd.h"
#include "fsd_internal.h"

using fsd::bf16_t;

namespace {

constexpr int64_t kTileM = 256;            // rows per GEMM tile: the chunk granule
// Rows per chunk of the pipelined LoRA linear: 85 tile-rows, so that the 255
// phase-A tiles (3 column tiles of 192 at rank 576) of the next chunk fill the
// last wave of the current chunk's phase-B tiles on 256 CUs.  Two chunks of T
// at rank 576 take 50.1 MB.
constexpr int64_t kPairChunkRows = 85 * kTileM;
// Chunk rows of the MXFP8 linear's schedule.  Its launches run twice as fast as
// the bf16 ones, but 170 and 255 row tiles measured no better than 85 on the 2K
// step (203.6 and 204.2 against 203.3 ms).
constexpr int64_t kMxPairChunkRows = 85 * kTileM;
constexpr int64_t kMaxOffsetBytes = 0x7fffffffLL;

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Bytes spanned by a rows x cols matrix with row stride ld (elements of size es).
inline int64_t span_bytes(int64_t rows, int64_t cols, int64_t ld, int64_t es) {
  if (rows <= 0 || cols <= 0) return 0;
  return ((rows - 1) * ld + cols) * es;
}

inline bool overlap(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
  if (!a || !b || abytes <= 0 || bbytes <= 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

inline int from_hip(hipError_t e) { return e == hipSuccess ? FSD_OK : FSD_EHIP; }

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

struct UpShape {
  const void *X, *W0, *T, *B;
  int64_t ldx, ldt;
  const float* bias;
  const void* residual;
  int64_t ldr;
  void* Y;
  int64_t ldy, M, N, K, r;
  int epi;
};

// Checks shared by phase B and the fused call (T may still be unset: has_t).
int validate_up(const UpShape& a, bool has_t) {
  if (a.M < 0 || a.K < 8 || a.N < 8 || a.r < 0) return FSD_EINVAL;
  if (a.K % 8 || a.N % 8 || a.r % 8) return FSD_EINVAL;
  if (a.epi != FSD_EPI_NONE && a.epi != FSD_EPI_SWIGLU) return FSD_EINVAL;
  if (a.epi == FSD_EPI_SWIGLU && (a.N % 16 || a.residual)) {
    return a.residual ? FSD_EUNSUPPORTED : FSD_EINVAL;
  }
  const int64_t nout = a.epi == FSD_EPI_SWIGLU ? a.N / 2 : a.N;
  if (!a.X || !a.W0 || !a.Y) return FSD_EINVAL;
  if (a.r > 0 && (!a.B || (has_t && !a.T))) return FSD_EINVAL;
  if (a.ldx < a.K || a.ldy < nout || a.ldx % 8 || a.ldy % 8) return FSD_EINVAL;
  if (a.r > 0 && has_t && (a.ldt < a.r || a.ldt % 8)) return FSD_EINVAL;
  if (a.residual && (a.ldr < nout || a.ldr % 8)) return FSD_EINVAL;
  if (!aligned16(a.X) || !aligned16(a.W0) || !aligned16(a.Y)) return FSD_EALIGN;
  if (a.r > 0 && (!aligned16(a.B) || (has_t && !aligned16(a.T)))) return FSD_EALIGN;
  if (a.residual && !aligned16(a.residual)) return FSD_EALIGN;
  if (a.bias && ((uintptr_t)a.bias & 3u)) return FSD_EALIGN;
  // 32-bit buffer offsets: whole weight matrices and one 256-row activation tile
  if ((a.N + kTileM) * a.K * 2 > kMaxOffsetBytes || (a.N + kTileM) * a.r * 2 > kMaxOffsetBytes)
    return FSD_EUNSUPPORTED;
  if (kTileM * a.ldx * 2 > kMaxOffsetBytes || kTileM * a.ldt * 2 > kMaxOffsetBytes)
    return FSD_EUNSUPPORTED;
  // the residual is fetched through one 256-row tile's buffer resource
  if (a.residual && kTileM * a.ldr * 2 > kMaxOffsetBytes) return FSD_EUNSUPPORTED;
  // aliasing
  const int64_t ybytes = span_bytes(a.M, nout, a.ldy, 2);
  if (overlap(a.Y, ybytes, a.X, span_bytes(a.M, a.K, a.ldx, 2)) ||
      overlap(a.Y, ybytes, a.W0, a.N * a.K * 2) ||
      overlap(a.Y, ybytes, a.bias, a.bias ? a.N * 4 : 0))
    return FSD_EINVAL;
  if (a.r > 0 && (overlap(a.Y, ybytes, a.B, a.N * a.r * 2) ||
                  (has_t && overlap(a.Y, ybytes, a.T, span_bytes(a.M, a.r, a.ldt, 2)))))
    return FSD_EINVAL;
  if (a.residual) {
    const bool same = a.residual == a.Y && a.ldr == a.ldy;
    if (!same && overlap(a.Y, ybytes, a.residual, span_bytes(a.M, nout, a.ldr, 2)))
      return FSD_EINVAL;
  }
  return FSD_OK;
}

fsd::GemmParams up_params(const UpShape& a) {
  fsd::GemmParams p;
  memset(&p, 0, sizeof(p));
  p.A0 = (const bf16_t*)a.X;  p.lda0 = a.ldx;
  p.B0 = (const bf16_t*)a.W0; p.ldb0 = a.K;
  p.A1 = (const bf16_t*)a.T;  p.lda1 = a.ldt;
  p.B1 = (const bf16_t*)a.B;  p.ldb1 = a.r;
  p.M = a.M; p.N = a.N; p.K0 = a.K; p.K1 = a.r;
  p.alpha = 1.0f;
  p.bias = a.bias;
  p.res = (const bf16_t*)a.residual; p.ldr = a.ldr;
  p.Y = (bf16_t*)a.Y; p.ldy = a.ldy;
  return p;
}

fsd::GemmParams down_params(const void* X, int64_t ldx, const void* A, float scale, void* T,
                            int64_t ldt, int64_t M, int64_t K, int64_t r) {
  fsd::GemmParams p;
  memset(&p, 0, sizeof(p));
  p.A0 = (const bf16_t*)X; p.lda0 = ldx;
  p.B0 = (const bf16_t*)A; p.ldb0 = K;
  p.M = M; p.N = r; p.K0 = K; p.K1 = 0;
  p.alpha = scale;
  p.Y = (bf16_t*)T; p.ldy = ldt;
  return p;
}

int validate_down(const void* X, int64_t ldx, const void* A, float scale, const void* T,
                  int64_t ldt, int64_t M, int64_t K, int64_t r) {
  if (M < 0 || K < 8 || r < 8 || K % 8 || r % 8) return FSD_EINVAL;
  if (!X || !A || !T) return FSD_EINVAL;
  if (!isfinite(scale)) return FSD_EINVAL;
  if (ldx < K || ldx % 8 || ldt < r || ldt % 8) return FSD_EINVAL;
  if (!aligned16(X) || !aligned16(A) || !aligned16(T)) return FSD_EALIGN;
  if ((r + kTileM) * K * 2 > kMaxOffsetBytes || kTileM * ldx * 2 > kMaxOffsetBytes)
    return FSD_EUNSUPPORTED;
  const int64_t tbytes = span_bytes(M, r, ldt, 2);
  if (overlap(T, tbytes, X, span_bytes(M, K, ldx, 2)) || overlap(T, tbytes, A, r * K * 2))
    return FSD_EINVAL;
  return FSD_OK;
}

// ---- MXFP8 operands --------------------------------------------------------
inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Scale bytes of `rows` rows over Kp (a multiple of 128) elements.
inline int64_t mx_scale_span(int64_t rows, int64_t Kp) {
  return (Kp / 128) * round_up(rows, kTileM) * 4;
}

// One MX operand: codes [rows, Kp] with row stride ld bytes plus its scales.
// A weight operand (whole_matrix) is addressed from its base; an activation
// operand from each 256-row tile.
int validate_mx_operand(const void* q, int64_t ld, const void* s, int64_t rows, int64_t Kp,
                        bool whole_matrix) {
  if (!q || !s || ld < Kp || ld % 16) return FSD_EINVAL;
  if (!aligned16(q) || ((uintptr_t)s & 3u)) return FSD_EALIGN;
  const int64_t span = whole_matrix ? (rows + kTileM) * ld : kTileM * ld;
  if (span > kMaxOffsetBytes || mx_scale_span(rows, Kp) > kMaxOffsetBytes)
    return FSD_EUNSUPPORTED;
  return FSD_OK;
}

// Output Y (bytes yb) must not overlap an operand's codes or scales.
inline bool mx_overlaps(const void* Y, int64_t yb, const void* q, int64_t ld, const void* s,
                        int64_t rows, int64_t Kp) {
  return overlap(Y, yb, q, span_bytes(rows, Kp, ld, 1)) ||
         overlap(Y, yb, s, mx_scale_span(rows, Kp));
}

// Shared checks of the MXFP8 phase-B inputs; `out` / `ob` is the first output
// (Y, or the E4M3 bytes of H), checked against every input for overlap.
int validate_mx_up_inputs(const void* Xq, int64_t ldxq, const void* Xs, const void* W0q,
                          const void* W0s, const void* Tq, int64_t ldtq, const void* Ts,
                          const void* Bq, const void* Bs, const float* bias, int64_t M,
                          int64_t N, int64_t K, int64_t r, const void* out, int64_t ob) {
  if (M < 0 || K < 32 || K % 32 || N < 8 || N % 8 || r < 0 || r % 32) return FSD_EINVAL;
  if (bias && ((uintptr_t)bias & 3u)) return FSD_EALIGN;
  const int64_t Kp = round_up(K, 128), rp = round_up(r, 128);
  int st = validate_mx_operand(Xq, ldxq, Xs, M, Kp, false);
  if (st == FSD_OK) st = validate_mx_operand(W0q, Kp, W0s, N, Kp, true);
  if (st == FSD_OK && r > 0) st = validate_mx_operand(Tq, ldtq, Ts, M, rp, false);
  if (st == FSD_OK && r > 0) st = validate_mx_operand(Bq, rp, Bs, N, rp, true);
  if (st != FSD_OK) return st;
  if (mx_overlaps(out, ob, Xq, ldxq, Xs, M, Kp) || mx_overlaps(out, ob, W0q, Kp, W0s, N, Kp) ||
      overlap(out, ob, bias, bias ? N * 4 : 0))
    return FSD_EINVAL;
  if (r > 0 && (mx_overlaps(out, ob, Tq, ldtq, Ts, M, rp) ||
                mx_overlaps(out, ob, Bq, rp, Bs, N, rp)))
    return FSD_EINVAL;
  return FSD_OK;
}

fsd::GemmParams mx_up_params(const void* Xq, int64_t ldxq, const void* Xs, const void* W0q,
                             const void* W0s, const void* Tq, int64_t ldtq, const void* Ts,
                             const void* Bq, const void* Bs, const float* bias, int64_t M,
                             int64_t N, int64_t K, int64_t r) {
  const int64_t Kp = round_up(K, 128), rp = round_up(r, 128);
  fsd::GemmParams p;
  memset(&p, 0, sizeof(p));
  p.A0 = Xq; p.lda0 = ldxq; p.sA0 = (const uint8_t*)Xs;
  p.B0 = W0q; p.ldb0 = Kp;  p.sB0 = (const uint8_t*)W0s;
  if (r > 0) {
    p.A1 = Tq; p.lda1 = ldtq; p.sA1 = (const uint8_t*)Ts;
    p.B1 = Bq; p.ldb1 = rp;   p.sB1 = (const uint8_t*)Bs;
  }
  p.M = M; p.N = N; p.K0 = Kp; p.K1 = rp;
  p.sMp = round_up(M, kTileM); p.sNp = round_up(N, kTileM);
  p.alpha = 1.0f;
  p.bias = bias;
  return p;
}

}  // namespace

extern "C" {

int fsd_abi_version(void) { return FSD_ABI_VERSION; }

const char* fsd_status_str(fsd_status status) {
  switch ((int)status) {
    case FSD_OK: return "FSD_OK";
    case FSD_EINVAL: return "FSD_EINVAL";
    case FSD_EALIGN: return "FSD_EALIGN";
    case FSD_EUNSUPPORTED: return "FSD_EUNSUPPORTED";
    case FSD_EWORKSPACE: return "FSD_EWORKSPACE";
    case FSD_EHIP: return "FSD_EHIP";
  }
  return "FSD_UNKNOWN";
}

int fsd_lora_merge(int n_adapters, const float* const* A_list, const float* const* B_list,
                   const int64_t* ranks, const float* scales, int64_t K, int64_t N, void* A_out,
                   void* B_out, void* stream) {
  if (n_adapters < 1 || n_adapters > 16 || !A_list || !B_list || !ranks) return FSD_EINVAL;
  if (K < 1 || N < 1 || !A_out || !B_out) return FSD_EINVAL;
  if (!aligned16(A_out) || !aligned16(B_out)) return FSD_EALIGN;
  int64_t R = 0;
  for (int i = 0; i < n_adapters; ++i) {
    if (!A_list[i] || !B_list[i] || ranks[i] < 1) return FSD_EINVAL;
    if (((uintptr_t)A_list[i] & 3u) || ((uintptr_t)B_list[i] & 3u)) return FSD_EALIGN;
    if (scales && !isfinite(scales[i])) return FSD_EINVAL;
    R += ranks[i];
  }
  if (overlap(A_out, R * K * 2, B_out, N * R * 2)) return FSD_EINVAL;
  for (int i = 0; i < n_adapters; ++i) {
    if (overlap(A_out, R * K * 2, A_list[i], ranks[i] * K * 4) ||
        overlap(A_out, R * K * 2, B_list[i], N * ranks[i] * 4) ||
        overlap(B_out, N * R * 2, A_list[i], ranks[i] * K * 4) ||
        overlap(B_out, N * R * 2, B_list[i], N * ranks[i] * 4))
      return FSD_EINVAL;
  }
  hipStream_t s = as_stream(stream);
  int64_t row0 = 0;
  for (int i = 0; i < n_adapters; ++i) {
    const float sc = scales ? scales[i] : 1.0f;
    hipError_t e = fsd::launch_merge_rows(A_list[i], ranks[i], K, (bf16_t*)A_out + row0 * K, K, s);
    if (e != hipSuccess) return FSD_EHIP;
    e = fsd::launch_merge_cols(B_list[i], N, ranks[i], sc, (bf16_t*)B_out + row0, R, s);
    if (e != hipSuccess) return FSD_EHIP;
    row0 += ranks[i];
  }
  return FSD_OK;
}

size_t fsd_lora_linear_workspace_bytes(int64_t M, int64_t r) {
  if (M <= 0 || r <= 0) return 0;
  const int64_t rows = M < 2 * kPairChunkRows ? M : 2 * kPairChunkRows;
  return (size_t)rows * (size_t)r * 2u;
}

int fsd_lora_down(const void* X, int64_t ldx, const void* A, float scale, void* T, int64_t ldt,
                  int64_t M, int64_t K, int64_t r, void* stream) {
  const int st = validate_down(X, ldx, A, scale, T, ldt, M, K, r);
  if (st != FSD_OK) return st;
  if (M == 0) return FSD_OK;
  return from_hip(fsd::launch_gemm(fsd::GEMM_DOWN,
                                   down_params(X, ldx, A, scale, T, ldt, M, K, r),
                                   as_stream(stream)));
}

int fsd_lora_up(const void* X, int64_t ldx, const void* W0, const void* T, int64_t ldt,
                const void* B, const float* bias, const void* residual, int64_t ldr, void* Y,
                int64_t ldy, int64_t M, int64_t N, int64_t K, int64_t r, int epilogue,
                void* stream) {
  const UpShape a{X, W0, T, B, ldx, ldt, bias, residual, ldr, Y, ldy, M, N, K, r, epilogue};
  const int st = validate_up(a, true);
  if (st != FSD_OK) return st;
  if (M == 0) return FSD_OK;
  const fsd::GemmKind kind = epilogue == FSD_EPI_SWIGLU ? fsd::GEMM_UP_SWIGLU : fsd::GEMM_UP;
  return from_hip(fsd::launch_gemm(kind, up_params(a), as_stream(stream)));
}

}  // extern "C"

namespace {

// The launch plan of the chunked LoRA linear (fsd_lora_linear): M rows at rank
// r through a workspace that holds `fit` rows of T (at least min(M, 256)).
//   SCHED_WHOLE: all M rows of T fit: phase A over all rows, then phase B;
//   SCHED_PAIRS: two chunks of at least 256 rows fit: chunks of R <=
//     kPairChunkRows rows (a multiple of 256) through two alternating halves of
//     the workspace; launch 0 is phase A of chunk 0, launch c + 1 is phase B of
//     chunk c together with phase A of chunk c + 1 (launch_gemm_pair);
//   SCHED_CHUNKS: 256-row multiples through one buffer, phase A then phase B
//     of each chunk.
// Chunks start on 256-row boundaries, so every output row is computed by the
// same tile arithmetic as without chunking: the result is bitwise identical.
enum { SCHED_WHOLE = 0, SCHED_PAIRS = 1, SCHED_CHUNKS = 2 };
struct Plan {
  int sched;
  int64_t R;         // rows per chunk
  int64_t nc;        // chunks
  int64_t launches;
};

Plan make_plan(int64_t M, int64_t r, int64_t ws_bytes) {
  Plan pl{SCHED_WHOLE, M, M > 0 ? 1 : 0, 0};
  if (M <= 0) return pl;
  if (r == 0) { pl.launches = 1; return pl; }
  const int64_t fit = ws_bytes / (r * 2);
  if (fit >= M) { pl.launches = 2; return pl; }
  if (fit >= 2 * kTileM) {
    pl.sched = SCHED_PAIRS;
    pl.R = (fit / 2) / kTileM * kTileM;
    if (pl.R > kPairChunkRows) pl.R = kPairChunkRows;
    pl.nc = (M + pl.R - 1) / pl.R;
    pl.launches = pl.nc + 1;
    return pl;
  }
  pl.sched = SCHED_CHUNKS;
  pl.R = fit / kTileM * kTileM;
  pl.nc = (M + pl.R - 1) / pl.R;
  pl.launches = 2 * pl.nc;
  return pl;
}

// Bytes of the workspace the plan touches.
int64_t plan_workspace_bytes(const Plan& pl, int64_t M, int64_t r) {
  if (r == 0 || M <= 0) return 0;
  if (pl.sched == SCHED_WHOLE) return M * r * 2;
  return (pl.sched == SCHED_PAIRS ? 2 : 1) * pl.R * r * 2;
}

// Launch `index` of the plan (arguments already validated).
int lora_linear_launch(const UpShape& a, const void* A, float scale, void* workspace,
                       const Plan& pl, int64_t index, hipStream_t s) {
  const int64_t M = a.M, r = a.r, K = a.K;
  const bool swiglu = a.epi == FSD_EPI_SWIGLU;
  const fsd::GemmKind kind = swiglu ? fsd::GEMM_UP_SWIGLU : fsd::GEMM_UP;
  auto rows = [&](int64_t c) { return c < pl.nc ? ((M - c * pl.R) < pl.R ? (M - c * pl.R) : pl.R) : 0; };
  auto chunk_up = [&](int64_t c, const void* T) {
    const int64_t m = c * pl.R;
    UpShape u = a;
    u.X = (const bf16_t*)a.X + m * a.ldx;
    u.M = rows(c);
    u.T = T;
    u.ldt = r;
    u.Y = (bf16_t*)a.Y + m * a.ldy;
    if (a.residual) u.residual = (const bf16_t*)a.residual + m * a.ldr;
    return up_params(u);
  };
  auto chunk_down = [&](int64_t c, void* T) {
    const int64_t mc = rows(c);
    const int64_t m = mc > 0 ? c * pl.R : 0;
    return down_params((const bf16_t*)a.X + m * a.ldx, a.ldx, A, scale, T, r, mc, K, r);
  };
  if (index < 0 || index >= pl.launches) return FSD_EINVAL;
  if (r == 0) return from_hip(fsd::launch_gemm(kind, chunk_up(0, nullptr), s));
  switch (pl.sched) {
    case SCHED_WHOLE:
      return from_hip(index == 0 ? fsd::launch_gemm(fsd::GEMM_DOWN, chunk_down(0, workspace), s)
                                 : fsd::launch_gemm(kind, chunk_up(0, workspace), s));
    case SCHED_PAIRS: {
      void* buf[2] = {workspace, (char*)workspace + pl.R * r * 2};
      if (index == 0) return from_hip(fsd::launch_gemm(fsd::GEMM_DOWN, chunk_down(0, buf[0]), s));
      const int64_t c = index - 1;
      return from_hip(fsd::launch_gemm_pair(swiglu, chunk_up(c, buf[c & 1]),
                                            chunk_down(c + 1, buf[(c + 1) & 1]), s));
    }
    default: {
      const int64_t c = index / 2;
      return from_hip((index & 1) == 0
                          ? fsd::launch_gemm(fsd::GEMM_DOWN, chunk_down(c, workspace), s)
                          : fsd::launch_gemm(kind, chunk_up(c, workspace), s));
    }
  }
}

// Validation of fsd_lora_linear's arguments against a workspace of ws_bytes.
int validate_linear(const UpShape& a, const void* A, float scale, const void* workspace,
                    int64_t ws_bytes) {
  int st = validate_up(a, false);
  if (st != FSD_OK) return st;
  if (!isfinite(scale)) return FSD_EINVAL;
  if (a.r == 0) return FSD_OK;
  const int64_t M = a.M, N = a.N, K = a.K, r = a.r;
  if (!A) return FSD_EINVAL;
  if (!aligned16(A)) return FSD_EALIGN;
  if ((r + kTileM) * K * 2 > kMaxOffsetBytes) return FSD_EUNSUPPORTED;
  const int64_t need_min = (M < kTileM ? M : kTileM) * r * 2;
  if (M > 0 && (!workspace || ws_bytes < need_min)) return FSD_EWORKSPACE;
  if (workspace && !aligned16(workspace)) return FSD_EALIGN;
  const int64_t nout = a.epi == FSD_EPI_SWIGLU ? N / 2 : N;
  const int64_t wbytes = plan_workspace_bytes(make_plan(M, r, ws_bytes), M, r);
  if (overlap(a.Y, span_bytes(M, nout, a.ldy, 2), workspace, wbytes) ||
      overlap(workspace, wbytes, a.X, span_bytes(M, K, a.ldx, 2)) ||
      overlap(workspace, wbytes, a.W0, N * K * 2) || overlap(workspace, wbytes, A, r * K * 2) ||
      overlap(workspace, wbytes, a.B, N * r * 2) ||
      overlap(workspace, wbytes, a.bias, a.bias ? N * 4 : 0) ||
      overlap(workspace, wbytes, a.residual, a.residual ? span_bytes(M, nout, a.ldr, 2) : 0))
    return FSD_EINVAL;
  return FSD_OK;
}

}  // namespace

// ---- scratch of fsd_lora_linear_noalloc ----------------------------------------
// T of the allocation-free LoRA linear lives in this file-scope device array:
// two 21,760-row chunks at rank 576 (FSD_NOALLOC_SCRATCH_BYTES).  Each GPU the
// library runs on holds its own copy until the process ends.  In host code the
// name `scratch` is only a stand-in for the symbol, not a device address: the
// address is looked up per device with hipGetSymbolAddress and only that
// pointer is ever passed to a kernel.
static_assert(FSD_NOALLOC_SCRATCH_BYTES == 2 * kPairChunkRows * 576 * 2,
              "the scratch holds two pipelined chunks of T at rank 576");
static __device__ __align__(256) char scratch[FSD_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The current device's scratch address (looked up once per device), or null
// with *err set.
void* device_scratch(int* err) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *err = FSD_EHIP;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      *err = FSD_EHIP;
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int fsd_lora_linear_noalloc(const void* X, int64_t ldx, const void* W0, const void* A,
                            const void* B, const float* bias, const void* residual, int64_t ldr,
                            float scale, void* Y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                            int64_t r, int epilogue, void* stream) {
  // the limit first (host arithmetic): 256 rows of T must fit in the scratch
  if (r > (int64_t)(FSD_NOALLOC_SCRATCH_BYTES / (kTileM * 2))) return FSD_EUNSUPPORTED;
  int err = FSD_OK;
  void* ws = r > 0 ? device_scratch(&err) : nullptr;
  if (r > 0 && !ws) return err;
  const int64_t ws_bytes = r > 0 ? (int64_t)FSD_NOALLOC_SCRATCH_BYTES : 0;
  const UpShape a{X, W0, ws, B, ldx, r, bias, residual, ldr, Y, ldy, M, N, K, r, epilogue};
  const int st = validate_linear(a, A, scale, ws, ws_bytes);
  if (st != FSD_OK) return st;
  const Plan pl = make_plan(M, r, ws_bytes);
  for (int64_t i = 0; i < pl.launches; ++i) {
    const int e = lora_linear_launch(a, A, scale, ws, pl, i, as_stream(stream));
    if (e != FSD_OK) return e;
  }
  return FSD_OK;
}

int64_t fsd_lora_linear_plan(int64_t M, int64_t r, size_t workspace_bytes, int64_t* chunk_rows,
                             int* schedule) {
  if (M < 0 || r < 0) return -1;
  const int64_t ws = workspace_bytes > (size_t)INT64_MAX ? INT64_MAX : (int64_t)workspace_bytes;
  const Plan pl = make_plan(M, r, ws);
  if (chunk_rows) *chunk_rows = pl.R;
  if (schedule) *schedule = pl.sched;
  return pl.launches;
}

int fsd_lora_linear_launch(const void* X, int64_t ldx, const void* W0, const void* A,
                           const void* B, const float* bias, const void* residual, int64_t ldr,
                           float scale, void* Y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                           int64_t r, int epilogue, void* workspace, size_t workspace_bytes,
                           int64_t index, void* stream) {
  const UpShape a{X, W0, workspace, B, ldx, r, bias, residual, ldr, Y, ldy, M, N, K, r, epilogue};
  const int64_t ws = workspace_bytes > (size_t)INT64_MAX ? INT64_MAX : (int64_t)workspace_bytes;
  const int st = validate_linear(a, A, scale, workspace, ws);
  if (st != FSD_OK) return st;
  const Plan pl = make_plan(M, r, ws);
  if (index < 0 || index >= pl.launches) return M == 0 && index == 0 ? FSD_OK : FSD_EINVAL;
  return lora_linear_launch(a, A, scale, workspace, pl, index, as_stream(stream));
}

int fsd_lora_linear(const void* X, int64_t ldx, const void* W0, const void* A, const void* B,
                    const float* bias, const void* residual, int64_t ldr, float scale, void* Y,
                    int64_t ldy, int64_t M, int64_t N, int64_t K, int64_t r, int epilogue,
                    void* workspace, size_t workspace_bytes, void* stream) {
  const UpShape a{X, W0, workspace, B, ldx, r, bias, residual, ldr, Y, ldy, M, N, K, r, epilogue};
  const int64_t ws = workspace_bytes > (size_t)INT64_MAX ? INT64_MAX : (int64_t)workspace_bytes;
  const int st = validate_linear(a, A, scale, workspace, ws);
  if (st != FSD_OK) return st;
  const Plan pl = make_plan(M, r, ws);
  for (int64_t i = 0; i < pl.launches; ++i) {
    const int e = lora_linear_launch(a, A, scale, workspace, pl, i, as_stream(stream));
    if (e != FSD_OK) return e;
  }
  return FSD_OK;
}

int fsd_renoise(const float* u, const float* eps, float sigma, float* z, int64_t n,
                void* stream) {
  if (n < 0 || !isfinite(sigma)) return FSD_EINVAL;
  if (n == 0) return FSD_OK;
  if (!u || !eps || !z) return FSD_EINVAL;
  if (!aligned16(u) || !aligned16(eps) || !aligned16(z)) return FSD_EALIGN;
  const int64_t b = n * 4;
  if ((z != u && overlap(z, b, u, b)) || (z != eps && overlap(z, b, eps, b))) return FSD_EINVAL;
  return from_hip(fsd::launch_renoise(u, eps, sigma, z, n, as_stream(stream)));
}

int fsd_euler_step(float* z, const float* v, float sigma, float sigma_next, int64_t n,
                   void* stream) {
  if (n < 0 || !isfinite(sigma) || !isfinite(sigma_next)) return FSD_EINVAL;
  if (n == 0) return FSD_OK;
  if (!z || !v) return FSD_EINVAL;
  if (!aligned16(z) || !aligned16(v)) return FSD_EALIGN;
  const int64_t b = n * 4;
  if (z != v && overlap(z, b, v, b)) return FSD_EINVAL;
  const float d = sigma_next - sigma;
  return from_hip(fsd::launch_euler(z, v, d, n, as_stream(stream)));
}

int fsd_token_embed(const float* z, const void* E, void* X, int64_t ldx, int64_t M, int64_t C,
                    int64_t D, void* stream) {
  if (M < 0 || C < 1 || C > 32 || D < 8 || D % 8) return FSD_EINVAL;
  if (M == 0) return FSD_OK;
  if (!z || !E || !X || ldx < D || ldx % 8) return FSD_EINVAL;
  if (!aligned16(X) || ((uintptr_t)z & 3u) || ((uintptr_t)E & 1u)) return FSD_EALIGN;
  if (C * D * 2 > kMaxOffsetBytes) return FSD_EUNSUPPORTED;
  const int64_t xb = span_bytes(M, D, ldx, 2);
  if (overlap(X, xb, z, M * C * 4) || overlap(X, xb, E, D * C * 2)) return FSD_EINVAL;
  return from_hip(fsd::launch_embed(z, (const bf16_t*)E, (bf16_t*)X, ldx, M, (int)C, D,
                                    as_stream(stream)));
}

int fsd_token_embed_mx(const float* z, const void* E, void* X, int64_t ldx, int64_t M,
                       int64_t C, int64_t D, void* Xq, int64_t ldxq, void* Xs, void* stream) {
  if (M < 0 || C < 1 || C > 32 || D < 128 || D % 8) return FSD_EINVAL;
  if (D % 128) return FSD_EUNSUPPORTED;
  if (!z || !E || !X || ldx < D || ldx % 8 || !Xq || !Xs || ldxq < D || ldxq % 16)
    return FSD_EINVAL;
  if (!aligned16(X) || ((uintptr_t)z & 3u) || ((uintptr_t)E & 1u) || !aligned16(Xq) ||
      ((uintptr_t)Xs & 3u))
    return FSD_EALIGN;
  if (C * D * 2 > kMaxOffsetBytes || mx_scale_span(M, D) > kMaxOffsetBytes)
    return FSD_EUNSUPPORTED;
  if (M == 0) return FSD_OK;
  const int64_t xb = span_bytes(M, D, ldx, 2);
  const int64_t qb = span_bytes(M, D, ldxq, 1), sb = mx_scale_span(M, D);
  const void* in[2] = {z, E};
  const int64_t inb[2] = {M * C * 4, D * C * 2};
  for (int i = 0; i < 2; ++i)
    if (overlap(X, xb, in[i], inb[i]) || overlap(Xq, qb, in[i], inb[i]) ||
        overlap(Xs, sb, in[i], inb[i]))
      return FSD_EINVAL;
  if (overlap(X, xb, Xq, qb) || overlap(X, xb, Xs, sb) || overlap(Xq, qb, Xs, sb))
    return FSD_EINVAL;
  return from_hip(fsd::launch_embed_mx(z, (const bf16_t*)E, (bf16_t*)X, ldx, M, (int)C, D,
                                       (uint8_t*)Xq, ldxq, (uint8_t*)Xs, as_stream(stream)));
}

int fsd_token_head(const void* H, int64_t ldh, const void* P, float* v, int64_t M, int64_t D,
                   int64_t C, void* stream) {
  if (M < 0 || C < 1 || C > 32 || D < 64 || D % 64) return FSD_EINVAL;
  if (M == 0) return FSD_OK;
  if (!H || !P || !v || ldh < D || ldh % 8) return FSD_EINVAL;
  if (!aligned16(H) || !aligned16(P) || ((uintptr_t)v & 3u)) return FSD_EALIGN;
  if (C * D * 2 > kMaxOffsetBytes || 128 * ldh * 2 > kMaxOffsetBytes) return FSD_EUNSUPPORTED;
  const int64_t vb = M * C * 4;
  if (overlap(v, vb, H, span_bytes(M, D, ldh, 2)) || overlap(v, vb, P, C * D * 2))
    return FSD_EINVAL;
  return from_hip(fsd::launch_head((const bf16_t*)H, ldh, (const bf16_t*)P, v, M, D, (int)C,
                                   as_stream(stream)));
}

int fsd_token_head_euler(const void* H, int64_t ldh, const void* P, float* z, int64_t M,
                         int64_t D, int64_t C, float sigma, float sigma_next, void* stream) {
  if (M < 0 || C < 1 || C > 32 || D < 64 || D % 64) return FSD_EINVAL;
  if (!isfinite(sigma) || !isfinite(sigma_next)) return FSD_EINVAL;
  if (M == 0) return FSD_OK;
  if (!H || !P || !z || ldh < D || ldh % 8) return FSD_EINVAL;
  if (!aligned16(H) || !aligned16(P) || ((uintptr_t)z & 3u)) return FSD_EALIGN;
  if (C * D * 2 > kMaxOffsetBytes || 128 * ldh * 2 > kMaxOffsetBytes) return FSD_EUNSUPPORTED;
  const int64_t zb = M * C * 4;
  if (overlap(z, zb, H, span_bytes(M, D, ldh, 2)) || overlap(z, zb, P, C * D * 2))
    return FSD_EINVAL;
  const float d = sigma_next - sigma;
  return from_hip(fsd::launch_head_euler((const bf16_t*)H, ldh, (const bf16_t*)P, z, d, M, D,
                                         (int)C, as_stream(stream)));
}

size_t fsd_mx_scale_bytes(int64_t M, int64_t K) {
  if (M < 0 || K < 0) return 0;
  return (size_t)(((K + 127) / 128) * ((M + 255) / 256 * 256) * 4);
}

int fsd_mx_quantize(const void* X, int64_t ldx, int64_t M, int64_t K, void* Q, int64_t ldq,
                    void* S, void* stream) {
  if (M < 0 || K < 32 || K % 32) return FSD_EINVAL;
  if (M == 0) return FSD_OK;
  const int64_t Kp = (K + 127) / 128 * 128;
  if (!X || !Q || !S || ldx < K || ldx % 8 || ldq < Kp || ldq % 16) return FSD_EINVAL;
  if (!aligned16(X) || !aligned16(Q) || ((uintptr_t)S & 3u)) return FSD_EALIGN;
  const int64_t qb = span_bytes(M, Kp, ldq, 1);
  const int64_t sb = (int64_t)fsd_mx_scale_bytes(M, K);
  const int64_t xb = span_bytes(M, K, ldx, 2);
  if (overlap(Q, qb, X, xb) || overlap(S, sb, X, xb) || overlap(S, sb, Q, qb)) return FSD_EINVAL;
  return from_hip(fsd::launch_mx_quantize((const bf16_t*)X, ldx, M, K, (uint8_t*)Q, ldq,
                                          (uint8_t*)S, as_stream(stream)));
}

int fsd_mx_lora_down(const void* Xq, int64_t ldxq, const void* Xs, const void* Aq,
                     const void* As, float scale, void* T, int64_t ldt, int64_t M, int64_t K,
                     int64_t r, void* stream) {
  if (M < 0 || K < 32 || K % 32 || r < 8 || r % 8 || !isfinite(scale)) return FSD_EINVAL;
  if (!T || ldt < r || ldt % 8) return FSD_EINVAL;
  if (!aligned16(T)) return FSD_EALIGN;
  const int64_t Kp = round_up(K, 128);
  int st = validate_mx_operand(Xq, ldxq, Xs, M, Kp, false);
  if (st == FSD_OK) st = validate_mx_operand(Aq, Kp, As, r, Kp, true);
  if (st != FSD_OK) return st;
  const int64_t tb = span_bytes(M, r, ldt, 2);
  if (mx_overlaps(T, tb, Xq, ldxq, Xs, M, Kp) || mx_overlaps(T, tb, Aq, Kp, As, r, Kp))
    return FSD_EINVAL;
  if (M == 0) return FSD_OK;
  fsd::GemmParams p;
  memset(&p, 0, sizeof(p));
  p.A0 = Xq; p.lda0 = ldxq; p.sA0 = (const uint8_t*)Xs;
  p.B0 = Aq; p.ldb0 = Kp;   p.sB0 = (const uint8_t*)As;
  p.M = M; p.N = r; p.K0 = Kp; p.K1 = 0;
  p.sMp = round_up(M, kTileM); p.sNp = round_up(r, kTileM);
  p.alpha = scale;
  p.Y = (bf16_t*)T; p.ldy = ldt;
  return from_hip(fsd::launch_gemm(fsd::GEMM_MX_DOWN, p, as_stream(stream)));
}

int fsd_mx_lora_up(const void* Xq, int64_t ldxq, const void* Xs, const void* W0q,
                   const void* W0s, const void* Tq, int64_t ldtq, const void* Ts,
                   const void* Bq, const void* Bs, const float* bias, const void* residual,
                   int64_t ldr, void* Y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                   int64_t r, int epilogue, void* stream) {
  if (epilogue != FSD_EPI_NONE && epilogue != FSD_EPI_SWIGLU) return FSD_EINVAL;
  const bool swiglu = epilogue == FSD_EPI_SWIGLU;
  if (N < 8 || (swiglu && N % 16)) return FSD_EINVAL;
  if (swiglu && (N % 128 || residual)) return FSD_EUNSUPPORTED;
  const int64_t nout = swiglu ? N / 2 : N;
  if (!Y || ldy < nout || ldy % 8) return FSD_EINVAL;
  if (residual && (ldr < nout || ldr % 8)) return FSD_EINVAL;
  if (!aligned16(Y) || (residual && !aligned16(residual))) return FSD_EALIGN;
  if (residual && kTileM * ldr * 2 > kMaxOffsetBytes) return FSD_EUNSUPPORTED;
  const int64_t yb = span_bytes(M, nout, ldy, 2);
  const int st = validate_mx_up_inputs(Xq, ldxq, Xs, W0q, W0s, Tq, ldtq, Ts, Bq, Bs, bias, M, N,
                                       K, r, Y, yb);
  if (st != FSD_OK) return st;
  if (residual) {
    const bool same = residual == Y && ldr == ldy;
    if (!same && overlap(Y, yb, residual, span_bytes(M, nout, ldr, 2))) return FSD_EINVAL;
  }
  if (M == 0) return FSD_OK;
  fsd::GemmParams p = mx_up_params(Xq, ldxq, Xs, W0q, W0s, Tq, ldtq, Ts, Bq, Bs, bias, M, N, K, r);
  p.res = (const bf16_t*)residual; p.ldr = ldr;
  p.Y = (bf16_t*)Y; p.ldy = ldy;
  const fsd::GemmKind kind = swiglu ? fsd::GEMM_MX_UP_SWIGLU : fsd::GEMM_MX_UP;
  return from_hip(fsd::launch_gemm(kind, p, as_stream(stream)));
}

int fsd_mx_lora_up_swiglu_mx(const void* Xq, int64_t ldxq, const void* Xs, const void* W0q,
                             const void* W0s, const void* Tq, int64_t ldtq, const void* Ts,
                             const void* Bq, const void* Bs, const float* bias, void* Hq,
                             int64_t ldhq, void* Hs, int64_t M, int64_t N, int64_t K, int64_t r,
                             void* stream) {
  if (N < 16 || N % 16) return FSD_EINVAL;
  if (N % 256) return FSD_EUNSUPPORTED;
  const int64_t F = N / 2;
  if (!Hq || !Hs || ldhq < F || ldhq % 16) return FSD_EINVAL;
  if (!aligned16(Hq) || ((uintptr_t)Hs & 3u)) return FSD_EALIGN;
  if (kTileM * ldhq > kMaxOffsetBytes || mx_scale_span(M, F) > kMaxOffsetBytes)
    return FSD_EUNSUPPORTED;
  const int64_t hb = span_bytes(M, F, ldhq, 1), hsb = mx_scale_span(M, F);
  int st = validate_mx_up_inputs(Xq, ldxq, Xs, W0q, W0s, Tq, ldtq, Ts, Bq, Bs, bias, M, N, K, r,
                                 Hq, hb);
  if (st == FSD_OK)
    st = validate_mx_up_inputs(Xq, ldxq, Xs, W0q, W0s, Tq, ldtq, Ts, Bq, Bs, bias, M, N, K, r,
                               Hs, hsb);
  if (st != FSD_OK) return st;
  if (overlap(Hq, hb, Hs, hsb)) return FSD_EINVAL;
  if (M == 0) return FSD_OK;
  fsd::GemmParams p = mx_up_params(Xq, ldxq, Xs, W0q, W0s, Tq, ldtq, Ts, Bq, Bs, bias, M, N, K, r);
  p.Yq = (uint8_t*)Hq; p.ldyq = ldhq;
  p.Ys = (uint8_t*)Hs; p.sYp = round_up(M, kTileM);
  return from_hip(fsd::launch_gemm(fsd::GEMM_MX_UP_SWIGLU_MX, p, as_stream(stream)));
}

int fsd_mx_lora_down_mx(const void* Xq, int64_t ldxq, const void* Xs, const void* Aq,
                        const void* As, float scale, void* Tq, int64_t ldtq, void* Ts, int64_t M,
                        int64_t K, int64_t r, void* stream) {
  if (M < 0 || K < 32 || K % 32 || r < 32 || r % 32 || !isfinite(scale)) return FSD_EINVAL;
  const int64_t Kp = round_up(K, 128), rp = round_up(r, 128);
  if (!Tq || !Ts || ldtq < rp || ldtq % 16) return FSD_EINVAL;
  if (!aligned16(Tq) || ((uintptr_t)Ts & 3u)) return FSD_EALIGN;
  if (mx_scale_span(M, rp) > kMaxOffsetBytes) return FSD_EUNSUPPORTED;
  int st = validate_mx_operand(Xq, ldxq, Xs, M, Kp, false);
  if (st == FSD_OK) st = validate_mx_operand(Aq, Kp, As, r, Kp, true);
  if (st != FSD_OK) return st;
  const int64_t tb = span_bytes(M, rp, ldtq, 1), sb = mx_scale_span(M, rp);
  if (mx_overlaps(Tq, tb, Xq, ldxq, Xs, M, Kp) || mx_overlaps(Tq, tb, Aq, Kp, As, r, Kp) ||
      mx_overlaps(Ts, sb, Xq, ldxq, Xs, M, Kp) || mx_overlaps(Ts, sb, Aq, Kp, As, r, Kp) ||
      overlap(Tq, tb, Ts, sb))
    return FSD_EINVAL;
  if (M == 0) return FSD_OK;
  fsd::GemmParams p;
  memset(&p, 0, sizeof(p));
  p.A0 = Xq; p.lda0 = ldxq; p.sA0 = (const uint8_t*)Xs;
  p.B0 = Aq; p.ldb0 = Kp;   p.sB0 = (const uint8_t*)As;
  p.M = M; p.N = r; p.K0 = Kp; p.K1 = 0;
  p.sMp = round_up(M, kTileM); p.sNp = round_up(r, kTileM);
  p.alpha = scale;
  p.Yq = (uint8_t*)Tq; p.ldyq = ldtq;
  p.Ys = (uint8_t*)Ts; p.sYp = round_up(M, kTileM);
  p.q0 = 0; p.q1 = r;
  return from_hip(fsd::launch_gemm(fsd::GEMM_MX_DOWN_Q, p, as_stream(stream)));
}

int fsd_mx_lora_up_q(const void* Xq, int64_t ldxq, const void* Xs, const void* W0q,
                     const void* W0s, const void* Tq, int64_t ldtq, const void* Ts,
                     const void* Bq, const void* Bs, const float* bias, const void* residual,
                     int64_t ldr, void* Y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                     int64_t r, int64_t q0, int64_t q1, void* Yq, int64_t ldyq, void* Ys,
                     void* stream) {
  if (N < 8 || q0 < 0 || q0 % 32 || q1 % 32 || q1 <= q0 || q1 > N) return FSD_EINVAL;
  const int64_t qkp = round_up(q1 - q0, 128);
  if (!Y || ldy < N || ldy % 8) return FSD_EINVAL;
  if (residual && (ldr < N || ldr % 8)) return FSD_EINVAL;
  if (!Yq || !Ys || ldyq < qkp || ldyq % 16) return FSD_EINVAL;
  if (!aligned16(Y) || (residual && !aligned16(residual)) || !aligned16(Yq) ||
      ((uintptr_t)Ys & 3u))
    return FSD_EALIGN;
  if (residual && kTileM * ldr * 2 > kMaxOffsetBytes) return FSD_EUNSUPPORTED;
  if (mx_scale_span(M, qkp) > kMaxOffsetBytes) return FSD_EUNSUPPORTED;
  const int64_t yb = span_bytes(M, N, ldy, 2);
  const int64_t qb = span_bytes(M, qkp, ldyq, 1), sb = mx_scale_span(M, qkp);
  int st = validate_mx_up_inputs(Xq, ldxq, Xs, W0q, W0s, Tq, ldtq, Ts, Bq, Bs, bias, M, N, K, r,
                                 Y, yb);
  if (st == FSD_OK)
    st = validate_mx_up_inputs(Xq, ldxq, Xs, W0q, W0s, Tq, ldtq, Ts, Bq, Bs, bias, M, N, K, r,
                               Yq, qb);
  if (st == FSD_OK)
    st = validate_mx_up_inputs(Xq, ldxq, Xs, W0q, W0s, Tq, ldtq, Ts, Bq, Bs, bias, M, N, K, r,
                               Ys, sb);
  if (st != FSD_OK) return st;
  const int64_t rb = residual ? span_bytes(M, N, ldr, 2) : 0;
  if (residual) {
    const bool same = residual == Y && ldr == ldy;
    if (!same && overlap(Y, yb, residual, rb)) return FSD_EINVAL;
  }
  if (overlap(Yq, qb, Ys, sb) || overlap(Yq, qb, Y, yb) || overlap(Ys, sb, Y, yb) ||
      overlap(Yq, qb, residual, rb) || overlap(Ys, sb, residual, rb))
    return FSD_EINVAL;
  if (M == 0) return FSD_OK;
  fsd::GemmParams p = mx_up_params(Xq, ldxq, Xs, W0q, W0s, Tq, ldtq, Ts, Bq, Bs, bias, M, N, K, r);
  p.res = (const bf16_t*)residual; p.ldr = ldr;
  p.Y = (bf16_t*)Y; p.ldy = ldy;
  p.Yq = (uint8_t*)Yq; p.ldyq = ldyq;
  p.Ys = (uint8_t*)Ys; p.sYp = round_up(M, kTileM);
  p.q0 = q0; p.q1 = q1;
  return from_hip(fsd::launch_gemm(fsd::GEMM_MX_UP_Q, p, as_stream(stream)));
}

}  // extern "C"

namespace {

// ---- the chunked MXFP8 LoRA linear -------------------------------------------
// T of one chunk in the workspace: E4M3 codes [R, rp] then their scales for R
// rows (rp = r rounded up to 128, R a multiple of 256): rp + rp/32 bytes per row.
inline int64_t mx_t_row_bytes(int64_t r) {
  const int64_t rp = round_up(r, 128);
  return rp + rp / 32;
}

// The largest chunk: 85 row tiles, and few enough rows that one chunk's T
// scales (R·rp/32 bytes) stay inside a buffer descriptor's 32-bit byte range.
inline int64_t mx_max_chunk_rows(int64_t r) {
  const int64_t rp = round_up(r, 128);
  const int64_t cap = kMaxOffsetBytes / (rp / 32) / kTileM * kTileM;
  return cap < kMxPairChunkRows ? cap : kMxPairChunkRows;
}

struct MxPlan {
  int64_t R, nc, launches;
};

// Chunks of R rows (a multiple of 256, at most mx_max_chunk_rows) through two
// halves of the workspace: launch 0 is phase A of chunk 0, launch c + 1 phase B
// of chunk c with phase A of chunk c + 1 (none after the last).  R = 0 when not
// even two 256-row chunks fit.
MxPlan make_mx_plan(int64_t M, int64_t r, int64_t ws_bytes) {
  MxPlan pl{0, 0, 0};
  if (M <= 0 || r <= 0) return pl;
  const int64_t fit = ws_bytes / mx_t_row_bytes(r);
  int64_t R = (fit / 2) / kTileM * kTileM;
  if (R > mx_max_chunk_rows(r)) R = mx_max_chunk_rows(r);
  if (R > round_up(M, kTileM)) R = round_up(M, kTileM);
  if (R < kTileM) return pl;
  pl.R = R;
  pl.nc = (M + R - 1) / R;
  pl.launches = pl.nc + 1;
  return pl;
}

struct MxLinear {
  const void* Xq; int64_t ldxq; const void* Xs;
  const void* Aq; const void* As; float scale;
  const void* W0q; const void* W0s; const void* Bq; const void* Bs;
  const float* bias; const void* residual; int64_t ldr;
  void* Y; int64_t ldy;
  int64_t M, N, K, r; int epi;
  int64_t q0, q1; void* Yq; int64_t ldyq; void* Ys;
};

int validate_mx_linear(const MxLinear& a, const void* ws, int64_t ws_bytes) {
  const bool swiglu = a.epi == FSD_EPI_SWIGLU;
  if (a.epi != FSD_EPI_NONE && !swiglu) return FSD_EINVAL;
  if (a.M < 0 || a.K < 32 || a.K % 32 || a.N < 8 || a.N % 8 || a.r < 32 || a.r % 32 ||
      !isfinite(a.scale))
    return FSD_EINVAL;
  const int64_t M = a.M, N = a.N, Kp = round_up(a.K, 128), rp = round_up(a.r, 128);
  const int64_t nout = swiglu ? N / 2 : N;
  if (swiglu) {
    if (N % 16) return FSD_EINVAL;
    if ((a.Y != nullptr) == (a.Yq != nullptr) || a.residual) return FSD_EINVAL;
    if (N % (a.Yq ? 256 : 128)) return FSD_EUNSUPPORTED;
    if (a.Yq && (a.q0 != 0 || a.q1 != nout)) return FSD_EINVAL;
  } else {
    if (!a.Y) return FSD_EINVAL;
    if (a.Yq && (a.q0 < 0 || a.q0 % 32 || a.q1 % 32 || a.q1 <= a.q0 || a.q1 > N))
      return FSD_EINVAL;
  }
  const int64_t qk = a.Yq ? a.q1 - a.q0 : 0, qkp = round_up(qk, 128);
  if (a.Y && (a.ldy < nout || a.ldy % 8)) return FSD_EINVAL;
  if (a.residual && (a.ldr < nout || a.ldr % 8)) return FSD_EINVAL;
  if (a.Yq && (!a.Ys || a.ldyq < qkp || a.ldyq % 16)) return FSD_EINVAL;
  if ((a.Y && !aligned16(a.Y)) || (a.residual && !aligned16(a.residual)) ||
      (a.Yq && (!aligned16(a.Yq) || ((uintptr_t)a.Ys & 3u))))
    return FSD_EALIGN;
  if (a.residual && kTileM * a.ldr * 2 > kMaxOffsetBytes) return FSD_EUNSUPPORTED;
  if (a.Yq && (kTileM * a.ldyq > kMaxOffsetBytes || mx_scale_span(M, qkp) > kMaxOffsetBytes))
    return FSD_EUNSUPPORTED;
  // the operands (phase B's T is the workspace: checked as an operand below)
  int st = validate_mx_operand(a.Xq, a.ldxq, a.Xs, M, Kp, false);
  if (st == FSD_OK) st = validate_mx_operand(a.Aq, Kp, a.As, a.r, Kp, true);
  if (st == FSD_OK) st = validate_mx_operand(a.W0q, Kp, a.W0s, N, Kp, true);
  if (st == FSD_OK) st = validate_mx_operand(a.Bq, rp, a.Bs, N, rp, true);
  if (st != FSD_OK) return st;
  if (a.bias && ((uintptr_t)a.bias & 3u)) return FSD_EALIGN;
  const MxPlan pl = make_mx_plan(M, a.r, ws_bytes);
  if (M > 0 && (!ws || pl.R == 0)) return FSD_EWORKSPACE;
  if (ws && !aligned16(ws)) return FSD_EALIGN;
  // outputs against every input, the workspace and each other
  const int64_t wsb = 2 * pl.R * mx_t_row_bytes(a.r);
  const void* in_p[10] = {a.Xq, a.Xs, a.Aq, a.As, a.W0q, a.W0s, a.Bq, a.Bs, a.bias, ws};
  const int64_t in_b[10] = {span_bytes(M, Kp, a.ldxq, 1), mx_scale_span(M, Kp),
                            a.r * Kp, mx_scale_span(a.r, Kp), N * Kp, mx_scale_span(N, Kp),
                            N * rp, mx_scale_span(N, rp), a.bias ? N * 4 : 0, wsb};
  const void* out_p[3] = {a.Y, a.Yq, a.Ys};
  const int64_t out_b[3] = {a.Y ? span_bytes(M, nout, a.ldy, 2) : 0,
                            a.Yq ? span_bytes(M, qkp, a.ldyq, 1) : 0,
                            a.Yq ? mx_scale_span(M, qkp) : 0};
  for (int o = 0; o < 3; ++o) {
    for (int i = 0; i < 10; ++i)
      if (overlap(out_p[o], out_b[o], in_p[i], in_b[i])) return FSD_EINVAL;
    for (int o2 = o + 1; o2 < 3; ++o2)
      if (overlap(out_p[o], out_b[o], out_p[o2], out_b[o2])) return FSD_EINVAL;
  }
  if (a.residual) {
    const int64_t rb = span_bytes(M, nout, a.ldr, 2);
    const bool same = a.residual == a.Y && a.ldr == a.ldy;
    if (!same && overlap(a.Y, out_b[0], a.residual, rb)) return FSD_EINVAL;
    if (overlap(a.Yq, out_b[1], a.residual, rb) || overlap(a.Ys, out_b[2], a.residual, rb) ||
        overlap(ws, wsb, a.residual, rb))
      return FSD_EINVAL;
  }
  for (int i = 0; i < 9; ++i)
    if (overlap(ws, wsb, in_p[i], in_b[i])) return FSD_EINVAL;
  return FSD_OK;
}

// Launch `index` of the plan (arguments already validated).
int mx_linear_launch(const MxLinear& a, void* ws, const MxPlan& pl, int64_t index, hipStream_t s) {
  if (index < 0 || index >= pl.launches) return FSD_EINVAL;
  const int64_t M = a.M, Mp = round_up(M, kTileM), Kp = round_up(a.K, 128);
  const int64_t rp = round_up(a.r, 128), R = pl.R;
  auto rows = [&](int64_t c) { return c < pl.nc ? ((M - c * R) < R ? (M - c * R) : R) : 0; };
  auto half_q = [&](int64_t c) { return (uint8_t*)ws + (c & 1) * R * mx_t_row_bytes(a.r); };
  auto half_s = [&](int64_t c) { return half_q(c) + R * rp; };
  auto chunk_down = [&](int64_t c) {
    const int64_t mc = rows(c), m = mc > 0 ? c * R : 0;
    fsd::GemmParams p;
    memset(&p, 0, sizeof(p));
    p.A0 = (const uint8_t*)a.Xq + m * a.ldxq; p.lda0 = a.ldxq;
    p.sA0 = (const uint8_t*)a.Xs; p.sa_g0 = m / 64; p.sMp = Mp;
    p.B0 = a.Aq; p.ldb0 = Kp; p.sB0 = (const uint8_t*)a.As; p.sNp = round_up(a.r, kTileM);
    p.M = mc; p.N = a.r; p.K0 = Kp; p.K1 = 0;
    p.alpha = a.scale;
    p.Yq = half_q(c); p.ldyq = rp; p.Ys = half_s(c); p.sYp = R;
    p.q0 = 0; p.q1 = a.r;
    return p;
  };
  auto chunk_up = [&](int64_t c) {
    const int64_t mc = rows(c), m = c * R;
    fsd::GemmParams p = mx_up_params((const uint8_t*)a.Xq + m * a.ldxq, a.ldxq, a.Xs, a.W0q,
                                     a.W0s, half_q(c), rp, half_s(c), a.Bq, a.Bs, a.bias, mc,
                                     a.N, a.K, a.r);
    p.sMp = Mp; p.sa_g0 = m / 64; p.sMp1 = R;
    if (a.residual) { p.res = (const bf16_t*)a.residual + m * a.ldr; p.ldr = a.ldr; }
    if (a.Y) { p.Y = (bf16_t*)a.Y + m * a.ldy; p.ldy = a.ldy; }
    if (a.Yq) {
      p.Yq = (uint8_t*)a.Yq + m * a.ldyq; p.ldyq = a.ldyq;
      p.Ys = (uint8_t*)a.Ys; p.sYp = Mp; p.sy_g0 = m / 64;
      p.q0 = a.q0; p.q1 = a.q1;
    }
    return p;
  };
  if (index == 0) return from_hip(fsd::launch_gemm(fsd::GEMM_MX_DOWN_Q, chunk_down(0), s));
  const int64_t c = index - 1;
  return from_hip(fsd::launch_gemm_pair_mx(a.epi == FSD_EPI_SWIGLU, a.Yq != nullptr,
                                           chunk_up(c), chunk_down(c + 1), s));
}

}  // namespace

extern "C" {

size_t fsd_mx_lora_linear_workspace_bytes(int64_t M, int64_t r) {
  if (M <= 0 || r <= 0) return 0;
  const int64_t cap = mx_max_chunk_rows(r);
  const int64_t rows = round_up(M, kTileM) < cap ? round_up(M, kTileM) : cap;
  return (size_t)(2 * rows * mx_t_row_bytes(r));
}

int fsd_mx_lora_linear_plan(int64_t M, int64_t r, size_t workspace_bytes, int64_t* launches,
                            int64_t* chunk_rows) {
  if (!launches || !chunk_rows) return FSD_EINVAL;
  if (M < 0 || r < 32 || r % 32 || workspace_bytes > (size_t)INT64_MAX) return FSD_EINVAL;
  const MxPlan pl = make_mx_plan(M, r, (int64_t)workspace_bytes);
  if (M > 0 && pl.R == 0) return FSD_EWORKSPACE;
  *launches = pl.launches;
  *chunk_rows = pl.R;
  return FSD_OK;
}

int fsd_mx_lora_linear_launch(const void* Xq, int64_t ldxq, const void* Xs, const void* Aq,
                              const void* As, float scale, const void* W0q, const void* W0s,
                              const void* Bq, const void* Bs, const float* bias,
                              const void* residual, int64_t ldr, void* Y, int64_t ldy, int64_t M,
                              int64_t N, int64_t K, int64_t r, int epilogue, int64_t q0,
                              int64_t q1, void* Yq, int64_t ldyq, void* Ys, void* workspace,
                              size_t workspace_bytes, int64_t index, void* stream) {
  if (workspace_bytes > (size_t)INT64_MAX) return FSD_EINVAL;
  const MxLinear a{Xq, ldxq, Xs, Aq, As, scale, W0q, W0s, Bq, Bs, bias, residual, ldr, Y, ldy,
                   M, N, K, r, epilogue, q0, q1, Yq, ldyq, Ys};
  const int st = validate_mx_linear(a, workspace, (int64_t)workspace_bytes);
  if (st != FSD_OK) return st;
  const MxPlan pl = make_mx_plan(M, r, (int64_t)workspace_bytes);
  if (M == 0) return index == 0 ? FSD_OK : FSD_EINVAL;
  return mx_linear_launch(a, workspace, pl, index, as_stream(stream));
}

int fsd_mx_lora_linear(const void* Xq, int64_t ldxq, const void* Xs, const void* Aq,
                       const void* As, float scale, const void* W0q, const void* W0s,
                       const void* Bq, const void* Bs, const float* bias, const void* residual,
                       int64_t ldr, void* Y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                       int64_t r, int epilogue, int64_t q0, int64_t q1, void* Yq, int64_t ldyq,
                       void* Ys, void* workspace, size_t workspace_bytes, void* stream) {
  if (workspace_bytes > (size_t)INT64_MAX) return FSD_EINVAL;
  const MxLinear a{Xq, ldxq, Xs, Aq, As, scale, W0q, W0s, Bq, Bs, bias, residual, ldr, Y, ldy,
                   M, N, K, r, epilogue, q0, q1, Yq, ldyq, Ys};
  const int st = validate_mx_linear(a, workspace, (int64_t)workspace_bytes);
  if (st != FSD_OK) return st;
  const MxPlan pl = make_mx_plan(M, r, (int64_t)workspace_bytes);
  for (int64_t i = 0; i < pl.launches; ++i) {
    const int e = mx_linear_launch(a, workspace, pl, i, as_stream(stream));
    if (e != FSD_OK) return e;
  }
  return FSD_OK;
}

int fsd_graph_begin(void* stream) {
  if (!stream) return FSD_EINVAL;     // the legacy default stream cannot be captured
  return from_hip(hipStreamBeginCapture(as_stream(stream), hipStreamCaptureModeThreadLocal));
}

int fsd_graph_end(void* stream, void** graph) {
  if (!stream || !graph) return FSD_EINVAL;
  *graph = nullptr;
  hipGraph_t g = nullptr;
  if (hipStreamEndCapture(as_stream(stream), &g) != hipSuccess || !g) return FSD_EHIP;
  hipGraphExec_t exec = nullptr;
  const hipError_t e = hipGraphInstantiate(&exec, g, nullptr, nullptr, 0);
  const hipError_t d = hipGraphDestroy(g);    // the instance does not need its template
  if (e != hipSuccess || !exec) return FSD_EHIP;
  if (d != hipSuccess) {
    (void)hipGraphExecDestroy(exec);
    return FSD_EHIP;
  }
  *graph = (void*)exec;
  return FSD_OK;
}

int fsd_graph_launch(void* graph, void* stream) {
  if (!graph) return FSD_EINVAL;
  return from_hip(hipGraphLaunch((hipGraphExec_t)graph, as_stream(stream)));
}

int fsd_graph_destroy(void* graph) {
  if (!graph) return FSD_OK;
  return from_hip(hipGraphExecDestroy((hipGraphExec_t)graph));
}

size_t fsd_attention_workspace_bytes(int64_t S, int64_t H, int64_t D) {
  if (S <= 0 || H <= 0 || D <= 0) return 0;
  return (size_t)(H * D * fsd::attention_padded_tokens(S) * 2);
}

int fsd_attention(const void* Q, const void* K, const void* V, int64_t ld, void* O, int64_t ldo,
                  int64_t S, int64_t H, int64_t D, float scale, void* workspace,
                  size_t workspace_bytes, void* stream) {
  if (S < 0 || H < 1 || D < 1 || !isfinite(scale) || !(scale > 0.0f)) return FSD_EINVAL;
  if (D != 128) return FSD_EUNSUPPORTED;
  if (H > 0x7fffffffLL / 128) return FSD_EINVAL;
  if (ld < H * D || ld % 8 || ldo < H * D || ldo % 8) return FSD_EINVAL;
  if (S == 0) return FSD_OK;
  if (!Q || !K || !V || !O) return FSD_EINVAL;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O)) return FSD_EALIGN;
  const int64_t Sp = fsd::attention_padded_tokens(S);
  const int64_t need = H * D * Sp * 2;
  if (!workspace || (int64_t)workspace_bytes < need) return FSD_EWORKSPACE;
  if (!aligned16(workspace)) return FSD_EALIGN;
  // 32-bit buffer offsets: a 256-row tile of Q / K / V, one head of the transpose
  if (256 * ld * 2 > kMaxOffsetBytes || D * Sp * 2 > kMaxOffsetBytes) return FSD_EUNSUPPORTED;
  if ((S + 255) / 256 * H > 0x7fffffffLL) return FSD_EUNSUPPORTED;
  const int64_t in_b = span_bytes(S, H * D, ld, 2);
  const int64_t ob = span_bytes(S, H * D, ldo, 2);
  if (overlap(O, ob, Q, in_b) || overlap(O, ob, K, in_b) || overlap(O, ob, V, in_b) ||
      overlap(O, ob, workspace, need) || overlap(workspace, need, Q, in_b) ||
      overlap(workspace, need, K, in_b) || overlap(workspace, need, V, in_b))
    return FSD_EINVAL;
  return from_hip(fsd::launch_attention((const bf16_t*)Q, (const bf16_t*)K, (const bf16_t*)V, ld,
                                        (bf16_t*)O, ldo, S, (int)H, scale, (bf16_t*)workspace,
                                        as_stream(stream)));
}

}  // extern "C"
