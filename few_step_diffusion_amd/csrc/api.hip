// C ABI of libfsd.so (include/fsd.h): argument validation, M-chunking of the
// LoRA linear through the caller's workspace, and kernel launches.
//
// Every entry point validates all arguments before it makes any HIP call, so
// an invalid request returns its status without touching the device.  The
// library keeps no state and never allocates, frees or synchronises.
#include <math.h>
#include <string.h>

#include "../../include/fsd.h"
#include "fsd_internal.h"

using fsd::bf16_t;

namespace {

constexpr int64_t kTileM = 256;            // rows per GEMM tile: the chunk granule
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

const char* fsd_status_str(int status) {
  switch (status) {
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
  return (size_t)M * (size_t)r * 2u;
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

int fsd_lora_linear(const void* X, int64_t ldx, const void* W0, const void* A, const void* B,
                    const float* bias, const void* residual, int64_t ldr, float scale, void* Y,
                    int64_t ldy, int64_t M, int64_t N, int64_t K, int64_t r, int epilogue,
                    void* workspace, size_t workspace_bytes, void* stream) {
  UpShape a{X, W0, workspace, B, ldx, r, bias, residual, ldr, Y, ldy, M, N, K, r, epilogue};
  int st = validate_up(a, false);
  if (st != FSD_OK) return st;
  if (!isfinite(scale)) return FSD_EINVAL;
  int64_t chunk = M;
  if (r > 0) {
    if (!A) return FSD_EINVAL;
    if (!aligned16(A)) return FSD_EALIGN;
    if ((r + kTileM) * K * 2 > kMaxOffsetBytes) return FSD_EUNSUPPORTED;
    const int64_t need_min = (M < kTileM ? M : kTileM) * r * 2;
    if (M > 0 && (!workspace || (int64_t)workspace_bytes < need_min)) return FSD_EWORKSPACE;
    if (workspace && !aligned16(workspace)) return FSD_EALIGN;
    const int64_t fit = (int64_t)(workspace_bytes / (size_t)(r * 2));
    if (fit < M) chunk = (fit / kTileM) * kTileM;
    if (M > 0 && chunk < 1) return FSD_EWORKSPACE;
    const int64_t nout = epilogue == FSD_EPI_SWIGLU ? N / 2 : N;
    const int64_t wbytes = (chunk < M ? chunk : M) * r * 2;
    if (overlap(Y, span_bytes(M, nout, ldy, 2), workspace, wbytes) ||
        overlap(workspace, wbytes, X, span_bytes(M, K, ldx, 2)) ||
        overlap(workspace, wbytes, W0, N * K * 2) || overlap(workspace, wbytes, A, r * K * 2) ||
        overlap(workspace, wbytes, B, N * r * 2) ||
        overlap(workspace, wbytes, bias, bias ? N * 4 : 0) ||
        overlap(workspace, wbytes, residual, residual ? span_bytes(M, nout, ldr, 2) : 0))
      return FSD_EINVAL;
  }
  if (M == 0) return FSD_OK;
  hipStream_t s = as_stream(stream);
  const fsd::GemmKind kind = epilogue == FSD_EPI_SWIGLU ? fsd::GEMM_UP_SWIGLU : fsd::GEMM_UP;
  for (int64_t m = 0; m < M; m += chunk) {
    const int64_t mc = (M - m) < chunk ? (M - m) : chunk;
    const bf16_t* Xc = (const bf16_t*)X + m * ldx;
    if (r > 0) {
      const hipError_t e = fsd::launch_gemm(
          fsd::GEMM_DOWN, down_params(Xc, ldx, A, scale, workspace, r, mc, K, r), s);
      if (e != hipSuccess) return FSD_EHIP;
    }
    UpShape c = a;
    c.X = Xc;
    c.M = mc;
    c.Y = (bf16_t*)Y + m * ldy;
    if (residual) c.residual = (const bf16_t*)residual + m * ldr;
    const hipError_t e = fsd::launch_gemm(kind, up_params(c), s);
    if (e != hipSuccess) return FSD_EHIP;
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
