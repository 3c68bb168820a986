/*
 * oracle.c — plain, slow, fp64 CPU reference of the refiner's hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library; the two meet only through
 * data.  Every function widens its inputs to double and keeps every
 * intermediate in double: no blocking, no reordering, no intermediate
 * rounding.  The only rounding functions (oracle_bf16_*) exist to define the
 * bit-exact result of the adapter merge.
 *
 * Sources:
 *   [EN] "Open-H3-Regenerate-2K: High-Resolution Video Refinement with
 *        Few-Step Diffusion" (agientry.com, English article)
 *   [CW] "Open-H3-Regenerate-2K：MiniMax H3 的开源 4K 精修方案"
 *        (comfyui-wiki.com news page)
 *
 * Parity pins (tests that tie this file to something other than itself) are
 * listed next to each function.  The velocity stand-in (oracle_standin_*) is
 * a synthetic block the pages do not describe: its composition is pinned only
 * through special cases (parity partially unpinned).
 *
 * Build: gcc -O2 -std=c11 -fPIC -shared oracle.c -o liboracle.so -lm -lpthread
 * (no -ffast-math: every sum is evaluated left to right as written).
 */
#define _GNU_SOURCE
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

int oracle_version(void) { return 1; }

/* ------------------------------------------------------------------ */
/* bfloat16 round-to-nearest-even, defined on the IEEE binary32 bits.  */
/* Pinned against torch's CPU float->bfloat16 cast on random and edge  */
/* values (tests).                                                      */
/* ------------------------------------------------------------------ */
uint16_t oracle_bf16_bits(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0) {
    return (uint16_t)((u >> 16) | 0x0040u); /* NaN stays a (quiet) NaN */
  }
  uint32_t lower = u & 0xffffu;     /* the 16 bits that are dropped */
  uint32_t upper = u >> 16;
  /* Round half to even: above the half-way point round up; at exactly the
     half-way point round up only when the kept part is odd. */
  if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;
  return (uint16_t)upper;
}

float oracle_bf16_value(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* ------------------------------------------------------------------ */
/* a0. Rank-axis merge ([CW] section "三个步如何完成工作").             */
/* A = [A_0; A_1; ...] stacks the down factors' rows; B = [s_0 B_0 |    */
/* s_1 B_1 | ...] stacks the up factors' columns, so that               */
/* B·A = sum_i s_i B_i·A_i (block matrix product).                      */
/* Pins: B·A equals the sum of the separate adapter deltas (checked     */
/* with numpy's matmul), the pages' fp32 merge error, concat order.     */
/* ------------------------------------------------------------------ */
void oracle_merge(int n_adapters, const float* const* A_list,
                  const float* const* B_list, const int64_t* ranks,
                  const double* scales, int64_t K, int64_t N, double* A_out,
                  double* B_out) {
  int64_t R = 0;
  for (int i = 0; i < n_adapters; ++i) R += ranks[i];
  int64_t row0 = 0;
  for (int i = 0; i < n_adapters; ++i) {
    const double s = scales ? scales[i] : 1.0;
    for (int64_t j = 0; j < ranks[i]; ++j)
      for (int64_t k = 0; k < K; ++k)
        A_out[(row0 + j) * K + k] = (double)A_list[i][j * K + k];
    for (int64_t n = 0; n < N; ++n)
      for (int64_t j = 0; j < ranks[i]; ++j)
        B_out[n * R + row0 + j] = s * (double)B_list[i][n * ranks[i] + j];
    row0 += ranks[i];
  }
}

/* The merge's bit-exact storage form: each element is s_i*b rounded once
   to binary32 (the product of two binary32 values is exact in double, so
   the cast is the single IEEE rounding), then rounded to bfloat16. */
void oracle_merge_bf16(int n_adapters, const float* const* A_list,
                       const float* const* B_list, const int64_t* ranks,
                       const float* scales, int64_t K, int64_t N,
                       uint16_t* A_out, uint16_t* B_out) {
  int64_t R = 0;
  for (int i = 0; i < n_adapters; ++i) R += ranks[i];
  int64_t row0 = 0;
  for (int i = 0; i < n_adapters; ++i) {
    const float s = scales ? scales[i] : 1.0f;
    for (int64_t j = 0; j < ranks[i]; ++j)
      for (int64_t k = 0; k < K; ++k)
        A_out[(row0 + j) * K + k] = oracle_bf16_bits(A_list[i][j * K + k]);
    for (int64_t n = 0; n < N; ++n)
      for (int64_t j = 0; j < ranks[i]; ++j) {
        const float p = (float)((double)s * (double)B_list[i][n * ranks[i] + j]);
        B_out[n * R + row0 + j] = oracle_bf16_bits(p);
      }
    row0 += ranks[i];
  }
}

/* ------------------------------------------------------------------ */
/* LoRA-adapted linear on one row, fp64 throughout.                      */
/*   t = x·Aᵀ                       (r values)                           */
/*   y[n] = x·W0[n]ᵀ + s·t·B[n]ᵀ + bias[n]                                */
/* x is a double row of length K; W0 [N,K], A [r,K], B [N,r] hold bf16  */
/* values widened to float.  Pins: exact rational arithmetic on micro   */
/* shapes, numpy float64 matmul, X = I revealing W0 + s·B·A, s = 0 and   */
/* r = 0 reducing to x·W0ᵀ.                                              */
/* ------------------------------------------------------------------ */
static void lora_row(const double* x, int64_t K, const float* W0,
                     const float* A, const float* B, const float* bias,
                     double s, int64_t N, int64_t r, double* t, double* y) {
  for (int64_t j = 0; j < r; ++j) {
    double acc = 0.0;
    const float* a = A + j * K;
    for (int64_t k = 0; k < K; ++k) acc += x[k] * (double)a[k];
    t[j] = acc;
  }
  for (int64_t n = 0; n < N; ++n) {
    double base = 0.0;
    const float* w = W0 + n * K;
    for (int64_t k = 0; k < K; ++k) base += x[k] * (double)w[k];
    double low = 0.0;
    const float* b = B + n * r;
    for (int64_t j = 0; j < r; ++j) low += t[j] * (double)b[j];
    y[n] = base + s * low + (bias ? (double)bias[n] : 0.0);
  }
}

/* SwiGLU (Shazeer, "GLU Variants Improve Transformer", 2020): the row is
   read as [G | U] halves, F = N/2, h[j] = silu(G[j])·U[j] with
   silu(g) = g·sigmoid(g) = g / (1 + exp(-g)).  Pins: silu(0) = 0,
   silu(1) = 1/(1+e^-1), silu(g) -> g for large g, -> 0 for very negative g. */
static void swiglu_row(const double* y, int64_t F, double* h) {
  for (int64_t j = 0; j < F; ++j) {
    const double g = y[j];
    const double u = y[F + j];
    h[j] = g / (1.0 + exp(-g)) * u;
  }
}

/* ------------------------------------------------------------------ */
/* Thread pool helper: run fn(i, ctx) for i in [0, count) on nthreads.  */
/* Each index is independent; threads only split the index range.       */
/* ------------------------------------------------------------------ */
typedef void (*index_fn)(int64_t i, void* ctx, double* scratch);
typedef struct {
  index_fn fn;
  void* ctx;
  int64_t begin, end;
  int64_t scratch_len;
} span_t;

static void* run_span(void* p) {
  span_t* sp = (span_t*)p;
  double* scratch = (double*)malloc(sizeof(double) * (size_t)(sp->scratch_len > 0 ? sp->scratch_len : 1));
  for (int64_t i = sp->begin; i < sp->end; ++i) sp->fn(i, sp->ctx, scratch);
  free(scratch);
  return NULL;
}

static int resolve_threads(int nthreads) {
  if (nthreads > 0) return nthreads;
  long c = sysconf(_SC_NPROCESSORS_ONLN);
  return c > 0 ? (int)c : 1;
}

static void parallel_for(int64_t count, int nthreads, int64_t scratch_len,
                         index_fn fn, void* ctx) {
  nthreads = resolve_threads(nthreads);
  if (nthreads > count) nthreads = (int)(count > 0 ? count : 1);
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  span_t* sp = (span_t*)malloc(sizeof(span_t) * (size_t)nthreads);
  for (int t = 0; t < nthreads; ++t) {
    sp[t].fn = fn;
    sp[t].ctx = ctx;
    sp[t].begin = count * t / nthreads;
    sp[t].end = count * (t + 1) / nthreads;
    sp[t].scratch_len = scratch_len;
  }
  for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, run_span, &sp[t]);
  run_span(&sp[0]);
  for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
  free(th);
  free(sp);
}

/* ------------------------------------------------------------------ */
/* a2-a4. LoRA linear on selected rows of X.                             */
/* X rows are taken as given (float values of bf16 inputs, or any       */
/* double-representable values); residual (optional) is [M, Nout] with  */
/* row stride ldr.  swiglu != 0 returns F = N/2 columns per row.         */
/* Y_out: double [nrows, Nout].                                          */
/* ------------------------------------------------------------------ */
typedef struct {
  const float* X; int64_t ldx; const int64_t* rows;
  const float *W0, *A, *B, *bias, *residual; int64_t ldr;
  double s; int64_t N, K, r; int swiglu; double* Y;
} lora_rows_ctx;

static void lora_rows_one(int64_t i, void* p, double* scratch) {
  lora_rows_ctx* c = (lora_rows_ctx*)p;
  const int64_t m = c->rows ? c->rows[i] : i;
  double* x = scratch;               /* K */
  double* t = x + c->K;              /* r */
  double* y = t + (c->r > 0 ? c->r : 1); /* N */
  for (int64_t k = 0; k < c->K; ++k) x[k] = (double)c->X[m * c->ldx + k];
  lora_row(x, c->K, c->W0, c->A, c->B, c->bias, c->s, c->N, c->r, t, y);
  const int64_t nout = c->swiglu ? c->N / 2 : c->N;
  double* out = c->Y + i * nout;
  if (c->swiglu) swiglu_row(y, c->N / 2, out);
  else memcpy(out, y, sizeof(double) * (size_t)nout);
  if (c->residual)
    for (int64_t n = 0; n < nout; ++n) out[n] += (double)c->residual[m * c->ldr + n];
}

void oracle_lora_linear_rows(const float* X, int64_t ldx, const int64_t* rows,
                             int64_t nrows, const float* W0, const float* A,
                             const float* B, const float* bias,
                             const float* residual, int64_t ldr, double scale,
                             int64_t N, int64_t K, int64_t r, int swiglu,
                             double* Y_out, int nthreads) {
  lora_rows_ctx c = {X, ldx, rows, W0, A, B, bias, residual, ldr,
                     scale, N, K, r, swiglu, Y_out};
  parallel_for(nrows, nthreads, K + (r > 0 ? r : 1) + N, lora_rows_one, &c);
}

/* Same linear map applied to double-precision rows (used to evaluate
   Freivalds' identity w·Y = (w·X)·W0ᵀ + s((w·X)·Aᵀ)·Bᵀ on a row that is
   itself a combination of input rows; no bias). */
typedef struct {
  const double* X; int64_t ldx;
  const float *W0, *A, *B; double s; int64_t N, K, r; double* Y;
} lora_drows_ctx;

static void lora_drows_one(int64_t i, void* p, double* scratch) {
  lora_drows_ctx* c = (lora_drows_ctx*)p;
  lora_row(c->X + i * c->ldx, c->K, c->W0, c->A, c->B, NULL, c->s, c->N, c->r, scratch,
           c->Y + i * c->N);
}

void oracle_lora_linear_drows(const double* X, int64_t ldx, int64_t nrows,
                              const float* W0, const float* A, const float* B,
                              double scale, int64_t N, int64_t K, int64_t r,
                              double* Y_out, int nthreads) {
  lora_drows_ctx c = {X, ldx, W0, A, B, scale, N, K, r, Y_out};
  parallel_for(nrows, nthreads, r > 0 ? r : 1, lora_drows_one, &c);
}

/* ------------------------------------------------------------------ */
/* a1. Renoise ([EN] section "Three steps instead of dozens", renoise   */
/* equation): z = (1 - sigma)·u + sigma·eps.                             */
/* Pins: sigma = 0 gives u, sigma = 1 gives eps; the Euler closed form. */
/* ------------------------------------------------------------------ */
void oracle_renoise(const float* u, const float* eps, double sigma, double* z,
                    int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    z[i] = (1.0 - sigma) * (double)u[i] + sigma * (double)eps[i];
}

/* ------------------------------------------------------------------ */
/* a5. Euler update ([EN] same section, schedule and update equation):  */
/*   z <- z + (sigma_next - sigma)·v.                                    */
/* Pin: with the flow-matching pair z_sigma = (1-sigma)x0 + sigma·eps,   */
/* v = eps - x0 ([EN] section "Training: learn what degradation         */
/* removed"), each step lands on z_{sigma_next} and the last on x0.      */
/* ------------------------------------------------------------------ */
void oracle_euler_step(double* z, const double* v, double sigma,
                       double sigma_next, int64_t n) {
  const double d = sigma_next - sigma;
  for (int64_t i = 0; i < n; ++i) z[i] = z[i] + d * v[i];
}

/* The whole sampler with the exact flow-matching velocity v = eps - x0:
   renoise at sigmas[0], then one Euler step per consecutive pair.
   z_hist: double [nsig, n]; row k is z after reaching sigmas[k]. */
void oracle_sampler_exact_velocity(const float* x0, const float* eps,
                                   const double* sigmas, int nsig,
                                   double* z_hist, int64_t n) {
  oracle_renoise(x0, eps, sigmas[0], z_hist, n);
  double* v = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  for (int64_t i = 0; i < n; ++i) v[i] = (double)eps[i] - (double)x0[i];
  for (int k = 1; k < nsig; ++k) {
    double* z = z_hist + (int64_t)k * n;
    memcpy(z, z_hist + (int64_t)(k - 1) * n, sizeof(double) * (size_t)n);
    oracle_euler_step(z, v, sigmas[k - 1], sigmas[k], n);
  }
  free(v);
}

/* ------------------------------------------------------------------ */
/* Velocity stand-in (synthetic; the pages give no transformer widths). */
/* Per token (one latent voxel, C channels):                             */
/*   x  = z·Eᵀ                       (D)      E [D, C]                   */
/*   q  = L_qkv(x)                   (3D)     output split [Q | K | V]    */
/*   h  = x + L_o(q[2D:3D])          (D)      attention reads only self  */
/*   h  = h + L_down(SwiGLU(L_gu(h)))         L_gu: D -> 2F, L_down: F -> D */
/*   v  = h·Pᵀ                       (C)      P [C, D]                   */
/* then the Euler update.  Every L_* is the LoRA linear above.           */
/* Pins: zero sublayers collapse it to v = z·(P·E)ᵀ; tokens are          */
/* independent (row permutation).                                        */
/* ------------------------------------------------------------------ */
/* Stand-in projections between the C-channel latent and width D:
   embed x[n] = sum_c z[c]·E[n, c] (E [D, C]); head v[c] = sum_n h[n]·P[c, n]
   (P [C, D]).  Pins: zero sublayers reduce the stand-in to z·(P·E)ᵀ. */
static void embed_row(const double* z, const float* E, int64_t C, int64_t D, double* x) {
  for (int64_t n = 0; n < D; ++n) {
    double acc = 0.0;
    for (int64_t ch = 0; ch < C; ++ch) acc += z[ch] * (double)E[n * C + ch];
    x[n] = acc;
  }
}

static void head_row(const double* h, const float* P, int64_t C, int64_t D, double* v) {
  for (int64_t ch = 0; ch < C; ++ch) {
    double acc = 0.0;
    for (int64_t n = 0; n < D; ++n) acc += h[n] * (double)P[ch * D + n];
    v[ch] = acc;
  }
}

/* Pins: exact rational sums on tiny shapes (C = 1, 24, 32, 70) and numpy
   float64 products (tests/test_oracle_pins.py). */
void oracle_embed_rows(const float* z, int64_t ntok, const float* E, int64_t C, int64_t D,
                       double* x_out) {
  double* zr = (double*)malloc(sizeof(double) * (size_t)(C > 0 ? C : 1));
  for (int64_t i = 0; i < ntok; ++i) {
    for (int64_t ch = 0; ch < C; ++ch) zr[ch] = (double)z[i * C + ch];
    embed_row(zr, E, C, D, x_out + i * D);
  }
  free(zr);
}

/* Rows of H have stride ldh >= D; only their first D entries are read.  Pins:
   exact rational sums on tiny shapes, ldh = D and ldh > D with non-finite
   values in the skipped columns (tests/test_oracle_pins.py). */
void oracle_head_rows(const float* H, int64_t ntok, int64_t ldh, const float* P, int64_t C,
                      int64_t D, double* v_out) {
  double* h = (double*)malloc(sizeof(double) * (size_t)D);
  for (int64_t i = 0; i < ntok; ++i) {
    for (int64_t n = 0; n < D; ++n) h[n] = (double)H[i * ldh + n];
    head_row(h, P, C, D, v_out + i * C);
  }
  free(h);
}

typedef struct {
  const float *W0, *A, *B, *bias;
  int64_t N, K, r;
  double scale;
} oracle_lora_layer;

typedef struct {
  const float* x0;  const float* eps;  /* [T, C] rows of the sampled tokens */
  const double* sigmas; int nsig;
  const float* E; const float* P; int64_t C, D, F;
  oracle_lora_layer L[4];              /* qkv, o, gate/up, down */
  double* z_hist;                      /* [nsig, T, C] */
  double* v_hist;                      /* [nsig-1, T, C] */
  int64_t ntok;
} standin_ctx;

static void standin_velocity(const standin_ctx* c, const double* z, double* v,
                             double* ws) {
  const int64_t C = c->C, D = c->D, F = c->F;
  double* x = ws;                 /* D   */
  double* q = x + D;              /* 3D  */
  double* h = q + 3 * D;          /* D   */
  double* o = h + D;              /* D   */
  double* gu = o + D;             /* 2F  */
  double* g = gu + 2 * F;         /* F   */
  double* t = g + F;              /* max r */
  embed_row(z, c->E, C, D, x);
  const oracle_lora_layer* L = c->L;
  lora_row(x, D, L[0].W0, L[0].A, L[0].B, L[0].bias, L[0].scale, 3 * D, L[0].r, t, q);
  lora_row(q + 2 * D, D, L[1].W0, L[1].A, L[1].B, L[1].bias, L[1].scale, D, L[1].r, t, o);
  for (int64_t n = 0; n < D; ++n) h[n] = x[n] + o[n];
  lora_row(h, D, L[2].W0, L[2].A, L[2].B, L[2].bias, L[2].scale, 2 * F, L[2].r, t, gu);
  swiglu_row(gu, F, g);
  lora_row(g, F, L[3].W0, L[3].A, L[3].B, L[3].bias, L[3].scale, D, L[3].r, t, o);
  for (int64_t n = 0; n < D; ++n) h[n] = h[n] + o[n];
  head_row(h, c->P, C, D, v);
}

static void standin_token(int64_t i, void* p, double* ws) {
  standin_ctx* c = (standin_ctx*)p;
  const int64_t C = c->C, T = c->ntok;
  double* z = c->z_hist + i * C;   /* row k at z_hist + (k*T + i)*C */
  oracle_renoise(c->x0 + i * C, c->eps + i * C, c->sigmas[0], z, C);
  for (int k = 1; k < c->nsig; ++k) {
    const double* zp = c->z_hist + ((int64_t)(k - 1) * T + i) * C;
    double* zn = c->z_hist + ((int64_t)k * T + i) * C;
    double* v = c->v_hist + ((int64_t)(k - 1) * T + i) * C;
    standin_velocity(c, zp, v, ws);
    memcpy(zn, zp, sizeof(double) * (size_t)C);
    oracle_euler_step(zn, v, c->sigmas[k - 1], c->sigmas[k], C);
  }
}

/* layers: 4 entries (qkv, o, gate/up, down) with N/K/r filled in by the
   caller: qkv N=3D K=D; o N=D K=D; gate/up N=2F K=D; down N=D K=F. */
void oracle_standin_refine(const float* x0, const float* eps, int64_t ntok,
                           const double* sigmas, int nsig, const float* E,
                           const float* P, int64_t C, int64_t D, int64_t F,
                           const oracle_lora_layer* layers, double* z_hist,
                           double* v_hist, int nthreads) {
  standin_ctx c;
  c.x0 = x0; c.eps = eps; c.sigmas = sigmas; c.nsig = nsig;
  c.E = E; c.P = P; c.C = C; c.D = D; c.F = F;
  int64_t rmax = 1;
  for (int i = 0; i < 4; ++i) {
    c.L[i] = layers[i];
    if (layers[i].r > rmax) rmax = layers[i].r;
  }
  c.z_hist = z_hist; c.v_hist = v_hist; c.ntok = ntok;
  parallel_for(ntok, nthreads, 6 * D + 3 * F + rmax, standin_token, &c);
}

/* The stand-in's velocity alone for given latent rows (double in). */
void oracle_standin_velocity(const double* z, int64_t ntok, const float* E,
                             const float* P, int64_t C, int64_t D, int64_t F,
                             const oracle_lora_layer* layers, double* v_out) {
  standin_ctx c;
  memset(&c, 0, sizeof(c));
  c.E = E; c.P = P; c.C = C; c.D = D; c.F = F;
  int64_t rmax = 1;
  for (int i = 0; i < 4; ++i) {
    c.L[i] = layers[i];
    if (layers[i].r > rmax) rmax = layers[i].r;
  }
  double* ws = (double*)malloc(sizeof(double) * (size_t)(6 * D + 3 * F + rmax));
  for (int64_t i = 0; i < ntok; ++i) standin_velocity(&c, z + i * C, v_out + i * C, ws);
  free(ws);
}
