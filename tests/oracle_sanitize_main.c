/*
 * Sanitizer driver for the oracle (test infrastructure): links oracle.c into
 * one program, built by tests/test_oracle_sanitizers.py with AddressSanitizer
 * and UndefinedBehaviorSanitizer (abort on the first report), and calls every
 * entry point on small shapes: the merge in both forms, the LoRA linear on
 * sampled rows (bias, residual, SwiGLU, r = 0, one and three threads), the
 * double-row form, renoise / Euler / the exact-velocity sampler, embed and
 * head, and the stand-in refine and velocity.  It prints a checksum so that
 * no call is optimised away; the test only asks for a clean exit.
 */
#include "../oracle/oracle.c"

#include <stdio.h>

static uint32_t rng_state = 12345u;
static float frand(void) {               /* xorshift32, uniform in [-1, 1) */
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 17;
  rng_state ^= rng_state << 5;
  return (float)((rng_state >> 8) * (1.0 / 8388608.0)) - 1.0f;
}
static float* fvec(int64_t n, float scale) {
  float* p = (float*)malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
  for (int64_t i = 0; i < n; ++i) p[i] = scale * frand();
  return p;
}
static double sum(const double* p, int64_t n) {
  double s = 0.0;
  for (int64_t i = 0; i < n; ++i) s += p[i];
  return s;
}

int main(void) {
  double check = 0.0;
  /* merge: three adapters, both forms */
  {
    const int64_t K = 24, N = 20, ranks[3] = {6, 3, 2}, R = 11;
    float* Al[3]; float* Bl[3];
    for (int i = 0; i < 3; ++i) { Al[i] = fvec(ranks[i] * K, 0.2f); Bl[i] = fvec(N * ranks[i], 0.1f); }
    const double sc[3] = {1.0, 0.5, 2.0};
    const float scf[3] = {1.0f, 0.5f, 2.0f};
    double* A = (double*)malloc(sizeof(double) * R * K);
    double* B = (double*)malloc(sizeof(double) * N * R);
    oracle_merge(3, (const float* const*)Al, (const float* const*)Bl, ranks, sc, K, N, A, B);
    uint16_t* Ab = (uint16_t*)malloc(2 * R * K);
    uint16_t* Bb = (uint16_t*)malloc(2 * N * R);
    oracle_merge_bf16(3, (const float* const*)Al, (const float* const*)Bl, ranks, scf, K, N, Ab, Bb);
    check += sum(A, R * K) + sum(B, N * R) + oracle_bf16_value(Ab[R * K - 1]) + oracle_bf16_value(Bb[0]);
    for (int i = 0; i < 3; ++i) { free(Al[i]); free(Bl[i]); }
    free(A); free(B); free(Ab); free(Bb);
  }
  /* LoRA linear on sampled rows: every option, one and three threads */
  {
    const int64_t M = 37, K = 48, N = 40, r = 12, ldx = 56, ldr = 44;
    float* X = fvec(M * ldx, 1.0f);
    float* W0 = fvec(N * K, 0.05f);
    float* A = fvec(r * K, 0.2f);
    float* B = fvec(N * r, 0.05f);
    float* bias = fvec(N, 0.1f);
    float* res = fvec(M * ldr, 1.0f);
    const int64_t rows[5] = {0, 1, 17, 35, 36};
    double* Y = (double*)malloc(sizeof(double) * 5 * N);
    for (int threads = 1; threads <= 3; threads += 2) {
      oracle_lora_linear_rows(X, ldx, rows, 5, W0, A, B, bias, res, ldr, 0.75, N, K, r, 0, Y, threads);
      check += sum(Y, 5 * N);
      oracle_lora_linear_rows(X, ldx, rows, 5, W0, A, B, bias, NULL, 0, 1.0, N, K, r, 1, Y, threads);
      check += sum(Y, 5 * N / 2);
      oracle_lora_linear_rows(X, ldx, rows, 5, W0, NULL, NULL, NULL, NULL, 0, 1.0, N, K, 0, 0, Y, threads);
      check += sum(Y, 5 * N);
    }
    double* Xd = (double*)malloc(sizeof(double) * 3 * K);
    for (int64_t i = 0; i < 3 * K; ++i) Xd[i] = X[i];
    oracle_lora_linear_drows(Xd, K, 3, W0, A, B, 0.5, N, K, r, Y, 2);
    check += sum(Y, 3 * N);
    free(X); free(W0); free(A); free(B); free(bias); free(res); free(Y); free(Xd);
  }
  /* sampler */
  {
    const int64_t n = 96;
    float* x0 = fvec(n, 1.0f);
    float* eps = fvec(n, 1.0f);
    const double sig[4] = {0.909, 0.857, 0.667, 0.0};
    double* z = (double*)malloc(sizeof(double) * 4 * n);
    oracle_sampler_exact_velocity(x0, eps, sig, 4, z, n);
    check += sum(z, 4 * n);
    double* v = (double*)malloc(sizeof(double) * n);
    for (int64_t i = 0; i < n; ++i) v[i] = (double)eps[i] - (double)x0[i];
    oracle_renoise(x0, eps, 0.909, z, n);
    oracle_euler_step(z, v, 0.909, 0.857, n);
    check += sum(z, n);
    free(x0); free(eps); free(z); free(v);
  }
  /* embed, head and the stand-in */
  {
    const int64_t T = 5, C = 24, D = 64, F = 96;
    float* z = fvec(T * C, 1.0f);
    float* E = fvec(D * C, 0.2f);
    float* P = fvec(C * D, 0.1f);
    double* x = (double*)malloc(sizeof(double) * T * D);
    oracle_embed_rows(z, T, E, C, D, x);
    check += sum(x, T * D);
    float* H = fvec(T * (D + 8), 1.0f);
    double* vv = (double*)malloc(sizeof(double) * T * C);
    oracle_head_rows(H, T, D + 8, P, C, D, vv);
    check += sum(vv, T * C);
    const int64_t Ns[4] = {3 * D, D, 2 * F, D}, Ks[4] = {D, D, D, F}, rs[4] = {16, 8, 0, 4};
    float* mats[4][4];
    oracle_lora_layer L[4];
    for (int i = 0; i < 4; ++i) {
      mats[i][0] = fvec(Ns[i] * Ks[i], 0.05f);
      mats[i][1] = fvec(rs[i] * Ks[i], 0.1f);
      mats[i][2] = fvec(Ns[i] * rs[i], 0.05f);
      mats[i][3] = fvec(Ns[i], 0.02f);
      L[i].W0 = mats[i][0]; L[i].A = rs[i] ? mats[i][1] : NULL; L[i].B = rs[i] ? mats[i][2] : NULL;
      L[i].bias = (i == 1) ? mats[i][3] : NULL;
      L[i].N = Ns[i]; L[i].K = Ks[i]; L[i].r = rs[i]; L[i].scale = 1.0;
    }
    float* x0 = fvec(T * C, 1.0f);
    float* eps = fvec(T * C, 1.0f);
    const double sig[4] = {0.909, 0.857, 0.667, 0.0};
    double* zh = (double*)malloc(sizeof(double) * 4 * T * C);
    double* vh = (double*)malloc(sizeof(double) * 3 * T * C);
    oracle_standin_refine(x0, eps, T, sig, 4, E, P, C, D, F, L, zh, vh, 2);
    check += sum(zh, 4 * T * C) + sum(vh, 3 * T * C);
    oracle_standin_velocity(zh, T, E, P, C, D, F, L, vv);
    check += sum(vv, T * C);
    for (int i = 0; i < 4; ++i)
      for (int j = 0; j < 4; ++j) free(mats[i][j]);
    free(z); free(E); free(P); free(x); free(H); free(vv); free(x0); free(eps); free(zh); free(vh);
  }
  printf("oracle sanitizer driver ok, checksum %.6e\n", check);
  return 0;
}
