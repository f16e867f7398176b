/* The CPU oracle (oracle/pararnn_oracle.c, compiled into this file) driven through every entry point, cell,
 * storage type and option on small seeded problems, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_sanitize_cpu.py): any invalid access or undefined operation stops
 * it.  It also checks a few exact facts (Newton run T times equals the unroll; the residual of the unroll is
 * rounding level; invalid arguments are rejected), and exits nonzero on the first that fails. */
#include "../../oracle/pararnn_oracle.c"

#include <stdio.h>

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static double urand(void) { /* xorshift64*, uniform in [-1, 1) */
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return (double)((g_state * 0x2545F4914F6CDD1Dull) >> 11) / 4503599627370496.0 - 1.0;
}
static int g_checks = 0;
#define EXPECT(c)                                                                        \
  do {                                                                                   \
    ++g_checks;                                                                          \
    if (!(c)) {                                                                          \
      fprintf(stderr, "oracle_run: check failed at line %d: %s\n", __LINE__, #c);       \
      return 1;                                                                          \
    }                                                                                    \
  } while (0)

static uint16_t to_bf16(float f) { /* truncation: any bf16 pattern will do for the sanitizers */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}

static double max_abs_diff(const double* a, const double* b, int64_t n) {
  double m = 0.0;
  for (int64_t i = 0; i < n; ++i) m = fmax(m, fabs(a[i] - b[i]));
  return m;
}

static int run_cell(int cell, int dtype, int64_t B, int64_t T, int64_t D, int64_t hs, int with_s0, int with_seg,
                    int nthreads) {
  const int G = gate_count(cell), S = state_size(cell);
  const int64_t N = B * T * D, nw = cell == OR_HGRU ? 3 * D * hs : (int64_t)G * D;
  void* pre[4] = {NULL, NULL, NULL, NULL};
  for (int g = 0; g < G; ++g) {
    if (dtype == OR_BF16) {
      uint16_t* p = (uint16_t*)malloc((size_t)N * sizeof(uint16_t));
      for (int64_t i = 0; i < N; ++i) p[i] = to_bf16((float)(1.5 * urand()));
      pre[g] = p;
    } else {
      float* p = (float*)malloc((size_t)N * sizeof(float));
      for (int64_t i = 0; i < N; ++i) p[i] = (float)(cell == OR_LINEAR && g == 0 ? 0.5 + 0.4 * urand() : 1.5 * urand());
      pre[g] = p;
    }
  }
  float* w = (float*)malloc((size_t)nw * sizeof(float));
  float* bias = (float*)malloc((size_t)G * D * sizeof(float));
  float* s0 = (float*)malloc((size_t)S * B * D * sizeof(float));
  unsigned char* seg = (unsigned char*)calloc((size_t)T, 1);
  float* g = (float*)malloc((size_t)N * sizeof(float));
  for (int64_t i = 0; i < nw; ++i) w[i] = (float)(0.5 * urand() / (cell == OR_HGRU ? sqrt((double)hs) : 1.0));
  for (int64_t i = 0; i < (int64_t)G * D; ++i) bias[i] = (float)(0.1 * urand());
  for (int64_t i = 0; i < (int64_t)S * B * D; ++i) s0[i] = (float)(0.5 * urand());
  if (cell == OR_SLSTM)
    for (int64_t i = 0; i < B * D; ++i) s0[B * D + i] = (float)(1.0 + 0.5 * urand()); /* n > 0 */
  for (int64_t t = 5; t < T; t += 11) seg[t] = 1;
  for (int64_t i = 0; i < N; ++i) g[i] = (float)urand();
  or_problem p;
  memset(&p, 0, sizeof p);
  p.cell = cell; p.dtype = dtype; p.B = B; p.T = T; p.D = D;
  for (int k = 0; k < 4; ++k) p.pre[k] = pre[k];
  p.w = w; p.bias = bias; p.s0 = with_s0 ? s0 : NULL; p.seg_start = with_seg ? seg : NULL;
  p.head_size = hs;
  const int64_t n = (int64_t)S * N;
  double* U = (double*)malloc((size_t)n * sizeof(double));
  double* H = (double*)malloc((size_t)n * sizeof(double));
  double resid[66], R = -1.0;
  int iters = 0, conv = 0;
  EXPECT(or_unroll(&p, U, nthreads) == OR_OK);
  EXPECT(or_residual(&p, U, &R, nthreads) == OR_OK && R <= 1e-12);
  if (cell != OR_SLSTM) {
    /* triangular exactness: T updates from the zero guess give the unroll */
    int K = (int)(T < 64 ? T : 64);
    int rc = or_newton(&p, NULL, 0, 0, K, 0.0, H, resid, &iters, &conv, nthreads);
    EXPECT(rc == OR_OK && iters == K);
    if (K == T) EXPECT(max_abs_diff(H, U, n) <= 1e-10);
  }
  int rc = or_newton(&p, NULL, 1, 2, 12, 1e-9, H, resid, &iters, &conv, nthreads);   /* warm, Picard, tol */
  EXPECT(rc == OR_OK || rc == OR_DIVERGED);
  float* guess = (float*)malloc((size_t)n * sizeof(float));
  for (int64_t i = 0; i < n; ++i) guess[i] = (float)U[i];
  rc = or_newton(&p, guess, 0, 0, 2, 1e-5, H, resid, &iters, &conv, nthreads);
  EXPECT(rc == OR_OK && iters == 1 && conv);
  double* d_pre = (double*)malloc((size_t)G * N * sizeof(double));
  double* d_w = (double*)malloc((size_t)nw * sizeof(double));
  double* d_bias = (double*)malloc((size_t)G * D * sizeof(double));
  double* d_s0 = (double*)malloc((size_t)S * B * D * sizeof(double));
  double* lam = (double*)malloc((size_t)n * sizeof(double));
  EXPECT(or_vjp(&p, U, g, d_pre, d_w, d_bias, d_s0, lam, nthreads) == OR_OK);
  EXPECT(or_vjp(&p, U, g, d_pre, d_w, d_bias, NULL, NULL, nthreads) == OR_OK);
  free(guess); free(d_pre); free(d_w); free(d_bias); free(d_s0); free(lam);
  free(U); free(H);
  for (int k = 0; k < 4; ++k) free(pre[k]);
  free(w); free(bias); free(s0); free(seg); free(g);
  return 0;
}

static int run_linear(int S, int dtype, int64_t B, int64_t T, int64_t D, int reverse, int with_s0, int with_seg) {
  const int64_t N = B * T * D, na = (S == 2 ? 4 : 1) * N, nb = (int64_t)S * N;
  const size_t esz = dtype == OR_BF16 ? 2 : 4;
  unsigned char* a = (unsigned char*)malloc((size_t)na * esz);
  unsigned char* b = (unsigned char*)malloc((size_t)nb * esz);
  for (int64_t i = 0; i < na; ++i) {
    float v = (float)(0.45 * urand());
    if (dtype == OR_BF16) ((uint16_t*)a)[i] = to_bf16(v); else ((float*)a)[i] = v;
  }
  for (int64_t i = 0; i < nb; ++i) {
    float v = (float)urand();
    if (dtype == OR_BF16) ((uint16_t*)b)[i] = to_bf16(v); else ((float*)b)[i] = v;
  }
  float* s0 = (float*)malloc((size_t)S * B * D * sizeof(float));
  for (int64_t i = 0; i < (int64_t)S * B * D; ++i) s0[i] = (float)urand();
  unsigned char* seg = (unsigned char*)calloc((size_t)T, 1);
  for (int64_t t = 3; t < T; t += 7) seg[t] = 1;
  double* out = (double*)malloc((size_t)nb * sizeof(double));
  EXPECT(or_linear_scan(S, B, T, D, dtype, a, b, with_s0 ? s0 : NULL, with_seg ? seg : NULL, reverse, out, 3) ==
         OR_OK);
  free(a); free(b); free(s0); free(seg); free(out);
  return 0;
}

int main(void) {
  for (int cell = OR_LINEAR; cell <= OR_HGRU; ++cell)
    for (int dtype = OR_F32; dtype <= OR_BF16; ++dtype)
      for (int v = 0; v < 4; ++v) {
        const int64_t hs = cell == OR_HGRU ? 4 : 1;
        if (run_cell(cell, dtype, 2, v == 3 ? 40 : 23, cell == OR_HGRU ? 8 : 6, hs, v & 1, (v >> 1) & 1, 1 + v))
          return 1;
      }
  for (int S = 1; S <= 2; ++S)
    for (int dtype = OR_F32; dtype <= OR_BF16; ++dtype)
      for (int v = 0; v < 8; ++v)
        if (run_linear(S, dtype, 2, 29, 5, v & 1, (v >> 1) & 1, (v >> 2) & 1)) return 1;
  /* empty problems and invalid arguments */
  {
    or_problem p;
    memset(&p, 0, sizeof p);
    p.cell = OR_GRU; p.B = 1; p.T = 0; p.D = 4;
    float wz[12] = {0};
    p.w = wz; p.bias = wz;
    double H[1], resid[4], R = 0.0;
    int it = 0, cv = 0;
    EXPECT(or_unroll(&p, H, 2) == OR_OK);
    EXPECT(or_residual(&p, H, &R, 2) == OR_OK && R == 0.0);
    EXPECT(or_newton(&p, NULL, 0, 0, 3, 0.0, H, resid, &it, &cv, 2) == OR_OK);
    EXPECT(or_newton(&p, NULL, 0, 0, 0, 0.0, H, resid, &it, &cv, 2) == OR_EINVAL);
    p.cell = 9;
    EXPECT(or_unroll(&p, H, 1) == OR_EINVAL);
    p.cell = OR_HGRU; p.head_size = 3;
    EXPECT(or_unroll(&p, H, 1) == OR_EINVAL);
    p.cell = OR_GRU; p.dtype = 5;
    EXPECT(or_unroll(&p, H, 1) == OR_EINVAL);
    p.dtype = OR_F32; p.T = -1;
    EXPECT(or_unroll(&p, H, 1) == OR_EINVAL);
    EXPECT(or_unroll(NULL, H, 1) == OR_EINVAL);
    EXPECT(or_linear_scan(3, 1, 4, 4, OR_F32, H, H, NULL, NULL, 0, H, 1) == OR_EINVAL);
  }
  {
    double u[4] = {0.3, -0.2, 0.7, 0.1}, wv[4] = {0.2, -0.3, 0.4, 0.1}, bv[4] = {0.0, 1.0, 0.0, 0.0};
    double s[4] = {0.1, 1.2, -0.3, 0.2}, sn[4], J[16], dfdu[16], wc[4];
    for (int cell = OR_LINEAR; cell <= OR_SLSTM; ++cell)
      EXPECT(or_cell_step(cell, u, wv, bv, s, sn, J, dfdu, wc) == OR_OK);
    double A[3 * 16 * 16], uh[3 * 16], bh[3 * 16], h[16], hn[16], Jh[256], dz[16], dc[16], dr[256], rh[16];
    for (int i = 0; i < 3 * 16 * 16; ++i) A[i] = 0.1 * urand();
    for (int i = 0; i < 48; ++i) { uh[i] = urand(); bh[i] = 0.1 * urand(); }
    for (int i = 0; i < 16; ++i) h[i] = 0.5 * urand();
    EXPECT(or_hgru_step(16, uh, A, bh, h, hn, Jh, dz, dc, dr, rh) == OR_OK);
    EXPECT(or_hgru_step(0, uh, A, bh, h, hn, Jh, dz, dc, dr, rh) == OR_EINVAL);
  }
  EXPECT(or_abi_version() == 7);
  printf("oracle_run: %d checks passed\n", g_checks);
  return 0;
}
