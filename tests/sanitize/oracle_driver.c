/*
 * Test driver: runs every entry point of oracle/ssd_oracle.c on small
 * problems (ragged chunks, groups, an initial state, packed sequences, the
 * gradients) under AddressSanitizer and UndefinedBehaviorSanitizer, plus the
 * shape rejections.  Built and run by tests/test_sanitizers.py; exits 0 when
 * every call returned what it should (the sanitizers abort on a finding).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_max_threads(int nthreads);
int oracle_ssd_fwd(const float* x, const float* dt_raw, const float* A, const float* B,
                   const float* C, const float* D, const float* z, const float* dt_bias,
                   double dt_min, double dt_max, const double* init, double* out,
                   double* final_states, const int32_t* seq_idx, int64_t batch,
                   int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate,
                   int64_t ngroups, const unsigned char* head_mask, int nthreads);
int oracle_ssd_chunk_intermediates(const float* x, const float* dt_raw, const float* A,
                                   const float* B, const float* dt_bias, double dt_min,
                                   double dt_max, const double* init, double* dt_out,
                                   double* cum_out, double* chunk_states, double* states_in,
                                   const int32_t* seq_idx, int64_t batch, int64_t seqlen,
                                   int64_t nheads, int64_t headdim, int64_t dstate,
                                   int64_t ngroups, int64_t chunk_size, int nthreads);
int oracle_ssd_bwd(const float* x, const float* dt_raw, const float* A, const float* B,
                   const float* C, const float* D, const float* z, const float* dt_bias,
                   double dt_min, double dt_max, const double* init, const int32_t* seq_idx,
                   const double* dout, const double* dfinal, double* dx, double* dz,
                   double* ddt_raw, double* dA, double* dB, double* dC, double* dD,
                   double* ddt_bias, double* dinit, int64_t batch, int64_t seqlen,
                   int64_t nheads, int64_t headdim, int64_t dstate, int64_t ngroups,
                   int nthreads);

static uint64_t rng = 88172645463325252ull;
static double uniform(void) {  /* xorshift64, in [-1, 1) */
  rng ^= rng << 13;
  rng ^= rng >> 7;
  rng ^= rng << 17;
  return (double)(rng >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}
static float* randf(size_t n, double scale) {
  float* p = malloc(n * sizeof(float));
  for (size_t i = 0; i < n; ++i) p[i] = (float)(scale * uniform());
  return p;
}
static double* randd(size_t n) {
  double* p = malloc(n * sizeof(double));
  for (size_t i = 0; i < n; ++i) p[i] = uniform();
  return p;
}
static double* zerosd(size_t n) { return calloc(n, sizeof(double)); }

static int finite_all(const double* p, size_t n) {
  for (size_t i = 0; i < n; ++i)
    if (!isfinite(p[i])) return 0;
  return 1;
}

#define CHECK(cond)                                                  \
  do {                                                               \
    if (!(cond)) {                                                   \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      return 1;                                                      \
    }                                                                \
  } while (0)

static int one_case(int64_t b, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G,
                    int64_t Q, int packed, int threads) {
  const size_t nx = (size_t)(b * L * H * P), nbc = (size_t)(b * L * G * N);
  const size_t ndt = (size_t)(b * L * H), nst = (size_t)(b * H * P * N);
  float *x = randf(nx, 1.0), *z = randf(nx, 1.0), *B = randf(nbc, 1.0), *C = randf(nbc, 1.0);
  float *dt = randf(ndt, 1.0), *A = randf((size_t)H, 1.0), *D = randf((size_t)H, 1.0);
  float* bias = randf((size_t)H, 1.0);
  for (int64_t h = 0; h < H; ++h) A[h] = -1.0f - fabsf(A[h]) * 15.0f;
  double* init = randd(nst);
  int32_t* seq = NULL;
  if (packed) {
    seq = malloc((size_t)(b * L) * sizeof(int32_t));
    for (int64_t i = 0; i < b * L; ++i) seq[i] = (int32_t)((i % L) / 5 + (i % 7 == 0));
  }
  double *out = zerosd(nx), *fin = zerosd(nst);
  CHECK(oracle_ssd_fwd(x, dt, A, B, C, D, z, bias, 0.0, INFINITY, init, out, fin, seq, b, L, H,
                       P, N, G, NULL, threads) == 0);
  CHECK(finite_all(out, nx) && finite_all(fin, nst));
  /* no optional inputs, a finite dt_limit, a head mask */
  unsigned char* mask = calloc((size_t)(b * H), 1);
  mask[b * H - 1] = 1;
  CHECK(oracle_ssd_fwd(x, dt, A, B, C, NULL, NULL, NULL, 0.01, 0.2, NULL, out, NULL, seq, b, L,
                       H, P, N, G, mask, threads) == 0);
  const int64_t nc = (L + Q - 1) / Q;
  const size_t nq = (size_t)(b * H * nc * Q), ncs = (size_t)(b * nc * H * P * N);
  double *d1 = zerosd(nq), *d2 = zerosd(nq), *s1 = zerosd(ncs), *s2 = zerosd(ncs);
  CHECK(oracle_ssd_chunk_intermediates(x, dt, A, B, bias, 0.0, INFINITY, init, d1, d2, s1, s2,
                                       seq, b, L, H, P, N, G, Q, threads) == 0);
  CHECK(finite_all(s1, ncs) && finite_all(s2, ncs));
  double *dout = randd(nx), *dfin = randd(nst);
  double *dx = zerosd(nx), *dz = zerosd(nx), *ddt = zerosd(ndt), *dA = zerosd((size_t)H);
  double *dB = zerosd(nbc), *dC = zerosd(nbc), *dD = zerosd((size_t)H);
  double *dbias = zerosd((size_t)H), *dinit = zerosd(nst);
  CHECK(oracle_ssd_bwd(x, dt, A, B, C, D, z, bias, 0.0, INFINITY, init, seq, dout, dfin, dx, dz,
                       ddt, dA, dB, dC, dD, dbias, dinit, b, L, H, P, N, G, threads) == 0);
  CHECK(finite_all(dx, nx) && finite_all(dB, nbc) && finite_all(dinit, nst));
  free(x); free(z); free(B); free(C); free(dt); free(A); free(D); free(bias); free(init);
  free(seq); free(out); free(fin); free(mask); free(d1); free(d2); free(s1); free(s2);
  free(dout); free(dfin); free(dx); free(dz); free(ddt); free(dA); free(dB); free(dC);
  free(dD); free(dbias); free(dinit);
  return 0;
}

int main(void) {
  /* ragged chunks, groups, packed sequences, one and several threads */
  if (one_case(2, 37, 4, 8, 4, 2, 16, 0, 1)) return 1;
  if (one_case(2, 37, 4, 8, 4, 2, 16, 1, 2)) return 1;
  if (one_case(1, 130, 6, 4, 8, 3, 64, 1, 3)) return 1;
  if (one_case(3, 1, 2, 2, 2, 1, 8, 0, 1)) return 1;
  if (one_case(1, 70, 2, 3, 5, 2, 70, 1, 1)) return 1;
  /* empty sequences and rejected shapes */
  double out[1], fin[4];
  float one[4] = {1, 1, 1, 1};
  if (oracle_ssd_fwd(one, one, one, one, one, NULL, NULL, NULL, 0.0, INFINITY, NULL, out, fin,
                     NULL, 1, 0, 1, 2, 2, 1, NULL, 1) != 0)
    return 1;
  if (oracle_ssd_fwd(one, one, one, one, one, NULL, NULL, NULL, 0.0, INFINITY, NULL, out, fin,
                     NULL, 1, 1, 3, 1, 1, 2, NULL, 1) != -1)
    return 1;
  if (oracle_ssd_bwd(one, one, one, one, one, NULL, NULL, NULL, 0.0, INFINITY, NULL, NULL, NULL,
                     NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1, 1, 2, 1, 1,
                     0, 1) != -1)
    return 1;
  puts("oracle sanitizer driver: ok");
  return 0;
}
