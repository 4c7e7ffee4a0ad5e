/*
 * Driver for the AddressSanitizer / UndefinedBehaviorSanitizer build of the
 * C oracle (oracle/kda_oracle.c) and the seeded input generator
 * (synth/synth.c): every generator kind and output type, blocks inside
 * larger tensors with strided outputs, and the oracle forward on small shapes
 * with every option and output combination plus its argument checks.  Built
 * and run by tests/test_sanitizers.py; a sanitizer finding aborts it.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int synth_fill(int kind, int out_dtype, uint64_t seed, uint64_t stream, int64_t B, int64_t T, int64_t H, int64_t D,
               int64_t b0, int64_t nb, int64_t t0, int64_t nt, int64_t h0, int64_t nh, double mean, double stdv,
               void* out, int64_t osb, int64_t ost, int64_t osh);
void synth_raw_uniform(uint64_t seed, uint64_t stream, uint64_t i0, int64_t n, double* out);
void synth_raw_bits(uint64_t seed, uint64_t stream, uint64_t i0, int64_t n, uint64_t* out);
int kda_oracle_forward(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, const float* q, const float* k,
                       const float* v, const float* beta, const float* z, const float* A, double g_min, double scale,
                       int l2norm, double l2_eps, const double* S0, const float* gate, const float* w, double rms_eps,
                       double* o, double* y, double* S_T, int nthreads, int decay);

static void* xmalloc(size_t n) {
  void* p = malloc(n ? n : 1);
  if (!p) {
    fprintf(stderr, "out of memory\n");
    exit(2);
  }
  return p;
}

static int failures = 0;
#define EXPECT(c)                                                     \
  do {                                                                \
    if (!(c)) {                                                       \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #c); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

/* fp32 tensor [B, T, H, D] of the given generator kind */
static float* gen(int kind, uint64_t stream, int64_t B, int64_t T, int64_t H, int64_t D, double mean, double sd) {
  float* x = (float*)xmalloc(sizeof(float) * (size_t)(B * T * H * D));
  EXPECT(synth_fill(kind, 0, 7, stream, B, T, H, D, 0, B, 0, T, 0, H, mean, sd, x, T * H * D, H * D, D) == 0);
  return x;
}

static void test_synth(void) {
  const int64_t B = 2, T = 9, H = 3;
  for (int kind = 0; kind <= 4; ++kind)
    for (int dt = 0; dt <= 2; ++dt)
      for (int64_t D = 1; D <= 300; D += 149) {
        if (kind == 1 && D > 1024) continue;
        const size_t es = dt == 0 ? 4 : dt == 1 ? 2 : 8;
        /* a block (1, 5, 2) at (1, 3, 1), written with padded strides */
        const int64_t osh = D + 3, ost = 2 * osh + 5, osb = 5 * ost + 7;
        const size_t n = (size_t)(osb * 1 + ost * 4 + osh * 1 + D);
        char* out = (char*)xmalloc(es * n);
        memset(out, 0, es * n);
        EXPECT(synth_fill(kind, dt, 11, 3, B, T, H, D, 1, 1, 3, 5, 1, 2, 0.5, 1.5, out, osb, ost, osh) == 0);
        free(out);
      }
  /* rejected blocks */
  float dummy[4];
  EXPECT(synth_fill(0, 0, 1, 1, 1, 1, 1, 4, 0, 2, 0, 1, 0, 1, 0, 1, dummy, 4, 4, 4) != 0);
  EXPECT(synth_fill(0, 7, 1, 1, 1, 1, 1, 4, 0, 1, 0, 1, 0, 1, 0, 1, dummy, 4, 4, 4) != 0);
  EXPECT(synth_fill(1, 0, 1, 1, 1, 1, 1, 2048, 0, 1, 0, 1, 0, 1, 0, 1, dummy, 4, 4, 4) != 0);
  double u[257];
  uint64_t bits[257];
  synth_raw_uniform(5, 2, 1000, 257, u);
  synth_raw_bits(5, 2, 1000, 257, bits);
  for (int i = 0; i < 257; ++i) EXPECT(u[i] > 0.0 && u[i] < 1.0);
}

static void test_oracle(void) {
  for (int64_t D = 16; D <= 64; D += 48)
    for (int decay = 0; decay <= 1; ++decay)
      for (int opt = 0; opt < 4; ++opt) {
        const int64_t B = 2, T = 70, H = 2;
        float* q = gen(0, 1, B, T, H, D, 0.0, 1.0);
        float* k = gen(0, 2, B, T, H, D, 0.0, 1.0);
        float* v = gen(0, 3, B, T, H, D, 0.0, 1.0);
        float* beta = gen(2, 4, B, T, H, 1, 0.0, 1.0);
        float* z = gen(0, 5, B, T, H, D, 0.0, 2.0);
        float* gate = gen(0, 6, B, T, H, D, 0.0, 1.0);
        float* A = gen(3, 8, 1, 1, H, 1, 0.2, 1.2);
        float* w = gen(3, 9, 1, 1, H, D, 0.5, 1.5);
        double* S0 = (double*)xmalloc(sizeof(double) * (size_t)(B * H * D * D));
        for (int64_t i = 0; i < B * H * D * D; ++i) S0[i] = 0.01 * (double)((i * 37) % 17 - 8);
        double* o = (double*)xmalloc(sizeof(double) * (size_t)(B * T * H * D));
        double* y = (double*)xmalloc(sizeof(double) * (size_t)(B * T * H * D));
        double* ST = (double*)xmalloc(sizeof(double) * (size_t)(B * H * D * D));
        /* opt 0: everything; 1: no S0, no w, no l2norm, o only; 2: y and S_T only, scale 0.5; 3: S_T only */
        const int rc = kda_oracle_forward(B, T, H, D, D, q, k, v, beta, z, A, -5.0, opt == 2 ? 0.5 : 1.0, opt != 1, 1e-6,
                                          opt == 1 ? NULL : S0, opt == 1 || opt == 3 ? NULL : gate,
                                          opt == 0 ? w : NULL, 1e-6, opt <= 1 ? o : NULL, opt == 0 || opt == 2 ? y : NULL,
                                          opt == 1 ? NULL : ST, 2, decay);
        EXPECT(rc == 0);
        free(q); free(k); free(v); free(beta); free(z); free(gate); free(A); free(w);
        free(S0); free(o); free(y); free(ST);
      }
  /* argument checks */
  float f[64] = {0};
  double d[64];
  EXPECT(kda_oracle_forward(1, 1, 0, 4, 4, f, f, f, f, f, f, -5, 1, 1, 1e-6, NULL, NULL, NULL, 1e-6, d, NULL, NULL, 1, 0) == -1);
  EXPECT(kda_oracle_forward(1, 1, 1, 4, 4, NULL, f, f, f, f, f, -5, 1, 1, 1e-6, NULL, NULL, NULL, 1e-6, d, NULL, NULL, 1, 0) == -1);
  EXPECT(kda_oracle_forward(1, 1, 1, 4, 4, f, f, f, f, f, f, -5, 1, 1, 1e-6, NULL, NULL, NULL, 1e-6, d, d, NULL, 1, 0) == -1);
  EXPECT(kda_oracle_forward(1, 1, 1, 4, 4, f, f, f, f, f, f, -5, 1, 1, 1e-6, NULL, NULL, NULL, 1e-6, d, NULL, NULL, 1, 2) == -1);
  /* T = 0: nothing to do, the state passes through */
  EXPECT(kda_oracle_forward(1, 0, 1, 4, 4, f, f, f, f, f, f, -5, 1, 1, 1e-6, NULL, NULL, NULL, 1e-6, NULL, NULL, d, 1, 0) == 0);
}

int main(void) {
  test_synth();
  test_oracle();
  if (failures) {
    fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  printf("san_c: ok\n");
  return 0;
}
