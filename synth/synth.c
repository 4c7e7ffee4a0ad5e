/*
 * Seeded synthetic inputs for the KDA forward and decode tests and benchmark.
 *
 * This module holds no arithmetic of the method itself; it only draws random
 * tensors with the distributions the workloads call for.  Both the oracle side
 * and the GPU side take their inputs from here.
 *
 * Generator: counter-based.  Element i of stream s under seed x is
 *     key  = mix64(x * GOLDEN + s)
 *     bits = mix64(key + (i + 1) * GOLDEN)
 * where mix64 is the splitmix64 output function (S. Vigna, "splitmix64.c",
 * derived from Steele, Lea and Flood, "Fast splittable pseudorandom number
 * generators", OOPSLA 2014) and GOLDEN = 0x9E3779B97F4A7C15.  A uniform in
 * [0,1) is (bits >> 11) * 2^-53.  Standard normals come in pairs from the
 * Box-Muller transform: pair m uses draws 2m and 2m+1, and element i takes
 * the cosine branch of pair i/2 when i is even, the sine branch when odd.
 *
 * Every value depends only on (seed, stream, flat index), so any sub-block
 * (a head, a time slab) can be regenerated on its own and equals the same
 * block of the full tensor bit for bit.
 *
 * Rounding to the storage type: fp64 -> fp32 (round to nearest even), then,
 * for bf16, fp32 -> bf16 (round to nearest even).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return mix64(seed * GOLDEN + stream);
}

static inline double uniform_at(uint64_t key, uint64_t i) {
  uint64_t b = mix64(key + (i + 1) * GOLDEN);
  return (double)(b >> 11) * (1.0 / 9007199254740992.0);
}

static inline void normal_pair(uint64_t key, uint64_t m, double* n0, double* n1) {
  double u1 = 1.0 - uniform_at(key, 2 * m); /* (0, 1] */
  double u2 = uniform_at(key, 2 * m + 1);   /* [0, 1) */
  double r = sqrt(-2.0 * log(u1));
  double th = 6.283185307179586476925286766559 * u2;
  *n0 = r * cos(th);
  *n1 = r * sin(th);
}

static inline double normal_at(uint64_t key, uint64_t i) {
  double n0, n1;
  normal_pair(key, i >> 1, &n0, &n1);
  return (i & 1) ? n1 : n0;
}

/* Normals for flat indices [base, base + n) into x. */
static inline void normals(uint64_t key, uint64_t base, int64_t n, double* x) {
  int64_t c = 0;
  if (n > 0 && (base & 1)) { x[0] = normal_at(key, base); c = 1; }
  for (; c + 1 < n; c += 2) normal_pair(key, (base + (uint64_t)c) >> 1, &x[c], &x[c + 1]);
  if (c < n) x[c] = normal_at(key, base + (uint64_t)c);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)(u >> 16) | ((u & 0xffff) ? 0x40 : 0);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

/* out_dtype: 0 = fp32, 1 = bf16 (stored as uint16 bit patterns), 2 = fp64 */
static inline void store(void* out, int64_t idx, double x, int out_dtype) {
  if (out_dtype == 0) {
    ((float*)out)[idx] = (float)x;
  } else if (out_dtype == 1) {
    ((uint16_t*)out)[idx] = f32_to_bf16_rne((float)x);
  } else {
    ((double*)out)[idx] = x;
  }
}

/* Distribution kinds. */
enum {
  SYNTH_NORMAL = 0,      /* mean + std * N(0,1)                                */
  SYNTH_UNIT_ROWS = 1,   /* N(0,1) rows scaled to unit L2 norm along last dim   */
  SYNTH_SIGMOID_NORMAL = 2, /* 1 / (1 + exp(-(mean + std*N(0,1))))            */
  SYNTH_UNIFORM = 3,     /* U(lo, hi) with lo = mean, hi = std                  */
  SYNTH_CONST = 4        /* the constant `mean`                                 */
};

/*
 * Fill the block b0.., t0.., h0.. (sizes nb, nt, nh, all of D) of a logical
 * tensor of shape [B, T, H, D] (row-major, D fastest).  The flat index of
 * element (b, t, h, c) is ((b*T + t)*H + h)*D + c.  Output element
 * (bi, ti, hi, c) of the block goes to out[bi*osb + ti*ost + hi*osh + c].
 */
int synth_fill(int kind, int out_dtype, uint64_t seed, uint64_t stream,
               int64_t B, int64_t T, int64_t H, int64_t D,
               int64_t b0, int64_t nb, int64_t t0, int64_t nt, int64_t h0, int64_t nh,
               double mean, double stdv, void* out, int64_t osb, int64_t ost, int64_t osh) {
  if (b0 < 0 || t0 < 0 || h0 < 0 || nb < 0 || nt < 0 || nh < 0 || D <= 0) return -1;
  if (b0 + nb > B || t0 + nt > T || h0 + nh > H) return -1;
  if (out_dtype < 0 || out_dtype > 2) return -1;
  if (kind == SYNTH_UNIT_ROWS && D > 1024) return -1;
  const uint64_t key = stream_key(seed, stream);
  const int64_t rows = nb * nt * nh;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const int64_t bi = r / (nt * nh);
    const int64_t ti = (r / nh) % nt;
    const int64_t hi = r % nh;
    const uint64_t base = (uint64_t)((((b0 + bi) * T + (t0 + ti)) * H + (h0 + hi)) * D);
    const int64_t ob = bi * osb + ti * ost + hi * osh;
    if (kind == SYNTH_UNIT_ROWS) {
      double x[1024];
      double ss = 0.0;
      normals(key, base, D, x);
      for (int64_t c = 0; c < D; ++c) ss += x[c] * x[c];
      double inv = 1.0 / sqrt(ss);
      for (int64_t c = 0; c < D; ++c) store(out, ob + c, x[c] * inv, out_dtype);
    } else if (kind == SYNTH_NORMAL || kind == SYNTH_SIGMOID_NORMAL) {
      double x[256];
      for (int64_t c0 = 0; c0 < D; c0 += 256) {
        int64_t n = D - c0 < 256 ? D - c0 : 256;
        normals(key, base + (uint64_t)c0, n, x);
        for (int64_t c = 0; c < n; ++c) {
          double y = mean + stdv * x[c];
          if (kind == SYNTH_SIGMOID_NORMAL) y = 1.0 / (1.0 + exp(-y));
          store(out, ob + c0 + c, y, out_dtype);
        }
      }
    } else {
      for (int64_t c = 0; c < D; ++c) {
        double y = kind == SYNTH_UNIFORM ? mean + (stdv - mean) * uniform_at(key, base + c) : mean;
        store(out, ob + c, y, out_dtype);
      }
    }
  }
  return 0;
}

/* Raw uniform draws, for testing the generator against its definition. */
void synth_raw_uniform(uint64_t seed, uint64_t stream, uint64_t i0, int64_t n, double* out) {
  const uint64_t key = stream_key(seed, stream);
  for (int64_t j = 0; j < n; ++j) out[j] = uniform_at(key, i0 + (uint64_t)j);
}

void synth_raw_bits(uint64_t seed, uint64_t stream, uint64_t i0, int64_t n, uint64_t* out) {
  const uint64_t key = stream_key(seed, stream);
  for (int64_t j = 0; j < n; ++j) out[j] = mix64(key + (i0 + (uint64_t)j + 1) * GOLDEN);
}
