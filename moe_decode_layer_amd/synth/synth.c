/*
 * Seeded synthetic inputs for the MoE decode layer.
 *
 * This file only draws random numbers and encodes them into the storage
 * formats the layer consumes (bf16 activations, fp32 router weights, FP8
 * e4m3fn expert weights with one fp32 scale per 32 contiguous K elements).
 * It holds none of the layer's own arithmetic: no dot product, no routing,
 * no activation, no dequantisation.  Both the GPU path and the CPU oracle
 * read the bytes produced here.
 *
 * Random numbers: counter-based SplitMix64.  Value i of the stream
 * (seed, tensor, a, row) is the SplitMix64 output function applied to
 * key + (i + 1) * 0x9E3779B97F4A7C15, where key chains the SplitMix64
 * output function over seed, (tensor << 32 | a) and row.  Every value
 * therefore depends only on its coordinates, never on thread count or
 * generation order.  Normals come from the Box-Muller transform on the
 * pair of values (2p, 2p + 1): u1 = (v_2p >> 11 + 1) * 2^-53 in (0, 1],
 * u2 = (v_2p+1 >> 11) * 2^-53 in [0, 1); element 2p takes r*cos(2*pi*u2)
 * and element 2p + 1 takes r*sin(2*pi*u2), r = sqrt(-2 ln u1).
 *
 * Built with gcc (-O2 -fopenmp); loaded through ctypes.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define SYNTH_ABI 2
#define GOLDEN_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint32_t tensor, uint32_t a, uint32_t row) {
  uint64_t k = mix64(seed + GOLDEN_GAMMA);
  k = mix64(k ^ (((uint64_t)tensor << 32) | (uint64_t)a));
  return mix64(k ^ (uint64_t)row);
}

static inline uint64_t stream_value(uint64_t key, uint64_t i) {
  return mix64(key + (i + 1) * GOLDEN_GAMMA);
}

/* n standard normals of stream key into out[0..n). */
static void normals(uint64_t key, int64_t n, double* out) {
  const double two_pi = 6.283185307179586476925286766559;
  for (int64_t p = 0; 2 * p < n; ++p) {
    uint64_t a = stream_value(key, (uint64_t)(2 * p));
    uint64_t b = stream_value(key, (uint64_t)(2 * p + 1));
    double u1 = (double)((a >> 11) + 1) * 0x1p-53;
    double u2 = (double)(b >> 11) * 0x1p-53;
    double r = sqrt(-2.0 * log(u1));
    out[2 * p] = r * cos(two_pi * u2);
    if (2 * p + 1 < n) out[2 * p + 1] = r * sin(two_pi * u2);
  }
}

/* fp64 -> bf16 bit pattern, round to nearest even, overflow to inf. */
uint16_t synth_bf16_encode(double v) {
  if (isnan(v)) return 0x7FC0;
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);                       /* a = f * 2^e, f in [0.5, 1) */
  int q = e - 8;                      /* 8 significant bits */
  if (q < -133) q = -133;             /* subnormal step of bf16 */
  double r = ldexp(nearbyint(ldexp(a, -q)), q);
  if (r > 0x1.FEp127) return sign | 0x7F80;
  float f = (float)r;                 /* exact: r is a bf16 value */
  uint32_t bits;
  memcpy(&bits, &f, 4);
  return sign | (uint16_t)((bits >> 16) & 0x7FFF);
}

/* fp64 -> OCP FP8 e4m3fn code, round to nearest even, saturate to +-448. */
uint8_t synth_e4m3fn_encode(double v) {
  if (isnan(v)) return 0x7F;
  uint8_t sign = signbit(v) ? 0x80 : 0;
  double a = fabs(v);
  if (a >= 448.0) return sign | 0x7E;
  if (a < 0x1p-6) {                   /* subnormal range, step 2^-9 */
    int m = (int)nearbyint(a * 0x1p9); /* m == 8 carries into the first normal code */
    return sign | (uint8_t)m;
  }
  int e;
  double f = frexp(a, &e);            /* a = f * 2^e, leading bit 2^(e-1) */
  int m = (int)nearbyint((2.0 * f - 1.0) * 8.0); /* 0..8 */
  int code = ((e - 1 + 7) << 3) + m;  /* m == 8 carries into the next binade */
  if (code > 0x7E) code = 0x7E;
  return sign | (uint8_t)code;
}

/* fp64 -> OCP FP4 E2M1 code (the MXFP4 element), round to nearest even,
   saturate to +-6.  Magnitudes of codes 0..7: 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
uint8_t synth_e2m1_encode(double v) {
  static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  uint8_t sign = signbit(v) ? 0x8 : 0;
  double a = fabs(v);
  if (isnan(v)) return 0x7;             /* no NaN code: the largest value */
  int best = 0;
  for (int c = 1; c < 8; ++c) {
    double d = fabs(a - mag[c]), db = fabs(a - mag[best]);
    if (d < db || (d == db && (c & 1) == 0)) best = c;   /* ties to the even code */
  }
  if (a >= 6.0) best = 7;
  return sign | (uint8_t)best;
}

int synth_abi(void) { return SYNTH_ABI; }

void synth_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int synth_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Raw standard normals of one stream (exposed for distribution tests). */
void synth_normal_f64(uint64_t seed, uint32_t tensor, uint32_t a, uint32_t row, int64_t n,
                      double* out) {
  normals(stream_key(seed, tensor, a, row), n, out);
}

/* Raw 64-bit values of one stream (exposed for tests). */
void synth_u64(uint64_t seed, uint32_t tensor, uint32_t a, uint32_t row, int64_t n,
               uint64_t* out) {
  uint64_t key = stream_key(seed, tensor, a, row);
  for (int64_t i = 0; i < n; ++i) out[i] = stream_value(key, (uint64_t)i);
}

/* x[t][h] = bf16(N(0, std^2)); row t is drawn from attempt attempts[t]. */
void synth_x_bf16(uint64_t seed, uint32_t tensor, int32_t T, int32_t H, double std,
                  const int32_t* attempts, uint16_t* out) {
#pragma omp parallel
  {
    double* buf = (double*)malloc(sizeof(double) * (size_t)H);
#pragma omp for schedule(static)
    for (int32_t t = 0; t < T; ++t) {
      normals(stream_key(seed, tensor, (uint32_t)attempts[t], (uint32_t)t), H, buf);
      for (int32_t h = 0; h < H; ++h) out[(int64_t)t * H + h] = synth_bf16_encode(std * buf[h]);
    }
    free(buf);
  }
}

/* w[r][k] = fp32(N(0, std^2)) for rows r in [0, R). */
void synth_f32(uint64_t seed, uint32_t tensor, uint32_t a, int32_t R, int32_t K, double std,
               float* out) {
#pragma omp parallel
  {
    double* buf = (double*)malloc(sizeof(double) * (size_t)K);
#pragma omp for schedule(static)
    for (int32_t r = 0; r < R; ++r) {
      normals(stream_key(seed, tensor, a, (uint32_t)r), K, buf);
      for (int32_t k = 0; k < K; ++k) out[(int64_t)r * K + k] = (float)(std * buf[k]);
    }
    free(buf);
  }
}

/*
 * One expert matrix [R][K] of N(0, std^2) weights, quantised per 32
 * contiguous K elements: scale = fp32(max|w| / 448) (1.0 for an all-zero
 * group), q = e4m3fn(w / scale).  q is [R][K] bytes, s is [R][K/32] fp32.
 * K must be a multiple of 32.
 */
void synth_fp8_g32(uint64_t seed, uint32_t tensor, uint32_t a, int32_t R, int32_t K,
                   double std, uint8_t* q, float* s) {
  const int32_t G = K / 32;
#pragma omp parallel
  {
    double* buf = (double*)malloc(sizeof(double) * (size_t)K);
#pragma omp for schedule(static)
    for (int32_t r = 0; r < R; ++r) {
      normals(stream_key(seed, tensor, a, (uint32_t)r), K, buf);
      for (int32_t g = 0; g < G; ++g) {
        const double* w = buf + 32 * g;
        double amax = 0.0;
        for (int j = 0; j < 32; ++j) {
          double m = fabs(std * w[j]);
          if (m > amax) amax = m;
        }
        float sc = amax > 0.0 ? (float)(amax / 448.0) : 1.0f;
        s[(int64_t)r * G + g] = sc;
        uint8_t* qq = q + (int64_t)r * K + 32 * g;
        for (int j = 0; j < 32; ++j) qq[j] = synth_e4m3fn_encode(std * w[j] / (double)sc);
      }
    }
    free(buf);
  }
}

/*
 * One expert matrix [R][K] of N(0, std^2) weights in an OCP MX format: each
 * block of 32 contiguous K elements shares the scale 2^X, X = floor(log2
 * max|w|) - emax of the element format (2 for E2M1, 8 for E4M3), clamped to
 * [-127, 127] and stored as the E8M0 code X + 127 (an all-zero block: code
 * 0); each element is w / 2^X encoded with round to nearest even, saturating.
 * fmt 1: MXFP8, q [R][K] e4m3fn codes; fmt 2: MXFP4, q [R][K/2], element 2j
 * in the low nibble of byte j.  s [R][K/32] E8M0 codes.  K a multiple of 32.
 */
void synth_mx_g32(uint64_t seed, uint32_t tensor, uint32_t a, int32_t R, int32_t K, double std,
                  int32_t fmt, uint8_t* q, uint8_t* s) {
  const int32_t G = K / 32;
  const int emax = fmt == 2 ? 2 : 8;
#pragma omp parallel
  {
    double* buf = (double*)malloc(sizeof(double) * (size_t)K);
#pragma omp for schedule(static)
    for (int32_t r = 0; r < R; ++r) {
      normals(stream_key(seed, tensor, a, (uint32_t)r), K, buf);
      for (int32_t g = 0; g < G; ++g) {
        const double* w = buf + 32 * g;
        double amax = 0.0;
        for (int j = 0; j < 32; ++j) {
          double m = fabs(std * w[j]);
          if (m > amax) amax = m;
        }
        int X = -127;
        if (amax > 0.0) {
          int e;
          frexp(amax, &e);               /* amax = f 2^e, f in [0.5, 1): floor(log2) = e - 1 */
          X = e - 1 - emax;
          if (X < -127) X = -127;
          if (X > 127) X = 127;
        }
        s[(int64_t)r * G + g] = (uint8_t)(X + 127);
        const double inv = ldexp(1.0, -X);
        for (int j = 0; j < 32; ++j) {
          const double v = std * w[j] * inv;
          const int64_t k = (int64_t)32 * g + j;
          if (fmt == 2) {
            const uint8_t c = synth_e2m1_encode(v);
            uint8_t* b = q + (int64_t)r * (K / 2) + k / 2;
            if ((k & 1) == 0) *b = c;
            else *b = (uint8_t)(*b | (c << 4));
          } else {
            q[(int64_t)r * K + k] = synth_e4m3fn_encode(v);
          }
        }
      }
    }
    free(buf);
  }
}
