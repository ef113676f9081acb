/*
 * synth.c — seeded, counter-based synthetic inputs for the decode-step path.
 *
 * This module is shared by the CPU oracle and the HIP library's tests and
 * benchmark.  It holds none of the decode method's arithmetic: it only draws
 * random numbers and rounds them to the storage types the workloads use
 * (fp16 bit patterns, fp32, small unsigned integer fields).
 *
 * Generator: the SplitMix64 sequence of Steele, Lea and Flood ("Fast
 * splittable pseudorandom number generators", OOPSLA 2014).  Its n-th output
 * for a state s is mix(s + n*GAMMA) with GAMMA = 0x9E3779B97F4A7C15, so any
 * element of any stream can be regenerated on its own (counter-based).  A
 * stream is identified by (seed, tensor id, sub-stream); its starting state is
 * a mix of the three, so streams do not overlap in practice.
 *
 * Normals: Box-Muller (cosine branch) in double from two uniforms drawn at
 * counters 2i and 2i+1 of the element's stream, rounded once to the storage
 * type with round-to-nearest-even.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC synth.c -lm
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* Starting state of stream (seed, tensor, sub). */
static inline uint64_t stream_key(uint64_t seed, uint64_t tensor, uint64_t sub) {
  uint64_t k = mix64(seed + GAMMA);
  k = mix64(k ^ (tensor * 0xD1B54A32D192ED03ULL + GAMMA));
  k = mix64(k ^ (sub * 0x8CB92BA72F3D8DD7ULL + GAMMA));
  return k;
}

/* n-th output (n >= 0) of the stream starting at key. */
static inline uint64_t draw(uint64_t key, uint64_t n) { return mix64(key + (n + 1) * GAMMA); }

/* Uniform double in (0, 1] with 53 random bits. */
static inline double unif_open0(uint64_t u) { return ((double)(u >> 11) + 1.0) * (1.0 / 9007199254740992.0); }
/* Uniform double in [0, 1). */
static inline double unif(uint64_t u) { return (double)(u >> 11) * (1.0 / 9007199254740992.0); }

static inline double std_normal(uint64_t key, uint64_t i) {
  const double u1 = unif_open0(draw(key, 2 * i));
  const double u2 = unif(draw(key, 2 * i + 1));
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925286766559 * u2);
}

/* double -> IEEE binary16 bit pattern, round to nearest even, subnormals kept,
 * overflow to +-inf.  Written from the binary16 format definition. */
uint16_t synth_f64_to_f16(double x) {
  uint16_t sign = 0;
  if (signbit(x)) { sign = 0x8000; x = -x; }
  if (isnan(x)) return (uint16_t)(sign | 0x7E00);
  if (x >= 65520.0) return (uint16_t)(sign | 0x7C00); /* rounds to inf */
  if (x < 0x1p-25) {
    /* below half the smallest subnormal: 0 (exactly half rounds to even = 0) */
    return sign;
  }
  int e;
  double f = frexp(x, &e); /* x = f * 2^e, f in [0.5, 1) */
  /* normal fp16: exponent field E = e - 1 + 15 in 1..30, value = 1.m * 2^(e-1) */
  int E = e - 1 + 15;
  double scaled;
  if (E >= 1) {
    scaled = ldexp(f, 11); /* in [1024, 2048): 11 significant bits incl. implicit */
  } else {
    /* subnormal: value = m * 2^-24 */
    scaled = ldexp(x, 24);
    E = 0;
  }
  double r = nearbyint(scaled); /* current rounding mode is round-to-nearest-even */
  uint32_t mant = (uint32_t)r;
  if (E >= 1) {
    if (mant == 2048) { mant = 1024; E += 1; }
    if (E >= 31) return (uint16_t)(sign | 0x7C00);
    return (uint16_t)(sign | (E << 10) | (mant - 1024));
  }
  /* subnormal (mant may round up to 1024 = smallest normal, which encodes correctly) */
  return (uint16_t)(sign | mant);
}

/* ---------------------------------------------------------------- raw draws */

void synth_u64(uint64_t seed, uint64_t tensor, uint64_t sub, uint64_t start, int64_t n, uint64_t* out) {
  const uint64_t key = stream_key(seed, tensor, sub);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = draw(key, start + (uint64_t)i);
}

/* Normal(mean, std) rounded to fp32; if absval, |N(mean, std)|. */
void synth_normal_f32(uint64_t seed, uint64_t tensor, uint64_t sub, uint64_t start, int64_t n, double mean,
                      double std, int absval, float* out) {
  const uint64_t key = stream_key(seed, tensor, sub);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    double v = mean + std * std_normal(key, start + (uint64_t)i);
    if (absval) v = fabs(v);
    out[i] = (float)v;
  }
}

/* Normal(mean, std) rounded to fp16 (bit patterns); if absval, |N(mean, std)|. */
void synth_normal_f16(uint64_t seed, uint64_t tensor, uint64_t sub, uint64_t start, int64_t n, double mean,
                      double std, int absval, uint16_t* out) {
  const uint64_t key = stream_key(seed, tensor, sub);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    double v = mean + std * std_normal(key, start + (uint64_t)i);
    if (absval) v = fabs(v);
    out[i] = synth_f64_to_f16(v);
  }
}

/* Integers uniform on [lo, hi] by the 64x64->128 multiply-shift map. */
void synth_uniform_i32(uint64_t seed, uint64_t tensor, uint64_t sub, uint64_t start, int64_t n, int32_t lo,
                       int32_t hi, int32_t* out) {
  const uint64_t key = stream_key(seed, tensor, sub);
  const uint64_t range = (uint64_t)((int64_t)hi - (int64_t)lo + 1);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    unsigned __int128 p = (unsigned __int128)draw(key, start + (uint64_t)i) * range;
    out[i] = (int32_t)((int64_t)lo + (int64_t)(uint64_t)(p >> 64));
  }
}

/* Uniform doubles in [0, 1) (used for Bernoulli decisions by the caller). */
void synth_uniform_f64(uint64_t seed, uint64_t tensor, uint64_t sub, uint64_t start, int64_t n, double* out) {
  const uint64_t key = stream_key(seed, tensor, sub);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = unif(draw(key, start + (uint64_t)i));
}

/* ------------------------------------------------------- Q4_K-style fields */
/*
 * Field arrays of an n_out x n_in block-quantized matrix, rows [r0, r1).
 * Superblock s = row*(n_in/256) + b (global index, so any slice regenerates
 * the same values):
 *   d[s], dmin[s] : fp16(|N(0, 0.01)|)              sub-streams 0 and 1
 *   sc[s][j]      : 6 raw bits (j = 0..7) of draw s  sub-stream 2
 *   m[s][j]       : 6 raw bits (j = 0..7) of draw s  sub-stream 3
 *   q[row][k]     : 4 raw bits; draw (row*n_in + k)/16 of sub-stream 4 holds
 *                   16 consecutive codes, code c at bits 4c..4c+3
 * Output arrays hold only rows [r0, r1) (row r0 first).
 */
void synth_q4k_fields(uint64_t seed, uint64_t tensor, int32_t n_out, int32_t n_in, int32_t r0, int32_t r1,
                      double d_std, uint16_t* d, uint16_t* dmin, uint8_t* sc, uint8_t* m, uint8_t* q) {
  (void)n_out;
  const int64_t nsb = n_in / 256;
  const uint64_t kd = stream_key(seed, tensor, 0), kdm = stream_key(seed, tensor, 1);
  const uint64_t ksc = stream_key(seed, tensor, 2), km = stream_key(seed, tensor, 3);
  const uint64_t kq = stream_key(seed, tensor, 4);
#pragma omp parallel for schedule(static)
  for (int64_t r = r0; r < r1; ++r) {
    const int64_t lr = r - r0;
    for (int64_t b = 0; b < nsb; ++b) {
      const uint64_t s = (uint64_t)(r * nsb + b);
      const int64_t ls = lr * nsb + b;
      d[ls] = synth_f64_to_f16(fabs(d_std * std_normal(kd, s)));
      dmin[ls] = synth_f64_to_f16(fabs(d_std * std_normal(kdm, s)));
      const uint64_t us = draw(ksc, s), um = draw(km, s);
      for (int j = 0; j < 8; ++j) {
        sc[ls * 8 + j] = (uint8_t)((us >> (6 * j)) & 63);
        m[ls * 8 + j] = (uint8_t)((um >> (6 * j)) & 63);
      }
    }
    const uint64_t base = (uint64_t)r * (uint64_t)n_in; /* n_in % 256 == 0, so base % 16 == 0 */
    uint8_t* qr = q + lr * (int64_t)n_in;
    for (int64_t k = 0; k < n_in; k += 16) {
      const uint64_t u = draw(kq, (base + (uint64_t)k) / 16);
      for (int c = 0; c < 16; ++c) qr[k + c] = (uint8_t)((u >> (4 * c)) & 15);
    }
  }
}

/* ---------------------------------------------- Gated DeltaNet step inputs */
/*
 * One step of inputs for nh independent heads (nh = layers*heads), T rows:
 * q, k : N(0,1) vectors of length dk, each L2-normalised in double, then fp32
 * v    : N(0,1) of length dv, fp32
 * g    : sigmoid(N(2, 0.5)), beta: sigmoid(N(0, 1)), fp32
 * Layout: q, k [T][nh][dk], v [T][nh][dv], g, beta [T][nh].
 * Stream tensor id encodes the step so every step regenerates on its own.
 */
void synth_gdn_step_inputs(uint64_t seed, uint64_t tensor, int32_t T, int32_t nh, int32_t dk, int32_t dv,
                           float* q, float* k, float* v, float* g, float* beta) {
  const uint64_t kq = stream_key(seed, tensor, 10), kk = stream_key(seed, tensor, 11);
  const uint64_t kv = stream_key(seed, tensor, 12), kg = stream_key(seed, tensor, 13);
  const uint64_t kb = stream_key(seed, tensor, 14);
#pragma omp parallel for schedule(static)
  for (int64_t th = 0; th < (int64_t)T * nh; ++th) {
    double nq = 0.0, nk = 0.0;
    double tq[512], tk[512];
    for (int i = 0; i < dk; ++i) {
      tq[i] = std_normal(kq, (uint64_t)(th * dk + i));
      tk[i] = std_normal(kk, (uint64_t)(th * dk + i));
      nq += tq[i] * tq[i];
      nk += tk[i] * tk[i];
    }
    nq = sqrt(nq);
    nk = sqrt(nk);
    for (int i = 0; i < dk; ++i) {
      q[th * dk + i] = (float)(tq[i] / nq);
      k[th * dk + i] = (float)(tk[i] / nk);
    }
    for (int i = 0; i < dv; ++i) v[th * dv + i] = (float)std_normal(kv, (uint64_t)(th * dv + i));
    const double zg = 2.0 + 0.5 * std_normal(kg, (uint64_t)th);
    const double zb = std_normal(kb, (uint64_t)th);
    g[th] = (float)(1.0 / (1.0 + exp(-zg)));
    beta[th] = (float)(1.0 / (1.0 + exp(-zb)));
  }
}
