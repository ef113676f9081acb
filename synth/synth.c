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
 * Normals: Box-Muller in double.  Pair p of a stream uses the uniforms at
 * counters 2p and 2p+1; element 2p is the cosine branch and element 2p+1 the
 * sine branch.  Each value is rounded once to its storage type with
 * round-to-nearest-even.
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

/* Normals come in Box-Muller pairs: pair p uses uniforms at counters 2p and
 * 2p+1; element 2p takes the cosine branch and element 2p+1 the sine branch. */
static inline void normal_pair(uint64_t key, uint64_t p, double* z0, double* z1) {
  const double u1 = unif_open0(draw(key, 2 * p));
  const double u2 = unif(draw(key, 2 * p + 1));
  const double r = sqrt(-2.0 * log(u1)), th = 6.283185307179586476925286766559 * u2;
  double sn, cs;
  sincos(th, &sn, &cs);
  *z0 = r * cs;
  *z1 = r * sn;
}

static inline double std_normal(uint64_t key, uint64_t i) {
  double z0, z1;
  normal_pair(key, i >> 1, &z0, &z1);
  return (i & 1) ? z1 : z0;
}

/* double -> IEEE binary16 bit pattern, round to nearest even, subnormals kept,
 * overflow to +-inf.  Written from the two formats' definitions: the double's
 * significand (53 bits with the implicit one) is shifted right to the 11 bits
 * a normal half keeps (or fewer for a subnormal half) and rounded to nearest,
 * ties to even, on the discarded bits. */
uint16_t synth_f64_to_f16(double x) {
  uint64_t b;
  memcpy(&b, &x, 8);
  const uint16_t sign = (uint16_t)((b >> 48) & 0x8000);
  const int e = (int)((b >> 52) & 0x7FF);
  uint64_t m = b & 0xFFFFFFFFFFFFFULL;
  if (e == 0x7FF) return (uint16_t)(sign | (m ? 0x7E00 : 0x7C00));
  if (e == 0) return sign; /* double zero or subnormal: far below half of 2^-24 */
  m |= 1ULL << 52;         /* value = m * 2^(e - 1075) */
  const int E = e - 1023 + 15; /* biased half exponent if normal */
  int shift;                   /* bits of m to discard */
  if (E >= 1) shift = 42;      /* keep 11 significant bits */
  else shift = 42 + (1 - E);   /* subnormal half: value = k * 2^-24 */
  if (shift > 63) return sign;
  const uint64_t keep = m >> shift, rem = m & ((1ULL << shift) - 1), half = 1ULL << (shift - 1);
  uint64_t q = keep + ((rem > half || (rem == half && (keep & 1))) ? 1 : 0);
  if (E >= 1) {
    int EE = E;
    if (q == 2048) { q = 1024; ++EE; }
    if (EE >= 31) return (uint16_t)(sign | 0x7C00);
    return (uint16_t)(sign | (EE << 10) | (q - 1024));
  }
  return (uint16_t)(sign | q); /* q == 1024 encodes the smallest normal */
}

/* ---------------------------------------------------------------- raw draws */

void synth_u64(uint64_t seed, uint64_t tensor, uint64_t sub, uint64_t start, int64_t n, uint64_t* out) {
  const uint64_t key = stream_key(seed, tensor, sub);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = draw(key, start + (uint64_t)i);
}

/* Fills out[0..n) with elements start..start+n of a normal stream, pairwise. */
#define NORMAL_FILL(STORE)                                                          \
  const uint64_t key = stream_key(seed, tensor, sub);                               \
  const uint64_t p0 = start >> 1, p1 = (start + (uint64_t)n + 1) >> 1;              \
  _Pragma("omp parallel for schedule(static)")                                      \
  for (int64_t pp = (int64_t)p0; pp < (int64_t)p1; ++pp) {                          \
    double z[2];                                                                    \
    normal_pair(key, (uint64_t)pp, &z[0], &z[1]);                                   \
    for (int b = 0; b < 2; ++b) {                                                   \
      const uint64_t e = 2 * (uint64_t)pp + b;                                      \
      if (e < start || e >= start + (uint64_t)n) continue;                          \
      double v = mean + std * z[b];                                                 \
      if (absval) v = fabs(v);                                                      \
      STORE;                                                                        \
    }                                                                               \
  }

/* Normal(mean, std) rounded to fp32; if absval, |N(mean, std)|. */
void synth_normal_f32(uint64_t seed, uint64_t tensor, uint64_t sub, uint64_t start, int64_t n, double mean,
                      double std, int absval, float* out) {
  NORMAL_FILL(out[e - start] = (float)v)
}

/* Normal(mean, std) rounded to fp16 (bit patterns); if absval, |N(mean, std)|. */
void synth_normal_f16(uint64_t seed, uint64_t tensor, uint64_t sub, uint64_t start, int64_t n, double mean,
                      double std, int absval, uint16_t* out) {
  NORMAL_FILL(out[e - start] = synth_f64_to_f16(v))
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
 *   d[s], dmin[s] : fp16(|N(0, 0.01)|): the two branches of Box-Muller pair s
 *                   of sub-stream 0
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
  const uint64_t kd = stream_key(seed, tensor, 0);
  const uint64_t ksc = stream_key(seed, tensor, 2), km = stream_key(seed, tensor, 3);
  const uint64_t kq = stream_key(seed, tensor, 4);
#pragma omp parallel for schedule(static)
  for (int64_t r = r0; r < r1; ++r) {
    const int64_t lr = r - r0;
    for (int64_t b = 0; b < nsb; ++b) {
      const uint64_t s = (uint64_t)(r * nsb + b);
      const int64_t ls = lr * nsb + b;
      double z0, z1;
      normal_pair(kd, s, &z0, &z1);
      d[ls] = synth_f64_to_f16(fabs(d_std * z0));
      dmin[ls] = synth_f64_to_f16(fabs(d_std * z1));
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
