/*
 * oracle.c — plain, slow, CPU reference of the multi-row speculative-decode
 * step.  TEST INFRASTRUCTURE ONLY: nothing in the product library links,
 * loads or calls this file.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg use it.
 *
 * Sources (the pages):
 *   [P2] richland.au, "Fusing the whole speculative-decoding cycle into one CUDA
 *        kernel" — section "What shipped": T = 1 + n_draft rows per pass,
 *        lm_head + verification on device, Gated DeltaNet state committed only
 *        through the surely-accepted token with drafts replayed from a
 *        (k, v, g, beta) ring, dp4a GEMV with shared activations; Q4_K_M weights.
 *   [P3] richland.au, "OpenJet's CUDA megakernel runs 4 coding agents" —
 *        section "Why it matters": each step streams all weights once and
 *        multiplies every loaded weight against all stacked rows (12 rows for
 *        4 agents x [token + 2 drafts]).
 *   [P4] pulse-3k2 mirror, "UPDATE: ... KL divergence" — section "Decode
 *        accuracy": speculative decoding is exact, greedy output is the main
 *        model's greedy choice.
 * The numeric definitions of the block format, the activation quantization,
 * the workloads and the delta rule come from the workload statement that
 * accompanies those pages (Q4_K-style superblocks of 256 weights with fp16 d
 * and dmin, eight 32-weight sub-blocks with 6-bit scale and min, 4-bit codes,
 * w = d*sc*q - dmin*m; activations quantized per 32 elements to int8 with an
 * fp32 scale; Gated DeltaNet rows (q, k, v, g, beta)).
 *
 * Rules: no SIMD intrinsics, no -ffast-math, no FMA contraction
 * (-ffp-contract=off); fp32 where the definition says fp32, double for every
 * accumulation; outputs rounded to fp32 where the GPU's dataflow stores fp32.
 *
 * Readings of the pages where they are silent:
 *   - activation scale s = fl32(amax/127) by IEEE division (amax over the
 *     group's non-NaN elements), codes clamp(rne(fl32(x/s)), -127, 127);
 *     s == 0 (an all-zero group, or amax/127 underflowing) gives zero codes,
 *     and an element whose x/s is NaN codes as 0;
 *   - the delta rule is S <- g (I - beta k k^T) S + beta k v^T with S of shape
 *     dk x dv and o = S^T q after the update; the literal printed form
 *     S <- g S (I - beta k k^T) + beta k v^T is kept behind a flag;
 *   - argmax ties go to the lowest index, NaN logits never win;
 *   - glue of the synthetic layer stack: pre-RMSNorm (unit gain, eps 1e-6)
 *     before each block, identity mixer, fp32 residual.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* IEEE binary16 bit pattern -> float (exact widening), from the format
 * definition: sign, 5-bit biased exponent, 10-bit fraction, subnormals. */
float orc_f16_to_f32(uint16_t h) {
  const int sign = (h >> 15) & 1, e = (h >> 10) & 31, f = h & 1023;
  double v;
  if (e == 0) v = ldexp((double)f, -24);
  else if (e == 31) v = f ? NAN : INFINITY;
  else v = ldexp(1024.0 + f, e - 25);
  return (float)(sign ? -v : v);
}

/* C1: dequantize one superblock row-slice to fp32, literally
 * w = f32(d)*sc[j]*q[k] - f32(dmin)*m[j] with each product rounded to fp32. */
static void dequant_row(const uint16_t* d, const uint16_t* dmin, const uint8_t* sc, const uint8_t* m,
                        const uint8_t* q, int32_t K, float* w) {
  const int nsb = K / 256;
  for (int b = 0; b < nsb; ++b) {
    const float dd = orc_f16_to_f32(d[b]), dm = orc_f16_to_f32(dmin[b]);
    for (int j = 0; j < 8; ++j) {
      const float a = dd * (float)sc[b * 8 + j];
      const float c = dm * (float)m[b * 8 + j];
      for (int i = 0; i < 32; ++i) {
        const int k = b * 256 + j * 32 + i;
        w[k] = a * (float)q[k] - c;
      }
    }
  }
}

void orc_dequant(const uint16_t* d, const uint16_t* dmin, const uint8_t* sc, const uint8_t* m, const uint8_t* q,
                 int32_t N, int32_t K, float* w) {
  const int nsb = K / 256;
#pragma omp parallel for schedule(static)
  for (int64_t o = 0; o < N; ++o)
    dequant_row(d + o * nsb, dmin + o * nsb, sc + o * nsb * 8, m + o * nsb * 8, q + o * (int64_t)K, K,
                w + o * (int64_t)K);
}

/* C2: per-32 symmetric int8 quantization of activation rows. */
void orc_quantize_rows(const float* x, int32_t T, int32_t K, int8_t* a8, float* s, int32_t* gsum) {
  const int ng = K / 32;
  for (int64_t t = 0; t < T; ++t) {
    for (int g = 0; g < ng; ++g) {
      const float* xg = x + t * K + g * 32;
      float amax = 0.0f;
      for (int i = 0; i < 32; ++i) {
        const float ax = fabsf(xg[i]);
        if (ax > amax) amax = ax;
      }
      int8_t* ag = a8 + t * K + g * 32;
      int32_t sum = 0;
      /* amax/127 is 0 for an all-zero group and also when it underflows (amax
       * at most 63 * 2^-149); such a group has no usable scale and gets s = 0
       * and zero codes */
      const float sg = amax / 127.0f;
      if (sg == 0.0f) {
        s[t * ng + g] = 0.0f;
        for (int i = 0; i < 32; ++i) ag[i] = 0;
      } else {
        s[t * ng + g] = sg;
        for (int i = 0; i < 32; ++i) {
          float r = nearbyintf(xg[i] / sg); /* round-half-to-even (default mode) */
          if (r != r) r = 0.0f;             /* a NaN element (or inf/inf) codes as 0 */
          if (r > 127.0f) r = 127.0f;
          if (r < -127.0f) r = -127.0f;
          ag[i] = (int8_t)r;
          sum += (int32_t)r;
        }
      }
      gsum[t * ng + g] = sum;
    }
  }
}

/* C3 on already-quantized rows: y[t][o] = fl32(sum_k w[o][k]*s[t][k/32]*a8[t][k]),
 * accumulated in double in increasing k. */
void orc_qgemv_q8(const uint16_t* d, const uint16_t* dmin, const uint8_t* sc, const uint8_t* m, const uint8_t* q,
                  int32_t N, int32_t K, const int8_t* a8, const float* s, int32_t T, float* y) {
  const int nsb = K / 256, ng = K / 32;
#pragma omp parallel
  {
    float* w = (float*)malloc(sizeof(float) * (size_t)K);
    double* acc = (double*)malloc(sizeof(double) * (size_t)T);
#pragma omp for schedule(static)
    for (int64_t o = 0; o < N; ++o) {
      dequant_row(d + o * nsb, dmin + o * nsb, sc + o * nsb * 8, m + o * nsb * 8, q + o * (int64_t)K, K, w);
      for (int t = 0; t < T; ++t) acc[t] = 0.0;
      for (int k = 0; k < K; ++k) {
        const double wk = (double)w[k];
        for (int t = 0; t < T; ++t)
          acc[t] += wk * (double)s[(int64_t)t * ng + k / 32] * (double)a8[(int64_t)t * K + k];
      }
      for (int t = 0; t < T; ++t) y[(int64_t)t * N + o] = (float)acc[t];
    }
    free(w);
    free(acc);
  }
}

/* C3: quantize x (C2) then GEMV.  Scratch for the codes is allocated here. */
void orc_qgemv(const uint16_t* d, const uint16_t* dmin, const uint8_t* sc, const uint8_t* m, const uint8_t* q,
               int32_t N, int32_t K, const float* x, int32_t T, float* y) {
  int8_t* a8 = (int8_t*)malloc((size_t)T * K);
  float* s = (float*)malloc(sizeof(float) * (size_t)T * (K / 32));
  int32_t* gs = (int32_t*)malloc(sizeof(int32_t) * (size_t)T * (K / 32));
  orc_quantize_rows(x, T, K, a8, s, gs);
  orc_qgemv_q8(d, dmin, sc, m, q, N, K, a8, s, T, y);
  free(a8);
  free(s);
  free(gs);
}

/* Exact integer partial sums P[t][o][b][j] = sum_{i<32} q[o][256b+32j+i] * a8[t][256b+32j+i]
 * (int64 arithmetic, stored int32: |P| <= 32*15*127). */
void orc_q4k_partials(const uint8_t* q, int32_t N, int32_t K, const int8_t* a8, int32_t T, int32_t* P) {
  const int ng = K / 32;
#pragma omp parallel for schedule(static)
  for (int64_t o = 0; o < N; ++o)
    for (int t = 0; t < T; ++t)
      for (int g = 0; g < ng; ++g) {
        int64_t acc = 0;
        for (int i = 0; i < 32; ++i)
          acc += (int64_t)q[o * (int64_t)K + g * 32 + i] * (int64_t)a8[(int64_t)t * K + g * 32 + i];
        P[((int64_t)t * N + o) * ng + g] = (int32_t)acc;
      }
}

/* h = fl32(g * u / (1 + exp(-g))) in double (SiLU(g) * u). */
void orc_silu_mul(const float* g, const float* u, int64_t n, float* h) {
  for (int64_t i = 0; i < n; ++i) {
    const double gg = (double)g[i];
    h[i] = (float)(gg * (double)u[i] / (1.0 + exp(-gg)));
  }
}

/* C4: y = W_d . q8(SiLU(W_g . q8(x)) * (W_u . q8(x))).  Weights are passed as
 * field arrays in the order gate, up, down. */
void orc_ffn(const uint16_t* gd, const uint16_t* gdm, const uint8_t* gsc, const uint8_t* gm, const uint8_t* gq,
             const uint16_t* ud, const uint16_t* udm, const uint8_t* usc, const uint8_t* um, const uint8_t* uq,
             const uint16_t* dd, const uint16_t* ddm, const uint8_t* dsc, const uint8_t* dm, const uint8_t* dq,
             int32_t H, int32_t F, const float* x, int32_t T, float* y, float* h_out /* may be NULL */) {
  float* g = (float*)malloc(sizeof(float) * (size_t)T * F);
  float* u = (float*)malloc(sizeof(float) * (size_t)T * F);
  float* h = h_out ? h_out : (float*)malloc(sizeof(float) * (size_t)T * F);
  orc_qgemv(gd, gdm, gsc, gm, gq, F, H, x, T, g);
  orc_qgemv(ud, udm, usc, um, uq, F, H, x, T, u);
  orc_silu_mul(g, u, (int64_t)T * F, h);
  orc_qgemv(dd, ddm, dsc, dm, dq, H, F, h, T, y);
  free(g);
  free(u);
  if (!h_out) free(h);
}

/* RMSNorm with unit gain: a = fl32(x / sqrt(mean(x^2) + eps)), in double. */
void orc_rmsnorm(const float* x, int32_t T, int32_t K, double eps, float* a) {
  for (int64_t t = 0; t < T; ++t) {
    double ss = 0.0;
    for (int k = 0; k < K; ++k) ss += (double)x[t * K + k] * (double)x[t * K + k];
    const double r = sqrt(ss / (double)K + eps);
    for (int k = 0; k < K; ++k) a[t * K + k] = (float)((double)x[t * K + k] / r);
  }
}

/* fl32 residual add: x[i] = fl32(x[i] + y[i]). */
void orc_residual_add(float* x, const float* y, int64_t n) {
  for (int64_t i = 0; i < n; ++i) x[i] = (float)((double)x[i] + (double)y[i]);
}

/* C6 (logits): logits[t][v] = sum_h f32(W[v][h]) * hid[t][h] in double, then the
 * argmax (lowest index among maxima; NaN never wins; -1 if every logit is NaN),
 * the runner-up, and for both the sum of |W[v][h] * hid[t][h]| (used for the
 * near-tie bound).  logits_out may be NULL. */
void orc_lmhead(const uint16_t* W, int32_t V, int32_t H, const float* hid, int32_t T, double* logits_out,
                int32_t* top1, double* top1_val, int32_t* top2, double* top2_val, double* abs1, double* abs2) {
  double* lg = logits_out ? logits_out : (double*)malloc(sizeof(double) * (size_t)T * V);
#pragma omp parallel
  {
    float* w = (float*)malloc(sizeof(float) * (size_t)H);
#pragma omp for schedule(static)
    for (int64_t v = 0; v < V; ++v) {
      for (int h = 0; h < H; ++h) w[h] = orc_f16_to_f32(W[v * (int64_t)H + h]);
      for (int t = 0; t < T; ++t) {
        double acc = 0.0;
        for (int h = 0; h < H; ++h) acc += (double)w[h] * (double)hid[(int64_t)t * H + h];
        lg[(int64_t)t * V + v] = acc;
      }
    }
    free(w);
  }
  for (int t = 0; t < T; ++t) {
    int32_t b1 = -1, b2 = -1;
    double v1 = -INFINITY, v2 = -INFINITY;
    for (int32_t v = 0; v < V; ++v) {
      const double x = lg[(int64_t)t * V + v];
      if (isnan(x)) continue;
      if (b1 < 0 || x > v1) {
        b2 = b1; v2 = v1;
        b1 = v; v1 = x;
      } else if (b2 < 0 || x > v2) {
        b2 = v; v2 = x;
      }
    }
    top1[t] = b1;
    top1_val[t] = v1;
    top2[t] = b2;
    top2_val[t] = v2;
    double s1 = 0.0, s2 = 0.0;
    for (int h = 0; h < H; ++h) {
      const double hh = (double)hid[(int64_t)t * H + h];
      if (b1 >= 0) s1 += fabs((double)orc_f16_to_f32(W[(int64_t)b1 * H + h]) * hh);
      if (b2 >= 0) s2 += fabs((double)orc_f16_to_f32(W[(int64_t)b2 * H + h]) * hh);
    }
    abs1[t] = s1;
    abs2[t] = s2;
  }
  if (!logits_out) free(lg);
}

/* C6 (verify): group g owns rows [gs[g], gs[g+1]) and the drafts
 * drafts[gs[g]-g .. gs[g+1]-g-2]; draft i of the group proposes the token of
 * row i+1, so it is accepted when it equals the argmax of row i.  n_acc[g] is
 * the number of leading accepted drafts; the group emits its n_acc accepted
 * drafts followed by the argmax of row n_acc (written at tokens[gs[g] + i]).
 * A row whose logits are all NaN has argmax -1, which no draft matches. */
void orc_verify(const int32_t* argmax, const int32_t* gs, int32_t G, const int32_t* drafts, int32_t* n_acc,
                int32_t* tokens) {
  for (int g = 0; g < G; ++g) {
    const int r = gs[g], n = gs[g + 1] - gs[g];
    const int32_t* dr = drafts + (r - g);
    int a = 0;
    while (a < n - 1 && argmax[r + a] >= 0 && dr[a] == argmax[r + a]) ++a;
    n_acc[g] = a;
    for (int i = 0; i < a; ++i) tokens[r + i] = dr[i];
    tokens[r + a] = argmax[r + a];
  }
}

/* C7: apply rows of the gated delta rule to one head's state S[i][j]
 * (i < dk key index, j < dv value index), in double:
 *   u = S^T k;  S <- g (S - beta k u^T) + beta k v^T  (= g (I - beta k k^T) S + beta k v^T)
 *   o = S^T q (after the update), rounded to fp32; o may be NULL.
 * literal != 0 applies the printed right-multiplied form
 *   S <- g S (I - beta k k^T) + beta k v^T   (needs dk == dv), kept for the record. */
void orc_gdn_rows(double* S, int32_t dk, int32_t dv, const float* q, const float* k, const float* v,
                  const float* g, const float* beta, int32_t nrows, int64_t row_stride_qk, int64_t row_stride_v,
                  int64_t row_stride_gb, float* o, int64_t row_stride_o, int literal) {
  double* u = (double*)malloc(sizeof(double) * (size_t)(dk > dv ? dk : dv));
  for (int r = 0; r < nrows; ++r) {
    const float* kr = k + r * row_stride_qk;
    const float* qr = q ? q + r * row_stride_qk : NULL;
    const float* vr = v + r * row_stride_v;
    const double gg = (double)g[r * row_stride_gb], bb = (double)beta[r * row_stride_gb];
    if (!literal) {
      for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += (double)kr[i] * S[(int64_t)i * dv + j];
        u[j] = acc;
      }
      for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) {
          const double ki = (double)kr[i];
          S[(int64_t)i * dv + j] = gg * (S[(int64_t)i * dv + j] - bb * ki * u[j]) + bb * ki * (double)vr[j];
        }
    } else {
      /* (S k)_i = sum_j S[i][j] k[j] */
      for (int i = 0; i < dk; ++i) {
        double acc = 0.0;
        for (int j = 0; j < dv; ++j) acc += S[(int64_t)i * dv + j] * (double)kr[j];
        u[i] = acc;
      }
      for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j)
          S[(int64_t)i * dv + j] =
              gg * (S[(int64_t)i * dv + j] - bb * u[i] * (double)kr[j]) + bb * (double)kr[i] * (double)vr[j];
    }
    if (o && qr) {
      for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += (double)qr[i] * S[(int64_t)i * dv + j];
        o[r * row_stride_o + j] = (float)acc;
      }
    }
  }
  free(u);
}

/* C7 + C8: one decode step of nh heads with rollback.  S (fp32, [nh][dk][dv])
 * is the committed state; rows t = 0..T-1 of q, k, v [T][nh][d] and g, beta
 * [T][nh] are applied in order and produce o [T][nh][dv]; the state committed
 * for the next step is S after rows 0..a only (recomputed from the step's
 * starting state), rounded to fp32. */
void orc_gdn_step(float* S, int32_t nh, int32_t dk, int32_t dv, const float* q, const float* k, const float* v,
                  const float* g, const float* beta, int32_t T, int32_t a, float* o) {
#pragma omp parallel
  {
    double* Sd = (double*)malloc(sizeof(double) * (size_t)dk * dv);
#pragma omp for schedule(static)
    for (int64_t h = 0; h < nh; ++h) {
      float* Sh = S + h * (int64_t)dk * dv;
      for (int64_t e = 0; e < (int64_t)dk * dv; ++e) Sd[e] = (double)Sh[e];
      orc_gdn_rows(Sd, dk, dv, q + h * dk, k + h * dk, v + h * dv, g + h, beta + h, T, (int64_t)nh * dk,
                   (int64_t)nh * dv, nh, o + h * dv, (int64_t)nh * dv, 0);
      for (int64_t e = 0; e < (int64_t)dk * dv; ++e) Sd[e] = (double)Sh[e];
      orc_gdn_rows(Sd, dk, dv, NULL, k + h * dk, v + h * dv, g + h, beta + h, a + 1, (int64_t)nh * dk,
                   (int64_t)nh * dv, nh, NULL, 0, 0);
      for (int64_t e = 0; e < (int64_t)dk * dv; ++e) Sh[e] = (float)Sd[e];
    }
    free(Sd);
  }
}

/* Full-attention decode of T query rows over a per-agent KV cache (the
 * model's full-attention layers; richland.au "Fusing the whole
 * speculative-decoding cycle into one CUDA kernel", section "What shipped":
 * split-K flash decoding over an fp16 KV cache).  Definition written out:
 *   row t of group g (index i in the group, ctx[g] cached positions before
 *   the step) and query head hq see positions j = 0 .. ctx[g] + i, the
 *   group's own newer rows hidden (causal among drafts);
 *   s_j = (q_t,hq . K_j) / sqrt(d),   w_j = exp(s_j - max s),
 *   o = (sum_j w_j V_j) / (sum_j w_j),  then o *= 1 / (1 + exp(-gate)) if a
 *   gate is given (the output gate of gated attention).
 * KV head of query head hq: hq / (Hq / Hkv) (grouped queries).
 * Layouts: q, gate, o [T][Hq][d] fp32; kc [G][Hkv][cap][d] and vc
 * [G][Hkv][d][cap] fp16 bits (V stored dimension-major); ctx [G];
 * gs [G+1] group starts.  Every accumulation is in double, the output is
 * rounded once to fp32. */
/* K and V element readers: fp16 caches, or q8_0 caches (blocks of 32 int8
 * codes with one fp16 scale; value = f32(scale) * code, exact in double). */
typedef struct {
  const uint16_t *kc, *vc;        /* fp16: [G][Hkv][cap][d], [G][Hkv][d][cap] */
  const int8_t *k8, *v8;          /* q8_0 codes: [G][Hkv][cap][d], [G][Hkv][cap/64][d][64] */
  const uint16_t *ks, *vs;        /* q8_0 scales: [G][Hkv][cap][d/32], [G][Hkv][cap/32][d] */
  const float* f16;               /* fp16 bit pattern -> value */
  int64_t cap, d;
} kv_src;

static double k_at(const kv_src* c, int64_t gh, int64_t j, int k) {
  if (c->kc) return (double)c->f16[c->kc[(gh * c->cap + j) * c->d + k]];
  return (double)c->f16[c->ks[(gh * c->cap + j) * (c->d / 32) + k / 32]] * (double)c->k8[(gh * c->cap + j) * c->d + k];
}

static double v_at(const kv_src* c, int64_t gh, int64_t j, int k) {
  if (c->vc) return (double)c->f16[c->vc[(gh * c->d + k) * c->cap + j]];
  return (double)c->f16[c->vs[(gh * (c->cap / 32) + j / 32) * c->d + k]] *
         (double)c->v8[((gh * (c->cap / 64) + j / 64) * c->d + k) * 64 + j % 64];
}

static void attn_rows(const float* q, const float* gate, int32_t T, int32_t Hq, const kv_src* c, int32_t Hkv,
                      const int32_t* ctx, const int32_t* gs, float* o);

void orc_attn_decode(const float* q, const float* gate, int32_t T, int32_t Hq, const uint16_t* kc,
                     const uint16_t* vc, int32_t Hkv, int32_t d, int32_t cap, const int32_t* ctx,
                     const int32_t* gs, int32_t G, float* o) {
  float* f16 = (float*)malloc(sizeof(float) * 65536);
  for (int b = 0; b < 65536; ++b) f16[b] = orc_f16_to_f32((uint16_t)b);
  kv_src c = {kc, vc, NULL, NULL, NULL, NULL, f16, cap, d};
  (void)G;
  attn_rows(q, gate, T, Hq, &c, Hkv, ctx, gs, o);
  free(f16);
}

/* The same attention over q8_0 caches (the pages keep the KV cache in q8_0
 * above about 80K positions; richland.au, "Fusing the whole speculative-
 * decoding cycle into one CUDA kernel", section "What shipped").  k8 [G][Hkv]
 * [cap][d] with ks [G][Hkv][cap][d/32] (scale of dims 32i..32i+31 of a
 * position); v8 [G][Hkv][cap/64][d][64] (tile-major: positions 64t..64t+63
 * of every dimension together) with vs [G][Hkv][cap/32][d] (scale of
 * positions 32i..32i+31 of a dimension).  d % 32 == 0, cap % 64 == 0. */
void orc_attn_decode_q8(const float* q, const float* gate, int32_t T, int32_t Hq, const int8_t* k8,
                        const uint16_t* ks, const int8_t* v8, const uint16_t* vs, int32_t Hkv, int32_t d,
                        int32_t cap, const int32_t* ctx, const int32_t* gs, int32_t G, float* o) {
  float* f16 = (float*)malloc(sizeof(float) * 65536);
  for (int b = 0; b < 65536; ++b) f16[b] = orc_f16_to_f32((uint16_t)b);
  kv_src c = {NULL, NULL, k8, v8, ks, vs, f16, cap, d};
  (void)G;
  attn_rows(q, gate, T, Hq, &c, Hkv, ctx, gs, o);
  free(f16);
}

static void attn_rows(const float* q, const float* gate, int32_t T, int32_t Hq, const kv_src* c, int32_t Hkv,
                      const int32_t* ctx, const int32_t* gs, float* o) {
  const int d = (int)c->d;
  const int gqa = Hq / Hkv;
  const double inv_sqrt_d = 1.0 / sqrt((double)d);
#pragma omp parallel
  {
    double* s = NULL;
    int64_t s_cap = 0;
    double* acc = (double*)malloc(sizeof(double) * d);
#pragma omp for schedule(dynamic)
    for (int64_t th = 0; th < (int64_t)T * Hq; ++th) {
      const int t = (int)(th / Hq), hq = (int)(th % Hq);
      int g = 0;
      while (!(gs[g] <= t && t < gs[g + 1])) ++g;
      const int64_t n = (int64_t)ctx[g] + (t - gs[g]) + 1;
      const int64_t gh = (int64_t)g * Hkv + hq / gqa;
      const float* qr = q + th * d;
      if (n > s_cap) {
        free(s);
        s_cap = n;
        s = (double*)malloc(sizeof(double) * n);
      }
      double mx = -INFINITY;
      for (int64_t j = 0; j < n; ++j) {
        double dot = 0.0;
        for (int k = 0; k < d; ++k) dot += (double)qr[k] * k_at(c, gh, j, k);
        s[j] = dot * inv_sqrt_d;
        if (s[j] > mx) mx = s[j];
      }
      double den = 0.0;
      for (int64_t j = 0; j < n; ++j) {
        s[j] = exp(s[j] - mx);
        den += s[j];
      }
      for (int k = 0; k < d; ++k) {
        double a = 0.0;
        for (int64_t j = 0; j < n; ++j) a += s[j] * v_at(c, gh, j, k);
        acc[k] = a / den;
      }
      for (int k = 0; k < d; ++k) {
        double y = acc[k];
        if (gate) y *= 1.0 / (1.0 + exp(-(double)gate[th * d + k]));
        o[th * d + k] = (float)y;
      }
    }
    free(acc);
    free(s);
  }
}
