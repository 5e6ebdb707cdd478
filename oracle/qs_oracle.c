/*
 * qs_oracle.c -- CPU oracle of the hierarchical INT8 KV cache.
 *
 * TEST INFRASTRUCTURE.  Plain, slow and written for a reader to check against the pages by
 * eye; it is the reference the GPU library is compared with and is never linked into it.
 * Built with gcc -O2 -ffp-contract=off and no fast-math, so every fp32 operation of the
 * quantizer is a single IEEE-754 operation in round-to-nearest-even.
 *
 * Sources (page titles and sections):
 *  [G]  QuantSpec Guide: Self-Speculative Decoding & Quantized KV (aifetchly blog)
 *  [R]  Pith review of arXiv:2502.10424, QuantSpec: Self-Speculative Decoding with
 *       Hierarchical Quantized KV Cache (pith.science)
 */
#include "qs_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------------------------------- */
/* fp16                                                                                      */
/* ---------------------------------------------------------------------------------------- */

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.  Normal
 * numbers are (1 + f/1024) * 2^(e-15); subnormals (e = 0) are (f/1024) * 2^-14; e = 31 is
 * infinity (f = 0) or NaN. */
float orc_half_to_float(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 31;
  int f = h & 1023;
  double v;
  if (e == 0) {
    v = ldexp((double)f, -24);
  } else if (e == 31) {
    v = f ? NAN : INFINITY;
  } else {
    v = ldexp((double)(1024 + f), e - 25);
  }
  return (float)(sign ? -v : v);
}

/* fp32 -> binary16, rounded to nearest with ties to even.  |x| is located between consecutive
 * binary16 values: below 2^-14 those are the multiples of 2^-24 (subnormals, bit pattern = the
 * multiple), from 2^E to 2^(E+1) the multiples of 2^(E-10); the count of quanta is rounded
 * with rint (ties to even in the default rounding mode) and a carry to 2^11 quanta moves to the
 * next binade.  Past the largest finite value (65504) the result is infinity. */
uint16_t orc_float_to_half(float x) {
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  if (isnan(x)) return (uint16_t)(sign | 0x7e00);
  double a = fabs((double)x);
  if (a == 0.0) return sign;
  int e2;
  frexp(a, &e2);           /* a = f 2^e2, f in [0.5, 1): a in [2^(e2-1), 2^e2) */
  int E = e2 - 1;
  if (E < -14) {           /* subnormal range: quanta of 2^-24 (1024 of them is 2^-14) */
    double n = rint(ldexp(a, 24));
    return (uint16_t)(sign | (uint16_t)n);
  }
  double n = rint(ldexp(a, 10 - E)); /* in [1024, 2048] */
  if (n == 2048.0) {
    n = 1024.0;
    ++E;
  }
  if (E > 15) return (uint16_t)(sign | 0x7c00);
  return (uint16_t)(sign | ((E + 15) << 10) | ((int)n - 1024));
}

/* ---------------------------------------------------------------------------------------- */
/* Quantizer and split                                                                       */
/* ---------------------------------------------------------------------------------------- */

/* Asymmetric 8-bit quantization of one group, in the order of the quantizer listing of [G]
 * ("Hierarchical Quantizer with Bit-Packing"), computed in fp32:
 *   mn, mx = min, max of the group
 *   s      = (mx - mn) / 255, then clamped to at least 1e-8
 *   z      = round(-mn / s)                                  (not clamped)
 *   c      = clamp(round(x / s) + z, 0, 255)
 * round() is round-half-to-even, like torch.round. */
void orc_quantize_group(const uint16_t* x, int n, int stride, float* s_out, float* z_out,
                        uint8_t* c, int cstride) {
  float mn = orc_half_to_float(x[0]);
  float mx = mn;
  for (int i = 1; i < n; ++i) {
    float v = orc_half_to_float(x[(size_t)i * stride]);
    if (v < mn) mn = v;
    if (v > mx) mx = v;
  }
  float s = (mx - mn) / 255.0f;
  if (s < 1e-8f) s = 1e-8f;
  float z = rintf(-mn / s);
  for (int i = 0; i < n; ++i) {
    float v = orc_half_to_float(x[(size_t)i * stride]);
    float q = rintf(v / s) + z;
    if (q < 0.0f) q = 0.0f;
    if (q > 255.0f) q = 255.0f;
    c[(size_t)i * cstride] = (uint8_t)q;
  }
  *s_out = s;
  *z_out = z;
}

/* The fp16 metadata format (a variant of the fp32 (scale, zero-point) pair of [G]'s quantizer,
 * which stores both in the input's dtype): from the fp32 s and z of a group, s and the offset
 * b = -(s z) -- the fp32 product, clamped to the finite half range -- each rounded to fp16.  A
 * code C then stands for s C + b = s (C - z) up to the roundings; a degenerate group (s clamped
 * to 1e-8, which rounds to 0) keeps its value in b. */
void orc_meta16(float s, float z, float* s16, float* b16) {
  float b = -(s * z);
  if (b > 65504.0f) b = 65504.0f;
  if (b < -65504.0f) b = -65504.0f;
  *s16 = orc_half_to_float(orc_float_to_half(s));
  *b16 = orc_half_to_float(orc_float_to_half(b));
}

/* Dequantizations with fp16 metadata (s, b), in fp64: s C8 + b (verify), s (2^4 C_U + off) + b
 * (draft). */
double orc_dequant16_full(uint8_t c8, float s, float b) {
  return (double)s * (double)c8 + (double)b;
}
double orc_dequant16_upper(uint8_t cu, float s, float b, int off) {
  return (double)s * (double)(16 * (int)cu + off) + (double)b;
}

/* C8 = 2^4 * C_U + C_L ([R] "What carries the argument", Fig. 3): the upper plane is the high
 * nibble and the lower "error-residual" plane the low nibble of the 8-bit code. */
static uint8_t upper_nibble(uint8_t c8) { return (uint8_t)(c8 >> 4); }
static uint8_t lower_nibble(uint8_t c8) { return (uint8_t)(c8 & 15); }

/* Target (verify) dequantization: (C8 - z) * s ([G] unpack_for_target), in fp64. */
double orc_dequant_full(uint8_t c8, float s, float z) {
  return ((double)c8 - (double)z) * (double)s;
}

/* Draft dequantization from the upper plane only: ((C_U << 4) + off - z) * s, off = 8 is the
 * midpoint centering of [G] unpack_for_draft, off = 0 the bare 2^4 * C_U of [R]. */
double orc_dequant_upper(uint8_t cu, float s, float z, int off) {
  return ((double)(16 * (int)cu + off) - (double)z) * (double)s;
}

/* A draft on the top k bits of the same 8-bit code, the verifier keeping all 8 ([R] "Editorial
 * extensions", "Reading between the lines": the 4/8 split generalizes to the top k bits for the
 * draft; the paper itself only uses k = 4).  The 8 - k dropped bits are replaced by off/16 of
 * their range, which for off = 8 sets the highest dropped bit -- [G]'s "| 0x08" centering of
 * the 4-bit draft, carried to every k -- and for k = 8 (nothing dropped) adds nothing.  So k = 4
 * is the draft above and k = 8 the verify dequantization. */
static int topk_code(uint8_t c8, int k, int off) {
  const int drop = 8 - k;
  return ((c8 >> drop) << drop) + ((off << drop) >> 4);
}
double orc_dequant_topk(uint8_t c8, float s, float z, int k, int off) {
  return ((double)topk_code(c8, k, off) - (double)z) * (double)s;
}
double orc_dequant16_topk(uint8_t c8, float s, float b, int k, int off) {
  return (double)s * (double)topk_code(c8, k, off) + (double)b;
}

/* ---------------------------------------------------------------------------------------- */
/* Cache                                                                                     */
/* ---------------------------------------------------------------------------------------- */

struct orc_cache {
  int L, B, H, D, G, T, NG, gamma_max, off;
  int meta16;       /* 1: ks/kz, vs/vz hold the fp16 (scale, offset) pairs, as floats   */
  uint8_t* kc;      /* [L][B][H][T][D] key codes                        */
  uint8_t* vc;      /* [L][B][H][T][D] value codes                      */
  float* ks;        /* [L][B][H][NG][D] key scale per group and channel */
  float* kz;        /* [L][B][H][NG][D] key zero-point                  */
  float* vs;        /* [L][B][H][T] value scale per token               */
  float* vz;        /* [L][B][H][T] value zero-point                    */
  uint16_t* tk;     /* [L][B][H][2G][D] fp16 tail ring (keys)           */
  uint16_t* tv;     /* [L][B][H][2G][D] fp16 tail ring (values)         */
  int* nq;          /* [L][B] quantized tokens                          */
  int* nt;          /* [L][B] tail tokens                               */
  int* head;        /* [L][B] ring slot of logical tail token 0         */
};

static size_t lbh(const orc_cache* c, int l, int b, int h) {
  return ((size_t)l * c->B + b) * c->H + h;
}

orc_cache* orc_create(int L, int B, int H, int D, int G, int T, int gamma_max, int off,
                      int meta16) {
  if (L < 1 || B < 1 || H < 1 || D < 2 || (D & 1) || G < 2 || (G & 1) || T < G || T % G ||
      gamma_max < 0 || gamma_max + 1 > G || (meta16 != 0 && meta16 != 1))
    return NULL;
  orc_cache* c = (orc_cache*)calloc(1, sizeof(orc_cache));
  if (!c) return NULL;
  c->L = L; c->B = B; c->H = H; c->D = D; c->G = G; c->T = T; c->NG = T / G;
  c->gamma_max = gamma_max; c->off = off; c->meta16 = meta16;
  size_t nbh = (size_t)L * B * H;
  c->kc = (uint8_t*)calloc(nbh * T * D, 1);
  c->vc = (uint8_t*)calloc(nbh * T * D, 1);
  c->ks = (float*)calloc(nbh * c->NG * D, sizeof(float));
  c->kz = (float*)calloc(nbh * c->NG * D, sizeof(float));
  c->vs = (float*)calloc(nbh * T, sizeof(float));
  c->vz = (float*)calloc(nbh * T, sizeof(float));
  c->tk = (uint16_t*)calloc(nbh * 2 * G * D, sizeof(uint16_t));
  c->tv = (uint16_t*)calloc(nbh * 2 * G * D, sizeof(uint16_t));
  c->nq = (int*)calloc((size_t)L * B, sizeof(int));
  c->nt = (int*)calloc((size_t)L * B, sizeof(int));
  c->head = (int*)calloc((size_t)L * B, sizeof(int));
  if (!c->kc || !c->vc || !c->ks || !c->kz || !c->vs || !c->vz || !c->tk || !c->tv || !c->nq ||
      !c->nt || !c->head) {
    orc_destroy(c);
    return NULL;
  }
  return c;
}

void orc_destroy(orc_cache* c) {
  if (!c) return;
  free(c->kc); free(c->vc); free(c->ks); free(c->kz); free(c->vs); free(c->vz);
  free(c->tk); free(c->tv); free(c->nq); free(c->nt); free(c->head);
  free(c);
}

/* Ring slot of logical tail position i of (l, b). */
static int slot_of(const orc_cache* c, int l, int b, int i) {
  return (c->head[l * c->B + b] + i) % (2 * c->G);
}

/* Tokens first .. first+count-1 of sequence b of k, v ([B][n_max][H][D]) to the back of the
 * full-precision buffer of (l, b). */
static void push_tokens(orc_cache* c, int l, int b, const uint16_t* k, const uint16_t* v,
                        int n_max, int first, int count) {
  int* nt = &c->nt[l * c->B + b];
  for (int i = 0; i < count; ++i) {
    int slot = slot_of(c, l, b, *nt + i);
    for (int h = 0; h < c->H; ++h) {
      const size_t src = (((size_t)b * n_max + first + i) * c->H + h) * c->D;
      const size_t dst = (lbh(c, l, b, h) * 2 * c->G + slot) * c->D;
      memcpy(&c->tk[dst], &k[src], (size_t)c->D * sizeof(uint16_t));
      memcpy(&c->tv[dst], &v[src], (size_t)c->D * sizeof(uint16_t));
    }
  }
  *nt += count;
}

/* New tokens go to the back of the full-precision buffer, unquantized ([G]
 * append_speculative_token; [R] "What carries the argument"). */
int orc_append(orc_cache* c, int layer, const uint16_t* k, const uint16_t* v, int n_max,
               const int* n) {
  if (!c || layer < 0 || layer >= c->L || !k || !v || n_max < 0) return 1;
  for (int b = 0; b < c->B; ++b) {
    int nb = n ? n[b] : n_max;
    if (nb < 0 || nb > n_max) return 1;
    if (c->nt[layer * c->B + b] + nb > 2 * c->G) return 2;
  }
  for (int b = 0; b < c->B; ++b) push_tokens(c, layer, b, k, v, n_max, 0, n ? n[b] : n_max);
  return 0;
}

/* Rejected speculative tokens are dropped from the full-precision buffer; the quantized tier
 * is never touched ([G] "Zero-Overhead Rollback"). */
int orc_rollback(orc_cache* c, int layer, const int* n_drop) {
  if (!c || layer < -1 || layer >= c->L) return 1;
  if (!n_drop) return 0;
  int l0 = layer < 0 ? 0 : layer, l1 = layer < 0 ? c->L : layer + 1;
  for (int l = l0; l < l1; ++l)
    for (int b = 0; b < c->B; ++b) {
      if (n_drop[b] < 0) return 1;
      if (n_drop[b] > c->nt[l * c->B + b]) return 3;
    }
  for (int l = l0; l < l1; ++l)
    for (int b = 0; b < c->B; ++b) c->nt[l * c->B + b] -= n_drop[b];
  return 0;
}

/* Quantizes the oldest G tail tokens (one ring half) of (l, b) into quantized group nq/G:
 * keys channel-wise over the G tokens, values token-wise over the D channels ([R] Fig. 7,
 * reference [128]); then the half is released ([G] "Periodic Group Quantization"). */
static void flush_one(orc_cache* c, int l, int b) {
  const int G = c->G, D = c->D;
  const int t0 = c->nq[l * c->B + b];
  const int g = t0 / G;
  const int head = c->head[l * c->B + b];
  for (int h = 0; h < c->H; ++h) {
    const size_t r = lbh(c, l, b, h);
    const uint16_t* tk = &c->tk[(r * 2 * G + head) * D]; /* G consecutive slots */
    const uint16_t* tv = &c->tv[(r * 2 * G + head) * D];
    uint8_t* kc = &c->kc[(r * c->T + t0) * D];
    uint8_t* vc = &c->vc[(r * c->T + t0) * D];
    for (int d = 0; d < D; ++d) /* key group: channel d over tokens t0 .. t0+G-1 */
      orc_quantize_group(&tk[d], G, D, &c->ks[(r * c->NG + g) * D + d],
                         &c->kz[(r * c->NG + g) * D + d], &kc[d], D);
    for (int t = 0; t < G; ++t) /* value group: token t over channels 0 .. D-1 */
      orc_quantize_group(&tv[(size_t)t * D], D, 1, &c->vs[r * c->T + t0 + t],
                         &c->vz[r * c->T + t0 + t], &vc[(size_t)t * D], 1);
    if (c->meta16) { /* the codes stay; the stored pairs become fp16 (scale, offset) */
      for (int d = 0; d < D; ++d) {
        float* ps = &c->ks[(r * c->NG + g) * D + d];
        float* pz = &c->kz[(r * c->NG + g) * D + d];
        orc_meta16(*ps, *pz, ps, pz);
      }
      for (int t = 0; t < G; ++t)
        orc_meta16(c->vs[r * c->T + t0 + t], c->vz[r * c->T + t0 + t], &c->vs[r * c->T + t0 + t],
                   &c->vz[r * c->T + t0 + t]);
    }
  }
  c->nq[l * c->B + b] += G;
  c->nt[l * c->B + b] -= G;
  c->head[l * c->B + b] = (head + G) % (2 * G);
}

/* "Quantize once": the prompt of sequence b (n_b tokens of k, v [B][n_max][H][D]) enters the
 * cache G tokens at a time, each group pushed through the full-precision buffer and quantized
 * once as it leaves ([G] "Core Architectural Blueprint" figure; "Periodic Group Quantization");
 * the n_b mod G remaining tokens stay in the buffer.  A prompt needs an empty buffer (its
 * tokens would otherwise come after younger ones).  Every sequence is checked first: 1 for a
 * bad argument, 3 for a non-empty buffer, 2 for a prompt past the capacity T. */
int orc_prefill(orc_cache* c, int layer, const uint16_t* k, const uint16_t* v, int n_max,
                const int* n) {
  if (!c || layer < 0 || layer >= c->L || !k || !v || n_max < 0) return 1;
  for (int b = 0; b < c->B; ++b) {
    int nb = n ? n[b] : n_max;
    if (nb < 0 || nb > n_max) return 1;
    if (nb == 0) continue;
    if (c->nt[layer * c->B + b] != 0) return 3;
    if (c->nq[layer * c->B + b] + (nb / c->G) * c->G > c->T) return 2;
  }
  for (int b = 0; b < c->B; ++b) {
    int nb = n ? n[b] : n_max;
    int g = 0;
    for (; (g + 1) * c->G <= nb; ++g) {
      push_tokens(c, layer, b, k, v, n_max, g * c->G, c->G);
      flush_one(c, layer, b);
    }
    push_tokens(c, layer, b, k, v, n_max, g * c->G, nb - g * c->G);
  }
  return 0;
}

int orc_flush(orc_cache* c, int layer, int min_tail, int* flushed) {
  if (!c || layer < -1 || layer >= c->L || min_tail > 2 * c->G) return 1;
  int need = min_tail > c->G ? min_tail : c->G;
  int l0 = layer < 0 ? 0 : layer, l1 = layer < 0 ? c->L : layer + 1;
  for (int l = l0; l < l1; ++l)
    for (int b = 0; b < c->B; ++b)
      if (c->nt[l * c->B + b] >= need && c->nq[l * c->B + b] + c->G > c->T) return 2;
  for (int l = l0; l < l1; ++l)
    for (int b = 0; b < c->B; ++b) {
      int sel = c->nt[l * c->B + b] >= need;
      if (sel) flush_one(c, l, b);
      if (flushed) flushed[b] = sel;
    }
  return 0;
}

/* ---------------------------------------------------------------------------------------- */
/* Attention                                                                                 */
/* ---------------------------------------------------------------------------------------- */

/* Dequantized code in the cache's metadata format from its top `bits` bits: 4 is the draft
 * (the upper plane), 8 the verify pass (both planes), 1..7 a top-k-bit draft. */
static double dequant(const orc_cache* c, uint8_t c8, float s, float x, int bits) {
  if (bits == 8) return c->meta16 ? orc_dequant16_full(c8, s, x) : orc_dequant_full(c8, s, x);
  if (bits == 4)
    return c->meta16 ? orc_dequant16_upper(upper_nibble(c8), s, x, c->off)
                     : orc_dequant_upper(upper_nibble(c8), s, x, c->off);
  return c->meta16 ? orc_dequant16_topk(c8, s, x, bits, c->off)
                   : orc_dequant_topk(c8, s, x, bits, c->off);
}

/* One query row of one (l, b, h): plain softmax attention in fp64 over the concatenation of
 *   - the nq quantized tokens, dequantized from the top `bits` bits of their codes (4: the draft
 *     formula, upper plane; 8: the verify formula, both planes), and
 *   - the first n_vis tail tokens in logical order (fp16 -> exact).
 * out_d = sum_j exp(s_j - max) v_jd / sum_j exp(s_j - max),  s_j = sm_scale * q . k_j. */
static void attend_row(const orc_cache* c, int l, int b, int h, const uint16_t* q, int bits,
                       int n_vis, double sm_scale, double* score, float* out) {
  const int D = c->D, G = c->G;
  const size_t r = lbh(c, l, b, h);
  const int nq = c->nq[l * c->B + b];
  const int n = nq + n_vis;
  double* qd = (double*)malloc((size_t)D * sizeof(double));
  double* acc = (double*)calloc((size_t)D, sizeof(double));
  for (int d = 0; d < D; ++d) qd[d] = orc_half_to_float(q[d]);

  for (int t = 0; t < nq; ++t) {
    const uint8_t* kc = &c->kc[(r * c->T + t) * D];
    const int g = t / G;
    double dot = 0.0;
    for (int d = 0; d < D; ++d) {
      float s = c->ks[(r * c->NG + g) * D + d], z = c->kz[(r * c->NG + g) * D + d];
      dot += qd[d] * dequant(c, kc[d], s, z, bits);
    }
    score[t] = sm_scale * dot;
  }
  for (int j = 0; j < n_vis; ++j) {
    const uint16_t* kt = &c->tk[(r * 2 * G + slot_of(c, l, b, j)) * D];
    double dot = 0.0;
    for (int d = 0; d < D; ++d) dot += qd[d] * (double)orc_half_to_float(kt[d]);
    score[nq + j] = sm_scale * dot;
  }

  double mx = -INFINITY;
  for (int j = 0; j < n; ++j)
    if (score[j] > mx) mx = score[j];
  double sum = 0.0;
  for (int j = 0; j < n; ++j) sum += exp(score[j] - mx);

  for (int t = 0; t < nq; ++t) {
    const double p = exp(score[t] - mx);
    const uint8_t* vc = &c->vc[(r * c->T + t) * D];
    const float s = c->vs[r * c->T + t], z = c->vz[r * c->T + t];
    for (int d = 0; d < D; ++d) acc[d] += p * dequant(c, vc[d], s, z, bits);
  }
  for (int j = 0; j < n_vis; ++j) {
    const double p = exp(score[nq + j] - mx);
    const uint16_t* vt = &c->tv[(r * 2 * G + slot_of(c, l, b, j)) * D];
    for (int d = 0; d < D; ++d) acc[d] += p * (double)orc_half_to_float(vt[d]);
  }
  for (int d = 0; d < D; ++d) out[d] = (float)(acc[d] / sum);
  free(qd);
  free(acc);
}

/* Draft pass on the top `bits` bits of every code (1..8); orc_attend_draft is bits = 4. */
int orc_attend_draft_bits(const orc_cache* c, int layer, const uint16_t* q, int bits,
                          double sm_scale, float* out) {
  if (!c || layer < 0 || layer >= c->L || !q || !out || bits < 1 || bits > 8) return 1;
  for (int b = 0; b < c->B; ++b)
    if (c->nq[layer * c->B + b] + c->nt[layer * c->B + b] == 0) return 3;
  double* score = (double*)malloc(((size_t)c->T + 2 * c->G) * sizeof(double));
  for (int b = 0; b < c->B; ++b)
    for (int h = 0; h < c->H; ++h) {
      const size_t row = ((size_t)b * c->H + h) * c->D;
      attend_row(c, layer, b, h, &q[row], bits, c->nt[layer * c->B + b], sm_scale, score,
                 &out[row]);
    }
  free(score);
  return 0;
}

int orc_attend_draft(const orc_cache* c, int layer, const uint16_t* q, double sm_scale,
                     float* out) {
  return orc_attend_draft_bits(c, layer, q, 4, sm_scale, out);
}

/* Query i of the verify block is the (nt - m + i)-th tail token itself: it sees the quantized
 * tier and tail positions 0 .. nt - m + i (causal). */
int orc_attend_verify(const orc_cache* c, int layer, const uint16_t* q, int m, double sm_scale,
                      float* out) {
  if (!c || layer < 0 || layer >= c->L || !q || !out || m < 1 || m > c->gamma_max + 1) return 1;
  for (int b = 0; b < c->B; ++b)
    if (m > c->nt[layer * c->B + b]) return 3;
  double* score = (double*)malloc(((size_t)c->T + 2 * c->G) * sizeof(double));
  for (int b = 0; b < c->B; ++b)
    for (int i = 0; i < m; ++i)
      for (int h = 0; h < c->H; ++h) {
        const size_t row = (((size_t)b * m + i) * c->H + h) * c->D;
        const int n_vis = c->nt[layer * c->B + b] - m + i + 1;
        attend_row(c, layer, b, h, &q[row], 8, n_vis, sm_scale, score, &out[row]);
      }
  free(score);
  return 0;
}

int orc_get_state(const orc_cache* c, int layer, int* nq, int* nt, int* head) {
  if (!c || layer < 0 || layer >= c->L) return 1;
  for (int b = 0; b < c->B; ++b) {
    if (nq) nq[b] = c->nq[layer * c->B + b];
    if (nt) nt[b] = c->nt[layer * c->B + b];
    if (head) head[b] = c->head[layer * c->B + b];
  }
  return 0;
}

/* Test support: sets the lower nibble of every stored code of `layer` (keys and values, rows
 * below nq) to `value`.  With value 8 and draft offset 8 the full code 16 C_U + 8 is exactly the
 * draft reconstruction's, so verify (m = 1) must then equal draft. */
int orc_set_lower_nibbles(orc_cache* c, int layer, int value) {
  if (!c || layer < 0 || layer >= c->L || value < 0 || value > 15) return 1;
  for (int b = 0; b < c->B; ++b)
    for (int h = 0; h < c->H; ++h) {
      const size_t r = lbh(c, layer, b, h);
      const size_t n = (size_t)c->nq[layer * c->B + b] * c->D;
      for (size_t i = 0; i < n; ++i) {
        uint8_t* k = &c->kc[r * c->T * c->D + i];
        uint8_t* v = &c->vc[r * c->T * c->D + i];
        *k = (uint8_t)((*k & 0xF0) | value);
        *v = (uint8_t)((*v & 0xF0) | value);
      }
    }
  return 0;
}

/* Test support: sets the low `nbits` bits (1..7) of every stored code of `layer` to `value`.
 * With nbits = 8 - k and value = the k-bit draft's replacement of the dropped bits, every code
 * equals its top-k reconstruction, so verify (m = 1) must equal the k-bit draft. */
int orc_set_low_bits(orc_cache* c, int layer, int nbits, int value) {
  if (!c || layer < 0 || layer >= c->L || nbits < 1 || nbits > 7 || value < 0 ||
      value >= (1 << nbits))
    return 1;
  const int keep = 0xFF ^ ((1 << nbits) - 1);
  for (int b = 0; b < c->B; ++b)
    for (int h = 0; h < c->H; ++h) {
      const size_t r = lbh(c, layer, b, h);
      const size_t n = (size_t)c->nq[layer * c->B + b] * c->D;
      for (size_t i = 0; i < n; ++i) {
        uint8_t* k = &c->kc[r * c->T * c->D + i];
        uint8_t* v = &c->vc[r * c->T * c->D + i];
        *k = (uint8_t)((*k & keep) | value);
        *v = (uint8_t)((*v & keep) | value);
      }
    }
  return 0;
}

int orc_read_codes(const orc_cache* c, int layer, int b, int h, int which_v, uint8_t* codes) {
  if (!c || layer < 0 || layer >= c->L || b < 0 || b >= c->B || h < 0 || h >= c->H || !codes)
    return 1;
  const size_t r = lbh(c, layer, b, h);
  memcpy(codes, &(which_v ? c->vc : c->kc)[r * c->T * c->D], (size_t)c->T * c->D);
  return 0;
}

int orc_read_meta(const orc_cache* c, int layer, int b, int h, float* kmeta, float* vmeta) {
  if (!c || layer < 0 || layer >= c->L || b < 0 || b >= c->B || h < 0 || h >= c->H) return 1;
  const size_t r = lbh(c, layer, b, h);
  if (kmeta)
    for (size_t i = 0; i < (size_t)c->NG * c->D; ++i) {
      kmeta[2 * i] = c->ks[r * c->NG * c->D + i];
      kmeta[2 * i + 1] = c->kz[r * c->NG * c->D + i];
    }
  if (vmeta)
    for (int t = 0; t < c->T; ++t) {
      vmeta[2 * t] = c->vs[r * c->T + t];
      vmeta[2 * t + 1] = c->vz[r * c->T + t];
    }
  return 0;
}

/* Arena layout of one layer, written out index by index from its definition:
 *   key planes   [B][H][T][D/2]         byte j of token row t: channel 2j in bits 0-3, 2j+1 in
 *                                       bits 4-7
 *   value planes [B][H][NG][2][D][G/4]  byte j of channel row d of half e of group g: token
 *                                       gG + eG/2 + 2j in bits 0-3, the next token in bits 4-7
 *   kmeta [B][H][NG][D][2], vmeta [B][H][T][2], tails [B][H][2G][D] (ring slots). */
int orc_export_layer(const orc_cache* c, int layer, uint8_t* uk, uint8_t* lk, uint8_t* uv,
                     uint8_t* lv, float* kmeta, float* vmeta, uint16_t* tail_k,
                     uint16_t* tail_v) {
  if (!c || layer < 0 || layer >= c->L) return 1;
  const int D = c->D, G = c->G, T = c->T, NG = c->NG;
  for (int b = 0; b < c->B; ++b)
    for (int h = 0; h < c->H; ++h) {
      const size_t r = lbh(c, layer, b, h);
      const size_t bh = (size_t)b * c->H + h;
      const int nq = c->nq[layer * c->B + b];
      for (int t = 0; t < T; ++t)
        for (int j = 0; j < D / 2; ++j) {
          uint8_t c0 = t < nq ? c->kc[(r * T + t) * D + 2 * j] : 0;
          uint8_t c1 = t < nq ? c->kc[(r * T + t) * D + 2 * j + 1] : 0;
          size_t o = (bh * T + t) * (D / 2) + j;
          if (uk) uk[o] = (uint8_t)(upper_nibble(c0) | (upper_nibble(c1) << 4));
          if (lk) lk[o] = (uint8_t)(lower_nibble(c0) | (lower_nibble(c1) << 4));
        }
      for (int g = 0; g < NG; ++g)
        for (int e = 0; e < 2; ++e)
          for (int d = 0; d < D; ++d)
            for (int j = 0; j < G / 4; ++j) {
              int t0 = g * G + e * (G / 2) + 2 * j, t1 = t0 + 1;
              uint8_t c0 = t0 < nq ? c->vc[(r * T + t0) * D + d] : 0;
              uint8_t c1 = t1 < nq ? c->vc[(r * T + t1) * D + d] : 0;
              size_t o = (((bh * NG + g) * 2 + e) * D + d) * (G / 4) + j;
              if (uv) uv[o] = (uint8_t)(upper_nibble(c0) | (upper_nibble(c1) << 4));
              if (lv) lv[o] = (uint8_t)(lower_nibble(c0) | (lower_nibble(c1) << 4));
            }
      if (kmeta)
        for (int g = 0; g < NG; ++g)
          for (int d = 0; d < D; ++d) {
            size_t o = ((bh * NG + g) * D + d) * 2;
            int live = (g + 1) * G <= nq;
            kmeta[o] = live ? c->ks[(r * NG + g) * D + d] : 0.0f;
            kmeta[o + 1] = live ? c->kz[(r * NG + g) * D + d] : 0.0f;
          }
      if (vmeta)
        for (int t = 0; t < T; ++t) {
          vmeta[(bh * T + t) * 2] = t < nq ? c->vs[r * T + t] : 0.0f;
          vmeta[(bh * T + t) * 2 + 1] = t < nq ? c->vz[r * T + t] : 0.0f;
        }
      if (tail_k)
        memcpy(&tail_k[bh * 2 * G * D], &c->tk[r * 2 * G * D], (size_t)2 * G * D * 2);
      if (tail_v)
        memcpy(&tail_v[bh * 2 * G * D], &c->tv[r * 2 * G * D], (size_t)2 * G * D * 2);
    }
  return 0;
}

/* The upper planes of the split-upper layout, in which the upper nibble C_U = 4 C_T + C_M of
 * every code is stored as two 2-bit planes, the top bits C_T = C8 >> 6 and the middle bits
 * C_M = (C8 >> 4) & 3, so that a 2-bit draft reads the C_T plane alone, a 4-bit draft both, and
 * verify both with the lower plane (unchanged, as in orc_export_layer).  A plane row is made of
 * 32-bit little-endian words, word w covering 16 entries 16w .. 16w+15 (channels of a key row,
 * tokens of a value row); nibble e (bits 4e .. 4e+3) of a word holds
 *   C_T plane: C_T(16w + e) in bits 4e+2 .. 4e+3, C_T(16w + 8 + e) in bits 4e .. 4e+1;
 *   C_M plane: C_M(16w + e) in bits 4e .. 4e+1,   C_M(16w + 8 + e) in bits 4e+2 .. 4e+3.
 * Shapes: key planes [B][H][T][D/4]; value planes [B][H][NG][2][D][G/8] (half e of group g,
 * channel d: tokens gG + eG/2 + 16w + ...).  Rows past nq are zero. */
static void split_word(const uint8_t* code16, size_t stride, uint8_t* tw, uint8_t* mw) {
  uint32_t t = 0, m = 0;
  for (int e = 0; e < 8; ++e) {
    const uint8_t a = code16[(size_t)e * stride], b = code16[(size_t)(8 + e) * stride];
    t |= (uint32_t)(a >> 6) << (4 * e + 2);
    t |= (uint32_t)(b >> 6) << (4 * e);
    m |= (uint32_t)((a >> 4) & 3) << (4 * e);
    m |= (uint32_t)((b >> 4) & 3) << (4 * e + 2);
  }
  for (int j = 0; j < 4; ++j) {
    tw[j] = (uint8_t)(t >> (8 * j));
    mw[j] = (uint8_t)(m >> (8 * j));
  }
}

int orc_export_upper_split(const orc_cache* c, int layer, uint8_t* tk, uint8_t* mk, uint8_t* tv,
                           uint8_t* mv) {
  if (!c || layer < 0 || layer >= c->L || !tk || !mk || !tv || !mv || c->D % 16 || c->G % 32)
    return 1;
  const int D = c->D, G = c->G, T = c->T, NG = c->NG;
  for (int b = 0; b < c->B; ++b)
    for (int h = 0; h < c->H; ++h) {
      const size_t r = lbh(c, layer, b, h);
      const size_t bh = (size_t)b * c->H + h;
      const int nq = c->nq[layer * c->B + b];
      for (int t = 0; t < T; ++t)
        for (int w = 0; w < D / 16; ++w) {
          const size_t o = (bh * T + t) * (D / 4) + 4 * w;
          if (t < nq) {
            split_word(&c->kc[(r * T + t) * D + 16 * w], 1, &tk[o], &mk[o]);
          } else {
            memset(&tk[o], 0, 4);
            memset(&mk[o], 0, 4);
          }
        }
      for (int g = 0; g < NG; ++g)
        for (int e = 0; e < 2; ++e)
          for (int d = 0; d < D; ++d)
            for (int w = 0; w < G / 32; ++w) {
              const int t0 = g * G + e * (G / 2) + 16 * w;
              const size_t o = (((bh * NG + g) * 2 + e) * D + d) * (G / 8) + 4 * w;
              if (t0 + 16 <= nq) {
                split_word(&c->vc[(r * T + t0) * D + d], (size_t)D, &tv[o], &mv[o]);
              } else {
                memset(&tv[o], 0, 4);
                memset(&mv[o], 0, 4);
              }
            }
    }
  return 0;
}

/* ---------------------------------------------------------------------------------------- */
/* Speculative accept / correct                                                              */
/* ---------------------------------------------------------------------------------------- */

/* softmax of one row in fp64, into out */
static void softmax_row(const float* x, int V, double* out) {
  double m = -INFINITY;
  for (int v = 0; v < V; ++v)
    if ((double)x[v] > m) m = x[v];
  double s = 0.0;
  for (int v = 0; v < V; ++v) {
    out[v] = m == -INFINITY ? 0.0 : exp((double)x[v] - m);
    s += out[v];
  }
  for (int v = 0; v < V; ++v) out[v] = s > 0.0 ? out[v] / s : 0.0;
}

/* The step after the target's verify pass, per sequence b ([G] "The Self-Speculative
 * Verification Loop" listing for the acceptance test; [R] major comment 1 on Algorithm 1 for
 * the correction from the normalised residual (p - q)_+, minor comment 5 for the token after
 * gamma acceptances, from p_{gamma+1}), in fp64:
 *   p_i = softmax(t_i) (rows 0 .. gamma), q_i = softmax(d_i) (rows 0 .. gamma-1);
 *   drafted token x_i is accepted iff u_i <= min(1, p_i(x_i) / (q_i(x_i) + 1e-8)), for
 *   i = 0, 1, .. until the first rejection j (a token outside [0, V) is rejected);
 *   the next token is the smallest v with sum_{w <= v} r(w) > u_gamma * sum_w r(w), where r is
 *   (p_j - q_j)_+ after a rejection at j, p_gamma after gamma acceptances, and p_j if the
 *   residual sums to zero.
 * margin[b] (test support, may be NULL): how far the decisions were from flipping -- the
 * smallest |u_i - min(1, ratio_i)| over the tests made, and for the sample the distance of
 * u_gamma from the CDF values around the chosen token, both in units of probability. */
int orc_spec_accept(const float* t, const float* d, const int* tokens, const float* u, int B,
                    int gamma, int V, int* n_acc, int* next, double* margin) {
  if (!t || !d || !tokens || !u || !n_acc || !next || B < 1 || gamma < 1 || V < 1) return 1;
  double* p = (double*)malloc(sizeof(double) * V);
  double* q = (double*)malloc(sizeof(double) * V);
  double* r = (double*)malloc(sizeof(double) * V);
  if (!p || !q || !r) {
    free(p); free(q); free(r);
    return 1;
  }
  for (int b = 0; b < B; ++b) {
    const float* tb = t + (size_t)b * (gamma + 1) * V;
    const float* db = d + (size_t)b * gamma * V;
    const float* ub = u + (size_t)b * (gamma + 1);
    double mg = INFINITY;
    int j = 0;
    for (; j < gamma; ++j) {
      const int x = tokens[(size_t)b * gamma + j];
      if (x < 0 || x >= V) break;
      softmax_row(tb + (size_t)j * V, V, p);
      softmax_row(db + (size_t)j * V, V, q);
      double acc = p[x] / (q[x] + 1e-8);
      if (acc > 1.0) acc = 1.0;
      const double gap = fabs((double)ub[j] - acc);
      if (gap < mg) mg = gap;
      if (!((double)ub[j] <= acc)) break;
    }
    softmax_row(tb + (size_t)j * V, V, p);
    double total = 0.0;
    if (j < gamma) {
      softmax_row(db + (size_t)j * V, V, q);
      for (int v = 0; v < V; ++v) {
        r[v] = p[v] > q[v] ? p[v] - q[v] : 0.0;
        total += r[v];
      }
    }
    if (total <= 0.0) {
      total = 0.0;
      for (int v = 0; v < V; ++v) {
        r[v] = p[v];
        total += r[v];
      }
    }
    int tok = 0;
    if (total > 0.0) {
      const double target = (double)ub[gamma] * total;
      double c = 0.0;
      tok = -1;
      for (int v = 0; v < V; ++v) {
        const double prev = c;
        c += r[v];
        if (c > target) {
          tok = v;
          const double gap = (target - prev) < (c - target) ? (target - prev) : (c - target);
          if (gap / total < mg) mg = gap / total;
          break;
        }
      }
      if (tok < 0)
        for (int v = V - 1; v >= 0; --v)
          if (r[v] > 0.0) {
            tok = v;
            break;
          }
    }
    n_acc[b] = j;
    next[b] = tok;
    if (margin) margin[b] = mg;
  }
  free(p); free(q); free(r);
  return 0;
}

