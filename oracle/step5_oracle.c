/*
 * Step-5 sparse-indexer path: CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the slow, plain reference that the
 * GPU library is checked against. Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark load it. The GPU library never includes,
 * links or calls anything here, and nothing here includes the GPU library's
 * headers.
 *
 * Sources (web pages; cited by title and section):
 *  [TF903-idx]   TensorFold pull request #903, "Step-5-Preview on one 256 GB
 *                Mac", commit note that turns on StepFun's CSA indexer for
 *                contexts to 1M tokens. It fixes the indexer's arithmetic:
 *                q = 16 heads with RMSNorm scaled by (1 + w); k = LayerNorm with
 *                bias; NEOX rotation of the first 32 dims; every completed
 *                8-token region summarised per dim as a softmax over z of k,
 *                rounded through bf16 to e4m3; a region's score is the sum over
 *                the group's heads of relu(e4m3(q_h) . summary) * w_h; the top
 *                512 by (-score, id) ascending; attention over those regions
 *                and the row's own region.
 *  [TF903-glue]  Same page, commit note on the native Step-5 family: the glue
 *                keeps StepFun's rounding points, among them zero-centred
 *                norms and the NEOX rotation read from bf16 cos/sin.
 *  [VLLM-proj]   vLLM, "vllm.models.step5.nvidia.model", class
 *                Step5FusedQKVIndexerLinear: the main attention's q, k, v and
 *                the indexer's q, k, z and the gate come from one product
 *                hidden @ W^T of the normed hidden state with one weight whose
 *                rows are [q | k | v | index_q | index_k | index_z | gate],
 *                split by column afterwards (split_indexer).
 *  [TF903-ref]   Same page, first commit note: the reference attends densely,
 *                which is exact while the indexer selects every region.
 *
 * Where the pages leave a rounding point or an order open, the reading used
 * here is the plainest one and is listed in the design notes of the
 * repository; every such choice is marked "reading:" below.
 *
 * Floating point: compile with -O2 -ffp-contract=off -fno-fast-math. Every
 * float operation below is one IEEE-754 binary32 operation rounded to nearest
 * even, unless it is written in double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#define O_OK 0
#define O_BAD 1

/* Geometry this oracle implements (the Step-5 DSA layer shapes). */
#define IDX_DIM 64   /* indexer head dim */
#define ROT_DIM 32   /* NEOX-rotated dims, pairs (i, i + 16) */
#define REGION 8     /* tokens per region */

/* ------------------------------------------------------------------------ */
/* Number formats                                                           */
/* ------------------------------------------------------------------------ */

float o_bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* fp32 -> bf16, round to nearest, ties to even (finite inputs). */
uint16_t o_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

/* OCP E4M3 (e4m3fn): 1 sign, 4 exponent bits (bias 7), 3 mantissa bits,
 * subnormals, no infinities, 0x7f/0xff are NaN, largest finite 448. */
double o_e4m3_to_f64(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) v = ldexp((double)m, -9);
  else v = ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

float o_e4m3_to_f32(uint8_t c) { return (float)o_e4m3_to_f64(c); }

/* bf16 -> e4m3: the nearest finite e4m3 value, ties to the even code.
 * reading: magnitudes past 448 saturate to 448 (no value in the path reaches
 * it: normalised, rotated and softmax-averaged data stay far below).
 * The search below walks the sorted table of non-negative codes, so that the
 * rule can be checked by eye. */
uint8_t o_bf16_to_e4m3(uint16_t h) {
  double v = (double)o_bf16_to_f32(h);
  uint8_t sign = (h & 0x8000u) ? 0x80 : 0x00;
  double a = fabs(v);
  if (a != a) return 0x7f | sign;
  if (a >= 448.0) return 0x7e | sign;
  /* largest code c in [0, 126] with value(c) <= a (codes are monotonic) */
  int lo = 0, hi = 126;
  while (lo < hi) {
    int mid = (lo + hi + 1) / 2;
    if (o_e4m3_to_f64((uint8_t)mid) <= a) lo = mid; else hi = mid - 1;
  }
  int c = lo;
  double below = o_e4m3_to_f64((uint8_t)c), above = o_e4m3_to_f64((uint8_t)(c + 1));
  double dlo = a - below, dhi = above - a;
  int pick;
  if (dlo < dhi) pick = c;
  else if (dhi < dlo) pick = c + 1;
  else pick = (c & 1) ? c + 1 : c;
  /* -0 keeps its sign bit (code 0x80), like every other value */
  return (uint8_t)pick | sign;
}

/* ------------------------------------------------------------------------ */
/* exp                                                                      */
/* ------------------------------------------------------------------------ */
/*
 * reading: the pages name a softmax but no exp routine. Bit-exact e4m3
 * summaries need one exp that every implementation computes identically, so
 * the path fixes it: Cody & Waite's (1980) reduction x = n*ln2 + r with
 * |r| <= ln2/2 and ln2 split in two parts, then e^r from its Taylor series
 * to degree 7 (coefficients 1/k!) in Horner form with fused multiply-adds,
 * then scaling by 2^n. Arguments below -87 are raised to -87, which keeps
 * every result a normal float (a softmax term that small is 0 to fp32
 * anyway next to the max term, which is exactly 1).
 */
#define O_L2E 0x1.715476p+0f        /* fp32(1 / ln 2) */
#define O_LN2_HI 0x1.62e4p-1f      /* ln 2 cut to 15 significant bits */
#define O_LN2_LO 0x1.7f7d1cp-20f   /* fp32(ln 2 - O_LN2_HI) */

float o_exp(float x) {
  static const float c[8] = {
      1.0f, 1.0f, 0.5f,
      0x1.555556p-3f,   /* fp32(1/6)    */
      0x1.555556p-5f,   /* fp32(1/24)   */
      0x1.111112p-7f,   /* fp32(1/120)  */
      0x1.6c16c2p-10f,  /* fp32(1/720)  */
      0x1.a01a02p-13f}; /* fp32(1/5040) */
  if (x < -87.0f) x = -87.0f;
  if (x > 88.0f) x = 88.0f;
  float t = x * O_L2E;
  float n = nearbyintf(t);
  float r = fmaf(-n, O_LN2_HI, x);
  r = fmaf(-n, O_LN2_LO, r);
  float p = c[7];
  for (int k = 6; k >= 0; --k) p = fmaf(p, r, c[k]);
  return ldexpf(p, (int)n);
}

/* ------------------------------------------------------------------------ */
/* Sums over the 64 dims of a head                                          */
/* ------------------------------------------------------------------------ */
/*
 * reading: the norms need mean(x) and mean(x^2) over 64 dims; the pages give
 * no order. The order fixed here is blocked pairwise: each run of 8 dims is
 * summed as a halving tree (strides 4, 2, 1) and the 8 run sums are summed
 * the same way.
 */
static float pair8(const float* a) {
  float b0 = a[0] + a[4], b1 = a[1] + a[5], b2 = a[2] + a[6], b3 = a[3] + a[7];
  float c0 = b0 + b2, c1 = b1 + b3;
  return c0 + c1;
}

float o_sum64(const float* x) {
  float s[8];
  for (int c = 0; c < 8; ++c) s[c] = pair8(x + 8 * c);
  return pair8(s);
}

/* NEOX rotation of dims [0, 32) at one position [TF903-idx, TF903-glue]:
 * pairs (i, i+16); cos_i and sin_i read from the bf16 table row of the
 * position (layout: cos_0..cos_15 | sin_0..sin_15). */
static void rope32(float* y, const uint16_t* cs_row) {
  float a[16], b[16];
  for (int i = 0; i < 16; ++i) { a[i] = y[i]; b[i] = y[i + 16]; }
  for (int i = 0; i < 16; ++i) {
    float c = o_bf16_to_f32(cs_row[i]), s = o_bf16_to_f32(cs_row[16 + i]);
    float ac = a[i] * c, bs = b[i] * s, bc = b[i] * c, as = a[i] * s;
    y[i] = ac - bs;
    y[i + 16] = bc + as;
  }
}

/* ------------------------------------------------------------------------ */
/* Step a1: indexer q prep [TF903-idx]                                      */
/* ------------------------------------------------------------------------ */
/* One head: RMSNorm over 64 dims with scale (1 + w) ("zero-centred"
 * [TF903-glue]), NEOX rotation at the row's position, bf16, then e4m3.
 * reading: fp32 throughout, one bf16 rounding at the end, then e4m3 of that
 * bf16 value (the summaries take the same bf16 -> e4m3 route). */
void o_q_prep_head(const uint16_t* x16, const float* w, float eps, const uint16_t* cs_row,
                   uint8_t* out) {
  float x[IDX_DIM], sq[IDX_DIM], y[IDX_DIM];
  for (int i = 0; i < IDX_DIM; ++i) { x[i] = o_bf16_to_f32(x16[i]); sq[i] = x[i] * x[i]; }
  float ms = o_sum64(sq) / 64.0f;
  float r = 1.0f / sqrtf(ms + eps);
  for (int i = 0; i < IDX_DIM; ++i) {
    float scale = 1.0f + w[i];
    y[i] = (x[i] * r) * scale;
  }
  rope32(y, cs_row);
  for (int i = 0; i < IDX_DIM; ++i) out[i] = o_bf16_to_e4m3(o_f32_to_bf16(y[i]));
}

/* q: bf16 [rows, idx_heads, 64] (row stride q_stride_row elements);
 * out: e4m3 [rows, idx_heads, 64]. */
int o_q_prep(const uint16_t* q, int64_t rows, int32_t idx_heads, int64_t q_stride_row,
             const float* w, float eps, const uint16_t* rope, int64_t rope_rows,
             const int64_t* row_pos, uint8_t* out, int nthreads) {
  for (int64_t r = 0; r < rows; ++r)
    if (row_pos[r] < 0 || row_pos[r] >= rope_rows) return O_BAD;
#pragma omp parallel for num_threads(nthreads) schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int h = 0; h < idx_heads; ++h)
      o_q_prep_head(q + r * q_stride_row + (int64_t)h * IDX_DIM, w, eps,
                    rope + row_pos[r] * ROT_DIM, out + (r * idx_heads + h) * IDX_DIM);
  return O_OK;
}

/* ------------------------------------------------------------------------ */
/* Step a2: indexer k prep [TF903-idx]                                      */
/* ------------------------------------------------------------------------ */
/* One (token, group): LayerNorm over 64 dims with weight and bias (biased
 * variance), NEOX rotation at the token's position, then bf16 (returned as
 * the fp32 value of that bf16). */
void o_k_prep_vec(const uint16_t* x16, const float* g, const float* b, float eps,
                  const uint16_t* cs_row, float* out) {
  float x[IDX_DIM], d[IDX_DIM], d2[IDX_DIM], y[IDX_DIM];
  for (int i = 0; i < IDX_DIM; ++i) x[i] = o_bf16_to_f32(x16[i]);
  float mu = o_sum64(x) / 64.0f;
  for (int i = 0; i < IDX_DIM; ++i) { d[i] = x[i] - mu; d2[i] = d[i] * d[i]; }
  float var = o_sum64(d2) / 64.0f;
  float r = 1.0f / sqrtf(var + eps);
  for (int i = 0; i < IDX_DIM; ++i) {
    float t = (d[i] * r) * g[i];
    y[i] = t + b[i];
  }
  rope32(y, cs_row);
  for (int i = 0; i < IDX_DIM; ++i) out[i] = o_bf16_to_f32(o_f32_to_bf16(y[i]));
}

/* ------------------------------------------------------------------------ */
/* Step a3: region summary [TF903-idx]                                      */
/* ------------------------------------------------------------------------ */
/* One (region, group): for each dim, softmax over the region's 8 tokens of
 * the raw z, weighting the prepared k; the weighted mean is rounded to bf16
 * and then to e4m3.
 * reading: max-subtracted softmax, unnormalised numerator and denominator
 * summed in token order, one division. */
void o_summary_vec(const float kp[REGION][IDX_DIM], const uint16_t* const z16[REGION],
                   uint8_t* out, double* shadow) {
  for (int dd = 0; dd < IDX_DIM; ++dd) {
    float z[REGION], e[REGION];
    for (int t = 0; t < REGION; ++t) z[t] = o_bf16_to_f32(z16[t][dd]);
    float m = z[0];
    for (int t = 1; t < REGION; ++t) m = fmaxf(m, z[t]);
    for (int t = 0; t < REGION; ++t) e[t] = o_exp(z[t] - m);
    float den = e[0];
    for (int t = 1; t < REGION; ++t) den = den + e[t];
    float num = e[0] * kp[0][dd];
    for (int t = 1; t < REGION; ++t) {
      float p = e[t] * kp[t][dd];
      num = num + p;
    }
    float s = num / den;
    out[dd] = o_bf16_to_e4m3(o_f32_to_bf16(s));
    if (shadow) {
      double m64 = (double)m, n64 = 0.0, d64 = 0.0;
      for (int t = 0; t < REGION; ++t) {
        double w = exp((double)z[t] - m64);
        d64 += w;
        n64 += w * (double)kp[t][dd];
      }
      shadow[dd] = n64 / d64;
    }
  }
}

/* k, z: bf16 [B, T, groups, 64] (element strides stride_b, stride_t; the 64
 * dims of a group are contiguous, groups are 64 apart), covering absolute
 * positions t0 .. t0 + T - 1 of each sequence, t0 a multiple of 8.
 * Writes summary[b][j] for every region j completed inside the span,
 * j = t0/8 .. (t0 + T)/8 - 1; summary is e4m3 [B, R_cap, groups, 64] with
 * batch stride s_stride_b bytes. shadow (nullable) gets the fp64 softmax
 * mean of the same bf16 k values, in summary's layout with R_cap regions. */
int o_summarize(const uint16_t* k, const uint16_t* z, int64_t B, int64_t T, int64_t t0,
                int32_t groups, int64_t stride_b, int64_t stride_t, const float* ln_w,
                const float* ln_b, float eps, const uint16_t* rope, int64_t rope_rows,
                uint8_t* summary, int64_t s_stride_b, int64_t R_cap, double* shadow,
                int nthreads) {
  if (t0 < 0 || t0 % REGION != 0 || T < 0) return O_BAD;
  int64_t j0 = t0 / REGION, nreg = T / REGION;
  if (j0 + nreg > R_cap || t0 + nreg * REGION > rope_rows) return O_BAD;
  int64_t units = B * nreg;
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 64)
  for (int64_t u = 0; u < units; ++u) {
    int64_t b = u / nreg, jr = u % nreg;
    for (int g = 0; g < groups; ++g) {
      float kp[REGION][IDX_DIM];
      const uint16_t* zp[REGION];
      for (int t = 0; t < REGION; ++t) {
        int64_t tl = jr * REGION + t;
        int64_t off = b * stride_b + tl * stride_t + (int64_t)g * IDX_DIM;
        o_k_prep_vec(k + off, ln_w, ln_b, eps, rope + (t0 + tl) * ROT_DIM, kp[t]);
        zp[t] = z + off;
      }
      int64_t so = b * s_stride_b + ((j0 + jr) * groups + g) * IDX_DIM;
      double* sh = shadow ? shadow + (b * R_cap + (j0 + jr)) * groups * IDX_DIM + g * IDX_DIM : NULL;
      o_summary_vec((const float(*)[IDX_DIM])kp, zp, summary + so, sh);
    }
  }
  return O_OK;
}

/* ------------------------------------------------------------------------ */
/* Step a4: region scores [TF903-idx]                                       */
/* ------------------------------------------------------------------------ */
/* Row r sits at absolute position p = row_pos[r] of sequence row_seq[r].
 * reading: its candidates are the completed regions before its own,
 * j < floor(p / 8); the own region is attended, never scored.
 * score(r, g, j) = sum over the group's heads h of relu(q8_h . S[j, g]) * w_h.
 * reading: each dot product is the exact sum (every e4m3 product is exact
 * and 64 of them add exactly in fp64) rounded once to fp32; relu maps -0 to
 * +0; the weighted terms are rounded products added in head order.
 * scores: fp32 [rows, groups, R_cap]; entries j >= floor(p/8) are left as
 * they were. w_head: fp32 [rows or 1, idx_heads] with row stride w_stride_row. */
int o_score(const uint8_t* q8, int32_t idx_heads, int32_t groups, const float* w_head,
            int64_t w_stride_row, const int32_t* row_seq, const int64_t* row_pos, int64_t rows,
            const uint8_t* summary, int64_t B, int64_t R_cap, int64_t s_stride_b, float* scores,
            int nthreads) {
  int hpg = idx_heads / groups;
  for (int64_t r = 0; r < rows; ++r) {
    if (row_seq[r] < 0 || row_seq[r] >= B || row_pos[r] < 0) return O_BAD;
    if (row_pos[r] / REGION > R_cap) return O_BAD;
  }
  int64_t units = rows * groups;
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
  for (int64_t u = 0; u < units; ++u) {
    int64_t r = u / groups;
    int g = (int)(u % groups);
    int64_t ncand = row_pos[r] / REGION;
    const uint8_t* S = summary + (int64_t)row_seq[r] * s_stride_b;
    const float* w = w_head + r * w_stride_row;
    double qv[16][IDX_DIM];
    for (int hh = 0; hh < hpg; ++hh)
      for (int d = 0; d < IDX_DIM; ++d)
        qv[hh][d] = o_e4m3_to_f64(q8[(r * idx_heads + g * hpg + hh) * IDX_DIM + d]);
    for (int64_t j = 0; j < ncand; ++j) {
      const uint8_t* sv = S + (j * groups + g) * IDX_DIM;
      double s64[IDX_DIM];
      for (int d = 0; d < IDX_DIM; ++d) s64[d] = o_e4m3_to_f64(sv[d]);
      float acc = 0.0f;
      for (int hh = 0; hh < hpg; ++hh) {
        double dot = 0.0;
        for (int d = 0; d < IDX_DIM; ++d) dot += qv[hh][d] * s64[d];
        float t = (float)dot;
        if (!(t > 0.0f)) t = 0.0f;
        float term = t * w[g * hpg + hh];
        acc = (hh == 0) ? term : acc + term;
      }
      scores[(r * groups + g) * R_cap + j] = acc;
    }
  }
  return O_OK;
}

/* ------------------------------------------------------------------------ */
/* Step a5: top-k selection [TF903-idx]                                     */
/* ------------------------------------------------------------------------ */
/* The min(topk, ncand) candidates first in the strict order (-score, id),
 * listed in that order (best first, equal scores by smaller id); the rest of
 * the topk slots are -1. -0 and +0 compare equal. */
typedef struct { float s; int32_t id; } o_cand;

static int o_cand_cmp(const void* pa, const void* pb) {
  const o_cand* a = (const o_cand*)pa;
  const o_cand* b = (const o_cand*)pb;
  if (a->s > b->s) return -1;
  if (a->s < b->s) return 1;
  return (a->id < b->id) ? -1 : (a->id > b->id);
}

int o_select(const float* scores, const int64_t* row_pos, int64_t rows, int32_t groups,
             int64_t R_cap, int32_t topk, int32_t* ids, float* sel_scores, int nthreads) {
  for (int64_t r = 0; r < rows; ++r)
    if (row_pos[r] < 0 || row_pos[r] / REGION > R_cap) return O_BAD;
  int64_t units = rows * groups;
  int bad = 0;
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
  for (int64_t u = 0; u < units; ++u) {
    int64_t ncand = row_pos[u / groups] / REGION;
    o_cand* c = (o_cand*)malloc((size_t)(ncand > 0 ? ncand : 1) * sizeof(o_cand));
    if (!c) { bad = 1; continue; }
    for (int64_t j = 0; j < ncand; ++j) { c[j].s = scores[u * R_cap + j]; c[j].id = (int32_t)j; }
    qsort(c, (size_t)ncand, sizeof(o_cand), o_cand_cmp);
    for (int32_t i = 0; i < topk; ++i) {
      int have = i < ncand;
      ids[u * topk + i] = have ? c[i].id : -1;
      if (sel_scores) sel_scores[u * topk + i] = have ? c[i].s : 0.0f;
    }
    free(c);
  }
  return bad ? O_BAD : O_OK;
}

/* ------------------------------------------------------------------------ */
/* Step a6: sparse attention [TF903-idx, TF903-ref]                         */
/* ------------------------------------------------------------------------ */
/* Row r (position p, sequence b) and query head h read KV head g = h / (q_heads / kv_heads)
 * over the tokens of its group's selected regions (ids >= 0 in sel) plus its
 * own region's tokens 8*floor(p/8) .. p; o = softmax(scale * q.K) V.
 * In fp64 from the bf16 inputs; out fp64 [rows, q_heads, head_dim] and
 * lse fp64 [rows, q_heads] (natural log of the softmax denominator, with
 * the scaled logits). k/v: bf16 [B, T_cap, kv_heads, head_dim] with element
 * strides kv_stride_b, kv_stride_t. sel: int32 [rows, kv_heads, topk]. */
int o_attend(const uint16_t* q, int64_t q_stride_row, int32_t q_heads, int32_t kv_heads,
             int32_t head_dim, const uint16_t* k, const uint16_t* v, int64_t kv_stride_b,
             int64_t kv_stride_t, int64_t T_cap, const int32_t* sel, int32_t topk,
             const int32_t* row_seq, const int64_t* row_pos, int64_t rows, double scale,
             double* out, double* lse, int nthreads) {
  int qpk = q_heads / kv_heads;
  for (int64_t r = 0; r < rows; ++r) {
    if (row_pos[r] < 0 || row_pos[r] >= T_cap || row_seq[r] < 0) return O_BAD;
    for (int g = 0; g < kv_heads; ++g)
      for (int i = 0; i < topk; ++i) {
        int32_t j = sel[(r * kv_heads + g) * topk + i];
        if (j >= 0 && (int64_t)j >= row_pos[r] / REGION) return O_BAD;
      }
  }
  int64_t units = rows * q_heads;
  int bad = 0;
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
  for (int64_t u = 0; u < units; ++u) {
    int64_t r = u / q_heads;
    int h = (int)(u % q_heads), g = h / qpk;
    int64_t p = row_pos[r];
    const uint16_t* kb = k + (int64_t)row_seq[r] * kv_stride_b + (int64_t)g * head_dim;
    const uint16_t* vb = v + (int64_t)row_seq[r] * kv_stride_b + (int64_t)g * head_dim;
    const int32_t* s = sel + (r * kv_heads + g) * topk;
    int64_t own0 = (p / REGION) * REGION;
    int64_t ntok = 0;
    int64_t* toks = (int64_t*)malloc((size_t)(topk * REGION + REGION) * sizeof(int64_t));
    double* lg = (double*)malloc((size_t)(topk * REGION + REGION) * sizeof(double));
    double qd[512];
    if (!toks || !lg || head_dim > 512) { bad = 1; free(toks); free(lg); continue; }
    for (int i = 0; i < topk; ++i)
      if (s[i] >= 0)
        for (int t = 0; t < REGION; ++t) toks[ntok++] = (int64_t)s[i] * REGION + t;
    for (int64_t t = own0; t <= p; ++t) toks[ntok++] = t;
    for (int d = 0; d < head_dim; ++d) qd[d] = (double)o_bf16_to_f32(q[r * q_stride_row + (int64_t)h * head_dim + d]);
    double mx = -INFINITY;
    for (int64_t i = 0; i < ntok; ++i) {
      const uint16_t* kr = kb + toks[i] * kv_stride_t;
      double dot = 0.0;
      for (int d = 0; d < head_dim; ++d) dot += qd[d] * (double)o_bf16_to_f32(kr[d]);
      lg[i] = scale * dot;
      if (lg[i] > mx) mx = lg[i];
    }
    double den = 0.0;
    double* o = out + u * head_dim;
    for (int d = 0; d < head_dim; ++d) o[d] = 0.0;
    for (int64_t i = 0; i < ntok; ++i) {
      double e = exp(lg[i] - mx);
      den += e;
      const uint16_t* vr = vb + toks[i] * kv_stride_t;
      for (int d = 0; d < head_dim; ++d) o[d] += e * (double)o_bf16_to_f32(vr[d]);
    }
    for (int d = 0; d < head_dim; ++d) o[d] /= den;
    if (lse) lse[u] = mx + log(den);
    free(toks);
    free(lg);
  }
  return bad ? O_BAD : O_OK;
}

/* ------------------------------------------------------------------------ */
/* Fused projection [VLLM-proj]                                             */
/* ------------------------------------------------------------------------ */
/* out[r, n] = sum over k of hidden[r, k] * w[n, k], the bf16 inputs widened
 * and the sum taken in fp64 in k order. hidden: bf16 [rows, hsize]
 * (contiguous rows); w: bf16 [n_out, hsize] (the weight's rows are output
 * columns); out: fp64 [rows, n_out]. The split into q, k, v and the indexer's
 * q, k, z and gate is by column ranges (oracle.py, project). */
int o_project(const uint16_t* hidden, int64_t rows, int64_t hsize, const uint16_t* w,
              int64_t n_out, double* out, int nthreads) {
  if (rows < 0 || hsize <= 0 || n_out <= 0) return O_BAD;
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
  for (int64_t r = 0; r < rows; ++r) {
    const uint16_t* hr = hidden + r * hsize;
    for (int64_t n = 0; n < n_out; ++n) {
      const uint16_t* wn = w + n * hsize;
      double acc = 0.0;
      for (int64_t k = 0; k < hsize; ++k)
        acc += (double)o_bf16_to_f32(hr[k]) * (double)o_bf16_to_f32(wn[k]);
      out[r * n_out + n] = acc;
    }
  }
  return O_OK;
}

/* ------------------------------------------------------------------------ */
/* Array forms of the helpers, for the tests' exhaustive sweeps             */
/* ------------------------------------------------------------------------ */
void o_f32_to_bf16_n(const float* x, uint16_t* y, int64_t n) {
  for (int64_t i = 0; i < n; ++i) y[i] = o_f32_to_bf16(x[i]);
}
void o_bf16_to_e4m3_n(const uint16_t* x, uint8_t* y, int64_t n) {
  for (int64_t i = 0; i < n; ++i) y[i] = o_bf16_to_e4m3(x[i]);
}
void o_exp_n(const float* x, float* y, int64_t n, int nthreads) {
#pragma omp parallel for num_threads(nthreads) schedule(static)
  for (int64_t i = 0; i < n; ++i) y[i] = o_exp(x[i]);
}
/* exp of the n inputs whose fp32 bit patterns are start, start + 1, ...
   (a sweep of a range of the domain without an input array) */
void o_exp_bits_range(uint32_t start, int64_t n, float* y, int nthreads) {
#pragma omp parallel for num_threads(nthreads) schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    const uint32_t b = start + (uint32_t)i;
    float x;
    memcpy(&x, &b, sizeof x);
    y[i] = o_exp(x);
  }
}
/* k prep of n vectors of 64 dims, all at their own positions pos[i] */
void o_k_prep_n(const uint16_t* x, int64_t n, const float* g, const float* b, float eps,
                const uint16_t* rope, const int64_t* pos, float* out) {
  for (int64_t i = 0; i < n; ++i)
    o_k_prep_vec(x + i * IDX_DIM, g, b, eps, rope + pos[i] * ROT_DIM, out + i * IDX_DIM);
}
