/*
 * oracle.c -- plain CPU oracle for the per-frame decode step of a
 * multi-codebook speech LM (one talker step + code-predictor micro-steps).
 *
 * TEST INFRASTRUCTURE.  Only tests/, the smoke check of __graft_entry__ and
 * the cpu_baseline leg of bench.py load this library.  It shares no code,
 * header, table or constant generator with the HIP library; both sides only
 * receive the same seeded input arrays.
 *
 * What it computes: greedy (or, with a temperature, sampled: see "sampling")
 * decoding with two pre-norm decoder-only stacks.
 * Every technique the pages apply to this loop (K/V caching in a per-layer
 * ring, a window padded to 256 with a -inf tail, gather-sums assembled on the
 * device, fixed arenas, graph replay, batching) is an exact reorganisation of
 * that plain definition, so this file computes the definition itself:
 *
 *   qwentts.cpp, pipeline-tts.h commit log:
 *     - "AR inputs on device" entry: the talker's input for a frame is the sum
 *       of the 16 frame code embeddings plus one text-or-pad overlay row; the
 *       code predictor takes c0 and each sampled sub-code from its group table.
 *     - "set_rows / bridge" entry: the talker's last hidden is handed to the
 *       predictor, which takes it as the first row of its prefill.
 *     - "per-layer K/V ring" entry: the talker appends one position per frame
 *       and attends over [0, cur_len+1); the predictor runs a 2-row prefill then
 *       14 single-row decodes on a 16-position cache reset every frame.
 *     - "persistent arena" entry: the talker window is padded to a multiple of
 *       256 with the causal mask carrying -inf over the padded tail.
 *   minicpm-o-4.5 single-GPU engine, docs/optimizations.md, core table:
 *     residual add + RMSNorm, q/k norm + RoPE, SiLU-multiply are the fused
 *     pieces of each block.
 *
 * Readings where the pages are silent (block structure as in a Qwen3-style
 * decoder: pre-norm, per-head q/k RMSNorm before NeoX half-split RoPE, GQA,
 * SiLU-multiply MLP, no biases, untied heads) are listed in the design doc and
 * pinned in tests/ against HuggingFace's Qwen3 implementation.
 *
 * Linear-weight formats: F32, BF16, Q8 (32 int8 + one fp16 scale) and Q4.
 * The qwentts.cpp commit log's TTFA table lists a 4-bit column without
 * defining its block; Q4 here is our own: 32 weights per fp16 scale d, two
 * 4-bit codes c per byte (even index in the low nibble), w = d * (c - 8).
 *
 * Arithmetic: every dot product, sum and elementwise function is evaluated in
 * double, sequentially in index order, and rounded to the storage precision of
 * the tensor it produces: float32 for activations, hidden states and logits;
 * bfloat16 (round to nearest even) for the K/V cache and for matmul operands
 * when the model says so.  Threads only split independent outputs, so results
 * do not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_E_ARG (-1)
#define ORC_E_RANGE (-2)
#define ORC_E_STATE (-3)
#define ORC_E_FULL (-4)

/* ----------------------------------------------------------------------- */
/* storage formats                                                          */

enum { ORC_LIN_F32 = 0, ORC_LIN_BF16 = 1, ORC_LIN_Q8 = 2, ORC_LIN_Q4 = 3 };
#define ORC_Q8_BLOCK 32 /* weights per scale, for both block formats */

typedef struct {
  int32_t H, nq, nkv, hd, F;
  int32_t Lt, Lp;
  int32_t G;       /* codebooks per frame; the predictor has G-1 heads */
  int32_t Vc, Vt;  /* codebook entries, overlay table rows */
  int32_t P;       /* talker positions */
  int32_t Q;       /* predictor positions (reset every frame) */
  int32_t lin;     /* ORC_LIN_* */
  int32_t tab_bf16, kv_bf16, act_bf16;
  double eps, theta;
} orc_model;

/* bfloat16 -> float is exact: the 16 bits are the high half of a float. */
static float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* float -> nearest bfloat16 (ties to even), returned widened to float. */
float orc_bf16_round(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) {
    u = (u | 0x00400000u) & 0xFFFF0000u; /* quiet NaN */
  } else {
    uint32_t lsb = (u >> 16) & 1u;
    u = (u + 0x7FFFu + lsb) & 0xFFFF0000u;
  }
  float r;
  memcpy(&r, &u, 4);
  return r;
}

/* IEEE binary16 -> float (exact), from the format's definition. */
float orc_f16_to_f32(uint16_t h) {
  int sign = (h >> 15) & 1;
  int exp = (h >> 10) & 0x1F;
  int man = h & 0x3FF;
  double v;
  if (exp == 0)
    v = ldexp((double)man, -24); /* subnormal: man * 2^-14 * 2^-10 */
  else if (exp == 31)
    v = man ? NAN : INFINITY;
  else
    v = ldexp(1.0 + man / 1024.0, exp - 15);
  return (float)(sign ? -v : v);
}

/* ----------------------------------------------------------------------- */
/* weights: a flat pointer table in a fixed order                           */
/*
 * Per linear weight two slots (values, q8 scales or NULL).
 * Global slots:
 *   0 code_emb [G][Vc][H]    1 text_emb [Vt][H]    2 t_norm [H]
 *   3,4 t_head [Vc][H]       5 p_norm [H]          6 .. 6+2(G-1)-1 p_heads
 * then per talker layer, then per predictor layer, ORC_LAYER_SLOTS each:
 *   +0 attn_norm  +1,2 wq  +3,4 wk  +5,6 wv  +7 q_norm  +8 k_norm  +9,10 wo
 *   +11 mlp_norm  +12,13 wg  +14,15 wu  +16,17 wd
 */
#define ORC_LAYER_SLOTS 18

typedef struct {
  const void *w;     /* float[N][K], bf16 bits[N][K], int8[N][K] (q8) or
                        uint8[N][K/2] (q4: weight k in byte k/2, low nibble for even k) */
  const uint16_t *d; /* q8 / q4 only: fp16 bits [N][K/32] */
  int32_t N, K;
} orc_lin;

typedef struct {
  const void *attn_norm, *q_norm, *k_norm, *mlp_norm;
  orc_lin wq, wk, wv, wo, wg, wu, wd;
} orc_layer;

typedef struct {
  orc_model m;
  int32_t B, Pcap;
  const void *code_emb, *text_emb, *t_norm, *p_norm;
  orc_lin t_head;
  orc_lin *p_heads; /* G-1 */
  orc_layer *tl, *pl;
  /* caches, values as float (already rounded to the cache's format) */
  float *tk, *tv; /* [B][Lt][Pcap][nkv][hd] */
  float *pk, *pv; /* [B][Lp][Q][nkv][hd] */
  int32_t *pos, *c0, *ready;
  float *bridge; /* [B][H] */
  float *rope_cos, *rope_sin; /* [max(Pcap,Q)][hd/2] */
  int32_t rope_rows;
  float inv_temp; /* sampling: float(1/T), 0 = greedy */
  int32_t top_k;  /* sampling: only the top_k largest logits compete (0: all) */
  uint64_t seed;
} orc_sess;

static double tab_get(const orc_model *m, const void *p, size_t i) {
  return m->tab_bf16 ? (double)bf16_to_f32(((const uint16_t *)p)[i])
                     : (double)((const float *)p)[i];
}

/* one row of a linear weight as doubles (Q8: w = f32(d) * q; Q4: w = f32(d) * (c - 8); exact) */
static void lin_row(const orc_model *m, const orc_lin *L, int32_t n, double *out) {
  size_t base = (size_t)n * L->K;
  if (m->lin == ORC_LIN_F32) {
    const float *w = (const float *)L->w + base;
    for (int32_t k = 0; k < L->K; ++k) out[k] = w[k];
  } else if (m->lin == ORC_LIN_BF16) {
    const uint16_t *w = (const uint16_t *)L->w + base;
    for (int32_t k = 0; k < L->K; ++k) out[k] = bf16_to_f32(w[k]);
  } else if (m->lin == ORC_LIN_Q4) {
    /* 4-bit blocks of our own definition: code c in 0..15 stands for c - 8 */
    const uint8_t *q = (const uint8_t *)L->w + base / 2;
    const uint16_t *d = L->d + (size_t)n * (L->K / ORC_Q8_BLOCK);
    for (int32_t k = 0; k < L->K; ++k) {
      const int c = k % 2 ? q[k / 2] >> 4 : q[k / 2] & 15;
      out[k] = (double)orc_f16_to_f32(d[k / ORC_Q8_BLOCK]) * (double)(c - 8);
    }
  } else {
    const int8_t *q = (const int8_t *)L->w + base;
    const uint16_t *d = L->d + (size_t)n * (L->K / ORC_Q8_BLOCK);
    for (int32_t k = 0; k < L->K; ++k)
      out[k] = (double)orc_f16_to_f32(d[k / ORC_Q8_BLOCK]) * (double)q[k];
  }
}

/* matmul operand: float activations, rounded to bf16 when the model says so */
static double act(const orc_model *m, float v) {
  return m->act_bf16 ? (double)orc_bf16_round(v) : (double)v;
}

/* ----------------------------------------------------------------------- */
/* primitives                                                               */

/* out[r][n] = sum_k W[n][k] * x~[r][k]  for r < R; x~ = act(x). */
static void mm(const orc_model *m, const orc_lin *L, int32_t R, const float *x,
               int32_t x_stride, float *out, int32_t out_stride) {
  const int32_t N = L->N, K = L->K;
  double *xt = (double *)malloc(sizeof(double) * (size_t)K * R); /* [K][R] */
  for (int32_t r = 0; r < R; ++r)
    for (int32_t k = 0; k < K; ++k) xt[(size_t)k * R + r] = act(m, x[(size_t)r * x_stride + k]);
#pragma omp parallel
  {
    double *wrow = (double *)malloc(sizeof(double) * K);
    double *acc = (double *)malloc(sizeof(double) * R);
#pragma omp for schedule(static)
    for (int32_t n = 0; n < N; ++n) {
      lin_row(m, L, n, wrow);
      for (int32_t r = 0; r < R; ++r) acc[r] = 0.0;
      for (int32_t k = 0; k < K; ++k) {
        const double w = wrow[k];
        const double *xk = xt + (size_t)k * R;
        for (int32_t r = 0; r < R; ++r) acc[r] += w * xk[r];
      }
      for (int32_t r = 0; r < R; ++r) out[(size_t)r * out_stride + n] = (float)acc[r];
    }
    free(wrow);
    free(acc);
  }
  free(xt);
}

/* RMSNorm: y_i = x_i / sqrt(mean(x^2) + eps) * g_i */
static void rmsnorm(const orc_model *m, const float *x, const void *g, int32_t n,
                    float *y) {
  double s = 0.0;
  for (int32_t i = 0; i < n; ++i) s += (double)x[i] * (double)x[i];
  const double r = 1.0 / sqrt(s / n + m->eps);
  for (int32_t i = 0; i < n; ++i) y[i] = (float)((double)x[i] * r * tab_get(m, g, i));
}

/* NeoX-style rotary embedding on one head: pairs (i, i + hd/2). */
static void rope(const orc_sess *s, float *v, int32_t p) {
  const int32_t h = s->m.hd / 2;
  const float *c = s->rope_cos + (size_t)p * h;
  const float *sn = s->rope_sin + (size_t)p * h;
  for (int32_t i = 0; i < h; ++i) {
    const double a = v[i], b = v[i + h];
    v[i] = (float)(a * c[i] - b * sn[i]);
    v[i + h] = (float)(b * c[i] + a * sn[i]);
  }
}

static float kv_store(const orc_model *m, float v) { return m->kv_bf16 ? orc_bf16_round(v) : v; }

/* ----------------------------------------------------------------------- */
/* sampling                                                                 */
/*
 * The pages decode greedily and keep the sampler inside the graph
 * (qwentts.cpp tests-branch log, "fused codec mode removed" entry), but they
 * define no distribution, so this one is our own: temperature sampling by the
 * Gumbel-max rule.  For a head's logits l and temperature T > 0 the code is
 *     argmax_n ( l_n * (1/T) + g_n ),   the lowest index winning ties,
 * with g_n = -log(-log(u_n)) standard Gumbel variates; the argmax of
 * Gumbel-perturbed scores is a draw from softmax(l / T).  u_n is the first
 * output word x of Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel
 * random numbers: as easy as 1, 2, 3", SC'11) at counter (n, j, q, slot) and
 * key (seed, 0), mapped to ((x >> 11) + 0.5) * 2^-53 in (0, 1).  j is the
 * code's index in its frame (0 = the talker's code), q the frame's talker
 * position (a talker head at position p decides frame q = p + 1; the
 * predictor of the frame at position q decides codes 1..G-1), slot the
 * stream.  1/T is rounded to float once; g is computed in double and rounded
 * to float once; the product and the sum are float operations.  T = 0 is the
 * greedy argmax.  With top_k = k > 0 only the k largest logits compete (the
 * draw is from softmax(l / T) restricted to them); among equal logits at the
 * boundary the lower indices are the larger, as in the argmax.
 */
#define ORC_PHILOX_M0 0xD2E7470EE14C6C93ULL
#define ORC_PHILOX_M1 0xCA5A826395121157ULL
#define ORC_PHILOX_W0 0x9E3779B97F4A7C15ULL /* golden ratio */
#define ORC_PHILOX_W1 0xBB67AE8584CAA73BULL /* sqrt(3) - 1 */

/* Philox4x64 with 10 rounds: each round multiplies words 0 and 2 by the two
   multipliers (128-bit products), crosses the high halves with words 1, 3 and
   the round key, and the key advances by the Weyl constants between rounds. */
void orc_prim_philox4x64(const uint64_t *ctr, const uint64_t *key, uint64_t *out) {
  uint64_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3], k0 = key[0], k1 = key[1];
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += ORC_PHILOX_W0; k1 += ORC_PHILOX_W1; }
    const unsigned __int128 p0 = (unsigned __int128)ORC_PHILOX_M0 * c0;
    const unsigned __int128 p1 = (unsigned __int128)ORC_PHILOX_M1 * c2;
    const uint64_t hi0 = (uint64_t)(p0 >> 64), lo0 = (uint64_t)p0;
    const uint64_t hi1 = (uint64_t)(p1 >> 64), lo1 = (uint64_t)p1;
    c0 = hi1 ^ c1 ^ k0;
    c1 = lo1;
    c2 = hi0 ^ c3 ^ k1;
    c3 = lo0;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* Gumbel variate of logit n of code j of frame q, stream slot */
float orc_prim_gumbel(uint64_t seed, int32_t slot, int32_t q, int32_t j, int32_t n) {
  const uint64_t ctr[4] = {(uint64_t)n, (uint64_t)j, (uint64_t)q, (uint64_t)slot};
  const uint64_t key[2] = {seed, 0};
  uint64_t x[4];
  orc_prim_philox4x64(ctr, key, x);
  const double u = ((double)(x[0] >> 11) + 0.5) * 0x1p-53;
  return (float)(-log(-log(u)));
}

/* argmax over n logits; the lowest index wins ties. */
static int32_t argmax(const float *x, int32_t n) {
  int32_t best = 0;
  for (int32_t i = 1; i < n; ++i)
    if (x[i] > x[best]) best = i;
  return best;
}

/*
 * Attention of one query head at position p over a cache laid out
 * [pos][nkv][hd] (kv head kh).  The window is [0, W): positions j > p are
 * masked by select -- their cache rows are never read, so padded or stale
 * rows (any bits, NaN included) cannot reach a sum, and a padded window gives
 * exactly the same result as an unpadded one.
 */
static void attend(const orc_model *m, const float *q, const float *kc, const float *vc,
                   int32_t kh, int32_t p, int32_t W, double *sc, float *o) {
  const int32_t hd = m->hd, stride = m->nkv * hd;
  const double scale = 1.0 / sqrt((double)hd);
  double mx = -INFINITY;
  for (int32_t j = 0; j < W; ++j) {
    if (j <= p) {
      const float *k = kc + (size_t)j * stride + (size_t)kh * hd;
      double d = 0.0;
      for (int32_t i = 0; i < hd; ++i) d += (double)q[i] * (double)k[i];
      sc[j] = d * scale;
      if (sc[j] > mx) mx = sc[j];
    } else {
      sc[j] = -INFINITY;
    }
  }
  double den = 0.0;
  for (int32_t j = 0; j < W; ++j) {
    sc[j] = (j <= p) ? exp(sc[j] - mx) : 0.0;
    den += sc[j];
  }
  for (int32_t i = 0; i < hd; ++i) {
    double a = 0.0;
    for (int32_t j = 0; j <= p && j < W; ++j)
      a += sc[j] * (double)vc[(size_t)j * stride + (size_t)kh * hd + i];
    o[i] = (float)(a / den);
  }
}

/* ----------------------------------------------------------------------- */
/* one decoder layer over R rows                                            */

typedef struct {
  float *k, *v;  /* cache base of this row's stream and layer: [cap][nkv][hd] */
  int32_t pos;   /* position of the row */
  int32_t W;     /* attention window */
} orc_row;

static void layer_fwd(const orc_sess *s, const orc_layer *L, int32_t R, float *x,
                      const orc_row *rows) {
  const orc_model *m = &s->m;
  const int32_t H = m->H, hd = m->hd, nq = m->nq, nkv = m->nkv, F = m->F;
  const int32_t qd = nq * hd, kd = nkv * hd;
  float *h = (float *)calloc((size_t)R * H, sizeof(float));
  float *q = (float *)malloc(sizeof(float) * (size_t)R * qd);
  float *k = (float *)malloc(sizeof(float) * (size_t)R * kd);
  float *v = (float *)malloc(sizeof(float) * (size_t)R * kd);
  float *o = (float *)malloc(sizeof(float) * (size_t)R * qd);
  float *d = (float *)malloc(sizeof(float) * (size_t)R * H);
  float *a = (float *)malloc(sizeof(float) * (size_t)R * F);
  float *u = (float *)malloc(sizeof(float) * (size_t)R * F);

  /* attention block */
  for (int32_t r = 0; r < R; ++r) rmsnorm(m, x + (size_t)r * H, L->attn_norm, H, h + (size_t)r * H);
  mm(m, &L->wq, R, h, H, q, qd);
  mm(m, &L->wk, R, h, H, k, kd);
  mm(m, &L->wv, R, h, H, v, kd);
  for (int32_t r = 0; r < R; ++r) {
    const int32_t p = rows[r].pos;
    for (int32_t hh = 0; hh < nq; ++hh) {
      float *qh = q + (size_t)r * qd + (size_t)hh * hd;
      rmsnorm(m, qh, L->q_norm, hd, qh);
      rope(s, qh, p);
    }
    for (int32_t kh = 0; kh < nkv; ++kh) {
      float *kk = k + (size_t)r * kd + (size_t)kh * hd;
      const float *vv = v + (size_t)r * kd + (size_t)kh * hd;
      rmsnorm(m, kk, L->k_norm, hd, kk);
      rope(s, kk, p);
      float *kdst = rows[r].k + (size_t)p * kd + (size_t)kh * hd;
      float *vdst = rows[r].v + (size_t)p * kd + (size_t)kh * hd;
      for (int32_t i = 0; i < hd; ++i) {
        kdst[i] = kv_store(m, kk[i]);
        vdst[i] = kv_store(m, vv[i]);
      }
    }
  }
  /* every row's K/V is in its cache before any row attends (rows of one
     stream in a prefill see each other causally through the mask) */
#pragma omp parallel
  {
    int32_t maxW = 0;
    for (int32_t r = 0; r < R; ++r)
      if (rows[r].W > maxW) maxW = rows[r].W;
    double *sc = (double *)malloc(sizeof(double) * (size_t)(maxW > 0 ? maxW : 1));
#pragma omp for schedule(static) collapse(2)
    for (int32_t r = 0; r < R; ++r)
      for (int32_t hh = 0; hh < nq; ++hh) {
        const int32_t kh = hh / (nq / nkv);
        attend(m, q + (size_t)r * qd + (size_t)hh * hd, rows[r].k, rows[r].v, kh, rows[r].pos,
               rows[r].W, sc, o + (size_t)r * qd + (size_t)hh * hd);
      }
    free(sc);
  }
  mm(m, &L->wo, R, o, qd, d, H);
  for (size_t i = 0; i < (size_t)R * H; ++i) x[i] = x[i] + d[i];

  /* MLP block: down(silu(gate) * up) */
  for (int32_t r = 0; r < R; ++r) rmsnorm(m, x + (size_t)r * H, L->mlp_norm, H, h + (size_t)r * H);
  mm(m, &L->wg, R, h, H, a, F);
  mm(m, &L->wu, R, h, H, u, F);
  for (size_t i = 0; i < (size_t)R * F; ++i) {
    const double g = a[i];
    a[i] = (float)(g / (1.0 + exp(-g)) * (double)u[i]);
  }
  mm(m, &L->wd, R, a, F, d, H);
  for (size_t i = 0; i < (size_t)R * H; ++i) x[i] = x[i] + d[i];

  free(h); free(q); free(k); free(v); free(o); free(d); free(a); free(u);
}

/* talker window: a multiple of 256 covering [0, p] */
static int32_t talker_window(int32_t p) { return 256 * ((p + 1 + 255) / 256); }

/* ----------------------------------------------------------------------- */
/* session                                                                  */

static void bind_lin(orc_lin *L, const void *const *t, int32_t slot, int32_t N, int32_t K) {
  L->w = t[slot];
  L->d = (const uint16_t *)t[slot + 1];
  L->N = N;
  L->K = K;
}

static void bind_layer(const orc_model *m, orc_layer *L, const void *const *t, int32_t b) {
  const int32_t H = m->H, qd = m->nq * m->hd, kd = m->nkv * m->hd;
  L->attn_norm = t[b + 0];
  bind_lin(&L->wq, t, b + 1, qd, H);
  bind_lin(&L->wk, t, b + 3, kd, H);
  bind_lin(&L->wv, t, b + 5, kd, H);
  L->q_norm = t[b + 7];
  L->k_norm = t[b + 8];
  bind_lin(&L->wo, t, b + 9, H, qd);
  L->mlp_norm = t[b + 11];
  bind_lin(&L->wg, t, b + 12, m->F, H);
  bind_lin(&L->wu, t, b + 14, m->F, H);
  bind_lin(&L->wd, t, b + 16, H, m->F);
}

int32_t orc_num_tensors(const orc_model *m) {
  return 6 + 2 * (m->G - 1) + ORC_LAYER_SLOTS * (m->Lt + m->Lp);
}

void orc_free(orc_sess *s) {
  if (!s) return;
  free(s->p_heads); free(s->tl); free(s->pl);
  free(s->tk); free(s->tv); free(s->pk); free(s->pv);
  free(s->pos); free(s->c0); free(s->ready); free(s->bridge);
  free(s->rope_cos); free(s->rope_sin);
  free(s);
}

/* Pcap: talker positions actually held per stream (<= P); positions past it
   are rejected, so a reduced allocation can never change a result. */
orc_sess *orc_new(const orc_model *m, const void *const *t, int32_t n_tensors, int32_t B,
                  int32_t Pcap) {
  if (!m || !t || B <= 0 || Pcap <= 0 || Pcap > m->P) return NULL;
  if (n_tensors != orc_num_tensors(m)) return NULL;
  if (m->hd % 2 || m->nq % m->nkv || m->G < 2 || m->Q < m->G) return NULL;
  if (m->lin < ORC_LIN_F32 || m->lin > ORC_LIN_Q4) return NULL;
  if (m->lin >= ORC_LIN_Q8 && (m->H % ORC_Q8_BLOCK || m->F % ORC_Q8_BLOCK ||
                               (m->nq * m->hd) % ORC_Q8_BLOCK))
    return NULL;
  orc_sess *s = (orc_sess *)calloc(1, sizeof(orc_sess));
  s->m = *m;
  s->B = B;
  s->Pcap = Pcap;
  s->code_emb = t[0];
  s->text_emb = t[1];
  s->t_norm = t[2];
  bind_lin(&s->t_head, t, 3, m->Vc, m->H);
  s->p_norm = t[5];
  s->p_heads = (orc_lin *)calloc((size_t)(m->G - 1), sizeof(orc_lin));
  for (int32_t j = 0; j < m->G - 1; ++j) bind_lin(&s->p_heads[j], t, 6 + 2 * j, m->Vc, m->H);
  int32_t base = 6 + 2 * (m->G - 1);
  s->tl = (orc_layer *)calloc((size_t)m->Lt, sizeof(orc_layer));
  s->pl = (orc_layer *)calloc((size_t)(m->Lp > 0 ? m->Lp : 1), sizeof(orc_layer));
  for (int32_t l = 0; l < m->Lt; ++l, base += ORC_LAYER_SLOTS) bind_layer(m, &s->tl[l], t, base);
  for (int32_t l = 0; l < m->Lp; ++l, base += ORC_LAYER_SLOTS) bind_layer(m, &s->pl[l], t, base);
  const size_t kd = (size_t)m->nkv * m->hd;
  s->tk = (float *)calloc((size_t)B * m->Lt * Pcap * kd, sizeof(float));
  s->tv = (float *)calloc((size_t)B * m->Lt * Pcap * kd, sizeof(float));
  s->pk = (float *)calloc((size_t)B * (m->Lp > 0 ? m->Lp : 1) * m->Q * kd, sizeof(float));
  s->pv = (float *)calloc((size_t)B * (m->Lp > 0 ? m->Lp : 1) * m->Q * kd, sizeof(float));
  s->pos = (int32_t *)calloc((size_t)B, sizeof(int32_t));
  s->c0 = (int32_t *)calloc((size_t)B, sizeof(int32_t));
  s->ready = (int32_t *)calloc((size_t)B, sizeof(int32_t));
  s->bridge = (float *)calloc((size_t)B * m->H, sizeof(float));
  if (!s->tk || !s->tv || !s->pk || !s->pv) {
    orc_free(s);
    return NULL;
  }
  /* rotary table: angle p * theta^(-2i/hd) in double, cos/sin rounded to float */
  const int32_t h = m->hd / 2;
  s->rope_rows = Pcap > m->Q ? Pcap : m->Q;
  s->rope_cos = (float *)malloc(sizeof(float) * (size_t)s->rope_rows * h);
  s->rope_sin = (float *)malloc(sizeof(float) * (size_t)s->rope_rows * h);
  for (int32_t p = 0; p < s->rope_rows; ++p)
    for (int32_t i = 0; i < h; ++i) {
      const double ang = (double)p * pow(m->theta, -2.0 * i / (double)m->hd);
      s->rope_cos[(size_t)p * h + i] = (float)cos(ang);
      s->rope_sin[(size_t)p * h + i] = (float)sin(ang);
    }
  return s;
}

static float *tcache(const orc_sess *s, float *base, int32_t b, int32_t l) {
  const size_t kd = (size_t)s->m.nkv * s->m.hd;
  return base + ((size_t)b * s->m.Lt + l) * s->Pcap * kd;
}
static float *pcache(const orc_sess *s, float *base, int32_t b, int32_t l) {
  const size_t kd = (size_t)s->m.nkv * s->m.hd;
  return base + ((size_t)b * s->m.Lp + l) * s->m.Q * kd;
}

/* Sum of table rows: codebook g row codes[g] for g < G (if codes), plus the
   overlay row text_id.  Exact sum in double, rounded once to float. */
static void gather_sum(const orc_sess *s, const int32_t *codes, int32_t text_id, float *out) {
  const orc_model *m = &s->m;
  for (int32_t i = 0; i < m->H; ++i) {
    double acc = 0.0;
    if (codes)
      for (int32_t g = 0; g < m->G; ++g)
        acc += tab_get(m, s->code_emb, ((size_t)g * m->Vc + codes[g]) * m->H + i);
    acc += tab_get(m, s->text_emb, (size_t)text_id * m->H + i);
    out[i] = (float)acc;
  }
}

/* The code a head's logits decide: greedy argmax, or with a temperature the
   Gumbel-max draw of code j of frame q for stream slot (see "sampling"). */
/* logit a ranks above logit b: larger value, or equal value and lower index */
static int ranks_above(const float *x, int32_t a, int32_t b) {
  return x[a] > x[b] || (x[a] == x[b] && a < b);
}

static int32_t choose(const orc_sess *s, const float *logits, int32_t n, int32_t slot, int32_t q, int32_t j) {
  if (s->inv_temp == 0.f) return argmax(logits, n);
  float best = -INFINITY;
  int32_t bi = 0;
  for (int32_t i = 0; i < n; ++i) {
    if (s->top_k > 0 && s->top_k < n) {
      /* member of the top k: fewer than k logits rank above it */
      int32_t above = 0;
      for (int32_t t = 0; t < n && above < s->top_k; ++t) above += ranks_above(logits, t, i);
      if (above >= s->top_k) continue;
    }
    const float scaled = logits[i] * s->inv_temp;
    const float v = scaled + orc_prim_gumbel(s->seed, slot, q, j, i);
    if (v > best) { best = v; bi = i; }
  }
  return bi;
}

/* talker final norm -> bridge, head -> logits, code 0 of frame q (the next one) */
static int32_t talker_tail(const orc_sess *s, const float *x, float *bridge, float *logits, int32_t slot,
                           int32_t q) {
  rmsnorm(&s->m, x, s->t_norm, s->m.H, bridge);
  mm(&s->m, &s->t_head, 1, bridge, s->m.H, logits, s->m.Vc);
  return choose(s, logits, s->m.Vc, slot, q, 0);
}

/* Sampling from now on: temperature T (0: greedy), top_k (0: every logit)
   and the Philox key seed. */
int32_t orc_set_sampler(orc_sess *s, float temperature, int32_t top_k, uint64_t seed) {
  if (!(temperature >= 0.f) || isinf(temperature) || top_k < 0) return ORC_E_ARG;
  s->inv_temp = temperature > 0.f ? (float)(1.0 / (double)temperature) : 0.f;
  s->top_k = top_k;
  s->seed = seed;
  return ORC_OK;
}

/*
 * Prefill of stream b with T prompt rows: row p = sum_g E_g[codes[p][g]] +
 * Tx[text[p]] (codes may be NULL: text rows only) at position p.  The cache
 * is reset (written over [0, T)), the last row's final-normed hidden becomes
 * the bridge and its head argmax the first frame's code 0.
 * dump_x0 [T][H] and dump_logits [Vc] may be NULL.
 */
int32_t orc_prefill(orc_sess *s, int32_t b, int32_t T, const int32_t *codes, const int32_t *text,
                    float *dump_x0, float *dump_logits) {
  const orc_model *m = &s->m;
  if (b < 0 || b >= s->B || T <= 0 || !text) return ORC_E_ARG;
  if (T > s->Pcap) return ORC_E_FULL;
  for (int32_t p = 0; p < T; ++p) {
    if (text[p] < 0 || text[p] >= m->Vt) return ORC_E_RANGE;
    if (codes)
      for (int32_t g = 0; g < m->G; ++g)
        if (codes[(size_t)p * m->G + g] < 0 || codes[(size_t)p * m->G + g] >= m->Vc) return ORC_E_RANGE;
  }
  float *x = (float *)malloc(sizeof(float) * (size_t)T * m->H);
  orc_row *rows = (orc_row *)malloc(sizeof(orc_row) * (size_t)T);
  for (int32_t p = 0; p < T; ++p)
    gather_sum(s, codes ? codes + (size_t)p * m->G : NULL, text[p], x + (size_t)p * m->H);
  if (dump_x0) memcpy(dump_x0, x, sizeof(float) * (size_t)T * m->H);
  for (int32_t l = 0; l < m->Lt; ++l) {
    for (int32_t p = 0; p < T; ++p) {
      rows[p].k = tcache(s, s->tk, b, l);
      rows[p].v = tcache(s, s->tv, b, l);
      rows[p].pos = p;
      rows[p].W = talker_window(p);
    }
    layer_fwd(s, &s->tl[l], T, x, rows);
  }
  float *logits = (float *)malloc(sizeof(float) * m->Vc);
  s->c0[b] = talker_tail(s, x + (size_t)(T - 1) * m->H, s->bridge + (size_t)b * m->H, logits, b, T);
  if (dump_logits) memcpy(dump_logits, logits, sizeof(float) * m->Vc);
  s->pos[b] = T;
  s->ready[b] = 1;
  free(logits);
  free(rows);
  free(x);
  return ORC_OK;
}

typedef struct {
  float *talker_logits; /* [n][B][Vc] */
  float *pred_logits;   /* [n][B][G-1][Vc] */
  float *bridge;        /* [n][B][H]   after the frame's talker step */
  float *x0;            /* [n][B][H]   talker input gather-sum */
  int32_t *gather;      /* [n][B][G+1] codes fed to the gather, then the overlay id */
  int32_t *tpos;        /* [n][B]      talker K/V write position */
  float *hidden;        /* [n][B][Lt][H] talker residual stream after each layer */
} orc_dump;

/*
 * Decode n frames for all B streams.  Frame f of stream b:
 *   1. code predictor, cache reset: rows [bridge, E_0[c0]] at positions 0, 1
 *      through Lp layers; head 0 on the final-normed row 1 gives c1.
 *   2. for j = 1 .. G-2: row E_j[c_j] at position j+1; head j gives c_{j+1}.
 *   3. codes[f] = (c0 .. c_{G-1}).
 *   4. talker step at position pos: input sum_g E_g[c_g] + Tx[overlay[f]];
 *      Lt layers; final norm -> bridge; head -> next c0; pos += 1.
 * With forced (teacher forcing, [n][B][G]) the codes fed back into the
 * predictor and the talker gather come from forced, while codes[] still gets
 * every argmax (codes[f][b][0] is the previous talker step's argmax).
 */
int32_t orc_decode(orc_sess *s, int32_t n, const int32_t *overlay, const int32_t *forced,
                   int32_t *codes, const orc_dump *dump) {
  const orc_model *m = &s->m;
  const int32_t B = s->B, H = m->H, G = m->G, Vc = m->Vc;
  if (n < 0 || !overlay || !codes) return ORC_E_ARG;
  for (int32_t b = 0; b < B; ++b) {
    if (!s->ready[b]) return ORC_E_STATE;
    if (s->pos[b] + n > s->Pcap) return ORC_E_FULL;
  }
  for (int32_t i = 0; i < n * B; ++i)
    if (overlay[i] < 0 || overlay[i] >= m->Vt) return ORC_E_RANGE;
  if (forced)
    for (int32_t i = 0; i < n * B * G; ++i)
      if (forced[i] < 0 || forced[i] >= Vc) return ORC_E_RANGE;

  float *x = (float *)malloc(sizeof(float) * (size_t)2 * B * H);
  float *hn = (float *)malloc(sizeof(float) * (size_t)H);
  float *logits = (float *)malloc(sizeof(float) * (size_t)Vc);
  int32_t *cin = (int32_t *)malloc(sizeof(int32_t) * (size_t)B * G);
  orc_row *rows = (orc_row *)malloc(sizeof(orc_row) * (size_t)2 * B);

  for (int32_t f = 0; f < n; ++f) {
    int32_t *cf = codes + (size_t)f * B * G;
    const int32_t *ff = forced ? forced + (size_t)f * B * G : NULL;
    for (int32_t b = 0; b < B; ++b) {
      cf[(size_t)b * G] = s->c0[b];
      cin[(size_t)b * G] = ff ? ff[(size_t)b * G] : s->c0[b];
    }
    /* 1. predictor prefill, two rows per stream */
    for (int32_t b = 0; b < B; ++b) {
      memcpy(x + (size_t)(2 * b) * H, s->bridge + (size_t)b * H, sizeof(float) * H);
      for (int32_t i = 0; i < H; ++i)
        x[(size_t)(2 * b + 1) * H + i] =
            (float)tab_get(m, s->code_emb, (size_t)cin[(size_t)b * G] * H + i);
    }
    for (int32_t l = 0; l < m->Lp; ++l) {
      for (int32_t b = 0; b < B; ++b)
        for (int32_t t = 0; t < 2; ++t) {
          rows[2 * b + t].k = pcache(s, s->pk, b, l);
          rows[2 * b + t].v = pcache(s, s->pv, b, l);
          rows[2 * b + t].pos = t;
          rows[2 * b + t].W = m->Q;
        }
      layer_fwd(s, &s->pl[l], 2 * B, x, rows);
    }
    for (int32_t b = 0; b < B; ++b) {
      rmsnorm(m, x + (size_t)(2 * b + 1) * H, s->p_norm, H, hn);
      mm(m, &s->p_heads[0], 1, hn, H, logits, Vc);
      const int32_t c = choose(s, logits, Vc, b, s->pos[b], 1);
      cf[(size_t)b * G + 1] = c;
      cin[(size_t)b * G + 1] = ff ? ff[(size_t)b * G + 1] : c;
      if (dump && dump->pred_logits)
        memcpy(dump->pred_logits + (((size_t)f * B + b) * (G - 1) + 0) * Vc, logits, sizeof(float) * Vc);
    }
    /* 2. predictor decodes */
    for (int32_t j = 1; j <= G - 2; ++j) {
      for (int32_t b = 0; b < B; ++b)
        for (int32_t i = 0; i < H; ++i)
          x[(size_t)b * H + i] = (float)tab_get(
              m, s->code_emb, ((size_t)j * Vc + cin[(size_t)b * G + j]) * H + i);
      for (int32_t l = 0; l < m->Lp; ++l) {
        for (int32_t b = 0; b < B; ++b) {
          rows[b].k = pcache(s, s->pk, b, l);
          rows[b].v = pcache(s, s->pv, b, l);
          rows[b].pos = j + 1;
          rows[b].W = m->Q;
        }
        layer_fwd(s, &s->pl[l], B, x, rows);
      }
      for (int32_t b = 0; b < B; ++b) {
        rmsnorm(m, x + (size_t)b * H, s->p_norm, H, hn);
        mm(m, &s->p_heads[j], 1, hn, H, logits, Vc);
        const int32_t c = choose(s, logits, Vc, b, s->pos[b], j + 1);
        cf[(size_t)b * G + j + 1] = c;
        cin[(size_t)b * G + j + 1] = ff ? ff[(size_t)b * G + j + 1] : c;
        if (dump && dump->pred_logits)
          memcpy(dump->pred_logits + (((size_t)f * B + b) * (G - 1) + j) * Vc, logits,
                 sizeof(float) * Vc);
      }
    }
    /* 4. talker step */
    for (int32_t b = 0; b < B; ++b) {
      gather_sum(s, cin + (size_t)b * G, overlay[(size_t)f * B + b], x + (size_t)b * H);
      if (dump && dump->x0) memcpy(dump->x0 + ((size_t)f * B + b) * H, x + (size_t)b * H, sizeof(float) * H);
      if (dump && dump->gather) {
        int32_t *gi = dump->gather + ((size_t)f * B + b) * (G + 1);
        for (int32_t g = 0; g < G; ++g) gi[g] = cin[(size_t)b * G + g];
        gi[G] = overlay[(size_t)f * B + b];
      }
      if (dump && dump->tpos) dump->tpos[(size_t)f * B + b] = s->pos[b];
    }
    for (int32_t l = 0; l < m->Lt; ++l) {
      for (int32_t b = 0; b < B; ++b) {
        rows[b].k = tcache(s, s->tk, b, l);
        rows[b].v = tcache(s, s->tv, b, l);
        rows[b].pos = s->pos[b];
        rows[b].W = talker_window(s->pos[b]);
      }
      layer_fwd(s, &s->tl[l], B, x, rows);
      if (dump && dump->hidden)
        for (int32_t b = 0; b < B; ++b)
          memcpy(dump->hidden + (((size_t)f * B + b) * m->Lt + l) * H, x + (size_t)b * H,
                 sizeof(float) * H);
    }
    for (int32_t b = 0; b < B; ++b) {
      s->c0[b] = talker_tail(s, x + (size_t)b * H, s->bridge + (size_t)b * H, logits, b, s->pos[b] + 1);
      if (dump && dump->talker_logits)
        memcpy(dump->talker_logits + ((size_t)f * B + b) * Vc, logits, sizeof(float) * Vc);
      if (dump && dump->bridge)
        memcpy(dump->bridge + ((size_t)f * B + b) * H, s->bridge + (size_t)b * H, sizeof(float) * H);
      s->pos[b] += 1;
    }
  }
  free(x); free(hn); free(logits); free(cin); free(rows);
  return ORC_OK;
}

/* ----------------------------------------------------------------------- */
/* state access                                                             */

int32_t orc_get_state(const orc_sess *s, int32_t b, int32_t *pos, int32_t *c0, float *bridge) {
  if (!s || b < 0 || b >= s->B) return ORC_E_ARG;
  if (pos) *pos = s->pos[b];
  if (c0) *c0 = s->c0[b];
  if (bridge) memcpy(bridge, s->bridge + (size_t)b * s->m.H, sizeof(float) * s->m.H);
  return ORC_OK;
}

int32_t orc_set_state(orc_sess *s, int32_t b, int32_t pos, int32_t c0, const float *bridge) {
  if (!s || b < 0 || b >= s->B || !bridge) return ORC_E_ARG;
  if (pos < 1 || pos > s->Pcap || c0 < 0 || c0 >= s->m.Vc) return ORC_E_RANGE;
  s->pos[b] = pos;
  s->c0[b] = c0;
  memcpy(s->bridge + (size_t)b * s->m.H, bridge, sizeof(float) * s->m.H);
  s->ready[b] = 1;
  return ORC_OK;
}

/* Talker cache of stream b, layer l, positions [p0, p0+np): k, v given as
   float [np][nkv][hd] (values already in the cache's format). */
int32_t orc_set_cache(orc_sess *s, int32_t b, int32_t l, int32_t p0, int32_t np, const float *k,
                      const float *v) {
  if (!s || b < 0 || b >= s->B || l < 0 || l >= s->m.Lt || p0 < 0 || np < 0 ||
      p0 + np > s->Pcap)
    return ORC_E_ARG;
  const size_t kd = (size_t)s->m.nkv * s->m.hd;
  memcpy(tcache(s, s->tk, b, l) + (size_t)p0 * kd, k, sizeof(float) * np * kd);
  memcpy(tcache(s, s->tv, b, l) + (size_t)p0 * kd, v, sizeof(float) * np * kd);
  return ORC_OK;
}

int32_t orc_get_cache(const orc_sess *s, int32_t b, int32_t l, int32_t p0, int32_t np, float *k,
                      float *v) {
  if (!s || b < 0 || b >= s->B || l < 0 || l >= s->m.Lt || p0 < 0 || np < 0 ||
      p0 + np > s->Pcap)
    return ORC_E_ARG;
  const size_t kd = (size_t)s->m.nkv * s->m.hd;
  memcpy(k, tcache(s, s->tk, b, l) + (size_t)p0 * kd, sizeof(float) * np * kd);
  memcpy(v, tcache(s, s->tv, b, l) + (size_t)p0 * kd, sizeof(float) * np * kd);
  return ORC_OK;
}

/* Fill the whole predictor cache of every stream with one value (NaN to show
   that stale rows from the previous frame never reach a sum). */
void orc_poison_predictor(orc_sess *s, float value) {
  const size_t n = (size_t)s->B * s->m.Lp * s->m.Q * s->m.nkv * s->m.hd;
  for (size_t i = 0; i < n; ++i) {
    s->pk[i] = value;
    s->pv[i] = value;
  }
}

/* ----------------------------------------------------------------------- */
/* primitives exported for the oracle's own pins                            */

void orc_prim_rmsnorm(const orc_model *m, const float *x, const void *g, int32_t n, float *y) {
  rmsnorm(m, x, g, n, y);
}

/* rotary embedding of one head (hd = m->hd) at position p, using a fresh
   table built for positions [0, p] */
void orc_prim_rope(const orc_model *m, float *v, int32_t p) {
  orc_sess s;
  memset(&s, 0, sizeof(s));
  s.m = *m;
  const int32_t h = m->hd / 2;
  s.rope_cos = (float *)malloc(sizeof(float) * (size_t)(p + 1) * h);
  s.rope_sin = (float *)malloc(sizeof(float) * (size_t)(p + 1) * h);
  for (int32_t i = 0; i < h; ++i) {
    const double ang = (double)p * pow(m->theta, -2.0 * i / (double)m->hd);
    s.rope_cos[(size_t)p * h + i] = (float)cos(ang);
    s.rope_sin[(size_t)p * h + i] = (float)sin(ang);
  }
  rope(&s, v, p);
  free(s.rope_cos);
  free(s.rope_sin);
}

/* one query head over a cache [W][nkv][hd] with kv head kh, position p */
void orc_prim_attend(const orc_model *m, const float *q, const float *kc, const float *vc,
                     int32_t kh, int32_t p, int32_t W, float *o) {
  double *sc = (double *)malloc(sizeof(double) * (size_t)(W > 0 ? W : 1));
  attend(m, q, kc, vc, kh, p, W, sc, o);
  free(sc);
}

/* out[r][n] = W x~[r] for a linear weight given as (w, d) with shape [N][K] */
void orc_prim_mm(const orc_model *m, const void *w, const uint16_t *d, int32_t N, int32_t K,
                 int32_t R, const float *x, float *out) {
  orc_lin L = {w, d, N, K};
  mm(m, &L, R, x, K, out, N);
}

int32_t orc_prim_argmax(const float *x, int32_t n) { return argmax(x, n); }

/* The sampler's choice for one head's logits (temperature 0: greedy). */
int32_t orc_prim_sample(const float *x, int32_t n, float temperature, int32_t top_k, uint64_t seed, int32_t slot,
                        int32_t q, int32_t j) {
  orc_sess s;
  memset(&s, 0, sizeof(s));
  if (orc_set_sampler(&s, temperature, top_k, seed) != ORC_OK) return ORC_E_ARG;
  return choose(&s, x, n, slot, q, j);
}

int32_t orc_prim_talker_window(int32_t p) { return talker_window(p); }

int32_t orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * Full recompute of the code predictor over R rows given outright (row 0 the
 * bridge, row j+1 the embedding of code j) as one causal sequence at
 * positions [0, R), in a scratch cache.  logits[j] = head_j(norm(row j+1)) for
 * j < R-1.  Pins the 2-row prefill + single-row decodes of orc_decode.
 */
int32_t orc_predictor_recompute(orc_sess *s, int32_t R, const float *rows_in, float *logits) {
  const orc_model *m = &s->m;
  if (R < 2 || R > m->Q || R - 1 > m->G - 1) return ORC_E_ARG;
  const size_t kd = (size_t)m->nkv * m->hd;
  float *x = (float *)malloc(sizeof(float) * (size_t)R * m->H);
  float *hn = (float *)malloc(sizeof(float) * m->H);
  float *kc = (float *)calloc((size_t)m->Q * kd, sizeof(float));
  float *vc = (float *)calloc((size_t)m->Q * kd, sizeof(float));
  orc_row *rows = (orc_row *)malloc(sizeof(orc_row) * (size_t)R);
  memcpy(x, rows_in, sizeof(float) * (size_t)R * m->H);
  for (int32_t l = 0; l < m->Lp; ++l) {
    for (int32_t r = 0; r < R; ++r) {
      rows[r].k = kc;
      rows[r].v = vc;
      rows[r].pos = r;
      rows[r].W = m->Q;
    }
    layer_fwd(s, &s->pl[l], R, x, rows);
  }
  for (int32_t j = 0; j < R - 1; ++j) {
    rmsnorm(m, x + (size_t)(j + 1) * m->H, s->p_norm, m->H, hn);
    mm(m, &s->p_heads[j], 1, hn, m->H, logits + (size_t)j * m->Vc, m->Vc);
  }
  free(x); free(hn); free(kc); free(vc); free(rows);
  return ORC_OK;
}
