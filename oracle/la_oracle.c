/*
 * Lookahead decoding oracle: a plain, slow CPU implementation of one
 * lookahead decoding step and of plain greedy decoding.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code,
 * header, table or helper with the HIP library and must never be called by
 * the product path.
 *
 * Source: "Break the Sequential Dependency of LLM Inference Using Lookahead
 * Decoding" (Fu, Bailis, Stoica, Zhang 2024), summary page.
 *   - Summary (in this file's words): each step guesses several future
 *     tokens at once by fixed-point (Jacobi) iteration on a window of
 *     guesses, turns the window's trajectories into n-grams kept in a store
 *     keyed by their first token, and checks stored n-grams against the
 *     model's own choices within the same step's forward pass, so the
 *     emitted tokens are those of one-token-at-a-time decoding.
 *   - Key points, "Tuning knobs": W = lookahead window, N = n-gram size,
 *     G = verification size.
 *   - Key points, "Main limitation": the per-step extra work is (W+G)(N-1)
 *     rows (120 / 80 / 56 for the near-optimal 7B / 13B / 34B settings).
 * The pages print no algorithm listing, mask, pool policy or model detail;
 * every such step below follows the plainest reading consistent with the
 * summary, and each is marked "reading".
 *
 * Model (reading: LLaMA-2 style, as the paper evaluates LLaMA-2): pre-norm
 * decoder, no biases, RMSNorm (eps from the config), rotary position
 * embedding on adjacent dimension pairs (2i, 2i+1) with angle
 * pos * theta^(-2i/dh), softmax attention with scale 1/sqrt(dh), grouped KV
 * heads (query head h reads KV head floor(h*Hkv/H)), SwiGLU feed-forward
 * silu(x Wg^T) * (x Wu^T) Wd^T, final RMSNorm and an untied LM head.
 *
 * Arithmetic: every value is held in double; weights are read as given
 * (fp32 values, or bfloat16 bit patterns widened exactly).  Each dot product
 * and each softmax sum runs in ascending index order in one thread, so every
 * result depends only on the (token, position) sequence a row can see and
 * never on the thread count.  Argmax decisions are taken on the logits
 * rounded to fp32 (the precision the HIP library's logits have), lowest
 * token id on ties.
 *
 * Storage precision (reading: the pages fix no number format).  With
 * act_bf16 = 0 nothing is rounded: the exact model.  With act_bf16 = 1 the
 * model of a bf16 datapath: every activation that a bf16 deployment keeps
 * in memory between operations is stored as bfloat16 (rounded to fp32,
 * then to 8 significant bits, ties to even at both steps), and everything
 * else stays exact:
 *   1. the attention block's normalized input, held as bf16(x * w) with the
 *      row's 1/rms(x) applied to the products (equal to RMSNorm then
 *      product in exact arithmetic);
 *   2. q and k after the rotary embedding, and v: the query and the KV
 *      cache (committed rows keep the rounded values);
 *   3. the attention probabilities exp(s - max) entering the weighted sum
 *      of values (the normalizer sums the unrounded ones);
 *   4. the attention output (input of the output projection);
 *   5. the FFN block's normalized input, as in 1;
 *   6. the SwiGLU output (input of the down projection);
 *   7. the LM head's input, RMSNorm(x) * w.
 * The residual stream and every sum stay exact.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
  int32_t n_layers, d_model, n_heads, n_kv_heads, head_dim, d_ffn, vocab;
  double rope_theta, rms_eps;
  int32_t W, N, G;
  int32_t max_ctx;
  int32_t wdtype; /* 0: float32 arrays; 1: bfloat16 bit patterns (uint16) */
  int32_t act_bf16; /* 1: bf16 storage of activations (see the header) */
} orc_config;

typedef struct {
  int32_t n_emitted;  /* k + 1 */
  int32_t tokens[32]; /* emitted tokens, last = new current token */
  int32_t accepted;   /* k */
  int32_t winner;     /* g*, -1 without candidates */
  int32_t n_candidates;
  int32_t kv_len;
} orc_result;

typedef struct orc {
  orc_config c;
  int T;        /* rows of one step: 1 + (W + G)(N - 1) */
  int kvdim;    /* n_kv_heads * head_dim */
  int qdim;     /* n_heads * head_dim */
  const void **w; /* 3 + 9 * n_layers weight pointers */
  double *kc, *vc; /* [layer][kv head][max_ctx][head_dim] */
  int32_t L;      /* committed KV length */
  int32_t cur;    /* current token (its KV is not committed yet) */
  int32_t *win;   /* [N-1][W], row 0 = level 1 (oldest) */
  int32_t *pool_len; /* [vocab] */
  int32_t *pool;     /* [vocab][G][N-1], oldest first */
  /* last forwarded block, kept for commit */
  int has_block;
  int32_t *btok, *bvalid;
  double *blk_k, *blk_v; /* [layer][T][kvdim] */
  double *logits;        /* [T][vocab] */
  /* sampling (temperature 0: greedy) */
  double temperature, top_p;
  int32_t top_k;
  uint64_t seed;
} orc;

/* ------------------------------------------------------------------------ */
/* weights                                                                  */

enum { W_EMB = 0, W_FNORM = 1, W_LM = 2, W_LAYER0 = 3 };
enum { L_ANORM = 0, L_Q, L_K, L_V, L_O, L_FNORM, L_GATE, L_UP, L_DOWN, L_NW };

static const void *lw(const orc *o, int layer, int which) {
  return o->w[W_LAYER0 + L_NW * layer + which];
}

static double bf16_to_double(uint16_t b) {
  union { uint32_t u; float f; } v;
  v.u = (uint32_t)b << 16;
  return (double)v.f;
}

/* bfloat16 storage of a value: the value rounded to fp32 (binary32, to
 * nearest even), then to the nearest bfloat16, i.e. to 8 significant bits,
 * ties to even (nearbyint in the default rounding mode); bfloat16 is the
 * upper half of a binary32 word, so the conversion is defined from fp32.
 * Exponents stay in fp32's normal range for every value a model produces. */
double orc_round_bf16(double v) {
  const double f = (double)(float)v;
  if (f == 0.0 || !isfinite(f)) return f;
  int e;
  const double m = frexp(f, &e); /* f = m 2^e, 0.5 <= |m| < 1 */
  return ldexp(nearbyint(ldexp(m, 8)), e - 8);
}
#define round_bf16 orc_round_bf16

/* A stored activation: rounded in bf16 storage mode, exact otherwise. */
static double stored(const orc *o, double v) {
  return o->c.act_bf16 ? round_bf16(v) : v;
}

static double wget(const void *p, size_t i, int dt) {
  return dt ? bf16_to_double(((const uint16_t *)p)[i])
            : (double)((const float *)p)[i];
}

/* Widen row n of a [rows][K] weight matrix into dst[K]. */
static void wrow(const void *p, size_t n, int K, int dt, double *dst) {
  size_t base = n * (size_t)K;
  if (dt) {
    const uint16_t *q = (const uint16_t *)p + base;
    for (int k = 0; k < K; k++) dst[k] = bf16_to_double(q[k]);
  } else {
    const float *q = (const float *)p + base;
    for (int k = 0; k < K; k++) dst[k] = (double)q[k];
  }
}

/* Y[r][n] = sum_k X[r][k] * Wt[n][k], k ascending, one thread per (n, all r).
 * Four rows run side by side; each row's sum is still sequential in k. */
static void matmul_wt(const double *X, int R, int K, const void *Wt, int Nout,
                      int dt, double *Y) {
#pragma omp parallel
  {
    double *row = (double *)malloc(sizeof(double) * (size_t)K);
#pragma omp for schedule(static)
    for (int n = 0; n < Nout; n++) {
      wrow(Wt, (size_t)n, K, dt, row);
      int r = 0;
      for (; r + 4 <= R; r += 4) {
        const double *x0 = X + (size_t)r * K, *x1 = x0 + K, *x2 = x1 + K,
                     *x3 = x2 + K;
        double s0 = 0, s1 = 0, s2 = 0, s3 = 0;
        for (int k = 0; k < K; k++) {
          s0 += x0[k] * row[k];
          s1 += x1[k] * row[k];
          s2 += x2[k] * row[k];
          s3 += x3[k] * row[k];
        }
        Y[(size_t)r * Nout + n] = s0;
        Y[(size_t)(r + 1) * Nout + n] = s1;
        Y[(size_t)(r + 2) * Nout + n] = s2;
        Y[(size_t)(r + 3) * Nout + n] = s3;
      }
      for (; r < R; r++) {
        const double *x = X + (size_t)r * K;
        double s = 0;
        for (int k = 0; k < K; k++) s += x[k] * row[k];
        Y[(size_t)r * Nout + n] = s;
      }
    }
    free(row);
  }
}

/* ------------------------------------------------------------------------ */
/* model pieces                                                             */

/* RMSNorm: x / sqrt(mean(x^2) + eps) * w */
static void rmsnorm(const orc *o, const double *x, int R, const void *w,
                    double *out) {
  int d = o->c.d_model, dt = o->c.wdtype;
  for (int r = 0; r < R; r++) {
    const double *xr = x + (size_t)r * d;
    double ss = 0;
    for (int i = 0; i < d; i++) ss += xr[i] * xr[i];
    double inv = 1.0 / sqrt(ss / d + o->c.rms_eps);
    for (int i = 0; i < d; i++)
      out[(size_t)r * d + i] = xr[i] * inv * wget(w, (size_t)i, dt);
  }
}

/* bf16 storage (1 and 5 of the header): the block input is held as
 * bf16(x * w); inv[r] = 1/rms(x_r) scales row r of the products instead. */
static void norm_input_bf16(const orc *o, const double *x, int R, const void *w,
                            double *out, double *inv) {
  int d = o->c.d_model, dt = o->c.wdtype;
  for (int r = 0; r < R; r++) {
    const double *xr = x + (size_t)r * d;
    double ss = 0;
    for (int i = 0; i < d; i++) ss += xr[i] * xr[i];
    inv[r] = 1.0 / sqrt(ss / d + o->c.rms_eps);
    for (int i = 0; i < d; i++)
      out[(size_t)r * d + i] = round_bf16(xr[i] * wget(w, (size_t)i, dt));
  }
}

static void scale_rows(double *y, int R, int n, const double *inv) {
  for (int r = 0; r < R; r++)
    for (int i = 0; i < n; i++) y[(size_t)r * n + i] *= inv[r];
}

static void round_all(double *y, size_t n) {
  for (size_t i = 0; i < n; i++) y[i] = round_bf16(y[i]);
}

/* Rotary embedding of one head vector at absolute position pos, rotating the
 * adjacent pairs (2i, 2i+1) by pos * theta^(-2i/dh). */
static void rope(const orc *o, double *v, int pos) {
  int dh = o->c.head_dim;
  for (int i = 0; i < dh / 2; i++) {
    double ang = (double)pos * pow(o->c.rope_theta, -2.0 * i / dh);
    double c = cos(ang), s = sin(ang);
    double a = v[2 * i], b = v[2 * i + 1];
    v[2 * i] = a * c - b * s;
    v[2 * i + 1] = a * s + b * c;
  }
}

static double silu(double g) { return g / (1.0 + exp(-g)); }

/*
 * Forward R rows through every layer.
 *   tok[R], pos[R]: token id and absolute position of each row;
 *   vis[R*R]: row r attends to row s (s != r allowed) iff vis[r*R + s];
 *   every row also attends to all committed cache positions 0..L-1.
 * Keys are visited in ascending position: the cache first, then the
 * visible rows sorted by position (ties by row index).
 * Outputs: bk/bv [layer][R][kvdim] (the rows' keys after RoPE, and values)
 * and logits [R][vocab] for rows with want[r] (all rows if want is NULL).
 */
static void forward(orc *o, int R, const int32_t *tok, const int32_t *pos,
                    const uint8_t *vis, double *bk, double *bv,
                    double *logits, const uint8_t *want) {
  const orc_config *c = &o->c;
  int d = c->d_model, dh = c->head_dim, H = c->n_heads, Hkv = c->n_kv_heads;
  int qd = o->qdim, kvd = o->kvdim, F = c->d_ffn, V = c->vocab, dt = c->wdtype;
  int L = o->L;
  double *x = malloc(sizeof(double) * (size_t)R * d);
  double *n = malloc(sizeof(double) * (size_t)R * d);
  double *q = malloc(sizeof(double) * (size_t)R * qd);
  double *att = malloc(sizeof(double) * (size_t)R * qd);
  double *tmp = malloc(sizeof(double) * (size_t)R * d);
  double *g = malloc(sizeof(double) * (size_t)R * F);
  double *u = malloc(sizeof(double) * (size_t)R * F);
  double *inv = malloc(sizeof(double) * (size_t)R);
  const int bf = c->act_bf16;
  /* per-row key order among the block rows */
  int *order = malloc(sizeof(int) * (size_t)R * R);
  int *nord = malloc(sizeof(int) * (size_t)R);
  for (int r = 0; r < R; r++) {
    int m = 0;
    for (int s = 0; s < R; s++)
      if (vis[(size_t)r * R + s]) {
        int j = m++;
        while (j > 0) {
          int p = order[(size_t)r * R + j - 1];
          if (pos[p] < pos[s] || (pos[p] == pos[s] && p < s)) break;
          order[(size_t)r * R + j] = p;
          j--;
        }
        order[(size_t)r * R + j] = s;
      }
    nord[r] = m;
  }

  for (int r = 0; r < R; r++)
    for (int i = 0; i < d; i++)
      x[(size_t)r * d + i] = wget(o->w[W_EMB], (size_t)tok[r] * d + i, dt);

  double scale = 1.0 / sqrt((double)dh);
  for (int l = 0; l < c->n_layers; l++) {
    double *lk = bk + (size_t)l * R * kvd, *lv = bv + (size_t)l * R * kvd;
    if (bf) norm_input_bf16(o, x, R, lw(o, l, L_ANORM), n, inv);
    else rmsnorm(o, x, R, lw(o, l, L_ANORM), n);
    matmul_wt(n, R, d, lw(o, l, L_Q), qd, dt, q);
    matmul_wt(n, R, d, lw(o, l, L_K), kvd, dt, lk);
    matmul_wt(n, R, d, lw(o, l, L_V), kvd, dt, lv);
    if (bf) {
      scale_rows(q, R, qd, inv);
      scale_rows(lk, R, kvd, inv);
      scale_rows(lv, R, kvd, inv);
    }
    for (int r = 0; r < R; r++) {
      for (int h = 0; h < H; h++) rope(o, q + (size_t)r * qd + h * dh, pos[r]);
      for (int h = 0; h < Hkv; h++) rope(o, lk + (size_t)r * kvd + h * dh, pos[r]);
    }
    if (bf) { /* 2: the query and the KV cache rows */
      round_all(q, (size_t)R * qd);
      round_all(lk, (size_t)R * kvd);
      round_all(lv, (size_t)R * kvd);
    }
    const double *ck = o->kc + (size_t)l * Hkv * c->max_ctx * dh;
    const double *cv = o->vc + (size_t)l * Hkv * c->max_ctx * dh;
#pragma omp parallel
    {
      double *sc = malloc(sizeof(double) * (size_t)(L + R));
#pragma omp for collapse(2) schedule(static)
      for (int r = 0; r < R; r++)
        for (int h = 0; h < H; h++) {
          int kh = (int)(((long)h * Hkv) / H);
          const double *qr = q + (size_t)r * qd + h * dh;
          int nk = L + nord[r];
          /* scores, in key order */
          for (int j = 0; j < nk; j++) {
            const double *kv = j < L ? ck + ((size_t)kh * c->max_ctx + j) * dh
                                     : lk + (size_t)order[(size_t)r * R + j - L] * kvd + kh * dh;
            double s = 0;
            for (int i = 0; i < dh; i++) s += qr[i] * kv[i];
            sc[j] = s * scale;
          }
          double m = -INFINITY;
          for (int j = 0; j < nk; j++) m = sc[j] > m ? sc[j] : m;
          double z = 0;
          for (int j = 0; j < nk; j++) {
            sc[j] = exp(sc[j] - m);
            z += sc[j];
          }
          double *out = att + (size_t)r * qd + h * dh;
          for (int i = 0; i < dh; i++) out[i] = 0;
          for (int j = 0; j < nk; j++) {
            const double *vv = j < L ? cv + ((size_t)kh * c->max_ctx + j) * dh
                                     : lv + (size_t)order[(size_t)r * R + j - L] * kvd + kh * dh;
            const double pj = stored(o, sc[j]); /* 3 */
            for (int i = 0; i < dh; i++) out[i] += pj * vv[i];
          }
          for (int i = 0; i < dh; i++) out[i] = stored(o, out[i] / z); /* 4 */
        }
      free(sc);
    }
    matmul_wt(att, R, qd, lw(o, l, L_O), d, dt, tmp);
    for (size_t i = 0; i < (size_t)R * d; i++) x[i] += tmp[i];
    if (bf) norm_input_bf16(o, x, R, lw(o, l, L_FNORM), n, inv);
    else rmsnorm(o, x, R, lw(o, l, L_FNORM), n);
    matmul_wt(n, R, d, lw(o, l, L_GATE), F, dt, g);
    matmul_wt(n, R, d, lw(o, l, L_UP), F, dt, u);
    if (bf) {
      scale_rows(g, R, F, inv);
      scale_rows(u, R, F, inv);
    }
    for (size_t i = 0; i < (size_t)R * F; i++) g[i] = stored(o, silu(g[i]) * u[i]); /* 6 */
    matmul_wt(g, R, F, lw(o, l, L_DOWN), d, dt, tmp);
    for (size_t i = 0; i < (size_t)R * d; i++) x[i] += tmp[i];
  }

  if (logits) {
    /* final norm + LM head over the wanted rows only */
    int nw = 0;
    for (int r = 0; r < R; r++) nw += want ? want[r] != 0 : 1;
    double *xs = malloc(sizeof(double) * (size_t)(nw ? nw : 1) * d);
    double *ls = malloc(sizeof(double) * (size_t)(nw ? nw : 1) * V);
    int m = 0;
    for (int r = 0; r < R; r++)
      if (!want || want[r]) memcpy(xs + (size_t)m++ * d, x + (size_t)r * d, sizeof(double) * d);
    rmsnorm(o, xs, nw, o->w[W_FNORM], n);
    if (bf) round_all(n, (size_t)nw * d); /* 7 */
    matmul_wt(n, nw, d, o->w[W_LM], V, dt, ls);
    m = 0;
    for (int r = 0; r < R; r++)
      if (!want || want[r]) memcpy(logits + (size_t)r * V, ls + (size_t)m++ * V, sizeof(double) * V);
    free(xs);
    free(ls);
  }
  free(x); free(n); free(q); free(att); free(tmp); free(g); free(u); free(inv);
  free(order); free(nord);
}

/* Copy one forwarded row's K/V (all layers) into cache position p. */
static void commit_row(orc *o, const double *bk, const double *bv, int R,
                       int row, int p) {
  const orc_config *c = &o->c;
  int dh = c->head_dim, kvd = o->kvdim;
  for (int l = 0; l < c->n_layers; l++)
    for (int h = 0; h < c->n_kv_heads; h++) {
      size_t dst = (((size_t)l * c->n_kv_heads + h) * c->max_ctx + p) * dh;
      size_t src = ((size_t)l * R + row) * kvd + (size_t)h * dh;
      memcpy(o->kc + dst, bk + src, sizeof(double) * dh);
      memcpy(o->vc + dst, bv + src, sizeof(double) * dh);
    }
}

/* Argmax over logits rounded to fp32; lowest token id on ties. */
static int argmax_f32(const double *lg, int V) {
  int best = 0;
  float bv = (float)lg[0];
  for (int i = 1; i < V; i++) {
    float v = (float)lg[i];
    if (v > bv) { bv = v; best = i; }
  }
  return best;
}

/* ------------------------------------------------------------------------ */
/* sampling ("Break the Sequential Dependency of LLM Inference Using
 * Lookahead Decoding", Summary: the method supports sampling as well as
 * greedy decoding, with no algorithm given, so all of this is a reading)   */

/* Philox4x32-10, the counter-based generator of Salmon, Moraes, Dror and
 * Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11): ten rounds;
 * each multiplies words 0 and 2 by two fixed 32-bit constants, keeps the
 * low halves and mixes the high halves with words 1 and 3 and the key;
 * the key advances by two Weyl increments between rounds. */
void orc_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
  uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
  uint32_t k0 = key_in[0], k1 = key_in[1];
  for (int r = 0; r < 10; r++) {
    uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    uint32_t n1 = (uint32_t)p1;
    uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    uint32_t n3 = (uint32_t)p0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* The uniform that draws the token at absolute sequence position pos
 * (prompt tokens at 0..P-1, the first generated token at P): Philox with
 * counter (pos low, pos high, 0, 0) and key (seed low, seed high); the top
 * 24 bits of word 0 scaled by 2^-24, so u in [0, 1) is exact in fp32.
 * Keying by position, not by step, makes a sampled lookahead run draw
 * every token with the same uniform as plain sampled decoding. */
double orc_uniform(uint64_t seed, int64_t pos) {
  uint32_t ctr[4] = {(uint32_t)pos, (uint32_t)((uint64_t)pos >> 32), 0u, 0u};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t out[4];
  orc_philox4x32_10(ctr, key, out);
  return (double)(out[0] >> 8) * (1.0 / 16777216.0);
}

typedef struct { double z; int32_t i; } orc_zi;

/* logit descending, lower token id first on equal logits */
static int zi_cmp(const void *pa, const void *pb) {
  const orc_zi *a = pa, *b = pb;
  if (a->z != b->z) return a->z > b->z ? -1 : 1;
  return a->i < b->i ? -1 : (a->i > b->i);
}

/*
 * One draw from a row of logits (reading):
 *   1. order the tokens by logit, descending, lower id first on ties;
 *   2. keep the first top_k of them (all when top_k is 0 or >= V);
 *   3. weights w = exp((z - z_max) / temperature) over the kept tokens;
 *      with top_p < 1 keep the shortest prefix whose weight sum reaches
 *      top_p times the kept total (at least one token);
 *   4. return the first kept token whose running weight sum exceeds
 *      u times the remaining total.
 * The decision takes the logits rounded to fp32 (as the argmax does) and
 * computes in double.  *margin (may be NULL) receives how far the draw is
 * from changing: the smallest of the distance from u to the ends of the
 * drawn token's interval and from the top-p cut to the running sums beside
 * it (fractions of the totals), and the logit gap at the top-k cut over
 * the temperature.  A logit error e moves each of these by about 2e/T at
 * most.
 */
int orc_sample_logits(const double *lg, int V, double temperature, int top_k, double top_p,
                      double u, double *margin) {
  orc_zi *a = malloc(sizeof(orc_zi) * (size_t)V);
  for (int j = 0; j < V; j++) {
    a[j].z = (double)(float)lg[j];
    a[j].i = j;
  }
  qsort(a, (size_t)V, sizeof(orc_zi), zi_cmp);
  int n = (top_k > 0 && top_k < V) ? top_k : V;
  double mg = INFINITY;
  if (n < V) mg = (a[n - 1].z - a[n].z) / temperature;
  double *w = malloc(sizeof(double) * (size_t)n);
  double tot = 0.0;
  for (int j = 0; j < n; j++) {
    w[j] = exp((a[j].z - a[0].z) / temperature);
    tot += w[j];
  }
  if (top_p < 1.0) {
    const double cut = top_p * tot;
    double run = 0.0;
    int m = n;
    for (int j = 0; j < n; j++) {
      const double prev = run;
      run += w[j];
      if (run >= cut) {
        m = j + 1;
        double d = fmin(cut - prev, run - cut) / tot;
        if (j == 0) d = (run - cut) / tot;  /* one token is always kept */
        mg = fmin(mg, d);
        break;
      }
    }
    n = m;
  }
  double z2 = 0.0;
  for (int j = 0; j < n; j++) z2 += w[j];
  const double target = u * z2;
  double run = 0.0;
  int pick = n - 1;
  for (int j = 0; j < n; j++) {
    if (run + w[j] > target) {
      pick = j;
      break;
    }
    run += w[j];
  }
  mg = fmin(mg, fmin(target - run, run + w[pick] - target) / z2);
  if (margin) *margin = mg;
  const int tok = a[pick].i;
  free(a);
  free(w);
  return tok;
}

/* The decision for a row whose output is the token at position pos:
 * greedy argmax, or a draw with that position's uniform. */
static int decide(const orc *o, const double *lg, int64_t pos, double *margin) {
  if (o->temperature > 0.0)
    return orc_sample_logits(lg, o->c.vocab, o->temperature, o->top_k, o->top_p,
                             orc_uniform(o->seed, pos), margin);
  if (margin) *margin = NAN;
  return argmax_f32(lg, o->c.vocab);
}

/* ------------------------------------------------------------------------ */
/* block layout and mask (reading of the Summary's 2D window + verification
 * branch in one pass)                                                      */

/* Row index of lookahead row (level l in 1..N-1, column j) and candidate row
 * (candidate g, index i in 1..N-1). Row 0 is the current token. */
static int row_la(const orc_config *c, int l, int j) { return 1 + (l - 1) * c->W + j; }
static int row_cand(const orc_config *c, int g, int i) {
  return 1 + (c->N - 1) * c->W + g * (c->N - 1) + (i - 1);
}

/* Decode a row index: kind 0 current, 1 lookahead (a = level, b = column),
 * 2 candidate (a = candidate, b = index). */
static void row_kind(const orc_config *c, int r, int *kind, int *a, int *b) {
  int nla = (c->N - 1) * c->W;
  if (r == 0) { *kind = 0; *a = 0; *b = 0; }
  else if (r <= nla) { *kind = 1; *a = 1 + (r - 1) / c->W; *b = (r - 1) % c->W; }
  else { *kind = 2; *a = (r - 1 - nla) / (c->N - 1); *b = 1 + (r - 1 - nla) % (c->N - 1); }
}

/* Relative position of a block row: 0 for the current token, l + j for
 * lookahead (l, j), i for candidate (g, i) (reading: consecutive positions
 * along each n-gram). */
int orc_row_pos(const orc_config *c, int r) {
  int k, a, b;
  row_kind(c, r, &k, &a, &b);
  return k == 0 ? 0 : (k == 1 ? a + b : b);
}

/* Does block row r see block row s? (reading)
 *   current token: itself only;
 *   lookahead (l, j): the current token, level-1 rows of columns j' <= j,
 *     and rows (l', j) of its own column for 2 <= l' <= l;
 *   candidate (g, i): the current token and (g, i') for i' <= i.
 * Lookahead and candidate groups never see each other, and candidates never
 * see other candidates. */
int orc_visible(const orc_config *c, int r, int s) {
  int kr, ar, br, ks, as, bs;
  row_kind(c, r, &kr, &ar, &br);
  row_kind(c, s, &ks, &as, &bs);
  if (ks == 0) return 1;
  if (kr == 0) return 0;
  if (kr == 1 && ks == 1) {
    if (as == 1) return bs <= br;
    return bs == br && as <= ar;
  }
  if (kr == 2 && ks == 2) return as == ar && bs <= br;
  return 0;
}

/* ------------------------------------------------------------------------ */
/* n-gram pool (reading of the Summary's n-gram store, keyed by lead token with at
 * most G tails per key): each key holds distinct (N-1)-token tails, oldest
 * first; inserting a tail already present moves it to the newest slot;
 * inserting a new tail into a full list drops the oldest.                  */

void orc_pool_insert(orc *o, int32_t key, const int32_t *tail) {
  int G = o->c.G, n1 = o->c.N - 1;
  if (G <= 0) return;
  int32_t *lst = o->pool + (size_t)key * G * n1;
  int len = o->pool_len[key];
  int found = -1;
  for (int e = 0; e < len && found < 0; e++)
    if (memcmp(lst + (size_t)e * n1, tail, sizeof(int32_t) * n1) == 0) found = e;
  int from;
  if (found >= 0) from = found;
  else if (len == G) from = 0;
  else from = len++;
  /* close the gap at `from`, then append at the end */
  for (int e = from; e + 1 < len; e++)
    memcpy(lst + (size_t)e * n1, lst + (size_t)(e + 1) * n1, sizeof(int32_t) * n1);
  memcpy(lst + (size_t)(len - 1) * n1, tail, sizeof(int32_t) * n1);
  o->pool_len[key] = len;
}

/* ------------------------------------------------------------------------ */
/* public API                                                               */

orc *orc_create(const orc_config *cfg, const void *const *weights) {
  const orc_config *c = cfg;
  if (c->n_layers < 1 || c->d_model < 1 || c->n_heads < 1 || c->n_kv_heads < 1 ||
      c->n_heads % c->n_kv_heads || c->head_dim < 2 || c->head_dim % 2 ||
      c->d_ffn < 1 || c->vocab < 2 || c->N < 2 || c->N > 32 || c->W < 0 ||
      c->G < 0 || c->max_ctx < 1)
    return NULL;
  orc *o = calloc(1, sizeof(orc));
  if (o) o->top_p = 1.0; /* greedy until orc_set_sampling */
  o->c = *cfg;
  o->T = 1 + (c->W + c->G) * (c->N - 1);
  o->kvdim = c->n_kv_heads * c->head_dim;
  o->qdim = c->n_heads * c->head_dim;
  int nw = W_LAYER0 + L_NW * c->n_layers;
  o->w = malloc(sizeof(void *) * nw);
  memcpy(o->w, weights, sizeof(void *) * nw);
  size_t kv = (size_t)c->n_layers * c->n_kv_heads * c->max_ctx * c->head_dim;
  o->kc = calloc(kv, sizeof(double));
  o->vc = calloc(kv, sizeof(double));
  o->win = calloc((size_t)(c->N - 1) * (c->W ? c->W : 1), sizeof(int32_t));
  o->pool_len = calloc((size_t)c->vocab, sizeof(int32_t));
  o->pool = calloc((size_t)c->vocab * (c->G ? c->G : 1) * (c->N - 1), sizeof(int32_t));
  o->btok = calloc((size_t)o->T, sizeof(int32_t));
  o->bvalid = calloc((size_t)o->T, sizeof(int32_t));
  o->blk_k = calloc((size_t)c->n_layers * o->T * o->kvdim, sizeof(double));
  o->blk_v = calloc((size_t)c->n_layers * o->T * o->kvdim, sizeof(double));
  o->logits = calloc((size_t)o->T * c->vocab, sizeof(double));
  if (!o->kc || !o->vc || !o->pool || !o->blk_k || !o->blk_v || !o->logits) {
    /* leave it to the caller to see NULL */
    free(o->kc); free(o->vc); free(o->win); free(o->pool_len); free(o->pool);
    free(o->btok); free(o->bvalid); free(o->blk_k); free(o->blk_v);
    free(o->logits); free(o->w); free(o);
    return NULL;
  }
  return o;
}

void orc_destroy(orc *o) {
  if (!o) return;
  free(o->kc); free(o->vc); free(o->win); free(o->pool_len); free(o->pool);
  free(o->btok); free(o->bvalid); free(o->blk_k); free(o->blk_v);
  free(o->logits); free(o->w); free(o);
}

int orc_rows(const orc *o) { return o->T; }
int orc_kv_len(const orc *o) { return o->L; }
int orc_current(const orc *o) { return o->cur; }

void orc_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int orc_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * Causal forward over `seq` starting at the committed length (positions
 * L..L+n-1); commits all n rows (L += n).  logits_all [n][vocab] receives
 * every row's logits when non-NULL; the last row's argmax is returned.
 * Returns -1 when the context would overflow.
 */
int orc_extend(orc *o, const int32_t *seq, int n, double *logits_all) {
  const orc_config *c = &o->c;
  if (n < 1 || o->L + n > c->max_ctx) return -1;
  int32_t *pos = malloc(sizeof(int32_t) * n);
  uint8_t *vis = calloc((size_t)n * n, 1);
  uint8_t *want = calloc((size_t)n, 1);
  for (int r = 0; r < n; r++) {
    pos[r] = o->L + r;
    for (int s = 0; s <= r; s++) vis[(size_t)r * n + s] = 1;
    want[r] = logits_all ? 1 : (r == n - 1);
  }
  double *bk = malloc(sizeof(double) * (size_t)c->n_layers * n * o->kvdim);
  double *bv = malloc(sizeof(double) * (size_t)c->n_layers * n * o->kvdim);
  double *lg = logits_all ? logits_all : malloc(sizeof(double) * (size_t)n * c->vocab);
  forward(o, n, seq, pos, vis, bk, bv, lg, want);
  for (int r = 0; r < n; r++) commit_row(o, bk, bv, n, r, o->L + r);
  o->L += n;
  /* the next token sits at position L: argmax, or a draw (sampling set) */
  int nxt = decide(o, lg + (size_t)(n - 1) * c->vocab, o->L, NULL);
  if (!logits_all) free(lg);
  free(pos); free(vis); free(want); free(bk); free(bv);
  return nxt;
}

/*
 * Prefill: empty the cache, run the prompt causally at positions 0..n-1,
 * set the current token to the argmax of the last row (the first generated
 * token, returned), install the initial window (N-1 levels x W, level 1
 * first; reading: the window starts full, no warm-up) and empty the pool.
 */
/* Seed the pool with every N-gram of a token sequence, in position order:
 * key seq[p], tail seq[p+1 .. p+N-1], for p = 0 .. n-N, each inserted with
 * the pool's policy (Key points, "Ablation": adding n-grams taken from the
 * prompt to the pool raises the speedup; reading: all prompt n-grams, in
 * order).  Returns 0, or -1 for a bad argument. */
int orc_seed_pool(orc *o, const int32_t *seq, int n) {
  const int n1 = o->c.N - 1;
  if (n < 0 || (n > 0 && !seq)) return -1;
  for (int i = 0; i < n; i++)
    if (seq[i] < 0 || seq[i] >= o->c.vocab) return -1;
  for (int p = 0; p + n1 < n; p++) orc_pool_insert(o, seq[p], seq + p + 1);
  return 0;
}

int orc_prefill(orc *o, const int32_t *prompt, int n, const int32_t *init_window,
                double *logits_all) {
  const orc_config *c = &o->c;
  o->L = 0;
  o->has_block = 0;
  memset(o->pool_len, 0, sizeof(int32_t) * (size_t)c->vocab);
  if (c->W > 0) {
    if (!init_window) return -1;
    memcpy(o->win, init_window, sizeof(int32_t) * (size_t)(c->N - 1) * c->W);
  }
  int t = orc_extend(o, prompt, n, logits_all);
  if (t < 0) return -1;
  o->cur = t;
  return t;
}

/*
 * Block rows for the next step from the state: row 0 = current token;
 * lookahead (l, j) = window level l, column j; candidate (g, i) = i-th token
 * of the g-th pool entry under the current token (oldest entry first;
 * reading).  valid[r] = 0 for candidate slots beyond the pool's entries.
 * Returns the candidate count.
 */
int orc_block_tokens(const orc *o, int32_t *tok, int32_t *valid) {
  const orc_config *c = &o->c;
  int n1 = c->N - 1;
  int nc = c->G > 0 ? o->pool_len[o->cur] : 0;
  tok[0] = o->cur;
  valid[0] = 1;
  for (int l = 1; l <= n1; l++)
    for (int j = 0; j < c->W; j++) {
      tok[row_la(c, l, j)] = o->win[(size_t)(l - 1) * c->W + j];
      valid[row_la(c, l, j)] = 1;
    }
  const int32_t *lst = o->pool + (size_t)o->cur * (c->G ? c->G : 1) * n1;
  for (int g = 0; g < c->G; g++)
    for (int i = 1; i <= n1; i++) {
      int r = row_cand(c, g, i);
      tok[r] = g < nc ? lst[(size_t)g * n1 + (i - 1)] : 0;
      valid[r] = g < nc;
    }
  return nc;
}

/*
 * Forward one block with the step mask at the current committed length:
 * every valid row sees the whole cache plus the block rows orc_visible
 * allows (invalid rows are left out entirely).  logits_out [T][vocab]
 * receives the valid rows' logits (NaN for invalid rows).  With keep != 0
 * the block is kept for orc_commit.
 */
int orc_forward_block(orc *o, const int32_t *tok, const int32_t *valid,
                      double *logits_out, int keep) {
  const orc_config *c = &o->c;
  int T = o->T;
  if (o->L + T > c->max_ctx) return -1;
  int R = 0;
  int *map = malloc(sizeof(int) * T);
  for (int r = 0; r < T; r++)
    if (valid[r]) map[R++] = r;
  int32_t *t2 = malloc(sizeof(int32_t) * R), *p2 = malloc(sizeof(int32_t) * R);
  uint8_t *vis = calloc((size_t)R * R, 1);
  for (int a = 0; a < R; a++) {
    t2[a] = tok[map[a]];
    p2[a] = o->L + orc_row_pos(c, map[a]);
    for (int b = 0; b < R; b++) vis[(size_t)a * R + b] = (uint8_t)orc_visible(c, map[a], map[b]);
  }
  double *bk = malloc(sizeof(double) * (size_t)c->n_layers * R * o->kvdim);
  double *bv = malloc(sizeof(double) * (size_t)c->n_layers * R * o->kvdim);
  double *lg = malloc(sizeof(double) * (size_t)R * c->vocab);
  forward(o, R, t2, p2, vis, bk, bv, lg, NULL);
  double *dst = keep ? o->logits : logits_out;
  if (dst) {
    for (size_t i = 0; i < (size_t)T * c->vocab; i++) dst[i] = NAN;
    for (int a = 0; a < R; a++)
      memcpy(dst + (size_t)map[a] * c->vocab, lg + (size_t)a * c->vocab, sizeof(double) * c->vocab);
  }
  if (keep) {
    if (logits_out) memcpy(logits_out, o->logits, sizeof(double) * (size_t)T * c->vocab);
    for (int l = 0; l < c->n_layers; l++)
      for (int a = 0; a < R; a++) {
        size_t s = ((size_t)l * R + a) * o->kvdim, d = ((size_t)l * T + map[a]) * o->kvdim;
        memcpy(o->blk_k + d, bk + s, sizeof(double) * o->kvdim);
        memcpy(o->blk_v + d, bv + s, sizeof(double) * o->kvdim);
      }
    memcpy(o->btok, tok, sizeof(int32_t) * T);
    memcpy(o->bvalid, valid, sizeof(int32_t) * T);
    o->has_block = 1;
  }
  free(map); free(t2); free(p2); free(vis); free(bk); free(bv); free(lg);
  return R;
}

/* Argmax of every valid row of the kept block (lowest id on ties, fp32). */
int orc_block_argmax(const orc *o, int32_t *amax) {
  if (!o->has_block) return -1;
  for (int r = 0; r < o->T; r++)
    amax[r] = o->bvalid[r] ? argmax_f32(o->logits + (size_t)r * o->c.vocab, o->c.vocab) : -1;
  return 0;
}

/* The decision of every valid row of the kept block: lookahead rows take
 * the argmax (they only propose n-grams; reading); the current-token row
 * and the candidate rows, whose outputs are the tokens verification emits,
 * take decide() for their output position, L + relative position + 1.
 * margin[T] (may be NULL) receives the draws' margins (NaN for argmax). */
int orc_block_select(const orc *o, int32_t *sel, double *margin) {
  if (!o->has_block) return -1;
  for (int r = 0; r < o->T; r++) {
    double m = NAN;
    int k, a, b;
    row_kind(&o->c, r, &k, &a, &b);
    const double *lg = o->logits + (size_t)r * o->c.vocab;
    if (!o->bvalid[r]) sel[r] = -1;
    else if (k == 1) sel[r] = argmax_f32(lg, o->c.vocab);
    else sel[r] = decide(o, lg, (int64_t)o->L + orc_row_pos(&o->c, r) + 1, &m);
    if (margin) margin[r] = m;
  }
  return 0;
}

/* Sampling for the tokens this context emits from now on (temperature 0:
 * greedy; top_k 0: no cut; top_p 1: no cut).  Returns -1 for bad values. */
int orc_set_sampling(orc *o, double temperature, int top_k, double top_p, uint64_t seed) {
  if (!(temperature >= 0.0) || top_k < 0 || !(top_p > 0.0 && top_p <= 1.0)) return -1;
  o->temperature = temperature;
  o->top_k = top_k;
  o->top_p = top_p;
  o->seed = seed;
  return 0;
}

/*
 * Finish the step for the kept block, given the per-row decisions amax[T]
 * (NULL: take the oracle's own, orc_block_select: argmax when greedy, the
 * draws when sampling).
 *   Verification (greedy; with sampling the same rule on the draws, so a
 *   candidate token is accepted exactly when it equals the token drawn at
 *   its position, which keeps every emitted token a draw from the model's
 *   distribution given the tokens before it): candidate g is accepted for k_g tokens, the
 *   longest prefix with cand[g][0] == argmax(row 0) and cand[g][i] ==
 *   argmax(row (g, i)) for 1 <= i < k_g; the winner g* is the lowest g with
 *   the largest k_g.  Emit cand[g*][0..k-1] and then the next greedy token
 *   (argmax of row (g*, k), or of row 0 when k = 0).
 *   KV: row 0 goes to position L, rows (g*, 1..k) to L+1..L+k; L += k + 1.
 *   Lookahead: the new level is the argmax of the last level's rows
 *   (reading); for j = 0..W-1 in order the n-gram (win[1][j], ...,
 *   win[N-1][j], new[j]) enters the pool keyed by win[1][j]; then every
 *   level moves down by one and the new level becomes level N-1 (reading:
 *   one level per step whatever k is).
 */
int orc_commit(orc *o, const int32_t *amax_in, orc_result *res) {
  const orc_config *c = &o->c;
  if (!o->has_block) return -1;
  int T = o->T, n1 = c->N - 1, W = c->W;
  int32_t *amax = malloc(sizeof(int32_t) * T);
  if (amax_in) memcpy(amax, amax_in, sizeof(int32_t) * T);
  else orc_block_select(o, amax, NULL);
  int nc = 0;
  for (int g = 0; g < c->G; g++) nc += o->bvalid[row_cand(c, g, 1)] != 0;
  int a0 = amax[0];
  int best_k = 0, best_g = -1;
  for (int g = 0; g < nc; g++) {
    int k = 0;
    while (k < n1) {
      int tokk = o->btok[row_cand(c, g, k + 1)];      /* cand[g][k] */
      int pred = k == 0 ? a0 : amax[row_cand(c, g, k)];
      if (tokk != pred) break;
      k++;
    }
    if (best_g < 0 || k > best_k) { best_k = k; best_g = g; }
  }
  int k = best_g >= 0 ? best_k : 0;
  memset(res, 0, sizeof(*res));
  for (int i = 0; i < k; i++) res->tokens[i] = o->btok[row_cand(c, best_g, i + 1)];
  int bonus = k == 0 ? a0 : amax[row_cand(c, best_g, k)];
  res->tokens[k] = bonus;
  res->n_emitted = k + 1;
  res->accepted = k;
  res->winner = best_g;
  res->n_candidates = nc;
  /* KV commit */
  commit_row(o, o->blk_k, o->blk_v, T, 0, o->L);
  for (int i = 1; i <= k; i++) commit_row(o, o->blk_k, o->blk_v, T, row_cand(c, best_g, i), o->L + i);
  o->L += k + 1;
  o->cur = bonus;
  res->kv_len = o->L;
  /* lookahead branch: new level, pool insert, shift */
  if (W > 0) {
    int32_t *ynew = malloc(sizeof(int32_t) * W);
    int32_t *tail = malloc(sizeof(int32_t) * n1);
    for (int j = 0; j < W; j++) ynew[j] = amax[row_la(c, n1, j)];
    for (int j = 0; j < W; j++) {
      for (int l = 2; l <= n1; l++) tail[l - 2] = o->win[(size_t)(l - 1) * W + j];
      tail[n1 - 1] = ynew[j];
      orc_pool_insert(o, o->win[j], tail);
    }
    for (int l = 1; l < n1; l++) memcpy(o->win + (size_t)(l - 1) * W, o->win + (size_t)l * W, sizeof(int32_t) * W);
    memcpy(o->win + (size_t)(n1 - 1) * W, ynew, sizeof(int32_t) * W);
    free(ynew);
    free(tail);
  }
  o->has_block = 0;
  free(amax);
  return 0;
}

/* One whole lookahead step with the oracle's own decisions. */
int orc_step(orc *o, orc_result *res, double *logits_out) {
  int32_t *tok = malloc(sizeof(int32_t) * o->T), *val = malloc(sizeof(int32_t) * o->T);
  orc_block_tokens(o, tok, val);
  int rc = orc_forward_block(o, tok, val, logits_out, 1);
  if (rc >= 0) rc = orc_commit(o, NULL, res);
  free(tok);
  free(val);
  return rc;
}

/* Plain one-token decoding: after orc_prefill, each call appends the
 * current token (one row at position L) and returns the next token (the
 * argmax, or the draw at its position when sampling is set). */
int orc_greedy_next(orc *o, double *logits_out) {
  int t = orc_extend(o, &o->cur, 1, logits_out);
  if (t < 0) return -1;
  o->cur = t;
  return t;
}

/* Rewind to committed length L (0 <= L <= the current length) with current
 * token cur: cache positions from L on are dropped; window and pool are
 * kept.  Tests use it to decode ahead with plain decoding and come back.
 * Returns 0, or -1 for a bad argument. */
int orc_rewind(orc *o, int L, int32_t cur) {
  if (L < 0 || L > o->L || cur < 0 || cur >= o->c.vocab) return -1;
  o->L = L;
  o->cur = cur;
  o->has_block = 0;
  return 0;
}

/* State inspection. */
void orc_get_window(const orc *o, int32_t *win) {
  memcpy(win, o->win, sizeof(int32_t) * (size_t)(o->c.N - 1) * o->c.W);
}
void orc_set_window(orc *o, const int32_t *win) {
  memcpy(o->win, win, sizeof(int32_t) * (size_t)(o->c.N - 1) * o->c.W);
}
void orc_set_current(orc *o, int32_t cur) { o->cur = cur; }
void orc_get_pool(const orc *o, int32_t *len, int32_t *tails) {
  memcpy(len, o->pool_len, sizeof(int32_t) * (size_t)o->c.vocab);
  if (o->c.G > 0)
    memcpy(tails, o->pool, sizeof(int32_t) * (size_t)o->c.vocab * o->c.G * (o->c.N - 1));
}
/* K/V of cache positions pos0..pos0+n-1 of one layer: [kv head][n][dh]. */
int orc_get_kv(const orc *o, int layer, int pos0, int n, double *k, double *v) {
  const orc_config *c = &o->c;
  if (layer < 0 || layer >= c->n_layers || pos0 < 0 || pos0 + n > c->max_ctx) return -1;
  for (int h = 0; h < c->n_kv_heads; h++)
    for (int p = 0; p < n; p++) {
      size_t s = (((size_t)layer * c->n_kv_heads + h) * c->max_ctx + pos0 + p) * c->head_dim;
      size_t d = ((size_t)h * n + p) * c->head_dim;
      memcpy(k + d, o->kc + s, sizeof(double) * c->head_dim);
      memcpy(v + d, o->vc + s, sizeof(double) * c->head_dim);
    }
  return 0;
}

/*
 * Masked attention of one layer on its own (the kernel-only workload):
 * q [T][H][dh]; k, v [Hkv][L + T][dh] where positions L..L+T-1 hold the
 * block rows in row order; out [T][H][dh].  Row r sees keys 0..L-1 and the
 * block rows orc_visible allows, among the valid ones (valid[r]; NULL = all
 * valid).  Inputs are bfloat16 bit patterns when bf16 != 0, else float32.
 * Invalid rows get zeros.  Keys visited in ascending position.
 */
void orc_attention(const orc_config *c, int L, const void *q, const void *k,
                   const void *v, int bf16, const int32_t *valid, double *out) {
  int T = 1 + (c->W + c->G) * (c->N - 1);
  int H = c->n_heads, Hkv = c->n_kv_heads, dh = c->head_dim;
  double scale = 1.0 / sqrt((double)dh);
#pragma omp parallel
  {
    double *sc = malloc(sizeof(double) * (size_t)(L + T));
    int *keys = malloc(sizeof(int) * (size_t)(L + T));
#pragma omp for collapse(2) schedule(static)
    for (int r = 0; r < T; r++)
      for (int h = 0; h < H; h++) {
        double *o = out + ((size_t)r * H + h) * dh;
        for (int i = 0; i < dh; i++) o[i] = 0;
        if (valid && !valid[r]) continue;
        int kh = (int)(((long)h * Hkv) / H);
        int nk = 0;
        for (int j = 0; j < L; j++) keys[nk++] = j;
        /* visible block rows sorted by relative position */
        int pr = orc_row_pos(c, r);
        for (int p = 0; p <= pr; p++)
          for (int s = 0; s < T; s++)
            if ((!valid || valid[s]) && orc_visible(c, r, s) && orc_row_pos(c, s) == p)
              keys[nk++] = L + s;
        for (int j = 0; j < nk; j++) {
          double s = 0;
          for (int i = 0; i < dh; i++)
            s += wget(q, ((size_t)r * H + h) * dh + i, bf16) *
                 wget(k, ((size_t)kh * (L + T) + keys[j]) * dh + i, bf16);
          sc[j] = s * scale;
        }
        double m = -INFINITY;
        for (int j = 0; j < nk; j++) m = sc[j] > m ? sc[j] : m;
        double z = 0;
        for (int j = 0; j < nk; j++) { sc[j] = exp(sc[j] - m); z += sc[j]; }
        for (int j = 0; j < nk; j++)
          for (int i = 0; i < dh; i++)
            o[i] += sc[j] * wget(v, ((size_t)kh * (L + T) + keys[j]) * dh + i, bf16);
        for (int i = 0; i < dh; i++) o[i] /= z;
      }
    free(sc);
    free(keys);
  }
}
