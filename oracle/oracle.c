/*
 * ORACLE — test infrastructure only.  A plain, slow, obviously ordered CPU implementation of the
 * Llama-architecture decoder step, used to check the GPU library and as the timed CPU baseline.
 * Only the tests, the smoke entry and the benchmark's CPU-baseline leg load it; the product path
 * never does.  It shares no code, header or table with the GPU library.
 *
 * Sources (page titles as printed):
 *   [bend]   bend-ml-llama@0.2.1.0 main.bend (jend.leeeet.dev): "The configuration", "The numeric
 *            pieces", "The key/value cache in flat arrays", "Grouped-query attention over the
 *            arrays", "A layer", "The model", "Sampling".  Every F32 operation there follows transformers'
 *            modeling_llama.py, and this file takes the same operations in the same order.
 *   [nest]   Llama 3.1 8B Instruct model card (nest.franknoh.dev): README "Validation" and
 *            `rope.linnet` (`tables`) for the llama3 frequency rescale; `attention.linnet`
 *            (`decode`, `prefill`, `decode_rows`) for positions and cache rows.
 *
 * Numerics: scalar F32 (float) throughout, built with -O2 -ffp-contract=off and no fast-math, so
 * every product and sum is rounded on its own, in the order written.  Dot products sum left to right
 * (the row product of a matmul); RMSNorm's sum of squares is the pairwise tree of [bend] `tree_sum`.
 * OpenMP splits only independent outputs (matrix rows, heads), so results do not depend on the
 * thread count.  bf16 tensors are uint16 bits widened exactly (bf16 is the upper half of an F32).
 * bf16 cache writes round F32 to bf16 with round-to-nearest-even (the reading taken for narrowing,
 * which the pages do not print).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ODT_F32 0
#define ODT_BF16 1

/* Cfg{kv, g, half, f, layers, vocab, eps, theta} ([bend] "The configuration") plus the llama3 rope
 * constants ([nest] rope.linnet), the head tying and the storage types. */
typedef struct {
  int32_t kv, g, half, f, layers, vocab;
  float eps, theta;
  int32_t llama3;
  float factor, low_freq_factor, high_freq_factor;
  float original_max_pos;
  int32_t tied;
  int32_t wdt, kvdt;
} ocfg;

/* LW: ln1, q, k, v, o, ln2, gate, up, down; row = output ([bend] "A layer", type LW) */
typedef struct {
  const void *ln1, *wq, *wk, *wv, *wo, *ln2, *wg, *wu, *wd;
} olayer;

typedef struct {
  const void *emb;     /* [vocab][dim] */
  const void *lm_head; /* [vocab][dim], NULL when tied (the LM head is the embedding) */
  const void *lnf;     /* [dim] */
  const olayer *layers;
} omodel;

static inline int o_head(const ocfg *c) { return 2 * c->half; }
static inline int o_heads(const ocfg *c) { return c->kv * c->g; }
static inline int o_dim(const ocfg *c) { return o_heads(c) * o_head(c); }
static inline int o_kvw(const ocfg *c) { return c->kv * o_head(c); }

/* bf16 -> F32: the bits become the upper half of an F32 (exact) */
static inline float o_get(const void *base, int dt, size_t i) {
  if (dt == ODT_F32) return ((const float *)base)[i];
  uint32_t u = (uint32_t)((const uint16_t *)base)[i] << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* F32 -> bf16, round to nearest even (NaN stays NaN) */
static inline uint16_t o_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static inline void o_put(void *base, int dt, size_t i, float v) {
  if (dt == ODT_F32)
    ((float *)base)[i] = v;
  else
    ((uint16_t *)base)[i] = o_bf16(v);
}

/* ---------------------------------------------------------------- numeric pieces ([bend]) ---- */

/* tree_sum: adjacent pairs added ([a,b,c,d,e] -> [a+b, c+d, e]) until one number is left */
float oracle_tree_sum(int n, const float *xs) {
  if (n <= 0) return 0.0f;
  float *buf = (float *)malloc(sizeof(float) * (size_t)n);
  memcpy(buf, xs, sizeof(float) * (size_t)n);
  int m = n;
  while (m > 1) {
    int k = 0;
    for (int i = 0; i + 1 < m; i += 2) buf[k++] = buf[i] + buf[i + 1];
    if (m & 1) buf[k++] = buf[m - 1];
    m = k;
  }
  float s = buf[0];
  free(buf);
  return s;
}

/* rmsnorm: g * (x * (1 / sqrt(tree_sum(x^2) / dim + eps))) */
void oracle_rmsnorm(int n, const float *x, const void *g, int gdt, float eps, float *out) {
  float *sq = (float *)malloc(sizeof(float) * (size_t)n);
  for (int i = 0; i < n; ++i) sq[i] = x[i] * x[i];
  float ms = oracle_tree_sum(n, sq) / (float)n;
  float r = 1.0f / sqrtf(ms + eps);
  for (int i = 0; i < n; ++i) out[i] = o_get(g, gdt, (size_t)i) * (x[i] * r);
  free(sq);
}

/* y = W x, W [rows][cols] row-major, each row's products summed left to right */
void oracle_matvec(int rows, int cols, const void *W, int wdt, const float *x, float *y) {
#pragma omp parallel for schedule(static)
  for (int r = 0; r < rows; ++r) {
    size_t base = (size_t)r * (size_t)cols;
    float acc = 0.0f;
    for (int c = 0; c < cols; ++c) acc = acc + o_get(W, wdt, base + (size_t)c) * x[c];
    y[r] = acc;
  }
}

/* silu(x) = x / (1 + exp(-x)) */
float oracle_silu(float x) { return x / (1.0f + expf(-x)); }

/* inv_freq[i] = 1 / theta^(2i / head), i < half; then, for llama3, the three-band rescale of
 * [nest] rope.linnet `tables` in its printed order: wavelength > original/low_freq_factor -> /factor;
 * wavelength < original/high_freq_factor -> unchanged; otherwise (1 - s) * inv/factor + s * inv with
 * s = (original / wavelength - low_freq_factor) / (high_freq_factor - low_freq_factor). */
void oracle_inv_freq(const ocfg *c, float *out) {
  const float hd = (float)o_head(c);
  const float PI = 3.14159265f;
  for (int i = 0; i < c->half; ++i) {
    float base = 1.0f / powf(c->theta, (float)(2 * i) / hd);
    if (!c->llama3) {
      out[i] = base;
      continue;
    }
    float wavelen = (2.0f * PI) / base;
    float low_wl = c->original_max_pos / c->low_freq_factor;
    float high_wl = c->original_max_pos / c->high_freq_factor;
    float smooth = (c->original_max_pos / wavelen - c->low_freq_factor) / (c->high_freq_factor - c->low_freq_factor);
    float smoothed = (1.0f - smooth) * (base / c->factor) + smooth * base;
    out[i] = (wavelen > low_wl) ? base / c->factor : ((wavelen < high_wl) ? base : smoothed);
  }
}

/* rot_at: cos and sin of t * inv_freq[i] (the angle rounded to F32 first) */
void oracle_rope_cs(const ocfg *c, int t, float *cs, float *sn) {
  float inv[1024];
  oracle_inv_freq(c, inv);
  for (int i = 0; i < c->half; ++i) {
    float a = (float)t * inv[i];
    cs[i] = cosf(a);
    sn[i] = sinf(a);
  }
}

/* rope of one head of 2*half: lo' = lo*c + (-hi)*s, hi' = hi*c + lo*s */
void oracle_rope_head(int half, const float *in, const float *cs, const float *sn, float *out) {
  for (int i = 0; i < half; ++i) {
    float lo = in[i], hi = in[half + i];
    float a = lo * cs[i];
    float b = (-hi) * sn[i];
    float d = hi * cs[i];
    float e = lo * sn[i];
    out[i] = a + b;
    out[half + i] = d + e;
  }
}

/* argmax: the first index of the largest value (strict >); (0, 0) for an empty list */
int oracle_argmax(int n, const float *xs, float *vmax) {
  if (n <= 0) {
    if (vmax) *vmax = 0.0f;
    return 0;
  }
  int bi = 0;
  float bv = xs[0];
  for (int i = 1; i < n; ++i)
    if (xs[i] > bv) {
      bv = xs[i];
      bi = i;
    }
  if (vmax) *vmax = bv;
  return bi;
}

/* ------------------------------------------------------- attention ([bend] head_att) ---- */

/* One query head over positions 0..t of its key/value head.  K, V point at that head's rows,
 * position p at [p*head, (p+1)*head).  scores = (K q) in order, scaled, softmax (max subtracted,
 * exp, running sum, divide), then out[d] = sum_p w_p * V[p][d], p ascending. */
void oracle_head_attention(int head, int t, float scale, const float *q, const void *K, const void *V, int kvdt,
                           float *out) {
  int n = t + 1;
  float *s = (float *)malloc(sizeof(float) * (size_t)n);
  for (int p = 0; p < n; ++p) {
    float acc = 0.0f;
    for (int d = 0; d < head; ++d) acc = acc + q[d] * o_get(K, kvdt, (size_t)p * head + d);
    s[p] = scale * acc;
  }
  float m = s[0];
  for (int p = 1; p < n; ++p) m = fmaxf(m, s[p]);
  float z = 0.0f;
  for (int p = 0; p < n; ++p) {
    s[p] = expf(s[p] - m);
    z = z + s[p];
  }
  for (int p = 0; p < n; ++p) s[p] = s[p] / z;
  for (int d = 0; d < head; ++d) {
    float acc = 0.0f;
    for (int p = 0; p < n; ++p) acc = acc + s[p] * o_get(V, kvdt, (size_t)p * head + d);
    out[d] = acc;
  }
  free(s);
}

/* ------------------------------------------------------------------ the model ---- */

/* Floats of one layer's trace: n1, q, k, v, qr, kr, attn, a, n2, m, y ([bend] type Act) */
int64_t oracle_trace_floats(const ocfg *c) {
  int64_t d = o_dim(c), kw = o_kvw(c);
  return 7 * d + 3 * kw + c->f;
}

/* cache layout: [layers][rows][kv][max_seq][head] */
static size_t o_slot(const ocfg *c, int rows, int max_seq, int l, int row, int j, int p) {
  return ((((size_t)l * rows + row) * c->kv + j) * (size_t)max_seq + p) * (size_t)o_head(c);
}

/*
 * One position of one cache row ([bend] forward / forward_pre with block; [nest] decode): token tok
 * at position pos (0-based), the row holding positions 0..pos-1.  Writes K (after RoPE) and V at pos
 * for every layer, returns the argmax of the logits (and fills logits) when logits != NULL, or -1 when
 * the final norm and LM head are skipped (a prompt position whose logits nobody reads).
 * Errors: -2 position outside [0, max_seq); -3 token outside [0, vocab).  Nothing is written then.
 * trace (nullable): per layer n1, q, k, v, qr, kr, attn, a, n2, m, y, each at full width.
 * hidden_out (nullable): the last layer's output before the final norm.
 */
int oracle_decode_row(const ocfg *c, const omodel *m, void *kc, void *vc, int rows, int max_seq, int row, int tok,
                      int pos, float *logits, float *trace, float *hidden_out) {
  if (pos < 0 || pos >= max_seq) return -2;
  if (tok < 0 || tok >= c->vocab) return -3;
  const int H = o_dim(c), KW = o_kvw(c), D = o_head(c), F = c->f, half = c->half;
  const int wdt = c->wdt, kvdt = c->kvdt;
  const float scale = 1.0f / sqrtf((float)D);
  float *x = (float *)malloc(sizeof(float) * H);
  float *n1 = (float *)malloc(sizeof(float) * H);
  float *q = (float *)malloc(sizeof(float) * H);
  float *k = (float *)malloc(sizeof(float) * KW);
  float *v = (float *)malloc(sizeof(float) * KW);
  float *qr = (float *)malloc(sizeof(float) * H);
  float *kr = (float *)malloc(sizeof(float) * KW);
  float *at = (float *)malloc(sizeof(float) * H);
  float *a = (float *)malloc(sizeof(float) * H);
  float *n2 = (float *)malloc(sizeof(float) * H);
  float *gt = (float *)malloc(sizeof(float) * F);
  float *up = (float *)malloc(sizeof(float) * F);
  float *mm = (float *)malloc(sizeof(float) * F);
  float *mo = (float *)malloc(sizeof(float) * H);
  float cs[1024], sn[1024];
  oracle_rope_cs(c, pos, cs, sn);

  for (int i = 0; i < H; ++i) x[i] = o_get(m->emb, wdt, (size_t)tok * H + i);

  for (int l = 0; l < c->layers; ++l) {
    const olayer *w = &m->layers[l];
    oracle_rmsnorm(H, x, w->ln1, wdt, c->eps, n1);
    oracle_matvec(H, H, w->wq, wdt, n1, q);
    oracle_matvec(KW, H, w->wk, wdt, n1, k);
    oracle_matvec(KW, H, w->wv, wdt, n1, v);
    for (int h = 0; h < o_heads(c); ++h) oracle_rope_head(half, q + h * D, cs, sn, qr + h * D);
    for (int j = 0; j < c->kv; ++j) oracle_rope_head(half, k + j * D, cs, sn, kr + j * D);
    /* KV.push: every kv head's rotated key and its value at position pos */
    for (int j = 0; j < c->kv; ++j) {
      size_t s = o_slot(c, rows, max_seq, l, row, j, pos);
      for (int d = 0; d < D; ++d) {
        o_put(kc, kvdt, s + d, kr[j * D + d]);
        o_put(vc, kvdt, s + d, v[j * D + d]);
      }
    }
    /* query head j*g + i reads key/value head j; outputs concatenated in query-head order */
#pragma omp parallel for schedule(static)
    for (int h = 0; h < o_heads(c); ++h) {
      int j = h / c->g;
      size_t s0 = o_slot(c, rows, max_seq, l, row, j, 0);
      size_t eb = (kvdt == ODT_F32) ? 4 : 2;
      oracle_head_attention(D, pos, scale, qr + h * D, (const char *)kc + s0 * eb, (const char *)vc + s0 * eb, kvdt,
                            at + h * D);
    }
    oracle_matvec(H, H, w->wo, wdt, at, a);
    float *x1 = x; /* x1 = x + a, in place */
    for (int i = 0; i < H; ++i) x1[i] = x[i] + a[i];
    oracle_rmsnorm(H, x1, w->ln2, wdt, c->eps, n2);
    oracle_matvec(F, H, w->wg, wdt, n2, gt);
    oracle_matvec(F, H, w->wu, wdt, n2, up);
    for (int i = 0; i < F; ++i) mm[i] = oracle_silu(gt[i]) * up[i];
    oracle_matvec(H, F, w->wd, wdt, mm, mo);
    for (int i = 0; i < H; ++i) x[i] = x1[i] + mo[i];
    if (trace) {
      float *tp = trace + (size_t)l * (size_t)oracle_trace_floats(c);
#define PUT(src, n)                              \
  do {                                           \
    memcpy(tp, src, sizeof(float) * (size_t)(n)); \
    tp += (n);                                   \
  } while (0)
      PUT(n1, H);
      PUT(q, H);
      PUT(k, KW);
      PUT(v, KW);
      PUT(qr, H);
      PUT(kr, KW);
      PUT(at, H);
      PUT(a, H);
      PUT(n2, H);
      PUT(mm, F);
      PUT(x, H);
#undef PUT
    }
  }
  if (hidden_out) memcpy(hidden_out, x, sizeof(float) * H);
  int result = -1;
  if (logits) {
    float *nf = n1;
    oracle_rmsnorm(H, x, m->lnf, wdt, c->eps, nf);
    const void *head_w = c->tied ? m->emb : m->lm_head;
    oracle_matvec(c->vocab, H, head_w, wdt, nf, logits);
    result = oracle_argmax(c->vocab, logits, NULL);
  }
  free(x); free(n1); free(q); free(k); free(v); free(qr); free(kr); free(at); free(a); free(n2);
  free(gt); free(up); free(mm); free(mo);
  return result;
}

/* Final norm + LM head + argmax of one hidden state ([bend] head_of + argmax). */
int oracle_lm_head(const ocfg *c, const omodel *m, const float *hidden, float *logits) {
  const int H = o_dim(c);
  float *nf = (float *)malloc(sizeof(float) * H);
  oracle_rmsnorm(H, hidden, m->lnf, c->wdt, c->eps, nf);
  oracle_matvec(c->vocab, H, c->tied ? m->emb : m->lm_head, c->wdt, nf, logits);
  free(nf);
  return oracle_argmax(c->vocab, logits, NULL);
}

/*
 * A prompt of S tokens at positions pos0..pos0+S-1 of one row, one position after another; only the
 * last position runs the final norm and LM head.  Returns its argmax, or an error (< -1) before any
 * write: -2 when pos0 < 0 or pos0 + S > max_seq, -3 for a token outside the vocabulary, -4 for S <= 0.
 */
int oracle_prefill_row(const ocfg *c, const omodel *m, void *kc, void *vc, int rows, int max_seq, int row,
                       const int32_t *toks, int S, int pos0, float *logits_last) {
  if (S <= 0) return -4;
  if (pos0 < 0 || (int64_t)pos0 + S > max_seq) return -2;
  for (int i = 0; i < S; ++i)
    if (toks[i] < 0 || toks[i] >= c->vocab) return -3;
  int r = -1;
  for (int i = 0; i < S; ++i)
    r = oracle_decode_row(c, m, kc, vc, rows, max_seq, row, toks[i], pos0 + i, (i == S - 1) ? logits_last : NULL,
                          NULL, NULL);
  return r;
}

/* F32 -> bf16 bits as the oracle rounds cache writes (exposed for tests) */
uint16_t oracle_bf16(float f) { return o_bf16(f); }

/* ------------------------------------------------------ sampling ([bend] "Sampling") ---- */
/*
 * Temperature, top-k and top-p with one uniform draw, every step an F32 operation in the order the
 * page gives.  Readings taken where the page leaves a step open: F32.exp is the correctly rounded
 * F32 exponential (here exp in double precision, rounded once to float); logits are finite, so the
 * IEEE comparisons the page uses never meet a NaN.
 */

/* lowbias32 (Chris Wellons, public domain): two xor-shift / odd-multiply rounds and a last xor-shift,
 * a bijection on 32-bit words ([bend] hash32). */
uint32_t oracle_hash32(uint32_t x) {
  x ^= x >> 16;
  x *= 2146121005u;
  x ^= x >> 15;
  x *= 2221713035u;
  x ^= x >> 16;
  return x;
}

/* draw n of a seed: the top 24 bits of hash32(hash32(seed) + n) scaled by 2^-24, exact in F32 and in
 * [0, 1) ([bend] uniform) */
float oracle_uniform(uint32_t seed, uint32_t n) {
  uint32_t h = oracle_hash32(oracle_hash32(seed) + n);
  return (float)(h >> 8) * 5.9604644775390625e-8f;
}

/* The k largest of xs[0..n), largest first, in one pass over xs ([bend] topk): a value enters while
 * fewer than k are held, or when it is strictly above the smallest held; it is placed after every held
 * value that is not smaller than it, so equal values keep id order (lower id first), and the list is
 * cut back to k.  Writes min(k, n) candidates and returns that count. */
int oracle_topk(int n, const float *xs, int k, int32_t *ids, float *vals) {
  int m = 0;
  if (k <= 0) return 0;
  for (int i = 0; i < n; ++i) {
    const float h = xs[i];
    if (!(m < k || h > vals[m - 1])) continue;
    int at = 0;
    while (at < m && !(vals[at] < h)) ++at; /* walk past the held values that are not smaller */
    int last = (m < k) ? m : k - 1;         /* the slot that receives the tail (the k-th drops off) */
    for (int j = last; j > at; --j) {
      vals[j] = vals[j - 1];
      ids[j] = ids[j - 1];
    }
    vals[at] = h;
    ids[at] = i;
    if (m < k) ++m;
  }
  return m;
}

/* exp(v/temp - top/temp): the weight of a candidate, 1 for the largest ([bend] weight) */
static float samp_weight(float v, float temp, float top) {
  const float a = v / temp;
  const float b = top / temp;
  const float d = a - b;
  return (float)exp((double)d);
}

/*
 * One draw ([bend] sample): top-k candidates; Z = their weights summed from 0 in candidate order;
 * lim = p * Z; the first candidate is always kept and each next one is kept while the running weight
 * before it is below lim ([bend] kept.go); z = the kept weight; target = u * z; the draw stops at the
 * first kept candidate whose running weight including itself is above target, or at the last kept one
 * ([bend] stops, pick.go).  Returns the drawn id (or -1 for n <= 0 or k <= 0) and, when the pointers
 * are not NULL, its logit, the kept count and the kept weight z.
 */
int oracle_sample(int n, const float *xs, float temp, int k, float p, float u, float *v_out, int32_t *n_kept,
                  float *z_out) {
  if (n <= 0 || k <= 0) return -1;
  const int kk = k < n ? k : n;
  int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * kk);
  float *vals = (float *)malloc(sizeof(float) * kk);
  const int m = oracle_topk(n, xs, k, ids, vals);
  const float top = vals[0];
  float Z = 0.0f;
  for (int j = 0; j < m; ++j) Z = Z + samp_weight(vals[j], temp, top);
  const float lim = p * Z;
  int kept = 0;
  float acc = 0.0f;
  for (int j = 0; j < m; ++j) {
    if (j > 0 && !(acc < lim)) break; /* the running weight before candidate j */
    acc = acc + samp_weight(vals[j], temp, top);
    ++kept;
  }
  const float z = acc;
  const float target = u * z;
  int pick = kept - 1;
  float run = 0.0f;
  for (int j = 0; j < kept - 1; ++j) {
    run = run + samp_weight(vals[j], temp, top);
    if (target < run) {
      pick = j;
      break;
    }
  }
  const int id = ids[pick];
  if (v_out) *v_out = vals[pick];
  if (n_kept) *n_kept = kept;
  if (z_out) *z_out = z;
  free(ids);
  free(vals);
  return id;
}
