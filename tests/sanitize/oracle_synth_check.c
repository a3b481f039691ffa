/*
 * Memory and undefined-behaviour check of the CPU oracle and the seeded input generator: this file
 * compiles both sources into one program with AddressSanitizer and UndefinedBehaviorSanitizer (see
 * tests/test_sanitize_cpu.py) and drives every entry point on tiny models, ragged spans and the error
 * paths.  Test infrastructure only; it is not part of the library.
 *
 * Besides running clean under the sanitizers it checks a few identities that hold bit for bit:
 * a prompt equals the same positions decoded one at a time (main.bend forward_pre against forward),
 * the standalone LM head equals the decode's own (main.bend head_of), and an error return writes
 * nothing (the room proof before KV.push).
 */
#include <stdio.h>
#include <stdlib.h>

#include "../../oracle/oracle.c"
#include "../../synth/synth.c"

static int fails = 0;
#define CHECK(cond, ...)                         \
  do {                                           \
    if (!(cond)) {                               \
      fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      fprintf(stderr, __VA_ARGS__);              \
      fprintf(stderr, "\n");                     \
      ++fails;                                   \
    }                                            \
  } while (0)

typedef struct {
  ocfg c;
  olayer *layers;
  omodel m;
  void *bufs[64];
  int nb;
} tmodel;

static void *tm_alloc(tmodel *t, size_t bytes) {
  void *p = malloc(bytes);
  t->bufs[t->nb++] = p;
  return p;
}

/* weights N(0, 0.02), gains 1 + N(0, 0.02), in the model's weight type, one seed per tensor */
static const void *tm_tensor(tmodel *t, uint32_t seed, size_t n, double mean) {
  if (t->c.wdt == ODT_F32) {
    float *p = (float *)tm_alloc(t, n * sizeof(float));
    synth_normal_f32(seed, 0, n, mean, 0.02, p);
    return p;
  }
  uint16_t *p = (uint16_t *)tm_alloc(t, n * sizeof(uint16_t));
  synth_normal_bf16(seed, 0, n, mean, 0.02, p);
  return p;
}

static void tm_init(tmodel *t, ocfg c) {
  memset(t, 0, sizeof(*t));
  t->c = c;
  const size_t H = o_dim(&c), KW = o_kvw(&c), F = c.f, V = c.vocab;
  t->layers = (olayer *)tm_alloc(t, sizeof(olayer) * c.layers);
  uint32_t s = 100;
  for (int l = 0; l < c.layers; ++l) {
    olayer *w = &t->layers[l];
    w->ln1 = tm_tensor(t, s++, H, 1.0);
    w->wq = tm_tensor(t, s++, H * H, 0.0);
    w->wk = tm_tensor(t, s++, KW * H, 0.0);
    w->wv = tm_tensor(t, s++, KW * H, 0.0);
    w->wo = tm_tensor(t, s++, H * H, 0.0);
    w->ln2 = tm_tensor(t, s++, H, 1.0);
    w->wg = tm_tensor(t, s++, F * H, 0.0);
    w->wu = tm_tensor(t, s++, F * H, 0.0);
    w->wd = tm_tensor(t, s++, H * F, 0.0);
  }
  t->m.emb = tm_tensor(t, s++, V * H, 0.0);
  t->m.lm_head = c.tied ? NULL : tm_tensor(t, s++, V * H, 0.0);
  t->m.lnf = tm_tensor(t, s++, H, 1.0);
  t->m.layers = t->layers;
}

static void tm_free(tmodel *t) {
  for (int i = 0; i < t->nb; ++i) free(t->bufs[i]);
}

static void check_model(ocfg c, const char *name) {
  tmodel t;
  tm_init(&t, c);
  const int rows = 2, max_seq = 12, S = 9, H = o_dim(&c);
  const size_t eb = c.kvdt == ODT_F32 ? 4 : 2;
  const size_t cache = (size_t)c.layers * rows * c.kv * max_seq * o_head(&c) * eb;
  void *k1 = calloc(cache, 1), *v1 = calloc(cache, 1), *k2 = calloc(cache, 1), *v2 = calloc(cache, 1);
  int32_t toks[9];
  synth_tokens(7, 3, S, (uint32_t)c.vocab, toks);
  float *lg1 = (float *)malloc(sizeof(float) * c.vocab), *lg2 = (float *)malloc(sizeof(float) * c.vocab);
  float *hid = (float *)malloc(sizeof(float) * H);
  float *tr = (float *)malloc(sizeof(float) * oracle_trace_floats(&c) * c.layers);
  int r1 = -1;
  for (int p = 0; p < S; ++p)
    r1 = oracle_decode_row(&c, &t.m, k1, v1, rows, max_seq, 1, toks[p], p, p == S - 1 ? lg1 : NULL, tr, hid);
  int r2 = oracle_prefill_row(&c, &t.m, k2, v2, rows, max_seq, 1, toks, S, 0, lg2);
  CHECK(r1 == r2 && r1 >= 0, "%s: prefill argmax %d vs decode %d", name, r2, r1);
  CHECK(memcmp(lg1, lg2, sizeof(float) * c.vocab) == 0, "%s: prefill logits differ from decode", name);
  CHECK(memcmp(k1, k2, cache) == 0 && memcmp(v1, v2, cache) == 0, "%s: prefill cache differs", name);
  int r3 = oracle_lm_head(&c, &t.m, hid, lg2);
  CHECK(r3 == r1 && memcmp(lg1, lg2, sizeof(float) * c.vocab) == 0, "%s: lm_head differs from decode", name);
  /* errors write nothing */
  CHECK(oracle_decode_row(&c, &t.m, k2, v2, rows, max_seq, 1, toks[0], max_seq, lg2, NULL, NULL) == -2, "%s", name);
  CHECK(oracle_decode_row(&c, &t.m, k2, v2, rows, max_seq, 1, toks[0], -1, lg2, NULL, NULL) == -2, "%s", name);
  CHECK(oracle_decode_row(&c, &t.m, k2, v2, rows, max_seq, 1, c.vocab, 0, lg2, NULL, NULL) == -3, "%s", name);
  CHECK(oracle_prefill_row(&c, &t.m, k2, v2, rows, max_seq, 1, toks, 0, 0, lg2) == -4, "%s", name);
  CHECK(oracle_prefill_row(&c, &t.m, k2, v2, rows, max_seq, 1, toks, S, max_seq - S + 1, lg2) == -2, "%s", name);
  CHECK(memcmp(k1, k2, cache) == 0 && memcmp(v1, v2, cache) == 0, "%s: an error wrote the cache", name);
  /* the last position of the cache, then row 0 untouched */
  CHECK(oracle_decode_row(&c, &t.m, k2, v2, rows, max_seq, 1, toks[1], max_seq - 1, lg2, NULL, NULL) >= 0, "%s",
        name);
  free(k1); free(v1); free(k2); free(v2); free(lg1); free(lg2); free(hid); free(tr);
  tm_free(&t);
}

static void check_pieces(void) {
  /* tree_sum on empty, one and odd lengths */
  float xs[7] = {1, 2, 3, 4, 5, 6, 7};
  CHECK(oracle_tree_sum(0, xs) == 0.0f, "tree_sum empty");
  CHECK(oracle_tree_sum(1, xs) == 1.0f, "tree_sum one");
  CHECK(oracle_tree_sum(7, xs) == 28.0f, "tree_sum seven");
  float v;
  CHECK(oracle_argmax(0, xs, &v) == 0 && v == 0.0f, "argmax empty");
  /* top-k and sampling: k above n, k = 1, equal values, p <= 0 and u at the edges */
  float lg[5] = {0.5f, 2.0f, 2.0f, -1.0f, 0.0f};
  int32_t ids[8];
  float vals[8];
  CHECK(oracle_topk(5, lg, 8, ids, vals) == 5 && ids[0] == 1 && ids[1] == 2, "topk ties keep id order");
  CHECK(oracle_topk(5, lg, 0, ids, vals) == 0, "topk k = 0");
  int32_t kept;
  float z, vo;
  CHECK(oracle_sample(5, lg, 0.7f, 8, 0.9f, 0.0f, &vo, &kept, &z) == 1, "sample u = 0");
  CHECK(oracle_sample(5, lg, 0.7f, 3, 0.0f, 0.99f, &vo, &kept, &z) == 1 && kept == 1, "sample p = 0");
  CHECK(oracle_sample(5, lg, 1.0f, 5, 1.0f, 0.9999999f, &vo, &kept, &z) >= 0, "sample u near 1");
  CHECK(oracle_sample(0, lg, 1.0f, 5, 1.0f, 0.5f, NULL, NULL, NULL) == -1, "sample empty");
  /* the generator over ragged spans: an odd start and length give the same values as the full span */
  float full[37], part[20];
  uint16_t fb[37], pb[20];
  synth_normal_f32(11, 0, 37, 0.0, 1.0, full);
  synth_normal_f32(11, 7, 20, 0.0, 1.0, part);
  synth_normal_bf16(11, 0, 37, 0.0, 1.0, fb);
  synth_normal_bf16(11, 7, 20, 0.0, 1.0, pb);
  CHECK(memcmp(full + 7, part, sizeof(part)) == 0 && memcmp(fb + 7, pb, sizeof(pb)) == 0, "normal spans");
  int32_t ir[50];
  synth_int_range(3, 5, 50, -4, 9, ir);
  for (int i = 0; i < 50; ++i) CHECK(ir[i] >= -4 && ir[i] <= 9, "int_range");
  float kf[33];
  uint16_t kb[33];
  synth_uniform_kv_f32(5, 1, 33, 1.0f / 8388608.0f, kf);
  synth_uniform_kv_bf16(5, 1, 33, 1.0f / 8388608.0f, kb);
  for (int i = 0; i < 33; ++i) CHECK(kf[i] >= -1.0f && kf[i] < 1.0f && kb[i] == o_bf16(kf[i]), "uniform kv");
  CHECK(synth_uniform(9, 4) == oracle_uniform(9, 4), "uniform draws agree");
}

int main(void) {
  /* kv, g, half, f, layers, vocab, eps, theta, llama3, factor, low, high, original, tied, wdt, kvdt */
  ocfg tiny = {2, 2, 4, 16, 2, 32, 1e-5f, 10000.0f, 0, 1, 1, 4, 8192, 1, ODT_F32, ODT_F32};
  ocfg tiny_bf16 = {2, 3, 8, 24, 2, 40, 1e-5f, 500000.0f, 1, 8.0f, 1.0f, 4.0f, 8192, 0, ODT_BF16, ODT_BF16};
  check_model(tiny, "tiny f32");
  check_model(tiny_bf16, "tiny bf16 llama3 untied");
  check_pieces();
  if (fails) {
    fprintf(stderr, "%d checks failed\n", fails);
    return 1;
  }
  printf("sanitized oracle and generator checks passed\n");
  return 0;
}
