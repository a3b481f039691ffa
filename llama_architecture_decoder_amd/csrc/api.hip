// Host side of the C ABI (include/llama_mi355x.h): argument checks, workspace layout, the rope
// cos/sin table, and the launch sequence of one decoder step.
//
// Step order (main.bend "A layer" block and "The model" forward; nest attention.linnet `decode`):
//   embed -> per layer [ rmsnorm+QKV GEMV -> RoPE+append+attention -> O GEMV + residual ->
//   rmsnorm+gate/up GEMV + SwiGLU -> down GEMV + residual ] -> rmsnorm + LM head GEMV + argmax.
// Every check that the host can make happens before the first launch, so an error leaves the caches
// and outputs untouched (main.bend's room proof before KV.push; needle's validation before use).
#include <math.h>
#include <stdint.h>

#include <cmath>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "common.h"

using namespace lm;

namespace {

constexpr uint32_t kWsMagic = 0x4c4d5357u;  // "LMSW"
// polls before an attention block of the q/k/v + attention launch stops waiting for its queries (each
// poll is a memory round trip of about a microsecond: ~0.1 s in all, against ~15 us for the product)
constexpr int kSpinLimit = 1 << 16;
// The O product runs inside the q/k/v + attention launch (F32 caches, one row) up to this many weight
// bytes.  Measured (us per step): SmolLM2-135M shape 633 -> 601, 360M 878 -> 858 (a launch boundary
// costs more than the in-launch wait for the attention outputs); the 1.7B shape's 16.8 MB gained
// nothing (290.4 vs 290.6 per 4-layer step: its weight stream competes with the attention's cache reads).
constexpr size_t kFuseOMaxBytes = 8u << 20;

// Caps on GEMV blocks per projection (blocks walk row groups with a grid stride).  Fewer blocks read
// the input vector fewer times (each block loads all of it); more blocks keep more loads in flight.
// Measured on MI355X at the 8B shape: the LM head is not monotonic in the cap (157 us at 384-416
// blocks, 170 at 512, 172-175 at 768-2048, 204 at 256; 1.05 GB); the gate/up product is fastest with
// one group per block (35.6 vs 35.9 us); the down product takes 19.5 us at 448-512 blocks, 19.7 at
// 768, 21-23 at 384, 576-1024.
// Batched rows: K slices are chosen for about rows_blocks blocks per product, rows_blocks_small up to
// rows_small rows.  Measured (8B shape, 4 layers): 32 rows of 8K..32K positions 2.352 ms per step at
// 256 against 2.368 at 512 (gate/up then takes one slice and no reduce launch, the other reduces read
// half the partials); the 256-request serving workload, mostly at 64 rows, 5776 tok/s at 256 against
// 5906 at 512.
struct Tun {
  int qkv = 1024, o = 512, gate_up = 4096, down = 512, lm = 384;
  int rows_blocks = 512, rows_blocks_small = 256, rows_small = 32;
};
const Tun &tun() {
  static const Tun t;
  return t;
}
// LM head blocks by the bytes of one row: the 8 KB rows of the 8B (bf16) and 1.7B (F32) shapes take
// tun().lm; shorter rows put fewer bytes in flight per block, so they take more blocks (measured, us per
// step: SmolLM2-360M's 3.75 KB rows 861 at 384 blocks, 852 at 768, 857 at 1536; SmolLM2-135M's 2.25 KB
// rows 600 at 384, 587 at 768, 584 at 1536, 581 at 2048)
int lm_grid_cap(int64_t row_bytes) { return row_bytes >= 8192 ? tun().lm : row_bytes >= 3072 ? 768 : kLmGridMax; }

struct Dims {
  int64_t head, heads, dim, kvw, f, vocab, layers, kv, g, half;
  int wb, kb;
};

Dims dims_of(const llama_cfg *c) {
  Dims d;
  d.kv = c->kv;
  d.g = c->g;
  d.half = c->half;
  d.head = 2 * (int64_t)c->half;
  d.heads = (int64_t)c->kv * c->g;
  d.dim = d.heads * d.head;
  d.kvw = (int64_t)c->kv * d.head;
  d.f = c->f;
  d.vocab = c->vocab;
  d.layers = c->layers;
  d.wb = c->weight_dtype == LLAMA_BF16 ? 2 : 4;
  d.kb = c->kv_dtype == LLAMA_BF16 ? 2 : 4;
  return d;
}

int check_cfg(const llama_cfg *c) {
  if (!c) return LLAMA_E_NULL;
  if (c->kv <= 0 || c->g <= 0 || c->half <= 0 || c->f <= 0 || c->layers <= 0 || c->vocab <= 0) return LLAMA_E_CONFIG;
  if (!(c->eps > 0.f) || !isfinite(c->eps) || !(c->theta > 0.f) || !isfinite(c->theta)) return LLAMA_E_CONFIG;
  if ((c->weight_dtype != LLAMA_F32 && c->weight_dtype != LLAMA_BF16) ||
      (c->kv_dtype != LLAMA_F32 && c->kv_dtype != LLAMA_BF16))
    return LLAMA_E_CONFIG;
  if (c->rope_llama3 != 0 && c->rope_llama3 != 1) return LLAMA_E_CONFIG;
  if (c->tied_lm_head != 0 && c->tied_lm_head != 1) return LLAMA_E_CONFIG;
  if (c->rope_llama3) {
    if (!(c->rope_factor > 0.f) || !(c->rope_low_freq_factor > 0.f) ||
        !(c->rope_high_freq_factor > c->rope_low_freq_factor) || c->rope_original_max_pos <= 0)
      return LLAMA_E_CONFIG;
  }
  const Dims d = dims_of(c);
  if (d.dim > (1 << 20) || d.f > (1 << 22) || d.layers > 4096 || d.vocab > (1 << 26)) return LLAMA_E_CONFIG;
  // shapes the kernels are instantiated for
  if (!attention_supported((int)d.head, c->g)) return LLAMA_E_UNSUPPORTED;
  if (d.dim % 8 || d.f % 8) return LLAMA_E_UNSUPPORTED;
  if (!gemv_supported(c->weight_dtype, (int)d.dim) || !gemv_supported(c->weight_dtype, (int)d.f))
    return LLAMA_E_UNSUPPORTED;
  return LLAMA_OK;
}

uint32_t cfg_key(const llama_cfg *c) {
  // FNV-1a over the fields (not the padding)
  uint32_t h = 0x811c9dc5u;
  auto mix = [&](const void *p, size_t n) {
    const unsigned char *b = (const unsigned char *)p;
    for (size_t i = 0; i < n; ++i) {
      h ^= b[i];
      h *= 0x01000193u;
    }
  };
  mix(&c->kv, 6 * sizeof(int32_t));
  mix(&c->eps, sizeof(float));
  mix(&c->theta, sizeof(float));
  mix(&c->rope_llama3, sizeof(int32_t));
  mix(&c->rope_factor, 3 * sizeof(float));
  mix(&c->rope_original_max_pos, sizeof(int32_t));
  mix(&c->tied_lm_head, 3 * sizeof(int32_t));
  return h;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct WsLayout {
  size_t status, done, epoch, tagged, group_done, att_t, rope_cs, rope_sn, x, x2, qkv, qrot, attn, m, part_o, part_ml, lm_v, lm_i, xhi, xlo, xhi2, xlo2, part,
      total;
  int nch;    // chunk slots per (row, kv head) of the attention partials
  int nch_f;  // chunk slots of the one-row launch that runs the q/k/v product with the attention
  int lm_ld;  // per-row stride of the LM head's block winners
  int mpad;   // token rows of the split operands (max_batch rounded up to 16)
};

// the matrix-core prefill: bf16 weights and cache, head 64 or 128, K of every product a multiple of 32
bool prefill_tiled_ok(const llama_cfg *c) {
  const int64_t dim = 2 * (int64_t)c->half * c->kv * c->g;
  return c->weight_dtype == LLAMA_BF16 && c->kv_dtype == LLAMA_BF16 && (c->half == 32 || c->half == 64) &&
         dim % 32 == 0 && c->f % 32 == 0;
}

// the matrix-core path for several decode rows: bf16 weights, K of every product a multiple of 128
bool rows_ok(const llama_cfg *c, int B) {
  const int dim = (int)(2 * (int64_t)c->half * c->kv * c->g);
  return B > 1 && gemm_rows_supported(c->weight_dtype, dim, B) && gemm_rows_supported(c->weight_dtype, c->f, B);
}

// K slices of each batched-rows product (q|k|v, o, gate/up, down)
struct RowsSlices {
  int qkv, o, gu, down;
};
RowsSlices rows_slices(const Dims &d, int rows) {
  const int H = (int)d.dim, KW = (int)d.kvw, F = (int)d.f;
  const int T = rows <= tun().rows_small ? tun().rows_blocks_small : tun().rows_blocks;
  return {gemm_rows_slices(H + 2 * KW, H, false, T), gemm_rows_slices(H, H, false, T),
          gemm_rows_slices(F, H, true, T), gemm_rows_slices(H, F, false, T)};
}

WsLayout ws_layout(const llama_cfg *c, int32_t max_batch, int32_t max_seq, int32_t max_prefill) {
  const Dims d = dims_of(c);
  // activation rows: a decode call's batch, or a prefill chunk when the matrix-core prefill runs
  const int32_t prows = prefill_tiled_ok(c) ? max_prefill : 0;
  const size_t rows = (size_t)(max_batch > prows ? max_batch : prows);
  WsLayout L;
  const int chunk = attention_chunk(c->kv_dtype, (int)d.head, (int)d.g);
  L.nch = (int)((max_seq + chunk - 1) / chunk);
  const int fchunk = qkv_attention_chunk(c->kv_dtype, (int)d.head, (int)d.g);
  L.nch_f = fchunk > 0 ? (int)((max_seq + fchunk - 1) / fchunk) : 0;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  L.status = take(64);
  // zeroed with the status word at init: chunk counters, the step counter and the tagged words
  L.done = take(sizeof(unsigned) * (size_t)max_batch * d.kv);
  L.epoch = take(sizeof(unsigned));
  L.tagged = take(sizeof(unsigned long long) * (size_t)(d.dim + 2 * d.kvw));
  L.group_done = take(sizeof(unsigned long long) * (size_t)(d.dim + 2 * d.kvw));  // at most a group per row
  L.att_t = take(sizeof(unsigned long long) * (size_t)d.dim);  // one row's attention outputs, tagged
  L.rope_cs = take(sizeof(float) * (size_t)max_seq * d.half);
  L.rope_sn = take(sizeof(float) * (size_t)max_seq * d.half);
  L.x = take(sizeof(float) * rows * d.dim);
  L.x2 = take(sizeof(float) * (size_t)d.dim);  // one row's residual stream after O (O in the fused launch)
  L.qkv = take(sizeof(float) * rows * (d.dim + 2 * d.kvw));
  L.qrot = take(sizeof(float) * (size_t)max_batch * d.dim);
  L.attn = take(sizeof(float) * rows * d.dim);
  // the F32 MLP activations of the GEMV path (decode rows one at a time, and the trace); the prefill's
  // gate/up product writes the down product's operands instead
  L.m = take(sizeof(float) * (size_t)max_batch * d.f);
  const size_t slots = std::max<size_t>((size_t)max_batch * L.nch, (size_t)L.nch_f);  // per kv head
  L.part_o = take(sizeof(float) * slots * d.kv * d.g * d.head);
  L.part_ml = take(sizeof(float) * slots * d.kv * d.g * 2);
  const bool rows_path = rows_ok(c, max_batch);
  L.lm_ld = kLmGridMax;
  if (rows_path && gemm_rows_blocks((int)d.vocab, false) > L.lm_ld) L.lm_ld = gemm_rows_blocks((int)d.vocab, false);
  L.lm_v = take(sizeof(float) * (size_t)max_batch * L.lm_ld);
  L.lm_i = take(sizeof(int) * (size_t)max_batch * L.lm_ld);
  L.mpad = rows_path ? (max_batch + 15) / 16 * 16 : 0;
  if (prows > 0 && gemm_tiled_rows(prows) > L.mpad) L.mpad = gemm_tiled_rows(prows);
  const int64_t kmax = d.dim > d.f ? d.dim : d.f;
  L.xhi = take(sizeof(uint16_t) * (size_t)L.mpad * kmax);
  L.xlo = take(sizeof(uint16_t) * (size_t)L.mpad * kmax);
  // batched rows: a second operand pair (the MLP's inner activations) and the K-slice partial sums
  // (and, for the matrix-core prefill, the down product's operands written by the gate/up product)
  const int64_t mrows = std::max<int64_t>(rows_path ? (max_batch + 15) / 16 * 16 : 0,
                                          prows > 0 ? gemm_tiled_rows(prows) : 0);
  L.xhi2 = take(sizeof(uint16_t) * (size_t)mrows * d.f);
  L.xlo2 = take(sizeof(uint16_t) * (size_t)mrows * d.f);
  size_t part = 0;
  if (rows_path) {
    auto need = [&](int slices, int64_t nout, int rows) {
      const size_t n = (size_t)slices * (size_t)rows * (size_t)nout;
      part = n > part ? n : part;
    };
    // every row count up to max_batch: the slices of the smaller counts' target, then of the larger
    for (int rows : {std::min<int>(max_batch, tun().rows_small), (int)max_batch}) {
      const RowsSlices S = rows_slices(d, rows);
      need(S.qkv, d.dim + 2 * d.kvw, rows);
      need(S.o, d.dim, rows);
      need(S.gu, 2 * d.f, rows);
      need(S.down, d.dim, rows);
    }
  }
  // the matrix-core prefill's K-slice partial sums (short prompts), for every chunk size up to prows
  for (int32_t m = 128; prows >= 2 && m < prows + 128; m += 128) {
    const int M = m < prows ? m : prows;
    const int H = (int)d.dim, KW = (int)d.kvw, F = (int)d.f;
    const size_t n[4] = {gemm_tiled_part_floats(M, H + 2 * KW, H, false), gemm_tiled_part_floats(M, H, H, false),
                         gemm_tiled_part_floats(M, F, H, true), gemm_tiled_part_floats(M, H, F, false)};
    for (size_t v : n) part = v > part ? v : part;
  }
  L.part = take(sizeof(float) * part);
  L.total = o;
  return L;
}

// inv_freq[i] = 1 / theta^(2i / head) (main.bend inv_freq), then the llama3 band rescale in the order
// nest rope.linnet `tables` prints it.  Plain F32 host arithmetic, no contraction.
void host_inv_freq(const llama_cfg *c, float *inv) {
#pragma clang fp contract(off)
  const float hd = (float)(2 * c->half);
  const float PI = 3.14159265f;
  const float orig = (float)c->rope_original_max_pos;
  for (int i = 0; i < c->half; ++i) {
    const float base = 1.0f / powf(c->theta, (float)(2 * i) / hd);
    if (!c->rope_llama3) {
      inv[i] = base;
      continue;
    }
    const float wavelen = (2.0f * PI) / base;
    const float low_wl = orig / c->rope_low_freq_factor;
    const float high_wl = orig / c->rope_high_freq_factor;
    const float smooth = (orig / wavelen - c->rope_low_freq_factor) / (c->rope_high_freq_factor - c->rope_low_freq_factor);
    const float scaled = base / c->rope_factor;
    const float t1 = (1.0f - smooth) * scaled;
    const float t2 = smooth * base;
    const float blended = t1 + t2;
    inv[i] = (wavelen > low_wl) ? scaled : ((wavelen < high_wl) ? base : blended);
  }
}

int hip_rc(hipError_t e) { return e == hipSuccess ? LLAMA_OK : LLAMA_E_HIP; }

// Opt-in kernel timing (llama_profile_enable): HIP events recorded on the caller's stream around
// every launch of a step, grouped by kernel class, read back by llama_profile_read.
struct Prof {
  bool on = false;
  std::vector<hipEvent_t> pool;
  size_t used = 0;
  std::vector<std::pair<int, std::pair<hipEvent_t, hipEvent_t>>> marks;
  hipEvent_t get() {
    if (used == pool.size()) {
      hipEvent_t e;
      if (hipEventCreate(&e) != hipSuccess) return nullptr;
      pool.push_back(e);
    }
    return pool[used++];
  }
};
Prof &prof() {
  static Prof p;
  return p;
}
struct ProfScope {
  // events handed to the launches of this scope (recorded by their dispatch packets); if no launch
  // used them, they are recorded on the stream around the scope instead
  int cls;
  hipStream_t s;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  ProfScope(int c, hipStream_t st) : cls(c), s(st) {
    if (!prof().on) return;
    e0 = prof().get();
    e1 = prof().get();
    if (!e0 || !e1) {
      e0 = e1 = nullptr;
      return;
    }
    LaunchEvents &ev = launch_events();
    ev.start = e0;
    ev.stop = e1;
    ev.used = false;
  }
  ~ProfScope() {
    if (!e0) return;
    LaunchEvents &ev = launch_events();
    const bool used = ev.used, stop_used = ev.stop_used;
    ev = LaunchEvents();
    if (!used) return;  // nothing was launched (an error path): drop the pair
    // a scope whose launches took only the start event (an operand split whose product belongs to the
    // next scope) ends where its work ends on the stream
    if (!stop_used && hipEventRecord(e1, s) != hipSuccess) return;
    prof().marks.push_back({cls, {e0, e1}});
  }
};

int check_ws(const llama_cfg *c, const llama_ws *ws) {
  if (!ws || !ws->base) return LLAMA_E_NULL;
  if (ws->magic != kWsMagic || ws->cfg_key != cfg_key(c)) return LLAMA_E_WORKSPACE;
  if (ws->max_batch <= 0 || ws->max_seq <= 0 || ws->max_prefill < 0) return LLAMA_E_WORKSPACE;
  if (ws_layout(c, ws->max_batch, ws->max_seq, ws->max_prefill).total > ws->bytes) return LLAMA_E_WORKSPACE;
  return LLAMA_OK;
}

int check_weights(const llama_cfg *c, const llama_weights *w) {
  if (!w || !w->emb || !w->final_norm || !w->layers) return LLAMA_E_NULL;
  if (!c->tied_lm_head && !w->lm_head) return LLAMA_E_NULL;
  for (int l = 0; l < c->layers; ++l) {
    const llama_layer_w &L = w->layers[l];
    if (!L.ln1 || !L.wq || !L.wk || !L.wv || !L.wo || !L.ln2 || !L.w_gate || !L.w_up || !L.w_down) return LLAMA_E_NULL;
    const void *ps[] = {L.ln1, L.wq, L.wk, L.wv, L.wo, L.ln2, L.w_gate, L.w_up, L.w_down};
    for (const void *p : ps)
      if (((uintptr_t)p) & 15u) return LLAMA_E_SHAPE;
  }
  if (((uintptr_t)w->emb & 15u) || ((uintptr_t)w->final_norm & 15u)) return LLAMA_E_SHAPE;
  if (w->lm_head && ((uintptr_t)w->lm_head & 15u)) return LLAMA_E_SHAPE;
  return LLAMA_OK;
}

int check_kv(const llama_cfg *c, const llama_kv *kv) {
  if (!kv || !kv->k || !kv->v) return LLAMA_E_NULL;
  const Dims d = dims_of(c);
  if (kv->layers != c->layers || kv->kv != c->kv || kv->head != d.head || kv->dtype != c->kv_dtype ||
      kv->rows <= 0 || kv->max_seq <= 0)
    return LLAMA_E_SHAPE;
  return LLAMA_OK;
}

struct Ctx {
  const llama_cfg *c;
  Dims d;
  const llama_weights *w;
  const llama_kv *kv;
  const llama_ws *ws;
  WsLayout L;
  hipStream_t s;
  char *base;
  // paged cache (decode: table [B][pages]; prefill: one row's table [pages]); row 0 of kv is the pool
  const int32_t *table = nullptr;
  int pages = 0, npages = 0;
  template <typename T>
  T *at(size_t off) const {
    return reinterpret_cast<T *>(base + off);
  }
};

void *layer_cache(const Ctx &x, void *cache, int l) {
  const size_t per_layer = (size_t)x.kv->rows * x.d.kv * (size_t)x.kv->max_seq * x.d.head * x.d.kb;
  return (char *)cache + per_layer * (size_t)l;
}

// LM head of batch entry b: logits (nullable) and next (nullable) from hidden h
int run_lm_head(const Ctx &x, const float *h, int b, float *logits, int32_t *next) {
  GemvArgs a = {};
  a.x = h;
  a.gain = x.w->final_norm;
  a.eps = x.c->eps;
  a.w[0] = x.c->tied_lm_head ? x.w->emb : x.w->lm_head;
  a.rs[0] = 0;
  a.rs[1] = a.rs[2] = a.rs[3] = (int)x.d.vocab;
  a.N = (int)x.d.vocab;
  a.K = (int)x.d.dim;
  a.y = logits;
  a.part_v = x.at<float>(x.L.lm_v) + (size_t)b * kLmGridMax;
  a.part_i = x.at<int>(x.L.lm_i) + (size_t)b * kLmGridMax;
  a.next = next;
  ProfScope ps(LLAMA_K_LM_HEAD, x.s);
  return hip_rc(launch_gemv(x.c->weight_dtype, EPI_ARGMAX, true, a, lm_grid_cap(x.d.dim * x.d.wb), x.s));
}

// Several token rows with bf16 weights: each projection is one matrix-core product over all rows (the
// weights stream once per step instead of once per row), on bf16 hi/lo operands.  The operands of the
// next product are formed where the previous one is finished: the residual + RMSNorm + split after o and
// down (k_rows_reduce_norm), the SwiGLU output straight from the gate/up product.
int run_step_rows(const Ctx &x, AttnArgs aa, RopeAppend ra, int tmax, int B, float *logits, int32_t *next,
                  bool want_head) {
  const Dims &d = x.d;
  const int H = (int)d.dim, KW = (int)d.kvw, F = (int)d.f, V = (int)d.vocab;
  const int mpad = (B + 15) / 16 * 16;
  float *xs = x.at<float>(x.L.x);
  float *qkv = x.at<float>(x.L.qkv);
  float *att = x.at<float>(x.L.attn);
  bf16_t *ahi = x.at<bf16_t>(x.L.xhi), *alo = x.at<bf16_t>(x.L.xlo);    // operands with K = dim
  bf16_t *bhi = x.at<bf16_t>(x.L.xhi2), *blo = x.at<bf16_t>(x.L.xlo2);  // operands with K = f
  float *part = x.at<float>(x.L.part);
  const int wdt = x.c->weight_dtype;
  const int qkv_stride = H + 2 * KW;
  const RowsSlices S = rows_slices(d, B);
  auto split = [&](const float *in, const void *gain) {
    SplitArgs sa = {};
    sa.x = in;
    sa.ldin = H;
    sa.gain = gain;
    sa.eps = x.c->eps;
    sa.K = H;
    sa.M = B;
    sa.xhi = ahi;
    sa.xlo = alo;
    sa.ldx = H;
    return hip_rc(launch_split(wdt, gain != nullptr, sa, mpad, x.s));
  };
  auto gemm = [&](GemvEpi epi, bool wide_in, const void *w0, const void *w1, const void *w2, int r1, int r2, int N,
                  int slices, float *y, int ldy, bool first, bool last) {
    GemmArgs ga = {};
    ga.xhi = wide_in ? bhi : ahi;
    ga.xlo = wide_in ? blo : alo;
    ga.K = wide_in ? F : H;
    ga.ldx = ga.K;
    ga.w[0] = w0;
    ga.w[1] = w1;
    ga.w[2] = w2;
    ga.rs[0] = 0;
    ga.rs[1] = r1;
    ga.rs[2] = r2;
    ga.rs[3] = N;
    ga.N = N;
    ga.M = B;
    ga.y = y;
    ga.ldy = ldy;
    ga.part = part;
    ga.ohi = bhi;
    ga.olo = blo;
    ga.ldo = F;
    ga.part_v = x.at<float>(x.L.lm_v);
    ga.part_i = x.at<int>(x.L.lm_i);
    ga.part_ld = x.L.lm_ld;
    if (epi == EPI_ROPE) ga.ra = ra;
    return hip_rc(launch_gemm_rows(epi, ga, slices, x.s, first, last));
  };
  auto reduce_norm = [&](int slices, const void *gain) {
    RowsNormArgs na = {};
    na.part = part;
    na.S = slices;
    na.M = B;
    na.N = H;
    na.x = xs;
    na.ldx = H;
    na.gain = gain;
    na.eps = x.c->eps;
    na.xhi = ahi;
    na.xlo = alo;
    na.ldo = H;
    return hip_rc(launch_rows_reduce_norm(wdt, na, x.s, true));
  };
  aa.ohi = ahi;
  aa.olo = alo;
  aa.ldo = H;
  int rc;
  {
    ProfScope ps(LLAMA_K_QKV, x.s);
    // layer 0's operands (also the zero rows that pad the batch to a 16-row tile; nothing writes those
    // rows afterwards); later layers' come from down
    if ((rc = split(xs, x.w->layers[0].ln1))) return rc;
  }
  for (int l = 0; l < (int)d.layers; ++l) {
    const llama_layer_w &lw = x.w->layers[l];
    aa.kc = ra.kc = layer_cache(x, x.kv->k, l);
    aa.vc = ra.vc = layer_cache(x, x.kv->v, l);
    {
      ProfScope ps(LLAMA_K_QKV, x.s);
      if ((rc = gemm(EPI_ROPE, false, lw.wq, lw.wk, lw.wv, H, H + KW, H + 2 * KW, S.qkv, qkv, qkv_stride, true, true)))
        return rc;
    }
    {
      ProfScope ps(LLAMA_K_ATTN, x.s);
      if ((rc = hip_rc(launch_attention(x.c->kv_dtype, (int)d.head, (int)d.g, aa, B, tmax, x.s)))) return rc;
    }
    {
      ProfScope ps(LLAMA_K_O, x.s);
      // the attention's outputs arrive as the O product's operands (aa.ohi / aa.olo)
      if ((rc = gemm(EPI_RESID, false, lw.wo, lw.wo, lw.wo, H, H, H, S.o, nullptr, H, true, false))) return rc;
      if ((rc = reduce_norm(S.o, lw.ln2))) return rc;
    }
    {
      ProfScope ps(LLAMA_K_GATE_UP, x.s);
      if ((rc = gemm(EPI_SWIGLU, false, lw.w_gate, lw.w_up, lw.w_up, F, F, F, S.gu, nullptr, F, true, true))) return rc;
    }
    {
      ProfScope ps(LLAMA_K_DOWN, x.s);
      const void *next_gain = l + 1 < (int)d.layers ? x.w->layers[l + 1].ln1 : x.w->final_norm;
      if ((rc = gemm(EPI_RESID, true, lw.w_down, lw.w_down, lw.w_down, H, H, H, S.down, nullptr, H, true, false)))
        return rc;
      if ((rc = reduce_norm(S.down, next_gain))) return rc;
    }
  }
  if (!want_head || (!logits && !next)) return LLAMA_OK;
  // the operands hold rmsnorm(x, final norm) (the last down's reduce)
  ProfScope ps(LLAMA_K_LM_HEAD, x.s);
  const void *wl = x.c->tied_lm_head ? x.w->emb : x.w->lm_head;
  if ((rc = gemm(EPI_ARGMAX, false, wl, wl, wl, V, V, V, 1, logits, V, true, next == nullptr))) return rc;
  if (next)
    return hip_rc(launch_argmax_final(x.at<float>(x.L.lm_v), x.at<int>(x.L.lm_i), gemm_rows_blocks(V, false),
                                      x.L.lm_ld, B, next, x.s));
  return LLAMA_OK;
}

// The matrix-core prefill's products whose activations go in as bf16 hi + lo (bit set: the F32 values to
// ~2^-17) rather than as bf16 (the hi half alone, half the matrix-core work)
enum { kProdQkv = 0, kProdO = 1, kProdGateUp = 2, kProdDown = 3 };
constexpr unsigned kPrefillLo = 0xFu;

// One piece of a packed pass: len consecutive positions pos0 .. of cache row `row` (paged: of table row
// `row`); out >= 0 asks for the logits / next token after its last position at entry `out`.
struct PackSeg {
  int row, pos0, len, out;
};

// One pass over S packed positions (S <= the workspace's max_prefill), nseg pieces end to end in `tokens`:
// matrix-core products over the S rows, RoPE + append of every position into its own request's cache,
// causal attention of each piece over its request's positions.  The LM head runs on the last position of
// each piece that asks for it.
int run_prefill_pass(const Ctx &x, const int32_t *tokens, const PackSeg *segs, int nseg, float *logits,
                     int32_t *next) {
  const Dims &d = x.d;
  if (nseg < 1 || nseg > kMaxSegments) return LLAMA_E_SHAPE;
  int S = 0;
  for (int i = 0; i < nseg; ++i) S += segs[i].len;
  const int H = (int)d.dim, KW = (int)d.kvw, F = (int)d.f;
  const int mpad = gemm_tiled_rows(S);
  float *xs = x.at<float>(x.L.x);
  float *qkv = x.at<float>(x.L.qkv);
  float *att = x.at<float>(x.L.attn);
  bf16_t *xhi = x.at<bf16_t>(x.L.xhi), *xlo = x.at<bf16_t>(x.L.xlo);
  bf16_t *mhi = x.at<bf16_t>(x.L.xhi2), *mlo = x.at<bf16_t>(x.L.xlo2);  // the down product's operands
  const int wdt = x.c->weight_dtype;
  const int qkv_stride = H + 2 * KW;
  int rc;
  {
    ProfScope ps(LLAMA_K_EMBED, x.s);
    rc = hip_rc(launch_embed(wdt, tokens, x.w->emb, H, (int)d.vocab, xs, S, x.at<int>(x.L.status), nullptr, x.s));
  }
  if (rc) return rc;
  auto split = [&](const float *in, const void *gain, int K) {
    SplitArgs sa = {};
    sa.x = in;
    sa.ldin = K;
    sa.gain = gain;
    sa.eps = x.c->eps;
    sa.K = K;
    sa.M = S;
    sa.xhi = xhi;
    sa.xlo = xlo;
    sa.ldx = K;
    return hip_rc(launch_split(wdt, gain != nullptr, sa, mpad, x.s));
  };
  // nn: for a residual product, the next product's RMSNorm gain (the reduce of a K-sliced product then
  // writes that product's operands itself; nn->done says so)
  auto gemm = [&](GemvEpi epi, const void *w0, const void *w1, const void *w2, int r1, int r2, int N, int K, float *y,
                  int ldy, const float *res, bool mlp_in, int product, bool first, NormNext *nn = nullptr,
                  int *defer_ks = nullptr) {
    GemmArgs ga = {};
    ga.lo = (kPrefillLo >> product) & 1;
    ga.xhi = mlp_in ? mhi : xhi;  // the down product reads the operands the gate/up product wrote
    ga.xlo = mlp_in ? mlo : xlo;
    if (epi == EPI_SWIGLU) {
      ga.ohi = mhi;
      ga.olo = mlo;
      ga.ldo = F;
    }
    ga.ldx = K;
    ga.w[0] = w0;
    ga.w[1] = w1;
    ga.w[2] = w2;
    ga.rs[0] = 0;
    ga.rs[1] = r1;
    ga.rs[2] = r2;
    ga.rs[3] = N;
    ga.N = N;
    ga.K = K;
    ga.M = S;
    ga.y = y;
    ga.ldy = ldy;
    ga.res = res;
    ga.ldres = ldy;
    ga.part = x.at<float>(x.L.part);  // short chunks split K (sized for every chunk up to max_prefill)
    // `first`: no operand split before it in its timing scope (the down product, or a product whose operands
    // the previous reduce wrote)
    return hip_rc(launch_gemm_tiled(epi, ga, x.s, true, first, nn, defer_ks));
  };
  auto norm_next = [&](const void *gain) {
    NormNext nn = {};
    nn.gain = gain;
    nn.gdtype = wdt;
    nn.eps = x.c->eps;
    nn.xhi = xhi;
    nn.xlo = xlo;
    nn.ldo = H;
    return nn;
  };
  bool x_split = false;  // the operands of rmsnorm(x, ln1) of the next layer are already written
  PrefillArgs pa = {};
  pa.qkv = qkv;
  pa.qkv_stride = qkv_stride;
  pa.kv = (int)d.kv;
  pa.g = (int)d.g;
  pa.heads = (int)(d.kv * d.g);
  pa.half = (int)d.half;
  pa.max_seq = x.kv->max_seq;
  pa.table = x.table;
  pa.pages = x.pages;
  pa.npages = x.npages;
  pa.status = x.at<int>(x.L.status);
  pa.S = S;
  pa.nseg = nseg;
  pa.seg_start[0] = 0;
  pa.seg_tile[0] = 0;
  for (int i = 0; i < nseg; ++i) {
    pa.seg_start[i + 1] = pa.seg_start[i] + segs[i].len;
    pa.seg_tile[i + 1] = pa.seg_tile[i] + (segs[i].len + kPrefillQT - 1) / kPrefillQT;
    pa.seg_pos0[i] = segs[i].pos0;
    pa.seg_row[i] = segs[i].row;
  }
  pa.rope_cs = x.at<float>(x.L.rope_cs);
  pa.rope_sn = x.at<float>(x.L.rope_sn);
  pa.out = att;
  pa.out_stride = H;
  pa.scale = 1.0f / sqrtf((float)d.head);
  for (int l = 0; l < (int)d.layers; ++l) {
    const llama_layer_w &lw = x.w->layers[l];
    {
      ProfScope ps(LLAMA_K_QKV, x.s);
      if (!x_split && (rc = split(xs, lw.ln1, H))) return rc;
      // in K slices: the RoPE + append launch adds the partial sums itself (no reduce launch)
      if ((rc = gemm(EPI_STORE, lw.wq, lw.wk, lw.wv, H, H + KW, H + 2 * KW, H, qkv, qkv_stride, nullptr, false,
                     kProdQkv, x_split, nullptr, &pa.ks)))
        return rc;
      pa.part = pa.ks > 1 ? x.at<float>(x.L.part) : nullptr;
    }
    pa.kc = reinterpret_cast<bf16_t *>(layer_cache(x, x.kv->k, l));
    pa.vc = reinterpret_cast<bf16_t *>(layer_cache(x, x.kv->v, l));
    {
      ProfScope ps(LLAMA_K_ATTN, x.s);
      if ((rc = hip_rc(launch_rope_rows(pa, x.s, true, false)))) return rc;
      if ((rc = hip_rc(launch_attn_prefill(pa, x.s, false, true)))) return rc;
    }
    {
      ProfScope ps(LLAMA_K_O, x.s);
      if ((rc = split(att, nullptr, H))) return rc;
      NormNext nn = norm_next(lw.ln2);
      if ((rc = gemm(EPI_RESID, lw.wo, lw.wo, lw.wo, H, H, H, H, xs, H, xs, false, kProdO, false, &nn))) return rc;
      x_split = nn.done;
    }
    {
      ProfScope ps(LLAMA_K_GATE_UP, x.s);
      if (!x_split && (rc = split(xs, lw.ln2, H))) return rc;
      // silu(gate) * up goes straight to the down product's operands (mhi / mlo), never to F32
      if ((rc = gemm(EPI_SWIGLU, lw.w_gate, lw.w_up, lw.w_up, F, F, F, H, nullptr, F, nullptr, false, kProdGateUp,
                     x_split)))
        return rc;
    }
    {
      ProfScope ps(LLAMA_K_DOWN, x.s);
      NormNext nn = norm_next(l + 1 < (int)d.layers ? x.w->layers[l + 1].ln1 : nullptr);
      if ((rc = gemm(EPI_RESID, lw.w_down, lw.w_down, lw.w_down, H, H, H, F, xs, H, xs, true, kProdDown, true,
                     l + 1 < (int)d.layers ? &nn : nullptr)))
        return rc;
      x_split = l + 1 < (int)d.layers && nn.done;
    }
  }
  if (!logits && !next) return LLAMA_OK;
  // one LM head per finished piece; they share the argmax partials, in stream order
  for (int i = 0; i < nseg; ++i) {
    const int o = segs[i].out;
    if (o < 0) continue;
    rc = run_lm_head(x, xs + (size_t)(pa.seg_start[i + 1] - 1) * H, 0,
                     logits ? logits + (size_t)o * d.vocab : nullptr, next ? next + o : nullptr);
    if (rc) return rc;
  }
  return LLAMA_OK;
}

// One step for B rows at positions pos[b] of cache rows row0 + b.  want_head = run the LM head.
int run_step(const Ctx &x, const int32_t *tokens, const int32_t *pos, int B, int row0, float *logits, int32_t *next,
             bool want_head, float *trace) {
  const Dims &d = x.d;
  const int H = (int)d.dim, KW = (int)d.kvw, F = (int)d.f;
  const int wdt = x.c->weight_dtype;
  float *xs = x.at<float>(x.L.x);
  float *qkv = x.at<float>(x.L.qkv);
  float *att = x.at<float>(x.L.attn);
  float *mm = x.at<float>(x.L.m);
  const int qkv_stride = H + 2 * KW;
  int rc;
  {
    ProfScope ps(LLAMA_K_EMBED, x.s);
    rc = hip_rc(launch_embed(wdt, tokens, x.w->emb, H, (int)d.vocab, xs, B, x.at<int>(x.L.status),
                             x.at<unsigned>(x.L.epoch), x.s));
  }
  if (rc) return rc;

  // attention: one block per (chunk of positions, kv head, row)
  int tmax = 0;
  for (int b = 0; b < B; ++b) tmax = pos[b] > tmax ? pos[b] : tmax;

  AttnArgs aa = {};
  aa.q = x.at<float>(x.L.qrot);
  aa.kv = (int)d.kv;
  aa.max_seq = x.kv->max_seq;
  aa.half = (int)d.half;
  aa.row0 = row0;
  aa.table = x.table;
  aa.pages = x.pages;
  aa.npages = x.npages;
  aa.status = x.at<int>(x.L.status);
  aa.out = att;
  aa.out_stride = H;
  aa.part_o = x.at<float>(x.L.part_o);
  aa.part_ml = x.at<float>(x.L.part_ml);
  aa.done = x.at<unsigned>(x.L.done);
  aa.nch = x.L.nch;
  aa.scale = 1.0f / sqrtf((float)d.head);
  for (int b = 0; b < B; ++b) aa.pos[b] = pos[b];

  // the q|k|v epilogue: RoPE and the cache append at each row's position
  RopeAppend ra = {};
  ra.qrot = x.at<float>(x.L.qrot);
  ra.kv_bf16 = x.c->kv_dtype == LLAMA_BF16;
  ra.max_seq = x.kv->max_seq;
  ra.half = (int)d.half;
  ra.hshift = d.half == 64 ? 6 : 5;
  ra.dim = H;
  ra.kvw = KW;
  ra.row0 = row0;
  ra.table = x.table;
  ra.pages = x.pages;
  ra.npages = x.npages;
  ra.status = x.at<int>(x.L.status);
  ra.rope_cs = x.at<float>(x.L.rope_cs);
  ra.rope_sn = x.at<float>(x.L.rope_sn);
  for (int b = 0; b < B; ++b) ra.pos[b] = pos[b];

  if (rows_ok(x.c, B) && !trace)
    return run_step_rows(x, aa, ra, tmax, B, logits, next, want_head);

  const int64_t tstride = 4 * d.dim + 2 * d.kvw + d.f;
  // one token row (contiguous cache, no trace): the q/k/v product and the attention in one launch, and
  // with F32 caches the O product too (its output goes to the second residual buffer x2, read by the
  // gate/up product and the down product's residual, so no block of the launch writes what another reads)
  bool fused = B == 1 && !trace && !x.table && x.L.nch_f > 0;
  const bool fuse_o = fused && qkv_attention_fuses_o(x.c->kv_dtype) && (size_t)H * H * d.wb <= kFuseOMaxBytes;
  float *x2 = x.at<float>(x.L.x2);
  for (int l = 0; l < (int)d.layers; ++l) {
    const llama_layer_w &lw = x.w->layers[l];
    aa.kc = ra.kc = layer_cache(x, x.kv->k, l);
    aa.vc = ra.vc = layer_cache(x, x.kv->v, l);
    auto qkv_args = [&](int b) {
      GemvArgs a = {};
      a.ra = ra;
      a.ra.qrot = ra.qrot + (size_t)b * H;
      a.ra.row0 = row0 + b;
      if (x.table) a.ra.table = x.table + (size_t)b * x.pages;  // the GEMV's one token row is row b
      a.ra.pos[0] = pos[b];
      a.x = xs + (size_t)b * H;
      a.gain = lw.ln1;
      a.eps = x.c->eps;
      a.w[0] = lw.wq;
      a.w[1] = lw.wk;
      a.w[2] = lw.wv;
      a.rs[0] = 0;
      a.rs[1] = H;
      a.rs[2] = H + KW;
      a.rs[3] = H + 2 * KW;
      a.N = H + 2 * KW;
      a.K = H;
      a.y = qkv + (size_t)b * qkv_stride;
      return a;
    };
    bool done = false, o_done = false;
    if (fused) {
      GemvArgs a = qkv_args(0);
      a.ra.tagged = x.at<unsigned long long>(x.L.tagged);
      a.ra.group_done = x.at<unsigned long long>(x.L.group_done);
      AttnArgs af = aa;
      af.tagged = a.ra.tagged;
      af.dim = H;
      af.kvw = KW;
      af.spin_limit = kSpinLimit;
      af.nch = x.L.nch_f;
      GemvArgs oa = {};
      if (fuse_o) {
        af.out_t = x.at<unsigned long long>(x.L.att_t);
        oa.xt = af.out_t;
        oa.spin_limit = kSpinLimit;
        oa.status = x.at<int>(x.L.status);
        oa.w[0] = lw.wo;
        oa.rs[0] = 0;
        oa.rs[1] = oa.rs[2] = oa.rs[3] = H;
        oa.N = H;
        oa.K = H;
        oa.y = x2;
        oa.res = xs;
      }
      ProfScope ps(LLAMA_K_QKV_ATTN, x.s);
      const hipError_t e = launch_qkv_attention(wdt, x.c->kv_dtype, (int)d.head, (int)d.g, a, af,
                                                fuse_o ? &oa : nullptr, tmax, x.at<unsigned>(x.L.epoch),
                                                (uint32_t)d.layers, (uint32_t)l + 1u, x.s);
      if (e == hipSuccess) {
        done = true;
        o_done = fuse_o;
      }
      else if (e == hipErrorNotSupported)
        fused = false;  // nothing was launched: the two launches below, for this and the later layers
      else
        return LLAMA_E_HIP;
    }
    if (!done) {
      for (int b = 0; b < B; ++b) {
        GemvArgs a = qkv_args(b);
        ProfScope ps(LLAMA_K_QKV, x.s);
        if ((rc = hip_rc(launch_gemv(wdt, EPI_ROPE, true, a, tun().qkv, x.s)))) return rc;
      }
      ProfScope ps(LLAMA_K_ATTN, x.s);
      if ((rc = hip_rc(launch_attention(x.c->kv_dtype, (int)d.head, (int)d.g, aa, B, tmax, x.s)))) return rc;
    }
    float *tr = trace ? trace + (size_t)l * tstride : nullptr;
    if (tr) {
      if ((rc = hip_rc(hipMemcpyAsync(tr, qkv, sizeof(float) * qkv_stride, hipMemcpyDeviceToDevice, x.s)))) return rc;
      if ((rc = hip_rc(hipMemcpyAsync(tr + qkv_stride, att, sizeof(float) * H, hipMemcpyDeviceToDevice, x.s))))
        return rc;
    }
    for (int b = 0; b < B && !o_done; ++b) {
      GemvArgs a = {};
      a.x = att + (size_t)b * H;
      a.w[0] = lw.wo;
      a.rs[0] = 0;
      a.rs[1] = a.rs[2] = a.rs[3] = H;
      a.N = H;
      a.K = H;
      a.y = xs + (size_t)b * H;
      a.res = xs + (size_t)b * H;
      ProfScope ps(LLAMA_K_O, x.s);
      if ((rc = hip_rc(launch_gemv(wdt, EPI_RESID, false, a, tun().o, x.s)))) return rc;
    }
    if (tr && (rc = hip_rc(hipMemcpyAsync(tr + qkv_stride + H, xs, sizeof(float) * H, hipMemcpyDeviceToDevice, x.s))))
      return rc;
    // the residual stream after O: x2 when the fused launch ran O (one row), else x in place
    float *xm = o_done ? x2 : xs;
    for (int b = 0; b < B; ++b) {
      GemvArgs a = {};
      a.x = xm + (size_t)b * H;
      a.gain = lw.ln2;
      a.eps = x.c->eps;
      a.w[0] = lw.w_gate;
      a.w[1] = lw.w_up;
      a.rs[0] = 0;
      a.rs[1] = a.rs[2] = a.rs[3] = F;
      a.N = F;
      a.K = H;
      a.y = mm + (size_t)b * F;
      ProfScope ps(LLAMA_K_GATE_UP, x.s);
      if ((rc = hip_rc(launch_gemv(wdt, EPI_SWIGLU, true, a, tun().gate_up, x.s)))) return rc;
    }
    for (int b = 0; b < B; ++b) {
      GemvArgs a = {};
      a.x = mm + (size_t)b * F;
      a.w[0] = lw.w_down;
      a.rs[0] = 0;
      a.rs[1] = a.rs[2] = a.rs[3] = H;
      a.N = H;
      a.K = F;
      a.y = xs + (size_t)b * H;
      a.res = xm + (size_t)b * H;
      ProfScope ps(LLAMA_K_DOWN, x.s);
      if ((rc = hip_rc(launch_gemv(wdt, EPI_RESID, false, a, tun().down, x.s)))) return rc;
    }
    if (tr) {
      if ((rc = hip_rc(hipMemcpyAsync(tr + qkv_stride + 2 * H, mm, sizeof(float) * F, hipMemcpyDeviceToDevice, x.s))))
        return rc;
      if ((rc = hip_rc(hipMemcpyAsync(tr + qkv_stride + 2 * H + F, xs, sizeof(float) * H, hipMemcpyDeviceToDevice,
                                      x.s))))
        return rc;
    }
  }
  if (want_head && (logits || next)) {
    for (int b = 0; b < B; ++b) {
      rc = run_lm_head(x, xs + (size_t)b * H, b, logits ? logits + (size_t)b * d.vocab : nullptr,
                       next ? next + b : nullptr);
      if (rc) return rc;
    }
  }
  return LLAMA_OK;
}

int make_ctx(const llama_cfg *c, const llama_weights *w, const llama_kv *kv, const llama_ws *ws, void *stream,
             Ctx *x) {
  int rc;
  if ((rc = check_cfg(c))) return rc;
  if (w && (rc = check_weights(c, w))) return rc;
  if (!w) return LLAMA_E_NULL;
  if (kv && (rc = check_kv(c, kv))) return rc;
  if ((rc = check_ws(c, ws))) return rc;
  x->c = c;
  x->d = dims_of(c);
  x->w = w;
  x->kv = kv;
  x->ws = ws;
  x->L = ws_layout(c, ws->max_batch, ws->max_seq, ws->max_prefill);
  x->s = (hipStream_t)stream;
  x->base = (char *)ws->base;
  return LLAMA_OK;
}

}  // namespace

extern "C" {

int llama_abi_version(void) { return 1; }

const char *llama_strerror(int code) {
  switch (code) {
    case LLAMA_OK: return "ok";
    case LLAMA_E_CONFIG: return "invalid config";
    case LLAMA_E_POS: return "position outside the cache";
    case LLAMA_E_TOKEN: return "token id outside the vocabulary";
    case LLAMA_E_SHAPE: return "shape mismatch";
    case LLAMA_E_NULL: return "required pointer is NULL";
    case LLAMA_E_WORKSPACE: return "workspace too small or not initialised for this config";
    case LLAMA_E_HIP: return "HIP runtime error";
    case LLAMA_E_UNSUPPORTED: return "not supported by this library";
    case LLAMA_E_PAGE: return "a page table entry outside the cache's page pool";
    case LLAMA_E_WAIT: return "a device-side wait for the step's queries gave up (outputs are NaN)";
    default: return "unknown error";
  }
}

int64_t llama_kv_cache_bytes(const llama_cfg *c, int32_t rows, int32_t max_seq) {
  int rc = check_cfg(c);
  if (rc) return rc;
  if (rows <= 0 || max_seq <= 0) return LLAMA_E_SHAPE;
  const Dims d = dims_of(c);
  return (int64_t)d.layers * rows * d.kv * (int64_t)max_seq * d.head * d.kb;
}

int kv_cache_alloc(const llama_cfg *c, int32_t rows, int32_t max_seq, void *k_mem, void *v_mem, size_t bytes_each,
                   llama_kv *out) {
  if (!out || !k_mem || !v_mem) return LLAMA_E_NULL;
  const int64_t need = llama_kv_cache_bytes(c, rows, max_seq);
  if (need < 0) return (int)need;
  if ((size_t)need > bytes_each) return LLAMA_E_WORKSPACE;
  if (((uintptr_t)k_mem & 15u) || ((uintptr_t)v_mem & 15u)) return LLAMA_E_SHAPE;
  const Dims d = dims_of(c);
  out->k = k_mem;
  out->v = v_mem;
  out->rows = rows;
  out->max_seq = max_seq;
  out->layers = c->layers;
  out->kv = c->kv;
  out->head = (int32_t)d.head;
  out->dtype = c->kv_dtype;
  return LLAMA_OK;
}

int64_t llama_workspace_bytes(const llama_cfg *c, int32_t max_batch, int32_t max_seq, int32_t max_prefill) {
  int rc = check_cfg(c);
  if (rc) return rc;
  if (max_batch <= 0 || max_batch > kMaxBatch || max_seq <= 0 || max_prefill < 0) return LLAMA_E_SHAPE;
  if ((int64_t)max_seq > (int64_t)kAttnMaxChunks * attention_chunk(c->kv_dtype, 2 * c->half, c->g))
    return LLAMA_E_UNSUPPORTED;
  if (max_prefill > 65535) return LLAMA_E_UNSUPPORTED;  // one grid row per prompt position
  return (int64_t)ws_layout(c, max_batch, max_seq, max_prefill).total;
}

int llama_workspace_init(const llama_cfg *c, int32_t max_batch, int32_t max_seq, int32_t max_prefill, void *mem,
                         size_t bytes, void *stream, llama_ws *out) {
  if (!mem || !out) return LLAMA_E_NULL;
  const int64_t need = llama_workspace_bytes(c, max_batch, max_seq, max_prefill);
  if (need < 0) return (int)need;
  if ((size_t)need > bytes) return LLAMA_E_WORKSPACE;
  if ((uintptr_t)mem & 255u) return LLAMA_E_SHAPE;
  const WsLayout L = ws_layout(c, max_batch, max_seq, max_prefill);
  hipStream_t s = (hipStream_t)stream;
  char *base = (char *)mem;
  int rc = hip_rc(launch_zero(base, L.rope_cs, s));  // the status word
  if (rc) return rc;
  // rope table: angle t * inv_freq[i] rounded to F32, then cos and sin (main.bend rot_at)
  const int half = c->half;
  std::vector<float> inv(half), cs((size_t)max_seq * half), sn((size_t)max_seq * half);
  host_inv_freq(c, inv.data());
  for (int t = 0; t < max_seq; ++t) {
    for (int i = 0; i < half; ++i) {
      const float a = (float)t * inv[i];
      cs[(size_t)t * half + i] = cosf(a);
      sn[(size_t)t * half + i] = sinf(a);
    }
  }
  if ((rc = hip_rc(hipMemcpyAsync(base + L.rope_cs, cs.data(), sizeof(float) * cs.size(), hipMemcpyHostToDevice, s))))
    return rc;
  if ((rc = hip_rc(hipMemcpyAsync(base + L.rope_sn, sn.data(), sizeof(float) * sn.size(), hipMemcpyHostToDevice, s))))
    return rc;
  if ((rc = hip_rc(hipStreamSynchronize(s)))) return rc;
  out->base = mem;
  out->bytes = bytes;
  out->max_batch = max_batch;
  out->max_seq = max_seq;
  out->max_prefill = max_prefill;
  out->cfg_key = cfg_key(c);
  out->magic = kWsMagic;
  return LLAMA_OK;
}

int64_t llama_trace_floats(const llama_cfg *c) {
  int rc = check_cfg(c);
  if (rc) return rc;
  const Dims d = dims_of(c);
  return d.layers * (4 * d.dim + 2 * d.kvw + d.f);
}

static int decode_common(const llama_cfg *c, const llama_weights *w, const llama_kv *kv, const int32_t *tokens,
                         const int32_t *pos_host, int32_t B, float *logits, int32_t *next, const llama_ws *ws,
                         void *stream, float *trace) {
  if (!kv || !tokens || !pos_host || !w || !ws) return LLAMA_E_NULL;
  // argument checks first (config, cache shape, batch, positions), then the bound buffers
  int rc = check_cfg(c);
  if (rc) return rc;
  if ((rc = check_kv(c, kv))) return rc;
  if (B <= 0 || B > kv->rows || B > kMaxBatch) return LLAMA_E_SHAPE;
  for (int b = 0; b < B; ++b)
    if (pos_host[b] < 0 || pos_host[b] >= kv->max_seq) return LLAMA_E_POS;
  if (logits && ((uintptr_t)logits & 3u)) return LLAMA_E_SHAPE;
  Ctx x;
  if ((rc = make_ctx(c, w, kv, ws, stream, &x))) return rc;
  if (B > ws->max_batch) return LLAMA_E_SHAPE;
  for (int b = 0; b < B; ++b)
    if (pos_host[b] >= ws->max_seq) return LLAMA_E_POS;
  return run_step(x, tokens, pos_host, B, 0, logits, next, true, trace);
}

int llama_decode_step(const llama_cfg *c, const llama_weights *w, const llama_kv *kv, const int32_t *tokens,
                      const int32_t *pos_host, int32_t B, float *logits, int32_t *next, const llama_ws *ws,
                      void *stream) {
  return decode_common(c, w, kv, tokens, pos_host, B, logits, next, ws, stream, nullptr);
}

int llama_decode_step_traced(const llama_cfg *c, const llama_weights *w, const llama_kv *kv, const int32_t *tokens,
                             const int32_t *pos_host, float *logits, int32_t *next, const llama_ws *ws, float *trace,
                             int64_t trace_floats, void *stream) {
  if (!trace) return LLAMA_E_NULL;
  const int64_t need = llama_trace_floats(c);
  if (need < 0) return (int)need;
  if (trace_floats < need) return LLAMA_E_SHAPE;
  return decode_common(c, w, kv, tokens, pos_host, 1, logits, next, ws, stream, trace);
}

int llama_generate_until(const llama_cfg *c, const llama_weights *w, const llama_kv *kv, const int32_t *token,
                         const int32_t *pos_host, int32_t B, int32_t max_new, int32_t eos, int32_t *produced,
                         int32_t *count, const llama_ws *ws, void *stream) {
  if (!kv || !token || !pos_host || !w || !ws || !produced || !count) return LLAMA_E_NULL;
  int rc = check_cfg(c);
  if (rc) return rc;
  if ((rc = check_kv(c, kv))) return rc;
  if (B <= 0 || B > kv->rows || B > kMaxBatch || max_new <= 0) return LLAMA_E_SHAPE;
  for (int b = 0; b < B; ++b)
    if (pos_host[b] < 0 || (int64_t)pos_host[b] + max_new > kv->max_seq) return LLAMA_E_POS;
  Ctx x;
  if ((rc = make_ctx(c, w, kv, ws, stream, &x))) return rc;
  if (B > ws->max_batch) return LLAMA_E_SHAPE;
  for (int b = 0; b < B; ++b)
    if ((int64_t)pos_host[b] + max_new > ws->max_seq) return LLAMA_E_POS;
  // step i reads the previous step's tokens (the caller's for i = 0) and writes produced[i][0..B); the
  // host waits for each step to see whether every row produced eos (the loop's scalar state)
  int32_t pos[kMaxBatch], last[kMaxBatch];
  *count = 0;
  int32_t n = 0;
  for (; n < max_new; ++n) {
    for (int b = 0; b < B; ++b) pos[b] = pos_host[b] + n;
    const int32_t *in = n == 0 ? token : produced + (size_t)(n - 1) * B;
    if ((rc = run_step(x, in, pos, B, 0, nullptr, produced + (size_t)n * B, true, nullptr))) return rc;
    if (hipStreamSynchronize(x.s) != hipSuccess) return LLAMA_E_HIP;
    if (hipMemcpy(last, produced + (size_t)n * B, sizeof(int32_t) * B, hipMemcpyDeviceToHost) != hipSuccess)
      return LLAMA_E_HIP;
    bool all = true;
    for (int b = 0; b < B; ++b) all = all && last[b] == eos;
    if (all) {
      ++n;
      break;
    }
  }
  *count = n;
  if (n < max_new && (rc = hip_rc(launch_zero(produced + (size_t)n * B, sizeof(int32_t) * (size_t)(max_new - n) * B,
                                             x.s))))
    return rc;
  return LLAMA_OK;
}

// the prompt of one cache row (or of one paged row when x.table is set) after the argument checks
static int prefill_common(const Ctx &x, const int32_t *tokens, int32_t S, int32_t pos0, int32_t row,
                          float *logits_last, int32_t *next) {
  int rc;
  if (prefill_tiled_ok(x.c) && x.ws->max_prefill >= 2 && S >= 2) {
    // chunks of at most max_prefill positions, each attending to everything before it in the cache
    for (int32_t c0 = 0; c0 < S; c0 += x.ws->max_prefill) {
      const int32_t n = S - c0 < x.ws->max_prefill ? S - c0 : x.ws->max_prefill;
      const PackSeg piece = {row, pos0 + c0, n, c0 + n == S ? 0 : -1};
      if ((rc = run_prefill_pass(x, tokens + c0, &piece, 1, logits_last, next))) return rc;
    }
    return LLAMA_OK;
  }
  // one position after another through the decode kernels (main.bend forward_pre per prompt
  // position); only the last runs the final norm, the LM head and the argmax
  for (int i = 0; i < S; ++i) {
    const int32_t p = pos0 + i;
    const bool last = (i == S - 1);
    rc = run_step(x, tokens + i, &p, 1, row, last ? logits_last : nullptr, last ? next : nullptr, last, nullptr);
    if (rc) return rc;
  }
  return LLAMA_OK;
}

int llama_prefill(const llama_cfg *c, const llama_weights *w, const llama_kv *kv, int32_t row, const int32_t *tokens,
                  int32_t S, int32_t pos0, float *logits_last, int32_t *next, const llama_ws *ws, void *stream) {
  if (!kv || !tokens || !w || !ws) return LLAMA_E_NULL;
  int rc = check_cfg(c);
  if (rc) return rc;
  if ((rc = check_kv(c, kv))) return rc;
  if (S <= 0 || row < 0 || row >= kv->rows) return LLAMA_E_SHAPE;
  if (pos0 < 0 || (int64_t)pos0 + S > kv->max_seq) return LLAMA_E_POS;
  Ctx x;
  if ((rc = make_ctx(c, w, kv, ws, stream, &x))) return rc;
  if ((int64_t)pos0 + S > ws->max_seq) return LLAMA_E_POS;
  return prefill_common(x, tokens, S, pos0, row, logits_last, next);
}

// paged cache checks: a table, whole pages in the pool, and the matrix-core attention (a wavefront's
// positions, and a prefill key tile, are one page)
static int check_paging(const llama_cfg *c, const llama_kv *kv, const int32_t *table, int32_t pages) {
  if (!table) return LLAMA_E_NULL;
  if (pages < 1 || kv->max_seq % kPageSize != 0) return LLAMA_E_SHAPE;
  if (!attention_paged_supported(c->kv_dtype, 2 * c->half, c->g)) return LLAMA_E_UNSUPPORTED;
  return LLAMA_OK;
}

int llama_decode_step_paged(const llama_cfg *c, const llama_weights *w, const llama_kv *kv, const int32_t *tokens,
                            const int32_t *pos_host, int32_t B, const int32_t *table, int32_t pages, float *logits,
                            int32_t *next, const llama_ws *ws, void *stream) {
  if (!kv || !tokens || !pos_host || !w || !ws) return LLAMA_E_NULL;
  int rc = check_cfg(c);
  if (rc) return rc;
  if ((rc = check_kv(c, kv))) return rc;
  if ((rc = check_paging(c, kv, table, pages))) return rc;
  if (B <= 0 || B > kMaxBatch) return LLAMA_E_SHAPE;
  for (int b = 0; b < B; ++b)
    if (pos_host[b] < 0 || (int64_t)pos_host[b] >= (int64_t)pages * kPageSize) return LLAMA_E_POS;
  if (logits && ((uintptr_t)logits & 3u)) return LLAMA_E_SHAPE;
  Ctx x;
  if ((rc = make_ctx(c, w, kv, ws, stream, &x))) return rc;
  if (B > ws->max_batch) return LLAMA_E_SHAPE;
  for (int b = 0; b < B; ++b)
    if (pos_host[b] >= ws->max_seq) return LLAMA_E_POS;
  x.table = table;
  x.pages = pages;
  x.npages = kv->max_seq / kPageSize;
  return run_step(x, tokens, pos_host, B, 0, logits, next, true, nullptr);
}

int llama_prefill_paged(const llama_cfg *c, const llama_weights *w, const llama_kv *kv, const int32_t *table,
                        int32_t pages, const int32_t *tokens, int32_t S, int32_t pos0, float *logits_last,
                        int32_t *next, const llama_ws *ws, void *stream) {
  if (!kv || !tokens || !w || !ws) return LLAMA_E_NULL;
  int rc = check_cfg(c);
  if (rc) return rc;
  if ((rc = check_kv(c, kv))) return rc;
  if ((rc = check_paging(c, kv, table, pages))) return rc;
  if (S <= 0) return LLAMA_E_SHAPE;
  if (pos0 < 0 || (int64_t)pos0 + S > (int64_t)pages * kPageSize) return LLAMA_E_POS;
  Ctx x;
  if ((rc = make_ctx(c, w, kv, ws, stream, &x))) return rc;
  if ((int64_t)pos0 + S > ws->max_seq) return LLAMA_E_POS;
  x.table = table;
  x.pages = pages;
  x.npages = kv->max_seq / kPageSize;
  return prefill_common(x, tokens, S, pos0, 0, logits_last, next);
}

int llama_prefill_packed(const llama_cfg *c, const llama_weights *w, const llama_kv *kv, const int32_t *table,
                         int32_t pages, const int32_t *tokens, int32_t nseg, const int32_t *seg_row,
                         const int32_t *seg_pos0, const int32_t *seg_len, float *logits, int32_t *next,
                         const llama_ws *ws, void *stream) {
  if (!kv || !tokens || !w || !ws || !seg_pos0 || !seg_len || (!table && !seg_row)) return LLAMA_E_NULL;
  int rc = check_cfg(c);
  if (rc) return rc;
  if ((rc = check_kv(c, kv))) return rc;
  if (table && (rc = check_paging(c, kv, table, pages))) return rc;
  if (nseg < 1 || nseg > kMaxSegments) return LLAMA_E_SHAPE;
  const int64_t room = table ? (int64_t)pages * kPageSize : (int64_t)kv->max_seq;
  int64_t total = 0;
  for (int i = 0; i < nseg; ++i) {
    if (seg_len[i] <= 0) return LLAMA_E_SHAPE;
    if (!table && (seg_row[i] < 0 || seg_row[i] >= kv->rows)) return LLAMA_E_SHAPE;
    if (seg_pos0[i] < 0 || (int64_t)seg_pos0[i] + seg_len[i] > room) return LLAMA_E_POS;
    total += seg_len[i];
  }
  if (total > INT32_MAX) return LLAMA_E_SHAPE;
  if (logits && ((uintptr_t)logits & 3u)) return LLAMA_E_SHAPE;
  Ctx x;
  if ((rc = make_ctx(c, w, kv, ws, stream, &x))) return rc;
  for (int i = 0; i < nseg; ++i)
    if ((int64_t)seg_pos0[i] + seg_len[i] > ws->max_seq) return LLAMA_E_POS;
  if (table) {
    x.table = table;
    x.pages = pages;
    x.npages = kv->max_seq / kPageSize;
  }
  const Dims &d = x.d;
  if (!(prefill_tiled_ok(c) && ws->max_prefill >= 2)) {
    // no matrix-core prefill for this config: segment after segment through the per-prompt path
    const int32_t *tok = tokens;
    for (int i = 0; i < nseg; ++i) {
      Ctx xs = x;
      if (table) xs.table = table + (size_t)i * pages;
      rc = prefill_common(xs, tok, seg_len[i], seg_pos0[i], table ? 0 : seg_row[i],
                          logits ? logits + (size_t)i * d.vocab : nullptr, next ? next + i : nullptr);
      if (rc) return rc;
      tok += seg_len[i];
    }
    return LLAMA_OK;
  }
  // passes of at most max_prefill packed positions; a segment that does not fit continues in the next
  // pass (its later positions attend to the earlier ones through the cache)
  PackSeg piece[kMaxSegments];
  int np = 0, fill = 0, seg = 0, done = 0;  // done: positions of segment `seg` already in a pass
  const int32_t *pass_tokens = tokens;
  while (seg < nseg) {
    const int take = std::min(seg_len[seg] - done, ws->max_prefill - fill);
    const bool ends = done + take == seg_len[seg];
    piece[np++] = {table ? seg : seg_row[seg], seg_pos0[seg] + done, take, ends ? seg : -1};
    fill += take;
    done += take;
    if (ends) {
      ++seg;
      done = 0;
    }
    if (fill == ws->max_prefill || seg == nseg) {
      if (fill == 1) {
        // a one-position pass: the decode kernels
        const PackSeg &p = piece[0];
        Ctx xs = x;
        if (table) xs.table = table + (size_t)p.row * pages;
        const bool head = p.out >= 0;
        rc = run_step(xs, pass_tokens, &p.pos0, 1, table ? 0 : p.row,
                      head && logits ? logits + (size_t)p.out * d.vocab : nullptr, head && next ? next + p.out : nullptr,
                      head, nullptr);
      } else {
        rc = run_prefill_pass(x, pass_tokens, piece, np, logits, next);
      }
      if (rc) return rc;
      pass_tokens += fill;
      np = 0;
      fill = 0;
    }
  }
  return LLAMA_OK;
}

int lm_head_argmax(const llama_cfg *c, const llama_weights *w, const float *hidden, int32_t B, float *logits,
                   int32_t *argmax, const llama_ws *ws, void *stream) {
  if (!hidden || !argmax) return LLAMA_E_NULL;
  Ctx x;
  int rc = make_ctx(c, w, nullptr, ws, stream, &x);
  if (rc) return rc;
  if (B <= 0 || B > ws->max_batch) return LLAMA_E_SHAPE;
  if ((uintptr_t)hidden & 15u) return LLAMA_E_SHAPE;
  for (int b = 0; b < B; ++b) {
    rc = run_lm_head(x, hidden + (size_t)b * x.d.dim, b, logits ? logits + (size_t)b * x.d.vocab : nullptr, argmax + b);
    if (rc) return rc;
  }
  return LLAMA_OK;
}

int llama_profile_enable(int on) {
  Prof &p = prof();
  p.on = on != 0;
  p.marks.clear();
  p.used = 0;
  return LLAMA_OK;
}

int llama_profile_read(int kernel_class, int64_t *launches, double *total_ms) {
  if (!launches || !total_ms) return LLAMA_E_NULL;
  Prof &p = prof();
  int64_t n = 0;
  double ms = 0.0;
  for (auto &m : p.marks) {
    if (m.first != kernel_class) continue;
    if (hipEventSynchronize(m.second.second) != hipSuccess) return LLAMA_E_HIP;
    float e = 0.f;
    if (hipEventElapsedTime(&e, m.second.first, m.second.second) != hipSuccess) return LLAMA_E_HIP;
    ms += e;
    ++n;
  }
  *launches = n;
  *total_ms = ms;
  return LLAMA_OK;
}

namespace {
int sample_k2(int k) {
  int k2 = 1;
  while (k2 < k) k2 <<= 1;
  return k2;
}
}  // namespace

int64_t llama_sample_scratch_bytes(int32_t B, int32_t V, int32_t k) {
  if (B < 0 || V < 1) return LLAMA_E_SHAPE;
  if (k < 1) return LLAMA_E_CONFIG;
  if (k > kSampleMaxK) return LLAMA_E_UNSUPPORTED;
  const int K2 = sample_k2(k);
  if (sample_candidates(V, K2) > kSampleCandMax) return LLAMA_E_UNSUPPORTED;
  return (int64_t)B * sample_chunks(V) * K2 * (int64_t)sizeof(uint64_t);
}

// The candidate keys of llama_sample_noalloc: a file-scope device array, one copy on each GPU the
// library runs on (kept until the process ends).  Host code must not pass `scratch` itself to a kernel
// (on the host it is only a stand-in for the device array): the device address comes from
// hipGetSymbolAddress, taken once per device with that device current and kept in `g_scratch`.
constexpr int64_t kNoAllocKeys = 64 * 4096;  // 64 rows of 16 chunks x 256 keys: 2 MiB
static __device__ __align__(256) uint64_t scratch[kNoAllocKeys];
namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices];

// the device address of this GPU's array, or nullptr (HIP error)
void *noalloc_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}
}  // namespace

int llama_sample_noalloc(const float *logits, int64_t ld, int32_t B, int32_t V, float temp, int32_t k, float p,
                         const uint32_t *seeds, uint32_t draw, const float *u, int32_t *ids, float *vals,
                         int32_t *topk_ids, void *stream) {
  const int64_t need = llama_sample_scratch_bytes(B, V, k);
  if (need < 0) return (int)need;
  if (need > kNoAllocKeys * (int64_t)sizeof(uint64_t)) return LLAMA_E_UNSUPPORTED;  // beyond the static buffer
  if (B == 0) return llama_sample(logits, ld, B, V, temp, k, p, seeds, draw, u, ids, vals, topk_ids, nullptr, 0,
                                  stream);
  void *buf = noalloc_scratch();
  if (!buf) return LLAMA_E_HIP;
  return llama_sample(logits, ld, B, V, temp, k, p, seeds, draw, u, ids, vals, topk_ids, buf,
                      (size_t)kNoAllocKeys * sizeof(uint64_t), stream);
}

int llama_sample(const float *logits, int64_t ld, int32_t B, int32_t V, float temp, int32_t k, float p,
                 const uint32_t *seeds, uint32_t draw, const float *u, int32_t *ids, float *vals, int32_t *topk_ids,
                 void *scratch, size_t scratch_bytes, void *stream) {
  const int64_t need = llama_sample_scratch_bytes(B, V, k);
  if (need < 0) return (int)need;
  if (ld < V) return LLAMA_E_SHAPE;
  if (!(temp > 0.f) || !std::isfinite(temp) || !std::isfinite(p)) return LLAMA_E_CONFIG;
  if (B == 0) return LLAMA_OK;
  if (!logits || !ids || (!seeds && !u)) return LLAMA_E_NULL;
  if (!scratch) return LLAMA_E_NULL;
  if ((size_t)need > scratch_bytes || ((uintptr_t)scratch & 7u)) return LLAMA_E_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  SampleArgs a{};
  a.logits = logits;
  a.ld = ld;
  a.V = V;
  a.k = k;
  a.K2 = sample_k2(k);
  a.nchunk = sample_chunks(V);
  a.temp = temp;
  a.p = p;
  a.seeds = seeds;
  a.draw = draw;
  a.u = u;
  a.ids = ids;
  a.vals = vals;
  a.topk_ids = topk_ids;
  a.cand = reinterpret_cast<uint64_t *>(scratch);
  ProfScope ps(LLAMA_K_SAMPLE, s);
  return hip_rc(launch_sample(a, B, s));
}

int llama_status(const llama_ws *ws, void *stream) {
  if (!ws || !ws->base) return LLAMA_E_NULL;
  if (ws->magic != kWsMagic) return LLAMA_E_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  int flag = 0;
  if (hipStreamSynchronize(s) != hipSuccess) return LLAMA_E_HIP;
  if (hipMemcpy(&flag, ws->base, sizeof(int), hipMemcpyDeviceToHost) != hipSuccess) return LLAMA_E_HIP;
  if (flag) {
    if (launch_zero(ws->base, 64, s) != hipSuccess || hipStreamSynchronize(s) != hipSuccess) return LLAMA_E_HIP;
    return (flag & 1) ? LLAMA_E_TOKEN : (flag & 2) ? LLAMA_E_PAGE : LLAMA_E_WAIT;
  }
  return LLAMA_OK;
}

}  // extern "C"
