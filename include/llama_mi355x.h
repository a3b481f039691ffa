/*
 * llama_mi355x.h — C ABI of the MI355X (gfx950) Llama-architecture decoder step.
 *
 * What it computes.  One decoder step of a Llama-architecture model: per layer RMSNorm, the Q/K/V
 * projections, RoPE (a head of 2*half numbers, number i rotated with number i + half, with optional
 * llama3 three-band frequency rescaling), a KV-cache append at the token's position, causal
 * grouped-query attention over positions 0..t (query head j*g + i reads key/value head j), the O
 * projection with its residual, RMSNorm, a SwiGLU MLP with its residual; then the final RMSNorm, the
 * tied or untied LM head and a greedy argmax (first index of the largest logit).
 *   Sources: bend-ml-llama@0.2.1.0 main.bend — "The configuration" (Cfg), "The numeric pieces"
 *   (rmsnorm, inv_freq, rope, silu), "The key/value cache in flat arrays" (KV.push), "Grouped-query
 *   attention" (gqa_head, causal), "A layer" (block), "The model" (forward, forward_pre, argmax);
 *   the Llama 3.1 8B Instruct model card (nest) — README (llama3 rope rule, untied head, entries
 *   decode / prefill / decode_rows) and rope.linnet `tables`.
 *
 * Conventions for every call.
 *   - Pointers are DEVICE pointers unless the name ends in _host.  The caller owns every buffer
 *     (weights, caches, workspace, outputs) and the stream; the library never allocates or frees
 *     device memory and keeps no pointer after a call returns.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default stream) unless stated.
 *   - Host-checkable errors are reported BEFORE anything is enqueued, so on error nothing is
 *     written (no cache slot, no output).  Token ids that live in device memory are range-checked
 *     by the kernels: an out-of-range id sets a sticky flag read by llama_status() and that row's
 *     outputs are not meaningful (its embedding is taken as zeros).
 *   - Positions: pos is the 0-based position of the token, i.e. the number of positions the cache
 *     row already holds.  A decode step writes K/V at pos and attends over 0..pos.
 *   - Not thread-safe for concurrent calls that share a workspace or a cache row.
 */
#ifndef LLAMA_MI355X_H
#define LLAMA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* storage types of weights and caches (arithmetic is always F32) */
enum { LLAMA_F32 = 0, LLAMA_BF16 = 1 };

/* return codes */
enum {
  LLAMA_OK = 0,
  LLAMA_E_CONFIG = -1,      /* a size <= 0, eps or theta <= 0 or not finite, bad rope constants, bad dtype */
  LLAMA_E_POS = -2,         /* pos < 0, pos >= max_seq, pos0 + S > max_seq (main.bend kv_room) */
  LLAMA_E_TOKEN = -3,       /* a token id outside [0, vocab) (sticky device flag, see llama_status) */
  LLAMA_E_SHAPE = -4,       /* B <= 0, B > cache rows or workspace batch, row out of range, S <= 0, cache
                               bound to another shape, S > workspace prefill capacity */
  LLAMA_E_NULL = -5,        /* a required pointer is NULL */
  LLAMA_E_WORKSPACE = -6,   /* workspace too small, not initialised, or initialised for another config */
  LLAMA_E_HIP = -7,         /* a HIP runtime call or launch failed */
  LLAMA_E_UNSUPPORTED = -8, /* valid but not built: head not in {64,128}, g not in {1,2,3,4,8}, dim or f not a
                               multiple of 8 or too wide, max_seq > 131072 */
  LLAMA_E_PAGE = -9,        /* a page table entry outside the pool (sticky device flag, see llama_status) */
  LLAMA_E_WAIT = -10        /* a device-side wait of a decode step gave up (sticky device flag, see llama_status) */
};

/*
 * Model config.  Cfg{kv, g, half, f, layers, vocab, eps, theta} (main.bend "The configuration"):
 * kv key/value heads, g query heads per key/value head, half = half a head (head = 2*half),
 * f the MLP inner width.  Derived: heads = kv*g, dim = heads*head, kvw = kv*head.
 * rope_llama3 = 1 applies the llama3 rescale of the frequency table (nest rope.linnet `tables`):
 * wavelength > original/low_freq_factor -> frequency/factor; wavelength < original/high_freq_factor ->
 * unchanged; otherwise the linear blend (1 - s)*f/factor + s*f.  tied_lm_head = 1 uses the
 * embedding as the LM head (main.bend head_of); 0 uses a separate lm_head matrix (nest card).
 * Supported: head in {64, 128}; dim and f multiples of 8.
 */
typedef struct llama_cfg {
  int32_t kv, g, half, f, layers, vocab;
  float eps, theta;
  int32_t rope_llama3;
  float rope_factor, rope_low_freq_factor, rope_high_freq_factor;
  int32_t rope_original_max_pos;
  int32_t tied_lm_head;
  int32_t weight_dtype; /* LLAMA_F32 | LLAMA_BF16: every weight, gain, the embedding and the LM head */
  int32_t kv_dtype;     /* LLAMA_F32 | LLAMA_BF16: the cache (F32 -> bf16 rounds to nearest even) */
} llama_cfg;

/* One layer's weights (main.bend type LW), row = output as PyTorch stores them:
 * ln1 [dim], wq [dim][dim], wk [kvw][dim], wv [kvw][dim], wo [dim][dim], ln2 [dim],
 * w_gate [f][dim], w_up [f][dim], w_down [dim][f].  Rows must start 16-byte aligned (true when
 * dim and f are multiples of 8 and each matrix starts 16-byte aligned). */
typedef struct llama_layer_w {
  const void *ln1, *wq, *wk, *wv, *wo, *ln2, *w_gate, *w_up, *w_down;
} llama_layer_w;

typedef struct llama_weights {
  const void *emb;              /* [vocab][dim]; also the LM head when tied */
  const void *lm_head;          /* [vocab][dim]; NULL iff cfg.tied_lm_head */
  const void *final_norm;       /* [dim] */
  const llama_layer_w *layers;  /* HOST array of cfg.layers entries, each holding device pointers */
} llama_weights;

/*
 * A KV cache bound to caller memory: one K array and one V array per (layer, row, kv head), position
 * p of head j at [p*head, (p+1)*head) (main.bend "The key/value cache in flat arrays"; the nest card's
 * cache_k/cache_v [Batch][KvHeads][MaxSeq][head] per layer).  Layout of k and v:
 * [layers][rows][kv][max_seq][head] in cfg.kv_dtype.  The cache needs no clearing: decoding never
 * reads past a row's own position.
 */
typedef struct llama_kv {
  void *k, *v;
  int32_t rows, max_seq;
  int32_t layers, kv, head, dtype; /* copied from the config by kv_cache_alloc, checked on use */
} llama_kv;

/* A workspace bound by llama_workspace_init: device scratch (activations, split-attention partials,
 * counters, the rope cos/sin table, the status flag) for batches up to max_batch, positions up to
 * max_seq and prompt chunks of up to max_prefill positions (the matrix-core prefill; 0 = none, at most
 * 65535).  Fill it only through llama_workspace_init. */
typedef struct llama_ws {
  void *base;
  size_t bytes;
  int32_t max_batch, max_seq, max_prefill;
  uint32_t cfg_key;  /* fingerprint of the config it was initialised for */
  uint32_t magic;
} llama_ws;

/* Bytes of ONE of the two cache arrays (K or V) for `rows` rows of max_seq positions; < 0 on error. */
int64_t llama_kv_cache_bytes(const llama_cfg *c, int32_t rows, int32_t max_seq);

/* Validate caller memory (k_mem, v_mem, each >= llama_kv_cache_bytes) and fill *out.  Writes no device
 * memory.  Errors: E_NULL, E_CONFIG, E_SHAPE (rows or max_seq <= 0), E_WORKSPACE (bytes_each too small). */
int kv_cache_alloc(const llama_cfg *c, int32_t rows, int32_t max_seq, void *k_mem, void *v_mem, size_t bytes_each,
                   llama_kv *out);

/* Bytes of workspace for the given capacities; < 0 on error. */
int64_t llama_workspace_bytes(const llama_cfg *c, int32_t max_batch, int32_t max_seq, int32_t max_prefill);

/* Bind `mem` (>= llama_workspace_bytes) as a workspace: clears its status flag and the attention
 * kernels' per-(row, kv head) completion counters (each call leaves them zero again), and uploads
 * the rope cos/sin table for positions 0..max_seq-1 (angle t*inv_freq[i] rounded to F32, then cos, sin;
 * main.bend rot_at).  Synchronous: returns after the stream has finished the upload. */
int llama_workspace_init(const llama_cfg *c, int32_t max_batch, int32_t max_seq, int32_t max_prefill, void *mem,
                         size_t bytes, void *stream, llama_ws *out);

/*
 * One decode step for B cache rows (main.bend forward; nest decode / decode_rows): batch entry b takes
 * token tokens[b] at position pos_host[b] of cache row b (rows 0..B-1).  Writes K/V of every layer at
 * that position, then (if logits != NULL) logits[b][vocab] F32 and (if next != NULL) next[b] = the
 * first index of the largest logit.  tokens: device int32 [B]; may alias next (greedy feeding).
 * Errors (nothing enqueued): E_NULL, E_CONFIG, E_SHAPE (B <= 0, B > kv->rows, B > ws->max_batch,
 * cache shape differs from the config), E_POS (pos < 0 or >= kv->max_seq or >= ws->max_seq),
 * E_WORKSPACE, E_HIP.
 */
int llama_decode_step(const llama_cfg *c, const llama_weights *w, const llama_kv *kv, const int32_t *tokens,
                      const int32_t *pos_host, int32_t B, float *logits, int32_t *next, const llama_ws *ws,
                      void *stream);

/*
 * The same step with a per-layer trace of intermediates for divergence bisection (B = 1 only).
 * trace: device F32 [layers][4*dim + 2*kvw + f] holding, per layer, in order: q [dim], k [kvw], v [kvw]
 * (projections before RoPE), attn [dim] (attention output), x1 [dim] (after the O projection and its
 * residual), m [f] (SwiGLU output), y [dim] (layer output) — main.bend type Act's q, k, v, attn, m, y.
 * trace_floats must be >= llama_trace_floats(c).
 */
int64_t llama_trace_floats(const llama_cfg *c);
int llama_decode_step_traced(const llama_cfg *c, const llama_weights *w, const llama_kv *kv, const int32_t *tokens,
                             const int32_t *pos_host, float *logits, int32_t *next, const llama_ws *ws,
                             float *trace, int64_t trace_floats, void *stream);

/*
 * A prompt of S tokens (device int32 [S]) into cache row `row` at positions pos0..pos0+S-1
 * (main.bend forward_pre for each prompt position; nest prefill<S>(tokens, pos)), then the final norm,
 * LM head and argmax after the last token only: logits_last [vocab] and next [1] (each optional).
 * Decoding continues at pos0 + S.  With bf16 weights and cache and a workspace whose max_prefill >= 2,
 * the prompt goes through each layer in chunks of up to max_prefill positions (matrix-core products over
 * the chunk, causal attention over the cache); otherwise one position after another through the decode
 * kernels.  Errors: E_SHAPE (S <= 0, row outside the cache), E_POS (pos0 < 0, pos0 + S > max_seq), plus
 * those of decode.
 */
int llama_prefill(const llama_cfg *c, const llama_weights *w, const llama_kv *kv, int32_t row, const int32_t *tokens,
                  int32_t S, int32_t pos0, float *logits_last, int32_t *next, const llama_ws *ws, void *stream);

/*
 * Greedy generation that stops early (nest card `generate_until`): for B rows of the cache, starting from
 * token[b] (device int32 [B]) at position pos_host[b], up to max_new decode steps; step i writes its
 * argmax tokens to produced[i][0..B) (device int32 [max_new][B], step-major) and feeds them to step i+1
 * at positions pos_host[b] + i + 1.  The loop ends after the first step at which every row's token equals
 * eos, or after max_new steps; *count (host) gets the steps taken and produced[count..max_new) is zeroed.
 * The host waits for each step (the stopping test), so unlike llama_decode_step this call returns when
 * the work is done.  Errors as llama_decode_step, plus E_POS when pos_host[b] + max_new exceeds the
 * cache or workspace max_seq, E_SHAPE for max_new <= 0, E_NULL for produced or count NULL.
 */
int llama_generate_until(const llama_cfg *c, const llama_weights *w, const llama_kv *kv, const int32_t *token,
                         const int32_t *pos_host, int32_t B, int32_t max_new, int32_t eos, int32_t *produced,
                         int32_t *count, const llama_ws *ws, void *stream);

/*
 * Paged cache (nest card `decode_paged` / `prefill_paged`: with one cache row, that row is a pool of
 * positions in pages of 64, and request b's positions lie in the pages its table row lists).  Cache row 0
 * of `kv` is the pool: kv->max_seq pool positions (a multiple of 64), npool = kv->max_seq / 64 pages, the
 * same page numbering in every layer and kv head.  Position p of a request with table row T (device
 * int32 [pages]) lives at pool position T[p / 64] * 64 + p % 64.  The table is read on the device: an
 * entry outside [0, npool) writes no key or value, reads page 0 instead, and sets the sticky status
 * (llama_status returns LLAMA_E_PAGE); the caller keeps the entries a step reaches valid.  Pages may be
 * shared by requests for reading (a common prefix); two requests writing one slot in one call race.
 * Needs a bf16 cache and the matrix-core attention (head 64 or 128 with its g; else E_UNSUPPORTED).
 *
 * llama_decode_step_paged: as llama_decode_step for B <= 64 requests, request b's table row at
 * table + b * pages (device int32 [B][pages]), its token at pos_host[b] < pages * 64 (E_POS beyond) and
 * below the workspace's max_seq; B is bounded by the workspace's max_batch, not by kv->rows.
 * llama_prefill_paged: as llama_prefill for one request whose table row is `table` [pages]
 * (pos0 + S <= pages * 64).
 */
int llama_decode_step_paged(const llama_cfg *c, const llama_weights *w, const llama_kv *kv, const int32_t *tokens,
                            const int32_t *pos_host, int32_t B, const int32_t *table, int32_t pages, float *logits,
                            int32_t *next, const llama_ws *ws, void *stream);
int llama_prefill_paged(const llama_cfg *c, const llama_weights *w, const llama_kv *kv, const int32_t *table,
                        int32_t pages, const int32_t *tokens, int32_t S, int32_t pos0, float *logits_last,
                        int32_t *next, const llama_ws *ws, void *stream);

/*
 * Packed prefill (nest cards `prefill_packed` and `prefill_paged`): the prompts of nseg <= 64 requests
 * packed end to end in `tokens` (device int32, segment 0's tokens first), no padding between them.
 * Segment s is seg_len[s] >= 1 consecutive positions seg_pos0[s] .. of one request; its keys and values go
 * to that request's cache and each of its positions attends over the request's positions 0 .. itself
 * (those already in the cache and those of the segment), never over another segment's request.
 *   table NULL  the request is cache row seg_row[s] (host int32 [nseg], each in [0, kv->rows));
 *               seg_pos0[s] + seg_len[s] <= kv->max_seq.
 *   table set   the paged pool of llama_decode_step_paged: segment s is the request of table row s
 *               (device int32 [nseg][pages]); seg_row is not read; seg_pos0[s] + seg_len[s] <= pages * 64.
 * With seg_pos0[s] = 0 for every segment this is the pages' packed prefill exactly (each prompt sees
 * only itself); a later start continues a request after positions it already holds (a chunk, or pages
 * shared with another request).  Segments of one request must not overlap in positions; two segments
 * writing one cache slot race.  The bf16 matrix-core path packs up to the workspace's max_prefill
 * positions per pass (a segment that does not fit continues in the next pass); other configs run the
 * segments one after another as llama_prefill.
 *   logits  device F32 [nseg][vocab], segment s's logits after its last position (optional)
 *   next    device int32 [nseg], their argmax (optional)
 * seg_row (table NULL), seg_pos0 and seg_len are host arrays, read before the call returns.  Errors
 * (nothing enqueued): E_NULL, E_SHAPE (nseg outside [1, 64], a length < 1, a row outside the cache,
 * misaligned logits), E_POS (a segment past its room or the workspace's max_seq), E_UNSUPPORTED (paged
 * without the matrix-core attention), and those of llama_prefill.
 */
int llama_prefill_packed(const llama_cfg *c, const llama_weights *w, const llama_kv *kv, const int32_t *table,
                         int32_t pages, const int32_t *tokens, int32_t nseg, const int32_t *seg_row,
                         const int32_t *seg_pos0, const int32_t *seg_len, float *logits, int32_t *next,
                         const llama_ws *ws, void *stream);

/*
 * Final RMSNorm + LM head + argmax of B hidden states (device F32 [B][dim], the last layer's output
 * before the final norm): main.bend head_of and argmax.  logits [B][vocab] optional, argmax [B] required.
 */
int lm_head_argmax(const llama_cfg *c, const llama_weights *w, const float *hidden, int32_t B, float *logits,
                   int32_t *argmax, const llama_ws *ws, void *stream);

/*
 * Sampling with temperature, top-k and top-p (main.bend "Sampling": topk, weight, total, kept, pick,
 * sample; draws from its `uniform`).  For each row b < B of logits (device F32, row b at
 * logits + b*ld, V values): the min(k, V) largest logits, largest first, equal logits in id order;
 * weights w_j = exp(v_j/temp - v_0/temp) in F32 (the exponential correctly rounded); running sums
 * S_j = S_{j-1} + w_j from 0 in that order, Z the last; top-p keeps candidate 0 and each next one while
 * the running sum before it is below p*Z; z = the running sum of the last kept one; with the uniform
 * u_b, the drawn candidate is the first kept one whose S_j is above u_b*z, else the last kept one.
 *   u_b      u[b] when `u` (device F32 [B], values in [0, 1)) is not NULL, else draw `draw` of the seed
 *            seeds[b] (device uint32 [B]): the top 24 bits of lowbias32(lowbias32(seed) + draw) times
 *            2^-24, so a (seed, draw) pair gives the same u whatever ran before.
 *   ids      device int32 [B]: the drawn token ids (required); vals: device F32 [B], their logits
 *            (optional); topk_ids: device int32 [B][k], the candidates in order, -1 past V (optional).
 *   scratch  device memory of at least llama_sample_scratch_bytes(B, V, k) bytes, 8-byte aligned,
 *            owned by the caller; it holds per-chunk candidates between the two kernels, so calls
 *            sharing one scratch buffer must be ordered on one stream.
 * Logits must be finite.  Runs on `stream`; every value is written on the device, nothing is
 * synchronised.  Errors (nothing launched): E_SHAPE (B < 0, V < 1, ld < V), E_CONFIG (k < 1, temp not
 * finite and > 0, p not finite), E_NULL (logits, ids or scratch NULL, or both seeds and u NULL),
 * E_WORKSPACE (scratch too small or misaligned), E_UNSUPPORTED (k > 256, or V above 8192 * (8192 / K2)
 * with K2 = k rounded up to a power of two: 262144 at k = 256).  B = 0 returns LLAMA_OK.
 */
int64_t llama_sample_scratch_bytes(int32_t B, int32_t V, int32_t k);

/*
 * llama_sample without a scratch argument, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation): the candidate keys live
 * in a static device array of the library (2 MiB on each GPU it runs on, held until the process
 * ends; llama_sample_scratch_bytes(B, V, k) must not exceed it: 64 rows of the 128256-token vocabulary
 * at k <= 256).  Same arguments, results and errors as llama_sample, plus E_UNSUPPORTED when the
 * candidates would not fit and E_HIP when the array's address cannot be obtained.  Nothing is
 * allocated.  Calls on one GPU share its array: two calls that overlap in time on one GPU (different
 * streams, or threads) race; order them on one stream.  The stream must belong to the current device.
 */
int llama_sample_noalloc(const float *logits, int64_t ld, int32_t B, int32_t V, float temp, int32_t k, float p,
                         const uint32_t *seeds, uint32_t draw, const float *u, int32_t *ids, float *vals,
                         int32_t *topk_ids, void *stream);
int llama_sample(const float *logits, int64_t ld, int32_t B, int32_t V, float temp, int32_t k, float p,
                 const uint32_t *seeds, uint32_t draw, const float *u, int32_t *ids, float *vals, int32_t *topk_ids,
                 void *scratch, size_t scratch_bytes, void *stream);

/*
 * Kernel timing for measurement.  While enabled, every kernel launch of the calls above is bracketed
 * by two HIP events recorded on the call's stream, grouped by kernel class; llama_profile_read waits
 * for the recorded events and returns the number of launches of one class and their summed elapsed
 * milliseconds since the last llama_profile_enable.  Events are created by the library on first use
 * and kept until the process ends; no device memory is allocated.  Not thread-safe.
 */
enum {
  LLAMA_K_EMBED = 0, LLAMA_K_QKV = 1, LLAMA_K_ATTN = 2, LLAMA_K_O = 3, LLAMA_K_GATE_UP = 4, LLAMA_K_DOWN = 5,
  LLAMA_K_LM_HEAD = 6, LLAMA_K_SAMPLE = 7, LLAMA_K_QKV_ATTN = 8
};
int llama_profile_enable(int on);
int llama_profile_read(int kernel_class, int64_t *launches, double *total_ms);

/* Synchronise `stream` and return the sticky device-side status, then clear it: LLAMA_OK, else LLAMA_E_TOKEN
 * (a token out of range), else LLAMA_E_PAGE (a page table entry outside the pool), else LLAMA_E_WAIT (an
 * attention block of a batch-1 step stopped waiting for the step's queries: its outputs are NaN; not
 * expected unless the GPU is shared with work that keeps the step's blocks from running). */
int llama_status(const llama_ws *ws, void *stream);

/* Static description of a return code. */
const char *llama_strerror(int code);

/* Version of the library ABI (this header): 1. */
int llama_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LLAMA_MI355X_H */
