// Internal to libllama_mi355x: types, launch descriptors and device helpers shared by the kernels
// and the host entry points.  Written for gfx950 (CDNA4): 64-lane wavefronts, 256-thread blocks.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "llama_mi355x.h"

namespace lm {

constexpr int kThreads = 256;   // every kernel runs 4 wavefronts of 64
constexpr int kMaxBatch = 64;   // rows of one decode call (positions travel as a kernel argument)
constexpr int kAttnMaxChunks = 512;  // chunks per (row, kv head): max_seq <= 512 * chunk (2 per merge thread)
constexpr int kLmGridMax = 2048;

typedef uint16_t bf16_t;  // bf16 kept as its bits; widened by a 16-bit shift (exact)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // one 16-byte load

// ------------------------------------------------------------------ device helpers ----

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Two F32 -> two bf16 (round to nearest even) in one instruction (v_cvt_pk_bf16_f32), a in the low half
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
// Matrix-core operands of two F32: hi = bf16(x), lo = bf16(x - hi) (x - hi is exact in F32), so
// hi + lo carries x to about 2^-17 relative
__device__ __forceinline__ void split_bf16x2(float a, float b, uint32_t &hi, uint32_t &lo) {
  hi = pack_bf16x2(a, b);
  lo = pack_bf16x2(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}

// F32 -> bf16 with round-to-nearest-even; NaN stays NaN
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// RoPE of one pair (main.bend rot_lo / rot_hi): lo' = lo*c + (-hi)*s, hi' = hi*c + lo*s, every product
// and sum rounded on its own (no fused multiply-add), as the F32 reference evaluates it.
__device__ __forceinline__ float rope_lo(float lo, float hi, float c, float s) {
#pragma clang fp contract(off)
  const float a = lo * c;
  const float b = (-hi) * s;
  return a + b;
}
__device__ __forceinline__ float rope_hi(float lo, float hi, float c, float s) {
#pragma clang fp contract(off)
  const float a = hi * c;
  const float b = lo * s;
  return a + b;
}

// The same two formulas as one: own*c + (sign*partner)*s, where partner is the number half a head away
// and sign is -1 in the first half (rot_lo) and +1 in the second (rot_hi).  Negation is exact, so this is
// bit-identical to rope_lo / rope_hi.
__device__ __forceinline__ float rope_pair(float own, float signed_partner, float c, float s) {
#pragma clang fp contract(off)
  const float a = own * c;
  const float b = signed_partner * s;
  return a + b;
}

// 16 bytes of a row: 4 F32 or 8 bf16, widened to F32
template <typename T>
struct Vec16;
template <>
struct Vec16<float> {
  static constexpr int E = 4;
  // the 16 bytes of 4 F32 values
  __device__ __forceinline__ static u32x4 pack(const float *v) {
    return u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
  }
  __device__ __forceinline__ static void unpack(const u32x4 &r, float *o) {
    o[0] = __uint_as_float(r.x);
    o[1] = __uint_as_float(r.y);
    o[2] = __uint_as_float(r.z);
    o[3] = __uint_as_float(r.w);
  }
};
template <>
struct Vec16<bf16_t> {
  static constexpr int E = 8;
  // the 16 bytes of 8 values that are bf16 numbers widened to F32 (their low 16 bits are zero)
  __device__ __forceinline__ static u32x4 pack(const float *v) {
    u32x4 r;
    r.x = (__float_as_uint(v[0]) >> 16) | (__float_as_uint(v[1]) & 0xffff0000u);
    r.y = (__float_as_uint(v[2]) >> 16) | (__float_as_uint(v[3]) & 0xffff0000u);
    r.z = (__float_as_uint(v[4]) >> 16) | (__float_as_uint(v[5]) & 0xffff0000u);
    r.w = (__float_as_uint(v[6]) >> 16) | (__float_as_uint(v[7]) & 0xffff0000u);
    return r;
  }
  __device__ __forceinline__ static void unpack(const u32x4 &r, float *o) {
    o[0] = __uint_as_float(r.x << 16);
    o[1] = __uint_as_float(r.x & 0xffff0000u);
    o[2] = __uint_as_float(r.y << 16);
    o[3] = __uint_as_float(r.y & 0xffff0000u);
    o[4] = __uint_as_float(r.z << 16);
    o[5] = __uint_as_float(r.z & 0xffff0000u);
    o[6] = __uint_as_float(r.w << 16);
    o[7] = __uint_as_float(r.w & 0xffff0000u);
  }
};

template <typename T>
__device__ __forceinline__ float load_scalar(const T *p, size_t i);
template <>
__device__ __forceinline__ float load_scalar<float>(const float *p, size_t i) {
  return p[i];
}
template <>
__device__ __forceinline__ float load_scalar<bf16_t>(const bf16_t *p, size_t i) {
  return bf16_to_f32(p[i]);
}

// streamed once per step: non-temporal 16-byte load
__device__ __forceinline__ u32x4 load_stream16(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ u32x4 load16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
// cache policy of a streaming buffer load (the non-temporal hint, as load_stream16)
constexpr int kBufferNT = 2;

// Block barrier that orders LDS only: waves publish LDS writes to each other, while global loads issued
// before it stay in flight (a full __syncthreads() also waits for every outstanding global access).
// Used wherever threads of a block exchange data through LDS and nothing through global memory.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
// the same for LDS data that one wavefront writes and reads itself
__device__ __forceinline__ void wave_lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// n (4 or 8) consecutive F32 from a 16-byte aligned address
template <int n>
__device__ __forceinline__ void load_f32(const float *p, float (&o)[n]) {
  static_assert(n % 4 == 0, "whole 16-byte vectors");
#pragma unroll
  for (int k = 0; k < n; k += 4) {
    const float4 v = *reinterpret_cast<const float4 *>(p + k);
    o[k] = v.x;
    o[k + 1] = v.y;
    o[k + 2] = v.z;
    o[k + 3] = v.w;
  }
}

// ---- cross-lane sums on VALU permutes (DPP within 16-lane rows, permlane swaps across rows)
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float xor16_sum(float v) {  // v + v of lane ^ 16
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float v) {  // v + v of lane ^ 32
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// Max over the lanes that share (lane % S), S = 16, 32 or 64 (whole rows or half-waves).
template <int S>
__device__ __forceinline__ float strided_max(float v) {
  static_assert(S >= 16, "row-aligned groups");
  if (S <= 16) v = xor16_max(v);
  if (S <= 32) v = xor32_max(v);
  return v;
}
// Sum over each aligned group of N lanes (N = 1, 2, 4, 8, 16, 32, 64); every lane of a group gets it.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if (N >= 2) v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]: lane ^ 1
  if (N >= 4) v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]: lane ^ 2
  if (N >= 8) v += dpp_f<0x141>(v);  // row_half_mirror: the other quad of the half row
  if (N >= 16) v += dpp_f<0x140>(v); // row_mirror: the other half of the row
  if (N >= 32) v = xor16_sum(v);
  if (N >= 64) v = xor32_sum(v);
  return v;
}
// Max over each aligned group of 16 lanes (a DPP row); every lane of the row gets it.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  return v;
}
// Sum over the lanes that share (lane % S), S = 8, 16, 32 or 64: one value per lane position of an
// S-lane group, summed over the 64/S groups of the wavefront.
template <int S>
__device__ __forceinline__ float strided_sum(float v) {
  if (S <= 8) v += dpp_f<0x128>(v);  // row_ror:8: lane ^ 8 within the row
  if (S <= 16) v = xor16_sum(v);
  if (S <= 32) v = xor32_sum(v);
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// -------------------------------------------------------------- launch descriptors ----

enum GemvEpi { EPI_STORE = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_ARGMAX = 3, EPI_ROPE = 4 };

// EPI_ROPE, the q|k|v projection's epilogue: y gets the projections as computed (before RoPE); the
// query heads are rotated into qrot and the key heads rotated and, with the value heads, stored at the
// token's position of its cache row (rounded to the cache type).  The weight rows are visited in an
// order that puts the two numbers of every RoPE pair (i, i + half of a head) side by side, so one
// thread holds both.
struct RopeAppend {
  float *qrot;                     // [M][dim] rotated queries
  void *kc, *vc;                   // this layer's cache [rows][kv][max_seq][head]
  int kv_bf16;                     // cache element type: 1 bf16, 0 F32
  int max_seq, half, dim, kvw;
  int hshift;                      // log2(half): half is 32 or 64
  int row0;                        // cache row of token row 0
  const float *rope_cs, *rope_sn;  // [max_seq][half]
  int pos[kMaxBatch];              // position of each token row
  // paged cache (table != nullptr): cache row 0 is a pool of max_seq positions in pages of kPageSize;
  // token row t's position p lies at pool position page_slot(table + t*pages, p)
  const int32_t *table;
  int pages, npages;               // entries per table row, pages in the pool
  int *status;                     // sticky flag word: bit 1 = a table entry outside the pool
  // nullable: each rotated query, and each key and value as the cache stores it, also goes to
  // tagged[P] (token row 0 only) as one 64-bit word (the tag in the high half, the F32 bits in the
  // low half), for attention blocks of the same launch (tagged_store / tagged_load)
  unsigned long long *tagged;
  // nullable (with tagged): one tagged word per row group of the product, written once the group's
  // outputs are out, so a waiting attention block can poll one word per group instead of every output
  unsigned long long *group_done;
};

// Paged caches: positions of a row lie in pages of kPageSize consecutive pool positions, page i of the
// row being pool page tr[i] (nest card `decode_paged` / `prefill_paged`: row b's positions lie in the
// pages table[b] lists).  An entry outside the pool sets bit 1 of the status word and yields -1.
constexpr int kPageSize = 64;
__device__ __forceinline__ int page_slot(const int32_t *tr, int p, int npages, int *status) {
  const int pg = tr[p / kPageSize];
  if (pg < 0 || pg >= npages) {
    if (status) atomicOr(status, 2);
    return -1;
  }
  return pg * kPageSize + p % kPageSize;
}

// logical row L of the stacked q|k|v rows -> the weight row it reads: inside the q and k heads,
// logical rows 2i and 2i+1 of a head are rows i and i + half
__device__ __forceinline__ int rope_row(int L, int qk_rows, int hshift) {
  if (L >= qk_rows) return L;
  const int w = L & ((2 << hshift) - 1);
  return (L - w) + (w >> 1) + ((w & 1) << hshift);
}

// pair index i (cos/sin column) of logical row L of the q and k heads
__device__ __forceinline__ int rope_pair_index(int L, int hshift) { return (L & ((2 << hshift) - 1)) >> 1; }

// Tagged words: a value and the tag of the launch that wrote it, stored and loaded as one naturally
// aligned 64-bit word with device-scope atomics (written through to memory; read past this XCD's L2).
// A reader takes a word only when its tag is the current launch's, and the 64-bit access is single-copy
// atomic, so the value it takes is the one stored with that tag: no fence or flag is needed.
__device__ __forceinline__ void tagged_store(unsigned long long *p, float v, uint32_t tag) {
  const unsigned long long w = ((unsigned long long)tag << 32) | (unsigned long long)__float_as_uint(v);
  __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long tagged_load(const unsigned long long *p) {
  return __hip_atomic_load(const_cast<unsigned long long *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// the epilogue for one logical row L of token row t: val = its projection, pv = its pair partner's,
// (c, s) = cos/sin of the token's position at the row's pair index (unused for value rows); `tag`
// labels the tagged copies (ra.tagged set)
__device__ __forceinline__ void rope_append(const RopeAppend &ra, float *y, int t, int L, float val, float pv, float c,
                                            float s, uint32_t tag = 0u) {
  const int dshift = ra.hshift + 1, D = 1 << dshift, qk = ra.dim + ra.kvw;
  const int p = ra.pos[t];
  int P = L;
  float out = val;
  if (L < qk) {
    const int w = L & (D - 1), i = w >> 1, upper = w & 1;
    P = (L - w) + i + (upper << ra.hshift);
    // rot_lo: lo*c - hi*s (own = lo); rot_hi: hi*c + lo*s (own = hi)
    out = rope_pair(val, upper ? pv : -pv, c, s);
  }
  y[P] = val;
  if (P < ra.dim) {
    if (ra.tagged)
      tagged_store(ra.tagged + P, out, tag);
    else
      ra.qrot[(size_t)t * ra.dim + P] = out;
    return;
  }
  const bool is_k = P < qk;
  const int r = is_k ? P - ra.dim : P - qk;  // row within the k (or v) heads
  const int j = r >> dshift, d = r & (D - 1);
  int crow = ra.row0 + t, slot = p;
  if (ra.table) {  // the pool row; an entry outside the pool writes nothing
    crow = 0;
    slot = page_slot(ra.table + (size_t)t * ra.pages, p, ra.npages, ra.status);
    if (slot < 0) return;
  }
  const size_t off = (((size_t)crow * (ra.kvw >> dshift) + j) * ra.max_seq + slot) * D + d;
  void *base = is_k ? ra.kc : ra.vc;
  float stored = out;
  if (ra.kv_bf16) {
    const uint16_t hb = f32_to_bf16(out);
    reinterpret_cast<bf16_t *>(base)[off] = hb;
    stored = bf16_to_f32(hb);
  } else {
    reinterpret_cast<float *>(base)[off] = out;
  }
  if (ra.tagged) tagged_store(ra.tagged + P, stored, tag);
}

struct GemvArgs {
  const float *x;      // input [K] (for the norm epilogues: the raw residual stream)
  const void *gain;    // RMSNorm gains [K] in the weight type, or nullptr for a plain input
  float eps;
  const void *w[3];    // stacked row blocks: row r in [rs[i], rs[i+1]) reads w[i] row (r - rs[i]);
  int rs[4];           // SWIGLU: w[0] = gate, w[1] = up, both N rows
  int N, K;
  float *y;            // output [N] (SWIGLU: silu(gate)*up; ARGMAX: logits, may be nullptr)
  const float *res;    // EPI_RESID: y = res + W x (res may alias y)
  int ngroups;         // row groups of R rows
  // EPI_ARGMAX
  float *part_v;       // [grid] per-block winners
  int *part_i;
  int32_t *next;       // nullable: argmax written by a one-block reduce
  RopeAppend ra;       // EPI_ROPE
  // nullable: the input as tagged words [K] written by another role of the same launch (the attention
  // outputs, for the O product in the launch that runs the q/k/v product with the attention); a wait
  // past spin_limit polls gives up with NaN inputs and status bit 3
  const unsigned long long *xt;
  int spin_limit;
  int *status;
};

// several token rows at once (matrix cores): operands split into bf16 hi/lo by k_split
struct SplitArgs {
  const float *x;      // [M][ldin] F32 rows
  int ldin;
  const void *gain;    // RMSNorm gains [K] (weight type) when normalising
  float eps;
  int K, M;            // row length, real rows (rows M..mpad-1 are written as zeros)
  bf16_t *xhi, *xlo;   // [mpad][ldx]
  int ldx;
};

struct GemmArgs {
  const bf16_t *xhi, *xlo;  // [mpad][ldx] operands from k_split
  int ldx;
  const void *w[3];    // as GemvArgs: stacked row blocks (rs), or w[0] = gate, w[1] = up
  int rs[4];
  int N, K, M;
  float *y;            // [M][ldy]
  int ldy;
  const float *res;    // EPI_RESID: y = res + X W^T
  int ldres;
  float *part_v;       // EPI_ARGMAX: [M][part_ld] per-block winners
  int *part_i;
  int part_ld;
  RopeAppend ra;       // EPI_ROPE
  // k_gemm_rows
  float *part;         // [S][M][N] partial sums of the K slices (SwiGLU: [S][M][2N], gate then up)
  int tiles_per_slice; // set by the launcher
  bf16_t *ohi, *olo;   // EPI_SWIGLU: the output as the next product's operands [mpad][ldo]
  int ldo;
  // k_gemm_tiled: K slices (set by the launcher); more than one leaves partial sums in `part` for a reduce
  int kslices;
  // k_gemm_tiled / k_gemm_big: 1 = multiply the operands' lo half too (F32 activations to ~2^-17),
  // 0 = the activations as bf16 (the hi half alone)
  int lo;
};

// x[t] += sum_s part[s][t][:], then the next product's operands from rmsnorm(x[t], gain)
struct RowsNormArgs {
  const float *part;   // [S][M][N]
  int S, M, N;
  float *x;            // [M][ldx] residual stream (updated in place)
  int ldx;
  const void *gain;    // RMSNorm gains [N] (weight type)
  float eps;
  bf16_t *xhi, *xlo;   // [mpad][ldo]
  int ldo;
};

struct AttnArgs {
  const float *q;      // [B][dim] rotated query heads
  void *kc, *vc;       // this layer's cache: [rows][kv][max_seq][head], positions 0..t stored
  int kv, max_seq, half;
  int row0;            // cache row of batch entry 0
  float *out;          // [B][dim]
  int out_stride;
  float *part_o;       // [B][kv][nch][g][head]
  float *part_ml;      // [B][kv][nch][g][2]
  int nch;             // chunk slots per (row, kv head) in the partial arrays
  unsigned *done;      // [B][kv] chunks finished per (row, kv head); zero between launches
  int direct;          // set by the launcher: one chunk per row, outputs written normalised
  // nullable: the outputs also as bf16 hi + lo matrix-core operands ([B][ldo]; hi = bf16(o), lo =
  // bf16(o - hi)), the form the batched O product reads, so no separate split launch is needed
  bf16_t *ohi, *olo;
  int ldo;
  float scale;         // 1/sqrt(head)
  int pos[kMaxBatch];
  // paged cache (as RopeAppend): row b's position p at pool position page_slot(table + b*pages, p) of row 0
  const int32_t *table;
  int pages, npages;
  int *status;
  // a launch that also runs the q/k/v product (one token row, contiguous cache row row0): the queries,
  // and the key and value at t, come from that product's tagged words (RopeAppend::tagged: query
  // number n at n, key head j number d at dim + j*head + d, value at dim + kvw + j*head + d)
  const unsigned long long *tagged;
  const unsigned long long *group_done;  // nullable: the product's per-row-group words (RopeAppend)
  int rows_per_group;                    // the product's rows per group (it divides head)
  int dim, kvw;
  int spin_limit;  // polls before a wait for them gives up (status bit 3; the outputs are then NaN)
  // nullable (one token row): the outputs also as tagged words [dim], for an O product in the same launch
  unsigned long long *out_t;
  // streamed attention (k_attn_stream; set by its launcher, sk_total = 0 otherwise): the step's chunks
  // in (row, kv head, chunk) order, sk_total of them, row b's first at sk_prefix[b]; sk_blocks blocks
  // take equal runs of them, and segment (b, j)'s partials are those of the blocks its chunks fall in
  int sk_total, sk_blocks, sk_rows;
  int sk_prefix[kMaxBatch];
};

// Prefill of S positions of one cache row (bf16 cache): RoPE + append and causal attention
// Prompts packed end to end (nest card `prefill_packed` / `prefill_paged`): the pass's S positions are
// nseg segments, segment s being packed rows seg_start[s] .. seg_start[s+1]-1, consecutive positions
// seg_pos0[s] .. of one request, whose keys and values go to cache row seg_row[s] (or, paged, to the pool
// slots of table row seg_row[s]) and whose queries attend over that request's positions 0 .. their own.
constexpr int kMaxSegments = 64;
constexpr int kPrefillQT = 32;  // query positions per prefill attention block
struct PrefillArgs {
  float *qkv;          // [S][qkv_stride]: q [dim] (rotated in place), k [kvw], v [kvw]
  int qkv_stride;
  bf16_t *kc, *vc;     // this layer's cache: [rows][kv][max_seq][head]
  int kv, g, heads, half, max_seq, S;
  const float *rope_cs, *rope_sn;  // [max_seq][half]
  float *out;          // [S][out_stride] attention output, heads concatenated
  int out_stride;
  float scale;         // 1/sqrt(head)
  // paged cache: every segment's cache row is 0 and its position p lies at pool position
  // page_slot(table + seg_row[s] * pages, p)
  const int32_t *table;
  int pages, npages;
  int *status;
  int nseg;
  int seg_start[kMaxSegments + 1];  // seg_start[0] = 0, seg_start[nseg] = S
  int seg_tile[kMaxSegments + 1];   // first query tile of each segment; seg_tile[nseg] = all tiles
  int seg_pos0[kMaxSegments];
  int seg_row[kMaxSegments];
  // nullable: the q|k|v rows are still the product's K-slice partial sums, part[z][i][n] for z < ks
  // (rows of qkv_stride numbers); the RoPE + append launch adds them in slice order first (the reduce the
  // product would otherwise launch), writing only the rotated queries back to qkv
  const float *part;
  int ks;
};

// the segment holding packed index i of a sorted start list (start[0] = 0, n >= 1 entries)
__device__ __forceinline__ int segment_of(const int *start, int n, int i) {
  int lo = 0, hi = n;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (i >= start[mid])
      lo = mid;
    else
      hi = mid;
  }
  return lo;
}

// Kernel timing: when the host sets `start`/`stop`, the next launch records them from its own dispatch
// packet (hipExtLaunchKernel), so they bracket exactly the kernel's execution; a launcher that issues
// several kernels gives `start` to the first and `stop` to the last.  Cleared once used.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
  bool used = false;       // some launch took an event
  bool stop_used = false;  // a launch took `stop`
};
LaunchEvents &launch_events();

template <typename F, typename... Args>
inline void launch(F kernel, dim3 grid, dim3 block, hipStream_t s, bool first, bool last, Args... args) {
  LaunchEvents &ev = launch_events();
  hipEvent_t e0 = first ? ev.start : nullptr, e1 = last ? ev.stop : nullptr;
  if (e0 || e1) {
    ev.used = true;
    if (e1) ev.stop_used = true;
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, e0, e1, 0, args...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
  }
}

// host-side launchers (one per kernel family); return hipSuccess or the launch error
hipError_t launch_gemv(int wdtype, GemvEpi epi, bool norm, const GemvArgs &a, int grid_cap, hipStream_t s);
int gemv_supported(int wdtype, int K);  // 1 if the chunk count per thread is instantiated
// rows' positions in a.pos[0..B-1], tmax = their maximum
hipError_t launch_attention(int kvdtype, int head, int g, const AttnArgs &a, int B, int tmax, hipStream_t s);
// the separate merge of nch chunk partials of `chunk` positions per (row, kv head)
hipError_t launch_attention_merge(int head, int g, const AttnArgs &a, int B, int nch, int chunk, hipStream_t s);
// The q/k/v product (one token row: GEMV with the RoPE + append epilogue) and the attention of that row
// in one launch (+ the merge of its chunks when that runs separately).  ga: the product's arguments
// (ga.ra.tagged set); aa: the attention's (aa.tagged, aa.nch slots per kv head for this launch's chunks).
// Each launch's tag is epoch[0] * tag_mul + tag_add (the step counter times the layers, plus the layer
// + 1).  Returns hipErrorNotSupported, having launched nothing, for shapes without an instantiation.
hipError_t launch_qkv_attention(int wdtype, int kvdtype, int head, int g, const GemvArgs &ga, const AttnArgs &aa,
                                const GemvArgs *oa, int tmax, const unsigned *epoch, uint32_t tag_mul,
                                uint32_t tag_add, hipStream_t s);
// whether that launch can also run the O product (oa non-null): its attention outputs are final in the
// launch (merged there), so the O blocks can poll them as tagged words
int qkv_attention_fuses_o(int kvdtype);
int qkv_attention_chunk(int kvdtype, int head, int g);  // positions per attention block of that launch (0: none)
int attention_supported(int head, int g);
int attention_paged_supported(int kvdtype, int head, int g);  // the matrix-core kernel (whole pages per wave)
int attention_chunk(int kvdtype, int head, int g);
// device-scope stores and loads (the scope bits on the instruction keep them coherent across the XCDs'
// L2 caches: a store is written through, a load does not hit a stale line)
__device__ __forceinline__ void store_dev(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_dev(const float *p) {
  return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
 // the smallest chunk of positions an attention block takes
int gemm_rows_supported(int wdtype, int K, int M);  // k_gemm_rows: bf16 weights, K % 128 == 0, 1 <= M <= 64
int gemm_rows_blocks(int N, bool swiglu);
int gemm_rows_slices(int N, int K, bool swiglu, int target);
// a split is always followed by its product: the split takes a timing scope's start event, the
// product (and, for the LM head, the argmax reduce) its stop event
hipError_t launch_split(int gdtype, bool norm, const SplitArgs &a, int mpad, hipStream_t s);
// S K slices; `first`/`last` mark the timing scope's first and last launch
hipError_t launch_gemm_rows(GemvEpi epi, GemmArgs a, int S, hipStream_t s, bool first, bool last);
hipError_t launch_rows_reduce_norm(int gdtype, const RowsNormArgs &a, hipStream_t s, bool last);
// many token rows (prefill): 128 x 128 tiles; the operands need gemm_tiled_rows(M) rows (zero-padded)
int gemm_tiled_rows(int M);
// K slices of a tiled product of M rows (more than one when the tiles alone would not fill the GPU) and
// the partial-sum floats they need in GemmArgs::part (0 for one slice)
int gemm_tiled_kslices(int M, int N, int K, bool swiglu);
size_t gemm_tiled_part_floats(int M, int N, int K, bool swiglu);
// For a residual product (y == res) that runs in K slices: the reduce also normalises the updated rows
// (RMSNorm with `gain`, of type gdtype) and writes them as the next product's bf16 hi/lo operands
// (k_rows_reduce_norm); `done` reports whether it did (else the caller splits them itself)
struct NormNext {
  const void *gain;
  int gdtype;
  float eps;
  bf16_t *xhi, *xlo;
  int ldo;
  bool done;
};
// first: the product's launch starts the profiling scope (no operand split launched before it).
// defer_ks (EPI_STORE): when non-null and the product runs in K slices, no reduce is launched; *defer_ks
// is the slice count (else 0) and the caller adds the partial sums itself (PrefillArgs::part)
hipError_t launch_gemm_tiled(GemvEpi epi, const GemmArgs &a, hipStream_t s, bool last, bool first = false,
                             NormNext *nn = nullptr, int *defer_ks = nullptr);
hipError_t launch_rope_rows(const PrefillArgs &a, hipStream_t s, bool first, bool last);
hipError_t launch_attn_prefill(const PrefillArgs &a, hipStream_t s, bool first, bool last);
// argmax of `rows` rows of per-block winners ([rows][ld], n valid per row) into next[rows]
hipError_t launch_argmax_final(const float *part_v, const int *part_i, int n, int ld, int rows, int32_t *next,
                               hipStream_t s);
// embedding rows of B tokens; `epoch` (nullable) is the step counter, advanced by one per launch
hipError_t launch_embed(int wdtype, const int32_t *tokens, const void *emb, int dim, int vocab, float *x, int B,
                        int *status, unsigned *epoch, hipStream_t s);

// sampling (temperature, top-k, top-p): per-row candidate keys of the first pass in `cand`
// [B][nchunk][K2]; the second pass selects from the nchunk*K2 <= kSampleCandMax keys of a row
constexpr int kSampleMaxK = 256;
constexpr int kSampleCandMax = 8192;
struct SampleArgs {
  const float *logits;
  int64_t ld;
  int V, k, K2, nchunk;
  float temp, p;
  const uint32_t *seeds;
  uint32_t draw;
  const float *u;
  int32_t *ids;
  float *vals;
  int32_t *topk_ids;
  uint64_t *cand;
};
int sample_chunks(int V);
int sample_candidates(int V, int K2);
hipError_t launch_sample(const SampleArgs &a, int B, hipStream_t s);
hipError_t launch_zero(void *p, size_t bytes, hipStream_t s);

}  // namespace lm
