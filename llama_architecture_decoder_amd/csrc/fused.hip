// The q/k/v product and the causal GQA attention of one token row in one launch (batch-1 decode).
//
// What it computes is unchanged from the two separate launches (main.bend "A layer": rmsnorm, the
// q/k/v projections, RoPE and the cache append at t, then "Grouped-query attention over the arrays":
// query head j*g+i over key/value head j, positions 0..t exactly, softmax, weighted V).  What changes is
// when the attention's cache reads happen: positions 0..t-1 were written by earlier steps, so the
// attention blocks stream them while the product's blocks stream the weights, and only the queries and
// the key and value at t wait for the product.
//
// Grid: blocks [0, nq) run the product (gemv_body with the RoPE + append epilogue), blocks from nq on
// are the attention blocks, (chunk c, kv head j) = (ab % nact, ab / nact).  The product's epilogue also
// writes each rotated query, and the key and value at t as the cache stores them, as tagged words
// (value + the launch's tag in one 64-bit word, tagged_store).  An attention block issues its cache loads
// for positions before t, then polls the tagged words of its kv head until every one carries this
// launch's tag; the chunk holding t takes that position's key and value from the words as well.  The
// tag is the device-side step counter (advanced by the step's embedding launch) times the layer count
// plus the layer + 1, so a graph replay of the step gets new tags too.
//
// Progress: the product's blocks never wait and come first in the grid, which the dispatcher starts in
// order, so every word a waiting block polls for is written by a block that is running or done.  A
// wait that outlasts spin_limit polls (~0.1 s) gives up: its block sets status bit 3 (llama_status:
// LLAMA_E_WAIT) and finishes with NaN queries, and while that bit is set every later wait ends at its
// first poll, so each launch always ends and a failure costs one wait.
#include <algorithm>

#include "attention_body.h"
#include "gemv_body.h"

namespace lm {

// positions per wavefront of the matrix-core role: 32 (chunks of 128)
constexpr int kFusedNpw = 32;
// Per cache type (measured, batch-1 decode with 4 full-width layers, us per step: 8B shape at
// positions 7936.., 1.7B shape at 767..):
//  - the merge: by a separate launch (kMergePlain), by the last chunk block of each kv head to finish
//    (kMergeSelf, finish_chunk_merge), or by all of the head's chunk blocks, each polling for the
//    others' partials as tagged words and merging a slice of the outputs.  bf16 / matrix cores:
//    separate, 505-507 us (last block 529-530, all blocks 514-532: the merge of 64 chunks waits for the
//    head's slowest one); F32: last block 289.6-289.8, all blocks 291.5-291.8, separate 293-296 us.
//  - the attention's cache loads before the poll for the queries (early) or after it (the product's
//    weight stream then has the memory to itself): bf16 early, F32 late.
//  - product blocks: as many as fit beside the attention's (kProductRoom), that many with the row
//    groups spread evenly (kProductBalanced: 2-4 us slower, every block then takes two rounds), or
//    one per row group (kProductAll; attention blocks that do not fit start as product blocks end).
//  - the wait: poll one word per product row group first (group words), or the outputs themselves.
//  For reference, the two launches without fusion: 505 us (8B), 295 us (1.7B).
enum { kProductRoom = 0, kProductBalanced = 1, kProductAll = 2 };
//  - the values' cache loads with the keys' (before the poll) or after the queries are seen (the scores
//    and the softmax then run while they are in flight; matrix-core role only): after, 501-502 vs
//    505-507 us at the 8B shape.
template <typename KT>
struct FusedPlan {
  static constexpr bool mfma = sizeof(KT) == 2;
  static constexpr int merge = mfma ? kMergePlain : kMergeSelf;
  static constexpr bool early_kv = mfma;
  static constexpr bool late_v = mfma;
  static constexpr int product = mfma ? kProductRoom : kProductAll;
  static constexpr bool group_words = !mfma;
};

// One wavefront polls the product's row-group words of kv head j (the query heads' groups, and in the
// chunk holding t the key and value head's) until every one carries this launch's tag, with a pause
// between polls; the block waits at a barrier.  A wait that outlasts spin_limit polls, or finds status
// bit 3 set, sets the bit and stops (poll_qkv then gives up at once).
template <int G, int D>
__device__ void wait_groups(const AttnArgs &a, int j, bool last, uint32_t tag) {
  if (threadIdx.x < 64) {
    const int R = a.rows_per_group;
    const int nqg = G * D / R, nkg = last ? D / R : 0;
    const int q0 = j * (G * D / R), k0 = (a.dim + j * D) / R, v0 = (a.dim + a.kvw + j * D) / R;
    const int n = nqg + 2 * nkg;
    int spins = 0;
    for (;;) {
      bool ok = true;
      for (int e = threadIdx.x; e < n; e += 64) {
        const int gi = e < nqg ? q0 + e : (e < nqg + nkg ? k0 + (e - nqg) : v0 + (e - nqg - nkg));
        ok &= (uint32_t)(tagged_load(a.group_done + gi) >> 32) == tag;
      }
      if (__all(ok)) break;
      ++spins;
      if (spins >= a.spin_limit ||
          ((spins & 63) == 0 && (__hip_atomic_load(a.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & 8))) {
        if (threadIdx.x == 0) atomicOr(a.status, 8);
        break;
      }
      __builtin_amdgcn_s_sleep(16);
    }
  }
  lds_barrier();
}

// The tagged words of kv head j: the g query heads into q_s and, in the chunk holding t, the key and
// value at t into kt_s / vt_s.  Every thread of the block calls it.  Returns false when the wait gave up
// (the words still missing are then NaN).
template <int G, int D>
__device__ bool poll_qkv(const AttnArgs &a, int j, bool last, uint32_t tag, float (&q_s)[G][D], float (&kt_s)[D],
                         float (&vt_s)[D]) {
  __shared__ int ok_s[kThreads / 64];
  __shared__ int stop_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const unsigned long long *tq = a.tagged + (size_t)j * G * D;
  const unsigned long long *tk = a.tagged + a.dim + (size_t)j * D;
  const unsigned long long *tv = tk + a.kvw;
  bool give_up = false;
  for (int it = 0;; ++it) {
    int ok = 1;
    for (int e = tid; e < G * D; e += kThreads) {
      const unsigned long long w = tagged_load(tq + e);
      const bool hit = (uint32_t)(w >> 32) == tag;
      if (hit || give_up) (&q_s[0][0])[e] = hit ? __uint_as_float((uint32_t)w) : __builtin_nanf("");
      ok &= hit;
    }
    if (last) {
      for (int e = tid; e < 2 * D; e += kThreads) {
        const unsigned long long w = tagged_load(e < D ? tk + e : tv + (e - D));
        const bool hit = (uint32_t)(w >> 32) == tag;
        if (hit || give_up) {
          const float v = hit ? __uint_as_float((uint32_t)w) : __builtin_nanf("");
          if (e < D)
            kt_s[e] = v;
          else
            vt_s[e - D] = v;
        }
        ok &= hit;
      }
    }
    const int wave_ok = __all(ok);
    if (lane == 0) ok_s[wave] = wave_ok;
    // a wait that gave up in this or an earlier launch (status bit 3, sticky until read) ends every
    // later wait at once, so a failure costs one wait, not one per launch
    if (tid == 0)
      stop_s = it >= a.spin_limit ||
               (__hip_atomic_load(a.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & 8) != 0;
    lds_barrier();  // also publishes the q_s / kt_s / vt_s writes
    int all = 1;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) all &= ok_s[w];
    if (all) return true;
    if (give_up) {
      if (tid == 0) atomicOr(a.status, 8);
      return false;
    }
    give_up = stop_s != 0;  // the next pass fills what is still missing with NaN, then returns
    lds_barrier();  // every wave has read ok_s and stop_s before they are written again
    __builtin_amdgcn_s_sleep(2);
  }
}

// Matrix-core attention role (bf16 cache): 4 wavefronts of NPW positions, as k_attn_mfma with keys
// loaded straight in the MFMA layout.
template <int D, int G, int NPW>
__device__ __forceinline__ void attn_role_mfma(const AttnArgs &a, int c, int j, int nact, uint32_t tag) {
  constexpr int NW = 4;
  using S = MfmaAttnShape<D, G, NPW, NW>;
  constexpr int CHUNK = S::CHUNK, NGI = S::NGI, KS = S::KS, LPR = S::LPR, PPI = S::PPI, NV = S::NV;
  const int t = a.pos[0];
  const bool last = c == nact - 1;
  const int tl = t > 0 ? t - 1 : 0;  // the cache holds positions 0..t-1 before the product appends t
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int pw0 = c * CHUNK + wave * NPW;
  __shared__ __attribute__((aligned(16))) float q_s[G][D];
  __shared__ __attribute__((aligned(16))) float kt_s[D], vt_s[D];

  const size_t head_off = ((size_t)a.row0 * a.kv + j) * (size_t)a.max_seq * D;
  const bf16_t *Kh = reinterpret_cast<const bf16_t *>(a.kc) + head_off;
  const bf16_t *Vh = reinterpret_cast<const bf16_t *>(a.vc) + head_off;
  // (1) keys in the B layout (lane l: position l%16 of a 16-key group, numbers 32 ks + 8(l/16) .. +8) and
  // value rows (lane l: 16 bytes at 8 (l%LPR) of row l/LPR); positions from t on read row t-1 for now
  const int qrow = lane & 15, qh8 = (lane >> 4) * 8;
  const int vl = lane % LPR, vg = lane / LPR;
  u32x4 kb[NGI][KS], vr[NV];
  auto load_k = [&]() {
#pragma unroll
    for (int gi = 0; gi < NGI; ++gi) {
      const int p = min(pw0 + 16 * gi + qrow, tl);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kb[gi][ks] = load_stream16(Kh + (size_t)p * D + 32 * ks + qh8);
    }
  };
  auto load_v = [&]() {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int p = min(pw0 + PPI * i + vg, tl);
      vr[i] = load_stream16(Vh + (size_t)p * D + 8 * vl);
    }
  };
  using P = FusedPlan<bf16_t>;
  if (P::early_kv) {
    load_k();
    if (!P::late_v) load_v();
  }
  // (2) the queries (and the key and value at t) from the product
  if (P::group_words) wait_groups<G, D>(a, j, last, tag);
  poll_qkv<G, D>(a, j, last, tag, q_s, kt_s, vt_s);
  if (!P::early_kv) load_k();
  if (!P::early_kv || P::late_v) load_v();
  if (last) {
#pragma unroll
    for (int gi = 0; gi < NGI; ++gi)
      if (pw0 + 16 * gi + qrow == t)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kb[gi][ks] = Vec16<bf16_t>::pack(&kt_s[32 * ks + qh8]);
  }
  // the lane's value row at t (if any) is taken from vt_s where it is used
  int vti = -1;
  if (last) {
    const int dp = t - pw0 - vg;
    if (dp >= 0 && dp % PPI == 0 && dp / PPI < NV) vti = dp / PPI;
  }
  float qf[KS][8];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) qf[ks][e] = q_s[min(qrow, G - 1)][32 * ks + qh8 + e];
  u32x4 qhi[KS], qlo[KS];
  q_fragments<D, G>(qf, qrow, qhi, qlo);
  auto getk = [&](int gi, u32x4(&kf)[KS]) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kf[ks] = kb[gi][ks];
  };
  mfma_attend<D, G, NPW, NW, P::merge>(a, c, j, 0, t, nact, pw0, qhi, qlo, getk, vr, vt_s, vti, tag);
}

// Vector-unit attention role (any cache type), as k_attn.
template <typename KT, int D, int G>
__device__ __forceinline__ void attn_role_valu(const AttnArgs &a, int c, int j, int nact, uint32_t tag) {
  using S = AttnShape<KT, D>;
  constexpr int E = S::E, LPR = S::LPR, PPR = S::PPR, NR = S::NR, CHUNK = S::CHUNK;
  const int t = a.pos[0];
  const bool last = c == nact - 1;
  const int tl = t > 0 ? t - 1 : 0;
  const int tid = threadIdx.x;
  const int li = tid % LPR, grp = tid / LPR;
  const int p0 = c * CHUNK;
  __shared__ __attribute__((aligned(16))) float q_s[G][D];
  __shared__ __attribute__((aligned(16))) float kt_s[D], vt_s[D];

  const size_t head_off = ((size_t)a.row0 * a.kv + j) * (size_t)a.max_seq * D;
  const KT *Kh = reinterpret_cast<const KT *>(a.kc) + head_off;
  const KT *Vh = reinterpret_cast<const KT *>(a.vc) + head_off;
  u32x4 kraw[NR], vraw[NR];
  auto load_kv = [&]() {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int p = min(p0 + r * PPR + grp, tl);
      kraw[r] = load_stream16(Kh + (size_t)p * D + li * E);
      vraw[r] = load_stream16(Vh + (size_t)p * D + li * E);
    }
  };
  using P = FusedPlan<KT>;
  if (P::early_kv) load_kv();
  if (P::group_words) wait_groups<G, D>(a, j, last, tag);
  poll_qkv<G, D>(a, j, last, tag, q_s, kt_s, vt_s);
  if (!P::early_kv) load_kv();
  if (last) {
#pragma unroll
    for (int r = 0; r < NR; ++r)
      if (p0 + r * PPR + grp == t) {
        kraw[r] = Vec16<KT>::pack(&kt_s[li * E]);
        vraw[r] = Vec16<KT>::pack(&vt_s[li * E]);
      }
  }
  valu_attend<KT, D, G, P::merge>(a, c, j, 0, t, nact, q_s, kraw, vraw, tag);
}

template <typename KT, int D, int G>
constexpr bool fused_mfma() {
  return sizeof(KT) == 2;
}
template <typename KT, int D, int G>
constexpr int fused_chunk() {
  if constexpr (fused_mfma<KT, D, G>())
    return MfmaAttnShape<D, G, kFusedNpw, 4>::CHUNK;
  else
    return AttnShape<KT, D>::CHUNK;
}

// the product and attention roles (blocks [0, nq) and [nq, nq + nact * kv))
template <typename WT, int KCH, typename KT, int D, int G>
__device__ __forceinline__ void qkv_attn_roles(const GemvArgs &g, const AttnArgs &a, int nq, int nact, uint32_t tag) {
  if ((int)blockIdx.x < nq) {
    gemv_body<WT, KCH, EPI_ROPE, true>(g, blockIdx.x, nq, tag);
    return;
  }
  const int ab = blockIdx.x - nq;
  const int c = ab % nact, j = ab / nact;
  if constexpr (fused_mfma<KT, D, G>())
    attn_role_mfma<D, G, kFusedNpw>(a, c, j, nact, tag);
  else
    attn_role_valu<KT, D, G>(a, c, j, nact, tag);
}

template <typename WT, int KCH, typename KT, int D, int G>
__global__ __launch_bounds__(kThreads) void k_qkv_attn(GemvArgs g, AttnArgs a, int nq, int nact, const unsigned *epoch,
                                                       uint32_t tag_mul, uint32_t tag_add) {
  qkv_attn_roles<WT, KCH, KT, D, G>(g, a, nq, nact, epoch[0] * tag_mul + tag_add);
}

// The same with the O product + residual as a third role (blocks from nq + na on; F32 plan): its weights
// stream while the attention finishes, and its input is the attention's outputs as tagged words (K = dim,
// as the q/k/v product's, so the same KCH).  A separate kernel, so that the launches without it keep the
// smaller argument block (measured: 4 us per step at the 1.7B shape with the O arguments always passed).
template <typename WT, int KCH, typename KT, int D, int G>
__global__ __launch_bounds__(kThreads) void k_qkv_attn_o(GemvArgs g, AttnArgs a, GemvArgs o, int nq, int nact, int na,
                                                         const unsigned *epoch, uint32_t tag_mul, uint32_t tag_add) {
  const uint32_t tag = epoch[0] * tag_mul + tag_add;
  if ((int)blockIdx.x >= nq + na) {
    gemv_body<WT, KCH, EPI_RESID, false, true>(o, blockIdx.x - nq - na, gridDim.x - nq - na, tag);
    return;
  }
  qkv_attn_roles<WT, KCH, KT, D, G>(g, a, nq, nact, tag);
}

// Product blocks: enough that the product streams at full rate, and as many as fit beside the attention
// blocks at four blocks per CU.  The matrix-core (bf16, 128-number heads) build needs 134 registers, so
// three fit and the attention blocks that do not start as product blocks end; capping it at 128
// registers for four per CU measured slower (507.8 against 505.8 us per 4-layer 8B step).
constexpr int kFusedResident = 1024;
constexpr int kFusedMinProduct = 256;
// Product blocks of the matrix-core build (three blocks per CU fit, 768 on the chip): measured at the 8B
// shape's 768 row groups, us per 4-layer step: 256 blocks 512.5, 384 505.8, 512 505.8-506.3, 576 505.3,
// 640 502.8-504.0, 704 505.0, 768 503.4-505.3
constexpr int kFusedProductMfma = 640;

template <typename T, int D, int G>
static hipError_t launch_dg(GemvArgs ga, AttnArgs aa, const GemvArgs *oa, int tmax, const unsigned *epoch,
                            uint32_t tag_mul, uint32_t tag_add, hipStream_t s) {
  constexpr int chunk = fused_chunk<T, D, G>();
  const int nact = tmax / chunk + 1;
  if (nact > aa.nch || nact > kAttnMaxChunks) return hipErrorNotSupported;
  constexpr int E = Vec16<T>::E;
  const int kch = (ga.K / E + kThreads - 1) / kThreads;
  const int R = 16 / kch >= 8 ? 8 : 16 / kch >= 4 ? 4 : 16 / kch >= 2 ? 2 : 1;  // RowsPerGroup<kch, 1>
  ga.ngroups = (ga.N + R - 1) / R;
  const int na = nact * aa.kv;
  // attention blocks wait only for the product's blocks, which come first in the grid and never wait;
  // beyond one resident round of attention blocks (F32 heads of 64 past ~4K positions) the two separate
  // launches are used
  if (na > kFusedResident) return hipErrorNotSupported;
  // product blocks: one per row group (F32), or, matrix-core build, kFusedProductMfma (measured), or the
  // room left beside the attention blocks, or that many with the row groups spread evenly (a block with
  // one group more than the others finishes a group's round trip later)
  int room = kFusedResident - na;
  if (room < kFusedMinProduct) room = kFusedMinProduct;
  const int per = (ga.ngroups + room - 1) / room;
  using P = FusedPlan<T>;
  const int nq = P::product == kProductAll        ? ga.ngroups
                 : P::product == kProductBalanced ? (ga.ngroups + per - 1) / per
                                                  : std::min(P::mfma ? kFusedProductMfma : room, ga.ngroups);
  if (P::group_words) {
    if (!ga.ra.group_done || D % R) return hipErrorNotSupported;
    aa.group_done = ga.ra.group_done;
    aa.rows_per_group = R;
  } else {
    ga.ra.group_done = nullptr;
  }
  aa.direct = nact == 1;
  const bool merge_launch = !aa.direct && P::merge == kMergePlain;
  // the O product in the same launch: only where the attention's outputs are final in this launch
  GemvArgs go = {};
  int no = 0;
  if (oa) {
    if (merge_launch || !aa.out_t || oa->K != ga.K || !oa->xt) return hipErrorNotSupported;
    go = *oa;
    go.ngroups = (go.N + R - 1) / R;  // K = dim: the q/k/v product's rows per group
    no = go.ngroups;
  } else {
    aa.out_t = nullptr;
  }
  const dim3 grid(nq + na + no);
  const bool last = !merge_launch;
  if (no > 0) {
    if constexpr (P::mfma) {
      return hipErrorNotSupported;  // the matrix-core plan merges in a separate launch
    } else {
      if (kch == 1)
        launch(k_qkv_attn_o<T, 1, T, D, G>, grid, dim3(kThreads), s, true, last, ga, aa, go, nq, nact, na, epoch,
               tag_mul, tag_add);
      else if (kch == 2)
        launch(k_qkv_attn_o<T, 2, T, D, G>, grid, dim3(kThreads), s, true, last, ga, aa, go, nq, nact, na, epoch,
               tag_mul, tag_add);
      else
        return hipErrorNotSupported;
    }
  } else if (kch == 1) {
    launch(k_qkv_attn<T, 1, T, D, G>, grid, dim3(kThreads), s, true, last, ga, aa, nq, nact, epoch, tag_mul, tag_add);
  } else if (kch == 2) {
    launch(k_qkv_attn<T, 2, T, D, G>, grid, dim3(kThreads), s, true, last, ga, aa, nq, nact, epoch, tag_mul, tag_add);
  } else {
    return hipErrorNotSupported;
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || !merge_launch) return e;
  return launch_attention_merge(D, G, aa, 1, nact, chunk, s);
}

template <typename T, int D>
static hipError_t launch_d(int g, const GemvArgs &ga, const AttnArgs &aa, const GemvArgs *oa, int tmax,
                           const unsigned *epoch, uint32_t tag_mul, uint32_t tag_add, hipStream_t s) {
  switch (g) {
    case 1: return launch_dg<T, D, 1>(ga, aa, oa, tmax, epoch, tag_mul, tag_add, s);
    case 3: return launch_dg<T, D, 3>(ga, aa, oa, tmax, epoch, tag_mul, tag_add, s);
    case 4: return launch_dg<T, D, 4>(ga, aa, oa, tmax, epoch, tag_mul, tag_add, s);
  }
  return hipErrorNotSupported;
}

hipError_t launch_qkv_attention(int wdtype, int kvdtype, int head, int g, const GemvArgs &ga, const AttnArgs &aa,
                                const GemvArgs *oa, int tmax, const unsigned *epoch, uint32_t tag_mul,
                                uint32_t tag_add, hipStream_t s) {
  if (wdtype != kvdtype || !ga.ra.tagged || !aa.tagged || ga.ra.table || aa.table) return hipErrorNotSupported;
  if (wdtype == LLAMA_BF16) {
    if (head == 64) return launch_d<bf16_t, 64>(g, ga, aa, oa, tmax, epoch, tag_mul, tag_add, s);
    if (head == 128) return launch_d<bf16_t, 128>(g, ga, aa, oa, tmax, epoch, tag_mul, tag_add, s);
  } else {
    if (head == 64) return launch_d<float, 64>(g, ga, aa, oa, tmax, epoch, tag_mul, tag_add, s);
    if (head == 128) return launch_d<float, 128>(g, ga, aa, oa, tmax, epoch, tag_mul, tag_add, s);
  }
  return hipErrorNotSupported;
}

int qkv_attention_fuses_o(int kvdtype) { return FusedPlan<float>::merge != kMergePlain && kvdtype == LLAMA_F32; }

int qkv_attention_chunk(int kvdtype, int head, int g) {
  if (g != 1 && g != 3 && g != 4) return 0;
  if (kvdtype == LLAMA_BF16) return head == 64 ? fused_chunk<bf16_t, 64, 1>() : fused_chunk<bf16_t, 128, 1>();
  return head == 64 ? fused_chunk<float, 64, 1>() : fused_chunk<float, 128, 1>();
}

}  // namespace lm
