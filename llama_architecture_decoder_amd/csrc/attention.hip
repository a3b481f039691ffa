// Causal grouped-query decode attention on gfx950.
//
// What it computes (main.bend "Grouped-query attention over the arrays", head_att / group_att /
// attention; nest attention.linnet `decode` / `decode_rows`): for cache row b at position t, query
// head h = j*g + i reads key/value head j (gqa_head); scores s_p = (q_h . K_j[p]) * (1/sqrt(head)) for
// p = 0..t exactly (causal / read_len), softmax over them, o_h = sum_p w_p V_j[p].  The rotated queries
// and the position-t key and value were produced by the q/k/v projection's epilogue (RoPE and the
// cache append, KV.push), so every position 0..t is read from the cache as stored.
//
// Work split (split-K over positions): block (c, j, b) takes chunk c of `chunk` positions of row b's
// head j and all g query heads of the group, so each K/V byte is read from HBM once for g heads.
// Two kernels: k_attn_mfma (bf16 caches) forms the scores on the matrix cores and the weighted V sum
// on the vector units; k_attn (any cache type) does both on the vector units.  Each chunk writes an
// unnormalised partial (o, m, l); the chunks of each (row, kv head) are merged in chunk order, so
// results do not depend on block timing: by a second small kernel, or for small merges by the last
// block of the (row, kv head) to finish (device-scope stores, loads and a completion counter).  When one chunk covers every row's positions
// the attention kernel normalises directly and no merge runs.
//
// k_attn: 256 threads = 256/LPR position groups of LPR lanes, LPR lanes covering one 16-byte slice each
// of a head row (head*bytes/16 lanes), so every load instruction of a wave reads whole contiguous rows.
// Every K and V load of a thread (8 rows each) is issued before any is used.  The query heads are
// staged once per block in LDS.  Each wavefront keeps its scores in registers and forms its own
// softmax pieces (max, exp-sum, exp-weighted V sum) with cross-lane permutes; the 4 wavefronts are
// combined through LDS.
#include <type_traits>

#include "common.h"

namespace lm {

// One normalised output o of row b at column col (of the row's dim outputs), and, when asked, its
// operand split for the batched O product (the bits k_split would give: hi = bf16(o) to nearest even,
// lo = bf16(o - hi))
__device__ __forceinline__ void put_out(const AttnArgs &a, int b, int col, float v) {
  a.out[(size_t)b * a.out_stride + col] = v;
  if (a.ohi) {
    const __bf16 h = (__bf16)v;
    const __bf16 l = (__bf16)(v - (float)h);
    a.ohi[(size_t)b * a.ldo + col] = __builtin_bit_cast(uint16_t, h);
    a.olo[(size_t)b * a.ldo + col] = __builtin_bit_cast(uint16_t, l);
  }
}

template <typename KT, int D>
struct AttnShape {
  static constexpr int E = Vec16<KT>::E;      // elements per 16-byte slice
  static constexpr int LPR = D / E;           // lanes per head row
  static constexpr int PPR = kThreads / LPR;  // positions per round
  static constexpr int NR = 8;                // rounds per thread: every K and V load issued up front
  static constexpr int CHUNK = NR * PPR;      // positions per block
};

// The end of a chunk when the merge runs in the last block of its (row b, kv head j): the partials went
// out with device-scope stores; once they have completed, one thread counts the chunk done with a
// device-scope atomic, and the block that brings the count to nact merges every chunk in chunk order:
// M = max_c m_c, w_c = 2^(m_c - M), L = sum_c w_c l_c, o = (sum_c w_c o_c) / L (maxima are base 2),
// reading the partials with device-scope loads, then clears the count for the next launch.
template <int G, int D>
__device__ void finish_chunk_merge(const AttnArgs &a, int b, int j, int nact, size_t slot) {
  constexpr int OPT = (G * D + kThreads - 1) / kThreads;  // outputs per thread
  constexpr int CB = 16;                                    // chunks per batch of loads
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ int last_s;
  __shared__ float w_s[kAttnMaxChunks * G];
  __shared__ float red_m[4][G], red_l[4][G];
  __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores have completed
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = __hip_atomic_fetch_add(&a.done[b * a.kv + j], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last_s = prev == (unsigned)(nact - 1);
  }
  __syncthreads();
  if (!last_s) return;
  const float *pml = a.part_ml + slot * (size_t)(G * 2);
  const float *po = a.part_o + slot * (size_t)(G * D);
  // (m, l) of chunks tid, tid + 256 for every head
  float mv[2][G], lv[2][G];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int cc = min(tid + k * kThreads, nact - 1);
#pragma unroll
    for (int q = 0; q < G; ++q) {
      mv[k][q] = load_dev(pml + (size_t)cc * G * 2 + 2 * q);
      lv[k][q] = load_dev(pml + (size_t)cc * G * 2 + 2 * q + 1);
    }
  }
  // the first batch of o partials goes out with them
  float ov[OPT][CB];
#pragma unroll
  for (int i = 0; i < OPT; ++i)
#pragma unroll
    for (int k = 0; k < CB; ++k)
      ov[i][k] = load_dev(po + (size_t)min(k, nact - 1) * G * D + min(tid + i * kThreads, G * D - 1));
#pragma unroll
  for (int q = 0; q < G; ++q) {
    float m = -INFINITY;
#pragma unroll
    for (int k = 0; k < 2; ++k)
      if (tid + k * kThreads < nact) m = fmaxf(m, mv[k][q]);
    m = wave_max(m);
    if (lane == 0) red_m[wave][q] = m;
  }
  lds_barrier();
#pragma unroll
  for (int q = 0; q < G; ++q) {
    const float M = fmaxf(fmaxf(red_m[0][q], red_m[1][q]), fmaxf(red_m[2][q], red_m[3][q]));
    float l = 0.f;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int cc = tid + k * kThreads;
      if (cc < nact) {
        const float w = __builtin_amdgcn_exp2f(mv[k][q] - M);
        w_s[cc * G + q] = w;
        l = fmaf(w, lv[k][q], l);
      }
    }
    l = wave_sum(l);
    if (lane == 0) red_l[wave][q] = l;
  }
  lds_barrier();
  float acc[OPT];
#pragma unroll
  for (int i = 0; i < OPT; ++i) acc[i] = 0.f;
  for (int c0 = 0; c0 < nact; c0 += CB) {
    if (c0 > 0) {
#pragma unroll
      for (int i = 0; i < OPT; ++i)
#pragma unroll
        for (int k = 0; k < CB; ++k)
          ov[i][k] = load_dev(po + (size_t)min(c0 + k, nact - 1) * G * D + min(tid + i * kThreads, G * D - 1));
    }
#pragma unroll
    for (int i = 0; i < OPT; ++i) {
      const int q = min(tid + i * kThreads, G * D - 1) / D;
#pragma unroll
      for (int k = 0; k < CB; ++k)
        if (c0 + k < nact) acc[i] = fmaf(w_s[(c0 + k) * G + q], ov[i][k], acc[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < OPT; ++i) {
    const int idx = tid + i * kThreads;
    if (idx < G * D) {
      const int q = idx / D;
      const float L = (red_l[0][q] + red_l[1][q]) + (red_l[2][q] + red_l[3][q]);
      put_out(a, b, j * G * D + idx, acc[i] / L);
    }
  }
  if (tid == 0) __hip_atomic_store(&a.done[b * a.kv + j], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename KT, int D, int G, bool SELF>
__global__ __launch_bounds__(kThreads) void k_attn(AttnArgs a) {
  using S = AttnShape<KT, D>;
  constexpr int E = S::E, LPR = S::LPR, PPR = S::PPR, NR = S::NR, CHUNK = S::CHUNK;
  static_assert(LPR >= 1 && LPR <= 64 && (64 % LPR) == 0, "row must fit a wavefront");
  const int c = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int t = a.pos[b];
  const int nact = t / CHUNK + 1;  // chunks covering 0..t
  if (c >= nact) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = tid % LPR, grp = tid / LPR;
  const int p0 = c * CHUNK;
  const int p1 = min(p0 + CHUNK, t + 1);

  __shared__ float q_s[G][D];                // rotated query heads of the group
  __shared__ float m_s[4][G];
  __shared__ float l_g[kThreads / LPR][G];
  __shared__ float o_g[kThreads / LPR][G][D];

  const size_t head_off = ((size_t)(a.row0 + b) * a.kv + j) * (size_t)a.max_seq * D;
  const KT *Kh = reinterpret_cast<const KT *>(a.kc) + head_off;
  const KT *Vh = reinterpret_cast<const KT *>(a.vc) + head_off;
  const float *qg = a.q + (size_t)b * (a.kv * G * D) + (size_t)j * G * D;

  // (1) the group's query heads, one 16-byte unit per thread, staged in LDS
  constexpr int NQ = G * D / 4;
  static_assert(NQ <= kThreads, "one staging unit per thread");
  float4 qv = make_float4(0.f, 0.f, 0.f, 0.f);
  if (tid < NQ) qv = *reinterpret_cast<const float4 *>(qg + tid * 4);

  // (2) every K and V row of this thread's positions, in flight together.  Loads are unconditional: a
  // position after t reads row t (inside the cache), and its value is never used.
  u32x4 kraw[NR], vraw[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int p = min(p0 + r * PPR + grp, t);
    kraw[r] = load_stream16(Kh + (size_t)p * D + li * E);
    vraw[r] = load_stream16(Vh + (size_t)p * D + li * E);
  }
  if (tid < NQ) *reinterpret_cast<float4 *>(&q_s[0][0] + tid * 4) = qv;
  lds_barrier();

  // (3) this thread's query slices [li*E, li*E + E) of the g heads
  const int d0 = li * E;
  float q[G][E];
#pragma unroll
  for (int i = 0; i < G; ++i)
#pragma unroll
    for (int e = 0; e < E; ++e) q[i][e] = q_s[i][d0 + e];

  // (4) scores of this thread's positions in base 2: s2 = (q . k) * (scale * log2 e), so that
  // exp(s - m) = exp2(s2 - m2); every lane of a position group gets the full dot product
  const float scale2 = a.scale * 1.4426950408889634f;
  float sc[NR][G];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int p = p0 + r * PPR + grp;
    float kf[E];
    Vec16<KT>::unpack(kraw[r], kf);
#pragma unroll
    for (int i = 0; i < G; ++i) {
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) acc = fmaf(q[i][e], kf[e], acc);
      const float dot = group_sum<LPR>(acc);  // every lane takes part in the row permutes
      sc[r][i] = (p < p1) ? dot * scale2 : -INFINITY;
    }
  }
  // (5) softmax pieces of this wavefront per head: max over its positions, 2^(s2 - max), their sum,
  // and sum_p e_p V[p] (per position group; the groups are summed through LDS below)
  float mw[G], lw[G], o[G][E];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    float m = sc[0][i];
#pragma unroll
    for (int r = 1; r < NR; ++r) m = fmaxf(m, sc[r][i]);
    mw[i] = strided_max<LPR < 16 ? 16 : LPR>(LPR < 16 ? fmaxf(m, dpp_f<0x128>(m)) : m);
    lw[i] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) o[i][e] = 0.f;
  }
  // exponent reference: the wavefront max, or 0 when none of its positions is in the chunk (every
  // score is then -inf and every weight 0; -inf - -inf would be NaN)
  float mref[G];
#pragma unroll
  for (int i = 0; i < G; ++i) mref[i] = (mw[i] == -INFINITY) ? 0.f : mw[i];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    float vf[E];
    Vec16<KT>::unpack(vraw[r], vf);
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const float w = __builtin_amdgcn_exp2f(sc[r][i] - mref[i]);  // -inf (masked) gives 0
      lw[i] += w;
#pragma unroll
      for (int e = 0; e < E; ++e) o[i][e] = fmaf(w, vf[e], o[i][e]);
    }
  }
  // per position group: (l, o) to LDS; the wavefront max is the same for its groups
  constexpr int NG = kThreads / LPR;  // position groups per block
#pragma unroll
  for (int i = 0; i < G; ++i) {
    if (li == 0) l_g[grp][i] = lw[i];
#pragma unroll
    for (int e = 0; e < E; ++e) o_g[grp][i][d0 + e] = o[i][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < G; ++i) m_s[wave][i] = mw[i];
  }
  lds_barrier();

  // (6) the position groups combined (a wavefront with no position of the chunk has max -inf,
  // weight 0); groups are summed in a fixed order
  constexpr int GPW = NG / 4;  // position groups per wavefront
  const size_t slot = ((size_t)b * a.kv + j) * (size_t)a.nch;
  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int i = idx / D, d = idx % D;
    const float M = fmaxf(fmaxf(m_s[0][i], m_s[1][i]), fmaxf(m_s[2][i], m_s[3][i]));
    float acc = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = (m_s[w][i] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_s[w][i] - M);
      float ow = 0.f, lsum = 0.f;
#pragma unroll
      for (int g2 = 0; g2 < GPW; ++g2) {
        ow += o_g[w * GPW + g2][i][d];
        lsum += l_g[w * GPW + g2][i];
      }
      acc = fmaf(f, ow, acc);
      L = fmaf(f, lsum, L);
    }
    if (a.direct) {
      put_out(a, b, j * G * D + idx, acc / L);
    } else if (SELF) {
      store_dev(&a.part_o[(slot + c) * (size_t)(G * D) + idx], acc);
      if (d == 0) {
        store_dev(&a.part_ml[(slot + c) * (size_t)(G * 2) + 2 * i], M);
        store_dev(&a.part_ml[(slot + c) * (size_t)(G * 2) + 2 * i + 1], L);
      }
    } else {
      a.part_o[(slot + c) * (size_t)(G * D) + idx] = acc;
      if (d == 0) {
        a.part_ml[(slot + c) * (size_t)(G * 2) + 2 * i] = M;
        a.part_ml[(slot + c) * (size_t)(G * 2) + 2 * i + 1] = L;
      }
    }
  }
  if (SELF && !a.direct) finish_chunk_merge<G, D>(a, b, j, nact, slot);
}

// ------------------------------------------------------------------ matrix-core scores ----
// k_attn_mfma (bf16 cache): each of the NW wavefronts takes chunk/NW consecutive positions, in groups of
// 16.
//   Scores: S[q][p] = Q K^T with v_mfma_f32_16x16x32_bf16, A = the group's query heads (rows q < g of
//   16; the F32 queries as bf16 hi + lo, so the products are those of the F32 values to ~2^-17) and
//   B = K^T (lane l: position l%16, 8 consecutive numbers at 8(l/16) of a 32-wide slice).  In large
//   launches keys are loaded as whole rows and reach that layout through a small per-wave LDS tile, 16
//   keys at a time; in small ones they are loaded in that layout directly.
//   Lane l then holds S[4(l/16) + r][l%16].
//   Softmax pieces per head over the wave's positions (max by DPP within 16-lane rows), the weights go
//   through LDS to the layout of the V loads (lane l: position l/LPR of PPI rows, numbers 8(l%LPR) .. +8),
//   and the weighted V sum runs on the vector units.  The wave's lane groups and the NW waves are combined
//   through LDS in a fixed order, as in k_attn.
typedef __bf16 abf16x8 __attribute__((ext_vector_type(8)));
typedef float af32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ af32x4 mfma16(u32x4 a, u32x4 b, af32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(abf16x8, a), __builtin_bit_cast(abf16x8, b), c, 0,
                                                 0, 0);
}

// 8 F32 -> bf16 hi (RNE) and lo = bf16(x - hi) (x - hi is exact), packed as MFMA operands
__device__ __forceinline__ void split8(const float (&f)[8], u32x4 &hi, u32x4 &lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) split_bf16x2(f[2 * e], f[2 * e + 1], h[e], l[e]);
  hi = u32x4{h[0], h[1], h[2], h[3]};
  lo = u32x4{l[0], l[1], l[2], l[3]};
}

template <int D, int G, int NPW_, int NW_ = 4>
struct MfmaAttnShape {
  static constexpr int NW = NW_;          // wavefronts per block
  static constexpr int NPW = NPW_;        // positions per wavefront
  static constexpr int CHUNK = NW * NPW;  // positions per block
  static constexpr int NGI = NPW / 16;    // 16-position score groups per wavefront
  static constexpr int KS = D / 32;       // 32-wide steps of a score
  static constexpr int LPR = D / 8;       // lanes per V row (16 bytes each)
  static constexpr int PPI = 64 / LPR;    // V rows per wavefront load
  static constexpr int NV = NPW / PPI;    // V loads per lane
  static constexpr int GP = G <= 4 ? 4 : 8;  // weights per position in LDS (padded)
  static constexpr int NG = NW * 64 / LPR;  // lane groups per block
  static constexpr int KROW = D + 8;      // LDS row of a wave's 16-key staging tile (bf16)
  static constexpr size_t LDS = sizeof(float) * (NW * NPW * GP + 2 * NW * G + (size_t)NG * G * D) + 2 * NW * 16 * KROW;
};

template <int D, int G, int NPW_, bool KROWS, bool SELF, int NW = 4>
__global__ __launch_bounds__(NW * 64) void k_attn_mfma(AttnArgs a) {
  using S = MfmaAttnShape<D, G, NPW_, NW>;
  static_assert(!SELF || NW == 4, "the in-kernel merge runs on 4 wavefronts");
  constexpr int CHUNK = S::CHUNK, NPW = S::NPW, NGI = S::NGI, KS = S::KS, LPR = S::LPR, PPI = S::PPI, NV = S::NV;
  constexpr int GP = S::GP, NG = S::NG;
  static_assert(G <= 8, "at most 8 query heads per kv head (two rows of the 16-row tile)");
  const int c = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int t = a.pos[b];
  const int nact = t / CHUNK + 1;
  if (c >= nact) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int pw0 = c * CHUNK + wave * NPW;  // this wavefront's first position
  const int p1 = min(c * CHUNK + CHUNK, t + 1);

  __shared__ __attribute__((aligned(16))) float p_s[NW][NPW][GP];
  __shared__ float m_s[NW][G], l_s[NW][G];
  __shared__ __attribute__((aligned(16))) float o_g[NG][G][D];
  __shared__ __attribute__((aligned(16))) bf16_t k_s[NW][16 * S::KROW];  // each wave's 16 keys in turn

  const size_t head_off = ((size_t)(a.table ? 0 : a.row0 + b) * a.kv + j) * (size_t)a.max_seq * D;
  const bf16_t *Kh = reinterpret_cast<const bf16_t *>(a.kc) + head_off;
  const bf16_t *Vh = reinterpret_cast<const bf16_t *>(a.vc) + head_off;
  // paged cache: the wave's positions (clamped to t) lie in one page, so one table entry places them all
  static_assert(kPageSize % NPW == 0, "a wavefront's positions must lie in one page");
  int pg0 = 0;
  if (a.table) {
    const int pe = min(pw0, t);
    const int sl = page_slot(a.table + (size_t)b * a.pages, pe, a.npages, a.status);
    pg0 = sl < 0 ? 0 : sl - pe % kPageSize;
  }
  auto phys = [&](int p) { return a.table ? pg0 + p % kPageSize : p; };

  // (1) loads, oldest first: the queries (lane l: head l%16 of the group, numbers 32 ks + 8(l/16) .. +8),
  // then keys and values in row slices (lane l: 16 bytes at 8 (l%LPR) of row l/LPR of PPI rows, so a load
  // reads whole rows; the MFMA layout would read 64-byte pieces of 16 rows, which streams slower).
  // Positions after t read row t (never used).
  const int qrow = lane & 15, qh8 = (lane >> 4) * 8;
  const float *qp = a.q + (size_t)b * (a.kv * G * D) + ((size_t)j * G + min(qrow, G - 1)) * D;
  float4 qv[KS][2];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qv[ks][0] = *reinterpret_cast<const float4 *>(qp + 32 * ks + qh8);
    qv[ks][1] = *reinterpret_cast<const float4 *>(qp + 32 * ks + qh8 + 4);
  }
  u32x4 kr[KROWS ? NV : 1], kb[KROWS ? 1 : NGI][KS], vr[NV];
  const int vl = lane % LPR, vg = lane / LPR;
  if (KROWS) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int p = phys(min(pw0 + PPI * i + vg, t));
      kr[i] = load_stream16(Kh + (size_t)p * D + 8 * vl);
    }
  } else {
#pragma unroll
    for (int gi = 0; gi < NGI; ++gi) {
      const int p = phys(min(pw0 + 16 * gi + qrow, t));
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kb[gi][ks] = load_stream16(Kh + (size_t)p * D + 32 * ks + qh8);
    }
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int p = phys(min(pw0 + PPI * i + vg, t));
    vr[i] = load_stream16(Vh + (size_t)p * D + 8 * vl);
  }

  // (2) query fragments: rows q >= g are zero
  u32x4 qhi[KS], qlo[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    float f[8] = {qv[ks][0].x, qv[ks][0].y, qv[ks][0].z, qv[ks][0].w,
                  qv[ks][1].x, qv[ks][1].y, qv[ks][1].z, qv[ks][1].w};
    if (qrow >= G) {
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = 0.f;
    }
    split8(f, qhi[ks], qlo[ks]);
  }

  // (3) scores, base 2: s2 = (q . k) * scale * log2 e; lane holds head 4(lane/16) + r, position
  // pw0 + 16 gi + lane%16
  const float scale2 = a.scale * 1.4426950408889634f;
  float sc[NGI][4];
  bf16_t *kw = k_s[wave];
  constexpr int IPG = 16 / PPI;  // key loads per 16-key group
#pragma unroll
  for (int gi = 0; gi < NGI; ++gi) {
    u32x4 kf[KS];
    if (KROWS) {
      // the group's 16 key rows through the wave's LDS tile into the B layout (lane l: key l%16, numbers
      // 32 ks + 8(l/16) .. +8); LDS operations of a wave complete in order
#pragma unroll
      for (int u = 0; u < IPG; ++u)
        *reinterpret_cast<u32x4 *>(&kw[(PPI * u + vg) * S::KROW + 8 * vl]) = kr[gi * IPG + u];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kf[ks] = *reinterpret_cast<const u32x4 *>(&kw[qrow * S::KROW + 32 * ks + qh8]);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kf[ks] = kb[gi][ks];
    }
    af32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      acc = mfma16(qhi[ks], kf[ks], acc);
      acc = mfma16(qlo[ks], kf[ks], acc);
    }
    const int p = pw0 + 16 * gi + qrow;
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[gi][r] = (p < p1) ? acc[r] * scale2 : -INFINITY;
  }
  // (4) per head: the wave's max, weights 2^(s2 - max) (reference 0 when the wave has no position of
  // the chunk: every weight is then 0), their sum
  const int qbase = 4 * (lane >> 4);  // heads held by this lane: qbase + r
  float mw[4], lw[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float m = sc[0][r];
#pragma unroll
    for (int gi = 1; gi < NGI; ++gi) m = fmaxf(m, sc[gi][r]);
    mw[r] = row16_max(m);
    const float mref = (mw[r] == -INFINITY) ? 0.f : mw[r];
    float l = 0.f;
#pragma unroll
    for (int gi = 0; gi < NGI; ++gi) {
      const float w = __builtin_amdgcn_exp2f(sc[gi][r] - mref);
      sc[gi][r] = w;
      l += w;
    }
    lw[r] = group_sum<16>(l);
  }
  if (qbase < G) {
#pragma unroll
    for (int gi = 0; gi < NGI; ++gi)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (qbase + r < GP) p_s[wave][16 * gi + qrow][qbase + r] = sc[gi][r];
    if (qrow == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (qbase + r < G) {
          m_s[wave][qbase + r] = mw[r];
          l_s[wave][qbase + r] = lw[r];
        }
    }
  }
  lds_barrier();

  // (5) o[q][e] = sum over this lane's positions of w[q] * V[p][8 vl + e]
  float o[G][8];
#pragma unroll
  for (int q = 0; q < G; ++q)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[q][e] = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    float w[GP];
#pragma unroll
    for (int k = 0; k < GP; k += 4) {
      const float4 w4 = *reinterpret_cast<const float4 *>(&p_s[wave][PPI * i + vg][k]);
      w[k] = w4.x;
      w[k + 1] = w4.y;
      w[k + 2] = w4.z;
      w[k + 3] = w4.w;
    }
    float vf[8];
    Vec16<bf16_t>::unpack(vr[i], vf);
#pragma unroll
    for (int q = 0; q < G; ++q)
#pragma unroll
      for (int e = 0; e < 8; ++e) o[q][e] = fmaf(w[q], vf[e], o[q][e]);
  }
  const int grp = tid / LPR;  // lane group of the block: wave * PPI + vg
#pragma unroll
  for (int q = 0; q < G; ++q) {
    *reinterpret_cast<float4 *>(&o_g[grp][q][8 * vl]) = make_float4(o[q][0], o[q][1], o[q][2], o[q][3]);
    *reinterpret_cast<float4 *>(&o_g[grp][q][8 * vl + 4]) = make_float4(o[q][4], o[q][5], o[q][6], o[q][7]);
  }
  lds_barrier();

  // (6) the waves combined (factor 2^(m_w - M), 0 for a wave without positions), lane groups summed in
  // a fixed order
  const size_t slot = ((size_t)b * a.kv + j) * (size_t)a.nch;
  for (int idx = tid; idx < G * D; idx += NW * 64) {
    const int q = idx / D, d = idx % D;
    float M = m_s[0][q];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, m_s[w][q]);
    float acc = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = (m_s[w][q] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_s[w][q] - M);
      float ow = 0.f;
#pragma unroll
      for (int g2 = 0; g2 < PPI; ++g2) ow += o_g[w * PPI + g2][q][d];
      acc = fmaf(f, ow, acc);
      L = fmaf(f, l_s[w][q], L);
    }
    if (a.direct) {
      put_out(a, b, j * G * D + idx, acc / L);
    } else if (SELF) {
      store_dev(&a.part_o[(slot + c) * (size_t)(G * D) + idx], acc);
      if (d == 0) {
        store_dev(&a.part_ml[(slot + c) * (size_t)(G * 2) + 2 * q], M);
        store_dev(&a.part_ml[(slot + c) * (size_t)(G * 2) + 2 * q + 1], L);
      }
    } else {
      a.part_o[(slot + c) * (size_t)(G * D) + idx] = acc;
      if (d == 0) {
        a.part_ml[(slot + c) * (size_t)(G * 2) + 2 * q] = M;
        a.part_ml[(slot + c) * (size_t)(G * 2) + 2 * q + 1] = L;
      }
    }
  }
  if (SELF && !a.direct) finish_chunk_merge<G, D>(a, b, j, nact, slot);
}

// Merge of the chunk partials of one (row, kv head), in chunk order (a separate launch: the kernel
// boundary makes the partials visible without cache-wide fences inside the attention kernel).
// Block (og, j, b) produces 64 consecutive outputs of query head i = og*64/head of group j:
// M = max_c m_c, w_c = exp(m_c - M), L = sum_c w_c l_c, o = (sum_c w_c o_c) / L.  The NW waves are NW
// chunk groups x 64 outputs (wave w takes chunks w, w + NW, ...); their sums are combined in a fixed
// order.  Every load is issued before the first use: NW * PER chunks in one memory round trip (NW = 16
// for one long row: 512 chunks took 34 us per layer in 8 rounds with 4 waves, 6.7 us in one with 16).
template <int G, int D, int NW>
__global__ __launch_bounds__(NW * 64) void k_attn_merge(AttnArgs a, int chunk) {
  constexpr int NT = NW * 64;
  constexpr int PER = NW >= 16 ? 32 : 16;  // partials per thread loaded up front; more in a loop
  constexpr int MLR = (kAttnMaxChunks + NT - 1) / NT;
  const int og = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int t = a.pos[b];
  const int nact = t / chunk + 1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = (og * 64) / D, d = (og * 64) % D + lane;
  __shared__ float w_s[kAttnMaxChunks];
  __shared__ float red[NW];
  __shared__ float acc_s[NW][64];
  const size_t slot = ((size_t)b * a.kv + j) * (size_t)a.nch;
  const float *pml0 = a.part_ml + slot * (size_t)(G * 2);
  const float *po0 = a.part_o + slot * (size_t)(G * D);
  // every load first: this thread's (m, l) of chunks tid, tid + NT, ... and its output's partial o of
  // chunks wave, wave + NW, ... (independent of the maxima: one memory round trip)
  float mv[MLR], lv[MLR];
#pragma unroll
  for (int k = 0; k < MLR; ++k) {
    const int cc = min(tid + k * NT, nact - 1);
    mv[k] = pml0[(size_t)cc * G * 2 + 2 * i];
    lv[k] = pml0[(size_t)cc * G * 2 + 2 * i + 1];
  }
  // (unconditional loads, chunks past the last clamped to it and unused: a load behind a branch would make
  // the wait counter hold the later loads until it lands, two round trips instead of one)
  float ov[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int cc = min(wave + NW * k, nact - 1);
    ov[k] = po0[(size_t)cc * G * D + i * D + d];
  }
  float M = -INFINITY;
#pragma unroll
  for (int k = 0; k < MLR; ++k)
    if (tid + k * NT < nact) M = fmaxf(M, mv[k]);
  M = wave_max(M);
  if (lane == 0) red[wave] = M;
  lds_barrier();
  M = red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) M = fmaxf(M, red[w]);
  lds_barrier();
  float L = 0.f;
#pragma unroll
  for (int k = 0; k < MLR; ++k) {
    const int cc = tid + k * NT;
    if (cc < nact) {
      const float w = __builtin_amdgcn_exp2f(mv[k] - M);  // maxima are in base 2
      w_s[cc] = w;
      L = fmaf(w, lv[k], L);
    }
  }
  L = wave_sum(L);
  if (lane == 0) red[wave] = L;
  lds_barrier();
  {
    float s2 = red[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) s2 += red[w];
    L = s2;
  }
  float acc = 0.f;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int cc = wave + NW * k;
    if (cc < nact) acc = fmaf(w_s[cc], ov[k], acc);
  }
  for (int base = NW * PER; base < nact; base += NW * PER) {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int cc = base + wave + NW * k;
      if (cc < nact) acc = fmaf(w_s[cc], po0[(size_t)cc * G * D + i * D + d], acc);
    }
  }
  acc_s[wave][lane] = acc;
  lds_barrier();
  if (wave == 0) {
    float sum = acc_s[0][lane];
#pragma unroll
    for (int w = 1; w < NW; ++w) sum += acc_s[w][lane];
    put_out(a, b, (j * G + i) * D + d, sum / L);
  }
}

// positions per wavefront of the matrix-core kernel: 64 (chunks of 256) measured faster than 32 or 128
// for both one row at 8K positions and 32 rows at 8K..32K
constexpr int kMfmaNpw = 64;
template <typename KT, int D, int G>
constexpr bool use_mfma() {
  return sizeof(KT) == 2 && MfmaAttnShape<D, G, kMfmaNpw>::LDS <= 64 * 1024;
}
template <typename KT, int D, int G>
constexpr int chunk_of() {
  if constexpr (use_mfma<KT, D, G>())
    return MfmaAttnShape<D, G, kMfmaNpw>::CHUNK;
  else
    return AttnShape<KT, D>::CHUNK;
}
template <typename KT, int D>
static int chunk_d(int g) {
  switch (g) {
    case 1: return chunk_of<KT, D, 1>();
    case 2: return chunk_of<KT, D, 2>();
    case 3: return chunk_of<KT, D, 3>();
    case 4: return chunk_of<KT, D, 4>();
    case 8: return chunk_of<KT, D, 8>();
  }
  return AttnShape<KT, D>::CHUNK;
}

int attention_chunk(int kvdtype, int head, int g) {
  if (kvdtype == LLAMA_BF16) return head == 64 ? chunk_d<bf16_t, 64>(g) : chunk_d<bf16_t, 128>(g);
  return head == 64 ? chunk_d<float, 64>(g) : chunk_d<float, 128>(g);
}

int attention_paged_supported(int kvdtype, int head, int g) {
  if (kvdtype != LLAMA_BF16 || !attention_supported(head, g)) return 0;
  auto ok = [](auto d, int gg) {
    constexpr int D = decltype(d)::value;
    switch (gg) {
      case 1: return use_mfma<bf16_t, D, 1>();
      case 2: return use_mfma<bf16_t, D, 2>();
      case 3: return use_mfma<bf16_t, D, 3>();
      case 4: return use_mfma<bf16_t, D, 4>();
      case 8: return use_mfma<bf16_t, D, 8>();
    }
    return false;
  };
  return head == 64 ? ok(std::integral_constant<int, 64>{}, g) : ok(std::integral_constant<int, 128>{}, g);
}

int attention_supported(int head, int g) {
  return (head == 64 || head == 128) && (g == 1 || g == 2 || g == 3 || g == 4 || g == 8);
}

// One attention launch (+ the merge when more than one chunk): chunks of `chunk` positions cover 0..tmax.
template <typename KT, int D, int G>
static hipError_t launch_g(AttnArgs a, int B, int tmax, hipStream_t s) {
  constexpr int chunk = chunk_of<KT, D, G>();
  const int nch_launch = tmax / chunk + 1;
  if (nch_launch > a.nch || nch_launch > kAttnMaxChunks) return hipErrorInvalidValue;
  const dim3 grid(nch_launch, a.kv, B);
  a.direct = (nch_launch == 1);
  const bool merge = !a.direct;
  // Small merges (few chunks x few outputs per (row, kv head)) run in the attention kernel's last block
  // per (row, kv head): measured faster than a separate launch for the 1.7B shape (8 chunks x 64 outputs:
  // 7.4 vs 10.0 us per layer), slower for the 8B shape at 8K positions (32 x 512: 16.3 vs 14.6 us) and
  // for 32 long rows.
  const bool self = merge && (long)nch_launch * G * D <= 4096;
  if constexpr (use_mfma<KT, D, G>()) {
    // keys as whole rows (through LDS) pay off when the launch streams many blocks per CU; a launch of
    // about one block per CU finishes sooner with the keys loaded straight in the MFMA layout, and with
    // 8 wavefronts of 32 positions rather than 4 of 64 (same chunk; one row at 8K: 14.4 vs 14.6 us per
    // layer with the merge)
    const bool krows = (long)B * a.kv * nch_launch >= 4096;
    if (krows && self) launch(k_attn_mfma<D, G, kMfmaNpw, true, true>, grid, dim3(kThreads), s, true, true, a);
    if (krows && !self) launch(k_attn_mfma<D, G, kMfmaNpw, true, false>, grid, dim3(kThreads), s, true, !merge, a);
    if (!krows && self) launch(k_attn_mfma<D, G, kMfmaNpw, false, true>, grid, dim3(kThreads), s, true, true, a);
    if (!krows && !self) launch(k_attn_mfma<D, G, kMfmaNpw / 2, false, false, 8>, grid, dim3(8 * 64), s, true, !merge, a);
  } else {
    if (self)
      launch(k_attn<KT, D, G, true>, grid, dim3(kThreads), s, true, true, a);
    else
      launch(k_attn<KT, D, G, false>, grid, dim3(kThreads), s, true, !merge, a);
  }
  if (merge && !self) {
    // 16 waves only when the merge has fewer blocks than the chip has CUs (one row): at 32 rows (2048
    // blocks of ~125 chunks) the 4-wave blocks were faster (11.8 vs 30.4 us per layer)
    const dim3 mg(G * D / 64, a.kv, B);
    if (nch_launch > 64 && (long)mg.x * mg.y * mg.z < 256)
      launch(k_attn_merge<G, D, 16>, mg, dim3(16 * 64), s, false, true, a, chunk);
    else
      launch(k_attn_merge<G, D, 4>, mg, dim3(kThreads), s, false, true, a, chunk);
  }
  return hipGetLastError();
}

template <typename KT, int D>
static hipError_t launch_d(int g, const AttnArgs &a, int B, int tmax, hipStream_t s) {
  switch (g) {
    case 1: return launch_g<KT, D, 1>(a, B, tmax, s);
    case 2: return launch_g<KT, D, 2>(a, B, tmax, s);
    case 3: return launch_g<KT, D, 3>(a, B, tmax, s);
    case 4: return launch_g<KT, D, 4>(a, B, tmax, s);
    case 8: return launch_g<KT, D, 8>(a, B, tmax, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attention(int kvdtype, int head, int g, const AttnArgs &a, int B, int tmax, hipStream_t s) {
  if (kvdtype == LLAMA_BF16) {
    if (head == 64) return launch_d<bf16_t, 64>(g, a, B, tmax, s);
    if (head == 128) return launch_d<bf16_t, 128>(g, a, B, tmax, s);
  } else {
    if (head == 64) return launch_d<float, 64>(g, a, B, tmax, s);
    if (head == 128) return launch_d<float, 128>(g, a, B, tmax, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace lm
