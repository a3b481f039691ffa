// Attention device code shared by the attention kernels and by the launch that runs the q/k/v product
// together with the attention: the block shapes, the tails that turn loaded keys and values into a
// chunk's partial (vector units: valu_attend; matrix cores: mfma_attend) and the in-kernel merge of the
// chunks (finish_chunk_merge).  What the kernels compute is described at the top of attention.hip.
#pragma once

#include "common.h"

namespace lm {

// One normalised output o of row b at column col (of the row's dim outputs), and, when asked, its
// operand split for the batched O product (the bits k_split would give: hi = bf16(o) to nearest even,
// lo = bf16(o - hi))
__device__ __forceinline__ void put_out(const AttnArgs &a, int b, int col, float v, uint32_t tag = 0u) {
  a.out[(size_t)b * a.out_stride + col] = v;
  if (a.out_t) tagged_store(a.out_t + col, v, tag);
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
__device__ void finish_chunk_merge(const AttnArgs &a, int b, int j, int nact, size_t slot, uint32_t tag = 0u) {
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
      put_out(a, b, j * G * D + idx, acc[i] / L, tag);
    }
  }
  if (tid == 0) __hip_atomic_store(&a.done[b * a.kv + j], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// How a chunk's result leaves the block when the positions take several chunks: plain stores of the
// partial for a separate merge launch, or device-scope stores and the merge in the last block of the kv
// head (finish_chunk_merge).
enum { kMergePlain = 0, kMergeSelf = 1 };

// A chunk's result for output idx (query head q, number d) of (row b, kv head j) in the merge mode.
template <int G, int D, int MODE>
__device__ __forceinline__ void emit_chunk(const AttnArgs &a, int b, int j, int c, size_t slot, int idx, int q, int d,
                                           float acc, float M, float L, uint32_t tag = 0u) {
  if (a.direct) {
    put_out(a, b, j * G * D + idx, acc / L, tag);
  } else if (MODE == kMergeSelf) {
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

// after every output of the chunk is emitted: the merge, where this block takes part in it
template <int G, int D, int MODE>
__device__ __forceinline__ void finish_chunk(const AttnArgs &a, int b, int j, int nact, size_t slot,
                                             uint32_t tag = 0u) {
  if (a.direct) return;
  if (MODE == kMergeSelf) finish_chunk_merge<G, D>(a, b, j, nact, slot, tag);
}

// Everything after the loads of k_attn: this thread's slices of the group's query heads from q_s (LDS,
// published by the caller's barrier), the scores of its positions, the softmax pieces per wavefront,
// the position groups combined in a fixed order into the chunk's partial (or, with one chunk, the
// output).
template <typename KT, int D, int G, int MODE>
__device__ __forceinline__ void valu_attend(const AttnArgs &a, int c, int j, int b, int t, int nact,
                                            const float (&q_s)[G][D], const u32x4 (&kraw)[AttnShape<KT, D>::NR],
                                            const u32x4 (&vraw)[AttnShape<KT, D>::NR], uint32_t tag = 0u) {
  using S = AttnShape<KT, D>;
  constexpr int E = S::E, LPR = S::LPR, PPR = S::PPR, NR = S::NR, CHUNK = S::CHUNK;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = tid % LPR, grp = tid / LPR;
  const int p0 = c * CHUNK;
  const int p1 = min(p0 + CHUNK, t + 1);

  __shared__ float m_s[4][G];
  __shared__ float l_g[kThreads / LPR][G];
  __shared__ float o_g[kThreads / LPR][G][D];

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
    emit_chunk<G, D, MODE>(a, b, j, c, slot, idx, i, d, acc, M, L, tag);
  }
  finish_chunk<G, D, MODE>(a, b, j, nact, slot, tag);
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

// Everything after the loads, for one wavefront's NPW positions starting at pw0 of chunk c of (row b,
// kv head j): scores on the matrix cores from the query fragments (qhi, qlo) and the keys (getk(gi, kf)
// supplies 16-key group gi in the B layout), the softmax pieces, the weighted V sum on the vector units,
// then the NW waves combined in a fixed order into the chunk's partial (or, with one chunk, the output).
// vt / vti (optional): this lane's value row vti is taken from vt (F32 values that are bf16 numbers)
// instead of vr[vti], at its use, so a load still in flight into vr is not waited for earlier.
template <int D, int G, int NPW, int NW, int MODE, typename GetK>
__device__ __forceinline__ void mfma_attend(const AttnArgs &a, int c, int j, int b, int t, int nact, int pw0,
                                            const u32x4 (&qhi)[D / 32], const u32x4 (&qlo)[D / 32], GetK getk,
                                            const u32x4 (&vr)[NPW / (64 / (D / 8))],
                                            const float *vt = nullptr, int vti = -1, uint32_t tag = 0u) {
  using S = MfmaAttnShape<D, G, NPW, NW>;
  constexpr int CHUNK = S::CHUNK, NGI = S::NGI, KS = S::KS, LPR = S::LPR, PPI = S::PPI, NV = S::NV;
  constexpr int GP = S::GP, NG = S::NG;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qrow = lane & 15;
  const int vl = lane % LPR, vg = lane / LPR;
  const int p1 = min(c * CHUNK + CHUNK, t + 1);

  __shared__ __attribute__((aligned(16))) float p_s[NW][NPW][GP];
  __shared__ float m_s[NW][G], l_s[NW][G];
  __shared__ __attribute__((aligned(16))) float o_g[NG][G][D];

  // (3) scores, base 2: s2 = (q . k) * scale * log2 e; lane holds head 4(lane/16) + r, position
  // pw0 + 16 gi + lane%16
  const float scale2 = a.scale * 1.4426950408889634f;
  float sc[NGI][4];
#pragma unroll
  for (int gi = 0; gi < NGI; ++gi) {
    u32x4 kf[KS];
    getk(gi, kf);
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
  // the weights are read back by the wave that wrote them (m_s and l_s only after the barrier below)
  wave_lds_barrier();

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
    if (vt && i == vti) load_f32<8>(vt + 8 * vl, vf);
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
    emit_chunk<G, D, MODE>(a, b, j, c, slot, idx, q, d, acc, M, L, tag);
  }
  finish_chunk<G, D, MODE>(a, b, j, nact, slot, tag);
}

// query fragments: lane l holds head l%16 (zero rows from G on), numbers 32 ks + 8(l/16) .. +8, as
// bf16 hi + lo
template <int D, int G>
__device__ __forceinline__ void q_fragments(const float (&f)[D / 32][8], int qrow, u32x4 (&qhi)[D / 32],
                                            u32x4 (&qlo)[D / 32]) {
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = qrow < G ? f[ks][e] : 0.f;
    split8(v, qhi[ks], qlo[ks]);
  }
}

}  // namespace lm
