// Causal grouped-query decode attention on gfx950, with RoPE and the KV-cache append fused in.
//
// What it computes (main.bend "Grouped-query attention over the arrays", head_att / group_att /
// attention; nest attention.linnet `decode` / `decode_rows`): for cache row b at position t, query
// head h = j*g + i reads key/value head j (gqa_head); scores s_p = (q_h . K_j[p]) * (1/sqrt(head)) for
// p = 0..t exactly (causal / read_len), softmax over them, o_h = sum_p w_p V_j[p].  Before that, the
// position's rotated key and its value are written at slot t of head j (KV.push): RoPE pairs number i
// with number i + half of a head, lo' = lo*c - hi*s, hi' = hi*c + lo*s (rot_lo / rot_hi), each product
// and sum rounded on its own; bf16 caches round to nearest even.  The position-t key and value that
// the scores use are the stored (rounded) ones, as a cache read would give.
//
// Work split (split-K over positions): block (c, j, b) takes chunk c of `chunk` positions of row b's
// head j and all g query heads of the group, so each K/V byte is read from HBM once for g heads.
// 256 threads = 256/LPR position groups of LPR lanes, LPR lanes covering one 16-byte slice each of a
// head row (head*bytes/16 lanes), so every load instruction of a wave reads whole contiguous rows.
// Every K and V load of a thread (8 rows each) is issued before any is used.  The query heads, the
// cos/sin row and the appended key/value are staged once per block in LDS.  Each wavefront keeps its
// scores in registers and forms its own softmax pieces (max, exp-sum, exp-weighted V sum) with
// cross-lane permutes; the 4 wavefronts are combined through LDS.  Each chunk writes an unnormalised
// partial (o, m, l); a second small kernel merges the chunks of each (row, kv head) in chunk order,
// so results do not depend on block timing.  When one chunk covers every row's positions the
// attention kernel normalises directly and no merge runs.
#include "common.h"

namespace lm {

template <typename KT>
struct KvStore;
template <>
struct KvStore<float> {
  __device__ __forceinline__ static float round_store(float *p, float v) {
    *p = v;
    return v;
  }
};
template <>
struct KvStore<bf16_t> {
  __device__ __forceinline__ static float round_store(bf16_t *p, float v) {
    const uint16_t b = f32_to_bf16(v);
    *p = b;
    return bf16_to_f32(b);
  }
};

template <typename KT, int D>
struct AttnShape {
  static constexpr int E = Vec16<KT>::E;      // elements per 16-byte slice
  static constexpr int LPR = D / E;           // lanes per head row
  static constexpr int PPR = kThreads / LPR;  // positions per round
  static constexpr int NR = 8;                // rounds per thread: every K and V load issued up front
  static constexpr int CHUNK = NR * PPR;      // positions per block
};

template <typename KT, int D, int G>
__global__ __launch_bounds__(kThreads) void k_attn(AttnArgs a) {
  using S = AttnShape<KT, D>;
  constexpr int E = S::E, LPR = S::LPR, PPR = S::PPR, NR = S::NR, CHUNK = S::CHUNK;
  static_assert(LPR >= 1 && LPR <= 64 && (64 % LPR) == 0, "row must fit a wavefront");
  constexpr int HALF = D / 2;
  const int c = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int t = a.pos[b];
  const int nact = t / CHUNK + 1;  // chunks covering 0..t
  if (c >= nact) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = tid % LPR, grp = tid / LPR;
  const int p0 = c * CHUNK;
  const int p1 = min(p0 + CHUNK, t + 1);
  const bool owner = (c == nact - 1);

  __shared__ float q_s[G][D];                // raw query heads of the group
  __shared__ float cs_s[HALF], sn_s[HALF];   // cos / sin of position t
  __shared__ float kr_s[D], vr_s[D];         // raw key / value of kv head j at t (owner block)
  __shared__ float kt_s[D], vt_s[D];         // the appended key (rotated) and value, as stored
  __shared__ float m_s[4][G];
  __shared__ float l_g[kThreads / LPR][G];
  __shared__ float o_g[kThreads / LPR][G][D];

  const size_t head_off = ((size_t)(a.row0 + b) * a.kv + j) * (size_t)a.max_seq * D;
  KT *Kh = reinterpret_cast<KT *>(a.kc) + head_off;
  KT *Vh = reinterpret_cast<KT *>(a.vc) + head_off;
  const float *qkv = a.qkv + (size_t)b * a.qkv_stride;
  const int dim = a.kv * G * D;

  // (1) small inputs, once per block, as 16-byte units: units [0, NQ) the query heads, [NQ, NQ+NC) the
  // cos/sin slices, then (owner block) the raw key and value of head j.  A thread takes units tid and
  // tid + 256.
  constexpr int NQ = G * D / 4, NC = HALF / 4, NK = D / 4, NU = NQ + NC + NK;
  static_assert(NU <= 2 * kThreads, "two staging units per thread");
  float4 sm[2][2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int u = tid + k * kThreads;
    sm[k][0] = sm[k][1] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (u < NQ) {
      sm[k][0] = *reinterpret_cast<const float4 *>(qkv + (size_t)j * G * D + u * 4);
    } else if (u < NQ + NC) {
      sm[k][0] = *reinterpret_cast<const float4 *>(a.rope_cs + (size_t)t * HALF + (u - NQ) * 4);
      sm[k][1] = *reinterpret_cast<const float4 *>(a.rope_sn + (size_t)t * HALF + (u - NQ) * 4);
    } else if (owner && u < NU) {
      const int w = u - NQ - NC;
      sm[k][0] = *reinterpret_cast<const float4 *>(qkv + dim + (size_t)j * D + w * 4);
      sm[k][1] = *reinterpret_cast<const float4 *>(qkv + dim + (size_t)a.kv * D + (size_t)j * D + w * 4);
    }
  }

  // (2) every K and V row of this thread's positions, in flight together.  Loads are unconditional: a
  // position at or after t reads row min(p, t - 1) (row 0 when t = 0), which is inside the cache, and
  // its value is never used (position t comes from this step's append).
  u32x4 kraw[NR], vraw[NR];
  const int plast = t > 0 ? t - 1 : 0;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int p = min(p0 + r * PPR + grp, plast);
    kraw[r] = load_stream16(Kh + (size_t)p * D + li * E);
    vraw[r] = load_stream16(Vh + (size_t)p * D + li * E);
  }

#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int u = tid + k * kThreads;
    if (u < NQ) {
      *reinterpret_cast<float4 *>(&q_s[0][0] + u * 4) = sm[k][0];
    } else if (u < NQ + NC) {
      *reinterpret_cast<float4 *>(cs_s + (u - NQ) * 4) = sm[k][0];
      *reinterpret_cast<float4 *>(sn_s + (u - NQ) * 4) = sm[k][1];
    } else if (owner && u < NU) {
      const int w = u - NQ - NC;
      *reinterpret_cast<float4 *>(kr_s + w * 4) = sm[k][0];
      *reinterpret_cast<float4 *>(vr_s + w * 4) = sm[k][1];
    }
  }
  lds_barrier();

  // (3) the owner appends position t: the rotated key (rot_lo / rot_hi) and the value, rounded as
  // stored; the scores use the stored values
  if (owner && tid < D) {
    const int d = tid, ic = d < HALF ? d : d - HALF;
    const float partner = d < HALF ? -kr_s[d + HALF] : kr_s[d - HALF];
    const float kr = rope_pair(kr_s[d], partner, cs_s[ic], sn_s[ic]);
    kt_s[d] = KvStore<KT>::round_store(Kh + (size_t)t * D + d, kr);
    vt_s[d] = KvStore<KT>::round_store(Vh + (size_t)t * D + d, vr_s[d]);
  }
  // rotated query slices [li*E, li*E + E) of the g heads
  const int d0 = li * E;
  const int dp = d0 < HALF ? d0 + HALF : d0 - HALF;
  const int ic0 = d0 < HALF ? d0 : d0 - HALF;
  const float sgn = d0 < HALF ? -1.f : 1.f;
  float q[G][E];
#pragma unroll
  for (int i = 0; i < G; ++i)
#pragma unroll
    for (int e = 0; e < E; ++e) q[i][e] = rope_pair(q_s[i][d0 + e], sgn * q_s[i][dp + e], cs_s[ic0 + e], sn_s[ic0 + e]);
  if (owner) {
    lds_barrier();  // kt_s / vt_s
    // the position-t row comes from this step's append: put its stored bits where a cache load would
    // have put them, so every round takes the same path
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      if (p0 + r * PPR + grp == t) {
        kraw[r] = Vec16<KT>::pack(&kt_s[d0]);
        vraw[r] = Vec16<KT>::pack(&vt_s[d0]);
      }
    }
  }

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
      a.out[(size_t)b * a.out_stride + (size_t)(j * G) * D + idx] = acc / L;
    } else {
      a.part_o[(slot + c) * (size_t)(G * D) + idx] = acc;
      if (d == 0) {
        a.part_ml[(slot + c) * (size_t)(G * 2) + 2 * i] = M;
        a.part_ml[(slot + c) * (size_t)(G * 2) + 2 * i + 1] = L;
      }
    }
  }
}

// Merge of the chunk partials of one (row, kv head), in chunk order (a separate launch: the kernel
// boundary makes the partials visible without cache-wide fences inside the attention kernel).
// Block (og, j, b) produces 64 consecutive outputs of query head i = og*64/head of group j:
// M = max_c m_c, w_c = exp(m_c - M), L = sum_c w_c l_c, o = (sum_c w_c o_c) / L.  The 256 threads are
// 4 chunk groups x 64 outputs; the 4 groups' sums are combined in a fixed order.
template <int G, int D>
__global__ __launch_bounds__(kThreads) void k_attn_merge(AttnArgs a, int chunk) {
  constexpr int PER = 16;  // partials per thread loaded up front (chunks 0..63); more in a loop
  const int og = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int t = a.pos[b];
  const int nact = t / chunk + 1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = (og * 64) / D, d = (og * 64) % D + lane;
  __shared__ float w_s[kAttnMaxChunks];
  __shared__ float red[4];
  __shared__ float acc_s[4][64];
  const size_t slot = ((size_t)b * a.kv + j) * (size_t)a.nch;
  const float *pml0 = a.part_ml + slot * (size_t)(G * 2);
  const float *po0 = a.part_o + slot * (size_t)(G * D);
  // every load first: this thread's (m, l) of chunks tid, tid + 256 and its output's partial o of
  // chunks wave, wave + 4, ..., wave + 60 (independent of the maxima: one memory round trip)
  float mv[2], lv[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int cc = min(tid + k * kThreads, nact - 1);
    mv[k] = pml0[(size_t)cc * G * 2 + 2 * i];
    lv[k] = pml0[(size_t)cc * G * 2 + 2 * i + 1];
  }
  float ov[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int cc = wave + 4 * k;
    if (cc < nact) ov[k] = po0[(size_t)cc * G * D + i * D + d];
  }
  float M = -INFINITY;
#pragma unroll
  for (int k = 0; k < 2; ++k)
    if (tid + k * kThreads < nact) M = fmaxf(M, mv[k]);
  M = wave_max(M);
  if (lane == 0) red[wave] = M;
  lds_barrier();
  M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  lds_barrier();
  float L = 0.f;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int cc = tid + k * kThreads;
    if (cc < nact) {
      const float w = __builtin_amdgcn_exp2f(mv[k] - M);  // maxima are in base 2
      w_s[cc] = w;
      L = fmaf(w, lv[k], L);
    }
  }
  L = wave_sum(L);
  if (lane == 0) red[wave] = L;
  lds_barrier();
  L = (red[0] + red[1]) + (red[2] + red[3]);
  float acc = 0.f;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int cc = wave + 4 * k;
    if (cc < nact) acc = fmaf(w_s[cc], ov[k], acc);
  }
  for (int base = 4 * PER; base < nact; base += 4 * PER) {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int cc = base + wave + 4 * k;
      if (cc < nact) acc = fmaf(w_s[cc], po0[(size_t)cc * G * D + i * D + d], acc);
    }
  }
  acc_s[wave][lane] = acc;
  lds_barrier();
  if (wave == 0) {
    const float sum = (acc_s[0][lane] + acc_s[1][lane]) + (acc_s[2][lane] + acc_s[3][lane]);
    a.out[(size_t)b * a.out_stride + (size_t)(j * G + i) * D + d] = sum / L;
  }
}

int attention_chunk(int kvdtype, int head) {
  if (kvdtype == LLAMA_BF16) return head == 64 ? AttnShape<bf16_t, 64>::CHUNK : AttnShape<bf16_t, 128>::CHUNK;
  return head == 64 ? AttnShape<float, 64>::CHUNK : AttnShape<float, 128>::CHUNK;
}

int attention_supported(int head, int g) {
  return (head == 64 || head == 128) && (g == 1 || g == 2 || g == 3 || g == 4 || g == 8);
}

template <typename KT, int D>
static hipError_t launch_d(int g, const AttnArgs &a, dim3 grid, bool merge, hipStream_t s) {
  const int chunk = AttnShape<KT, D>::CHUNK;
  switch (g) {
#define CASE(G)                                                                                     \
  case G:                                                                                           \
    launch(k_attn<KT, D, G>, grid, dim3(kThreads), s, true, !merge, a);                             \
    if (merge) launch(k_attn_merge<G, D>, dim3(G * D / 64, grid.y, grid.z), dim3(kThreads), s, false, \
                      true, a, chunk);                                                              \
    break;
    CASE(1) CASE(2) CASE(3) CASE(4) CASE(8)
#undef CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attention(int kvdtype, int head, int g, AttnArgs a, int B, int nch_launch, hipStream_t s) {
  if (nch_launch > a.nch || nch_launch > kAttnMaxChunks) return hipErrorInvalidValue;
  const dim3 grid(nch_launch, a.kv, B);
  a.direct = (nch_launch == 1);
  const bool merge = !a.direct;
  if (kvdtype == LLAMA_BF16) {
    if (head == 64) return launch_d<bf16_t, 64>(g, a, grid, merge, s);
    if (head == 128) return launch_d<bf16_t, 128>(g, a, grid, merge, s);
  } else {
    if (head == 64) return launch_d<float, 64>(g, a, grid, merge, s);
    if (head == 128) return launch_d<float, 128>(g, a, grid, merge, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace lm
