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
// Every K and V load of a thread (8 rows each) is issued before any is used.  Scores go to LDS; per head
// the chunk max and exp-sum; then the exp-weighted V sum.  Each chunk writes an unnormalised partial
// (o, m, l); a second small kernel merges the chunks of each (row, kv head) in chunk order, so results
// do not depend on block timing.  When one chunk covers every row's positions the attention kernel
// normalises directly and no merge runs.
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
  const int c = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int t = a.pos[b];
  const int nact = t / CHUNK + 1;  // chunks covering 0..t
  if (c >= nact) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = tid % LPR, grp = tid / LPR;
  const int p0 = c * CHUNK;
  const int p1 = min(p0 + CHUNK, t + 1);
  const int half = a.half;

  __shared__ float s_sc[G][CHUNK];
  __shared__ float kt_s[D], vt_s[D];
  __shared__ float m_s[G], l_s[G];
  __shared__ float o_s[4][G][D];

  const size_t head_off = ((size_t)(a.row0 + b) * a.kv + j) * (size_t)a.max_seq * D;
  KT *Kh = reinterpret_cast<KT *>(a.kc) + head_off;
  KT *Vh = reinterpret_cast<KT *>(a.vc) + head_off;
  const float *qkv = a.qkv + (size_t)b * a.qkv_stride;
  const int dim = a.kv * G * D;
  const float *cs = a.rope_cs + (size_t)t * half;
  const float *sn = a.rope_sn + (size_t)t * half;

  // (1) the small inputs first, so that waiting for them does not wait for the K/V stream: this lane's
  // query slices [li*E, li*E + E) of the g heads and the slices half a head away, the cos/sin slice,
  // and (for the append) the raw key/value slices of kv head j
  const int d0 = li * E;                      // first number of this lane's slice
  const int dp = d0 < half ? d0 + half : d0 - half;  // partner slice
  const int ic = d0 < half ? d0 : d0 - half;  // frequency index of the slice
  const float sgn = d0 < half ? -1.f : 1.f;
  float qo[G][E], qp[G][E], cv[E], sv[E], ko[E], kp[E], vo[E];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const float *qh = qkv + (size_t)(j * G + i) * D;
    load_f32(qh + d0, qo[i]);
    load_f32(qh + dp, qp[i]);
  }
  load_f32(cs + ic, cv);
  load_f32(sn + ic, sv);
  const bool owner = (c == nact - 1);
  const float *kh = qkv + dim + (size_t)j * D;
  const float *vh = qkv + dim + (size_t)a.kv * D + (size_t)j * D;
  if (owner && grp == 0) {
    load_f32(kh + d0, ko);
    load_f32(kh + dp, kp);
    load_f32(vh + d0, vo);
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

  // (3) rotated query slices (rot_lo / rot_hi)
  float q[G][E];
#pragma unroll
  for (int i = 0; i < G; ++i)
#pragma unroll
    for (int e = 0; e < E; ++e) q[i][e] = rope_pair(qo[i][e], sgn * qp[i][e], cv[e], sv[e]);

  // (4) the block whose chunk holds t appends this position's rotated key and its value (lanes of the
  // first position group, one slice each); the scores read them back from LDS as stored
  if (owner && grp == 0) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float kr = rope_pair(ko[e], sgn * kp[e], cv[e], sv[e]);
      kt_s[d0 + e] = KvStore<KT>::round_store(Kh + (size_t)t * D + d0 + e, kr);
      vt_s[d0 + e] = KvStore<KT>::round_store(Vh + (size_t)t * D + d0 + e, vo[e]);
    }
  }
  lds_barrier();

  // ---- scores of positions p0..p1-1, scaled after the dot product
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int p = p0 + r * PPR + grp;
    float kf[E];
    if (p < t) {
      Vec16<KT>::unpack(kraw[r], kf);
    } else if (p == t) {
#pragma unroll
      for (int e = 0; e < E; ++e) kf[e] = kt_s[li * E + e];
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) kf[e] = 0.f;
    }
    float s[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) acc = fmaf(q[i][e], kf[e], acc);
      s[i] = group_sum<LPR>(acc);
    }
    if (li == 0 && p < p1) {
#pragma unroll
      for (int i = 0; i < G; ++i) s_sc[i][r * PPR + grp] = a.scale * s[i];
    }
  }
  lds_barrier();

  // ---- per head over this chunk: max, exp(s - max), their sum
  const int n = p1 - p0;
  for (int i = wave; i < G; i += 4) {
    float m = -INFINITY;
    for (int p = lane; p < n; p += 64) m = fmaxf(m, s_sc[i][p]);
    m = wave_max(m);
    float l = 0.f;
    for (int p = lane; p < n; p += 64) {
      const float e = expf(s_sc[i][p] - m);
      s_sc[i][p] = e;
      l += e;
    }
    l = wave_sum(l);
    if (lane == 0) {
      m_s[i] = m;
      l_s[i] = l;
    }
  }
  lds_barrier();

  // ---- sum_p e_p V[p]
  float o[G][E];
#pragma unroll
  for (int i = 0; i < G; ++i)
#pragma unroll
    for (int e = 0; e < E; ++e) o[i][e] = 0.f;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int p = p0 + r * PPR + grp;
    if (p < p1) {
      float vf[E];
      if (p < t) {
        Vec16<KT>::unpack(vraw[r], vf);
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) vf[e] = vt_s[li * E + e];
      }
#pragma unroll
      for (int i = 0; i < G; ++i) {
        const float w = s_sc[i][r * PPR + grp];
#pragma unroll
        for (int e = 0; e < E; ++e) o[i][e] = fmaf(w, vf[e], o[i][e]);
      }
    }
  }
  // position groups inside a wavefront, then the 4 wavefronts
#pragma unroll
  for (int i = 0; i < G; ++i)
#pragma unroll
    for (int e = 0; e < E; ++e) o[i][e] = strided_sum<LPR>(o[i][e]);
  if (lane < LPR) {
#pragma unroll
    for (int i = 0; i < G; ++i)
#pragma unroll
      for (int e = 0; e < E; ++e) o_s[wave][i][li * E + e] = o[i][e];
  }
  lds_barrier();

  const int o_base = (j * G) * D;
  if (a.direct) {
    // a single chunk covers 0..t (every row of the launch): normalise here, no merge pass
    for (int idx = tid; idx < G * D; idx += kThreads) {
      const int i = idx / D, d = idx % D;
      const float sum = (o_s[0][i][d] + o_s[1][i][d]) + (o_s[2][i][d] + o_s[3][i][d]);
      a.out[(size_t)b * a.out_stride + o_base + idx] = sum / l_s[i];
    }
    return;
  }
  const size_t slot = ((size_t)b * a.kv + j) * (size_t)a.nch;
  float *po = a.part_o + (slot + c) * (size_t)(G * D);
  float *pml = a.part_ml + (slot + c) * (size_t)(G * 2);
  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int i = idx / D, d = idx % D;
    po[idx] = (o_s[0][i][d] + o_s[1][i][d]) + (o_s[2][i][d] + o_s[3][i][d]);
  }
  if (tid < G) {
    pml[2 * tid] = m_s[tid];
    pml[2 * tid + 1] = l_s[tid];
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
      const float w = expf(mv[k] - M);
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
#define CASE(G)                                                                                        \
  case G:                                                                                              \
    hipLaunchKernelGGL((k_attn<KT, D, G>), grid, dim3(kThreads), 0, s, a);                             \
    if (merge)                                                                                         \
      hipLaunchKernelGGL((k_attn_merge<G, D>), dim3(G * D / 64, grid.y, grid.z), dim3(kThreads), 0, s, \
                         a, chunk);                                                                    \
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
