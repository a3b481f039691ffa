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
// Pass 1: scores into LDS; per-head chunk max and exp-sum; pass 2: the exp-weighted V sum.  Each chunk
// writes an unnormalised partial (o, m, l); the last block to finish a (b, j) (an atomic counter that
// it resets) merges the chunks in chunk order, so the result does not depend on block timing.
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

template <typename KT, int D, int G>
__global__ __launch_bounds__(kThreads) void k_attn(AttnArgs a) {
  constexpr int E = Vec16<KT>::E;        // elements per 16-byte slice
  constexpr int LPR = D / E;             // lanes per head row
  constexpr int PPR = kThreads / LPR;    // positions per round
  static_assert(LPR >= 1 && LPR <= 64 && (64 % LPR) == 0, "row must fit a wavefront");
  const int c = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int t = a.pos[b];
  const int nact = (t + a.chunk) / a.chunk;  // chunks covering 0..t
  if (c >= nact) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = tid % LPR, grp = tid / LPR;
  const int p0 = c * a.chunk;
  const int p1 = min(p0 + a.chunk, t + 1);
  const int half = a.half;

  __shared__ float s_sc[G][kAttnChunkMax];
  __shared__ float kt_s[D], vt_s[D];
  __shared__ float m_s[G], l_s[G];
  __shared__ float o_s[4][G][D];
  __shared__ int last_s;

  const size_t head_off = ((size_t)(a.row0 + b) * a.kv + j) * (size_t)a.max_seq * D;
  KT *Kh = reinterpret_cast<KT *>(a.kc) + head_off;
  KT *Vh = reinterpret_cast<KT *>(a.vc) + head_off;
  const float *qkv = a.qkv + (size_t)b * a.qkv_stride;
  const int dim = a.kv * G * D;
  const float *cs = a.rope_cs + (size_t)t * half;
  const float *sn = a.rope_sn + (size_t)t * half;

  // rotated query slices of the g heads: lane li holds numbers [li*E, li*E + E)
  float q[G][E];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const float *qh = qkv + (size_t)(j * G + i) * D;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int d = li * E + e;
      if (d < half) {
        q[i][e] = rope_lo(qh[d], qh[d + half], cs[d], sn[d]);
      } else {
        const int dd = d - half;
        q[i][e] = rope_hi(qh[dd], qh[d], cs[dd], sn[dd]);
      }
    }
  }

  // the block whose chunk holds t appends this position's key (rotated) and value
  if (c == nact - 1) {
    const float *kh = qkv + dim + (size_t)j * D;
    const float *vh = qkv + dim + (size_t)a.kv * D + (size_t)j * D;
    for (int d = tid; d < D; d += kThreads) {
      float kr;
      if (d < half) {
        kr = rope_lo(kh[d], kh[d + half], cs[d], sn[d]);
      } else {
        const int dd = d - half;
        kr = rope_hi(kh[dd], kh[d], cs[dd], sn[dd]);
      }
      kt_s[d] = KvStore<KT>::round_store(Kh + (size_t)t * D + d, kr);
      vt_s[d] = KvStore<KT>::round_store(Vh + (size_t)t * D + d, vh[d]);
    }
  }
  __syncthreads();

  // ---- pass 1: scores of positions p0..p1-1
  const int n = p1 - p0;
  const int rounds = (n + PPR - 1) / PPR;
  for (int it = 0; it < rounds; it += 4) {
    u32x4 kr[4];
    float kf[4][E];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int p = p0 + (it + u) * PPR + grp;
      if (it + u < rounds && p < t) kr[u] = load_stream16(Kh + (size_t)p * D + li * E);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int p = p0 + (it + u) * PPR + grp;
      if (it + u < rounds && p < p1) {
        if (p < t) {
          Vec16<KT>::unpack(kr[u], kf[u]);
        } else {
#pragma unroll
          for (int e = 0; e < E; ++e) kf[u][e] = kt_s[li * E + e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) kf[u][e] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int p = p0 + (it + u) * PPR + grp;
      float s[G];
#pragma unroll
      for (int i = 0; i < G; ++i) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) acc = fmaf(q[i][e], kf[u][e], acc);
#pragma unroll
        for (int o = LPR / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
        s[i] = acc;
      }
      if (li == 0 && it + u < rounds && p < p1) {
#pragma unroll
        for (int i = 0; i < G; ++i) s_sc[i][p - p0] = a.scale * s[i];
      }
    }
  }
  __syncthreads();

  // ---- softmax pieces per head over this chunk: max, exp(s - max), their sum
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
  __syncthreads();

  // ---- pass 2: sum_p e_p V[p]
  float o[G][E];
#pragma unroll
  for (int i = 0; i < G; ++i)
#pragma unroll
    for (int e = 0; e < E; ++e) o[i][e] = 0.f;
  for (int it = 0; it < rounds; it += 4) {
    u32x4 vr[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int p = p0 + (it + u) * PPR + grp;
      if (it + u < rounds && p < t) vr[u] = load_stream16(Vh + (size_t)p * D + li * E);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int p = p0 + (it + u) * PPR + grp;
      if (it + u < rounds && p < p1) {
        float vf[E];
        if (p < t) {
          Vec16<KT>::unpack(vr[u], vf);
        } else {
#pragma unroll
          for (int e = 0; e < E; ++e) vf[e] = vt_s[li * E + e];
        }
#pragma unroll
        for (int i = 0; i < G; ++i) {
          const float w = s_sc[i][p - p0];
#pragma unroll
          for (int e = 0; e < E; ++e) o[i][e] = fmaf(w, vf[e], o[i][e]);
        }
      }
    }
  }
  // position groups inside a wavefront, then the 4 wavefronts
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
    for (int i = 0; i < G; ++i)
#pragma unroll
      for (int e = 0; e < E; ++e) o[i][e] += __shfl_xor(o[i][e], off);
  if (lane < LPR) {
#pragma unroll
    for (int i = 0; i < G; ++i)
#pragma unroll
      for (int e = 0; e < E; ++e) o_s[wave][i][li * E + e] = o[i][e];
  }
  __syncthreads();

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

  // ---- the last chunk block of (b, j) merges all chunks in chunk order
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const int prev = atomicAdd(a.counter + (size_t)b * a.kv + j, 1);
    last_s = (prev == nact - 1);
  }
  __syncthreads();
  if (!last_s) return;
  __threadfence();
  const float *po0 = a.part_o + slot * (size_t)(G * D);
  const float *pml0 = a.part_ml + slot * (size_t)(G * 2);
  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int i = idx / D, d = idx % D;
    float M = -INFINITY;
    for (int cc = 0; cc < nact; ++cc) M = fmaxf(M, __builtin_nontemporal_load(pml0 + (size_t)cc * G * 2 + 2 * i));
    float acc = 0.f, L = 0.f;
    for (int cc = 0; cc < nact; ++cc) {
      const float w = expf(__builtin_nontemporal_load(pml0 + (size_t)cc * G * 2 + 2 * i) - M);
      L = fmaf(w, __builtin_nontemporal_load(pml0 + (size_t)cc * G * 2 + 2 * i + 1), L);
      acc = fmaf(w, __builtin_nontemporal_load(po0 + (size_t)cc * G * D + idx), acc);
    }
    a.out[(size_t)b * a.out_stride + (size_t)(j * G + i) * D + d] = acc / L;
  }
  if (tid == 0) a.counter[(size_t)b * a.kv + j] = 0;
}

int attention_supported(int head, int g) {
  return (head == 64 || head == 128) && (g == 1 || g == 2 || g == 3 || g == 4 || g == 8);
}

template <typename KT, int D>
static hipError_t launch_d(int g, const AttnArgs &a, dim3 grid, hipStream_t s) {
  switch (g) {
#define CASE(G)                                                                   \
  case G:                                                                         \
    hipLaunchKernelGGL((k_attn<KT, D, G>), grid, dim3(kThreads), 0, s, a);        \
    break;
    CASE(1) CASE(2) CASE(3) CASE(4) CASE(8)
#undef CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attention(int kvdtype, int head, int g, const AttnArgs &a, int B, int nch_launch, hipStream_t s) {
  const dim3 grid(nch_launch, a.kv, B);
  if (kvdtype == LLAMA_BF16) {
    if (head == 64) return launch_d<bf16_t, 64>(g, a, grid, s);
    if (head == 128) return launch_d<bf16_t, 128>(g, a, grid, s);
  } else {
    if (head == 64) return launch_d<float, 64>(g, a, grid, s);
    if (head == 128) return launch_d<float, 128>(g, a, grid, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace lm
