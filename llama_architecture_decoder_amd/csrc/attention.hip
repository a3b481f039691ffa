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
#include <algorithm>
#include <type_traits>

#include "attention_body.h"

namespace lm {

template <typename KT, int D, int G, bool SELF>
__global__ __launch_bounds__(kThreads) void k_attn(AttnArgs a) {
  using S = AttnShape<KT, D>;
  constexpr int E = S::E, LPR = S::LPR, PPR = S::PPR, NR = S::NR, CHUNK = S::CHUNK;
  static_assert(LPR >= 1 && LPR <= 64 && (64 % LPR) == 0, "row must fit a wavefront");
  const int c = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int t = a.pos[b];
  const int nact = t / CHUNK + 1;  // chunks covering 0..t
  if (c >= nact) return;
  const int tid = threadIdx.x;
  const int li = tid % LPR, grp = tid / LPR;
  const int p0 = c * CHUNK;

  __shared__ float q_s[G][D];  // rotated query heads of the group

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
  valu_attend<KT, D, G, SELF ? kMergeSelf : kMergePlain>(a, c, j, b, t, nact, q_s, kraw, vraw);
}

template <int D, int G, int NPW_, bool KROWS, bool SELF, int NW = 4>
__global__ __launch_bounds__(NW * 64) void k_attn_mfma(AttnArgs a) {
  using S = MfmaAttnShape<D, G, NPW_, NW>;
  static_assert(!SELF || NW == 4, "the in-kernel merge runs on 4 wavefronts");
  constexpr int CHUNK = S::CHUNK, NPW = S::NPW, NGI = S::NGI, KS = S::KS, LPR = S::LPR, PPI = S::PPI, NV = S::NV;
  static_assert(G <= 8, "at most 8 query heads per kv head (two rows of the 16-row tile)");
  const int c = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int t = a.pos[b];
  const int nact = t / CHUNK + 1;
  if (c >= nact) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int pw0 = c * CHUNK + wave * NPW;  // this wavefront's first position

  __shared__ __attribute__((aligned(16))) bf16_t k_s[KROWS ? NW : 1][16 * S::KROW];  // each wave's 16 keys in turn

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
  float qf[KS][8];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) load_f32<8>(qp + 32 * ks + qh8, qf[ks]);
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
  q_fragments<D, G>(qf, qrow, qhi, qlo);

  bf16_t *kw = k_s[KROWS ? wave : 0];
  constexpr int IPG = 16 / PPI;  // key loads per 16-key group
  auto getk = [&](int gi, u32x4(&kf)[KS]) {
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
  };
  mfma_attend<D, G, NPW, NW, SELF ? kMergeSelf : kMergePlain>(a, c, j, b, t, nact, pw0, qhi, qlo, getk, vr);
}

// positions per wavefront of the matrix-core kernel: 64 (chunks of 256) measured faster than 32 or 128
// for both one row at 8K positions and 32 rows at 8K..32K
constexpr int kMfmaNpw = 64;

// Streamed attention for long rows and many blocks (batched rows, long contexts).  The step's chunks
// of 256 positions, in (row, kv head, chunk) order, are cut into sk_blocks equal runs (two blocks per
// CU, all resident); block k takes run k, crossing from one (row, kv head) segment to the next, and
// writes one partial per segment it touches (the merge combines a segment's partials in block order,
// which is position order).  Each wavefront keeps a running softmax over its 64 positions of every
// chunk (running maximum m and sum l per query head, its output slices rescaled by 2^(m_old - m_new)
// when the maximum grows), so a segment's result is the same combination of the same terms as in the
// one-chunk-per-block kernel.  The next chunk's keys are requested as soon as this chunk's scores are
// formed (their registers are free), its values as soon as this chunk's weighted sum is done, so every
// block keeps about a chunk of loads in flight from its first chunk to its last.  Against one block per
// chunk (32 rows of 8K..32K positions): the chunk partials' stores (40 MB per layer, interleaved with
// the cache stream) cost far more than their bytes (~39 us of a ~426 us launch), and spans of 4 or 8
// chunks per block left the launch's last round ragged.
#ifndef STREAM_NPW
#define STREAM_NPW 64
#endif
constexpr int kStreamNpw = STREAM_NPW;  // positions per wavefront and chunk in the streamed kernel
template <int D, int G>
__global__ __launch_bounds__(kThreads, 2) void k_attn_stream(AttnArgs a) {
  using S = MfmaAttnShape<D, G, kStreamNpw, 4>;
  constexpr int NW = 4, NPW = S::NPW, CHUNK = S::CHUNK, NGI = S::NGI, KS = S::KS, LPR = S::LPR, PPI = S::PPI;
  constexpr int NV = S::NV, GP = S::GP, IPG = 16 / PPI;
  const int nb = gridDim.x, T = a.sk_total;
  const int g0 = (int)((long)blockIdx.x * T / nb), g1 = (int)((long)(blockIdx.x + 1) * T / nb);
  if (g0 >= g1) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qrow = lane & 15, qh8 = (lane >> 4) * 8, qbase = 4 * (lane >> 4);
  const int vl = lane % LPR, vg = lane / LPR;

  __shared__ __attribute__((aligned(16))) bf16_t k_s[NW][16 * S::KROW];  // each wave's 16 keys in turn
  __shared__ __attribute__((aligned(16))) u32x4 q_s[KS][2][64];            // query fragments (hi, lo) by lane
  __shared__ __attribute__((aligned(16))) float p_s[NW][NPW][GP];          // each wave's weights
  __shared__ float r_s[NW][G];                                              // each wave's rescale factors
  __shared__ float m_s[NW][G], l_s[NW][G];
  __shared__ __attribute__((aligned(16))) float o_w[NW][G][D];             // each wave's output slices

  // the block whose run holds chunk g: the last k with k * T / nb <= g
  auto blk = [&](int g) { return (int)(((long)(g + 1) * nb - 1) / T); };
  // where the run starts: row b (the last whose first chunk is at or before g0), kv head j, chunk c
  int b;
  {
    int lo = 0, hi = a.sk_rows - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.sk_prefix[mid] <= g0) lo = mid;
      else hi = mid - 1;
    }
    b = lo;
  }
  int t = a.pos[b];
  int n = t / CHUNK + 1;  // chunks of each of row b's segments
  int j = (g0 - a.sk_prefix[b]) / n, c = (g0 - a.sk_prefix[b]) % n;

  const bf16_t *Kc = reinterpret_cast<const bf16_t *>(a.kc);
  const bf16_t *Vc = reinterpret_cast<const bf16_t *>(a.vc);
  auto seg_off = [&](int bb, int jj) { return ((size_t)(a.row0 + bb) * a.kv + jj) * (size_t)a.max_seq * D; };
  // Requests go through buffer descriptors of the segment's rows 0..tt (scalar registers): lane l asks
  // for 16 bytes at 8 (l%LPR) of row l/LPR of each PPI-row group of its 64 positions (whole rows per
  // load), one 32-bit offset register per request; a row past tt is outside the descriptor, so the
  // hardware returns zeros without a memory access (their scores are masked, their weights 0).  `rest`:
  // the requests after the run's last chunk, all outside, fetch nothing.
  u32x4 kr[NV], vr[NV];
  auto rsrc = [&](const bf16_t *base, int tt) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t *>(base), (short)0, (tt + 1) * D * 2, 0x00020000);
  };
  // (`rest` sets the offset's top bit, past any descriptor: arithmetic, not a branch around each request)
  auto voff = [&](int cc, bool rest, int i) {
    return (uint32_t)((cc * CHUNK + wave * NPW + PPI * i + vg) * D * 2 + 16 * vl) | ((uint32_t)rest << 31);
  };
  // requests i0 .. i1-1 of a chunk's keys / values
  auto load_k = [&](__amdgpu_buffer_rsrc_t r, int cc, bool rest, int i0, int i1) {
#pragma unroll
    for (int i = i0; i < i1; ++i) kr[i] = __builtin_amdgcn_raw_buffer_load_b128(r, voff(cc, rest, i), 0, kBufferNT);
  };
  auto load_v = [&](__amdgpu_buffer_rsrc_t r, int cc, bool rest, int i0, int i1) {
#pragma unroll
    for (int i = i0; i < i1; ++i) vr[i] = __builtin_amdgcn_raw_buffer_load_b128(r, voff(cc, rest, i), 0, kBufferNT);
  };
  size_t off = seg_off(b, j);
  __amdgpu_buffer_rsrc_t rk = rsrc(Kc + off, t), rv = rsrc(Vc + off, t);
  load_k(rk, c, false, 0, NV);
  load_v(rv, c, false, 0, NV);
  // the segment's query fragments (the same for every wavefront) into LDS, read per key group: registers
  // go to the loads of two chunks in flight.  The barrier also orders the previous segment's reads of
  // the combine arrays before any later write.
  auto load_q = [&]() {
    if (wave == 0) {
      const float *qp = a.q + (size_t)b * (a.kv * G * D) + ((size_t)j * G + min(qrow, G - 1)) * D;
      float qf[KS][8];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) load_f32<8>(qp + 32 * ks + qh8, qf[ks]);
      u32x4 qhi[KS], qlo[KS];
      q_fragments<D, G>(qf, qrow, qhi, qlo);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        q_s[ks][0][lane] = qhi[ks];
        q_s[ks][1][lane] = qlo[ks];
      }
    }
    lds_barrier();
  };
  load_q();

  // LDS operations of a wave complete in order; a wave barrier between its writes and its reads
  auto wave_sync = [] {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  };
  bf16_t *kw = k_s[wave];
  const float scale2 = a.scale * 1.4426950408889634f;
  float mrun[4], lrun[4];  // this lane's heads qbase + r: running maximum (base 2) and sum
  float o[G][8];
  auto reset = [&] {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      mrun[r] = -INFINITY;
      lrun[r] = 0.f;
    }
#pragma unroll
    for (int q = 0; q < G; ++q)
#pragma unroll
      for (int e = 0; e < 8; ++e) o[q][e] = 0.f;
  };
  reset();

  for (int g = g0; g < g1; ++g) {
    // the chunk after this one in the run
    int b2 = b, j2 = j, c2 = c + 1;
    if (c2 >= n) {
      c2 = 0;
      if (++j2 >= a.kv) {
        j2 = 0;
        ++b2;
      }
    }
    const bool more = g + 1 < g1;
    const int t2 = more ? a.pos[b2] : t;
    const size_t off2 = more ? seg_off(b2, j2) : off;
    const __amdgpu_buffer_rsrc_t rk2 = rsrc(Kc + off2, t2), rv2 = rsrc(Vc + off2, t2);

    const int pw0 = c * CHUNK + wave * NPW;
    const int p1 = min(c * CHUNK + CHUNK, t + 1);
    // (1) scores, base 2, on the matrix cores: the 16 keys of group gi through the wave's LDS tile into
    // the B layout (lane l: key l%16, numbers 32 ks + 8(l/16) .. +8)
    float sc[NGI][4];
#pragma unroll
    for (int gi = 0; gi < NGI; ++gi) {
#pragma unroll
      for (int u = 0; u < IPG; ++u)
        *reinterpret_cast<u32x4 *>(&kw[(PPI * u + vg) * S::KROW + 8 * vl]) = kr[gi * IPG + u];
      wave_sync();
      u32x4 kf[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kf[ks] = *reinterpret_cast<const u32x4 *>(&kw[qrow * S::KROW + 32 * ks + qh8]);
      wave_sync();
      af32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        acc = mfma16(q_s[ks][0][lane], kf[ks], acc);
        acc = mfma16(q_s[ks][1][lane], kf[ks], acc);
      }
      const int p = pw0 + 16 * gi + qrow;
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[gi][r] = (p < p1) ? acc[r] * scale2 : -INFINITY;
      // (2) the next chunk's keys go out as their registers free up: the first half after the first
      // half of the groups (the scheduling barriers keep the compiler from hoisting these requests above
      // the use of the registers they refill, which would need a second set of registers)
      if (gi == NGI / 2 - 1 || gi == NGI - 1) {
        __builtin_amdgcn_sched_barrier(0);
        load_k(rk2, c2, !more, gi == NGI - 1 ? NV / 2 : 0, gi == NGI - 1 ? NV : NV / 2);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // (3) per head: the new running maximum, the factor for what was summed so far, this chunk's
    // weights 2^(s2 - max) and their sum (reference 0 while no position has been seen: every weight 0)
    float fr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float m = sc[0][r];
#pragma unroll
      for (int gi = 1; gi < NGI; ++gi) m = fmaxf(m, sc[gi][r]);
      const float mn = fmaxf(mrun[r], row16_max(m));
      const float mref = (mn == -INFINITY) ? 0.f : mn;
      fr[r] = (mrun[r] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mrun[r] - mref);
      float l = 0.f;
#pragma unroll
      for (int gi = 0; gi < NGI; ++gi) {
        const float w = __builtin_amdgcn_exp2f(sc[gi][r] - mref);
        sc[gi][r] = w;
        l += w;
      }
      lrun[r] = fmaf(lrun[r], fr[r], group_sum<16>(l));
      mrun[r] = mn;
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
          if (qbase + r < G) r_s[wave][qbase + r] = fr[r];
      }
    }
    wave_sync();
    // (4) o[q][e] = f[q] * o[q][e] + sum over this lane's positions of w[q] * V[p][8 vl + e]
#pragma unroll
    for (int q = 0; q < G; ++q) {
      const float f = r_s[wave][q];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[q][e] *= f;
    }
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
      // (5) the next chunk's values, each half as its registers free up
      if (i == NV - 1) {
        __builtin_amdgcn_sched_barrier(0);
        load_v(rv2, c2, !more, 0, NV);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    wave_sync();  // this chunk's weights and factors are read before the next chunk writes them

    if (!more || b2 != b || j2 != j) {
      // (6) the segment's partial: the wave's lane groups summed (lanes that share lane % LPR hold the
      // same numbers), the waves combined in a fixed order (factor 2^(m_w - M), 0 for a wave without
      // positions); slot = this block's place among the blocks the segment's chunks fall in
#pragma unroll
      for (int q = 0; q < G; ++q)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[q][e] = strided_sum<LPR>(o[q][e]);
      if (vg == 0) {
#pragma unroll
        for (int q = 0; q < G; ++q) {
          *reinterpret_cast<float4 *>(&o_w[wave][q][8 * vl]) = make_float4(o[q][0], o[q][1], o[q][2], o[q][3]);
          *reinterpret_cast<float4 *>(&o_w[wave][q][8 * vl + 4]) = make_float4(o[q][4], o[q][5], o[q][6], o[q][7]);
        }
      }
      if (qbase < G && qrow == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (qbase + r < G) {
            m_s[wave][qbase + r] = mrun[r];
            l_s[wave][qbase + r] = lrun[r];
          }
      }
      lds_barrier();
      const int part = (int)blockIdx.x - blk(a.sk_prefix[b] + j * n);
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
          acc = fmaf(f, o_w[w][q][d], acc);
          L = fmaf(f, l_s[w][q], L);
        }
        emit_chunk<G, D, kMergePlain>(a, b, j, part, slot, idx, q, d, acc, M, L);
      }
      reset();
      if (more) {
        b = b2;
        j = j2;
        t = t2;
        n = t / CHUNK + 1;
        off = off2;
        rk = rk2;
        rv = rv2;
        load_q();
      }
    }
    c = c2;
  }
}

// Merge of the chunk partials of one (row, kv head), in chunk order (a separate launch: the kernel
// boundary makes the partials visible without cache-wide fences inside the attention kernel).
// Block (og, j, b) produces 64 consecutive outputs of query head i = og*64/head of group j:
// M = max_c m_c, w_c = exp(m_c - M), L = sum_c w_c l_c, o = (sum_c w_c o_c) / L.  The NW waves are NW
// chunk groups x 64 outputs (wave w takes chunks w, w + NW, ...); their sums are combined in a fixed
// order.  Every load is issued before the first use: NW * PER chunks in one memory round trip (NW = 16
// for one long row: 512 chunks took 34 us per layer in 8 rounds with 4 waves, 6.7 us in one with 16;
// one row of 64 chunks: 16 waves of 4 chunks 0.33 us per layer faster than 4 of 16, 1 wave of 64 2.5 us
// slower).
template <int G, int D, int NW, int PER>
__global__ __launch_bounds__(NW * 64) void k_attn_merge(AttnArgs a, int chunk) {
  constexpr int NT = NW * 64;
  constexpr int MLR = (kAttnMaxChunks + NT - 1) / NT;
  const int og = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int t = a.pos[b];
  int nact = t / chunk + 1;
  if (a.sk_total) {
    // streamed attention: the segment's partials are those of the blocks its chunks fall in
    const int nb = a.sk_blocks, T = a.sk_total, g = a.sk_prefix[b] + j * nact;
    auto blk = [&](int x) { return (int)(((long)(x + 1) * nb - 1) / T); };
    nact = blk(g + nact - 1) - blk(g) + 1;
  }
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

// Merge of the streamed kernel's partials when no segment has more than kFewParts of them (long rows
// over a resident grid: 2-3 each): block = one (row, kv head) segment, each thread OPT of its g*head
// outputs; every part's (m, l, o) requested before any is used (one memory round trip), then
// M = max_c m_c, w_c = 2^(m_c - M), L = sum_c w_c l_c, o = (sum_c w_c o_c) / L in part (= position) order.
// Against the general merge (2048 blocks of 64 outputs at 32 rows x 8 kv heads): no LDS, no barriers.
constexpr int kFewParts = 8;
template <int G, int D>
__global__ __launch_bounds__(kThreads) void k_attn_merge_few(AttnArgs a, int chunk) {
  constexpr int NO = G * D, OPT = (NO + kThreads - 1) / kThreads;
  const int j = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int n = a.pos[b] / chunk + 1;
  const int nb = a.sk_blocks, T = a.sk_total, g = a.sk_prefix[b] + j * n;
  auto blk = [&](int x) { return (int)(((long)(x + 1) * nb - 1) / T); };
  const int nparts = blk(g + n - 1) - blk(g) + 1;  // <= kFewParts (checked by the launcher)
  const size_t slot = ((size_t)b * a.kv + j) * (size_t)a.nch;
  const float *pml = a.part_ml + slot * (size_t)(G * 2);
  const float *po = a.part_o + slot * (size_t)NO;
  float mv[OPT][kFewParts], lv[OPT][kFewParts], ov[OPT][kFewParts];
#pragma unroll
  for (int i = 0; i < OPT; ++i) {
    const int idx = min(tid + i * kThreads, NO - 1), q = idx / D;
#pragma unroll
    for (int k = 0; k < kFewParts; ++k) {
      const int cc = min(k, nparts - 1);  // unconditional (clamped): one wait for all of them
      mv[i][k] = pml[(size_t)cc * G * 2 + 2 * q];
      lv[i][k] = pml[(size_t)cc * G * 2 + 2 * q + 1];
      ov[i][k] = po[(size_t)cc * NO + idx];
    }
  }
#pragma unroll
  for (int i = 0; i < OPT; ++i) {
    const int idx = tid + i * kThreads;
    float M = mv[i][0];
#pragma unroll
    for (int k = 1; k < kFewParts; ++k)
      if (k < nparts) M = fmaxf(M, mv[i][k]);
    float L = 0.f, acc = 0.f;
#pragma unroll
    for (int k = 0; k < kFewParts; ++k)
      if (k < nparts) {
        const float w = __builtin_amdgcn_exp2f(mv[i][k] - M);  // maxima are in base 2
        L = fmaf(w, lv[i][k], L);
        acc = fmaf(w, ov[i][k], acc);
      }
    if (idx < NO) put_out(a, b, j * NO + idx, acc / L);
  }
}

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

template <int G, int D>
static hipError_t merge_g(const AttnArgs &a, int B, int nch_launch, int chunk, hipStream_t s) {
  // 16 waves only when the merge has fewer blocks than the chip has CUs (one row): at 32 rows (2048
  // blocks of ~125 chunks) the 4-wave blocks were faster (11.8 vs 30.4 us per layer)
  const dim3 mg(G * D / 64, a.kv, B);
  const bool one_round = (long)mg.x * mg.y * mg.z < 256;
  if (one_round && nch_launch > 64)
    launch(k_attn_merge<G, D, 16, 32>, mg, dim3(16 * 64), s, false, true, a, chunk);
  else if (one_round)
    launch(k_attn_merge<G, D, 16, 4>, mg, dim3(16 * 64), s, false, true, a, chunk);
  else
    launch(k_attn_merge<G, D, 4, 16>, mg, dim3(kThreads), s, false, true, a, chunk);
  return hipGetLastError();
}

hipError_t launch_attention_merge(int head, int g, const AttnArgs &a, int B, int nch, int chunk, hipStream_t s) {
  auto by_g = [&](auto d) -> hipError_t {
    constexpr int D = decltype(d)::value;
    switch (g) {
      case 1: return merge_g<1, D>(a, B, nch, chunk, s);
      case 2: return merge_g<2, D>(a, B, nch, chunk, s);
      case 3: return merge_g<3, D>(a, B, nch, chunk, s);
      case 4: return merge_g<4, D>(a, B, nch, chunk, s);
      case 8: return merge_g<8, D>(a, B, nch, chunk, s);
    }
    return hipErrorInvalidValue;
  };
  if (head == 64) return by_g(std::integral_constant<int, 64>{});
  if (head == 128) return by_g(std::integral_constant<int, 128>{});
  return hipErrorInvalidValue;
}

// Blocks of the streamed attention: two per CU of the current device (its kernel fits two per CU), all
// resident at once; 0 if the count cannot be read
static int stream_blocks() {
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cached[dev] == 0) {
    int cu = 0;
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0) return 0;
    cached[dev] = 2 * cu;
  }
  return cached[dev];
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
    const long nblk = (long)B * a.kv * nch_launch;
    const bool krows = nblk >= 4096;
    if (krows && !self && !a.table && stream_blocks() > 0) {
      // the streamed kernel: equal runs of the step's chunks over a resident grid, then the merge
      constexpr int schunk = MfmaAttnShape<D, G, kStreamNpw, 4>::CHUNK;
      long total = 0;
      for (int b = 0; b < B; ++b) {
        a.sk_prefix[b] = (int)total;
        total += (long)a.kv * (a.pos[b] / schunk + 1);
      }
      a.sk_total = (int)total;
      a.sk_rows = B;
      a.sk_blocks = (int)std::min<long>(stream_blocks(), total);
      a.direct = 0;
      launch(k_attn_stream<D, G>, dim3(a.sk_blocks), dim3(kThreads), s, true, false, a);
      // the most parts a segment has: the blocks its chunks fall in
      int most = 0;
      for (int b = 0; b < B; ++b) {
        const int n = a.pos[b] / schunk + 1;
        for (int j = 0; j < a.kv; ++j) {
          const long g = a.sk_prefix[b] + (long)j * n;
          const long first = ((g + 1) * a.sk_blocks - 1) / total, last = ((g + n) * a.sk_blocks - 1) / total;
          most = std::max(most, (int)(last - first + 1));
        }
      }
      if (most <= kFewParts) {
        launch(k_attn_merge_few<G, D>, dim3(a.kv, B), dim3(kThreads), s, false, true, a, schunk);
        return hipGetLastError();
      }
      return merge_g<G, D>(a, B, nch_launch, schunk, s);
    }
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
  if (merge && !self) return merge_g<G, D>(a, B, nch_launch, chunk, s);
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
