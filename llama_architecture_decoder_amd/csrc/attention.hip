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

template <int G, int D>
static hipError_t merge_g(const AttnArgs &a, int B, int nch_launch, int chunk, hipStream_t s) {
  // 16 waves only when the merge has fewer blocks than the chip has CUs (one row): at 32 rows (2048
  // blocks of ~125 chunks) the 4-wave blocks were faster (11.8 vs 30.4 us per layer)
  const dim3 mg(G * D / 64, a.kv, B);
  if (nch_launch > 64 && (long)mg.x * mg.y * mg.z < 256)
    launch(k_attn_merge<G, D, 16>, mg, dim3(16 * 64), s, false, true, a, chunk);
  else
    launch(k_attn_merge<G, D, 4>, mg, dim3(kThreads), s, false, true, a, chunk);
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
