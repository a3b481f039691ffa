// Sampling with temperature, top-k and top-p from F32 logits (bend-ml-llama main.bend, "Sampling":
// topk, weight, total, kept, stops/pick, sample; draws from its lowbias32-based `uniform`).
//
// Two passes, both on 64-bit keys that order candidates exactly as the page's top-k does: the high
// word is the logit's bits mapped to an unsigned order (−0 and +0 share one key, as they compare
// equal), the low word is 0xFFFFFFFF − id, so a larger key is a larger logit or, for equal logits,
// the lower id.  Keys are unique; 0 marks an empty slot (no real key is 0).
//
//   k_topk_chunk   block (c, b): the 8192 logits of chunk c of row b, 32 keys per thread in
//                  registers; their K2 largest (K2 = k rounded up to a power of two), sorted, out.
//   k_sample_rows  block b: the nchunk lists of row b, the K2 largest of them, then the draw.
//
// Selection of the K2 largest of a block's keys (block_select) looks closely only at what can be
// among them.  Each thread takes the maxima of G disjoint groups of its keys (G = 1, 2, 4 as K2 <= 64,
// 128, 256); each wavefront finds (a lower bound on) the m-th largest of its 64*G maxima, m =
// ceil(K2/4), by a bitwise search with ballots; T, the smallest of the four, has at least K2 keys at
// or above it (m distinct maxima in each wavefront), so every key of the answer is >= T.  The keys >= T are appended to LDS
// (offsets from a wavefront prefix sum built from ballots of the count bits, one LDS atomic per
// wavefront) and each finds its rank by counting the held keys above it (LDS broadcast reads); ranks
// below K2 are the sorted answer.  More than 1024 survivors go through a bitonic network over LDS
// instead, and if more than the buffer holds pass T (adversarial orders only), the buffer's K2-th
// largest becomes the new T and the keys are scanned again.
//
// The draw keeps the page's F32 order: each candidate's weight exp(v/temp − top/temp) (the
// exponential computed in double and rounded once, i.e. the correctly rounded F32 value), one
// running sum from 0 in candidate order (one thread; the others wait), Z = the last running sum,
// lim = p*Z, kept = the candidates up to the first one after which the running sum is not below lim,
// z = the running sum of the last kept one, target = u*z, and the draw is the first kept candidate
// whose running sum is above target, or the last kept one.  Every partial sum the page forms (total,
// kept.go, pick.go) is one of these running sums, so the comparisons see the same F32 values.
#include "common.h"

namespace lm {

namespace {

constexpr int kT = 256;        // threads per block of both passes
constexpr int kChunk = 8192;   // logits per block of the first pass (32 per thread)
constexpr int kCap = 2048;     // keys the selection buffer holds

__device__ __forceinline__ uint32_t order_bits(float v) {
  uint32_t b = __float_as_uint(v);
  if ((b & 0x7FFFFFFFu) == 0u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float from_order(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

__device__ __forceinline__ uint64_t cand_key(float v, int id) {
  return ((uint64_t)order_bits(v) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)id);
}

// lowbias32 (Chris Wellons, public domain)
__device__ __forceinline__ uint32_t lowbias32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7FEB352Du;
  x ^= x >> 15;
  x *= 0x846CA68Bu;
  x ^= x >> 16;
  return x;
}

// draw n of a seed: 24 bits scaled by 2^-24, in [0, 1)
__device__ __forceinline__ float uniform_draw(uint32_t seed, uint32_t n) {
  return (float)(lowbias32(lowbias32(seed) + n) >> 8) * 0x1p-24f;
}

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int m) {
  const int lo = __shfl_xor((int)(uint32_t)v, m);
  const int hi = __shfl_xor((int)(uint32_t)(v >> 32), m);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

__device__ __forceinline__ uint64_t readlane64(uint64_t v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}

// lanes below this one whose bit is set in m
__device__ __forceinline__ int below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// the m-th largest (m >= 1) of the keys v[0..R) of the wavefront's 64 lanes (distinct keys, 0 = empty;
// 0 when fewer than m are nonzero): the largest x with at least m keys >= x, built from the top bit.
// The high words (the logits) are searched first; the low words (the ids) only when more than a few
// keys share the high word found, so for logits without ties the result is x with a zero low word,
// still a bound with at least m keys at or above it.
template <int R>
__device__ __forceinline__ uint64_t wave_mth_largest(const uint64_t (&v)[R], int m) {
  uint32_t hi[R], lo[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    hi[r] = (uint32_t)(v[r] >> 32);
    lo[r] = (uint32_t)v[r];
  }
  uint32_t xh = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = xh | (1u << bit);
    int n = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) n += __popcll(__ballot(hi[r] >= c));
    if (n >= m) xh = c;
  }
  int above = 0, equal = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    above += __popcll(__ballot(hi[r] > xh));
    equal += __popcll(__ballot(hi[r] == xh));
  }
  uint32_t xl = 0;
  if (equal > 4) {
    const int need = m - above;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t c = xl | (1u << bit);
      int n = 0;
#pragma unroll
      for (int r = 0; r < R; ++r) n += __popcll(__ballot(hi[r] == xh && lo[r] >= c));
      if (n >= need) xl = c;
    }
  }
  return ((uint64_t)xh << 32) | xl;
}

// bitonic sort, descending, of s[0..n) (n a power of two) by the whole block
__device__ __forceinline__ void lds_sort_desc(uint64_t *s, int n) {
  for (int size = 2; size <= n; size <<= 1)
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      __syncthreads();
      for (int i = threadIdx.x; i < (n >> 1); i += kT) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const uint64_t x = s[lo], y = s[hi];
        const bool desc = (lo & size) == 0;
        if ((x < y) == desc) {
          s[lo] = y;
          s[hi] = x;
        }
      }
    }
  __syncthreads();
}

constexpr int kRankMax = 1024;  // survivors ranked by counting; more are sorted by the network

struct SelectLds {
  uint64_t buf[kCap];
  uint64_t wt[kT / 64];
  unsigned long long tmin;
  int count;
};

template <int G, int NPT>
__device__ __forceinline__ uint64_t wave_threshold(const uint64_t (&key)[NPT], int m) {
  uint64_t mx[G];
#pragma unroll
  for (int g = 0; g < G; ++g) mx[g] = 0ull;
#pragma unroll
  for (int j = 0; j < NPT; ++j) mx[j % G] = key[j] > mx[j % G] ? key[j] : mx[j % G];
  return wave_mth_largest<G>(mx, m);
}

// A lower bound T >= 1 on the K2-th largest of the block's keys (thread t holds key[j]; 0 = empty):
// the smallest over the wavefronts of the m-th largest of their group maxima (at least K2 keys are
// >= T), or 1 when there are fewer nonzero keys than that finds.  Ends with a barrier.
template <int NPT>
__device__ uint64_t maxima_threshold(const uint64_t (&key)[NPT], int K2, SelectLds &L) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m = (K2 + 3) / 4;
  const uint64_t tw = K2 <= 64 ? wave_threshold<1>(key, m)
                               : K2 <= 128 ? wave_threshold<2>(key, m) : wave_threshold<4>(key, m);
  if (lane == 0) L.wt[wave] = tw;
  __syncthreads();
  uint64_t T = L.wt[0];
#pragma unroll
  for (int w = 1; w < kT / 64; ++w) T = L.wt[w] < T ? L.wt[w] : T;
  return T == 0ull ? 1ull : T;
}

// The K2 largest of the block's keys (thread t holds key[j]; 0 = empty), sorted descending, into
// dst[0..K2) (0 past the real keys), given T >= 1 with at least K2 keys >= T or every nonzero key >= T;
// dst may be global or LDS memory.  Every thread of the block calls it with the same T; it ends with a
// barrier.
template <int NPT>
__device__ void block_select(const uint64_t (&key)[NPT], uint64_t T, int K2, SelectLds &L, uint64_t *dst) {
  static_assert(NPT <= 32, "pass masks are 32 bits");
  const int tid = threadIdx.x, lane = tid & 63;
  if (tid == 0) L.count = 0;
  __syncthreads();
  int cnt;
  for (;;) {
    uint32_t pm = 0;
#pragma unroll
    for (int j = 0; j < NPT; ++j) pm |= (key[j] >= T ? 1u : 0u) << j;
    const int c = __popc(pm);
    // exclusive prefix and total of c over the wavefront, one ballot per bit of c (c <= 32)
    int off = 0, tot = 0;
#pragma unroll
    for (int bit = 0; bit < 6; ++bit) {
      const uint64_t bm = __ballot((c >> bit) & 1);
      off += below(bm) << bit;
      tot += __popcll(bm) << bit;
    }
    int base = 0;
    if (lane == 0 && tot) base = atomicAdd(&L.count, tot);
    int pos = __shfl(base, 0) + off;
#pragma unroll
    for (int j = 0; j < NPT; ++j)
      if ((pm >> j) & 1u) {
        if (pos < kCap) L.buf[pos] = key[j];
        ++pos;
      }
    __syncthreads();
    cnt = L.count;
    if (cnt <= kCap) break;
    // too many passed: the K2-th largest of those held is a higher bound with K2 keys at or above it
    lds_sort_desc(L.buf, kCap);
    T = L.buf[K2 - 1];
    __syncthreads();
    if (tid == 0) L.count = 0;
    __syncthreads();
  }
  if (cnt <= kRankMax) {
    const int c8 = (cnt + 7) & ~7;
    if (tid < c8 - cnt) L.buf[cnt + tid] = 0ull;
    __syncthreads();
    const ulonglong2 *b2 = reinterpret_cast<const ulonglong2 *>(L.buf);
    for (int i = tid; i < cnt; i += kT) {
      const uint64_t me = L.buf[i];
      int r = 0;
      for (int j = 0; j < c8 / 2; j += 4) {
        const ulonglong2 p0 = b2[j], p1 = b2[j + 1], p2 = b2[j + 2], p3 = b2[j + 3];
        r += (p0.x > me) + (p0.y > me) + (p1.x > me) + (p1.y > me) + (p2.x > me) + (p2.y > me) + (p3.x > me) +
             (p3.y > me);
      }
      if (r < K2) dst[r] = me;
    }
    for (int i = cnt + tid; i < K2; i += kT) dst[i] = 0ull;
  } else {
    int n = 1;
    while (n < cnt) n <<= 1;
    for (int i = cnt + tid; i < n; i += kT) L.buf[i] = 0ull;
    lds_sort_desc(L.buf, n);
    for (int i = tid; i < K2; i += kT) dst[i] = L.buf[i];
  }
  __syncthreads();
}

__global__ __launch_bounds__(kT) void k_topk_chunk(const float *logits, int64_t ld, int V, int K2, uint64_t *cand) {
  __shared__ SelectLds L;
  const int c = blockIdx.x, b = blockIdx.y, nchunk = gridDim.x;
  const float *row = logits + (int64_t)b * ld;
  const int base = c * kChunk;
  uint64_t key[kChunk / kT];
#pragma unroll
  for (int j = 0; j < kChunk / kT; ++j) {
    // branch-free, so every load is issued before any is used (the index is clamped into the row)
    const int id = base + j * kT + (int)threadIdx.x;
    const float v = row[id < V ? id : V - 1];
    key[j] = cand_key(v, id) & (0ull - (uint64_t)(id < V));
  }
  const uint64_t T = maxima_threshold<kChunk / kT>(key, K2, L);
  block_select<kChunk / kT>(key, T, K2, L, cand + ((int64_t)b * nchunk + c) * K2);
}

__device__ __forceinline__ float lane_of(const float (&r)[4], int j) {
  const int q = j >> 6, l = j & 63;
  const float x = q == 0 ? r[0] : q == 1 ? r[1] : q == 2 ? r[2] : r[3];
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

__device__ __forceinline__ int lane_of(const int (&r)[4], int j) {
  const int q = j >> 6, l = j & 63;
  const int x = q == 0 ? r[0] : q == 1 ? r[1] : q == 2 ? r[2] : r[3];
  return __builtin_amdgcn_readlane(x, l);
}

// the first j (candidate order, lanes of groups 0..3) whose flag is set, or `none`
__device__ __forceinline__ int first_set(const bool (&f)[4], int none) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint64_t m = __ballot(f[q]);
    if (m) return 64 * q + __builtin_ctzll(m);
  }
  return none;
}

template <int NPT>
__global__ __launch_bounds__(kT) void k_sample_rows(SampleArgs a) {
  __shared__ SelectLds L;
  __shared__ uint64_t top[kSampleMaxK];
  __shared__ float wv[kSampleMaxK], Sv[kSampleMaxK];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int K2 = a.K2, total = a.nchunk * K2;
  const uint64_t *src = a.cand + (int64_t)b * total;
  uint64_t key[NPT];
#pragma unroll
  for (int j = 0; j < NPT; ++j) {
    const int i = j * kT + tid;
    key[j] = src[i < total ? i : total - 1] & (0ull - (uint64_t)(i < total));
  }
  // each list is sorted, so q = ceil(K2 / nl) entries of each of nl lists are >= the smallest of their
  // q-th entries: T.  A last chunk holding fewer than q logits is left out of the bound.
  int nl = a.nchunk, q = (K2 + nl - 1) / nl;
  if (nl > 1 && a.V - (nl - 1) * kChunk < q) {
    nl -= 1;
    q = (K2 + nl - 1) / nl;
  }
  if (tid == 0) L.tmin = ~0ull;
  __syncthreads();
  uint64_t tl = ~0ull;
  for (int c = tid; c < nl; c += kT) {
    const uint64_t e = src[(int64_t)c * K2 + q - 1];
    tl = e < tl ? e : tl;
  }
  if (tl != ~0ull) atomicMin(&L.tmin, (unsigned long long)tl);
  __syncthreads();
  const uint64_t T = L.tmin;
  block_select<NPT>(key, T == 0ull ? 1ull : T, K2, L, top);

  const int keff = a.k < a.V ? a.k : a.V;
  const float temp = a.temp;
  const float topv = from_order((uint32_t)(top[0] >> 32));
  if (tid < kSampleMaxK) {
    float w = 0.f;
    if (tid < keff) {
      const float v = from_order((uint32_t)(top[tid] >> 32));
      const float qv = v / temp;
      const float qt = topv / temp;
      const float d = qv - qt;
      w = (float)exp((double)d);
    }
    wv[tid] = w;
  }
  __syncthreads();
  // running sums in candidate order, one after another (adding the zero weights past keff changes no
  // sum that is used)
  if (tid == 0) {
    float acc = 0.f;
    const float4 *w4 = reinterpret_cast<const float4 *>(wv);
    for (int j = 0; j < keff; j += 4) {
      const float4 q = w4[j >> 2];
      const float s0 = acc + q.x;
      const float s1 = s0 + q.y;
      const float s2 = s1 + q.z;
      const float s3 = s2 + q.w;
      *reinterpret_cast<float4 *>(Sv + j) = make_float4(s0, s1, s2, s3);
      acc = s3;
    }
  }
  __syncthreads();
  if (tid >= 64) return;
  const int lane = tid;
  float S[4];
  int id[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int j = 64 * q + lane;
    S[q] = Sv[j];
    id[q] = j < keff ? (int)(0xFFFFFFFFu - (uint32_t)top[j]) : -1;
  }
  const float acc = Sv[keff - 1];
  const float Z = acc;
  const float lim = a.p * Z;
  bool f[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int j = 64 * q + lane;
    f[q] = j <= keff - 2 && !(S[q] < lim);
  }
  const int kept = first_set(f, keff - 1) + 1;
  const float z = lane_of(S, kept - 1);
  const float u = a.u ? a.u[b] : uniform_draw(a.seeds[b], a.draw);
  const float target = u * z;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int j = 64 * q + lane;
    f[q] = j <= kept - 2 && target < S[q];
  }
  const int pick = first_set(f, kept - 1);
  const int pid = lane_of(id, pick);
  if (lane == 0) {
    a.ids[b] = pid;
    if (a.vals) a.vals[b] = a.logits[(int64_t)b * a.ld + pid];
  }
  if (a.topk_ids) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int j = 64 * q + lane;
      if (j < a.k) a.topk_ids[(int64_t)b * a.k + j] = id[q];
    }
  }
}

}  // namespace

int sample_chunks(int V) { return (V + kChunk - 1) / kChunk; }

int sample_candidates(int V, int K2) { return sample_chunks(V) * K2; }

hipError_t launch_sample(const SampleArgs &a, int B, hipStream_t s) {
  launch(k_topk_chunk, dim3(a.nchunk, B), dim3(kT), s, true, false, a.logits, a.ld, a.V, a.K2, a.cand);
  if (a.nchunk * a.K2 <= 4 * kT)
    launch(k_sample_rows<4>, dim3(B), dim3(kT), s, false, true, a);
  else
    launch(k_sample_rows<kSampleCandMax / kT>, dim3(B), dim3(kT), s, false, true, a);
  return hipGetLastError();
}

}  // namespace lm
