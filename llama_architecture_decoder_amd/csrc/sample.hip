// Sampling with temperature, top-k and top-p from F32 logits (bend-ml-llama main.bend, "Sampling":
// topk, weight, total, kept, stops/pick, sample; draws from its lowbias32-based `uniform`).
//
// Two passes, both on 64-bit keys that order candidates exactly as the page's top-k does: the high
// word is the logit's bits mapped to an unsigned order (−0 and +0 share one key, as they compare
// equal), the low word is 0xFFFFFFFF − id, so a larger key is a larger logit or, for equal logits,
// the lower id.  Keys are unique; 0 marks an empty slot (no real key is 0).
//
//   k_topk_chunk   block (c, b): the 4096 logits of chunk c of row b into LDS as keys, a bitonic
//                  sort, the K2 largest out (K2 = k rounded up to a power of two).
//   k_sample_rows  block b: the nchunk sorted lists of row b into LDS with every odd list reversed,
//                  which is the state of a bitonic sort after its runs of K2, so the sort continues
//                  from runs of 2*K2; then one wavefront does the draw.
//
// The draw keeps the page's F32 order: each candidate's weight exp(v/temp − top/temp) (the
// exponential computed in double and rounded once, i.e. the correctly rounded F32 value), one
// running sum from 0 in candidate order (lanes hand their weights to the sum through readlane, and
// each lane keeps the partial sums of its candidates), Z = the last running sum, lim = p*Z, kept =
// the candidates up to the first one after which the running sum is not below lim, z = the running
// sum of the last kept one, target = u*z, and the draw is the first kept candidate whose running
// sum is above target, or the last kept one.  Every partial sum the page forms (total, kept.go,
// pick.go) is one of these running sums, so the comparisons see the same F32 values.
#include "common.h"

namespace lm {

namespace {

constexpr int kChunk = 4096;   // logits per block of the first pass
constexpr int kSortT = 1024;   // threads per block of both passes

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

// bitonic sort of s[0..n) (n a power of two) into descending order, starting from runs of size0/2
// that are already sorted, alternately descending and ascending
__device__ __forceinline__ void bitonic_desc(uint64_t *s, int n, int size0) {
  for (int size = size0; size <= n; size <<= 1)
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      __syncthreads();
      for (int i = threadIdx.x; i < (n >> 1); i += kSortT) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const uint64_t a = s[lo], b = s[hi];
        const bool desc = (lo & size) == 0;
        if ((a < b) == desc) {
          s[lo] = b;
          s[hi] = a;
        }
      }
    }
  __syncthreads();
}

__global__ __launch_bounds__(kSortT) void k_topk_chunk(const float *logits, int64_t ld, int V, int K2,
                                                      uint64_t *cand) {
  __shared__ uint64_t s[kChunk];
  const int c = blockIdx.x, b = blockIdx.y, nchunk = gridDim.x;
  const float *row = logits + (int64_t)b * ld;
  const int base = c * kChunk;
  for (int j = threadIdx.x; j < kChunk; j += kSortT) {
    const int id = base + j;
    s[j] = id < V ? cand_key(row[id], id) : 0ull;
  }
  bitonic_desc(s, kChunk, 2);
  uint64_t *out = cand + ((int64_t)b * nchunk + c) * K2;
  for (int j = threadIdx.x; j < K2; j += kSortT) out[j] = s[j];
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

template <int NMAX>
__global__ __launch_bounds__(kSortT) void k_sample_rows(SampleArgs a) {
  __shared__ uint64_t s[NMAX];
  const int b = blockIdx.x;
  const int K2 = a.K2, n2 = a.n2;
  const uint64_t *src = a.cand + (int64_t)b * a.nchunk * K2;
  for (int j = threadIdx.x; j < n2; j += kSortT) {
    const int c = j / K2, r = j - c * K2;
    s[j] = c < a.nchunk ? src[(int64_t)c * K2 + ((c & 1) ? K2 - 1 - r : r)] : 0ull;
  }
  bitonic_desc(s, n2, 2 * K2);
  if (threadIdx.x >= 64) return;

  const int lane = threadIdx.x;
  const int keff = a.k < a.V ? a.k : a.V;
  const float temp = a.temp;
  const float top = from_order((uint32_t)(s[0] >> 32));
  float w[4], S[4];
  int id[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int j = 64 * q + lane;
    w[q] = 0.f;
    S[q] = 0.f;
    id[q] = -1;
    if (j < keff) {
      const uint64_t key = s[j];
      const float v = from_order((uint32_t)(key >> 32));
      id[q] = (int)(0xFFFFFFFFu - (uint32_t)key);
      const float qv = v / temp;
      const float qt = top / temp;
      const float d = qv - qt;
      w[q] = (float)exp((double)d);
    }
  }
  // running sums in candidate order; lane l of group q keeps the one that ends at candidate 64q+l
  float acc = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int n = keff - 64 * q < 64 ? keff - 64 * q : 64;
    for (int l = 0; l < n; ++l) {
      acc = acc + __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w[q]), l));
      if (lane == l) S[q] = acc;
    }
  }
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

int sample_sort_size(int V, int K2) {
  int n = 1;
  while (n < sample_chunks(V) * K2) n <<= 1;
  return n < K2 ? K2 : n;
}

hipError_t launch_sample(const SampleArgs &a, int B, hipStream_t s) {
  launch(k_topk_chunk, dim3(a.nchunk, B), dim3(kSortT), s, true, false, a.logits, a.ld, a.V, a.K2, a.cand);
  if (a.n2 <= 1024)
    launch(k_sample_rows<1024>, dim3(B), dim3(kSortT), s, false, true, a);
  else if (a.n2 <= 4096)
    launch(k_sample_rows<4096>, dim3(B), dim3(kSortT), s, false, true, a);
  else
    launch(k_sample_rows<kSampleSortMax>, dim3(B), dim3(kSortT), s, false, true, a);
  return hipGetLastError();
}

}  // namespace lm
