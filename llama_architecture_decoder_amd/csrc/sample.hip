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
//   k_sample_rows  block b: the nchunk lists of row b, the K2 largest of them, then one wavefront
//                  does the draw.
//
// Selection of the K2 largest of a block's keys (block_select) sorts only what can be among them.
// Each wavefront sorts its 64 per-thread maxima in registers and takes the m-th largest, m =
// ceil(K2/4); T, the smallest of the four, has at least K2 keys at or above it (m distinct maxima in
// each wavefront), so every key of the answer is >= T.  The keys >= T are appended to LDS (positions
// from ballots, one LDS atomic per wavefront) and sorted: in registers by one wavefront when there
// are at most 256, else by a bitonic network over LDS.  If more than the LDS buffer holds pass T (only
// for adversarial orders), the buffer's K2-th largest becomes the new T and the keys are scanned again.
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

// bitonic sort, descending, of the 64*R keys of one wavefront (element r*64 + lane in a[r])
template <int R>
__device__ __forceinline__ void wave_sort_desc(uint64_t (&a)[R]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int size = 2; size <= 64 * R; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (stride >= 64) {
        const int rs = stride >> 6;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if (r & rs) continue;
          const bool desc = ((r * 64 + lane) & size) == 0;
          const uint64_t x = a[r], y = a[r | rs];
          if ((x < y) == desc) {
            a[r] = y;
            a[r | rs] = x;
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const uint64_t o = shfl_xor64(a[r], stride);
          const bool desc = ((r * 64 + lane) & size) == 0;
          const bool low = (lane & stride) == 0;
          const bool keep_max = low == desc;
          a[r] = keep_max ? (a[r] > o ? a[r] : o) : (a[r] < o ? a[r] : o);
        }
      }
    }
  }
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

template <int R>
__device__ __forceinline__ void wave0_sort(uint64_t *buf) {
  uint64_t a[R];
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int r = 0; r < R; ++r) a[r] = buf[r * 64 + lane];
  wave_sort_desc<R>(a);
#pragma unroll
  for (int r = 0; r < R; ++r) buf[r * 64 + lane] = a[r];
}

struct SelectLds {
  uint64_t buf[kCap];
  uint64_t wt[kT / 64];
  int count;
};

// The K2 largest of the block's keys (thread t holds key[j]; 0 = empty), sorted descending, into
// L.buf[0..K2) (0 past the real keys).  Every thread of the block calls it.
template <int NPT>
__device__ void block_select(const uint64_t (&key)[NPT], int K2, SelectLds &L) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint64_t mx[1] = {0ull};
#pragma unroll
  for (int j = 0; j < NPT; ++j) mx[0] = key[j] > mx[0] ? key[j] : mx[0];
  wave_sort_desc<1>(mx);
  const int m = (K2 + 3) / 4;
  const uint64_t tw = readlane64(mx[0], m - 1);
  if (lane == 0) L.wt[wave] = tw;
  if (tid == 0) L.count = 0;
  __syncthreads();
  uint64_t T = L.wt[0];
#pragma unroll
  for (int w = 1; w < kT / 64; ++w) T = L.wt[w] < T ? L.wt[w] : T;
  if (T == 0ull) T = 1ull;
  int cnt;
  for (;;) {
    int total = 0;
#pragma unroll
    for (int j = 0; j < NPT; ++j) total += __popcll(__ballot(key[j] >= T));
    int base = 0;
    if (lane == 0 && total) base = atomicAdd(&L.count, total);
    base = __shfl(base, 0);
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
      const bool pass = key[j] >= T;
      const uint64_t bm = __ballot(pass);
      const int pos = base + below(bm);
      if (pass && pos < kCap) L.buf[pos] = key[j];
      base += __popcll(bm);
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
  int n = 64;
  while (n < cnt || n < K2) n <<= 1;
  for (int i = cnt + tid; i < n; i += kT) L.buf[i] = 0ull;
  __syncthreads();
  if (n <= 256) {
    if (wave == 0) {
      if (n == 64)
        wave0_sort<1>(L.buf);
      else if (n == 128)
        wave0_sort<2>(L.buf);
      else
        wave0_sort<4>(L.buf);
    }
    __syncthreads();
  } else {
    lds_sort_desc(L.buf, n);
  }
}

__global__ __launch_bounds__(kT) void k_topk_chunk(const float *logits, int64_t ld, int V, int K2, uint64_t *cand) {
  __shared__ SelectLds L;
  const int c = blockIdx.x, b = blockIdx.y, nchunk = gridDim.x;
  const float *row = logits + (int64_t)b * ld;
  const int base = c * kChunk;
  uint64_t key[kChunk / kT];
#pragma unroll
  for (int j = 0; j < kChunk / kT; ++j) {
    const int id = base + j * kT + (int)threadIdx.x;
    key[j] = id < V ? cand_key(row[id], id) : 0ull;
  }
  block_select<kChunk / kT>(key, K2, L);
  uint64_t *out = cand + ((int64_t)b * nchunk + c) * K2;
  for (int j = threadIdx.x; j < K2; j += kT) out[j] = L.buf[j];
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
  const int b = blockIdx.x;
  const int K2 = a.K2, total = a.nchunk * K2;
  const uint64_t *src = a.cand + (int64_t)b * total;
  uint64_t key[NPT];
#pragma unroll
  for (int j = 0; j < NPT; ++j) {
    const int i = j * kT + (int)threadIdx.x;
    key[j] = i < total ? src[i] : 0ull;
  }
  block_select<NPT>(key, K2, L);
  if (threadIdx.x >= 64) return;

  const int lane = threadIdx.x;
  const int keff = a.k < a.V ? a.k : a.V;
  const float temp = a.temp;
  const float top = from_order((uint32_t)(L.buf[0] >> 32));
  float w[4], S[4];
  int id[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int j = 64 * q + lane;
    w[q] = 0.f;
    S[q] = 0.f;
    id[q] = -1;
    if (j < keff) {
      const uint64_t key = L.buf[j];
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
