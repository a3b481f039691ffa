// Device-side writer of pre-filled cache positions: the same integer-exact uniform draws as synth.c's
// synth_uniform_kv_* (draw n of a seed = top 24 bits of lowbias32(lowbias32(seed) + n); value =
// (int)(draw - 2^23) * step in one F32 multiply; bf16 caches round that F32 with round-to-nearest-even
// on its bits), so the bytes equal the host's and a long cache is filled in place without a host copy.
// Like synth.c it draws numbers only.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kMaxHeads = 64;

struct HeadSeeds {
  uint32_t h[kMaxHeads];  // lowbias32(seed) of each kv head's stream
};

__device__ __forceinline__ uint32_t lowbias32(uint32_t x) {
  x ^= x >> 16;
  x *= 2146121005u;
  x ^= x >> 15;
  x *= 2221713035u;
  x ^= x >> 16;
  return x;
}

__device__ __forceinline__ float draw_value(uint32_t hs, uint32_t n, float step) {
  const int32_t iv = (int32_t)(lowbias32(hs + n) >> 8) - 8388608;
  return (float)iv * step;
}

__device__ __forceinline__ uint32_t bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);  // the draws are finite
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// grid (slices, heads): thread i of the launch writes 8 consecutive elements of its head
template <bool BF16>
__global__ __launch_bounds__(256) void k_fill(HeadSeeds s, void *base, int64_t head_stride, int64_t n8, float step) {
  const int j = blockIdx.y;
  const uint32_t hs = s.h[j];
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < n8; c += (int64_t)gridDim.x * 256) {
    const uint32_t n0 = (uint32_t)(c * 8);
    if (BF16) {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w[e] = bf16_bits(draw_value(hs, n0 + 2 * e, step)) | (bf16_bits(draw_value(hs, n0 + 2 * e + 1, step)) << 16);
      uint4 *dst = reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(base) + (size_t)j * head_stride) + c;
      *dst = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
      float *dst = reinterpret_cast<float *>(base) + (size_t)j * head_stride + (size_t)c * 8;
      float4 a, b;
      a.x = draw_value(hs, n0 + 0, step);
      a.y = draw_value(hs, n0 + 1, step);
      a.z = draw_value(hs, n0 + 2, step);
      a.w = draw_value(hs, n0 + 3, step);
      b.x = draw_value(hs, n0 + 4, step);
      b.y = draw_value(hs, n0 + 5, step);
      b.z = draw_value(hs, n0 + 6, step);
      b.w = draw_value(hs, n0 + 7, step);
      reinterpret_cast<float4 *>(dst)[0] = a;
      reinterpret_cast<float4 *>(dst)[1] = b;
    }
  }
}

}  // namespace

// Fill elements 0 .. n-1 of `heads` arrays spaced head_stride elements apart from `base` (one kv head's
// positions 0 .. n/head-1 each), draws 0 .. n-1 of the stream whose seed is seeds_host[j].  n must be a
// multiple of 8 and below 2^32, base 16-byte aligned, head_stride a multiple of 8.  Returns 0, or -1 for
// bad arguments (nothing launched), or the HIP error of the launch.  Asynchronous on `stream`.
extern "C" int synth_dev_fill_kv(const uint32_t *seeds_host, int heads, void *base, int64_t head_stride, int64_t n,
                                 float step, int bf16, void *stream) {
  if (!seeds_host || !base || heads <= 0 || heads > kMaxHeads || n < 0 || n % 8 || n >= (int64_t(1) << 32) ||
      head_stride % 8 || head_stride < n || (reinterpret_cast<uintptr_t>(base) & 15))
    return -1;
  if (n == 0) return 0;
  HeadSeeds s;
  for (int j = 0; j < heads; ++j) s.h[j] = seeds_host[j];
  const int64_t n8 = n / 8;
  int64_t blocks = (n8 + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  const dim3 grid((unsigned)blocks, (unsigned)heads);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (bf16)
    hipLaunchKernelGGL(k_fill<true>, grid, dim3(256), 0, st, s, base, head_stride, n8, step);
  else
    hipLaunchKernelGGL(k_fill<false>, grid, dim3(256), 0, st, s, base, head_stride, n8, step);
  return (int)hipGetLastError();
}
