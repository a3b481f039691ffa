// Embedding gather and workspace clearing.
//
// Embedding (main.bend forward: the embedding row of the token, Bands.read_row; bf16 rows widened
// exactly, bf16 being the upper half of an F32): x[b] = emb[tokens[b]], one 16-byte slice per thread.
// Token ids live in device memory (the previous step's argmax may feed them), so the range check
// happens here: an id outside
// [0, vocab) sets the sticky status flag and the row's input becomes zeros, so no out-of-bounds read
// can happen.
#include "common.h"

namespace lm {

template <typename WT>
__global__ __launch_bounds__(kThreads) void k_embed(const int32_t *tokens, const WT *emb, int dim, int vocab,
                                                    float *x, int *status, unsigned *epoch) {
  // block (s, b): 16-byte slices s*256 + tid of row b (dim is a multiple of 8)
  constexpr int E = Vec16<WT>::E;
  const int b = blockIdx.y;
  // the step counter (tags of the step's tagged words): the launch boundary publishes it to the
  // step's later launches
  if (epoch && blockIdx.x == 0 && b == 0 && threadIdx.x == 0) epoch[0] = epoch[0] + 1u;
  const int tok = tokens[b];
  const int ci = blockIdx.x * kThreads + threadIdx.x;
  if (ci * E >= dim) return;
  float *xb = x + (size_t)b * dim + (size_t)ci * E;
  float v[E];
  if (tok < 0 || tok >= vocab) {
    if (ci == 0) atomicOr(status, 1);
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = 0.f;
  } else {
    Vec16<WT>::unpack(load16(emb + (size_t)tok * dim + (size_t)ci * E), v);
  }
#pragma unroll
  for (int e = 0; e < E; e += 4) *reinterpret_cast<float4 *>(xb + e) = make_float4(v[e], v[e + 1], v[e + 2], v[e + 3]);
}

__global__ void k_zero(uint32_t *p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0u;
}

hipError_t launch_embed(int wdtype, const int32_t *tokens, const void *emb, int dim, int vocab, float *x, int B,
                        int *status, unsigned *epoch, hipStream_t s) {
  const int E = wdtype == LLAMA_BF16 ? 8 : 4;
  const dim3 grid((dim / E + kThreads - 1) / kThreads, B);
  if (wdtype == LLAMA_BF16)
    launch(k_embed<bf16_t>, grid, dim3(kThreads), s, true, true, tokens, reinterpret_cast<const bf16_t *>(emb), dim,
           vocab, x, status, epoch);
  else
    launch(k_embed<float>, grid, dim3(kThreads), s, true, true, tokens, reinterpret_cast<const float *>(emb), dim,
           vocab, x, status, epoch);
  return hipGetLastError();
}

LaunchEvents &launch_events() {
  static thread_local LaunchEvents ev;
  return ev;
}

hipError_t launch_zero(void *p, size_t bytes, hipStream_t s) {
  const size_t n = bytes / 4;
  if (n == 0) return hipSuccess;
  size_t blocks = (n + kThreads - 1) / kThreads;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_zero, dim3((unsigned)blocks), dim3(kThreads), 0, s, reinterpret_cast<uint32_t *>(p), n);
  return hipGetLastError();
}

}  // namespace lm
