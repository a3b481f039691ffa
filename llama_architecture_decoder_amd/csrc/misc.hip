// Embedding gather and workspace clearing.
//
// Embedding (main.bend forward: the embedding row of the token, Bands.read_row; bf16 rows widened
// exactly, bf16 being the upper half of an F32): x[b] = emb[tokens[b]].  Token ids live in device
// memory (the previous step's argmax may feed them), so the range check happens here: an id outside
// [0, vocab) sets the sticky status flag and the row's input becomes zeros, so no out-of-bounds read
// can happen.
#include "common.h"

namespace lm {

template <typename WT>
__global__ __launch_bounds__(kThreads) void k_embed(const int32_t *tokens, const WT *emb, int dim, int vocab,
                                                    float *x, int *status) {
  const int b = blockIdx.x;
  const int tok = tokens[b];
  float *xb = x + (size_t)b * dim;
  if (tok < 0 || tok >= vocab) {
    if (threadIdx.x == 0) atomicOr(status, 1);
    for (int i = threadIdx.x; i < dim; i += kThreads) xb[i] = 0.f;
    return;
  }
  const WT *row = emb + (size_t)tok * dim;
  for (int i = threadIdx.x; i < dim; i += kThreads) xb[i] = load_scalar<WT>(row, i);
}

__global__ void k_zero(uint32_t *p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0u;
}

hipError_t launch_embed(int wdtype, const int32_t *tokens, const void *emb, int dim, int vocab, float *x, int B,
                        int *status, hipStream_t s) {
  if (wdtype == LLAMA_BF16)
    hipLaunchKernelGGL((k_embed<bf16_t>), dim3(B), dim3(kThreads), 0, s, tokens,
                       reinterpret_cast<const bf16_t *>(emb), dim, vocab, x, status);
  else
    hipLaunchKernelGGL((k_embed<float>), dim3(B), dim3(kThreads), 0, s, tokens, reinterpret_cast<const float *>(emb),
                       dim, vocab, x, status);
  return hipGetLastError();
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
