// HBM-streaming matrix-vector products for the batch-1 decode step on gfx950.
//
// y = W x with W [N][K] row-major (row = output, main.bend type LW), F32 or bf16 weights, F32
// arithmetic.  The projections of main.bend "A layer" (block): q/k/v from the attention norm, o with
// the first residual, gate/up from the MLP norm with SwiGLU (silu(g) * u, silu(z) = z / (1 + e^-z)),
// down with the second residual; the q/k/v projection can also finish with RoPE and the cache append
// (EPI_ROPE); and "The model" head_of: logits = W_lm * rmsnorm(x, lnf) with the
// argmax of main.bend `argmax` (first index of the largest value).
//
// The work split and reduction order are described with the block's body in gemv_body.h.
#include "gemv_body.h"

namespace lm {

template <typename WT, int KCH, int EPI, bool NORM>
__global__ __launch_bounds__(kThreads) void k_gemv(GemvArgs a) {
  gemv_body<WT, KCH, EPI, NORM>(a, blockIdx.x, gridDim.x, 0u);
}

// The per-block winners of the LM head, reduced by one block in a second launch: larger value wins,
// equal values keep the lower index, so the result is the first index of the largest logit whatever
// the order of the blocks (main.bend argmax).  Every logit NaN: index 0, as an empty list gives.
__global__ __launch_bounds__(kThreads) void k_argmax_final(const float *part_v, const int *part_i, int n, int ld,
                                                         int32_t *next) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  part_v += (size_t)blockIdx.x * ld;
  part_i += (size_t)blockIdx.x * ld;
  __shared__ float sv[4];
  __shared__ int si[4];
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  constexpr int PER = 8;  // partials per thread per pass, loaded before any compare
  for (int base = 0; base < n; base += PER * kThreads) {
    float vv[PER];
    int iv[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int ix = min(base + tid + k * kThreads, n - 1);
      vv[k] = part_v[ix];
      iv[k] = part_i[ix];
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      if (base + tid + k * kThreads < n && (vv[k] > bv || (vv[k] == bv && iv[k] < bi))) {
        bv = vv[k];
        bi = iv[k];
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o);
    const int oi = __shfl_xor(bi, o);
    if (ov > bv || (ov == bv && oi < bi)) {
      bv = ov;
      bi = oi;
    }
  }
  if (lane == 0) {
    sv[wave] = bv;
    si[wave] = bi;
  }
  lds_barrier();
  if (tid == 0) {
    float fv = sv[0];
    int fi = si[0];
    for (int w = 1; w < 4; ++w)
      if (sv[w] > fv || (sv[w] == fv && si[w] < fi)) {
        fv = sv[w];
        fi = si[w];
      }
    next[blockIdx.x] = (fi == 0x7fffffff) ? 0 : fi;
  }
}

hipError_t launch_argmax_final(const float *part_v, const int *part_i, int n, int ld, int rows, int32_t *next,
                               hipStream_t s) {
  launch(k_argmax_final, dim3(rows), dim3(kThreads), s, false, true, part_v, part_i, n, ld, next);
  return hipGetLastError();
}

template <typename WT, int EPI, bool NORM>
static hipError_t dispatch_kch(int kch, dim3 grid, const GemvArgs &a, hipStream_t s, bool last) {
  switch (kch) {
#define CASE(k)                                                                        \
  case k:                                                                              \
    launch(k_gemv<WT, k, EPI, NORM>, grid, dim3(kThreads), s, true, last, a);          \
    break;
    CASE(1) CASE(2) CASE(3) CASE(4) CASE(5) CASE(6) CASE(7) CASE(8)
#undef CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

static int rows_per_group(int kch, int pairs) {
  int raw = 16 / (kch * pairs);
  return raw >= 8 ? 8 : raw >= 4 ? 4 : raw >= 2 ? 2 : 1;
}

int gemv_supported(int wdtype, int K) {
  const int E = wdtype == LLAMA_BF16 ? 8 : 4;
  if (K <= 0 || K % E) return 0;
  const int kch = (K / E + kThreads - 1) / kThreads;
  return kch >= 1 && kch <= 8;
}

template <typename WT>
static hipError_t launch_typed(GemvEpi epi, bool norm, GemvArgs a, int grid_cap, hipStream_t s) {
  const int E = Vec16<WT>::E;
  const int kch = (a.K / E + kThreads - 1) / kThreads;
  const int R = rows_per_group(kch, epi == EPI_SWIGLU ? 2 : 1);
  a.ngroups = (a.N + R - 1) / R;
  int grid = a.ngroups < grid_cap ? a.ngroups : grid_cap;
  if (epi == EPI_ARGMAX && grid > kLmGridMax) grid = kLmGridMax;
  if (grid < 1) grid = 1;
  const dim3 g(grid);
  if (epi == EPI_STORE && norm) return dispatch_kch<WT, EPI_STORE, true>(kch, g, a, s, true);
  if (epi == EPI_ROPE && norm) {
    if (R % 2) return hipErrorInvalidValue;
    return dispatch_kch<WT, EPI_ROPE, true>(kch, g, a, s, true);
  }
  if (epi == EPI_STORE && !norm) return dispatch_kch<WT, EPI_STORE, false>(kch, g, a, s, true);
  if (epi == EPI_RESID && !norm) return dispatch_kch<WT, EPI_RESID, false>(kch, g, a, s, true);
  if (epi == EPI_SWIGLU && norm) return dispatch_kch<WT, EPI_SWIGLU, true>(kch, g, a, s, true);
  if (epi == EPI_ARGMAX && norm) {
    const bool reduce = a.next != nullptr;
    hipError_t e = dispatch_kch<WT, EPI_ARGMAX, true>(kch, g, a, s, !reduce);
    if (e != hipSuccess || !reduce) return e;
    return launch_argmax_final(a.part_v, a.part_i, grid, grid, 1, a.next, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemv(int wdtype, GemvEpi epi, bool norm, const GemvArgs &a, int grid_cap, hipStream_t s) {
  if (wdtype == LLAMA_BF16) return launch_typed<bf16_t>(epi, norm, a, grid_cap, s);
  return launch_typed<float>(epi, norm, a, grid_cap, s);
}

}  // namespace lm
