// Matrix products for several tokens at once (batched decode rows) on gfx950 matrix cores.
//
// Y[M][N] = X[M][K] W[N][K]^T with bf16 weights (row = output, main.bend type LW) and M <= 64 token rows
// (nest card `decode_rows`: every cache row one token).  Weights are streamed from HBM once per call, as
// in the single-token GEMV; the matrix cores do the products.  X is F32: it is carried as two bf16
// operands, hi = bf16(X) and lo = bf16(X - hi) (X - hi is exact in F32), and both meet the same weight
// fragment, so products are exact and the result matches an F32 product to about 2^-17 relative.
//
// v_mfma_f32_16x16x32_bf16: A (16 x 32) lane l holds A[l%16][8(l/16) .. +8], B (32 x 16) lane l holds
// B[8(l/16) .. +8][l%16], C (16 x 16) lane l holds C[4(l/16) + r][l%16], r < 4.  Here A = a 16-token tile
// of X, B = 16 weight rows transposed: lane l loads 16 contiguous bytes of weight row n0 + l%16.
// A block owns 16 weight rows (two sets for SwiGLU: gate and up); its 4 wavefronts take interleaved
// 32-element K steps (a block step reads 256 contiguous bytes of each row) and their sums are added in a
// fixed order through LDS.  Epilogues as the GEMV: store, residual, SwiGLU, RoPE + cache append, LM head
// (+ block winners).
#include "common.h"

namespace lm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// X -> (hi, lo) bf16 operands, optionally RMS-normalised first: X = g * (x * (1 / sqrt(sum x^2 / K + eps)))
// (main.bend rmsnorm).  Block b = token row b; rows b >= M (padding to a 16-row tile) are zeros.
template <typename GT, bool NORM>
__global__ __launch_bounds__(kThreads) void k_split(SplitArgs a) {
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  bf16_t *hi = a.xhi + (size_t)b * a.ldx;
  bf16_t *lo = a.xlo + (size_t)b * a.ldx;
  if (b >= a.M) {
    for (int k = 2 * tid; k < a.K; k += 2 * kThreads) {
      *reinterpret_cast<uint32_t *>(hi + k) = 0u;
      *reinterpret_cast<uint32_t *>(lo + k) = 0u;
    }
    return;
  }
  const float *x = a.x + (size_t)b * a.ldin;
  float r = 1.f;
  if (NORM) {
    __shared__ float ss_w[4];
    float ss = 0.f;
    for (int k = tid; k < a.K; k += kThreads) ss += x[k] * x[k];
    ss = wave_sum(ss);
    if (lane == 0) ss_w[wave] = ss;
    lds_barrier();
    const float tot = (ss_w[0] + ss_w[1]) + (ss_w[2] + ss_w[3]);
    r = 1.0f / sqrtf(tot / (float)a.K + a.eps);
  }
  const GT *g = reinterpret_cast<const GT *>(a.gain);
  // pairs of numbers (K is even): one packed conversion per pair
  for (int k = 2 * tid; k < a.K; k += 2 * kThreads) {
    const float v0 = NORM ? load_scalar<GT>(g, k) * (x[k] * r) : x[k];
    const float v1 = NORM ? load_scalar<GT>(g, k + 1) * (x[k + 1] * r) : x[k + 1];
    uint32_t h, l;
    split_bf16x2(v0, v1, h, l);
    *reinterpret_cast<uint32_t *>(hi + k) = h;
    *reinterpret_cast<uint32_t *>(lo + k) = l;
  }
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

template <int MT, int EPI>
__global__ __launch_bounds__(kThreads) void k_gemm_skinny(GemmArgs a) {
  constexpr int PAIRS = (EPI == EPI_SWIGLU) ? 2 : 1;
  constexpr int U = 4;  // K steps per wavefront per iteration (loads in flight)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * 16;
  const int nl = lane & 15, q = lane >> 4;
  const int row = min(n0 + nl, a.N - 1);
  const bf16_t *wrow[PAIRS];
  if (EPI == EPI_SWIGLU) {
    wrow[0] = reinterpret_cast<const bf16_t *>(a.w[0]) + (size_t)row * a.K;
    wrow[PAIRS - 1] = reinterpret_cast<const bf16_t *>(a.w[1]) + (size_t)row * a.K;
  } else {
    const int wr = EPI == EPI_ROPE ? rope_row(row, a.ra.dim + a.ra.kvw, a.ra.hshift) : row;
    const bf16_t *base = reinterpret_cast<const bf16_t *>(wr >= a.rs[2] ? a.w[2] : (wr >= a.rs[1] ? a.w[1] : a.w[0]));
    const int r0 = wr >= a.rs[2] ? a.rs[2] : (wr >= a.rs[1] ? a.rs[1] : 0);
    wrow[0] = base + (size_t)(wr - r0) * a.K;
  }
  f32x4 acc[PAIRS][MT];
#pragma unroll
  for (int p = 0; p < PAIRS; ++p)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[p][m] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int ksteps = a.K / 32;
  for (int ks0 = wave; ks0 < ksteps; ks0 += 4 * U) {
    u32x4 wv[PAIRS][U], xh[U][MT], xl[U][MT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ks = min(ks0 + 4 * u, ksteps - 1);  // a step past the end repeats the last one, unused
      const size_t ko = (size_t)ks * 32 + q * 8;
#pragma unroll
      for (int p = 0; p < PAIRS; ++p) wv[p][u] = load_stream16(wrow[p] + ko);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        xh[u][m] = load16(a.xhi + (size_t)(m * 16 + nl) * a.ldx + ko);
        xl[u][m] = load16(a.xlo + (size_t)(m * 16 + nl) * a.ldx + ko);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (ks0 + 4 * u < ksteps) {
#pragma unroll
        for (int p = 0; p < PAIRS; ++p)
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            acc[p][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xh[u][m]), as_bf16x8(wv[p][u]), acc[p][m], 0, 0, 0);
            acc[p][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xl[u][m]), as_bf16x8(wv[p][u]), acc[p][m], 0, 0, 0);
          }
      }
    }
  }

  // the 4 wavefronts' sums, added in a fixed order; lane l holds C[4q + r][nl] of each tile
  __shared__ float red[4][PAIRS][MT * 16][16];
#pragma unroll
  for (int p = 0; p < PAIRS; ++p)
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave][p][m * 16 + 4 * q + r][nl] = acc[p][m][r];
  lds_barrier();
  for (int idx = tid; idx < MT * 16 * 16; idx += kThreads) {
    const int t = idx / 16, j = idx % 16, n = n0 + j;
    float v[PAIRS];
#pragma unroll
    for (int p = 0; p < PAIRS; ++p) v[p] = (red[0][p][t][j] + red[1][p][t][j]) + (red[2][p][t][j] + red[3][p][t][j]);
    if (t < a.M && n < a.N) {
      float *y = a.y + (size_t)t * a.ldy + n;
      if (EPI == EPI_STORE) {
        *y = v[0];
      } else if (EPI == EPI_RESID) {
        *y = a.res[(size_t)t * a.ldres + n] + v[0];
      } else if (EPI == EPI_SWIGLU) {
        *y = (v[0] / (1.0f + expf(-v[0]))) * v[PAIRS - 1];
      } else if (EPI == EPI_ROPE) {
        const int j2 = j ^ 1;  // the pair partner (logical rows 2i, 2i+1), in this block's 16 rows
        const float pv = (red[0][0][t][j2] + red[1][0][t][j2]) + (red[2][0][t][j2] + red[3][0][t][j2]);
        const size_t ci = (size_t)a.ra.pos[t] * a.ra.half + rope_pair_index(n, a.ra.hshift);
        const bool qk = n < a.ra.dim + a.ra.kvw;
        rope_append(a.ra, a.y + (size_t)t * a.ldy, t, n, v[0], pv, qk ? a.ra.rope_cs[ci] : 0.f,
                    qk ? a.ra.rope_sn[ci] : 0.f);
      } else if (a.y) {
        *y = v[0];
      }
    }
    if (EPI == EPI_ARGMAX) red[0][0][t][j] = (t < a.M && n < a.N) ? v[0] : -INFINITY;
  }
  if (EPI == EPI_ARGMAX) {
    lds_barrier();
    // winner of this block's 16 rows for every token: first index of the largest value
    for (int t = tid; t < MT * 16; t += kThreads) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
      for (int j = 0; j < 16; ++j) {
        const float v = red[0][0][t][j];
        if (v > bv) {
          bv = v;
          bi = n0 + j;
        }
      }
      if (t < a.M) {
        a.part_v[(size_t)t * a.part_ld + blockIdx.x] = bv;
        a.part_i[(size_t)t * a.part_ld + blockIdx.x] = bi;
      }
    }
  }
}

int gemm_skinny_supported(int wdtype, int K, int M) {
  return wdtype == LLAMA_BF16 && K % 32 == 0 && M >= 1 && M <= kMaxBatch;
}

hipError_t launch_split(int gdtype, bool norm, const SplitArgs &a, int mpad, hipStream_t s) {
  const dim3 g(mpad);
  if (norm) {
    if (gdtype == LLAMA_BF16)
      launch(k_split<bf16_t, true>, g, dim3(kThreads), s, true, false, a);
    else
      launch(k_split<float, true>, g, dim3(kThreads), s, true, false, a);
  } else {
    launch(k_split<float, false>, g, dim3(kThreads), s, true, false, a);
  }
  return hipGetLastError();
}

template <int MT>
static hipError_t launch_mt(GemvEpi epi, const GemmArgs &a, hipStream_t s, bool last) {
  const dim3 g((a.N + 15) / 16);
  switch (epi) {
    case EPI_STORE: launch(k_gemm_skinny<MT, EPI_STORE>, g, dim3(kThreads), s, false, last, a); break;
    case EPI_RESID: launch(k_gemm_skinny<MT, EPI_RESID>, g, dim3(kThreads), s, false, last, a); break;
    case EPI_SWIGLU: launch(k_gemm_skinny<MT, EPI_SWIGLU>, g, dim3(kThreads), s, false, last, a); break;
    case EPI_ARGMAX: launch(k_gemm_skinny<MT, EPI_ARGMAX>, g, dim3(kThreads), s, false, last, a); break;
    case EPI_ROPE: launch(k_gemm_skinny<MT, EPI_ROPE>, g, dim3(kThreads), s, false, last, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_skinny(GemvEpi epi, const GemmArgs &a, hipStream_t s, bool last) {
  const int mt = (a.M + 15) / 16;
  switch (mt) {
    case 1: return launch_mt<1>(epi, a, s, last);
    case 2: return launch_mt<2>(epi, a, s, last);
    case 3: return launch_mt<3>(epi, a, s, last);
    case 4: return launch_mt<4>(epi, a, s, last);
  }
  return hipErrorInvalidValue;
}

int gemm_skinny_blocks(int N) { return (N + 15) / 16; }

}  // namespace lm
