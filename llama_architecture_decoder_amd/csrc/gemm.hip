// Matrix products for several tokens at once (batched decode rows) on gfx950 matrix cores.
//
// Y[M][N] = X[M][K] W[N][K]^T with bf16 weights (row = output, main.bend type LW) and M <= 64 token rows
// (nest card `decode_rows`: every cache row one token).  Weights are streamed from HBM once per call, as
// in the single-token GEMV; the matrix cores do the products.  X is F32: it is carried as two bf16
// operands, hi = bf16(X) and lo = bf16(X - hi) (X - hi is exact in F32), and both meet the same weight
// fragment, so products are exact and the result matches an F32 product to about 2^-17 relative.
//
// v_mfma_f32_16x16x32_bf16: A (16 x 32) lane l holds A[l%16][8(l/16) .. +8], B (32 x 16) lane l holds
// B[8(l/16) .. +8][l%16], C (16 x 16) lane l holds C[4(l/16) + r][l%16], r < 4.  A = a 16-token tile of
// X (from LDS), B = 16 weight rows transposed: lane l loads 16 contiguous bytes of weight row l%16.
//
// k_gemm_rows: block (bx, s) owns 128 consecutive outputs (wave w: outputs 32w .. +32 as two 16-row
// tiles; SwiGLU: 64 outputs, wave w's tiles are the gate and the up rows of outputs 16w .. +16) over the
// s-th slice of K.  X tiles of 128 columns are staged in LDS once for the 4 waves (double buffered up to
// 2 token tiles); each wave keeps the weight loads of the next two tiles (one at 4 token tiles) in flight
// while it multiplies the current one.  The
// weights are loaded in 256-byte runs of a row (the MFMA layout would give 64-byte pieces of 16 rows per
// load, which streams from HBM markedly slower) and rearranged through the wave's own LDS tile.  With one slice
// the epilogue runs in the kernel; with several, each slice writes its partial sums and a reduce kernel
// adds them in slice order (deterministic) and runs the epilogue.  The number of slices is chosen so
// the launch has at most 512 blocks (two resident per CU): at these sizes every CU must see all of X, so
// X re-reads, not weights, decide how many output rows a block should own.
//
// Epilogues: STORE, RESID (y = res + XW^T), SWIGLU (silu(gate) * up, written straight as the next
// product's bf16 hi/lo operands), ROPE (RoPE + cache append, as the GEMV), ARGMAX (LM head: logits and
// per-block winners).  The residual + RMSNorm + split of the next product's input are fused into the
// reduce kernel k_rows_reduce_norm (one block per token row).
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
  // four numbers per thread when K allows (16-byte loads), else pairs (K is even): one packed conversion
  // per pair
  if (a.K % 4 == 0 && a.ldin % 4 == 0 && a.ldx % 4 == 0) {
    for (int k = 4 * tid; k < a.K; k += 4 * kThreads) {
      const float4 v = *reinterpret_cast<const float4 *>(x + k);
      float f[4] = {v.x, v.y, v.z, v.w};
      if (NORM)
#pragma unroll
        for (int e = 0; e < 4; ++e) f[e] = load_scalar<GT>(g, k + e) * (f[e] * r);
      uint32_t h0, l0, h1, l1;
      split_bf16x2(f[0], f[1], h0, l0);
      split_bf16x2(f[2], f[3], h1, l1);
      *reinterpret_cast<uint2 *>(hi + k) = make_uint2(h0, h1);
      *reinterpret_cast<uint2 *>(lo + k) = make_uint2(l0, l1);
    }
    return;
  }
  for (int k = 2 * tid; k < a.K; k += 2 * kThreads) {
    const float v0 = NORM ? load_scalar<GT>(g, k) * (x[k] * r) : x[k];
    const float v1 = NORM ? load_scalar<GT>(g, k + 1) * (x[k + 1] * r) : x[k + 1];
    uint32_t h, l;
    split_bf16x2(v0, v1, h, l);
    *reinterpret_cast<uint32_t *>(hi + k) = h;
    *reinterpret_cast<uint32_t *>(lo + k) = l;
  }
}

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

constexpr int kRT = 128;           // K columns per tile
constexpr int kRowsOut = 128;      // outputs per block (SwiGLU: 64)
constexpr int kLdt = kRT + 8;      // LDS row of an X tile (bf16): 272 bytes, 16-byte reads of 16 rows hit distinct banks

// weight row (in the stacked q|k|v or plain matrix) that output n of the epilogue reads
template <int EPI>
__device__ __forceinline__ const bf16_t *weight_row(const GemmArgs &a, int n, int which) {
  if (EPI == EPI_SWIGLU) return reinterpret_cast<const bf16_t *>(a.w[which]) + (size_t)n * a.K;
  const int wr = EPI == EPI_ROPE ? rope_row(n, a.ra.dim + a.ra.kvw, a.ra.hshift) : n;
  const int seg = wr >= a.rs[2] ? 2 : (wr >= a.rs[1] ? 1 : 0);
  return reinterpret_cast<const bf16_t *>(a.w[seg]) + (size_t)(wr - a.rs[seg]) * a.K;
}

// Two blocks per CU: from 3 token tiles on, one X buffer (to fit the LDS) and, at 4 tiles, the weights
// requested one tile ahead instead of two (to fit the registers without spilling).  Measured against
// one block per CU with two buffers: 40-row decode 9% faster, 64-row decode 10% faster.
template <int MT, int EPI, bool PART>
__global__ __launch_bounds__(kThreads, 2) void k_gemm_rows(GemmArgs a) {
  constexpr bool SW = EPI == EPI_SWIGLU;
  constexpr int ROWS = SW ? kRowsOut / 2 : kRowsOut;
  constexpr int XCH = MT * 16 * kRT / 8 / kThreads;  // 16-byte chunks of one X array per thread per tile (= MT)
  constexpr int XB = MT >= 3 ? 1 : 2;  // X tile buffers
  __shared__ __attribute__((aligned(16))) bf16_t xs[XB][2][MT * 16 * kLdt];  // [buffer][hi, lo]
  __shared__ __attribute__((aligned(16))) bf16_t ws[4][32 * kLdt];          // each wave's weight tile
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, q8 = (lane >> 4) * 8;
  const int nb = blockIdx.x * ROWS;
  const int ntile_all = a.K / kRT;
  const int t0 = blockIdx.y * a.tiles_per_slice;
  const int nt = min(a.tiles_per_slice, ntile_all - t0);  // >= 1 (slices are never empty)

  // The wave's 32 weight rows (SwiGLU: rows 0..15 gate, 16..31 up) are read in runs of 256 bytes: load
  // i brings rows 4i .. 4i+3, lane l the 16 bytes at 8 (l%16) of row 4i + l/16.  They reach the MFMA
  // layout (lane l: row l%16 of a 16-row tile) through the wave's own LDS tile.
  const bf16_t *wrow[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 4 * i + (lane >> 4);
    const int n = min(SW ? nb + 16 * wave + (r & 15) : nb + 32 * wave + r, a.N - 1);
    wrow[i] = weight_row<EPI>(a, n, SW ? r >> 4 : 0) + (size_t)t0 * kRT + l16 * 8;
  }
  // X staging: chunk c = tid + 256 i is row c / 16, columns 8 (c % 16) .. +8 of the tile
  const bf16_t *xg[2][XCH];
  int xo[XCH];
#pragma unroll
  for (int i = 0; i < XCH; ++i) {
    const int c = tid + kThreads * i, r = c >> 4, cc = (c & 15) * 8;
    xo[i] = r * kLdt + cc;
    xg[0][i] = a.xhi + (size_t)r * a.ldx + (size_t)t0 * kRT + cc;
    xg[1][i] = a.xlo + (size_t)r * a.ldx + (size_t)t0 * kRT + cc;
  }
  bf16_t *wl = ws[wave];

  u32x4 xr[2][XCH];
  u32x4 w0[8], w1[8], w2[8];
  auto load_x = [&](int t) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < XCH; ++i) xr[h][i] = load16(xg[h][i] + (size_t)t * kRT);
  };
  auto stash_x = [&](int buf) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < XCH; ++i) *reinterpret_cast<u32x4 *>(&xs[buf][h][xo[i]]) = xr[h][i];
  };
  auto load_w = [&](u32x4 (&w)[8], int t) {
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = load_stream16(wrow[i] + (size_t)t * kRT);
  };
  f32x4 acc[MT][2];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int buf, const u32x4 (&w)[8]) {
    // the weight tile into the wave's LDS rows (LDS operations of a wave complete in order, so the
    // reads below see these writes and the writes of the next tile follow these reads)
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4 *>(&wl[(4 * i + (lane >> 4)) * kLdt + l16 * 8]) = w[i];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 b[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = *reinterpret_cast<const u32x4 *>(&wl[(16 * j + l16) * kLdt + ks * 32 + q8]);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const int off = (m * 16 + l16) * kLdt + ks * 32 + q8;
        const u32x4 ah = *reinterpret_cast<const u32x4 *>(&xs[buf][0][off]);
        const u32x4 al = *reinterpret_cast<const u32x4 *>(&xs[buf][1][off]);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[m][j] = mfma16(ah, b[j], acc[m][j]);
          acc[m][j] = mfma16(al, b[j], acc[m][j]);
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  };
  // one tile: the X tile after it (LDS, distance 1) and the weights two tiles ahead (registers, a ring of
  // three) are requested first, X before weights so that waiting for X leaves the weights in flight; LDS
  // barriers do not wait for global loads
  constexpr int WD = MT >= 4 ? 1 : 2;  // how many tiles ahead the weights are requested
  auto step = [&](int t, const u32x4 (&wcur)[8], u32x4 (&wahead)[8]) {
    if (t + 1 < nt) load_x(t + 1);
    if (t + WD < nt) load_w(wahead, t + WD);
    compute(XB == 2 ? (t & 1) : 0, wcur);
    if (t + 1 < nt) {
      if (XB == 1) lds_barrier();  // every wave is done with the one X tile
      stash_x(XB == 2 ? ((t + 1) & 1) : 0);
      lds_barrier();
    }
  };
  load_x(0);
  load_w(w0, 0);
  if (WD == 2 && nt > 1) load_w(w1, 1);
  stash_x(0);
  lds_barrier();
  if constexpr (WD == 2) {
    for (int t = 0; t < nt; t += 3) {
      step(t, w0, w2);
      if (t + 1 >= nt) break;
      step(t + 1, w1, w0);
      if (t + 2 >= nt) break;
      step(t + 2, w2, w1);
    }
  } else {
    for (int t = 0; t < nt; t += 2) {
      step(t, w0, w1);
      if (t + 1 >= nt) break;
      step(t + 1, w1, w0);
    }
  }

  // lane holds C[token 4(lane/16) + r][output l16] of tile (m, j)
  if (PART) {
    // partial sums of this slice: part[s][t][n], n over the N (SwiGLU: 2N, gate then up) outputs
    const int nout = SW ? 2 * a.N : a.N;
    float *pp = a.part + (size_t)blockIdx.y * a.M * nout;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = m * 16 + (lane >> 4) * 4 + r;
        if (t >= a.M) continue;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int n = SW ? nb + 16 * wave + l16 : nb + 32 * wave + 16 * j + l16;
          if (n < a.N) pp[(size_t)t * nout + (SW ? j * a.N : 0) + n] = acc[m][j][r];
        }
      }
    return;
  }
  if (EPI == EPI_ARGMAX) {
    // per token: this block's largest logit and its first index
    __shared__ float bv_s[4][MT * 16];
    __shared__ int bi_s[4][MT * 16];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = m * 16 + (lane >> 4) * 4 + r;
        float bv = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int n = nb + 32 * wave + 16 * j + l16;
          const float v = acc[m][j][r];
          if (t < a.M && n < a.N) {
            if (a.y) a.y[(size_t)t * a.ldy + n] = v;
            if (v > bv) {
              bv = v;
              bi = n;
            }
          }
        }
        // over the 16 lanes of the row (outputs l16); ties keep the lower index
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
          const float ov = __shfl_xor(bv, o);
          const int oi = __shfl_xor(bi, o);
          if (ov > bv || (ov == bv && oi < bi)) {
            bv = ov;
            bi = oi;
          }
        }
        if (l16 == 0) {
          bv_s[wave][t] = bv;
          bi_s[wave][t] = bi;
        }
      }
    lds_barrier();
    for (int t = tid; t < a.M; t += kThreads) {
      float bv = bv_s[0][t];
      int bi = bi_s[0][t];
#pragma unroll
      for (int w = 1; w < 4; ++w)
        if (bv_s[w][t] > bv || (bv_s[w][t] == bv && bi_s[w][t] < bi)) {
          bv = bv_s[w][t];
          bi = bi_s[w][t];
        }
      a.part_v[(size_t)t * a.part_ld + blockIdx.x] = bv;
      a.part_i[(size_t)t * a.part_ld + blockIdx.x] = bi;
    }
    return;
  }
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = m * 16 + (lane >> 4) * 4 + r;
      if (SW) {
        // m = silu(gate) * up, straight to the next product's operands: lanes l, l+1 hold outputs n, n+1
        const int n = nb + 16 * wave + l16;
        const float gt = acc[m][0][r], up = acc[m][1][r];
        const float v = (gt / (1.0f + expf(-gt))) * up;
        const float v1 = __shfl_xor(v, 1);
        if (t < a.M && n < a.N && (n & 1) == 0) {
          uint32_t h, l;
          split_bf16x2(v, v1, h, l);
          *reinterpret_cast<uint32_t *>(a.ohi + (size_t)t * a.ldo + n) = h;
          *reinterpret_cast<uint32_t *>(a.olo + (size_t)t * a.ldo + n) = l;
        }
        continue;
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = nb + 32 * wave + 16 * j + l16;
        const float v = acc[m][j][r];
        if (EPI == EPI_ROPE) {
          const float pv = __shfl_xor(v, 1);  // the pair partner: logical rows 2i, 2i + 1
          if (t < a.M && n < a.N) {
            const bool qk = n < a.ra.dim + a.ra.kvw;
            const size_t ci = (size_t)a.ra.pos[t] * a.ra.half + rope_pair_index(n, a.ra.hshift);
            rope_append(a.ra, a.y + (size_t)t * a.ldy, t, n, v, pv, qk ? a.ra.rope_cs[ci] : 0.f,
                        qk ? a.ra.rope_sn[ci] : 0.f);
          }
        } else if (t < a.M && n < a.N) {
          float *y = a.y + (size_t)t * a.ldy + n;
          *y = EPI == EPI_RESID ? a.res[(size_t)t * a.ldres + n] + v : v;
        }
      }
    }
}

// Sum of the slices' partial sums in slice order, then the epilogue; thread = a pair of outputs (n, n+1)
// of token row blockIdx.y.  ROPE needs both numbers of a pair; SWIGLU writes the next operands.
template <int EPI>
__global__ __launch_bounds__(kThreads) void k_rows_reduce(GemmArgs a, int S) {
  constexpr bool SW = EPI == EPI_SWIGLU;
  const int t = blockIdx.y;
  const int n = 2 * (blockIdx.x * kThreads + threadIdx.x);
  if (n >= a.N) return;
  const int nout = SW ? 2 * a.N : a.N;
  const float *pp = a.part + (size_t)t * nout + n;
  const size_t sstride = (size_t)a.M * nout;
  float v0 = 0.f, v1 = 0.f, u0 = 0.f, u1 = 0.f;
  for (int s = 0; s < S; ++s) {
    const float2 p = *reinterpret_cast<const float2 *>(pp + s * sstride);
    v0 += p.x;
    v1 += p.y;
    if (SW) {
      const float2 q = *reinterpret_cast<const float2 *>(pp + s * sstride + a.N);
      u0 += q.x;
      u1 += q.y;
    }
  }
  if (SW) {
    const float m0 = (v0 / (1.0f + expf(-v0))) * u0, m1 = (v1 / (1.0f + expf(-v1))) * u1;
    uint32_t h, l;
    split_bf16x2(m0, m1, h, l);
    *reinterpret_cast<uint32_t *>(a.ohi + (size_t)t * a.ldo + n) = h;
    *reinterpret_cast<uint32_t *>(a.olo + (size_t)t * a.ldo + n) = l;
  } else if (EPI == EPI_ROPE) {
    float *y = a.y + (size_t)t * a.ldy;
    float c = 0.f, s = 0.f;
    if (n < a.ra.dim + a.ra.kvw) {
      const size_t ci = (size_t)a.ra.pos[t] * a.ra.half + rope_pair_index(n, a.ra.hshift);
      c = a.ra.rope_cs[ci];
      s = a.ra.rope_sn[ci];
    }
    rope_append(a.ra, y, t, n, v0, v1, c, s);
    rope_append(a.ra, y, t, n + 1, v1, v0, c, s);
  } else {
    float *y = a.y + (size_t)t * a.ldy + n;
    if (EPI == EPI_RESID) {
      const float *r = a.res + (size_t)t * a.ldres + n;
      v0 += r[0];
      v1 += r[1];
    }
    y[0] = v0;
    y[1] = v1;
  }
}

// x[t] = x[t] + sum of the slices' partials (slice order), stored; then the next product's operands
// g * (x * (1 / sqrt(sum x^2 / N + eps))) as bf16 hi + lo (main.bend rmsnorm).  Block = token row t, 1024
// threads with 4 consecutive numbers each, every slice's partial loaded before any is added.
constexpr int kNormThreads = 1024;
template <typename GT>
__global__ __launch_bounds__(kNormThreads) void k_rows_reduce_norm(RowsNormArgs a) {
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float *pp = a.part + (size_t)t * a.N;
  const size_t sstride = (size_t)a.M * a.N;
  float *x = a.x + (size_t)t * a.ldx;
  float ss = 0.f;
  for (int n = 4 * tid; n < a.N; n += 4 * kNormThreads) {
    const float4 r = *reinterpret_cast<const float4 *>(x + n);  // the residual stream
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (a.S == 2) {  // the usual split: both partials, no clamped repeats
      const float4 p0 = *reinterpret_cast<const float4 *>(pp + n), p1 = *reinterpret_cast<const float4 *>(pp + sstride + n);
      acc = make_float4((acc.x + p0.x) + p1.x, (acc.y + p0.y) + p1.y, (acc.z + p0.z) + p1.z, (acc.w + p0.w) + p1.w);
    }
    for (int s0 = 0; s0 < a.S && a.S != 2; s0 += 8) {
      float4 p[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        p[k] = *reinterpret_cast<const float4 *>(pp + (size_t)min(s0 + k, a.S - 1) * sstride + n);
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (s0 + k < a.S) {
          acc.x += p[k].x;
          acc.y += p[k].y;
          acc.z += p[k].z;
          acc.w += p[k].w;
        }
    }
    const float4 v = make_float4(r.x + acc.x, r.y + acc.y, r.z + acc.z, r.w + acc.w);
    *reinterpret_cast<float4 *>(x + n) = v;
    ss += (v.x * v.x + v.y * v.y) + (v.z * v.z + v.w * v.w);
  }
  __shared__ float ss_w[kNormThreads / 64];
  ss = wave_sum(ss);
  if (lane == 0) ss_w[wave] = ss;
  lds_barrier();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < kNormThreads / 64; ++w) tot += ss_w[w];
  const float r = 1.0f / sqrtf(tot / (float)a.N + a.eps);
  const GT *g = reinterpret_cast<const GT *>(a.gain);
  for (int n = 4 * tid; n < a.N; n += 4 * kNormThreads) {
    const float4 v = *reinterpret_cast<const float4 *>(x + n);  // this thread's own store above
    uint32_t h0, l0, h1, l1;
    split_bf16x2(load_scalar<GT>(g, n) * (v.x * r), load_scalar<GT>(g, n + 1) * (v.y * r), h0, l0);
    split_bf16x2(load_scalar<GT>(g, n + 2) * (v.z * r), load_scalar<GT>(g, n + 3) * (v.w * r), h1, l1);
    *reinterpret_cast<uint2 *>(a.xhi + (size_t)t * a.ldo + n) = make_uint2(h0, h1);
    *reinterpret_cast<uint2 *>(a.xlo + (size_t)t * a.ldo + n) = make_uint2(l0, l1);
  }
}

int gemm_rows_supported(int wdtype, int K, int M) {
  return wdtype == LLAMA_BF16 && K % kRT == 0 && M >= 1 && M <= kMaxBatch;
}

int gemm_rows_blocks(int N, bool swiglu) {
  const int rows = swiglu ? kRowsOut / 2 : kRowsOut;
  return (N + rows - 1) / rows;
}

// K slices for at most `target` blocks in all (one round of resident blocks: a second, partial round
// would cost as much as the first), never an empty slice
int gemm_rows_slices(int N, int K, bool swiglu, int target) {
  const int nb = gemm_rows_blocks(N, swiglu);
  const int ntile = K / kRT;
  int s = target / nb;
  if (s < 1) s = 1;
  if (s > ntile) s = ntile;
  const int per = (ntile + s - 1) / s;
  return (ntile + per - 1) / per;
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

template <int MT, bool PART>
static void launch_rows_mt(GemvEpi epi, const GemmArgs &a, dim3 g, hipStream_t s, bool first, bool last) {
  switch (epi) {
    case EPI_STORE: launch(k_gemm_rows<MT, EPI_STORE, PART>, g, dim3(kThreads), s, first, last, a); break;
    case EPI_RESID: launch(k_gemm_rows<MT, EPI_RESID, PART>, g, dim3(kThreads), s, first, last, a); break;
    case EPI_SWIGLU: launch(k_gemm_rows<MT, EPI_SWIGLU, PART>, g, dim3(kThreads), s, first, last, a); break;
    case EPI_ROPE: launch(k_gemm_rows<MT, EPI_ROPE, PART>, g, dim3(kThreads), s, first, last, a); break;
    case EPI_ARGMAX:
      if constexpr (!PART) launch(k_gemm_rows<MT, EPI_ARGMAX, false>, g, dim3(kThreads), s, first, last, a);
      break;
  }
}

template <int MT>
static hipError_t launch_rows(GemvEpi epi, const GemmArgs &a, int S, bool part, hipStream_t s, bool first, bool last) {
  const dim3 g(gemm_rows_blocks(a.N, epi == EPI_SWIGLU), S);
  if (part)
    launch_rows_mt<MT, true>(epi, a, g, s, first, last);
  else
    launch_rows_mt<MT, false>(epi, a, g, s, first, last);
  return hipGetLastError();
}

hipError_t launch_gemm_rows(GemvEpi epi, GemmArgs a, int S, hipStream_t s, bool first, bool last) {
  if (a.K % kRT != 0 || a.M < 1 || a.M > kMaxBatch || S < 1) return hipErrorInvalidValue;
  if (S > 1 && epi == EPI_ARGMAX) return hipErrorInvalidValue;
  const int ntile = a.K / kRT;
  a.tiles_per_slice = (ntile + S - 1) / S;
  if ((S - 1) * a.tiles_per_slice >= ntile) return hipErrorInvalidValue;  // an empty slice
  // RESID always leaves partial sums (slice 0 alone when S = 1): k_rows_reduce_norm adds them to the
  // residual stream and forms the next product's operands
  const bool part = S > 1 || epi == EPI_RESID;
  const bool reduce = S > 1 && epi != EPI_RESID;
  hipError_t e = hipErrorInvalidValue;
  switch ((a.M + 15) / 16) {
    case 1: e = launch_rows<1>(epi, a, S, part, s, first, last && !reduce); break;
    case 2: e = launch_rows<2>(epi, a, S, part, s, first, last && !reduce); break;
    case 3: e = launch_rows<3>(epi, a, S, part, s, first, last && !reduce); break;
    case 4: e = launch_rows<4>(epi, a, S, part, s, first, last && !reduce); break;
  }
  if (e != hipSuccess || !reduce) return e;
  const dim3 g((a.N / 2 + kThreads - 1) / kThreads, a.M);
  switch (epi) {
    case EPI_STORE: launch(k_rows_reduce<EPI_STORE>, g, dim3(kThreads), s, false, last, a, S); break;
    case EPI_SWIGLU: launch(k_rows_reduce<EPI_SWIGLU>, g, dim3(kThreads), s, false, last, a, S); break;
    case EPI_ROPE: launch(k_rows_reduce<EPI_ROPE>, g, dim3(kThreads), s, false, last, a, S); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_rows_reduce_norm(int gdtype, const RowsNormArgs &a, hipStream_t s, bool last) {
  if (a.N % 4 != 0) return hipErrorInvalidValue;
  if (gdtype == LLAMA_BF16)
    launch(k_rows_reduce_norm<bf16_t>, dim3(a.M), dim3(kNormThreads), s, false, last, a);
  else
    launch(k_rows_reduce_norm<float>, dim3(a.M), dim3(kNormThreads), s, false, last, a);
  return hipGetLastError();
}

}  // namespace lm
