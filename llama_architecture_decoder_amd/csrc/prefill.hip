// Prefill of S prompt positions at once (bf16 weights and cache) on gfx950 matrix cores.
//
// The prompt is the decode step applied to positions pos0 .. pos0+S-1 in order, where position i sees
// cache positions 0 .. pos0+i (main.bend forward_pre per prompt position; nest prefill.linnet states the
// same pass with the causal `seen` mask).  All S positions of a layer are done together:
//   * projections: Y[S][N] = X[S][K] W[N][K]^T as tiled MFMA products (X = bf16 hi + lo of the F32
//     activations, so the products carry about 16 significant bits of X and W is exact);
//   * RoPE + cache append for all S positions (the decode kernels' arithmetic, element for element);
//   * causal grouped-query attention over the cache, flash style: key tiles of 64 positions stream
//     through LDS once per (32-position query tile, kv head) and serve the g query heads of the group;
//     scores and probabilities stay in registers (softmax with a running maximum, base 2).
#include <type_traits>

#include "common.h"

namespace lm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// v_mfma_f32_32x32x16_bf16: A (32 x 16) lane l holds A[l%32][8(l/32) .. +8]; B (16 x 32) lane l holds
// B[8(l/32) .. +8][l%32]; C (32 x 32) lane l holds C[8(r/4) + 4(l/32) + r%4][l%32], r < 16.
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// ------------------------------------------------------------------------ tiled product ----
// Block: 128 token rows x 256 weight rows (SwiGLU: 128 gate rows + the same 128 up rows), K in steps of
// 32 through double-buffered LDS.  Wave (wm, wn) owns 64 x 128 of the block as 2 x 4 tiles of 32 x 32, so
// each k step reads 2 (x hi, lo) A fragments and 4 B fragments from LDS for 16 MFMAs: the LDS traffic per
// MFMA (reads + the staging writes) stays well under what the LDS delivers while the matrix cores run.
// Two blocks share a CU (80 KB of LDS each, at most 256 registers per lane), so one block's matrix work
// covers the other's wait for its next tiles: measured 7% faster over the 4096-position prefill than one
// block per CU with more registers.
constexpr int kTM = 128, kTN = 256, kTK = 32;
constexpr int kRowA = kTK + 8;  // LDS row of a tile: 40 bf16 = 80 bytes (16-byte reads of 16 rows hit distinct banks)

// A SwiGLU output v of token row t, unit n: F32 into y, or (a.ohi set) straight as the down product's
// bf16 operands, hi = bf16(v) to nearest even, lo = bf16(v - hi) (the bits k_split would give)
__device__ __forceinline__ void swiglu_store(const GemmArgs &a, int t, int n, float v) {
  if (a.ohi) {
    const __bf16 h = (__bf16)v;
    a.ohi[(size_t)t * a.ldo + n] = __builtin_bit_cast(uint16_t, h);
    a.olo[(size_t)t * a.ldo + n] = __builtin_bit_cast(uint16_t, (__bf16)(v - (float)h));
  } else {
    a.y[(size_t)t * a.ldy + n] = v;
  }
}

// LO: the A operand's lo half is multiplied too (hi + lo carry the F32 activations to ~2^-17); without
// it the product takes A as bf16 (hi, rounded to nearest even)
template <int EPI, bool LO>
__global__ __launch_bounds__(kThreads, 2) void k_gemm_tiled(GemmArgs a) {
  constexpr bool SW = EPI == EPI_SWIGLU;
  constexpr int AC = (LO ? 2 : 1) * kTM * (kTK / 8) / kThreads;  // 16-byte chunks of A (hi, lo) per thread
  constexpr int BC = kTN * (kTK / 8) / kThreads;      // of B
  __shared__ __attribute__((aligned(16))) bf16_t s_a[2][2][kTM * kRowA];  // [buffer][hi, lo]
  __shared__ __attribute__((aligned(16))) bf16_t s_b[2][kTN * kRowA];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * kTM;
  const int n0 = blockIdx.x * (SW ? kTN / 2 : kTN);

  // staging: 16-byte chunk c of a tile (rows of 32 columns) is row c / 4, columns 8 (c % 4) .. +8; A chunks
  // c < 512 are hi, the rest lo
  const bf16_t *ga[AC], *gb[BC];
  int ao[AC], bo[BC];
#pragma unroll
  for (int i = 0; i < AC; ++i) {
    const int c = tid + kThreads * i, h = c / (kTM * 4), cr = c % (kTM * 4), r = cr >> 2, cc = (cr & 3) * 8;
    ao[i] = h * kTM * kRowA + r * kRowA + cc;
    ga[i] = (h ? a.xlo : a.xhi) + (size_t)(m0 + r) * a.ldx + cc;
  }
#pragma unroll
  for (int i = 0; i < BC; ++i) {
    const int c = tid + kThreads * i, r = c >> 2, cc = (c & 3) * 8;
    bo[i] = r * kRowA + cc;
    const bf16_t *base;
    if (SW) {
      const int n = min(n0 + (r & 127), a.N - 1);
      base = reinterpret_cast<const bf16_t *>(r < 128 ? a.w[0] : a.w[1]) + (size_t)n * a.K;
    } else {
      const int n = min(n0 + r, a.N - 1);
      const int seg = n >= a.rs[2] ? 2 : (n >= a.rs[1] ? 1 : 0);
      base = reinterpret_cast<const bf16_t *>(a.w[seg]) + (size_t)(n - a.rs[seg]) * a.K;
    }
    gb[i] = base + cc;
  }

  u32x4 ra[AC], rb[BC];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int i = 0; i < AC; ++i) ra[i] = load16(ga[i] + k0);
#pragma unroll
    for (int i = 0; i < BC; ++i) rb[i] = load16(gb[i] + k0);
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < AC; ++i) *reinterpret_cast<u32x4 *>(&s_a[buf][0][ao[i]]) = ra[i];
#pragma unroll
    for (int i = 0; i < BC; ++i) *reinterpret_cast<u32x4 *>(&s_b[buf][bo[i]]) = rb[i];
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // K slice blockIdx.z of gridDim.z: steps kz0 .. kz0 + nst - 1
  const int nst = a.K / kTK / (int)gridDim.z;
  const int kz = (int)blockIdx.z * nst * kTK;
#pragma unroll
  for (int i = 0; i < AC; ++i) ga[i] += kz;
#pragma unroll
  for (int i = 0; i < BC; ++i) gb[i] += kz;
  fetch(0);
  stash(0);
  __syncthreads();
  const int l32 = lane & 31, hsel = (lane >> 5) * 8;
  for (int s = 0; s < nst; ++s) {
    const int buf = s & 1;
    if (s + 1 < nst) fetch((s + 1) * kTK);
#pragma unroll
    for (int kk = 0; kk < kTK / 16; ++kk) {
      const int ko = kk * 16 + hsel;
      u32x4 ah[2], al[2], b[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = wm * 64 + i * 32 + l32;
        ah[i] = *reinterpret_cast<const u32x4 *>(&s_a[buf][0][row * kRowA + ko]);
        if (LO) al[i] = *reinterpret_cast<const u32x4 *>(&s_a[buf][1][row * kRowA + ko]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // SwiGLU: tiles 0, 1 are gate rows, 2, 3 the up rows of the same outputs
        const int brow = SW ? ((j >> 1) * 128 + wn * 64 + (j & 1) * 32 + l32) : (wn * 128 + j * 32 + l32);
        b[j] = *reinterpret_cast<const u32x4 *>(&s_b[buf][brow * kRowA + ko]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] = mfma32(ah[i], b[j], acc[i][j]);
          if (LO) acc[i][j] = mfma32(al[i], b[j], acc[i][j]);
        }
    }
    if (s + 1 < nst) stash(buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds C[8(r/4) + 4(lane/32) + r%4][lane%32] of each tile
  if (gridDim.z > 1) {
    // a K slice: raw sums to part[z][t][n] (SwiGLU: gate at n, up at N + n); k_tiled_reduce finishes
    const int nout = SW ? 2 * a.N : a.N;
    float *pz = a.part + (size_t)blockIdx.z * a.M * nout;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (t >= a.M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = SW ? n0 + wn * 64 + (j & 1) * 32 + l32 : n0 + wn * 128 + j * 32 + l32;
          if (n < a.N) pz[(size_t)t * nout + (SW && j >= 2 ? a.N : 0) + n] = acc[i][j][r];
        }
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (t >= a.M) continue;
      if (SW) {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int n = n0 + wn * 64 + jj * 32 + l32;
          if (n < a.N) {
            const float gt = acc[i][jj][r], up = acc[i][2 + jj][r];
            swiglu_store(a, t, n, (gt / (1.0f + expf(-gt))) * up);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = n0 + wn * 128 + j * 32 + l32;
          if (n >= a.N) continue;
          float *y = a.y + (size_t)t * a.ldy + n;
          if (EPI == EPI_RESID)
            *y = a.res[(size_t)t * a.ldres + n] + acc[i][j][r];
          else
            *y = acc[i][j][r];
        }
      }
    }
}

// The K slices' partial sums of a tiled product, added in slice order, then its epilogue: thread =
// two consecutive outputs of token row blockIdx.y.
template <int EPI>
__global__ __launch_bounds__(kThreads) void k_tiled_reduce(GemmArgs a, int S) {
  constexpr bool SW = EPI == EPI_SWIGLU;
  const int t = blockIdx.y;
  const int n = 2 * (blockIdx.x * kThreads + threadIdx.x);
  if (n >= a.N) return;
  const int nout = SW ? 2 * a.N : a.N;
  const float *pp = a.part + (size_t)t * nout + n;
  const size_t zs = (size_t)a.M * nout;
  float v0 = 0.f, v1 = 0.f, u0 = 0.f, u1 = 0.f;
  for (int z = 0; z < S; ++z) {
    const float2 p = *reinterpret_cast<const float2 *>(pp + z * zs);
    v0 += p.x;
    v1 += p.y;
    if (SW) {
      const float2 q = *reinterpret_cast<const float2 *>(pp + z * zs + a.N);
      u0 += q.x;
      u1 += q.y;
    }
  }
  if (SW) {
    swiglu_store(a, t, n, (v0 / (1.0f + expf(-v0))) * u0);
    swiglu_store(a, t, n + 1, (v1 / (1.0f + expf(-v1))) * u1);
    return;
  }
  float *y = a.y + (size_t)t * a.ldy + n;
  {
    if (EPI == EPI_RESID) {
      v0 += a.res[(size_t)t * a.ldres + n];
      v1 += a.res[(size_t)t * a.ldres + n + 1];
    }
    y[0] = v0;
    y[1] = v1;
  }
}

// ------------------------------------------------------------------ large-tile product ----
// Long prompts (M of at least 1024 rows): 256x256 block tiles, 8 waves of 64x128 (2x4 MFMA 32x32x16
// tiles, the same per-wave work as k_gemm_tiled), one block per CU.  The operand tiles of a K step (A hi,
// A lo, B: 256 rows x 32 bf16 each, 48 KB) go from global memory straight into LDS (global_load_lds, 16
// bytes a lane, no registers), three stages deep, so a step's loads are issued two steps before it is
// multiplied.  A row of a tile is 64 bytes = 4 chunks of 16; chunk c of row r is stored at position
// c ^ ((r / 4) % 4): the loads write whole 1 KB runs, and the MFMA operand reads (32 rows, one chunk
// each, two chunks a lane pair) run at the conflict-free rate (measured: 6.6 cycles per wavefront read
// on this layout and on 80-byte padded rows, 17 on plain 64-byte rows, ~8.7 for swizzles that use row
// bit 1).  Tiles are ordered in groups of 4 M x 8 N tiles and each XCD takes an equal run of that
// order, so the operands a group shares stay in that XCD's L2 and no XCD has more tiles than another.
constexpr int kBM = 256, kBN = 256, kBK = 32;
constexpr int kBWaves = 8;  // waves of the large-tile kernel (4 or 8; measured the same)
constexpr int kBTile = kBM * kBK;       // bf16 per operand tile of a stage
constexpr int kBGroupM = 4, kBGroupN = 8, kXcds = 8;

__device__ __forceinline__ int bswz(int row) { return (row >> 2) & 3; }

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land at LDS byte address
// lds + 16 l (lds is the same for the whole wavefront, passed in M0).  Issued as inline assembly: the
// compiler then adds no wait of its own for these loads (it cannot tell which stage buffer a pending one
// writes at the loop head, and would wait for all); the kernel waits for them explicitly (wait_vm).  M0
// is used by nothing else in these kernels.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_load16(const bf16_t *g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void *)(p);
}

// s_waitcnt for at most N vector-memory operations in flight and no LDS operation in flight (gfx9
// encoding; expcnt left at its maximum)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}

// the workgroup barrier without a memory fence, after wait_vm: every wave's loads into the stage about to
// be read are complete and every wave's reads of earlier stages have returned (so a buffer refilled after
// the barrier is no longer being read); the compiler may not move memory accesses across it (it may move
// the products, which only touch registers)
__device__ __forceinline__ void bar_nofence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

struct BigPlan {
  int mt, nt, groups_m, groups_n, per_xcd, blocks, kslices;
};

static BigPlan big_plan(int M, int N, int K, bool swiglu) {
  BigPlan p;
  const int tn = swiglu ? kBN / 2 : kBN;
  p.mt = (M + kBM - 1) / kBM;
  p.nt = (N + tn - 1) / tn;
  p.groups_m = (p.mt + kBGroupM - 1) / kBGroupM;
  p.groups_n = (p.nt + kBGroupN - 1) / kBGroupN;
  const int order = p.groups_m * p.groups_n * kBGroupM * kBGroupN;  // tiles in grouped order
  p.per_xcd = (order + kXcds - 1) / kXcds;
  p.blocks = p.per_xcd * kXcds;
  const int tiles = p.mt * p.nt, steps = K / kBK;
  p.kslices = 1;
  // one block per CU: at least two rounds of 256 tiles, keep at least 32 steps of K per slice
  while (tiles * p.kslices < 512 && p.kslices < 8 && N % 2 == 0 && steps % (2 * p.kslices) == 0 &&
         steps / (2 * p.kslices) >= 32)
    p.kslices *= 2;
  return p;
}

// NW waves: 8 (4 x 2 waves of 64 x 128, two per SIMD) or 4 (2 x 2 waves of 128 x 128, one per SIMD with
// 256 accumulators, a quarter fewer operand reads per product)
// LO: as k_gemm_tiled (without it a stage holds [A hi | B] and each step does half the products)
template <int EPI, int NW, bool LO>
__global__ __launch_bounds__(NW * 64, 1) void k_gemm_big(GemmArgs a, BigPlan plan) {
  constexpr bool SW = EPI == EPI_SWIGLU;
  constexpr int WM = NW / 2, TMW = kBM / WM, MI = TMW / 32;  // waves along M, rows per wave, 32-row tiles
  constexpr int NOP = LO ? 3 : 2;                              // operand tiles per stage
  constexpr int SPW = 16 / NW, LPW = NOP * SPW;                // 1 KB segments per operand, loads per wave
  // three stages, each [A hi | A lo | B] (or [A hi | B])
  __shared__ __attribute__((aligned(1024))) bf16_t st0[NOP * kBTile];
  __shared__ __attribute__((aligned(1024))) bf16_t st1[NOP * kBTile];
  __shared__ __attribute__((aligned(1024))) bf16_t st2[NOP * kBTile];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // tile of this block: the tiles in grouped order (groups of 4 M x 8 N tiles, M fastest inside a group)
  // are cut into 8 equal runs; XCD x (= block % 8, the dispatch order) takes run x in order
  const int b = blockIdx.x, x = b % kXcds, l = b / kXcds;
  const int q = x * plan.per_xcd + l;
  const int gi = q / (kBGroupM * kBGroupN), w = q % (kBGroupM * kBGroupN);
  const int tm = (gi % plan.groups_m) * kBGroupM + w % kBGroupM;
  const int tnn = (gi / plan.groups_m) * kBGroupN + w / kBGroupM;
  if (gi >= plan.groups_m * plan.groups_n || tm >= plan.mt || tnn >= plan.nt) return;
  const int m0 = tm * kBM;
  const int n0 = tnn * (SW ? kBN / 2 : kBN);

  // this thread's LPW 16-byte loads of a stage: wave segment g = part * NW + wave (1 KB = 16 rows) of
  // operand o (0 A hi, 1 A lo, 2 B; without LO 0 A hi, 1 B); lane -> row 16 g + lane / 4, stored
  // position lane % 4
  const bf16_t *gp[LPW];
  uint32_t lo[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int o = i / SPW, g = (i % SPW) * NW + wave;
    const int row = g * 16 + (lane >> 2), c = (lane & 3) ^ bswz(row);
    lo[i] = (uint32_t)(o * kBTile + g * 512) * 2;  // byte offset of the wavefront's 1 KB within the stage
    if (o < NOP - 1) {
      const int t = min(m0 + row, a.M - 1);
      gp[i] = (o ? a.xlo : a.xhi) + (size_t)t * a.ldx + c * 8;
    } else if (SW) {
      const int n = min(n0 + (row & 127), a.N - 1);
      gp[i] = reinterpret_cast<const bf16_t *>(row < 128 ? a.w[0] : a.w[1]) + (size_t)n * a.K + c * 8;
    } else {
      const int n = min(n0 + row, a.N - 1);
      const int seg = n >= a.rs[2] ? 2 : (n >= a.rs[1] ? 1 : 0);
      gp[i] = reinterpret_cast<const bf16_t *>(a.w[seg]) + (size_t)(n - a.rs[seg]) * a.K + c * 8;
    }
  }
  // K slice blockIdx.y of gridDim.y
  const int nst = a.K / kBK / (int)gridDim.y;
  const int kz = (int)blockIdx.y * nst * kBK;
  const uint32_t sb0 = lds_addr(st0), sb1 = lds_addr(st1), sb2 = lds_addr(st2);
  auto issue = [&](uint32_t stage, int k) {
#pragma unroll
    for (int i = 0; i < LPW; ++i) lds_load16(gp[i] + kz + k, stage + lo[i]);
  };

  f32x16 acc[MI][4];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int l32 = lane & 31, hsel = lane >> 5;
  int arow[MI], brow[4];
#pragma unroll
  for (int i = 0; i < MI; ++i) arow[i] = wm * TMW + i * 32 + l32;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    brow[j] = SW ? ((j >> 1) * 128 + wn * 64 + (j & 1) * 32 + l32) : (wn * 128 + j * 32 + l32);
  // the step's operand reads (two halves of K) and its products
  auto compute = [&](const bf16_t *stage) {
    u32x4 ah[2][MI], al[2][MI], bf[2][4];
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int c = kk * 2 + hsel;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bf[kk][j] = *reinterpret_cast<const u32x4 *>(stage + (NOP - 1) * kBTile + brow[j] * kBK +
                                                     ((c ^ bswz(brow[j])) << 3));
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int off = arow[i] * kBK + ((c ^ bswz(arow[i])) << 3);
        ah[kk][i] = *reinterpret_cast<const u32x4 *>(stage + off);
        if (LO) al[kk][i] = *reinterpret_cast<const u32x4 *>(stage + kBTile + off);
      }
    }
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(ah[kk][i], bf[kk][j], acc[i][j]);
      if (LO) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(al[kk][i], bf[kk][j], acc[i][j]);
      }
    }
    // (the compiler's own interleaving of these reads and products: explicit groups -- the first half's
    // reads, half or a quarter of the products, the second half's reads, the rest; or all reads first --
    // measured 1.8-2.9% slower over an 8-layer 4096-position prefill)
  };
  // step t multiplies stage t % 3; its loads were issued two steps earlier.  At step t the wave waits
  // for its own loads of stage t (those of stage t + 1, issued later, may still be in flight), then the
  // barrier makes every wave's part visible and ends every read of stage t - 1, whose buffer the loads
  // of stage t + 2 then refill.
  issue(sb0, 0);
  if (nst > 1) issue(sb1, kBK);
  // steady state (every step refills): straight-line code, so the compiler's own wait for loads into
  // LDS sees which buffer each pending load writes and adds none
  int t = 0;
  for (; t + 4 < nst; t += 3) {
    wait_vm<LPW>();
    bar_nofence();
    issue(sb2, (t + 2) * kBK);
    compute(st0);
    wait_vm<LPW>();
    bar_nofence();
    issue(sb0, (t + 3) * kBK);
    compute(st1);
    wait_vm<LPW>();
    bar_nofence();
    issue(sb1, (t + 4) * kBK);
    compute(st2);
  }
  // the last two to four steps (stages t and t + 1 are in st0 and st1)
  auto step = [&](const bf16_t *cur, uint32_t refill, int u) {
    if (u + 1 < nst)
      wait_vm<LPW>();
    else
      wait_vm<0>();
    bar_nofence();
    if (u + 2 < nst) issue(refill, (u + 2) * kBK);
    compute(cur);
  };
  for (; t < nst; t += 3) {
    step(st0, sb2, t);
    if (t + 1 < nst) step(st1, sb0, t + 1);
    if (t + 2 < nst) step(st2, sb1, t + 2);
  }

  // epilogue: lane holds C[8(r/4) + 4(lane/32) + r%4][lane%32] of each 32x32 tile
  if (gridDim.y > 1) {
    const int nout = SW ? 2 * a.N : a.N;
    float *pz = a.part + (size_t)blockIdx.y * a.M * nout;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = m0 + wm * TMW + i * 32 + 8 * (r >> 2) + 4 * hsel + (r & 3);
        if (t >= a.M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = SW ? n0 + wn * 64 + (j & 1) * 32 + l32 : n0 + wn * 128 + j * 32 + l32;
          if (n < a.N) pz[(size_t)t * nout + (SW && j >= 2 ? a.N : 0) + n] = acc[i][j][r];
        }
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = m0 + wm * TMW + i * 32 + 8 * (r >> 2) + 4 * hsel + (r & 3);
      if (t >= a.M) continue;
      if (SW) {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int n = n0 + wn * 64 + jj * 32 + l32;
          if (n < a.N) {
            const float gt = acc[i][jj][r], up = acc[i][2 + jj][r];
            swiglu_store(a, t, n, (gt / (1.0f + expf(-gt))) * up);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = n0 + wn * 128 + j * 32 + l32;
          if (n >= a.N) continue;
          float *y = a.y + (size_t)t * a.ldy + n;
          if (EPI == EPI_RESID)
            *y = a.res[(size_t)t * a.ldres + n] + acc[i][j][r];
          else
            *y = acc[i][j][r];
        }
      }
    }
}

// the large-tile kernel for M of at least 1024 rows and enough tiles for the chip
static bool use_big(int M, int N, int K, bool swiglu) {
  if (M < 1024 || K % kBK != 0) return false;
  const BigPlan p = big_plan(M, N, K, swiglu);
  return p.mt * p.nt * p.kslices >= 512;
}

int gemm_tiled_rows(int M) { return (M + kTM - 1) / kTM * kTM; }

int gemm_tiled_kslices(int M, int N, int K, bool swiglu) {
  const int blocks = ((M + kTM - 1) / kTM) * ((N + (swiglu ? kTN / 2 : kTN) - 1) / (swiglu ? kTN / 2 : kTN));
  const int steps = K / kTK;
  int ks = 1;
  // two blocks per CU: aim for 512, keep at least 8 steps of K per slice
  while (blocks * ks < 512 && ks < 16 && N % 2 == 0 && steps % (2 * ks) == 0 && steps / (2 * ks) >= 8) ks *= 2;
  return ks;
}

size_t gemm_tiled_part_floats(int M, int N, int K, bool swiglu) {
  const int ks = use_big(M, N, K, swiglu) ? big_plan(M, N, K, swiglu).kslices : gemm_tiled_kslices(M, N, K, swiglu);
  return ks > 1 ? (size_t)ks * M * (swiglu ? 2 * (size_t)N : (size_t)N) : 0;
}

hipError_t launch_gemm_tiled(GemvEpi epi, const GemmArgs &a0, hipStream_t s, bool last, bool first, NormNext *nn,
                             int *defer_ks) {
  if (a0.K % kTK != 0 || a0.M <= 0) return hipErrorInvalidValue;
  GemmArgs a = a0;
  if (nn) nn->done = false;
  if (defer_ks) *defer_ks = 0;
  // the K slices' reduce: plain, or (residual in place) with the RMSNorm + operand split of the next product
  auto reduce = [&](auto epi_c, int ks) {
    constexpr int E = decltype(epi_c)::value;
    if (E == EPI_STORE && defer_ks) {
      *defer_ks = ks;
      return;
    }
    if (E == EPI_RESID && nn && a.y == a.res && a.ldy == a.ldres && a.N % 4 == 0) {
      RowsNormArgs r = {};
      r.part = a.part;
      r.S = ks;
      r.M = a.M;
      r.N = a.N;
      r.x = a.y;
      r.ldx = a.ldy;
      r.gain = nn->gain;
      r.eps = nn->eps;
      r.xhi = nn->xhi;
      r.xlo = nn->xlo;
      r.ldo = nn->ldo;
      nn->done = launch_rows_reduce_norm(nn->gdtype, r, s, last) == hipSuccess;
      return;
    }
    const dim3 rg((a.N / 2 + kThreads - 1) / kThreads, a.M);
    launch(k_tiled_reduce<E>, rg, dim3(kThreads), s, false, last, a, ks);
  };
  const int mt = (a.M + kTM - 1) / kTM;
  const bool sw = epi == EPI_SWIGLU;
  if (use_big(a.M, a.N, a.K, sw)) {
    BigPlan p = big_plan(a.M, a.N, a.K, sw);
    if (!a.part) p.kslices = 1;
    a.kslices = p.kslices;
    const int ks = a.kslices;
    const dim3 g(p.blocks, ks);
    auto big = [&](auto epi_c) {
      constexpr int E = decltype(epi_c)::value;
      if (a.lo)
        launch(k_gemm_big<E, kBWaves, true>, g, dim3(kBWaves * 64), s, first, last && ks == 1, a, p);
      else
        launch(k_gemm_big<E, kBWaves, false>, g, dim3(kBWaves * 64), s, first, last && ks == 1, a, p);
      if (ks > 1) reduce(epi_c, ks);
    };
    switch (epi) {
      case EPI_STORE: big(std::integral_constant<int, EPI_STORE>{}); break;
      case EPI_RESID: big(std::integral_constant<int, EPI_RESID>{}); break;
      case EPI_SWIGLU: big(std::integral_constant<int, EPI_SWIGLU>{}); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  a.kslices = a.part ? gemm_tiled_kslices(a.M, a.N, a.K, sw) : 1;
  const int ks = a.kslices;
  auto tiled = [&](auto epi_c) {
    constexpr int E = decltype(epi_c)::value;
    const dim3 g(E == EPI_SWIGLU ? (a.N + kTN / 2 - 1) / (kTN / 2) : (a.N + kTN - 1) / kTN, mt, ks);
    if (a.lo)
      launch(k_gemm_tiled<E, true>, g, dim3(kThreads), s, first, last && ks == 1, a);
    else
      launch(k_gemm_tiled<E, false>, g, dim3(kThreads), s, first, last && ks == 1, a);
    if (ks > 1) reduce(epi_c, ks);
  };
  switch (epi) {
    case EPI_STORE: tiled(std::integral_constant<int, EPI_STORE>{}); break;
    case EPI_RESID: tiled(std::integral_constant<int, EPI_RESID>{}); break;
    case EPI_SWIGLU: tiled(std::integral_constant<int, EPI_SWIGLU>{}); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------ RoPE + cache append ----
// Block i = packed row i, position p of its segment's request: the query heads are rotated in place in
// the qkv rows; the key heads are rotated and, with the value heads, stored at that position of the
// request's cache (bf16 with round-to-nearest-even).  Each pair (d, d + half) uses rot_lo / rot_hi
// (main.bend rope) with the position's cos/sin from the table.
__global__ __launch_bounds__(kThreads) void k_rope_rows(PrefillArgs a) {
  const int i = blockIdx.x;
  const int sg = segment_of(a.seg_start, a.nseg, i);
  const int p = a.seg_pos0[sg] + i - a.seg_start[sg];
  const int crow = a.table ? 0 : a.seg_row[sg];
  const int half = a.half, D = 2 * half;
  // the cache slot of position p: itself in row crow, or its place in the page pool (row 0); an entry
  // outside the pool writes no key or value
  const int slot = a.table ? page_slot(a.table + (size_t)a.seg_row[sg] * a.pages, p, a.npages, a.status) : p;
  float *row = a.qkv + (size_t)i * a.qkv_stride;
  // numbers n .. n+3 of this row: the product's outputs, or its K slices added in slice order (0 + p0 +
  // p1 ..., the order k_tiled_reduce adds them in)
  const size_t zs = (size_t)a.S * a.qkv_stride;
  auto val4 = [&](int n) {
    if (!a.part) return *reinterpret_cast<const float4 *>(row + n);
    const float *pp = a.part + (size_t)i * a.qkv_stride + n;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int z = 0; z < a.ks; ++z) {
      const float4 q = *reinterpret_cast<const float4 *>(pp + z * zs);
      v.x += q.x;
      v.y += q.y;
      v.z += q.z;
      v.w += q.w;
    }
    return v;
  };
  const float *cs = a.rope_cs + (size_t)p * half, *sn = a.rope_sn + (size_t)p * half;
  // four pairs (d .. d+3 with d+half .. d+half+3) per thread: half is a multiple of 4
  const int hq = half / 4, nq = a.heads * hq, nk = a.kv * hq;
  for (int k = threadIdx.x; k < nq + nk; k += kThreads) {
    const bool isq = k < nq;
    const int kk = isq ? k : k - nq;
    const int h = kk / hq, d = (kk - h * hq) * 4;
    const int base = isq ? h * D : a.heads * D + h * D;
    const float4 lo4 = val4(base + d), hi4 = val4(base + d + half);
    const float4 c4 = *reinterpret_cast<const float4 *>(cs + d), s4 = *reinterpret_cast<const float4 *>(sn + d);
    const float lo[4] = {lo4.x, lo4.y, lo4.z, lo4.w}, hi[4] = {hi4.x, hi4.y, hi4.z, hi4.w};
    const float c[4] = {c4.x, c4.y, c4.z, c4.w}, sv[4] = {s4.x, s4.y, s4.z, s4.w};
    float nlo[4], nhi[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      nlo[e] = rope_pair(lo[e], -hi[e], c[e], sv[e]);
      nhi[e] = rope_pair(hi[e], lo[e], c[e], sv[e]);
    }
    if (isq) {
      *reinterpret_cast<float4 *>(row + base + d) = make_float4(nlo[0], nlo[1], nlo[2], nlo[3]);
      *reinterpret_cast<float4 *>(row + base + d + half) = make_float4(nhi[0], nhi[1], nhi[2], nhi[3]);
    } else if (slot >= 0) {
      bf16_t *kd = a.kc + ((size_t)(crow * a.kv + h) * a.max_seq + slot) * D;
      *reinterpret_cast<uint2 *>(kd + d) =
          make_uint2(f32_to_bf16(nlo[0]) | ((uint32_t)f32_to_bf16(nlo[1]) << 16),
                     f32_to_bf16(nlo[2]) | ((uint32_t)f32_to_bf16(nlo[3]) << 16));
      *reinterpret_cast<uint2 *>(kd + d + half) =
          make_uint2(f32_to_bf16(nhi[0]) | ((uint32_t)f32_to_bf16(nhi[1]) << 16),
                     f32_to_bf16(nhi[2]) | ((uint32_t)f32_to_bf16(nhi[3]) << 16));
    }
  }
  if (slot < 0) return;
  const int v0 = a.heads * D + a.kv * D;
  for (int k = 4 * threadIdx.x; k < a.kv * D; k += 4 * kThreads) {
    const int h = k / D, d = k - h * D;
    const float4 v = val4(v0 + k);
    *reinterpret_cast<uint2 *>(a.vc + ((size_t)(crow * a.kv + h) * a.max_seq + slot) * D + d) =
        make_uint2(f32_to_bf16(v.x) | ((uint32_t)f32_to_bf16(v.y) << 16),
                   f32_to_bf16(v.z) | ((uint32_t)f32_to_bf16(v.w) << 16));
  }
}

// ------------------------------------------------------------------ causal attention ----
// Block (query tile of 32 consecutive positions of one segment, kv head j, head quarter z; the order is
// below): wave w takes
// query head j*g + 4z + w (idle when that is >= g; it still helps stage the tiles); the keys are the
// segment's request's positions 0 .. the query's own, from its cache row or its pages.  Per key tile of
// 64 positions:
//   S^T[key][q] = K Q^T (K from LDS as the A operand, the wave's rotated queries as bf16 hi + lo B
//   fragments held in registers), so each lane owns one query column: 32 of the tile's 64 scores, the
//   other 32 in lane ^ 32.  Softmax with a running maximum in base 2 (the queries carry scale * log2(e)).
//   O^T[d][q] += V^T P^T: P^T is the score accumulator itself, split into bf16 hi + lo; the 16 keys a
//   B fragment covers are taken in the order the accumulator holds them (a sum does not care), and
//   V^T fragments are read from an LDS copy of V stored transposed, in the same key order.
constexpr int kQT = kPrefillQT;  // query positions per block
constexpr int kKT = 64;   // key positions per tile

template <int D>
struct FlashShape {
  static constexpr int KROW = D + 8;        // LDS row of K (bf16): 16-byte reads of 16 rows hit distinct banks
  static constexpr int VROW = kKT + 4;      // LDS row of V^T (bf16): one d, 64 keys
  static constexpr int KS = D / 16;         // k16 steps of a score product
  static constexpr int DT = D / 32;         // 32-row tiles of O^T
};

// Two blocks per CU (at most 256 registers per lane, 68 KB of LDS each at head 128): 6% faster over the
// 4096-position prefill than one block with more registers.
template <int D>
__global__ __launch_bounds__(kThreads, 2) void k_attn_prefill(PrefillArgs a) {
  using F = FlashShape<D>;
  __shared__ __attribute__((aligned(16))) bf16_t s_k[2][kKT * F::KROW];   // double buffered
  __shared__ __attribute__((aligned(16))) bf16_t s_vt[2][D * F::VROW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // block b: kv head b % kv, then head quarter and query tile from b / kv.  Query tiles are the
  // segments' own tiles of kQT positions in order (the last of each ragged), taken from the end so that
  // the longest start first.  Consecutive blocks go to consecutive XCDs, so with 8 kv heads each XCD runs
  // one head's tiles and its L2 keeps that head's keys and values.
  const int zq = (a.g + 3) / 4, nq_tiles = a.seg_tile[a.nseg];
  const int j = (int)blockIdx.x % a.kv, rest = (int)blockIdx.x / a.kv;
  const int zz = rest % zq;
  const int tile_id = nq_tiles - 1 - rest / zq;
  const int sg = segment_of(a.seg_tile, a.nseg, tile_id);
  const int qt = tile_id - a.seg_tile[sg];
  const int r0 = a.seg_start[sg], len = a.seg_start[sg + 1] - r0, pos0 = a.seg_pos0[sg];
  const int crow = a.table ? 0 : a.seg_row[sg];
  const int32_t *tr = a.table ? a.table + (size_t)a.seg_row[sg] * a.pages : nullptr;
  const int hi_in_group = zz * 4 + wave;
  const bool active = hi_in_group < a.g;
  const int head = j * a.g + (active ? hi_in_group : 0);
  const int l32 = lane & 31, hsel = lane >> 5;
  const int q_i = qt * kQT + l32;                     // index of this lane's query in its segment
  const int q_row = r0 + min(q_i, len - 1);           // its packed row (tail lanes repeat the last)
  const int q_pos = pos0 + min(q_i, len - 1);         // its cache position
  const int last_pos = pos0 + min(qt * kQT + kQT - 1, len - 1);
  const int first_pos = pos0 + qt * kQT;              // every lane's query is at or after it
  const bf16_t *Kh = a.kc + (size_t)(crow * a.kv + j) * a.max_seq * D;
  const bf16_t *Vh = a.vc + (size_t)(crow * a.kv + j) * a.max_seq * D;

  const float sc = a.scale * 1.4426950408889634f;
  // the wave's rotated queries as B fragments: lane holds q[q_i][16 ks + 8 hsel .. +8], hi and lo
  u32x4 qh[F::KS], ql[F::KS];
  {
    const float *q = a.qkv + (size_t)q_row * a.qkv_stride + head * D;
#pragma unroll
    for (int ks = 0; ks < F::KS; ++ks) {
      const float4 v0 = *reinterpret_cast<const float4 *>(q + ks * 16 + hsel * 8);
      const float4 v1 = *reinterpret_cast<const float4 *>(q + ks * 16 + hsel * 8 + 4);
      // the query times scale * log2(e), so the products are the base-2 softmax's exponents
      const float f[8] = {v0.x * sc, v0.y * sc, v0.z * sc, v0.w * sc, v1.x * sc, v1.y * sc, v1.z * sc, v1.w * sc};
      uint32_t h4[4], l4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) split_bf16x2(f[2 * e], f[2 * e + 1], h4[e], l4[e]);
      qh[ks] = u32x4{h4[0], h4[1], h4[2], h4[3]};
      ql[ks] = u32x4{l4[0], l4[1], l4[2], l4[3]};
    }
  }

  f32x16 o[F::DT];
#pragma unroll
  for (int t = 0; t < F::DT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[t][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int ntiles = last_pos / kKT + 1;
  // K (row-major) and V (transposed) of positions k0 .. k0+63 (past last_pos: clamped, masked): the next
  // tile's loads are in flight in registers while the current tile is multiplied, then written to the
  // other LDS buffer; one barrier per tile
  constexpr int KCH = kKT * D / 8;            // 16-byte chunks of the K tile
  constexpr int KPT = (KCH + kThreads - 1) / kThreads;
  constexpr int VCH = (kKT / 4) * (D / 8);    // (4 keys x 8 numbers) pieces of the V tile
  u32x4 kreg[KPT], vreg[4];
  // the V piece of this thread: 8 lanes read 128 contiguous bytes of a key row, and a wavefront covers 8
  // d-chunks x 8 key quads, so the stash's transposed 8-byte writes of one instruction fall in 16
  // distinct bank pairs (conflict-free)
  const int v_dc = lane % 8 + 8 * (wave % (D / 64)), v_kq = lane / 8 + 8 * (wave / (D / 64));
  static_assert(VCH == kKT / 4 * D / 8 && D % 64 == 0, "8 x 8 pieces per wavefront");
  // paged cache: a tile's positions k0 .. k0+63 (k0 a multiple of the page size, clamped to last_pos)
  // lie in one page
  static_assert(kKT == kPageSize, "a key tile is one page");
  auto fetch = [&](int k0) {
    int base = k0;  // cache slot of position k0
    if (tr) {
      const int sl = page_slot(tr, k0, a.npages, a.status);
      base = sl < 0 ? 0 : sl;
    }
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + i * kThreads;
      if (KCH % kThreads == 0 || c < KCH) {
        const int r = c / (D / 8), cc = (c % (D / 8)) * 8;
        kreg[i] = load16(Kh + (size_t)(base + min(k0 + r, last_pos) - k0) * D + cc);
      }
    }
    if (tid < VCH) {
      const int dc = v_dc, kq = v_kq;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        vreg[u] = load16(Vh + (size_t)(base + min(k0 + 4 * kq + u, last_pos) - k0) * D + dc * 8);
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + i * kThreads;
      if (KCH % kThreads == 0 || c < KCH) {
        const int r = c / (D / 8), cc = (c % (D / 8)) * 8;
        *reinterpret_cast<u32x4 *>(&s_k[buf][r * F::KROW + cc]) = kreg[i];
      }
    }
    // V: this thread's 4 consecutive keys x 8 consecutive numbers go to 8 rows of 4 keys of V^T
    if (tid < VCH) {
      const int dc = v_dc, kq = v_kq;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // number e of keys 0 and 1 (2 and 3) as one word: bytes 0-1 or 2-3 of each (v_perm_b32)
        const int w = e >> 1;
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t p01 = __builtin_amdgcn_perm(vreg[1][w], vreg[0][w], sel);
        const uint32_t p23 = __builtin_amdgcn_perm(vreg[3][w], vreg[2][w], sel);
        *reinterpret_cast<u32x2 *>(&s_vt[buf][(dc * 8 + e) * F::VROW + 4 * kq]) = u32x2{p01, p23};
      }
    }
  };
  fetch(0);
  stash(0);
  __syncthreads();
  for (int tile = 0; tile < ntiles; ++tile) {
    const int k0 = tile * kKT, buf = tile & 1;
    if (tile + 1 < ntiles) fetch(k0 + kKT);

    if (active) {
      // scores S^T for keys k0 + 32 mt + (8(r/4) + 4 hsel + r%4), query q_i
      f32x16 s[2];
      // the matrix-core phases at a raised wave priority, so the other block's wavefront on this SIMD
      // fills the softmax phases (8-layer 4096-position prefill 27.42 -> 27.21 ms)
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[mt][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < F::KS; ++ks) {
        u32x4 kf[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
          kf[mt] = *reinterpret_cast<const u32x4 *>(&s_k[buf][(mt * 32 + l32) * F::KROW + ks * 16 + hsel * 8]);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) s[mt] = mfma32(kf[mt], qh[ks], s[mt]);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) s[mt] = mfma32(kf[mt], ql[ks], s[mt]);
      }
      __builtin_amdgcn_s_setprio(0);
      float mt_max = -INFINITY;
      // the causal mask only where the tile reaches past the block's first query
      if (k0 + kKT - 1 <= first_pos) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            mt_max = fmaxf(mt_max, s[mt][r]);
          }
      } else {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + mt * 32 + 8 * (r >> 2) + 4 * hsel + (r & 3);
            const float v = key <= q_pos ? s[mt][r] : -INFINITY;
            s[mt][r] = v;
            mt_max = fmaxf(mt_max, v);
          }
      }
      mt_max = fmaxf(mt_max, __shfl_xor(mt_max, 32));
      const float m_new = fmaxf(m_run, mt_max);  // finite: key 0 is visible to every query
      // 2^x as the hardware's exponential (results below 2^-126 flush to zero: against a sum >= 1)
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      float lsum = 0.f;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pr = __builtin_amdgcn_exp2f(s[mt][r] - m_new);
          s[mt][r] = pr;
          lsum += pr;
        }
      lsum += __shfl_xor(lsum, 32);
      l_run = l_run * alpha + lsum;
      // the accumulators change only where the maximum grew (elsewhere alpha is exactly 1)
      if (!__all(m_new == m_run)) {
#pragma unroll
        for (int t = 0; t < F::DT; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[t][r] *= alpha;
      }
      m_run = m_new;
      // O^T += V^T P^T over the tile's 4 groups of 16 keys
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int mt = kk >> 1, r0 = (kk & 1) * 8;
        uint32_t ph[4], pl[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) split_bf16x2(s[mt][r0 + 2 * e], s[mt][r0 + 2 * e + 1], ph[e], pl[e]);
        const u32x4 pfh = u32x4{ph[0], ph[1], ph[2], ph[3]}, pfl = u32x4{pl[0], pl[1], pl[2], pl[3]};
        // keys of slot e of half hsel within the 16-group: 8(e/4) + 4 hsel + e%4
        const int kb = kk * 16 + 4 * hsel;
        u32x4 vf[F::DT];
#pragma unroll
        for (int t = 0; t < F::DT; ++t) {
          const bf16_t *vr = &s_vt[buf][(t * 32 + l32) * F::VROW + kb];
          const u32x2 lo4 = *reinterpret_cast<const u32x2 *>(vr);
          const u32x2 hi4 = *reinterpret_cast<const u32x2 *>(vr + 8);
          vf[t] = u32x4{lo4[0], lo4[1], hi4[0], hi4[1]};
        }
#pragma unroll
        for (int t = 0; t < F::DT; ++t) o[t] = mfma32(vf[t], pfh, o[t]);
#pragma unroll
        for (int t = 0; t < F::DT; ++t) o[t] = mfma32(vf[t], pfl, o[t]);
      }
    }
    // the other buffer was last read in the previous tile, before the previous barrier
    __builtin_amdgcn_s_setprio(0);
    if (tile + 1 < ntiles) stash(buf ^ 1);
    __syncthreads();
  }

  if (active && q_i < len) {
    const float inv = 1.0f / l_run;
    float *out = a.out + (size_t)q_row * a.out_stride + head * D;
#pragma unroll
    for (int t = 0; t < F::DT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) out[t * 32 + 8 * (r >> 2) + 4 * hsel + (r & 3)] = o[t][r] * inv;
  }
}

hipError_t launch_rope_rows(const PrefillArgs &a, hipStream_t s, bool first, bool last) {
  if (a.nseg < 1 || a.nseg > kMaxSegments || a.seg_start[a.nseg] != a.S) return hipErrorInvalidValue;
  launch(k_rope_rows, dim3(a.S), dim3(kThreads), s, first, last, a);
  return hipGetLastError();
}

hipError_t launch_attn_prefill(const PrefillArgs &a, hipStream_t s, bool first, bool last) {
  if (a.nseg < 1 || a.nseg > kMaxSegments || a.seg_start[a.nseg] != a.S) return hipErrorInvalidValue;
  const dim3 g(a.seg_tile[a.nseg] * a.kv * ((a.g + 3) / 4));
  if (a.half == 64)
    launch(k_attn_prefill<128>, g, dim3(kThreads), s, first, last, a);
  else if (a.half == 32)
    launch(k_attn_prefill<64>, g, dim3(kThreads), s, first, last, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace lm
