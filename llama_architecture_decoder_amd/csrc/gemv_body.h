// The batch-1 matrix-vector product as a device function (one block's share of the row groups), used
// by the GEMV kernels and by the launch that runs the q/k/v product together with the attention.
//
// y = W x with W [N][K] row-major (row = output, main.bend type LW), F32 or bf16 weights, F32
// arithmetic.  One 256-thread block owns R consecutive rows at a time (a row group) and the whole block
// splits K: thread t reads 16-byte chunk j*256 + t of every row of the group, so each block instruction
// streams 4 KB of contiguous row bytes and a thread's slice of x is the same for every row (x lives in
// registers, at most 8 chunks = 64 floats).  Blocks walk row groups with a stride, so the per-block
// prologue (loading x and, for the norm variants, its sum of squares) is paid once per block rather
// than once per group.  Each thread issues R*KCH independent 16-byte loads (~16) before it uses any,
// which keeps ~64 KB in flight per block.
//
// Reduction: the R (or 2R) per-thread partial sums are reduced across the wavefront with a
// transposing butterfly (R-1 + 6-log2 R shuffles instead of 6R), then across the 4 waves through LDS
// in a fixed order, so results are deterministic.
#pragma once

#include "common.h"

namespace lm {


template <int KCH, int PAIRS>
struct RowsPerGroup {
  static constexpr int loads = 16;
  static constexpr int raw = loads / (KCH * PAIRS);
  static constexpr int value = raw >= 8 ? 8 : raw >= 4 ? 4 : raw >= 2 ? 2 : 1;
};

// Reduce n = 2^k values per lane across the 64 lanes.  After the call, value index r's wave sum is in
// v[0] of every lane whose lane id / (64 / n) == r.
template <int n>
__device__ __forceinline__ void wave_transpose_sum(float (&v)[n], int lane) {
  int count = n;
  int off = 32;
#pragma unroll
  for (int step = 0; step < 6; ++step) {
    if (count > 1) {
      const int halfc = count / 2;
      const bool up = (lane & off) != 0;
      // the lane-dependent choice as a bitwise select: as a conditional, the compiler may turn it into
      // an index into v and move v to scratch memory
      const uint32_t m = up ? 0xffffffffu : 0u;
#pragma unroll
      for (int i = 0; i < n / 2; ++i) {
        if (i < halfc) {
          const uint32_t x = __float_as_uint(v[i]), y = __float_as_uint(v[i + halfc]);
          const float send = __uint_as_float((x & m) | (y & ~m));
          const float keep = __uint_as_float((y & m) | (x & ~m));
          v[i] = keep + __shfl_xor(send, off);
        }
      }
      count = halfc;
    } else {
      v[0] += __shfl_xor(v[0], off);
    }
    off >>= 1;
  }
}
template <>
__device__ __forceinline__ void wave_transpose_sum<1>(float (&v)[1], int lane) {
  v[0] = wave_sum(v[0]);
}

// The input slice of this thread (chunks j*256 + tid, E numbers each) from tagged words a.xt written by
// another role of the same launch, polled until every word carries this launch's tag.  A wait past
// spin_limit polls (at once when status bit 3 is already set) gives up: the missing inputs are NaN and
// bit 3 is set.
template <int KCH, int E>
__device__ void poll_tagged_input(const GemvArgs &a, float (&xr)[KCH][E], int nchunk, uint32_t tag) {
  __shared__ int ok_s[kThreads / 64];
  __shared__ int stop_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  bool give_up = false;
  for (int it = 0;; ++it) {
    bool ok = true;
#pragma unroll
    for (int j = 0; j < KCH; ++j) {
      const int ci = min(j * kThreads + tid, nchunk - 1);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const unsigned long long w = tagged_load(a.xt + (size_t)ci * E + e);
        const bool hit = (uint32_t)(w >> 32) == tag;
        if (hit)
          xr[j][e] = __uint_as_float((uint32_t)w);
        else if (give_up)
          xr[j][e] = __builtin_nanf("");
        ok &= hit;
      }
    }
    const int wave_ok = __all(ok);
    if (lane == 0) ok_s[wave] = wave_ok;
    if (tid == 0)
      stop_s = it >= a.spin_limit ||
               (__hip_atomic_load(a.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & 8) != 0;
    lds_barrier();
    int all = 1;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) all &= ok_s[w];
    const bool stop = stop_s != 0;
    lds_barrier();  // ok_s and stop_s are read by every wave before they are written again
    if (all) return;
    if (give_up) {
      if (tid == 0) atomicOr(a.status, 8);
      return;
    }
    give_up = stop;
    __builtin_amdgcn_s_sleep(2);
  }
}

template <typename WT>
__device__ __forceinline__ const WT *row_ptr(const GemvArgs &a, int r) {
  int blk = (r >= a.rs[1]) + (r >= a.rs[2]);
  return reinterpret_cast<const WT *>(a.w[blk]) + (size_t)(r - a.rs[blk]) * (size_t)a.K;
}

// One block's share of a product: row groups bid, bid + nblk, ...  `tag` labels the tagged copies the
// q/k/v epilogue writes when a.ra.tagged is set (a launch that also runs the attention), and, with XT,
// the tagged input words this launch's other role writes (a.xt): the first group's weights are then
// requested before the wait for the input.
template <typename WT, int KCH, int EPI, bool NORM, bool XT = false>
__device__ __forceinline__ void gemv_body(const GemvArgs &a, int bid, int nblk, uint32_t tag) {
  constexpr int E = Vec16<WT>::E;
  constexpr int PAIRS = (EPI == EPI_SWIGLU) ? 2 : 1;
  constexpr int R = RowsPerGroup<KCH, PAIRS>::value;
  constexpr int NV = R * PAIRS;  // partial sums per thread per group
  static_assert(EPI != EPI_ROPE || NORM, "the RoPE epilogue's cos/sin reach LDS through the norm prologue's barrier");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nchunk = a.K / E;
  const bool ragged = (nchunk % kThreads) != 0;  // uniform: some threads' last chunk is past K

  __shared__ float red[4][NV];
  __shared__ float ss_w[4];
  // Every load below is unconditional (indices clamped, unwanted values zeroed afterwards): the wait
  // counter then sees one straight sequence (cos/sin, x, gains, weights), so the norm prologue waits for
  // x and the gains only, not for the weights behind them.
  __shared__ float rope_s[EPI == EPI_ROPE ? 2 * 64 : 1];  // cos | sin of the position (half <= 64)
  float rope_v = 0.f;
  if (EPI == EPI_ROPE) {
    // the table row of the position: cos for threads 0..half-1, sin for half..2*half-1 (pointers chosen
    // from uniform values, the element index clamped)
    const int hf = a.ra.half;
    const float *tab = tid < hf ? a.ra.rope_cs : a.ra.rope_sn;
    rope_v = tab[(size_t)a.ra.pos[0] * hf + min(tid < hf ? tid : tid - hf, hf - 1)];
  }

  // ---- the input slice of this thread: chunks j*256 + tid (a chunk past K reads the last chunk and is
  // zeroed)
  static_assert(!XT || !NORM, "a tagged input is not normalised");
  float xr[KCH][E];
#pragma unroll
  for (int j = 0; j < KCH && !XT; ++j) {
    const int ci = min(j * kThreads + tid, nchunk - 1);
#pragma unroll
    for (int e = 0; e < E; e += 4) {
      float4 v = *reinterpret_cast<const float4 *>(a.x + (size_t)ci * E + e);
      xr[j][e + 0] = v.x;
      xr[j][e + 1] = v.y;
      xr[j][e + 2] = v.z;
      xr[j][e + 3] = v.w;
    }
  }
  // the norm gains of the slice (also independent of everything else)
  u32x4 gr[NORM ? KCH : 1];
  if (NORM) {
    const WT *g = reinterpret_cast<const WT *>(a.gain);
#pragma unroll
    for (int j = 0; j < KCH; ++j) gr[j] = load16(g + (size_t)min(j * kThreads + tid, nchunk - 1) * E);
  }

  // the weights of a row group: unconditional loads (a row past N reads row N-1, whose result is never
  // stored; a chunk past the row end reads the row's last chunk and is zeroed)
  auto load_group = [&](int grp, u32x4 (&wv)[NV][KCH]) {
    const int row0 = grp * R;
#pragma unroll
    for (int p = 0; p < PAIRS; ++p) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int crow = min(row0 + r, a.N - 1);
        const WT *wp = (EPI == EPI_SWIGLU) ? reinterpret_cast<const WT *>(a.w[p]) + (size_t)crow * (size_t)a.K
                       : (EPI == EPI_ROPE) ? row_ptr<WT>(a, rope_row(crow, a.ra.dim + a.ra.kvw, a.ra.hshift))
                                           : row_ptr<WT>(a, crow);
#pragma unroll
        for (int j = 0; j < KCH; ++j) {
          const int ci = min(j * kThreads + tid, nchunk - 1);
          wv[p * R + r][j] = load_stream16(wp + (size_t)ci * E);
        }
      }
    }
  };
  // the first group's weights go out before the norm prologue (loads complete in order: the prologue
  // waits for x and the gains only, and the weights stream meanwhile)
  u32x4 wv[NV][KCH];
  int grp = bid;
  load_group(min(grp, a.ngroups - 1), wv);  // the launch has at most one block per group
  if (XT) poll_tagged_input<KCH, E>(a, xr, nchunk, tag);
#pragma unroll
  for (int j = 0; j < KCH; ++j)
    if (j * kThreads + tid >= nchunk)
#pragma unroll
      for (int e = 0; e < E; ++e) xr[j][e] = 0.f;
  if (EPI == EPI_ROPE && tid < 2 * a.ra.half) rope_s[tid] = rope_v;  // published by the norm's barrier

  if (NORM) {
    // RMSNorm prologue: g * (x * (1 / sqrt(sum(x^2) / K + eps)))
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < KCH; ++j)
#pragma unroll
      for (int e = 0; e < E; ++e) ss += xr[j][e] * xr[j][e];
    ss = wave_sum(ss);
    if (lane == 0) ss_w[wave] = ss;
    lds_barrier();
    const float tot = (ss_w[0] + ss_w[1]) + (ss_w[2] + ss_w[3]);
    const float r = 1.0f / sqrtf(tot / (float)a.K + a.eps);
#pragma unroll
    for (int j = 0; j < KCH; ++j) {
      float gv[E];
      Vec16<WT>::unpack(gr[j], gv);
#pragma unroll
      for (int e = 0; e < E; ++e) xr[j][e] = gv[e] * (xr[j][e] * r);  // chunks past K: x = 0
    }
  }

  float best_v = -INFINITY;
  int best_i = 0x7fffffff;

  for (; grp < a.ngroups; grp += nblk) {
    const int row0 = grp * R;
    if (grp != bid) load_group(grp, wv);
    if (ragged) {  // a chunk past the row end contributes exact zeros, whatever was stored there
#pragma unroll
      for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int j = 0; j < KCH; ++j)
          if (j * kThreads + tid >= nchunk) wv[v][j] = u32x4{0u, 0u, 0u, 0u};
    }
    float acc[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < KCH; ++j) {
        float wf[E];
        Vec16<WT>::unpack(wv[v][j], wf);
#pragma unroll
        for (int e = 0; e < E; ++e) s = fmaf(wf[e], xr[j][e], s);
      }
      acc[v] = s;
    }
    wave_transpose_sum<NV>(acc, lane);
    constexpr int span = 64 / NV;
    if ((lane % span) == 0) red[wave][lane / span] = acc[0];
    lds_barrier();
    if (tid < R) {
      const int row = row0 + tid;
      float val[PAIRS];
#pragma unroll
      for (int p = 0; p < PAIRS; ++p) {
        const int v = p * R + tid;
        val[p] = (red[0][v] + red[1][v]) + (red[2][v] + red[3][v]);
      }
      if (row < a.N) {
        if (EPI == EPI_STORE) {
          a.y[row] = val[0];
        } else if (EPI == EPI_RESID) {
          a.y[row] = a.res[row] + val[0];
        } else if (EPI == EPI_SWIGLU) {
          const float gt = val[0], up = val[PAIRS - 1];
          a.y[row] = (gt / (1.0f + expf(-gt))) * up;
        } else if (EPI == EPI_ROPE) {
          // the pair partner is logical row row ^ 1, in this group (R is even)
          const int v2 = tid ^ 1;
          const float pv = (red[0][v2] + red[1][v2]) + (red[2][v2] + red[3][v2]);
          const int ci = rope_pair_index(row, a.ra.hshift);
          rope_append(a.ra, a.y, 0, row, val[0], pv, rope_s[ci], rope_s[a.ra.half + ci], tag);
        } else {  // EPI_ARGMAX
          if (a.y) a.y[row] = val[0];
        }
      }
      if (EPI == EPI_ARGMAX) red[0][tid] = (row < a.N) ? val[0] : -INFINITY;
    }
    if (EPI == EPI_ROPE && a.ra.group_done) {
      // the group's outputs were issued by threads < R before this barrier; its word follows them
      lds_barrier();
      if (tid == 0) tagged_store(a.ra.group_done + grp, 0.f, tag);
    }
    if (EPI == EPI_ARGMAX) {
      lds_barrier();
      if (tid == 0) {
        // rows in increasing order, strict >: the first index of the largest value
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const float v = red[0][r];
          if (v > best_v) {
            best_v = v;
            best_i = row0 + r;
          }
        }
      }
    }
    lds_barrier();
  }

  if (EPI == EPI_ARGMAX && tid == 0) {
    a.part_v[bid] = best_v;
    a.part_i[bid] = best_i;
  }
}

}  // namespace lm
