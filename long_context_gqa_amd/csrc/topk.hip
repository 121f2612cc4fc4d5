// Top-k candidate selection over the vocabulary: each row's k highest
// logits, value descending, the lower index first among equal values.
//
// Stage 1 (topk_slice): one workgroup per (row, slice of 8,192 columns). Each
//   lane holds 32 of the slice's values in registers; each wave finds its
//   best k through a threshold (the k-th best lane maximum), compacts the few
//   values that can still be in the answer, and sorts them with a 64-lane
//   bitonic network; wave 0 sorts the 4k wave winners the same way. The
//   logits are read once.
// Stage 2 (topk_merge): one wave per row takes the best k of the slices'
//   candidates the same way and writes them in order.
#include <stdint.h>

#include "sv_common.h"
#include "sv_topk.h"

namespace sv {

namespace {

struct Cand {
  float v;
  int i;  // INT32_MAX: no candidate
};

__device__ __forceinline__ bool beats(Cand b, Cand a) {
  // b ranks before a: larger value, or equal value and lower index
  return b.v > a.v || (b.v == a.v && b.i < a.i);
}

__device__ __forceinline__ Cand wave_best(Cand x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    Cand y{__shfl_xor(x.v, o), __shfl_xor(x.i, o)};
    if (beats(y, x)) x = y;
  }
  return x;
}

constexpr int kPerLane = kTopkSlice / kThreads;  // 32 values per lane
constexpr Cand kNone = {-INFINITY, INT32_MAX};

// Sort one candidate per lane across the wave, best first (bitonic network
// over lane ids; indices are unique, so every pair has one better member).
__device__ __forceinline__ Cand bitonic64(Cand c, int lane) {
#pragma unroll
  for (int k = 2; k <= kWave; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const Cand o{__shfl_xor(c.v, j), __shfl_xor(c.i, j)};
      const bool best_first = (lane & k) == 0 || k == kWave;  // this run sorts best first
      const bool low = (lane & j) == 0;                         // lower lane of the pair
      const bool take = (low == best_first) ? beats(o, c) : beats(c, o);
      if (take) c = o;
    }
  }
  return c;
}

// The wave's best k (k <= 16) of the N values per lane (v, idx), in order,
// written to out[0..k-1]. The k-th best lane maximum t ranks no earlier than
// the wave's k-th best value, so only values ranking at or before t can be
// in the answer; they sit in at most k lanes (at most k*N of them) and are
// compacted into buf, then sorted (one per lane) or, when more than 64,
// taken by k rounds of a wave maximum.
template <int N>
__device__ __forceinline__ void wave_topk(const float (&v)[N], const int (&idx)[N], int k, Cand* out, Cand* buf,
                                          int lane) {
  Cand lb = kNone;
#pragma unroll
  for (int u = 0; u < N; ++u) {
    const Cand c{v[u], idx[u]};
    if (beats(c, lb)) lb = c;
  }
  const Cand srt = bitonic64(lb, lane);
  const Cand t{__shfl(srt.v, k - 1), __shfl(srt.i, k - 1)};
  int count = 0;
#pragma unroll
  for (int u = 0; u < N; ++u) {
    const Cand c{v[u], idx[u]};
    const bool pred = c.i != INT32_MAX && !beats(t, c);
    const uint64_t m = __ballot(pred);
    if (pred) buf[count + __popcll(m & ((1ull << lane) - 1ull))] = c;
    count += __popcll(m);
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (count <= kWave) {
    Cand c = lane < count ? buf[lane] : kNone;
    c = bitonic64(c, lane);
    if (lane < k) out[lane] = c;
  } else {
    // rare (many values tied or clustered in a few lanes): k rounds
    const int per = (count + kWave - 1) / kWave;  // <= N
    Cand h[N];
#pragma unroll
    for (int e = 0; e < N; ++e) h[e] = (e < per && lane + e * kWave < count) ? buf[lane + e * kWave] : kNone;
    auto best_of = [&]() {
      Cand b = kNone;
#pragma unroll
      for (int e = 0; e < N; ++e)
        if (beats(h[e], b)) b = h[e];
      return b;
    };
    Cand mine = best_of();
    for (int r = 0; r < k; ++r) {
      const Cand w = wave_best(mine);
      if (lane == 0) out[r] = w;
      if (w.i != INT32_MAX && mine.i == w.i) {
#pragma unroll
        for (int e = 0; e < N; ++e)
          if (h[e].i == w.i) h[e] = kNone;
        mine = best_of();
      }
    }
  }
}

}  // namespace

template <bool VEC4>
__global__ __launch_bounds__(kThreads) void topk_slice_kernel(const float* __restrict__ logits, int vocab, int k,
                                                              int n_slices, float2* ws) {
  const int sl = blockIdx.x, row = blockIdx.y, tid = threadIdx.x;
  const int lane = tid % kWave, wave = tid / kWave;
  const int lo = sl * kTopkSlice, hi = min(lo + kTopkSlice, vocab);
  const float* rp = logits + (size_t)row * vocab;
  // value u of this lane is column lo + 4*(tid + 256*(u/4)) + u%4
  float v[kPerLane];
  int idx[kPerLane];
#pragma unroll
  for (int u = 0; u < kPerLane; ++u) {
    const int col = lo + 4 * (tid + (u / 4) * kThreads) + u % 4;
    idx[u] = col < hi ? col : INT32_MAX;
  }
  if (VEC4) {
#pragma unroll
    for (int g = 0; g < kPerLane / 4; ++g) {
      const int col = lo + 4 * (tid + g * kThreads);
      const float4 x = col < hi ? *reinterpret_cast<const float4*>(rp + col)
                                : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      v[4 * g] = x.x;
      v[4 * g + 1] = x.y;
      v[4 * g + 2] = x.z;
      v[4 * g + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int u = 0; u < kPerLane; ++u) v[u] = idx[u] != INT32_MAX ? rp[idx[u]] : -INFINITY;
  }
  __shared__ Cand buf[kWavesPerGroup][kMaxTopk * kPerLane];
  __shared__ Cand wl[kWavesPerGroup * kMaxTopk];
  wave_topk<kPerLane>(v, idx, k, &wl[wave * k], buf[wave], lane);
  __syncthreads();
  if (wave == 0) {
    // the best k of the 4k wave winners (k <= 16: one per lane)
    Cand c = lane < kWavesPerGroup * k ? wl[lane] : kNone;
    c = bitonic64(c, lane);
    if (lane < k) ws[((size_t)row * n_slices + sl) * k + lane] = make_float2(c.v, __int_as_float(c.i));
  }
}

// One wave per row: the best k of the row's n_slices * k slice candidates.
__global__ __launch_bounds__(kThreads) void topk_merge_kernel(const float2* __restrict__ ws, int rows, int n_slices,
                                                              int k, int32_t* out_ids, float* out_vals) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int row = blockIdx.x * kWavesPerGroup + wave;
  __shared__ Cand buf[kWavesPerGroup][kMaxTopk * kMergePerLane];
  __shared__ Cand res[kWavesPerGroup][kMaxTopk];
  if (row >= rows) return;  // (no workgroup barrier below)
  const int n = n_slices * k;  // <= kWave * kMergePerLane
  float v[kMergePerLane];
  int idx[kMergePerLane];
#pragma unroll
  for (int e = 0; e < kMergePerLane; ++e) {
    const int j = lane + e * kWave;
    v[e] = -INFINITY;
    idx[e] = INT32_MAX;
    if (j < n) {
      const float2 p = ws[(size_t)row * n + j];
      v[e] = p.x;
      idx[e] = __float_as_int(p.y);
    }
  }
  wave_topk<kMergePerLane>(v, idx, k, res[wave], buf[wave], lane);
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (lane < k) {
    const Cand c = res[wave][lane];
    out_ids[(size_t)row * k + lane] = c.i == INT32_MAX ? -1 : c.i;
    out_vals[(size_t)row * k + lane] = c.v;
  }
}

void launch_topk(const TopkLaunch& a, hipStream_t s) {
  dim3 g1(a.n_slices, a.rows);
  if (a.vocab % 4 == 0)
    hipLaunchKernelGGL((topk_slice_kernel<true>), g1, dim3(kThreads), 0, s, a.logits, a.vocab, a.k, a.n_slices, a.ws);
  else
    hipLaunchKernelGGL((topk_slice_kernel<false>), g1, dim3(kThreads), 0, s, a.logits, a.vocab, a.k, a.n_slices,
                       a.ws);
  hipLaunchKernelGGL(topk_merge_kernel, dim3((a.rows + kWavesPerGroup - 1) / kWavesPerGroup), dim3(kThreads), 0, s,
                     a.ws, a.rows, a.n_slices, a.k, a.out_ids, a.out_vals);
}

}  // namespace sv
