// Top-k candidate selection over the vocabulary: each row's k highest
// logits, value descending, the lower index first among equal values.
//
// Stage 1 (topk_slice): one workgroup per (row, slice of 8,192 columns, or
//   16,384 when there are few rows to spread). Each lane holds 32 (64) of the
//   slice's values in registers. A threshold from the k-th largest of the 64
//   four-lane group maxima leaves the few values that can still be in the
//   answer; they are compacted and sorted once with a 64-lane bitonic
//   network (or, when more than 64, each wave finds its best k and wave 0
//   merges the 4k winners). The logits are read once.
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

constexpr Cand kNone = {-INFINITY, INT32_MAX};

// The value of lane (lane ^ J) without the LDS crossbar: DPP quad
// permutations (xor 1, 2), row shifts (xor 4: lane +4 where bit 2 is clear,
// -4 where set), a row rotation (xor 8), and the gfx950 row/half swaps
// (xor 16, 32: the swapped copy of the other row or half).
template <int J>
__device__ __forceinline__ int xor_lane(int x, int lane) {
  if constexpr (J == 1) {
    return __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
  } else if constexpr (J == 2) {
    return __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
  } else if constexpr (J == 4) {
    const int up = __builtin_amdgcn_update_dpp(x, x, 0x104, 0xF, 0xF, false);  // row_shl:4 (lane + 4)
    const int dn = __builtin_amdgcn_update_dpp(x, x, 0x114, 0xF, 0xF, false);  // row_shr:4 (lane - 4)
    return (lane & 4) ? dn : up;
  } else if constexpr (J == 8) {
    return __builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, false);  // row_ror:8
  } else if constexpr (J == 16) {
    const auto p = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return (lane & 16) ? (int)p[0] : (int)p[1];
  } else {
    static_assert(J == 32, "xor distance");
    const auto p = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return (lane & 32) ? (int)p[0] : (int)p[1];
  }
}

template <int J>
__device__ __forceinline__ Cand xor_cand(Cand c, int lane) {
  return Cand{__int_as_float(xor_lane<J>(__float_as_int(c.v), lane)), xor_lane<J>(c.i, lane)};
}

// One compare-exchange stage of the bitonic network: run length K, distance J.
template <int K, int J>
__device__ __forceinline__ Cand bitonic_stage(Cand c, int lane) {
  const Cand o = xor_cand<J>(c, lane);
  const bool best_first = (lane & K) == 0 || K == kWave;  // this run sorts best first
  const bool low = (lane & J) == 0;                         // lower lane of the pair
  const bool take = (low == best_first) ? beats(o, c) : beats(c, o);
  return take ? o : c;
}

template <int K, int J>
__device__ __forceinline__ Cand bitonic_merge(Cand c, int lane) {
  c = bitonic_stage<K, J>(c, lane);
  if constexpr (J > 1) c = bitonic_merge<K, J / 2>(c, lane);
  return c;
}

// Sort one candidate per lane across the wave, best first (bitonic network
// over lane ids; indices are unique, so every pair has one better member).
__device__ __forceinline__ Cand bitonic64(Cand c, int lane) {
  c = bitonic_merge<2, 1>(c, lane);
  c = bitonic_merge<4, 2>(c, lane);
  c = bitonic_merge<8, 4>(c, lane);
  c = bitonic_merge<16, 8>(c, lane);
  c = bitonic_merge<32, 16>(c, lane);
  c = bitonic_merge<64, 32>(c, lane);
  return c;
}

// Values only, largest first (the same network).
template <int K, int J>
__device__ __forceinline__ float vstage(float x, int lane) {
  const float o = __int_as_float(xor_lane<J>(__float_as_int(x), lane));
  const bool best_first = (lane & K) == 0 || K == kWave;
  const bool low = (lane & J) == 0;
  return (low == best_first) ? fmaxf(x, o) : fminf(x, o);
}
template <int K, int J>
__device__ __forceinline__ float vmerge(float x, int lane) {
  x = vstage<K, J>(x, lane);
  if constexpr (J > 1) x = vmerge<K, J / 2>(x, lane);
  return x;
}
__device__ __forceinline__ float vsort64(float x, int lane) {
  x = vmerge<2, 1>(x, lane);
  x = vmerge<4, 2>(x, lane);
  x = vmerge<8, 4>(x, lane);
  x = vmerge<16, 8>(x, lane);
  x = vmerge<32, 16>(x, lane);
  x = vmerge<64, 32>(x, lane);
  return x;
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
  const Cand t{__int_as_float(__builtin_amdgcn_readlane(__float_as_int(srt.v), k - 1)),
               __builtin_amdgcn_readlane(srt.i, k - 1)};
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

// Column of this lane's value u in a slice starting at lo (increasing in u).
__device__ __forceinline__ int slice_col(int lo, int tid, int u) { return lo + 4 * (tid + (u / 4) * kThreads) + u % 4; }

// The slice stage of one wave: its best k of the lane values v (column
// slice_col(lo, tid, u), valid below hi), written to out[0..k-1]. As
// wave_topk, specialised: a lane's columns increase with u, so its maximum
// needs value compares only (the first of equal values has the lowest
// column), and the values that can still be in the answer are found by a
// cheap test against the threshold's value first (v >= t.v), the exact rank
// test only when some lane passes it.
template <int NPL>
__device__ __forceinline__ void slice_wave_topk(const float (&v)[NPL], int lo, int hi, int tid, int k, Cand* out,
                                                Cand* buf, int lane) {
  Cand lb = kNone;
  if (slice_col(lo, tid, 0) < hi) {
    lb = Cand{v[0], slice_col(lo, tid, 0)};
#pragma unroll
    for (int u = 1; u < NPL; ++u)
      if (v[u] > lb.v) lb = Cand{v[u], slice_col(lo, tid, u)};  // (past hi, v is -inf and never wins)
  }
  const Cand srt = bitonic64(lb, lane);
  const Cand t{__int_as_float(__builtin_amdgcn_readlane(__float_as_int(srt.v), k - 1)),
               __builtin_amdgcn_readlane(srt.i, k - 1)};
  int count = 0;
#pragma unroll
  for (int u = 0; u < NPL; ++u) {
    if (__ballot(v[u] >= t.v)) {  // (uniform) some lane may hold a candidate here
      const Cand c{v[u], slice_col(lo, tid, u)};
      const bool pred = c.i < hi && !beats(t, c);
      const uint64_t m = __ballot(pred);
      if (pred) buf[count + __popcll(m & ((1ull << lane) - 1ull))] = c;
      count += __popcll(m);
    }
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (count <= kWave) {
    Cand c = lane < count ? buf[lane] : kNone;
    c = bitonic64(c, lane);
    if (lane < k) out[lane] = c;
  } else {
    // rare (many values tied or clustered in a few lanes): k rounds of a
    // wave maximum over the compacted values
    Cand mine = kNone;
    for (int e = lane; e < count; e += kWave)
      if (beats(buf[e], mine)) mine = buf[e];
    for (int r = 0; r < k; ++r) {
      const Cand w = wave_best(mine);
      if (lane == 0) out[r] = w;
      if (w.i != INT32_MAX && mine.i == w.i) {
        mine = kNone;
        for (int e = lane; e < count; e += kWave)
          if (buf[e].i != w.i && beats(buf[e], mine) && beats(w, buf[e])) mine = buf[e];
      }
    }
  }
}

// NPL values per lane: slices of NPL * 256 columns.
//
// The slice's answer is found with one threshold for the whole workgroup:
// every group of 4 lanes gives its largest value, and the k-th largest t of
// these 64 group maxima has at least k values at or above it, so the k-th
// best value of the slice is >= t and every value of the answer is >= t.
// The values >= t (about 18 for random data) are compacted into LDS and, when
// they fit one per lane, sorted once by wave 0. Otherwise (many values tied
// or clustered) each wave finds its best k with the per-wave threshold of
// slice_wave_topk and wave 0 merges the 4k winners.
template <bool VEC4, int NPL, bool NT>
__global__ __launch_bounds__(kThreads) void topk_slice_kernel(const float* __restrict__ logits, int vocab, int k,
                                                              int n_slices, float2* ws) {
  const int sl = blockIdx.x, row = blockIdx.y, tid = threadIdx.x;
  const int lane = tid % kWave, wave = tid / kWave;
  const int lo = sl * NPL * kThreads, hi = min(lo + NPL * kThreads, vocab);
  const float* rp = logits + (size_t)row * vocab;
  float v[NPL];
  if (VEC4) {
#pragma unroll
    for (int g = 0; g < NPL / 4; ++g) {
      const int col = slice_col(lo, tid, 4 * g);
      const float4 x = col < hi ? load4<NT>(rp + col)
                                : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      v[4 * g] = x.x;
      v[4 * g + 1] = x.y;
      v[4 * g + 2] = x.z;
      v[4 * g + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int u = 0; u < NPL; ++u) {
      const int col = slice_col(lo, tid, u);
      v[u] = col < hi ? rp[col] : -INFINITY;
    }
  }
  constexpr int kCap = kMaxTopk * NPL;  // per-wave compaction capacity
  __shared__ Cand buf[kWavesPerGroup][kCap];
  __shared__ Cand wl[kWavesPerGroup * kMaxTopk];
  __shared__ float s_g[kWave];
  __shared__ int s_cnt[kWavesPerGroup];
  // the group maxima (values past hi are -inf)
  float m = v[0];
#pragma unroll
  for (int u = 1; u < NPL; ++u) m = fmaxf(m, v[u]);
  m = fmaxf(m, __int_as_float(xor_lane<1>(__float_as_int(m), lane)));
  m = fmaxf(m, __int_as_float(xor_lane<2>(__float_as_int(m), lane)));
  if ((lane & 3) == 0) s_g[wave * (kWave / 4) + lane / 4] = m;
  __syncthreads();
  const float gs = vsort64(s_g[lane], lane);
  const float t = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gs), k - 1));
  // compact this wave's values >= t (the count is kept even past capacity)
  int count = 0;
#pragma unroll
  for (int u = 0; u < NPL; ++u) {
    if (__ballot(v[u] >= t)) {  // (uniform) some lane holds one here
      const int col = slice_col(lo, tid, u);
      const bool pred = v[u] >= t && col < hi;
      const uint64_t mk = __ballot(pred);
      const int pos = count + __popcll(mk & ((1ull << lane) - 1ull));
      if (pred && pos < kCap) buf[wave][pos] = Cand{v[u], col};
      count += __popcll(mk);
    }
  }
  if (lane == 0) s_cnt[wave] = count;
  __syncthreads();
  const int c0 = s_cnt[0], c1 = s_cnt[1], c2 = s_cnt[2], c3 = s_cnt[3];
  const int total = c0 + c1 + c2 + c3;  // (uniform over the workgroup)
  if (total <= kWave) {
    if (wave == 0) {
      Cand c = kNone;
      if (lane < total) {
        const int w = lane >= c0 + c1 + c2 ? 3 : lane >= c0 + c1 ? 2 : lane >= c0 ? 1 : 0;
        const int base = w == 0 ? 0 : w == 1 ? c0 : w == 2 ? c0 + c1 : c0 + c1 + c2;
        c = buf[w][lane - base];
      }
      c = bitonic64(c, lane);
      if (lane < k) ws[((size_t)row * n_slices + sl) * k + lane] = make_float2(c.v, __int_as_float(c.i));
    }
    return;
  }
  slice_wave_topk<NPL>(v, lo, hi, tid, k, &wl[wave * k], buf[wave], lane);
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
  const bool vec4 = a.vocab % 4 == 0, wide = a.slice == kTopkSliceWide;
  const bool once = (long long)a.rows * a.vocab * (long long)sizeof(float) >= kStreamOnceBytes;
  if (vec4 && wide && once)
    hipLaunchKernelGGL((topk_slice_kernel<true, kTopkSliceWide / kThreads, true>), g1, dim3(kThreads), 0, s,
                       a.logits, a.vocab, a.k, a.n_slices, a.ws);
  else if (vec4 && wide)
    hipLaunchKernelGGL((topk_slice_kernel<true, kTopkSliceWide / kThreads, false>), g1, dim3(kThreads), 0, s,
                       a.logits, a.vocab, a.k, a.n_slices, a.ws);
  else if (vec4 && once)
    hipLaunchKernelGGL((topk_slice_kernel<true, kTopkSlice / kThreads, true>), g1, dim3(kThreads), 0, s, a.logits,
                       a.vocab, a.k, a.n_slices, a.ws);
  else if (vec4)
    hipLaunchKernelGGL((topk_slice_kernel<true, kTopkSlice / kThreads, false>), g1, dim3(kThreads), 0, s, a.logits, a.vocab,
                       a.k, a.n_slices, a.ws);
  else if (wide)
    hipLaunchKernelGGL((topk_slice_kernel<false, kTopkSliceWide / kThreads, false>), g1, dim3(kThreads), 0, s, a.logits,
                       a.vocab, a.k, a.n_slices, a.ws);
  else
    hipLaunchKernelGGL((topk_slice_kernel<false, kTopkSlice / kThreads, false>), g1, dim3(kThreads), 0, s, a.logits,
                       a.vocab, a.k, a.n_slices, a.ws);
  hipLaunchKernelGGL(topk_merge_kernel, dim3((a.rows + kWavesPerGroup - 1) / kWavesPerGroup), dim3(kThreads), 0, s,
                     a.ws, a.rows, a.n_slices, a.k, a.out_ids, a.out_vals);
}

}  // namespace sv
