// Merge of split-KV attention partials (o normalised per split, lse) into the
// final fp16 rows: LSE = ln sum_s exp(lse_s), out = sum_s exp(lse_s - LSE) o_s,
// skipping empty splits (lse = -inf).
//
// One wave per (row, head): the lanes first reduce the split lse values
// (max, then sum of exponentials), then each lane accumulates a float4 slice
// of the channels over the splits — reads of one split are 1 KB contiguous.
#include "sv_common.h"

namespace sv {

namespace {
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
}  // namespace

__global__ __launch_bounds__(kThreads) void merge_kernel(MergeArgs a) {
  const int lane = threadIdx.x % kWave;
  const long long item = (long long)blockIdx.x * kWavesPerGroup + threadIdx.x / kWave;
  const long long n_items = (long long)a.num_rows * a.num_heads;
  if (item >= n_items) return;
  const int row = (int)(item / a.num_heads);
  int S = a.num_splits;
  if (a.kv_lens) {
    // merge launched by the verify entry point: a request covered by a single
    // chunk was written directly, and chunks past its length hold nothing
    int dummy = 0;
    const int b = row / a.q_len;
    const int kv = clamp_kv_len(a.kv_lens[b], a.max_kv_len, a.max_pages, a.page_size, &dummy);
    const int nch = kv > 0 ? (kv + a.chunk - 1) / a.chunk : 1;
    if (nch <= 1) return;
    S = min(S, nch);
  }
  const size_t split_stride_l = (size_t)a.num_rows * a.num_heads;
  const size_t split_stride_o = split_stride_l * a.head_dim;

  float mx = -INFINITY;
  for (int s = lane; s < S; s += kWave) mx = fmaxf(mx, a.part_lse[(size_t)s * split_stride_l + item]);
  mx = wave_max(mx);
  const float ref = (mx == -INFINITY) ? 0.f : mx;
  float tot = 0.f;
  for (int s = lane; s < S; s += kWave) {
    const float l = a.part_lse[(size_t)s * split_stride_l + item];
    tot += (l == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((l - ref) * kLog2e);
  }
  tot = wave_sum(tot);
  const float inv = tot > 0.f ? 1.f / tot : 0.f;

  const int D4 = a.head_dim / 4;
  for (int d4 = lane; d4 < D4; d4 += kWave) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < S; ++s) {
      const float l = a.part_lse[(size_t)s * split_stride_l + item];
      if (l == -INFINITY) continue;
      const float w = __builtin_amdgcn_exp2f((l - ref) * kLog2e);
      const float4 o = reinterpret_cast<const float4*>(a.part_o + (size_t)s * split_stride_o +
                                                       item * a.head_dim)[d4];
      acc.x += w * o.x;
      acc.y += w * o.y;
      acc.z += w * o.z;
      acc.w += w * o.w;
    }
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    h4 hv = {(_Float16)(acc.x * inv), (_Float16)(acc.y * inv), (_Float16)(acc.z * inv),
             (_Float16)(acc.w * inv)};
    reinterpret_cast<h4*>(a.out + item * a.head_dim)[d4] = hv;
  }
  if (a.out_lse && lane == 0)
    a.out_lse[item] = tot > 0.f ? ref + __builtin_amdgcn_logf(tot) * kLn2 : -INFINITY;
}

void launch_merge(const MergeArgs& a, hipStream_t s) {
  const long long n_items = (long long)a.num_rows * a.num_heads;
  const unsigned blocks = (unsigned)((n_items + kWavesPerGroup - 1) / kWavesPerGroup);
  hipLaunchKernelGGL(merge_kernel, dim3(blocks), dim3(kThreads), 0, s, a);
}

}  // namespace sv
