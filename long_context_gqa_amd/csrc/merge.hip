// Merge of split-KV attention partials (o normalised per split, lse) into the
// final fp16 rows: LSE = ln sum_s exp(lse_s), out = sum_s exp(lse_s - LSE) o_s,
// skipping empty splits (lse = -inf).
//
// Few items (rows x heads): one workgroup per (row, head). Its threads first
// reduce the split lse values (max, then the sum of exponentials); then wave
// w accumulates splits w, w+4, ... with each lane owning a float4 of channels
// and four splits' loads in flight at a time; the four waves' sums are added
// through LDS. Many items: one wave per (row, head), the same arithmetic
// with wave reductions only.
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

__device__ __forceinline__ float block_reduce(float v, float* red, bool is_max) {
  v = is_max ? wave_max(v) : wave_sum(v);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if (threadIdx.x % kWave == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
  for (int k = 1; k < kWavesPerGroup; ++k) r = is_max ? fmaxf(r, red[k]) : r + red[k];
  return r;
}

// The splits to merge for packed row `row`: all of them for a standalone
// merge; for the verify entry point the chunks the attention kernel wrote
// for the row's request (0: nothing to merge, the row was written directly
// or belongs to no request).
__device__ __forceinline__ int item_splits(const MergeArgs& a, int row) {
  int S = a.num_splits;
  if (a.counters || a.balanced) return S;  // claimed work, balanced chunks: every workgroup wrote its slot
  if (a.kv_lens) {
    // merge launched by the verify entry point: a request covered by a single
    // chunk was written directly, and chunks past its length hold nothing
    int dummy = 0;
    int b = row / a.q_len;
    int q_b = a.q_len;
    if (a.q_start) {
      // packed rows: the request is the last b with q_start[b] <= row; rows
      // of no request (past the block, or of a marked request) are skipped
      int lo = 0, hi = a.batch - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (a.q_start[mid] <= row) lo = mid;
        else hi = mid - 1;
      }
      b = lo;
      int st = 0;
      const int n = block_rows(a.q_start, b, a.batch, a.q_len, &st, &dummy);
      if (row < st || row >= st + n) return 0;
      q_b = n;
    }
    const int kv = clamp_kv_len(a.kv_lens[b], a.max_kv_len, a.max_pages, a.page_size, &dummy);
    // the chunks the attention wrote: the block's live key steps in chunks
    // of a.chunk / 16 steps (the count the attention kernel uses)
    int n_sink, w0;
    const int total = live_steps(kv, kv - q_b, a.window, a.sink, &n_sink, &w0);
    const int cs = a.chunk / 16;
    const int nch = total > 0 ? (total + cs - 1) / cs : 1;
    if (nch <= 1) return 0;
    S = min(S, nch);
  }
  return S;
}

// Claimed work: each grain counter must have ended at the number of grains
// it deals plus the number of waves that claim from it (each fails once),
// and each group's tally of grains taken (word 1 of its first counter's
// line) at the group's grain count; anything else means a counter did not
// start at zero (bit 0x10): one that started a little above zero skips its
// first grains yet ends at the clean value, which only the tally shows.
// Either way both are left at zero for the next call. Runs once, in block 0,
// after the attention kernel has finished.
__device__ __forceinline__ void settle_counters(const MergeArgs& a) {
  const int groups = a.batch * a.num_kv_heads;
  const int C = a.counters ? claim_counters(a.num_splits, groups) : 1;
  if (!a.counters || blockIdx.x != 0 || (int)threadIdx.x >= groups * C) return;
  const int q = (int)threadIdx.x / C, c = (int)threadIdx.x % C;  // group q = b * Hkv + g
  int dummy = 0;
  const int kv = clamp_kv_len(a.kv_lens[q / a.num_kv_heads], a.max_kv_len, a.max_pages, a.page_size, &dummy);
  int f, pool0, n_grains;
  claim_layout(kv > 0 ? (kv + 15) / 16 : 0, a.num_splits, &f, &pool0, &n_grains);
  // counter c of C deals its grains to S / 2 / C * 8 waves, each of which
  // fails once
  const int want = counter_grains(n_grains, c, C) + a.num_splits / 2 / C * 8;
  int32_t* const ctr = a.counters + threadIdx.x * kCounterStride;
  bool dirty = *ctr != want;
  *ctr = 0;
  if (c == 0) {
    dirty = dirty || ctr[1] != n_grains;
    ctr[1] = 0;
  }
  if (dirty && a.flags) atomicOr(a.flags, 0x10);
}

__global__ __launch_bounds__(kThreads) void merge_kernel(MergeArgs a) {
  settle_counters(a);
  __shared__ float red[kWavesPerGroup];
  __shared__ float4 acc_s[kWavesPerGroup - 1][kWave];
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const long long item = blockIdx.x;  // (row, head)
  const int row = (int)(item / a.num_heads);
  const int S = item_splits(a, row);
  if (S <= 0) return;
  const size_t sl = (size_t)a.num_rows * a.num_heads;  // stride between splits (lse)
  const size_t so = sl * a.head_dim;                     // stride between splits (o)
  const float* lse = a.part_lse + item;
  const float* po = a.part_o + item * a.head_dim;

  // Up to 64 splits of 256 channels (every launch of the verify entry point
  // with a workgroup per item): wave w takes splits w, w + 4, ..., lane l
  // channels 4l..4l+3, and every load goes out at once (one round trip);
  // the split maximum and the sums meet in LDS.
  constexpr int kPer = 16;
  if (S <= kWavesPerGroup * kPer && a.head_dim == 4 * kWave) {
    float lv[kPer];
    float4 ov[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int s = w + kWavesPerGroup * k;
      lv[k] = -INFINITY;
      ov[k] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (s < S) {
        lv[k] = lse[s * sl];
        ov[k] = reinterpret_cast<const float4*>(po + s * so)[lane];
      }
    }
    float m = -INFINITY;
#pragma unroll
    for (int k = 0; k < kPer; ++k) m = fmaxf(m, lv[k]);
    if (lane == 0) red[w] = m;
    __syncthreads();
    float M = red[0];
#pragma unroll
    for (int k = 1; k < kWavesPerGroup; ++k) M = fmaxf(M, red[k]);
    const float ref = (M == -INFINITY) ? 0.f : M;
    float t = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const float wgt = (lv[k] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((lv[k] - ref) * kLog2e);
      t += wgt;
      acc.x += wgt * ov[k].x;
      acc.y += wgt * ov[k].y;
      acc.z += wgt * ov[k].z;
      acc.w += wgt * ov[k].w;
    }
    __syncthreads();  // every wave has read red
    if (lane == 0) red[w] = t;
    if (w > 0) acc_s[w - 1][lane] = acc;
    __syncthreads();
    if (w == 0) {
      float tot = red[0];
#pragma unroll
      for (int k = 1; k < kWavesPerGroup; ++k) {
        tot += red[k];
        const float4 u = acc_s[k - 1][lane];
        acc.x += u.x;
        acc.y += u.y;
        acc.z += u.z;
        acc.w += u.w;
      }
      const float inv = tot > 0.f ? 1.f / tot : 0.f;
      typedef _Float16 h4 __attribute__((ext_vector_type(4)));
      h4 hv = {(_Float16)(acc.x * inv), (_Float16)(acc.y * inv), (_Float16)(acc.z * inv),
               (_Float16)(acc.w * inv)};
      reinterpret_cast<h4*>(a.out + item * a.head_dim)[lane] = hv;
      if (a.out_lse && lane == 0)
        a.out_lse[item] = tot > 0.f ? ref + __builtin_amdgcn_logf(tot) * kLn2 : -INFINITY;
    }
    return;
  }

  float mx = -INFINITY;
  for (int s = threadIdx.x; s < S; s += kThreads) mx = fmaxf(mx, lse[s * sl]);
  mx = block_reduce(mx, red, true);
  const float ref = (mx == -INFINITY) ? 0.f : mx;
  float tot = 0.f;
  for (int s = threadIdx.x; s < S; s += kThreads) {
    const float l = lse[s * sl];
    tot += (l == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((l - ref) * kLog2e);
  }
  tot = block_reduce(tot, red, false);
  const float inv = tot > 0.f ? 1.f / tot : 0.f;

  const int D4 = a.head_dim / 4;
  // uniform trip count: every lane passes the same barriers
  for (int base = 0; base < D4; base += kWave) {
    const int d4 = base + lane;
    const bool on = d4 < D4;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (on) {
      int s = w;
      for (; s + 3 * kWavesPerGroup < S; s += 4 * kWavesPerGroup) {
        float l[4];
        float4 o[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          l[u] = lse[(s + u * kWavesPerGroup) * sl];
          o[u] = reinterpret_cast<const float4*>(po + (s + u * kWavesPerGroup) * so)[d4];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float wgt = (l[u] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((l[u] - ref) * kLog2e);
          acc.x += wgt * o[u].x;
          acc.y += wgt * o[u].y;
          acc.z += wgt * o[u].z;
          acc.w += wgt * o[u].w;
        }
      }
      for (; s < S; s += kWavesPerGroup) {
        const float l = lse[s * sl];
        const float wgt = (l == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((l - ref) * kLog2e);
        const float4 o = reinterpret_cast<const float4*>(po + s * so)[d4];
        acc.x += wgt * o.x;
        acc.y += wgt * o.y;
        acc.z += wgt * o.z;
        acc.w += wgt * o.w;
      }
      if (w > 0) acc_s[w - 1][lane] = acc;
    }
    __syncthreads();
    if (w == 0 && on) {
#pragma unroll
      for (int k = 0; k < kWavesPerGroup - 1; ++k) {
        const float4 t = acc_s[k][lane];
        acc.x += t.x;
        acc.y += t.y;
        acc.z += t.z;
        acc.w += t.w;
      }
      typedef _Float16 h4 __attribute__((ext_vector_type(4)));
      h4 hv = {(_Float16)(acc.x * inv), (_Float16)(acc.y * inv), (_Float16)(acc.z * inv),
               (_Float16)(acc.w * inv)};
      reinterpret_cast<h4*>(a.out + item * a.head_dim)[d4] = hv;
    }
    __syncthreads();
  }
  if (a.out_lse && threadIdx.x == 0)
    a.out_lse[item] = tot > 0.f ? ref + __builtin_amdgcn_logf(tot) * kLn2 : -INFINITY;
}

// One wave per (row, head), for launches with many items (each with few
// splits): no workgroup barriers. Each lane owns a float4 of channels; up to
// 16 splits are loaded at once, more four at a time with wave reductions of
// the lse values.
__global__ __launch_bounds__(kThreads) void merge_wave_kernel(MergeArgs a) {
  settle_counters(a);
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const long long item = (long long)blockIdx.x * kWavesPerGroup + w;
  if (item >= (long long)a.num_rows * a.num_heads) return;
  const int row = (int)(item / a.num_heads);
  const int S = item_splits(a, row);
  if (S <= 0) return;
  const size_t sl = (size_t)a.num_rows * a.num_heads;
  const size_t so = sl * a.head_dim;
  const float* lse = a.part_lse + item;
  const float* po = a.part_o + item * a.head_dim;
  typedef _Float16 h4 __attribute__((ext_vector_type(4)));
  // Up to 16 splits of 256 channels: every lane loads its float4 of all
  // splits and every split's lse at once (one round trip), then reduces in
  // registers.
  constexpr int kOnce = 16;
  if (S <= kOnce && a.head_dim == 4 * kWave) {
    float lv[kOnce];
    float4 ov[kOnce];
#pragma unroll
    for (int s = 0; s < kOnce; ++s) {
      lv[s] = -INFINITY;
      ov[s] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (s < S) {
        lv[s] = lse[s * sl];
        ov[s] = reinterpret_cast<const float4*>(po + s * so)[lane];
      }
    }
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < kOnce; ++s) M = fmaxf(M, lv[s]);
    const float ref = (M == -INFINITY) ? 0.f : M;
    float t = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int s = 0; s < kOnce; ++s) {
      const float wgt = (lv[s] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((lv[s] - ref) * kLog2e);
      t += wgt;
      acc.x += wgt * ov[s].x;
      acc.y += wgt * ov[s].y;
      acc.z += wgt * ov[s].z;
      acc.w += wgt * ov[s].w;
    }
    const float inv = t > 0.f ? 1.f / t : 0.f;
    h4 hv = {(_Float16)(acc.x * inv), (_Float16)(acc.y * inv), (_Float16)(acc.z * inv), (_Float16)(acc.w * inv)};
    reinterpret_cast<h4*>(a.out + item * a.head_dim)[lane] = hv;
    if (a.out_lse && lane == 0) a.out_lse[item] = t > 0.f ? ref + __builtin_amdgcn_logf(t) * kLn2 : -INFINITY;
    return;
  }
  float mx = -INFINITY;
  for (int s = lane; s < S; s += kWave) mx = fmaxf(mx, lse[s * sl]);
  mx = wave_max(mx);
  const float ref = (mx == -INFINITY) ? 0.f : mx;
  float tot = 0.f;
  for (int s = lane; s < S; s += kWave) {
    const float l = lse[s * sl];
    tot += (l == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((l - ref) * kLog2e);
  }
  tot = wave_sum(tot);
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  const int D4 = a.head_dim / 4;
  for (int d4 = lane; d4 < D4; d4 += kWave) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    int s = 0;
    for (; s + 3 < S; s += 4) {
      float l[4];
      float4 o[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        l[u] = lse[(s + u) * sl];
        o[u] = reinterpret_cast<const float4*>(po + (s + u) * so)[d4];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float wgt = (l[u] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((l[u] - ref) * kLog2e);
        acc.x += wgt * o[u].x;
        acc.y += wgt * o[u].y;
        acc.z += wgt * o[u].z;
        acc.w += wgt * o[u].w;
      }
    }
    for (; s < S; ++s) {
      const float l = lse[s * sl];
      const float wgt = (l == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((l - ref) * kLog2e);
      const float4 o = reinterpret_cast<const float4*>(po + s * so)[d4];
      acc.x += wgt * o.x;
      acc.y += wgt * o.y;
      acc.z += wgt * o.z;
      acc.w += wgt * o.w;
    }
    h4 hv = {(_Float16)(acc.x * inv), (_Float16)(acc.y * inv), (_Float16)(acc.z * inv), (_Float16)(acc.w * inv)};
    reinterpret_cast<h4*>(a.out + item * a.head_dim)[d4] = hv;
  }
  if (a.out_lse && lane == 0) a.out_lse[item] = tot > 0.f ? ref + __builtin_amdgcn_logf(tot) * kLn2 : -INFINITY;
}

// Few items (e.g. one long request: many splits each): a workgroup per item
// spreads its splits over four waves; many items: a wave per item.
constexpr long long kWaveMergeItems = 4096;

void launch_merge(const MergeArgs& a, hipStream_t s) {
  const long long n_items = (long long)a.num_rows * a.num_heads;
  if (n_items >= kWaveMergeItems)
    hipLaunchKernelGGL(merge_wave_kernel, dim3((unsigned)((n_items + kWavesPerGroup - 1) / kWavesPerGroup)),
                       dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(merge_kernel, dim3((unsigned)n_items), dim3(kThreads), 0, s, a);
}

}  // namespace sv
