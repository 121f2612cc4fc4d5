// Greedy acceptance of a verify block: block-wise argmax over fp32 logits,
// then the longest prefix of drafts that match, the bonus token and the new
// cache length.
//
// Stage 1 (argmax_partial): one workgroup per (row, slice of 8,192 columns);
//   every thread issues all of its float4 loads first, then keeps the winner
//   under the rule "larger value, then lower index"; winners are combined
//   with the same rule across the wave (shuffles) and across the 4 waves
//   (LDS). Output (value, index) per (row, slice).
// Stage 2 (accept_finalize): one workgroup per request reduces the slices of
//   all its q_len rows at once (a team of lanes per row) and walks the drafts.
// The logits are read once; the scan is HBM-bound.
#include <stdint.h>

#include "sv_common.h"
#include "sv_accept.h"

namespace sv {

namespace {

struct Best {
  float v;
  int i;
};

__device__ __forceinline__ Best better(Best a, Best b) {
  // larger value wins; equal values: lower index wins. NaN never wins.
  if (b.v > a.v || (b.v == a.v && b.i < a.i)) return b;
  return a;
}

__device__ __forceinline__ Best wave_best(Best x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    Best y;
    y.v = __shfl_xor(x.v, o);
    y.i = __shfl_xor(x.i, o);
    x = better(x, y);
  }
  return x;
}

}  // namespace

template <bool VEC4, bool NT>
__global__ __launch_bounds__(kThreads) void argmax_partial_kernel(const float* __restrict__ logits,
                                                                  int vocab, int slice,
                                                                  int n_slices, float2* ws,
                                                                  const int32_t* q_start, int batch,
                                                                  int max_rows) {
  const int sl = blockIdx.x, row = blockIdx.y;
  if (q_start) {
    // packed widths: only rows q_start[0] .. q_start[batch]-1 exist
    const int lo_row = q_start[0], hi_row = q_start[batch];
    if (row < lo_row || row >= hi_row || row >= max_rows) return;
  }
  const int lo = sl * slice, hi = min(lo + slice, vocab);
  const float* rp = logits + (size_t)row * vocab;
  Best b{-INFINITY, INT32_MAX};
  if (VEC4) {
    // columns [lo, hi) with lo, hi multiples of 4 (vocab % 4 == 0); all of a
    // thread's loads are issued before any is used
    constexpr int kPer = kAcceptSlice / (4 * kThreads);
    float4 v[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int c = lo + 4 * (threadIdx.x + u * kThreads);
      v[u] = c < hi ? load4<NT>(rp + c)
                    : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int c = lo + 4 * (threadIdx.x + u * kThreads);
      b = better(b, Best{v[u].x, c});
      b = better(b, Best{v[u].y, c + 1});
      b = better(b, Best{v[u].z, c + 2});
      b = better(b, Best{v[u].w, c + 3});
    }
  } else {
    for (int c = lo + threadIdx.x; c < hi; c += kThreads) b = better(b, Best{rp[c], c});
  }
  b = wave_best(b);
  __shared__ Best sb[kWavesPerGroup];
  const int w = threadIdx.x / kWave;
  if (threadIdx.x % kWave == 0) sb[w] = b;
  __syncthreads();
  if (threadIdx.x == 0) {
    Best r = sb[0];
    for (int k = 1; k < kWavesPerGroup; ++k) r = better(r, sb[k]);
    ws[(size_t)row * n_slices + sl] = make_float2(r.v, __int_as_float(r.i));
  }
}

// One workgroup per request: the slices of all its rows are reduced at once
// (each row by a team of lanes), then one thread walks the drafts.
__global__ __launch_bounds__(kThreads) void accept_finalize_kernel(AcceptLaunch a) {
  __shared__ int am_s[kMaxAcceptRows];
  __shared__ int dr_s[kMaxAcceptRows];
  __shared__ int kv_s;
  __shared__ Best red[kThreads];
  const int b = blockIdx.x, tid = threadIdx.x;
  const float2* __restrict__ ws = a.ws;
  const int n_slices = a.n_slices;
  // the request's rows r0 .. r0+q_len-1, and where the draft checked against
  // row j sits: d_{j+1} of the padded draft matrix, or the block id one row on
  int q_len = a.q_len, r0 = b * a.q_len;
  const int32_t* dp = a.draft_ids;
  if (!a.q_start) {
    if (q_len > 1) dp += (size_t)b * (q_len - 1);
  } else {
    int flag_bits = 0;
    q_len = block_rows(a.q_start, b, a.batch, a.q_len, &r0, &flag_bits);
    if (q_len == 0) {
      // no block (width 0, or marked): nothing accepted, no bonus, length kept
      if (tid == 0) {
        a.accept_len[b] = 0;
        a.bonus_ids[b] = -1;
        if (a.kv_lens_out) a.kv_lens_out[b] = a.kv_lens_in[b];
        if (flag_bits && a.flags) atomicOr(a.flags, flag_bits);
      }
      return;
    }
    dp = a.block_ids + r0 + 1;
  }
  // the drafts and the length go to LDS up front, beside the slice reads, so
  // the walk below is no chain of dependent global loads
  for (int j = tid; j < q_len - 1; j += kThreads) dr_s[j] = dp[j];
  if (tid == kThreads - 1 && a.kv_lens_out) kv_s = a.kv_lens_in[b];
  // team of lanes per row: the largest power of two with q_len teams <= 256
  int team = kThreads;
  while (team > 1 && team * q_len > kThreads) team >>= 1;
  for (int j0 = 0; j0 < q_len; j0 += kThreads / team) {
    const int j = j0 + tid / team, k = tid % team;
    Best x{-INFINITY, INT32_MAX};
    if (j < q_len) {
      const size_t row = (size_t)r0 + j;
      for (int s = k; s < n_slices; s += team) {
        const float2 p = ws[row * n_slices + s];
        x = better(x, Best{p.x, __float_as_int(p.y)});
      }
    }
    red[tid] = x;
    __syncthreads();
    for (int w = team / 2; w > 0; w >>= 1) {
      if (k < w) red[tid] = better(red[tid], red[tid + w]);
      __syncthreads();
    }
    if (k == 0 && j < q_len) {
      const int am = (red[tid].i == INT32_MAX) ? 0 : red[tid].i;
      am_s[j] = am;
      if (a.argmax_ids) a.argmax_ids[(size_t)r0 + j] = am;
    }
    __syncthreads();
  }
  if (tid == 0) {
    int acc = 0;
    while (acc < q_len - 1 && dr_s[acc] == am_s[acc]) ++acc;
    a.accept_len[b] = acc;
    a.bonus_ids[b] = am_s[acc];
    if (a.kv_lens_out) a.kv_lens_out[b] = kv_s - q_len + 1 + acc;
  }
}

void launch_greedy_accept(const AcceptLaunch& a, hipStream_t s) {
  const int max_rows = a.batch * a.q_len;
  dim3 g1(a.n_slices, max_rows);
  const bool once = (long long)max_rows * a.vocab * (long long)sizeof(float) >= kStreamOnceBytes;
  if (a.vocab % 4 == 0 && once)
    hipLaunchKernelGGL((argmax_partial_kernel<true, true>), g1, dim3(kThreads), 0, s, a.logits, a.vocab,
                       a.slice, a.n_slices, a.ws, a.q_start, a.batch, max_rows);
  else if (a.vocab % 4 == 0)
    hipLaunchKernelGGL((argmax_partial_kernel<true, false>), g1, dim3(kThreads), 0, s, a.logits, a.vocab,
                       a.slice, a.n_slices, a.ws, a.q_start, a.batch, max_rows);
  else
    hipLaunchKernelGGL((argmax_partial_kernel<false, false>), g1, dim3(kThreads), 0, s, a.logits, a.vocab,
                       a.slice, a.n_slices, a.ws, a.q_start, a.batch, max_rows);
  hipLaunchKernelGGL(accept_finalize_kernel, dim3(a.batch), dim3(kThreads), 0, s, a);
}

}  // namespace sv
