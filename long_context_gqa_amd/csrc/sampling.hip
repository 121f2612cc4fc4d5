// Stochastic acceptance of a verify block by rejection sampling: draft
// d_{j+1} is kept while u_j * q_j(d) < p_j(d), with p_j = softmax(row j / T);
// the final token is drawn by inverse CDF with u_final from the residual
// max(p_A - q_A, 0) of the first rejected row A (or from p_{q-1} when every
// draft is kept).
//
// Stage 1 (row_stats): one workgroup per (row, slice of 8,192 columns): the
//   slice's max of z = logit * log2(e)/T and sum of 2^(z - max), combined
//   across threads, waves and (in stage 2) slices. One HBM pass over the
//   logits.
// Stage 2 (walk_residual): one workgroup per (slice, request): the row
//   statistics of the request's rows, the acceptance walk (a few element
//   reads), then the sum over this slice of the weight the final draw uses.
// Stage 3 (draw): one workgroup per request: the slice where the cumulative
//   weight passes u_final * total, then a scan inside that slice.
#include <stdint.h>

#include "sv_common.h"
#include "sv_sampling.h"

namespace sv {

namespace {

struct Stat {
  float m, s;  // max of z; sum of 2^(z - m)
};

__device__ __forceinline__ Stat combine(Stat a, Stat b) {
  const float m = fmaxf(a.m, b.m);
  if (m == -INFINITY) return Stat{-INFINITY, 0.f};
  return Stat{m, a.s * __builtin_amdgcn_exp2f(a.m - m) + b.s * __builtin_amdgcn_exp2f(b.m - m)};
}

__device__ __forceinline__ Stat wave_stat(Stat x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    Stat y{__shfl_xor(x.m, o), __shfl_xor(x.s, o)};
    x = combine(x, y);
  }
  return x;
}

__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Statistics (M, 1/S) of row `row` from its slices' (m, s), by one wave: lane
// k takes slice k (n_slices <= 64), then the wave combines; every lane gets
// the result.
__device__ __forceinline__ void row_stat_wave(const float2* __restrict__ ws1, int n_slices, size_t row, int lane,
                                              float* M, float* invS) {
  Stat t{-INFINITY, 0.f};
  if (lane < n_slices) {
    const float2 v = ws1[row * n_slices + lane];
    t = Stat{v.x, v.y};
  }
  t = wave_stat(t);
  *M = t.m;
  *invS = t.s > 0.f ? 1.f / t.s : 0.f;
}

__device__ __forceinline__ float wave_incl_scan(float v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  return v;
}

}  // namespace

template <bool VEC4, bool NT>
__global__ __launch_bounds__(kThreads) void row_stats_kernel(const float* __restrict__ logits, int vocab,
                                                             int slice, int n_slices, float c, float2* ws1) {
  const int sl = blockIdx.x, row = blockIdx.y;
  const int lo = sl * slice, hi = min(lo + slice, vocab);
  const float* rp = logits + (size_t)row * vocab;
  Stat st{-INFINITY, 0.f};
  if (VEC4) {
    constexpr int kPer = kSampleSlice / (4 * kThreads);
    float4 v[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int col = lo + 4 * (threadIdx.x + u * kThreads);
      v[u] = col < hi ? load4<NT>(rp + col)
                      : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    }
    float m = -INFINITY;
#pragma unroll
    for (int u = 0; u < kPer; ++u) m = fmaxf(m, fmaxf(fmaxf(v[u].x, v[u].y), fmaxf(v[u].z, v[u].w)) * c);
    float s = 0.f;
    if (m != -INFINITY) {
#pragma unroll
      for (int u = 0; u < kPer; ++u)
        s += (__builtin_amdgcn_exp2f(v[u].x * c - m) + __builtin_amdgcn_exp2f(v[u].y * c - m)) +
             (__builtin_amdgcn_exp2f(v[u].z * c - m) + __builtin_amdgcn_exp2f(v[u].w * c - m));
    }
    st = Stat{m, s};
  } else {
    float m = -INFINITY;
    for (int col = lo + threadIdx.x; col < hi; col += kThreads) m = fmaxf(m, rp[col] * c);
    float s = 0.f;
    if (m != -INFINITY)
      for (int col = lo + threadIdx.x; col < hi; col += kThreads) s += __builtin_amdgcn_exp2f(rp[col] * c - m);
    st = Stat{m, s};
  }
  st = wave_stat(st);
  __shared__ Stat sb[kWavesPerGroup];
  const int w = threadIdx.x / kWave;
  if (threadIdx.x % kWave == 0) sb[w] = st;
  __syncthreads();
  if (threadIdx.x == 0) {
    Stat r = sb[0];
    for (int k = 1; k < kWavesPerGroup; ++k) r = combine(r, sb[k]);
    ws1[(size_t)row * n_slices + sl] = make_float2(r.m, r.s);
  }
}

// Request b's row statistics (in LDS) and whether each draft passes its test
// u_j * q_j(d) < p_j(d) (an id outside the vocabulary never does): the
// tested elements are loaded for all drafts at once, then each wave combines
// the slice statistics of every fourth row.
__device__ __forceinline__ void request_tests(const SampleLaunch& a, int b, float* M, float* invS, int* keep) {
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  __shared__ float s_ld[kMaxSampleRows], s_qu[kMaxSampleRows];
  for (int j = tid; j < a.q_len - 1; j += kThreads) {
    const int d = a.draft_ids[(size_t)b * (a.q_len - 1) + j];
    const bool ok = d >= 0 && d < a.vocab;
    s_ld[j] = ok ? a.logits[((size_t)b * a.q_len + j) * a.vocab + d] : 0.f;
    // u * q(d), or +inf for an id that is never kept
    s_qu[j] = ok ? a.u_accept[(size_t)b * (a.q_len - 1) + j] *
                       a.draft_probs[((size_t)b * (a.q_len - 1) + j) * a.vocab + d]
                 : INFINITY;
  }
  for (int j = wave; j < a.q_len; j += kWavesPerGroup) {
    float m, is;
    row_stat_wave(a.ws1, a.n_slices, (size_t)b * a.q_len + j, lane, &m, &is);
    if (lane == 0) {
      M[j] = m;
      invS[j] = is;
    }
  }
  __syncthreads();
  for (int j = tid; j < a.q_len; j += kThreads)
    keep[j] = (j < a.q_len - 1) ? (int)(s_qu[j] < __builtin_amdgcn_exp2f(s_ld[j] * a.c - M[j]) * invS[j]) : 0;
  __syncthreads();
}

template <bool VEC4>
__global__ __launch_bounds__(kThreads) void walk_residual_kernel(SampleLaunch a) {
  const int sl = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  __shared__ float M[kMaxSampleRows], invS[kMaxSampleRows];
  __shared__ int keep[kMaxSampleRows];
  __shared__ int s_acc;
  // every row's statistics and every draft's test in parallel; the walk
  // then stops at the first draft that fails (the same in every workgroup)
  request_tests(a, b, M, invS, keep);
  if (tid == 0) {
    int acc = 0;
    while (acc < a.q_len - 1 && keep[acc]) ++acc;
    s_acc = acc;
  }
  __syncthreads();
  const int A = s_acc;
  const bool residual = A < a.q_len - 1;
  const size_t row = (size_t)b * a.q_len + A;
  const float* lp = a.logits + row * a.vocab;
  const float* qp = residual ? a.draft_probs + ((size_t)b * (a.q_len - 1) + A) * a.vocab : nullptr;
  const float Mr = M[A], iS = invS[A];
  const int lo = sl * a.slice, hi = min(lo + a.slice, a.vocab);
  float sum = 0.f;
  if (VEC4) {
    for (int col = lo + 4 * tid; col < hi; col += 4 * kThreads) {
      const float4 l4 = *reinterpret_cast<const float4*>(lp + col);
      float4 p4 = make_float4(__builtin_amdgcn_exp2f(l4.x * a.c - Mr) * iS, __builtin_amdgcn_exp2f(l4.y * a.c - Mr) * iS,
                              __builtin_amdgcn_exp2f(l4.z * a.c - Mr) * iS, __builtin_amdgcn_exp2f(l4.w * a.c - Mr) * iS);
      if (residual) {
        const float4 q4 = *reinterpret_cast<const float4*>(qp + col);
        p4 = make_float4(fmaxf(p4.x - q4.x, 0.f), fmaxf(p4.y - q4.y, 0.f), fmaxf(p4.z - q4.z, 0.f),
                         fmaxf(p4.w - q4.w, 0.f));
      }
      sum += (p4.x + p4.y) + (p4.z + p4.w);
    }
  } else {
    for (int col = lo + tid; col < hi; col += kThreads) {
      float p = __builtin_amdgcn_exp2f(lp[col] * a.c - Mr) * iS;
      if (residual) p = fmaxf(p - qp[col], 0.f);
      sum += p;
    }
  }
  sum = wave_sum_f(sum);
  __shared__ float red[kWavesPerGroup];
  if (tid % kWave == 0) red[tid / kWave] = sum;
  __syncthreads();
  if (tid == 0) {
    float t = 0.f;
    for (int k = 0; k < kWavesPerGroup; ++k) t += red[k];
    a.ws2[(size_t)b * a.n_slices + sl] = t;
    if (sl == 0) a.ws_acc[b] = A;
  }
}

// Weight of column col of request b's chosen row (residual or p).
__device__ __forceinline__ float weight(const float* lp, const float* qp, float c, float Mr, float iS, int col) {
  float p = __builtin_amdgcn_exp2f(lp[col] * c - Mr) * iS;
  if (qp) p = fmaxf(p - qp[col], 0.f);
  return p;
}

template <bool VEC4>
__global__ __launch_bounds__(kThreads) void draw_kernel(SampleLaunch a) {
  const int b = blockIdx.x, tid = threadIdx.x;
  __shared__ int s_k, s_mode, s_best, s_last, s_pos;
  __shared__ float s_base, s_target, s_M, s_iS;
  __shared__ float s_wt[kWavesPerGroup];
  const int A = a.ws_acc[b];
  const bool residual = A < a.q_len - 1;
  const size_t row = (size_t)b * a.q_len + A;
  if (tid < kWave) {
    // wave 0: the row's statistics, the slices' weights (the residual's, or
    // p's from the statistics when the residual is zero everywhere or every
    // draft was kept), the total, and the slice where the cumulative weight
    // passes u_final * total (a prefix scan over the slices, one per lane)
    const int lane = tid;
    float M, iS;
    row_stat_wave(a.ws1, a.n_slices, row, lane, &M, &iS);
    const bool in = lane < a.n_slices;
    const float wr = in ? a.ws2[(size_t)b * a.n_slices + lane] : 0.f;
    float tot = wave_sum_f(wr);
    int mode = residual ? 1 : 0;
    if (residual && !(tot > 0.f)) mode = 0;
    float w = wr;
    if (mode == 0 && residual) {
      // p's slice sums from the row statistics
      w = 0.f;
      if (in) {
        const float2 v = a.ws1[row * a.n_slices + lane];
        w = v.y * __builtin_amdgcn_exp2f(v.x - M) * iS;
      }
      tot = wave_sum_f(w);
    }
    const float target = a.u_final[b] * tot;
    const float cum = wave_incl_scan(w, lane);
    const uint64_t past = __ballot(in && cum > target);
    const uint64_t pos = __ballot(in && w > 0.f);
    // the first slice past the target (uniform across the wave), or when
    // rounding put the target past the total, the last positive weight
    const int k = past ? __builtin_ctzll(past) : (pos ? 63 - __builtin_clzll(pos) : 0);
    const float base = __shfl(cum, k) - __shfl(w, k);
    if (lane == 0) {
      s_last = past ? 0 : 1;
      s_k = k;
      s_base = past ? base : 0.f;
      s_target = target;
      s_mode = mode;
      s_best = INT32_MAX;
      s_M = M;
      s_iS = iS;
    }
  }
  if (tid == 0) s_pos = -1;
  __syncthreads();
  // The chosen slice: thread tid's 32 consecutive columns' weights in
  // registers (read with 16-byte loads), their sum, the block's exclusive
  // prefix of the sums (wave scans, then the earlier waves' totals), and the
  // first column whose running weight passes the target.
  const float* lp = a.logits + row * a.vocab;
  const float* qp = s_mode == 1 ? a.draft_probs + ((size_t)b * (a.q_len - 1) + A) * a.vocab : nullptr;
  const int lo = s_k * kSampleSlice, hi = min(lo + kSampleSlice, a.vocab);
  constexpr int kPer = kSampleSlice / kThreads;  // consecutive columns per thread
  const int c0 = lo + tid * kPer;
  const float Mr = s_M, iS = s_iS;
  float w[kPer];
  if (VEC4 && c0 + kPer <= hi) {
#pragma unroll
    for (int j = 0; j < kPer / 4; ++j) {
      const float4 l4 = *reinterpret_cast<const float4*>(lp + c0 + 4 * j);
      w[4 * j] = __builtin_amdgcn_exp2f(l4.x * a.c - Mr) * iS;
      w[4 * j + 1] = __builtin_amdgcn_exp2f(l4.y * a.c - Mr) * iS;
      w[4 * j + 2] = __builtin_amdgcn_exp2f(l4.z * a.c - Mr) * iS;
      w[4 * j + 3] = __builtin_amdgcn_exp2f(l4.w * a.c - Mr) * iS;
      if (qp) {
        const float4 q4 = *reinterpret_cast<const float4*>(qp + c0 + 4 * j);
        w[4 * j] = fmaxf(w[4 * j] - q4.x, 0.f);
        w[4 * j + 1] = fmaxf(w[4 * j + 1] - q4.y, 0.f);
        w[4 * j + 2] = fmaxf(w[4 * j + 2] - q4.z, 0.f);
        w[4 * j + 3] = fmaxf(w[4 * j + 3] - q4.w, 0.f);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < kPer; ++i) w[i] = c0 + i < hi ? weight(lp, qp, a.c, Mr, iS, c0 + i) : 0.f;
  }
  float loc = 0.f;
#pragma unroll
  for (int i = 0; i < kPer; ++i) loc += w[i];
  const int lane = tid % kWave, wave = tid / kWave;
  const float inc = wave_incl_scan(loc, lane);
  if (lane == kWave - 1) s_wt[wave] = inc;
  __syncthreads();
  float woff = 0.f;
  for (int v = 0; v < wave; ++v) woff += s_wt[v];
  const float excl = s_base + woff + (inc - loc);
  int last = -1;  // this thread's last column of positive weight
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    if (w[i] > 0.f) last = c0 + i;
  if (last >= 0) atomicMax(&s_pos, last);
  if (!s_last && excl + loc > s_target) {  // the crossing is in this thread's columns
    float run = excl;
    int hit = INT32_MAX;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      run += w[i];
      if (hit == INT32_MAX && run > s_target) hit = c0 + i;
    }
    if (hit != INT32_MAX) atomicMin(&s_best, hit);
  }
  __syncthreads();
  if (tid == 0) {
    // the crossing; or, when rounding put the target past the total (or past
    // this slice's own sum), the last column of positive weight
    int tok = s_best;
    if (s_last || tok == INT32_MAX) tok = s_pos >= 0 ? s_pos : hi - 1;
    a.accept_len[b] = A;
    a.token_ids[b] = tok;
    if (a.kv_lens_out) a.kv_lens_out[b] = a.kv_lens_in[b] - a.q_len + 1 + A;
  }
}

void launch_rejection_accept(const SampleLaunch& a, hipStream_t s) {
  dim3 g1(a.n_slices, a.batch * a.q_len), g2(a.n_slices, a.batch);
  const bool once = (long long)a.batch * a.q_len * a.vocab * (long long)sizeof(float) >= kStreamOnceBytes;
  if (a.vocab % 4 == 0) {
    if (once)
      hipLaunchKernelGGL((row_stats_kernel<true, true>), g1, dim3(kThreads), 0, s, a.logits, a.vocab, a.slice,
                         a.n_slices, a.c, a.ws1);
    else
      hipLaunchKernelGGL((row_stats_kernel<true, false>), g1, dim3(kThreads), 0, s, a.logits, a.vocab, a.slice,
                         a.n_slices, a.c, a.ws1);
    hipLaunchKernelGGL((walk_residual_kernel<true>), g2, dim3(kThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL((row_stats_kernel<false, false>), g1, dim3(kThreads), 0, s, a.logits, a.vocab, a.slice, a.n_slices,
                       a.c, a.ws1);
    hipLaunchKernelGGL((walk_residual_kernel<false>), g2, dim3(kThreads), 0, s, a);
  }
  if (a.vocab % 4 == 0)
    hipLaunchKernelGGL((draw_kernel<true>), dim3(a.batch), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((draw_kernel<false>), dim3(a.batch), dim3(kThreads), 0, s, a);
}

}  // namespace sv
