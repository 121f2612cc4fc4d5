// Preparing a verify block and appending its K/V to the paged cache.
//
// prepare_block (one workgroup): request b with committed length L_b and
//   block width q_b gets the packed rows q_start[b] .. q_start[b]+q_b-1
//   (q_start is the exclusive prefix sum of the widths), row i the position
//   L_b + i, the cache slot page_table[b][pos / P] * P + pos % P reserved for
//   it, and (optionally) the block id t0 (i = 0) or draft d_i; the cache
//   length the verify pass sees is L_b + q_b. The requests are taken 256 at a
//   time: a scan of the widths in LDS plus a running carry, then each thread
//   writes its own request's rows.
// append_kv: one thread per 16 bytes of a new K or V row copies it into its
//   slot; rows whose slot is -1 (no reserved page) are skipped.
#include <stdint.h>

#include "sv_block.h"
#include "sv_common.h"

namespace sv {

__global__ __launch_bounds__(kThreads) void prepare_block_kernel(PrepareArgs a) {
  __shared__ int scan[kThreads];
  __shared__ int carry_s;
  const int tid = threadIdx.x;
  int flag_bits = 0;
  if (tid == 0) carry_s = 0;
  __syncthreads();
  for (int c = 0; c < a.batch; c += kThreads) {
    const int b = c + tid;
    int qb = 0, L = 0;
    if (b < a.batch) {
      qb = a.q_lens[b];
      if (qb < 0 || qb > a.max_width) {
        flag_bits |= 0x8;
        qb = 0;
      }
      L = a.seq_lens[b];
      if (L < 0 || L > 0x7fffffff - a.max_width) {  // (keeps L_b + q_b in int32)
        flag_bits |= 0x1;
        L = L < 0 ? 0 : 0x7fffffff - a.max_width;
      }
    }
    // inclusive scan of the widths of this group of requests
    scan[tid] = qb;
    __syncthreads();
    for (int o = 1; o < kThreads; o <<= 1) {
      const int v = tid >= o ? scan[tid - o] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    const int carry = carry_s;
    const int start = carry + scan[tid] - qb;
    if (b < a.batch) {
      a.q_start[b] = start;
      if (a.kv_lens_out) a.kv_lens_out[b] = L + qb;
      const int32_t* pt = a.page_table + (size_t)b * a.max_pages;
      for (int i = 0; i < qb; ++i) {
        const int r = start + i;
        const long long pos = (long long)L + i;
        int slot = -1;
        if (pos < (long long)a.max_pages * a.page_size) {
          const int pid = pt[pos / a.page_size];
          if (pid >= 0 && pid < a.num_pages) slot = pid * a.page_size + (int)(pos % a.page_size);
        }
        if (slot < 0) flag_bits |= 0x4;
        if (a.positions) a.positions[r] = (int)pos;
        a.cache_slot[r] = slot;
        if (a.block_ids) a.block_ids[r] = i == 0 ? a.last_tokens[b] : a.draft_ids[(size_t)b * (a.max_width - 1) + i - 1];
      }
    }
    __syncthreads();  // every thread has read carry_s
    if (tid == kThreads - 1) carry_s = carry + scan[tid];
    __syncthreads();
  }
  if (tid == 0) a.q_start[a.batch] = carry_s;
  if (flag_bits && a.flags) atomicOr(a.flags, flag_bits);
}

__global__ __launch_bounds__(kThreads) void append_kv_kernel(AppendArgs a) {
  // rows q_start[0] .. q_start[batch]-1 exist; a 16-byte piece per thread
  const int chunks = a.head_dim / 8;  // 16-byte pieces per (row, KV head)
  const long long item = (long long)blockIdx.x * kThreads + threadIdx.x;
  const long long per_row = (long long)a.num_kv_heads * chunks;
  const int row = (int)(item / per_row);
  if (row >= a.max_rows) return;
  const int lo_row = a.q_start[0], hi_row = a.q_start[a.batch];
  if (row < lo_row || row >= hi_row) return;
  const int rem = (int)(item % per_row);
  const int h = rem / chunks, c = rem % chunks;
  const int slot = a.cache_slot[row];
  if (slot < 0) return;
  if ((long long)slot >= (long long)a.num_pages * a.page_size) {
    if (a.flags) atomicOr(a.flags, 0x4);
    return;
  }
  const int page = slot / a.page_size, s = slot % a.page_size;
  const size_t src = ((size_t)row * a.num_kv_heads + h) * a.head_dim + 8 * c;
  const size_t dst = (((size_t)page * a.num_kv_heads + h) * a.page_size + s) * a.head_dim + 8 * c;
  const uint4 kv = *reinterpret_cast<const uint4*>(a.new_k + src);
  const uint4 vv = *reinterpret_cast<const uint4*>(a.new_v + src);
  *reinterpret_cast<uint4*>(a.k_pages + dst) = kv;
  *reinterpret_cast<uint4*>(a.v_pages + dst) = vv;
}

// E4M3 byte of y (|y| <= 448): the nearest finite value, ties to the even
// code, the sign of y kept. Normal range (|y| >= 2^-6): the fp32 mantissa
// rounded to 3 bits, to nearest even; below it, multiples of 2^-9 (2^-6 itself
// is code 0x08).
__device__ __forceinline__ uint32_t e4m3_rne(float y) {
  const uint32_t bits = __float_as_uint(y);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const float ay = fabsf(y);
  uint32_t code;
  if (ay >= 0.015625f) {
    const uint32_t ab = __float_as_uint(ay);
    int e = (int)(ab >> 23) - 127;  // -6 .. 8
    uint32_t q = (ab >> 20) & 7u;
    const uint32_t rem = ab & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) ++q;
    if (q == 8u) {
      q = 0u;
      ++e;
    }
    code = ((uint32_t)(e + 7) << 3) | q;
  } else {
    code = (uint32_t)rintf(ay * 512.f);  // exact scaling; round to nearest even
  }
  return sign | code;
}

// One wave per (row, KV head): lane l quantises channels 4l .. 4l+3 of each
// 256-channel group; the 16 lanes of a 64-channel block share its largest
// |x|. scale = fp16(amax / 448) (1.0 where that is 0), code = E4M3 of
// clamp(x / scale, +-448); both divisions rounded to nearest.
__global__ __launch_bounds__(kThreads) void append_kv_fp8_kernel(AppendFp8Args a) {
  const int lane = threadIdx.x % kWave;
  const long long item = (long long)blockIdx.x * kWavesPerGroup + threadIdx.x / kWave;
  const int row = (int)(item / a.num_kv_heads), h = (int)(item % a.num_kv_heads);
  if (row >= a.max_rows) return;
  if (row < a.q_start[0] || row >= a.q_start[a.batch]) return;
  const int slot = a.cache_slot[row];
  if (slot < 0) return;
  if ((long long)slot >= (long long)a.num_pages * a.page_size) {
    if (a.flags && lane == 0) atomicOr(a.flags, 0x4);
    return;
  }
  const int page = slot / a.page_size, s = slot % a.page_size;
  const size_t src = ((size_t)row * a.num_kv_heads + h) * a.head_dim;
  const size_t dst = (((size_t)page * a.num_kv_heads + h) * a.page_size + s) * a.head_dim;
  const int nb = a.head_dim / 64;
#pragma unroll
  for (int kv = 0; kv < 2; ++kv) {
    const _Float16* in = (kv ? a.new_v : a.new_k) + src;
    uint8_t* out = (kv ? a.v_pages : a.k_pages) + dst;
    _Float16* sc_out = (kv ? a.v_scales : a.k_scales) + dst / 64;
    for (int c0 = 4 * lane; c0 - 4 * lane < a.head_dim; c0 += 4 * kWave) {
      const bool on = c0 < a.head_dim;  // (uniform trip count: every lane shuffles)
      float x[4] = {0.f, 0.f, 0.f, 0.f};
      if (on) {
        typedef _Float16 h4 __attribute__((ext_vector_type(4)));
        const h4 v = *reinterpret_cast<const h4*>(in + c0);
#pragma unroll
        for (int k = 0; k < 4; ++k) x[k] = (float)v[k];
      }
      float m = fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3])));
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
      _Float16 sc = (_Float16)__fdiv_rn(m, 448.f);
      if (sc == (_Float16)0.f) sc = (_Float16)1.f;
      if (on) {
        const float fs = (float)sc;
        uint32_t packed = 0u;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float y = fminf(fmaxf(__fdiv_rn(x[k], fs), -448.f), 448.f);
          packed |= e4m3_rne(y) << (8 * k);
        }
        *reinterpret_cast<uint32_t*>(out + c0) = packed;
        if ((lane & 15) == 0 && c0 / 64 < nb) sc_out[c0 / 64] = sc;
      }
    }
  }
}

void launch_prepare_block(const PrepareArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(prepare_block_kernel, dim3(1), dim3(kThreads), 0, s, a);
}

void launch_append_kv_fp8(const AppendFp8Args& a, hipStream_t s) {
  const long long items = (long long)a.max_rows * a.num_kv_heads;  // one wave each
  const long long groups = (items + kWavesPerGroup - 1) / kWavesPerGroup;
  hipLaunchKernelGGL(append_kv_fp8_kernel, dim3((unsigned)groups), dim3(kThreads), 0, s, a);
}

void launch_append_kv(const AppendArgs& a, hipStream_t s) {
  const long long items = (long long)a.max_rows * a.num_kv_heads * (a.head_dim / 8);
  const long long groups = (items + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(append_kv_kernel, dim3((unsigned)groups), dim3(kThreads), 0, s, a);
}

}  // namespace sv
