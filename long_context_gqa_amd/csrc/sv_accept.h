// Launch descriptor of the greedy-accept kernels (internal header).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

struct AcceptLaunch {
  const float* logits;
  const int32_t* draft_ids;  // uniform widths: [batch, q_len-1]
  const int32_t* block_ids;  // packed widths: [rows] = t0, d1, .. per request
  const int32_t* q_start;    // packed widths: row offsets [batch+1]; NULL for uniform
  int32_t* flags;
  int32_t batch, q_len, vocab, slice, n_slices;  // q_len: the (largest) width
  int32_t* accept_len;
  int32_t* bonus_ids;
  int32_t* argmax_ids;
  const int32_t* kv_lens_in;
  int32_t* kv_lens_out;
  float2* ws;  // [batch*q_len, n_slices] (value, index bits)
};

constexpr int kAcceptSlice = 8192;  // vocabulary columns per argmax workgroup
constexpr int kMaxAcceptRows = 1024;  // largest q_len sv_greedy_accept takes

void launch_greedy_accept(const AcceptLaunch& a, hipStream_t s);

}  // namespace sv
