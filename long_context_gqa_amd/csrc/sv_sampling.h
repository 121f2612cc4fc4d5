// Launch descriptor of the rejection-sampling acceptance kernels (internal
// header).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

struct SampleLaunch {
  const float* logits;       // [batch*q_len, vocab]
  const int32_t* draft_ids;  // [batch, q_len-1]
  const float* draft_probs;  // [batch, q_len-1, vocab]
  const float* u_accept;     // [batch, q_len-1]
  const float* u_final;      // [batch]
  int32_t batch, q_len, vocab, slice, n_slices;
  float c;  // log2(e) / temperature
  int32_t* accept_len;
  int32_t* token_ids;
  const int32_t* kv_lens_in;
  int32_t* kv_lens_out;
  float2* ws1;     // [batch*q_len, n_slices] per-slice (max, sum) of the rows
  float* ws2;      // [batch, n_slices] per-slice weight of the final draw
  int32_t* ws_acc;  // [batch] drafts kept
};

constexpr int kSampleSlice = 8192;   // vocabulary columns per workgroup
constexpr int kMaxSampleRows = 64;   // largest q_len sv_rejection_accept takes

void launch_rejection_accept(const SampleLaunch& a, hipStream_t s);

}  // namespace sv
