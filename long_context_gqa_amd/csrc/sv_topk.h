// Launch descriptor of the top-k candidate kernels (internal header).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

struct TopkLaunch {
  const float* logits;  // [rows, vocab]
  int32_t rows, vocab, k, n_slices, slice;  // slice: kTopkSlice or kTopkSliceWide
  float2* ws;           // [rows, n_slices, k] (value, index bits)
  int32_t* out_ids;     // [rows, k]
  float* out_vals;      // [rows, k]
};

constexpr int kTopkSlice = 8192;     // vocabulary columns per stage-1 workgroup (bounds the workspace)
constexpr int kTopkSliceWide = 16384;  // the wider slices used for few rows
constexpr int kMaxTopk = 16;         // largest k
constexpr int kMergePerLane = 8;     // stage 2: one wave holds n_slices * k <= 512 candidates

void launch_topk(const TopkLaunch& a, hipStream_t s);

}  // namespace sv
