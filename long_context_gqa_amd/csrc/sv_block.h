// Launch descriptors of the block-preparation and KV-append kernels
// (internal header).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

struct PrepareArgs {
  const int32_t* seq_lens;     // [batch] committed lengths L_b
  const int32_t* q_lens;       // [batch] block widths, 0..max_width
  const int32_t* page_table;   // [batch, max_pages]
  const int32_t* last_tokens;  // NULL, or [batch] t0 of each block
  const int32_t* draft_ids;    // with last_tokens and max_width > 1: [batch, max_width-1]
  int32_t* q_start;            // [batch+1] (written)
  int32_t* positions;          // NULL or [rows] (written)
  int32_t* cache_slot;         // [rows] page*P + slot, -1 if unreserved (written)
  int32_t* kv_lens_out;        // NULL or [batch] L_b + q_b (written)
  int32_t* block_ids;          // NULL or [rows] (written)
  int32_t* flags;
  int32_t batch, max_width, max_pages, page_size, num_pages;
};

struct AppendArgs {
  const _Float16* new_k;  // [rows, Hkv, D]
  const _Float16* new_v;
  const int32_t* cache_slot;
  const int32_t* q_start;  // [batch+1]
  _Float16* k_pages;       // [num_pages, Hkv, P, D]
  _Float16* v_pages;
  int32_t* flags;
  int32_t batch, max_rows, num_kv_heads, head_dim, page_size, num_pages;
};

// Appending into an FP8 cache: the rows are quantised per 64-channel block.
struct AppendFp8Args {
  const _Float16* new_k;  // [rows, Hkv, D]
  const _Float16* new_v;
  const int32_t* cache_slot;
  const int32_t* q_start;  // [batch+1]
  uint8_t* k_pages;        // [num_pages, Hkv, P, D] E4M3 codes
  uint8_t* v_pages;
  _Float16* k_scales;      // [num_pages, Hkv, P, D/64]
  _Float16* v_scales;
  int32_t* flags;
  int32_t batch, max_rows, num_kv_heads, head_dim, page_size, num_pages;
};

void launch_prepare_block(const PrepareArgs& a, hipStream_t s);
void launch_append_kv(const AppendArgs& a, hipStream_t s);
void launch_append_kv_fp8(const AppendFp8Args& a, hipStream_t s);

}  // namespace sv
