// Shared device/host definitions of the HIP path (internal header).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kHeadDim = 256;
constexpr int kWave = 64;
constexpr int kWavesPerGroup = 4;
constexpr int kThreads = kWave * kWavesPerGroup;
constexpr int kStep = 16;        // tokens per wave step (one MFMA M/K block)
constexpr int kMaxQLen = 512;    // rows per request: a verify block, or an extend chunk after a prefix
constexpr int kMaxRows = 8192;   // q_len * (Hq/Hkv) per KV head
constexpr int kRowStride = kHeadDim + 4;  // fp32 LDS row stride of the combine buffer

// Arguments of the verify-attention kernel (passed by value).
struct AttnArgs {
  const _Float16* q;
  const void* k_pages;
  const void* v_pages;
  const _Float16* k_scales;
  const _Float16* v_scales;
  const int32_t* page_table;
  const int32_t* kv_lens;
  const int32_t* q_start;  // NULL: every request has q_len rows; else packed row offsets [batch+1]
  _Float16* out;
  float* out_lse;
  float* part_o;    // [S, B*q_len, Hq, D] (q_len: the largest width)
  float* part_lse;  // [S, B*q_len, Hq]
  int32_t* flags;
  int32_t batch, q_len, num_q_heads, num_kv_heads, group, page_size;
  int32_t num_pages, max_pages, max_kv_len, chunk, num_splits;
  int32_t row_blocks;  // workgroups per (chunk, KV head, request), each of up to 48 rows
  int32_t units;       // num_splits * num_kv_heads * batch, numbered split-major
  int32_t window, sink;  // sliding window (0: full attention) and leading sink positions
  float scale_log2;  // sm_scale * log2(e)
  int32_t* counters;  // claimed work: the grain counters of every (request, KV head) group
  int32_t balanced;   // XCD-balanced static chunks (see xcd_chunk_start)
};

struct MergeArgs {
  const float* part_o;
  const float* part_lse;
  _Float16* out;
  float* out_lse;
  const int32_t* kv_lens;  // optional: per-request number of chunks
  const int32_t* q_start;  // optional (with kv_lens): packed row offsets [batch+1]
  int32_t num_splits, num_rows, num_heads, head_dim;
  int32_t q_len, chunk, max_kv_len, max_pages, page_size, batch;
  int32_t window, sink;  // as in AttnArgs (the chunks tile the block's live key steps)
  // claimed work: the grain counters to check and clear (NULL otherwise),
  // and the flag word for a counter that did not start at zero
  int32_t* counters;
  int32_t num_kv_heads;
  int32_t* flags;
  int32_t balanced;  // every split slot holds a partial (XCD-balanced static chunks)
};

// Cache policy of one-pass streams (the K/V of a verify pass read by one
// workgroup each, the logit scans). A pass of at least kStreamOnceBytes reads
// non-temporally (the nt bit): on MI355X such a stream reads measurably faster
// that way (a page gather in the verify kernel's order: 6.95 against 6.16
// TB/s). A smaller pass keeps the default policy, under which the 256 MB
// Infinity Cache can keep its bytes for the next reader (read again and again,
// a 17 MB verify pass and an 8 MB logit scan are a few percent slower with
// the nt bit).
constexpr long long kStreamOnceBytes = 32LL << 20;

// a 16-byte load, non-temporal when NT
template <bool NT>
__device__ __forceinline__ float4 load4(const float* p) {
  if constexpr (NT) {
    const floatx4 v = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
  } else {
    return *reinterpret_cast<const float4*>(p);
  }
}

// Length of request b as the kernels use it: the stored value clamped to the
// host bound and to what the page table can address. Shared by the attention
// and merge kernels so both see the same number of chunks.
__device__ inline int clamp_kv_len(int raw, int max_kv_len, int max_pages, int page_size, int* flag_bits) {
  int bound = max_kv_len;
  long long addressable = (long long)max_pages * page_size;
  if (addressable < bound) bound = (int)addressable;
  int v = raw;
  if (v > bound) { v = bound; *flag_bits |= 0x1; }
  if (v < 0) v = 0;
  return v;
}

// Rows of request b in a block packed request by request (row offsets
// q_start[0..batch]): returns the width q_start[b+1] - q_start[b] and sets
// *start. A width outside 0..max_width or rows outside 0..batch*max_width
// mark the request (bit 0x8) and give it width 0, so no access leaves
// buffers sized for batch*max_width rows.
__device__ inline int block_rows(const int32_t* q_start, int b, int batch, int max_width, int* start,
                                 int* flag_bits) {
  const int s = q_start[b], e = q_start[b + 1];
  if (s < 0 || e < s || e - s > max_width || (long long)e > (long long)batch * max_width) {
    *flag_bits |= 0x8;
    *start = 0;
    return 0;
  }
  *start = s;
  return e - s;
}

// The 16-token key steps a verify block whose first row is at position L
// reads from a cache of kv positions. Without a window (window 0): every step
// from position 0. With a sliding window of `window` positions and `sink`
// leading positions: the block sees [0, sink) and [L + 1 - window, kv), so
// the steps are *n_sink from position 0 (the sink part the window does not
// cover), then steps from *a2 (the window part, from a 16-aligned position).
// Key chunks tile these steps (chunk s = steps [s*cs, (s+1)*cs)); the
// attention and merge kernels both count them here.
__device__ inline int live_steps(int kv, int L, int window, int sink, int* n_sink, int* a2) {
  *n_sink = 0;
  *a2 = 0;
  if (kv <= 0) return 0;
  if (window == 0) return (kv + 15) / 16;
  const int wlo = L + 1 - window > 0 ? L + 1 - window : 0;
  const int s_end = sink < wlo ? sink : wlo;
  const int ns = (s_end + 15) / 16;
  int w0 = (wlo / 16) * 16;
  if (w0 < 16 * ns) w0 = 16 * ns;
  *n_sink = ns;
  *a2 = w0;
  return ns + (kv > w0 ? (kv - w0 + 15) / 16 : 0);
}

// Claimed work for a (request, KV head) group whose keys are split over S
// workgroups (4 waves each): wave w of workgroup s first takes the static
// segment of steps [(4s + w) * f, (4s + w + 1) * f), f up to 64 (about three
// quarters of the steps over all waves, 0 for short caches); the steps from
// pool0 = 4 * S * f on form grains of kGrain steps that the group's waves
// claim one at a time from its counters (below). Every wave stops after its
// first ticket past its counter's last grain, so each counter ends at its
// grain count plus its wave count: the merge checks that and clears it.
constexpr int kGrain = 4;
// Each (request, KV head) group's grains are dealt over C counters (grain
// c + k * C is ticket k of counter c), so that no one address takes every
// claim of the group. C is the largest power of two up to kClaimCounters that
// divides S / 2 and leaves room for every group's counters; wave w of
// workgroup slot s claims from counter (w + 4 * (s / 8)) mod C. Slots s and
// s + 1 .. s + 7 sit on the 8 different XCDs, so every counter's waves are
// spread over all XCDs, S / 2 / C * 8 of them per counter. Counter c of group
// q sits in slot q * C + c.
constexpr int kClaimCounters = 16;
constexpr int kCounterSlots = 128;
__host__ __device__ inline int claim_counters(int splits, int groups) {
  int c = kClaimCounters;
  while (c > 1 && ((splits / 2) % c != 0 || c * groups > kCounterSlots)) c /= 2;
  return c;
}
// each counter on its own 256-byte line (int32 stride), in a block of 32 KB
constexpr int kCounterStride = 64;
// the number of grains counter c of C deals
__device__ inline int counter_grains(int n_grains, int c, int C) {
  return n_grains > c ? (n_grains - c + C - 1) / C : 0;
}
__device__ inline void claim_layout(int total, int splits, int* f, int* pool0, int* n_grains) {
  const int waves = splits * kWavesPerGroup;
  int ff = (int)((3LL * total) / (4LL * waves));
  if (ff > 64) ff = 64;
  if (ff < 4) ff = 0;
  *f = ff;
  *pool0 = waves * ff;
  *n_grains = total > *pool0 ? (total - *pool0 + kGrain - 1) / kGrain : 0;
}

// XCD-balanced static chunks for one long request. The S workgroups of each
// (request, KV head) group are spread over the 8 XCDs (slot s of the group
// runs on XCD s mod 8, as workgroup ids go round-robin over the XCDs), and
// since odd XCDs stream their keys measurably slower than even ones, a slot
// on an even XCD gets a longer chunk: slot weights 1 + w and 1 - w (w =
// kXcdWeight / 1000), so slot s starts at step
//     floor(total * (1000 s + kXcdWeight (s mod 2)) / (1000 S))   (S even).
// The boundaries are integers fixed by the length alone: the result is the
// same to the bit on every call.
constexpr int kXcdWeight = 70;  // best of 0..130 in an interleaved sweep at 512K
__host__ __device__ inline int xcd_chunk_start(int total, int s, int S) {
  return (int)(((long long)total * (1000LL * s + kXcdWeight * (s & 1))) / (1000LL * S));
}

void launch_verify_attention(const AttnArgs& a, int rb, bool fp8, bool claim, bool stream_once, hipStream_t s);
// 49 to 96 rows per KV head, fp16 keys, a large pass (verify_rows.hip): one
// workgroup per (chunk, KV head, request), rb row blocks per half; chunks of
// at most kRowsMaxChunk tokens (the workgroup keeps the chunk's cache rows in
// LDS)
void launch_verify_rows(const AttnArgs& a, int rb, hipStream_t s);
constexpr int kRowsMaxChunk = 32768;
void launch_merge(const MergeArgs& a, hipStream_t s);

}  // namespace sv
