// Host side of the C ABI declared in include/sv.h: argument validation, the
// split planner, workspace layout and kernel launches. No allocation, no
// host synchronisation, no device reads: every call is safe to record in a
// HIP graph.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "sv.h"
#include "sv_accept.h"
#include "sv_block.h"
#include "sv_common.h"
#include "sv_sampling.h"
#include "sv_topk.h"

namespace {

thread_local char g_err[512] = "";

sv_status fail(sv_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

sv_status ok() {
  g_err[0] = 0;
  return SV_OK;
}

sv_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(SV_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

// Compute units of the current device, cached per device.
int cu_count() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lk(mu);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct Plan {
  int rb, row_blocks;  // row blocks of 16 per workgroup; workgroups per (chunk, KV head, request)
  int splits, chunk;   // key chunks and their length in tokens
  bool claim;          // the keys of each (request, KV head) are claimed in grains (splits = slots per group)
  bool balanced;       // XCD-balanced static chunks (splits = slots per group, a multiple of 8)
  bool stream_once;    // one row tile and a large pass: the K/V copies go non-temporal
  int halves;          // 2 or 3: the two-half kernel (verify_rows.hip) with that many row blocks per half
  size_t part_o_bytes, part_lse_bytes, ws_bytes;
};

// The first 32 KB of a split workspace hold the claimed-work counters (up to
// 128 counters, each on its own 256-byte line; up to 16 per (request, KV
// head) group); the partials follow.
constexpr size_t kCounterBytes = sv::kCounterSlots * sv::kCounterStride * 4;

constexpr int kMinChunk = 128;         // tokens; below this the partial traffic dominates
// largest automatic chunk for a batch of requests: 16 MiB of K/V per
// (request, KV head), i.e. 16,384 fp16 tokens or 32,768 FP8 tokens (528 B per
// token, taken as half of fp16's 1,024). Smaller chunks balance ragged
// lengths better but pay each workgroup's fixed cost more often: on the
// 32-request 8K-131K batch 8K-token chunks took 1,682 us at q=16 and 1,448 us
// at q=8, 16K-token ones 1,638 and 1,437 us.
constexpr int kBatchChunkCap = 16384;
// the same for the two-half kernel, which holds 96 rows per workgroup: 8K
// tokens (on the 32-request batch at q=16, 6K / 8K / 12K / 16K-token chunks
// took 1,452 / 1,446 / 1,528 / 1,520 us)
constexpr int kRowsBatchChunkCap = 8192;
// shortest automatic chunk for the two-half kernel: its pipeline takes five
// edge rounds per chunk, and below this the row tiles are faster (one
// request at q = 16 over 8K / 20K / 65K / 131K positions: 39.4 / 46.6 / 72.4
// / 124 us with chunks of 192 / 320 / 1,024 / 2,048 tokens, against 33.3 /
// 40.0 / 65.7 / 128.9 us with the row tiles; four requests of 16.5K with
// 1,088-token chunks: 76.2 against 67.5 us)
constexpr int kRowsMinChunk = 2048;
constexpr int kGroupsPerCU = 1;        // workgroups per CU the automatic plan aims at (LDS and registers allow one)

sv_status validate(const sv_verify_params* p) {
  if (!p) return fail(SV_ERR_INVALID_ARGUMENT, "params is NULL");
  if (p->batch < 1) return fail(SV_ERR_INVALID_ARGUMENT, "batch must be >= 1 (got %d)", p->batch);
  if (p->q_len < 1 || p->q_len > sv::kMaxQLen)
    return fail(SV_ERR_UNSUPPORTED, "q_len must be in 1..%d (got %d)", sv::kMaxQLen, p->q_len);
  if (p->num_kv_heads < 1 || p->num_q_heads < 1 || p->num_q_heads % p->num_kv_heads != 0)
    return fail(SV_ERR_INVALID_ARGUMENT, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                p->num_q_heads, p->num_kv_heads);
  const int G = p->num_q_heads / p->num_kv_heads;
  if (p->q_len * G > sv::kMaxRows)
    return fail(SV_ERR_UNSUPPORTED, "q_len * (num_q_heads/num_kv_heads) = %d exceeds %d rows per KV head",
                p->q_len * G, sv::kMaxRows);
  if (p->head_dim != sv::kHeadDim)
    return fail(SV_ERR_UNSUPPORTED, "head_dim must be %d (got %d)", sv::kHeadDim, p->head_dim);
  if (p->page_size < 16 || p->page_size % 16 != 0 || p->page_size > 4096)
    return fail(SV_ERR_UNSUPPORTED, "page_size must be a multiple of 16 in 16..4096 (got %d)", p->page_size);
  if (p->num_pages < 1) return fail(SV_ERR_INVALID_ARGUMENT, "num_pages must be >= 1");
  if ((long long)p->num_pages * p->num_kv_heads * p->page_size > 0xffffffffLL)
    return fail(SV_ERR_UNSUPPORTED, "num_pages * num_kv_heads * page_size must be below 2^32 (cache rows)");
  if (p->max_pages_per_req < 1) return fail(SV_ERR_INVALID_ARGUMENT, "max_pages_per_req must be >= 1");
  if (p->max_kv_len < p->q_len)
    return fail(SV_ERR_INVALID_ARGUMENT, "max_kv_len (%d) must be >= q_len (%d)", p->max_kv_len, p->q_len);
  if ((long long)p->max_kv_len > (long long)p->max_pages_per_req * p->page_size)
    return fail(SV_ERR_INVALID_ARGUMENT, "max_kv_len (%d) exceeds max_pages_per_req * page_size (%lld)",
                p->max_kv_len, (long long)p->max_pages_per_req * p->page_size);
  if (p->kv_dtype != SV_KV_FP16 && p->kv_dtype != SV_KV_FP8_E4M3)
    return fail(SV_ERR_UNSUPPORTED, "unknown kv_dtype %d", (int)p->kv_dtype);
  if (!(p->sm_scale > 0.f) || p->sm_scale > 1e6f)
    return fail(SV_ERR_INVALID_ARGUMENT, "sm_scale must be positive and finite");
  if (p->num_splits < 0) return fail(SV_ERR_INVALID_ARGUMENT, "num_splits must be >= 0");
  if (p->window < 0 || p->sink < 0) return fail(SV_ERR_INVALID_ARGUMENT, "window and sink must be >= 0");
  if (p->window == 0 && p->sink != 0)
    return fail(SV_ERR_INVALID_ARGUMENT, "sink positions need a window (window 0 is full attention)");
  if (p->batch > 65535 || p->num_kv_heads > 65535)
    return fail(SV_ERR_UNSUPPORTED, "batch and num_kv_heads must be <= 65535");
  if (p->options & ~SV_VERIFY_CLAIMED_WORK)
    return fail(SV_ERR_INVALID_ARGUMENT, "unknown options bits 0x%x", (unsigned)p->options);
  return ok();
}

sv_status make_plan(const sv_verify_params* p, Plan* pl) {
  sv_status st = validate(p);
  if (st != SV_OK) return st;
  const int G = p->num_q_heads / p->num_kv_heads;
  const int R = p->q_len * G;
  const int rbt = (R + 15) / 16;
  // more than 48 rows: several workgroups of up to 48 rows (3 row blocks of
  // 16) read the same keys, the rows dealt out evenly
  pl->row_blocks = (rbt + 2) / 3;
  pl->rb = (rbt + pl->row_blocks - 1) / pl->row_blocks;
  // positions the chunks tile: the whole context, or with a sliding window
  // at most the sink, the window and the block (plus 16-token alignment)
  long long maxkv = p->max_kv_len;
  if (p->window > 0) {
    const long long live = (long long)p->sink + p->window + p->q_len + 48;
    const long long whole = (maxkv + 15) / 16 * 16;
    maxkv = live < whole ? live : whole;
  }
  // K/V bytes of the pass if every request were max_kv_len long (or its
  // window): K and V rows of D channels, plus FP8's scale per 64 channels
  const long long row_bytes = p->kv_dtype == SV_KV_FP8_E4M3 ? 2LL * (sv::kHeadDim + sv::kHeadDim / 64 * 2)
                                                            : 2LL * sv::kHeadDim * 2;
  const bool large = (long long)p->batch * p->num_kv_heads * maxkv * row_bytes >= sv::kStreamOnceBytes;
  // 49 to 96 rows with fp16 keys over a large pass: one workgroup of two row
  // halves reads each key once (verify_rows.hip) instead of two row tiles
  // sharing it through L2; short passes keep the row tiles (a few rounds per
  // chunk do not fill the two-half kernel's pipeline)
  pl->halves = 0;
  if (p->kv_dtype == SV_KV_FP16 && R > 48 && R <= 96 && large) {
    pl->halves = R <= 64 ? 2 : 3;
    pl->row_blocks = 1;
    pl->rb = pl->halves;
  }
  // split count and chunk length for the kernel chosen so far
  auto size_splits = [&](long long* S_out, long long* chunk_out) {
    const long long rgs = pl->row_blocks;  // workgroups per (chunk, KV head, request)
    long long S;
    if (p->num_splits > 0) {
      S = p->num_splits;
    } else {
      // Enough chunks for one workgroup per CU when every request is as long
      // as max_kv_len; for batches (whose lengths may be ragged) also cap the
      // chunk so that the work is cut into pieces small enough to balance.
      const long long groups = (long long)p->batch * p->num_kv_heads * rgs;
      const long long target = (long long)kGroupsPerCU * cu_count();
      S = (target + groups - 1) / groups;
      long long chunk = (maxkv + S - 1) / S;
      const long long cap = pl->halves ? kRowsBatchChunkCap
                            : p->kv_dtype == SV_KV_FP8_E4M3 ? 2LL * kBatchChunkCap : kBatchChunkCap;
      if (p->batch > 1 && chunk > cap) {
        // a whole multiple of the fill count keeps full rounds of workgroups
        S *= chunk / cap;
        chunk = (maxkv + S - 1) / S;
      }
      if (chunk < kMinChunk) chunk = kMinChunk;
      S = (maxkv + chunk - 1) / chunk;
      if (S < 1) S = 1;
      if (rgs > 1) {
        // the row tiles of a unit all run on the unit's XCD (unit mod 8), so a
        // unit count that is a multiple of 8 spreads the work over every XCD
        const long long hb = (long long)p->batch * p->num_kv_heads;
        long long need = 8;
        while (need > 1 && hb % (8 / need * 2) == 0) need /= 2;  // 8 / gcd(8, hb)
        const long long S8 = (S + need - 1) / need * need;
        if (maxkv >= S8 * kMinChunk) S = S8;
      }
    }
    long long chunk = (maxkv + S - 1) / S;
    chunk = (chunk + 63) / 64 * 64;
    if (chunk < 64) chunk = 64;
    *S_out = S;
    *chunk_out = chunk;
  };
  auto use_row_tiles = [&]() {
    pl->halves = 0;
    pl->row_blocks = (rbt + 2) / 3;
    pl->rb = (rbt + pl->row_blocks - 1) / pl->row_blocks;
  };
  long long S, chunk;
  size_splits(&S, &chunk);
  if (pl->halves && p->num_splits > 0 && chunk > sv::kRowsMaxChunk) {
    // a forced split count with longer chunks than the two-half kernel
    // holds: the row tiles instead
    use_row_tiles();
    size_splits(&S, &chunk);
  } else if (pl->halves && p->num_splits == 0) {
    if (chunk > sv::kRowsMaxChunk) {
      chunk = sv::kRowsMaxChunk;
    } else if (chunk < kRowsMinChunk) {
      // too short for the two-half kernel's pipeline
      use_row_tiles();
      size_splits(&S, &chunk);
    }
  }
  S = (maxkv + chunk - 1) / chunk;
  if (S * p->num_kv_heads * p->batch * 2 * pl->row_blocks > 0x7fffffffLL)
    return fail(SV_ERR_UNSUPPORTED, "too many workgroups (%lld splits)", S);
  // On request only (the rounding then varies between calls): one long
  // request with fp16 keys, full attention and one row tile, whose
  // workgroups of each KV head (S a multiple of 8, so every head has
  // workgroups on all 8 XCDs) claim its keys in grains, which evens out XCDs
  // that stream at different rates. Only where every wave has about 64 steps
  // or more. Batches keep the static order: their lengths may be ragged
  // (only the device knows), and there the longest-first order of fixed
  // chunks beats an equal number of workgroups per request.
  pl->claim = false;
  if ((p->options & SV_VERIFY_CLAIMED_WORK) && p->batch == 1 && p->window == 0 && p->kv_dtype == SV_KV_FP16 &&
      pl->row_blocks == 1 && pl->halves == 0 && p->num_kv_heads <= sv::kCounterSlots) {
    const long long S8 = p->num_splits > 0 ? S : (S + 7) / 8 * 8;
    if (S8 >= 8 && S8 % 8 == 0 && (maxkv + 15) / 16 >= 64LL * sv::kWavesPerGroup * S8) {
      S = S8;
      pl->claim = true;
    }
  }
  // The default for long caches with fp16 keys, full attention and one row
  // tile, when every request's S workgroups per KV head fit on the GPU in one
  // round (one long request, or a batch of at most 256 / (Hkv * S)): static
  // chunks spread over the 8 XCDs, the ones on even XCDs longer
  // (xcd_chunk_start), which recovers what claiming does without giving up
  // reproducible bits. Each request's chunks follow its own length, so a
  // ragged batch of this size still ends with its longest request's slots.
  pl->balanced = false;
  if (!pl->claim && p->window == 0 && pl->row_blocks == 1 && pl->halves == 0 && p->kv_dtype == SV_KV_FP16) {
    const long long S8 = p->num_splits > 0 ? S : (S + 7) / 8 * 8;
    if (S8 >= 8 && S8 % 8 == 0 && (maxkv + 15) / 16 >= 64LL * sv::kWavesPerGroup * S8 &&
        (long long)p->batch * p->num_kv_heads * S8 <= cu_count()) {
      S = S8;
      pl->balanced = true;
    }
  }
  pl->splits = (int)S;
  pl->chunk = (int)chunk;
  pl->stream_once = pl->row_blocks == 1 && large;
  if (S > 1) {
    const size_t rows = (size_t)p->batch * p->q_len * p->num_q_heads;
    pl->part_o_bytes = align256((size_t)S * rows * sv::kHeadDim * sizeof(float));
    pl->part_lse_bytes = align256((size_t)S * rows * sizeof(float));
    pl->ws_bytes = kCounterBytes + pl->part_o_bytes + pl->part_lse_bytes;
  } else {
    pl->part_o_bytes = pl->part_lse_bytes = 0;
    pl->ws_bytes = 0;
  }
  return ok();
}

}  // namespace

extern "C" {

size_t sv_verify_workspace_bytes(const sv_verify_params* p) {
  Plan pl;
  if (make_plan(p, &pl) != SV_OK) return 0;
  return pl.ws_bytes;
}

sv_status sv_verify_plan(const sv_verify_params* p, int32_t* num_splits, int32_t* chunk_tokens) {
  Plan pl;
  sv_status st = make_plan(p, &pl);
  if (st != SV_OK) return st;
  if (num_splits) *num_splits = pl.splits;
  if (chunk_tokens) *chunk_tokens = pl.chunk;
  return ok();
}

sv_status sv_verify_plan_kernel(const sv_verify_params* p, int32_t* kernel) {
  if (!kernel) return fail(SV_ERR_INVALID_ARGUMENT, "kernel is NULL");
  Plan pl;
  sv_status st = make_plan(p, &pl);
  if (st != SV_OK) return st;
  *kernel = pl.halves ? SV_KERNEL_TWO_HALVES : SV_KERNEL_ROW_TILES;
  return ok();
}

}  // extern "C"

namespace {

sv_status verify_attention_impl(const sv_verify_params* p, const int32_t* q_start, const void* q,
                                const void* k_pages, const void* v_pages, const void* k_scales,
                                const void* v_scales, const int32_t* page_table, const int32_t* kv_lens,
                                void* out, float* out_lse, void* workspace, size_t workspace_bytes,
                                int32_t* status_flags, void* stream) {
  Plan pl;
  sv_status st = make_plan(p, &pl);
  if (st != SV_OK) return st;
  if (!q || !k_pages || !v_pages || !page_table || !kv_lens || !out)
    return fail(SV_ERR_INVALID_ARGUMENT, "q, k_pages, v_pages, page_table, kv_lens and out must be non-NULL");
  if (p->kv_dtype == SV_KV_FP8_E4M3) {
    if (!k_scales || !v_scales)
      return fail(SV_ERR_INVALID_ARGUMENT, "FP8 KV needs k_scales and v_scales");
  } else if (k_scales || v_scales) {
    return fail(SV_ERR_INVALID_ARGUMENT, "k_scales/v_scales must be NULL for fp16 KV");
  }
  if (pl.ws_bytes > 0) {
    if (!workspace || workspace_bytes < pl.ws_bytes)
      return fail(SV_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes (got %zu)", pl.ws_bytes,
                  workspace ? workspace_bytes : (size_t)0);
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
      return fail(SV_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  sv::AttnArgs a;
  a.q = static_cast<const _Float16*>(q);
  a.k_pages = k_pages;
  a.v_pages = v_pages;
  a.k_scales = static_cast<const _Float16*>(k_scales);
  a.v_scales = static_cast<const _Float16*>(v_scales);
  a.page_table = page_table;
  a.kv_lens = kv_lens;
  a.q_start = q_start;
  a.out = static_cast<_Float16*>(out);
  a.out_lse = out_lse;
  char* const ws = static_cast<char*>(workspace);
  a.part_o = pl.ws_bytes ? reinterpret_cast<float*>(ws + kCounterBytes) : nullptr;
  a.part_lse = pl.ws_bytes ? reinterpret_cast<float*>(ws + kCounterBytes + pl.part_o_bytes) : nullptr;
  const bool claim = pl.claim && !q_start;
  // a dirty counter block is reported only through the flag word
  if (claim && !status_flags)
    return fail(SV_ERR_INVALID_ARGUMENT, "SV_VERIFY_CLAIMED_WORK needs a status_flags word");
  a.counters = claim ? reinterpret_cast<int32_t*>(ws) : nullptr;
  a.flags = status_flags;
  a.batch = p->batch;
  a.q_len = p->q_len;
  a.num_q_heads = p->num_q_heads;
  a.num_kv_heads = p->num_kv_heads;
  a.group = p->num_q_heads / p->num_kv_heads;
  a.page_size = p->page_size;
  a.num_pages = p->num_pages;
  a.max_pages = p->max_pages_per_req;
  a.max_kv_len = p->max_kv_len;
  a.chunk = pl.chunk;
  a.num_splits = pl.splits;
  a.scale_log2 = p->sm_scale * 1.44269504088896340736f;
  a.row_blocks = pl.row_blocks;
  a.units = pl.splits * p->num_kv_heads * p->batch;
  a.window = p->window;
  a.sink = p->sink;
  a.balanced = (pl.balanced && !q_start) ? 1 : 0;
  if (pl.halves) {
    // (the plan keeps these by construction; the kernel's tables rely on them)
    if (pl.chunk > sv::kRowsMaxChunk || pl.chunk % 64 != 0 || p->q_len * a.group > 32 * pl.halves)
      return fail(SV_ERR_UNSUPPORTED, "internal plan error: two-half kernel with chunk %d, %d rows", pl.chunk,
                  p->q_len * a.group);
    sv::launch_verify_rows(a, pl.halves, s);
  } else
    sv::launch_verify_attention(a, pl.rb, p->kv_dtype == SV_KV_FP8_E4M3, claim, pl.stream_once, s);
  st = check_launch("verify_attn");
  if (st != SV_OK) return st;
  if (pl.splits > 1) {
    sv::MergeArgs m;
    m.part_o = a.part_o;
    m.part_lse = a.part_lse;
    m.out = a.out;
    m.out_lse = out_lse;
    m.kv_lens = kv_lens;
    m.q_start = q_start;
    m.batch = p->batch;
    m.window = p->window;
    m.sink = p->sink;
    m.num_splits = pl.splits;
    m.num_rows = p->batch * p->q_len;
    m.num_heads = p->num_q_heads;
    m.head_dim = sv::kHeadDim;
    m.q_len = p->q_len;
    m.chunk = pl.chunk;
    m.max_kv_len = p->max_kv_len;
    m.max_pages = p->max_pages_per_req;
    m.page_size = p->page_size;
    m.counters = a.counters;
    m.num_kv_heads = p->num_kv_heads;
    m.flags = status_flags;
    m.balanced = a.balanced;
    sv::launch_merge(m, s);
    st = check_launch("verify_merge");
    if (st != SV_OK) return st;
  }
  return ok();
}

// Scratch of the allocation-free entry point: the workspace of one verify
// call, in the library's own device memory (zero at load, which the
// claimed-work counters at its start need; every call leaves them zero).
// Each device that runs the library holds one copy until the process ends.
// In host code `scratch` names a host-side stand-in, never the device
// memory: its device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// The device address of `scratch` on the current device, looked up on the
// first call there (with that device current) and kept per device.
sv_status scratch_address(void** ptr) {
  static std::mutex mu;
  static void* cache[64] = {nullptr};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SV_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(SV_ERR_UNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(mu);
  if (!cache[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(SV_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    cache[dev] = p;
  }
  *ptr = cache[dev];
  return SV_OK;
}

}  // namespace

extern "C" {

size_t sv_verify_scratch_bytes(void) { return kScratchBytes; }

sv_status sv_verify_attention_noalloc(const sv_verify_params* p, const void* q, const void* k_pages,
                                      const void* v_pages, const void* k_scales, const void* v_scales,
                                      const int32_t* page_table, const int32_t* kv_lens, void* out,
                                      float* out_lse, int32_t* status_flags, void* stream) {
  Plan pl;
  sv_status st = make_plan(p, &pl);
  if (st != SV_OK) return st;
  if (pl.ws_bytes > kScratchBytes)
    return fail(SV_ERR_WORKSPACE_TOO_SMALL,
                "this plan needs %zu bytes of workspace; the library's scratch holds %zu "
                "(use sv_verify_attention with a workspace)",
                pl.ws_bytes, kScratchBytes);
  void* ws = nullptr;
  if (pl.ws_bytes > 0) {
    st = scratch_address(&ws);
    if (st != SV_OK) return st;
  }
  return verify_attention_impl(p, nullptr, q, k_pages, v_pages, k_scales, v_scales, page_table, kv_lens, out,
                               out_lse, ws, pl.ws_bytes, status_flags, stream);
}

sv_status sv_verify_attention(const sv_verify_params* p, const void* q, const void* k_pages,
                              const void* v_pages, const void* k_scales, const void* v_scales,
                              const int32_t* page_table, const int32_t* kv_lens, void* out,
                              float* out_lse, void* workspace, size_t workspace_bytes,
                              int32_t* status_flags, void* stream) {
  return verify_attention_impl(p, nullptr, q, k_pages, v_pages, k_scales, v_scales, page_table, kv_lens, out,
                               out_lse, workspace, workspace_bytes, status_flags, stream);
}

sv_status sv_verify_attention_ragged(const sv_verify_params* p, const int32_t* q_start, const void* q,
                                     const void* k_pages, const void* v_pages, const void* k_scales,
                                     const void* v_scales, const int32_t* page_table, const int32_t* kv_lens,
                                     void* out, float* out_lse, void* workspace, size_t workspace_bytes,
                                     int32_t* status_flags, void* stream) {
  if (!q_start) return fail(SV_ERR_INVALID_ARGUMENT, "q_start must be non-NULL");
  return verify_attention_impl(p, q_start, q, k_pages, v_pages, k_scales, v_scales, page_table, kv_lens, out,
                               out_lse, workspace, workspace_bytes, status_flags, stream);
}

sv_status sv_verify_merge(const float* part_o, const float* part_lse, int32_t num_splits,
                          int32_t num_rows, int32_t num_heads, int32_t head_dim, void* out,
                          float* out_lse, void* stream) {
  if (!part_o || !part_lse || !out)
    return fail(SV_ERR_INVALID_ARGUMENT, "part_o, part_lse and out must be non-NULL");
  if (num_splits < 1 || num_rows < 1 || num_heads < 1)
    return fail(SV_ERR_INVALID_ARGUMENT, "num_splits, num_rows and num_heads must be >= 1");
  if (head_dim < 4 || head_dim > 1024 || head_dim % 4 != 0)
    return fail(SV_ERR_UNSUPPORTED, "head_dim must be a multiple of 4 in 4..1024 (got %d)", head_dim);
  if (reinterpret_cast<uintptr_t>(part_o) % 16 || reinterpret_cast<uintptr_t>(out) % 8)
    return fail(SV_ERR_INVALID_ARGUMENT, "part_o must be 16-byte and out 8-byte aligned");
  sv::MergeArgs m;
  m.part_o = part_o;
  m.part_lse = part_lse;
  m.out = static_cast<_Float16*>(out);
  m.out_lse = out_lse;
  m.kv_lens = nullptr;
  m.q_start = nullptr;
  m.counters = nullptr;
  m.num_kv_heads = 0;
  m.flags = nullptr;
  m.balanced = 0;
  m.batch = 0;
  m.window = 0;
  m.sink = 0;
  m.num_splits = num_splits;
  m.num_rows = num_rows;
  m.num_heads = num_heads;
  m.head_dim = head_dim;
  m.q_len = 1;
  m.chunk = 1;
  m.max_kv_len = 0;
  m.max_pages = 0;
  m.page_size = 0;
  sv::launch_merge(m, static_cast<hipStream_t>(stream));
  return check_launch("verify_merge");
}

size_t sv_greedy_accept_workspace_bytes(int32_t batch, int32_t q_len, int32_t vocab) {
  if (batch < 1 || q_len < 1 || vocab < 1) return 0;
  const size_t slices = ((size_t)vocab + sv::kAcceptSlice - 1) / sv::kAcceptSlice;
  return align256((size_t)batch * q_len * slices * sizeof(float2));
}

}  // extern "C"

namespace {

sv_status greedy_accept_impl(const float* logits, const int32_t* draft_ids, const int32_t* block_ids,
                             const int32_t* q_start, int32_t batch, int32_t q_len, int32_t vocab,
                             int32_t* accept_len, int32_t* bonus_ids, int32_t* argmax_ids,
                             const int32_t* kv_lens_in, int32_t* kv_lens_out, void* workspace,
                             size_t workspace_bytes, int32_t* status_flags, void* stream) {
  if (batch < 1 || q_len < 1 || vocab < 1)
    return fail(SV_ERR_INVALID_ARGUMENT, "batch, q_len and vocab must be >= 1");
  if ((long long)batch * q_len > 65535)
    return fail(SV_ERR_UNSUPPORTED, "batch * q_len must be <= 65535");
  if (q_len > sv::kMaxAcceptRows)
    return fail(SV_ERR_UNSUPPORTED, "q_len must be <= %d", sv::kMaxAcceptRows);
  if (!logits || !accept_len || !bonus_ids)
    return fail(SV_ERR_INVALID_ARGUMENT, "logits, accept_len and bonus_ids must be non-NULL");
  if (q_start) {
    if (q_len > 1 && !block_ids) return fail(SV_ERR_INVALID_ARGUMENT, "block_ids is NULL");
  } else if (q_len > 1 && !draft_ids) {
    return fail(SV_ERR_INVALID_ARGUMENT, "draft_ids is NULL");
  }
  if ((kv_lens_in == nullptr) != (kv_lens_out == nullptr))
    return fail(SV_ERR_INVALID_ARGUMENT, "kv_lens_in and kv_lens_out must be both NULL or both set");
  if (vocab % 4 == 0 && reinterpret_cast<uintptr_t>(logits) % 16)
    return fail(SV_ERR_INVALID_ARGUMENT, "logits must be 16-byte aligned");
  const size_t need = sv_greedy_accept_workspace_bytes(batch, q_len, vocab);
  if (!workspace || workspace_bytes < need)
    return fail(SV_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes (got %zu)", need,
                workspace ? workspace_bytes : (size_t)0);
  sv::AcceptLaunch a;
  a.logits = logits;
  a.draft_ids = draft_ids;
  a.block_ids = block_ids;
  a.q_start = q_start;
  a.flags = status_flags;
  a.batch = batch;
  a.q_len = q_len;
  a.vocab = vocab;
  a.slice = sv::kAcceptSlice;
  a.n_slices = (vocab + sv::kAcceptSlice - 1) / sv::kAcceptSlice;
  a.accept_len = accept_len;
  a.bonus_ids = bonus_ids;
  a.argmax_ids = argmax_ids;
  a.kv_lens_in = kv_lens_in;
  a.kv_lens_out = kv_lens_out;
  a.ws = static_cast<float2*>(workspace);
  sv::launch_greedy_accept(a, static_cast<hipStream_t>(stream));
  return check_launch("greedy_accept");
}

}  // namespace

extern "C" {

sv_status sv_greedy_accept(const float* logits, const int32_t* draft_ids, int32_t batch,
                           int32_t q_len, int32_t vocab, int32_t* accept_len, int32_t* bonus_ids,
                           int32_t* argmax_ids, const int32_t* kv_lens_in, int32_t* kv_lens_out,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return greedy_accept_impl(logits, draft_ids, nullptr, nullptr, batch, q_len, vocab, accept_len, bonus_ids,
                            argmax_ids, kv_lens_in, kv_lens_out, workspace, workspace_bytes, nullptr, stream);
}

sv_status sv_greedy_accept_ragged(const float* logits, const int32_t* block_ids, const int32_t* q_start,
                                  int32_t batch, int32_t max_q_len, int32_t vocab, int32_t* accept_len,
                                  int32_t* bonus_ids, int32_t* argmax_ids, const int32_t* kv_lens_in,
                                  int32_t* kv_lens_out, void* workspace, size_t workspace_bytes,
                                  int32_t* status_flags, void* stream) {
  if (!q_start) return fail(SV_ERR_INVALID_ARGUMENT, "q_start must be non-NULL");
  return greedy_accept_impl(logits, nullptr, block_ids, q_start, batch, max_q_len, vocab, accept_len, bonus_ids,
                            argmax_ids, kv_lens_in, kv_lens_out, workspace, workspace_bytes, status_flags,
                            stream);
}

sv_status sv_prepare_block(const int32_t* seq_lens, const int32_t* q_lens, const int32_t* page_table,
                           int32_t batch, int32_t max_q_len, int32_t max_pages_per_req, int32_t page_size,
                           int32_t num_pages, const int32_t* last_tokens, const int32_t* draft_ids,
                           int32_t* q_start, int32_t* positions, int32_t* cache_slot, int32_t* kv_lens_out,
                           int32_t* block_ids, int32_t* status_flags, void* stream) {
  if (batch < 1 || max_q_len < 1)
    return fail(SV_ERR_INVALID_ARGUMENT, "batch and max_q_len must be >= 1");
  if ((long long)batch * max_q_len > 0x7fffffffLL)
    return fail(SV_ERR_UNSUPPORTED, "batch * max_q_len must fit in int32");
  if (page_size < 1 || max_pages_per_req < 1 || num_pages < 1)
    return fail(SV_ERR_INVALID_ARGUMENT, "page_size, max_pages_per_req and num_pages must be >= 1");
  if ((long long)num_pages * page_size > 0x7fffffffLL)
    return fail(SV_ERR_UNSUPPORTED, "num_pages * page_size must fit in int32 (flat cache slots)");
  if (!seq_lens || !q_lens || !page_table || !q_start || !cache_slot)
    return fail(SV_ERR_INVALID_ARGUMENT, "seq_lens, q_lens, page_table, q_start and cache_slot must be non-NULL");
  if ((last_tokens == nullptr) != (block_ids == nullptr))
    return fail(SV_ERR_INVALID_ARGUMENT, "last_tokens and block_ids must be both NULL or both set");
  if (last_tokens && max_q_len > 1 && !draft_ids)
    return fail(SV_ERR_INVALID_ARGUMENT, "draft_ids is NULL");
  sv::PrepareArgs a;
  a.seq_lens = seq_lens;
  a.q_lens = q_lens;
  a.page_table = page_table;
  a.last_tokens = last_tokens;
  a.draft_ids = draft_ids;
  a.q_start = q_start;
  a.positions = positions;
  a.cache_slot = cache_slot;
  a.kv_lens_out = kv_lens_out;
  a.block_ids = block_ids;
  a.flags = status_flags;
  a.batch = batch;
  a.max_width = max_q_len;
  a.max_pages = max_pages_per_req;
  a.page_size = page_size;
  a.num_pages = num_pages;
  sv::launch_prepare_block(a, static_cast<hipStream_t>(stream));
  return check_launch("prepare_block");
}

sv_status sv_append_kv(const void* new_k, const void* new_v, const int32_t* cache_slot, const int32_t* q_start,
                       int32_t batch, int32_t max_rows, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                       int32_t num_pages, sv_kv_dtype kv_dtype, void* k_pages, void* v_pages,
                       int32_t* status_flags, void* stream) {
  if (batch < 1 || max_rows < 1 || num_kv_heads < 1)
    return fail(SV_ERR_INVALID_ARGUMENT, "batch, max_rows and num_kv_heads must be >= 1");
  if (kv_dtype != SV_KV_FP16)
    return fail(SV_ERR_UNSUPPORTED, "sv_append_kv writes fp16 pages only (FP8 pages: sv_append_kv_fp8)");
  if (head_dim < 8 || head_dim % 8 != 0 || head_dim > 4096)
    return fail(SV_ERR_UNSUPPORTED, "head_dim must be a multiple of 8 in 8..4096 (got %d)", head_dim);
  if (page_size < 1 || num_pages < 1)
    return fail(SV_ERR_INVALID_ARGUMENT, "page_size and num_pages must be >= 1");
  if ((long long)num_pages * page_size > 0x7fffffffLL)
    return fail(SV_ERR_UNSUPPORTED, "num_pages * page_size must fit in int32 (flat cache slots)");
  if ((long long)max_rows * num_kv_heads * (head_dim / 8) > 0x7fffffffLL * sv::kThreads)
    return fail(SV_ERR_UNSUPPORTED, "too many rows");
  if (!new_k || !new_v || !cache_slot || !q_start || !k_pages || !v_pages)
    return fail(SV_ERR_INVALID_ARGUMENT, "new_k, new_v, cache_slot, q_start, k_pages and v_pages must be non-NULL");
  const uintptr_t al = reinterpret_cast<uintptr_t>(new_k) | reinterpret_cast<uintptr_t>(new_v) |
                       reinterpret_cast<uintptr_t>(k_pages) | reinterpret_cast<uintptr_t>(v_pages);
  if (al % 16) return fail(SV_ERR_INVALID_ARGUMENT, "new_k, new_v, k_pages and v_pages must be 16-byte aligned");
  sv::AppendArgs a;
  a.new_k = static_cast<const _Float16*>(new_k);
  a.new_v = static_cast<const _Float16*>(new_v);
  a.cache_slot = cache_slot;
  a.q_start = q_start;
  a.k_pages = static_cast<_Float16*>(k_pages);
  a.v_pages = static_cast<_Float16*>(v_pages);
  a.flags = status_flags;
  a.batch = batch;
  a.max_rows = max_rows;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.page_size = page_size;
  a.num_pages = num_pages;
  sv::launch_append_kv(a, static_cast<hipStream_t>(stream));
  return check_launch("append_kv");
}

sv_status sv_append_kv_fp8(const void* new_k, const void* new_v, const int32_t* cache_slot, const int32_t* q_start,
                           int32_t batch, int32_t max_rows, int32_t num_kv_heads, int32_t head_dim,
                           int32_t page_size, int32_t num_pages, void* k_pages, void* v_pages, void* k_scales,
                           void* v_scales, int32_t* status_flags, void* stream) {
  if (batch < 1 || max_rows < 1 || num_kv_heads < 1)
    return fail(SV_ERR_INVALID_ARGUMENT, "batch, max_rows and num_kv_heads must be >= 1");
  if (head_dim < 64 || head_dim % 64 != 0 || head_dim > 4096)
    return fail(SV_ERR_UNSUPPORTED, "head_dim must be a multiple of 64 in 64..4096 (got %d)", head_dim);
  if (page_size < 1 || num_pages < 1)
    return fail(SV_ERR_INVALID_ARGUMENT, "page_size and num_pages must be >= 1");
  if ((long long)num_pages * page_size > 0x7fffffffLL)
    return fail(SV_ERR_UNSUPPORTED, "num_pages * page_size must fit in int32 (flat cache slots)");
  if ((long long)max_rows * num_kv_heads > 0x7fffffffLL)
    return fail(SV_ERR_UNSUPPORTED, "too many rows");
  if (!new_k || !new_v || !cache_slot || !q_start || !k_pages || !v_pages || !k_scales || !v_scales)
    return fail(SV_ERR_INVALID_ARGUMENT,
                "new_k, new_v, cache_slot, q_start, k_pages, v_pages, k_scales and v_scales must be non-NULL");
  if ((reinterpret_cast<uintptr_t>(new_k) | reinterpret_cast<uintptr_t>(new_v)) % 8 ||
      (reinterpret_cast<uintptr_t>(k_pages) | reinterpret_cast<uintptr_t>(v_pages)) % 4 ||
      (reinterpret_cast<uintptr_t>(k_scales) | reinterpret_cast<uintptr_t>(v_scales)) % 2)
    return fail(SV_ERR_INVALID_ARGUMENT, "new_k/new_v must be 8-byte, pages 4-byte and scales 2-byte aligned");
  sv::AppendFp8Args a;
  a.new_k = static_cast<const _Float16*>(new_k);
  a.new_v = static_cast<const _Float16*>(new_v);
  a.cache_slot = cache_slot;
  a.q_start = q_start;
  a.k_pages = static_cast<uint8_t*>(k_pages);
  a.v_pages = static_cast<uint8_t*>(v_pages);
  a.k_scales = static_cast<_Float16*>(k_scales);
  a.v_scales = static_cast<_Float16*>(v_scales);
  a.flags = status_flags;
  a.batch = batch;
  a.max_rows = max_rows;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.page_size = page_size;
  a.num_pages = num_pages;
  sv::launch_append_kv_fp8(a, static_cast<hipStream_t>(stream));
  return check_launch("append_kv_fp8");
}

size_t sv_rejection_accept_workspace_bytes(int32_t batch, int32_t q_len, int32_t vocab) {
  if (batch < 1 || q_len < 1 || vocab < 1) return 0;
  const size_t slices = ((size_t)vocab + sv::kSampleSlice - 1) / sv::kSampleSlice;
  return align256((size_t)batch * q_len * slices * sizeof(float2)) + align256((size_t)batch * slices * sizeof(float)) +
         align256((size_t)batch * sizeof(int32_t));
}

sv_status sv_rejection_accept(const float* logits, const int32_t* draft_ids, const float* draft_probs,
                              int32_t batch, int32_t q_len, int32_t vocab, float temperature, const float* u_accept,
                              const float* u_final, int32_t* accept_len, int32_t* token_ids,
                              const int32_t* kv_lens_in, int32_t* kv_lens_out, void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (batch < 1 || q_len < 1 || vocab < 1)
    return fail(SV_ERR_INVALID_ARGUMENT, "batch, q_len and vocab must be >= 1");
  if (q_len > sv::kMaxSampleRows) return fail(SV_ERR_UNSUPPORTED, "q_len must be <= %d", sv::kMaxSampleRows);
  if ((long long)vocab > 64LL * sv::kSampleSlice)
    return fail(SV_ERR_UNSUPPORTED, "vocab must be <= %d", 64 * sv::kSampleSlice);
  if ((long long)batch * q_len > 65535) return fail(SV_ERR_UNSUPPORTED, "batch * q_len must be <= 65535");
  if (!(temperature > 0.f) || temperature > 1e30f)
    return fail(SV_ERR_INVALID_ARGUMENT, "temperature must be positive and finite");
  if (!logits || !u_final || !accept_len || !token_ids)
    return fail(SV_ERR_INVALID_ARGUMENT, "logits, u_final, accept_len and token_ids must be non-NULL");
  if (q_len > 1 && (!draft_ids || !draft_probs || !u_accept))
    return fail(SV_ERR_INVALID_ARGUMENT, "draft_ids, draft_probs and u_accept must be non-NULL when q_len > 1");
  if ((kv_lens_in == nullptr) != (kv_lens_out == nullptr))
    return fail(SV_ERR_INVALID_ARGUMENT, "kv_lens_in and kv_lens_out must be both NULL or both set");
  if (vocab % 4 == 0 && ((reinterpret_cast<uintptr_t>(logits) | reinterpret_cast<uintptr_t>(draft_probs)) % 16))
    return fail(SV_ERR_INVALID_ARGUMENT, "logits and draft_probs must be 16-byte aligned");
  const size_t need = sv_rejection_accept_workspace_bytes(batch, q_len, vocab);
  if (!workspace || workspace_bytes < need)
    return fail(SV_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes (got %zu)", need,
                workspace ? workspace_bytes : (size_t)0);
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return fail(SV_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  sv::SampleLaunch a;
  a.logits = logits;
  a.draft_ids = draft_ids;
  a.draft_probs = draft_probs;
  a.u_accept = u_accept;
  a.u_final = u_final;
  a.batch = batch;
  a.q_len = q_len;
  a.vocab = vocab;
  a.slice = sv::kSampleSlice;
  a.n_slices = (vocab + sv::kSampleSlice - 1) / sv::kSampleSlice;
  a.c = 1.44269504088896340736f / temperature;
  a.accept_len = accept_len;
  a.token_ids = token_ids;
  a.kv_lens_in = kv_lens_in;
  a.kv_lens_out = kv_lens_out;
  char* w = static_cast<char*>(workspace);
  a.ws1 = reinterpret_cast<float2*>(w);
  w += align256((size_t)batch * q_len * a.n_slices * sizeof(float2));
  a.ws2 = reinterpret_cast<float*>(w);
  w += align256((size_t)batch * a.n_slices * sizeof(float));
  a.ws_acc = reinterpret_cast<int32_t*>(w);
  sv::launch_rejection_accept(a, static_cast<hipStream_t>(stream));
  return check_launch("rejection_accept");
}

size_t sv_topk_candidates_workspace_bytes(int32_t rows, int32_t vocab, int32_t k) {
  if (rows < 1 || vocab < 1 || k < 1) return 0;
  const size_t slices = ((size_t)vocab + sv::kTopkSlice - 1) / sv::kTopkSlice;
  return align256((size_t)rows * slices * k * sizeof(float2));
}

sv_status sv_topk_candidates(const float* logits, int32_t rows, int32_t vocab, int32_t k, int32_t* out_ids,
                             float* out_values, void* workspace, size_t workspace_bytes, void* stream) {
  if (rows < 1 || vocab < 1) return fail(SV_ERR_INVALID_ARGUMENT, "rows and vocab must be >= 1");
  if (k < 1 || k > sv::kMaxTopk) return fail(SV_ERR_UNSUPPORTED, "k must be in 1..%d (got %d)", sv::kMaxTopk, k);
  if (k > vocab) return fail(SV_ERR_INVALID_ARGUMENT, "k (%d) exceeds vocab (%d)", k, vocab);
  if (rows > 65535) return fail(SV_ERR_UNSUPPORTED, "rows must be <= 65535");
  const long long slices = ((long long)vocab + sv::kTopkSlice - 1) / sv::kTopkSlice;
  if (slices * k > (long long)sv::kWave * sv::kMergePerLane)
    return fail(SV_ERR_UNSUPPORTED, "vocab too large for k = %d (at most %d columns)", k,
                sv::kWave * sv::kMergePerLane / k * sv::kTopkSlice);
  if (!logits || !out_ids || !out_values)
    return fail(SV_ERR_INVALID_ARGUMENT, "logits, out_ids and out_values must be non-NULL");
  if (vocab % 4 == 0 && reinterpret_cast<uintptr_t>(logits) % 16)
    return fail(SV_ERR_INVALID_ARGUMENT, "logits must be 16-byte aligned");
  const size_t need = sv_topk_candidates_workspace_bytes(rows, vocab, k);
  if (!workspace || workspace_bytes < need)
    return fail(SV_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes (got %zu)", need,
                workspace ? workspace_bytes : (size_t)0);
  sv::TopkLaunch a;
  a.logits = logits;
  a.rows = rows;
  a.vocab = vocab;
  a.k = k;
  // few rows: wider slices (fewer, fuller workgroups); the workspace is sized
  // for the narrow ones
  a.slice = rows <= 64 ? sv::kTopkSliceWide : sv::kTopkSlice;
  a.n_slices = (int)(((long long)vocab + a.slice - 1) / a.slice);
  a.ws = static_cast<float2*>(workspace);
  a.out_ids = out_ids;
  a.out_vals = out_values;
  sv::launch_topk(a, static_cast<hipStream_t>(stream));
  return check_launch("topk_candidates");
}

const char* sv_status_string(sv_status s) {
  switch (s) {
    case SV_OK: return "SV_OK";
    case SV_ERR_INVALID_ARGUMENT: return "SV_ERR_INVALID_ARGUMENT";
    case SV_ERR_UNSUPPORTED: return "SV_ERR_UNSUPPORTED";
    case SV_ERR_WORKSPACE_TOO_SMALL: return "SV_ERR_WORKSPACE_TOO_SMALL";
    case SV_ERR_HIP: return "SV_ERR_HIP";
  }
  return "SV_ERR_UNKNOWN";
}

const char* sv_last_error(void) { return g_err; }

int32_t sv_version(void) { return 200; }

}  // extern "C"
