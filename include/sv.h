/*
 * sv.h — C ABI of the target-verify path of speculative decoding on MI355X
 * (gfx950): paged causal grouped-query attention of a verify block, the
 * merge of split-KV partials, greedy and stochastic (rejection-sampling)
 * acceptance, top-k candidate selection; blocks of one width or of a width
 * per request, and the preparation and K/V append of a block.
 *
 * Conventions shared by every entry point
 *   - Pointers are DEVICE pointers unless marked "host".
 *   - Every call is asynchronous and ordered on `stream` (0 = the null
 *     stream). No call allocates device memory, synchronises the host, or
 *     reads device memory from the host; each is safe to record in a HIP
 *     graph. The caller owns every buffer and keeps it alive until the
 *     stream has passed the call.
 *   - Host-detectable errors (null pointers, unsupported shapes, a workspace
 *     that is too small) return a status without launching anything; the
 *     detail is in sv_last_error() (thread-local).
 *   - Device-side contract violations (a length larger than the host bound
 *     or smaller than the block, a page id outside the pool) cannot be
 *     reported synchronously: kernels clamp so that no access leaves the
 *     buffers, and OR a bit into *status_flags when that pointer is not
 *     NULL (SV_FLAG_*). The caller zeroes the flag word.
 *   - The library keeps no state between calls apart from the last-error
 *     string and a per-device cache of the compute-unit count.
 */
#ifndef SV_H_
#define SV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SV_OK = 0,
  SV_ERR_INVALID_ARGUMENT = 1,
  SV_ERR_UNSUPPORTED = 2,
  SV_ERR_WORKSPACE_TOO_SMALL = 3,
  SV_ERR_HIP = 4
} sv_status;

typedef enum { SV_KV_FP16 = 0, SV_KV_FP8_E4M3 = 1 } sv_kv_dtype;

/* Bits OR-ed into *status_flags by the kernels. */
#define SV_FLAG_KV_LEN_ABOVE_BOUND 0x1 /* kv_lens[b] > max_kv_len or > max_pages_per_req*page_size; clamped */
#define SV_FLAG_KV_LEN_BELOW_BLOCK 0x2 /* kv_lens[b] < q_len; rows that see no key give 0 output, -inf lse */
#define SV_FLAG_PAGE_ID_OUT_OF_RANGE 0x4 /* page id < 0 or >= num_pages; page 0 read instead
                                           (sv_prepare_block, sv_append_kv: the row's slot is -1 / skipped) */
#define SV_FLAG_BAD_BLOCK_WIDTH 0x8 /* a width outside 0..max, or packed rows outside 0..batch*max;
                                       that request is treated as having no block */
#define SV_FLAG_WORKSPACE_NOT_ZERO 0x10 /* the work counters in the first 32 KB of the verify
                                           workspace were not zero at a call with
                                           SV_VERIFY_CLAIMED_WORK: the result is wrong (they are
                                           zero again afterwards) */

/* Bits of sv_verify_params.options. */
#define SV_VERIFY_CLAIMED_WORK 0x1 /* opt-in run-time balancing of one long request (see
                                      sv_verify_attention); results are then reproducible
                                      to rounding only, and status_flags must be non-NULL */

/*
 * Shape and layout of one verify call (host struct).
 *
 * The verify block: a request with committed prefix L appends q_len known
 * tokens (the current token and q_len-1 drafts) and the target evaluates all
 * rows in one causal pass, row i seeing the prefix and block rows 0..i
 * (worked example "Why the target output stayed the same" on the page "MTP
 * and DFlash2 at long context on XPU"; verify table of section 1.1 on the
 * page "DFlash -> dLLM self-spec, part 1"). The block's own K/V are already
 * in the paged cache and kv_lens counts them: row i of request b attends to
 * cache positions 0 .. kv_lens[b] - q_len + i.
 *
 * The same call serves an extend chunk: up to 512 new tokens processed on
 * top of a cached prefix, a short prefill after it (the glossary at the end
 * of the page "DFlash -> dLLM self-spec, part 1"); its rows attend causally
 * exactly as a verify block's do, so q_len may exceed the block sizes 8 and 16.
 *
 * Sink + sliding window (window > 0; the opt-in sparse mode of the PocketLLM
 * page, "Implemented execution path" and "Validated performance"): row i at
 * position p = kv_lens[b] - q_len + i attends only to the positions t <= p
 * with t < sink or t > p - window (the window includes the row itself); the
 * cache layout is unchanged and chunks the block cannot see are not read.
 * window = 0 (with sink = 0) is full attention.
 */
typedef struct {
  int32_t batch;             /* B >= 1 requests */
  int32_t q_len;             /* rows per request, 1..512 (a verify block, or an extend chunk) */
  int32_t num_q_heads;       /* Hq; query head h uses KV head h / (Hq/Hkv) */
  int32_t num_kv_heads;      /* Hkv, divides Hq; q_len * Hq/Hkv <= 8192 */
  int32_t head_dim;          /* D, must be 256 */
  int32_t page_size;         /* P tokens per page: a multiple of 16, at most 4096 */
  int32_t num_pages;         /* pages in the pool (bounds page ids) */
  int32_t max_pages_per_req; /* row stride of page_table */
  int32_t max_kv_len;        /* host upper bound on every kv_lens[b]; sizes the grid */
  sv_kv_dtype kv_dtype;
  float sm_scale;            /* softmax scale, e.g. 1/sqrt(D) */
  int32_t num_splits;        /* 0 = automatic; > 0 forces the number of key chunks */
  int32_t window;            /* 0 = full attention; > 0: a sliding window of this many positions */
  int32_t sink;              /* with a window: leading positions every row also sees (0 = none) */
  int32_t options;           /* SV_VERIFY_* bits; 0 = the default, bit-reproducible plan */
} sv_verify_params;

/*
 * Bytes of workspace sv_verify_attention needs for these parameters (0 when
 * one key chunk covers max_kv_len). Depends only on the host fields. Its
 * first 32 KB hold the work counters of the SV_VERIFY_CLAIMED_WORK option
 * and must be zero before the workspace's first use with that option, e.g.
 * filled with zeros once when it is allocated: every verify call leaves them
 * zero again, so a workspace serves any number of verify calls (also of other
 * shapes), one at a time, but should not be shared with other entry points'
 * scratch. The default plan never reads them. The partials follow.
 */
size_t sv_verify_workspace_bytes(const sv_verify_params* p);

/*
 * Number of key chunks (splits) the planner uses for these parameters, and
 * the chunk length in tokens. Chunks are anchored at absolute position 0:
 * chunk s covers cache positions [s*chunk, (s+1)*chunk). With a sliding
 * window the chunks instead tile the positions a block can see (its sink
 * positions, then its window, in 16-position steps), so the split count
 * follows sink + window + q_len rather than max_kv_len. One exception: for
 * one long request (batch 1, full attention, q_len*Hq/Hkv <= 48, a split
 * count that is a multiple of 8 and max_kv_len >= 4096 * splits) the chunks
 * of each KV head are spread over the GPU's 8 XCDs and those that run on the
 * faster even XCDs are a few percent longer; their bounds are 16-position
 * steps fixed by the request's length, and `chunk` is then the nominal
 * length. Host only.
 */
sv_status sv_verify_plan(const sv_verify_params* p, int32_t* num_splits, int32_t* chunk_tokens);

/*
 * The attention kernel the planner launches for these parameters (both
 * compute the same attention, equal to rounding; they differ in how a
 * workgroup covers the rows of a KV head):
 *   SV_KERNEL_ROW_TILES   up to 48 rows per workgroup; more rows as row tiles
 *                         (workgroups on the same keys, shared through L2)
 *   SV_KERNEL_TWO_HALVES  49 to 96 rows in one workgroup of two row halves
 *                         that split the output channels; taken for fp16
 *                         keys over a pass of 32 MB or more (batch x KV
 *                         heads x max_kv_len x 1 KB; with a window, its
 *                         span instead of max_kv_len) whose chunks are at
 *                         least 2,048 positions long (any length up to 32,768
 *                         when num_splits is forced)
 * Host only; the status is that of the plan (as for sv_verify_plan), and
 * SV_ERR_INVALID_ARGUMENT for a NULL `kernel`.
 */
typedef enum { SV_KERNEL_ROW_TILES = 0, SV_KERNEL_TWO_HALVES = 1 } sv_verify_kernel;
sv_status sv_verify_plan_kernel(const sv_verify_params* p, int32_t* kernel);

/*
 * Causal GQA of every verify row over the paged cache (the target-verify
 * attention; split-context decode with compact online-softmax partials as on
 * the PocketLLM page "Qwen3.8-27B-FP8", section "Implemented execution
 * path", generalised to a verify block).
 *
 *   q           [batch*q_len, Hq, D] fp16, row r = b*q_len + i
 *   k_pages     [num_pages, Hkv, P, D] fp16, or E4M3 bytes (kv_dtype FP8)
 *   v_pages     same layout and type as k_pages
 *   k_scales    FP8 only: [num_pages, Hkv, P, D/64] fp16 — one scale per
 *               token, KV head and 64-channel block (value = e4m3 * scale);
 *               must be NULL for fp16
 *   v_scales    same as k_scales
 *   page_table  [batch, max_pages_per_req] int32: position t of request b is
 *               slot t % P of page page_table[b*max_pages_per_req + t / P]
 *   kv_lens     [batch] int32, q_len <= kv_lens[b] <= max_kv_len
 *   out         [batch*q_len, Hq, D] fp16 (written)
 *   out_lse     NULL or [batch*q_len, Hq] fp32: natural-log sum of
 *               exp(sm_scale * q.k) over the row's visible keys
 *   workspace   device buffer of sv_verify_workspace_bytes(p) bytes, 256-byte
 *               aligned; its first 32 KB zero (see sv_verify_workspace_bytes)
 *   status_flags NULL or one int32 word (see SV_FLAG_*)
 *
 * Arithmetic: fp16 (or exactly dequantised E4M3) inputs, fp32 accumulation;
 * the result does not depend on the number of splits beyond rounding.
 * Deterministic: every key chunk and the order of its softmax updates are
 * fixed by the host fields and the device lengths, so repeated calls give the
 * same bits, and so do calls whose physical pages are permuted (with the page
 * table permuted alike).
 *
 * One exception, only on request (p->options & SV_VERIFY_CLAIMED_WORK): for
 * one request (batch 1) with fp16 keys, full attention, q_len*Hq/Hkv <= 48, a
 * split count that is a multiple of 8 and max_kv_len >= 4096 * splits (at
 * least 64 key steps of 16 per wave, e.g. 256K tokens at the automatic 64
 * splits), the waves of each KV head claim 64-key grains at run time, which
 * evens out compute units that stream at different rates; the order of the
 * softmax updates, and with it the rounding, then varies between calls.
 * That mode needs status_flags (SV_ERR_INVALID_ARGUMENT otherwise), since a
 * workspace whose counters are not zero is reported only there
 * (SV_FLAG_WORKSPACE_NOT_ZERO). Elsewhere the option is ignored.
 */
sv_status sv_verify_attention(const sv_verify_params* p, const void* q, const void* k_pages,
                              const void* v_pages, const void* k_scales, const void* v_scales,
                              const int32_t* page_table, const int32_t* kv_lens, void* out,
                              float* out_lse, void* workspace, size_t workspace_bytes,
                              int32_t* status_flags, void* stream);

/*
 * sv_verify_attention for callers that cannot allocate device memory or pass
 * a workspace (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): the same operation and the same kernels, with the
 * workspace in the library's own device scratch of sv_verify_scratch_bytes()
 * bytes (32 MiB), which each GPU the library runs on holds until the process
 * ends. No allocation, no host synchronisation.
 *
 * Arguments and results as for sv_verify_attention, minus the workspace.
 * A plan whose workspace exceeds the scratch (sv_verify_workspace_bytes(p) >
 * sv_verify_scratch_bytes(), e.g. very large batches of q_len 16) returns
 * SV_ERR_WORKSPACE_TOO_SMALL without launching. Every call on a GPU shares
 * that GPU's scratch: calls that may overlap on one GPU (other streams,
 * other threads) race and must be serialised by the caller. The first call
 * on a device looks the scratch's device address up (hipGetSymbolAddress)
 * with that device current; SV_ERR_HIP if that fails.
 */
size_t sv_verify_scratch_bytes(void);
sv_status sv_verify_attention_noalloc(const sv_verify_params* p, const void* q, const void* k_pages,
                                      const void* v_pages, const void* k_scales, const void* v_scales,
                                      const int32_t* page_table, const int32_t* kv_lens, void* out,
                                      float* out_lse, int32_t* status_flags, void* stream);

/*
 * Merge of split-KV partials into the final attention output (the merge
 * step of compact online-softmax partials, PocketLLM page, "Implemented
 * execution path"): for every (row, head)
 *     LSE = ln sum_s exp(part_lse[s]),  out = sum_s exp(part_lse[s] - LSE) * part_o[s]
 * over the partials whose lse is not -inf (an empty split). A row whose
 * partials are all empty gets out = 0 and lse = -inf.
 *
 *   part_o    [num_splits, num_rows, num_heads, head_dim] fp32, each partial
 *             normalised over its own key range
 *   part_lse  [num_splits, num_rows, num_heads] fp32
 *   out       [num_rows, num_heads, head_dim] fp16
 *   out_lse   NULL or [num_rows, num_heads] fp32
 * head_dim must be a multiple of 4 and at most 1024.
 */
sv_status sv_verify_merge(const float* part_o, const float* part_lse, int32_t num_splits,
                          int32_t num_rows, int32_t num_heads, int32_t head_dim, void* out,
                          float* out_lse, void* stream);

/*
 * Verify blocks of different widths per request (the adaptive verify width
 * of the PocketLLM page's DFlash2 runs; per-request verify lengths chosen by
 * a scheduler, DSpark in section 1.7.2 of the page "DFlash -> dLLM
 * self-spec, part 1"). The same attention as sv_verify_attention, with the
 * rows of the requests packed one after another:
 *
 *   q_start     [batch+1] int32 device: request b owns rows
 *               q_start[b] .. q_start[b+1]-1 of q / out / out_lse, i.e. a
 *               block of q_b = q_start[b+1] - q_start[b] rows, 0 <= q_b <= p->q_len,
 *               and all rows lie in 0 .. batch*p->q_len - 1 (sv_prepare_block
 *               writes such offsets). Row i of request b attends to cache
 *               positions 0 .. kv_lens[b] - q_b + i. A request with q_b = 0
 *               is skipped; one that breaks the rule is skipped and flagged
 *               (SV_FLAG_BAD_BLOCK_WIDTH).
 *   p->q_len    the largest width; the plan, the workspace size and the
 *               kernels' row blocks are those of a uniform call of that width
 *   q, out      [rows, Hq, D] fp16 (rows = q_start[batch]); out_lse [rows, Hq]
 * Every other argument is as for sv_verify_attention. Rows outside every
 * request's range are not written.
 */
sv_status sv_verify_attention_ragged(const sv_verify_params* p, const int32_t* q_start, const void* q,
                                     const void* k_pages, const void* v_pages, const void* k_scales,
                                     const void* v_scales, const int32_t* page_table, const int32_t* kv_lens,
                                     void* out, float* out_lse, void* workspace, size_t workspace_bytes,
                                     int32_t* status_flags, void* stream);

/* Bytes of workspace sv_greedy_accept (and sv_greedy_accept_ragged with
 * q_len = its max_q_len) needs. */
size_t sv_greedy_accept_workspace_bytes(int32_t batch, int32_t q_len, int32_t vocab);

/*
 * Greedy acceptance of a verify block (worked example "Why the target output
 * stayed the same", page "MTP and DFlash2 at long context on XPU"; glossary
 * entries "bonus token" and "accept length" and section 1.6.1 on the page
 * "DFlash -> dLLM self-spec, part 1"). Row j's logits are the target's
 * choice after t0, d1..dj, so draft d_{j+1} is checked against row j:
 *     am_j       = argmax of logits row b*q_len + j (lowest index on ties)
 *     accept_len = largest A <= q_len-1 with draft_ids[b][j] == am_j for all j < A
 *     bonus      = am_A   (the first mismatching row; the last row if all match)
 *     kv_lens_out[b] = kv_lens_in[b] - q_len + 1 + accept_len  (prefix + A drafts + bonus)
 *
 *   logits      [batch*q_len, vocab] fp32, finite (NaN order is unspecified)
 *   draft_ids   [batch, q_len-1] int32 (may be NULL when q_len == 1)
 *   accept_len  [batch] int32 (written)
 *   bonus_ids   [batch] int32 (written)
 *   argmax_ids  NULL or [batch*q_len] int32 (written)
 *   kv_lens_in, kv_lens_out  both NULL, or both [batch] int32 (may alias)
 *   workspace   sv_greedy_accept_workspace_bytes() bytes, 256-byte aligned
 * Two launches (the slice scan, then one workgroup per request that reduces
 * the slices and walks the drafts); nothing is kept between calls.
 */
sv_status sv_greedy_accept(const float* logits, const int32_t* draft_ids, int32_t batch,
                           int32_t q_len, int32_t vocab, int32_t* accept_len, int32_t* bonus_ids,
                           int32_t* argmax_ids, const int32_t* kv_lens_in, int32_t* kv_lens_out,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Greedy acceptance of packed blocks of different widths (same rule as
 * sv_greedy_accept, rows packed as for sv_verify_attention_ragged).
 *
 *   logits      [rows, vocab] fp32, rows = q_start[batch]
 *   block_ids   [rows] int32: request b's rows hold its block t0, d1, ..,
 *               d_{q_b-1} (as sv_prepare_block writes them), so the draft
 *               checked against row j is the id one row later; may be NULL
 *               when max_q_len == 1
 *   q_start     [batch+1] int32 packed row offsets, widths 0..max_q_len
 *   accept_len, bonus_ids [batch] int32 (written); argmax_ids NULL or [rows]
 *   kv_lens_out[b] = kv_lens_in[b] - q_b + 1 + accept_len[b]
 * A request without a block (q_b = 0, or flagged SV_FLAG_BAD_BLOCK_WIDTH)
 * gets accept_len 0, bonus -1 and kv_lens_out = kv_lens_in.
 * workspace: sv_greedy_accept_workspace_bytes(batch, max_q_len, vocab) bytes.
 */
sv_status sv_greedy_accept_ragged(const float* logits, const int32_t* block_ids, const int32_t* q_start,
                                  int32_t batch, int32_t max_q_len, int32_t vocab, int32_t* accept_len,
                                  int32_t* bonus_ids, int32_t* argmax_ids, const int32_t* kv_lens_in,
                                  int32_t* kv_lens_out, void* workspace, size_t workspace_bytes,
                                  int32_t* status_flags, void* stream);

/*
 * Block preparation of one verify round (the fused step that yields the
 * block's token ids, positions and cache locations, section 1.3.3 of the
 * page "DFlash -> dLLM self-spec, part 1"; slots reserved ahead of time,
 * section 1.3.2 "KV over-allocation"). For request b with committed length
 * L_b = seq_lens[b] and width q_b = q_lens[b]:
 *     q_start[b]   = q_0 + .. + q_{b-1};  q_start[batch] = total rows
 *     positions[q_start[b] + i]  = L_b + i                      (i < q_b)
 *     cache_slot[q_start[b] + i] = page_table[b][(L_b+i) / P] * P + (L_b+i) % P
 *     kv_lens_out[b] = L_b + q_b       (the cache length the verify pass sees)
 *     block_ids[q_start[b] + i] = last_tokens[b] (i = 0) or draft_ids[b][i-1]
 *
 *   seq_lens, q_lens  [batch] int32; 0 <= q_lens[b] <= max_q_len (else the
 *               width is taken as 0 and SV_FLAG_BAD_BLOCK_WIDTH set)
 *   page_table  [batch, max_pages_per_req] int32, pages of the pool that
 *               sv_verify_attention reads; a position past the row or on a
 *               page id outside 0..num_pages-1 gets cache_slot -1
 *               (SV_FLAG_PAGE_ID_OUT_OF_RANGE)
 *   last_tokens NULL, or [batch] int32: t0 of each block (with block_ids)
 *   draft_ids   [batch, max_q_len-1] int32, padded (may be NULL when
 *               max_q_len == 1 or last_tokens is NULL)
 *   q_start     [batch+1] int32 (written)
 *   positions   NULL or [batch*max_q_len] int32 (first q_start[batch] written)
 *   cache_slot  [batch*max_q_len] int32 (first q_start[batch] written)
 *   kv_lens_out NULL or [batch] int32 (written; may alias seq_lens)
 *   block_ids   NULL or [batch*max_q_len] int32 (written)
 * One workgroup; cost grows with batch (about a microsecond per 256 requests).
 */
sv_status sv_prepare_block(const int32_t* seq_lens, const int32_t* q_lens, const int32_t* page_table,
                           int32_t batch, int32_t max_q_len, int32_t max_pages_per_req, int32_t page_size,
                           int32_t num_pages, const int32_t* last_tokens, const int32_t* draft_ids,
                           int32_t* q_start, int32_t* positions, int32_t* cache_slot, int32_t* kv_lens_out,
                           int32_t* block_ids, int32_t* status_flags, void* stream);

/*
 * Writing a block's K and V into its reserved cache slots (the append of
 * the verify block before the verify pass, section 1.3.2 of the page
 * "DFlash -> dLLM self-spec, part 1"):
 *     k_pages[slot / P, h, slot % P, :] = new_k[r, h, :]   (same for V)
 * for every packed row r in q_start[0] .. q_start[batch]-1 (clamped to
 * max_rows) with slot = cache_slot[r] >= 0.
 *
 *   new_k, new_v  [rows, num_kv_heads, head_dim] fp16, 16-byte aligned
 *   cache_slot    [rows] int32 flat slots page*P + slot, or -1 (skipped);
 *                 a slot >= num_pages*page_size is skipped and flagged
 *                 (SV_FLAG_PAGE_ID_OUT_OF_RANGE)
 *   q_start       [batch+1] int32 (e.g. from sv_prepare_block)
 *   max_rows      host bound on q_start[batch]: sizes the grid
 *   k_pages, v_pages  [num_pages, num_kv_heads, page_size, head_dim], written
 *   kv_dtype      SV_KV_FP16 only (FP8 pages: SV_ERR_UNSUPPORTED; use sv_append_kv_fp8)
 * Rows that share a slot race; prepare_block never gives two rows one slot
 * when the page table maps distinct positions to distinct slots.
 */
sv_status sv_append_kv(const void* new_k, const void* new_v, const int32_t* cache_slot, const int32_t* q_start,
                       int32_t batch, int32_t max_rows, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                       int32_t num_pages, sv_kv_dtype kv_dtype, void* k_pages, void* v_pages,
                       int32_t* status_flags, void* stream);

/*
 * The same append into an FP8 cache (the E4M3 pages with one fp16 scale per
 * token, KV head and 64-channel block of the page "Qwen3.8-27B-FP8",
 * sections "Implemented execution path" and "KV cache dtype and the
 * 262,144-token boundary"): each new row is quantised per 64-channel block,
 *     scale = fp16(amax / 448)   (amax = largest |x| of the block; 1.0 where
 *                                 the fp16 value would be 0)
 *     code  = E4M3 of clamp(x / scale, -448, 448), nearest value, ties to
 *             the even code, the sign kept (-0 gives 0x80)
 * with both divisions in fp32 rounded to nearest, and written with its scales:
 *     k_pages[slot / P, h, slot % P, :]        = codes of new_k[r, h, :]
 *     k_scales[slot / P, h, slot % P, 0..D/64) = their scales   (same for V)
 *
 *   new_k, new_v  [rows, num_kv_heads, head_dim] fp16, 8-byte aligned
 *   head_dim      a multiple of 64 (the verify attention reads 256)
 *   k_pages, v_pages    [num_pages, num_kv_heads, page_size, head_dim] uint8, 4-byte aligned
 *   k_scales, v_scales  [num_pages, num_kv_heads, page_size, head_dim/64] fp16
 *   other arguments, the skipped and flagged slots and the races as in sv_append_kv.
 */
sv_status sv_append_kv_fp8(const void* new_k, const void* new_v, const int32_t* cache_slot, const int32_t* q_start,
                           int32_t batch, int32_t max_rows, int32_t num_kv_heads, int32_t head_dim,
                           int32_t page_size, int32_t num_pages, void* k_pages, void* v_pages, void* k_scales,
                           void* v_scales, int32_t* status_flags, void* stream);

/* Bytes of workspace sv_rejection_accept needs. */
size_t sv_rejection_accept_workspace_bytes(int32_t batch, int32_t q_len, int32_t vocab);

/*
 * Stochastic acceptance of a verify block: rejection sampling against the
 * target's and the draft's probabilities (the sampling case of "Why the
 * target output stayed the same", page "MTP and DFlash2 at long context on
 * XPU"; a verify post-processing step in section 1.1 of the page "DFlash ->
 * dLLM self-spec, part 1"). With p_j = softmax(logits row b*q_len + j / T):
 *     draft d_{j+1} = draft_ids[b][j] is kept while
 *         u_accept[b][j] * draft_probs[b][j][d] < p_j(d)    (j = 0, 1, ..)
 *     accept_len[b] = A, the number kept
 *     token_ids[b]  = the inverse-CDF draw with u_final[b] (the smallest v
 *         whose cumulative weight exceeds u_final * total weight) from
 *         max(p_A - draft_probs[b][A], 0) when A < q_len-1 (from p_A if that
 *         residual is zero everywhere), else from p_{q_len-1}
 *     kv_lens_out[b] = kv_lens_in[b] - q_len + 1 + A
 *
 *   logits       [batch*q_len, vocab] fp32, finite
 *   draft_ids    [batch, q_len-1] int32 (an id outside 0..vocab-1 is never kept)
 *   draft_probs  [batch, q_len-1, vocab] fp32: row j is the distribution
 *                d_{j+1} was drawn from
 *   temperature  > 0 (the logits are divided by it; no top-k/top-p filter)
 *   u_accept     [batch, q_len-1] fp32 uniforms on [0, 1); u_final [batch]
 *                (the caller's random numbers: the call itself is
 *                deterministic)
 *   accept_len, token_ids [batch] int32 (written)
 *   kv_lens_in, kv_lens_out  both NULL, or both [batch] int32 (may alias)
 *   workspace    sv_rejection_accept_workspace_bytes() bytes, 256-byte aligned
 * Arithmetic is fp32; q_len <= 64; batch * q_len <= 65535; vocab <= 524,288. The three NULL
 * draft pointers are allowed when q_len == 1.
 */
sv_status sv_rejection_accept(const float* logits, const int32_t* draft_ids, const float* draft_probs,
                              int32_t batch, int32_t q_len, int32_t vocab, float temperature, const float* u_accept,
                              const float* u_final, int32_t* accept_len, int32_t* token_ids,
                              const int32_t* kv_lens_in, int32_t* kv_lens_out, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Bytes of workspace sv_topk_candidates needs. */
size_t sv_topk_candidates_workspace_bytes(int32_t rows, int32_t vocab, int32_t k);

/*
 * Top-k candidate selection over the vocabulary (the draft side's per-position
 * top-16 candidate sets of DFlash2: page "MTP and DFlash2 at long context on
 * XPU", the DFlash2 description — a local top 16 per shard, then a top 16 of
 * the gathered candidates, equal to the unsharded set; the PocketLLM page's
 * split top-16 with one comparator). For every row:
 *     out_ids[row][0..k-1] = the k columns with the largest logits, in order:
 *     larger value first, the lower column index first among equal values
 *     out_values[row][j]   = logits[row][out_ids[row][j]]
 *
 *   logits      [rows, vocab] fp32 (NaN order is unspecified; -inf allowed)
 *   k           1..16, k <= vocab; vocab <= 512/k * 8,192 columns (262,144 at k = 16)
 *   out_ids     [rows, k] int32 (written); out_values [rows, k] fp32 (written)
 *   workspace   sv_topk_candidates_workspace_bytes() bytes
 * rows <= 65535. The same kernels give the top k of any slice union, so a
 * vocabulary-sharded head can run them per shard and merge the per-shard
 * lists with this call on the gathered candidates.
 */
sv_status sv_topk_candidates(const float* logits, int32_t rows, int32_t vocab, int32_t k, int32_t* out_ids,
                             float* out_values, void* workspace, size_t workspace_bytes, void* stream);

const char* sv_status_string(sv_status s);
const char* sv_last_error(void);

/* Library version as major*10000 + minor*100 + patch. */
int32_t sv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SV_H_ */
