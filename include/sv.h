/*
 * sv.h — C ABI of the target-verify path of speculative decoding on MI355X
 * (gfx950): paged causal grouped-query attention of a verify block, the
 * merge of split-KV partials, and greedy acceptance.
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
#define SV_FLAG_PAGE_ID_OUT_OF_RANGE 0x4 /* page id < 0 or >= num_pages; page 0 read instead */

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
 */
typedef struct {
  int32_t batch;             /* B >= 1 requests */
  int32_t q_len;             /* verify rows per request, 1..16 */
  int32_t num_q_heads;       /* Hq; query head h uses KV head h / (Hq/Hkv) */
  int32_t num_kv_heads;      /* Hkv, divides Hq; q_len * Hq/Hkv <= 96 */
  int32_t head_dim;          /* D, must be 256 */
  int32_t page_size;         /* P tokens per page: a multiple of 16, at most 4096 */
  int32_t num_pages;         /* pages in the pool (bounds page ids) */
  int32_t max_pages_per_req; /* row stride of page_table */
  int32_t max_kv_len;        /* host upper bound on every kv_lens[b]; sizes the grid */
  sv_kv_dtype kv_dtype;
  float sm_scale;            /* softmax scale, e.g. 1/sqrt(D) */
  int32_t num_splits;        /* 0 = automatic; > 0 forces the number of key chunks */
} sv_verify_params;

/*
 * Bytes of workspace sv_verify_attention needs for these parameters (0 when
 * one key chunk covers max_kv_len). Depends only on the host fields.
 */
size_t sv_verify_workspace_bytes(const sv_verify_params* p);

/*
 * Number of key chunks (splits) the planner uses for these parameters, and
 * the chunk length in tokens. Chunks are anchored at absolute position 0:
 * chunk s covers cache positions [s*chunk, (s+1)*chunk). Host only.
 */
sv_status sv_verify_plan(const sv_verify_params* p, int32_t* num_splits, int32_t* chunk_tokens);

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
 *               aligned; contents need no initialisation
 *   status_flags NULL or one int32 word (see SV_FLAG_*)
 *
 * Arithmetic: fp16 (or exactly dequantised E4M3) inputs, fp32 accumulation;
 * the result does not depend on the number of splits beyond rounding.
 */
sv_status sv_verify_attention(const sv_verify_params* p, const void* q, const void* k_pages,
                              const void* v_pages, const void* k_scales, const void* v_scales,
                              const int32_t* page_table, const int32_t* kv_lens, void* out,
                              float* out_lse, void* workspace, size_t workspace_bytes,
                              int32_t* status_flags, void* stream);

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

/* Bytes of workspace sv_greedy_accept needs. */
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
 */
sv_status sv_greedy_accept(const float* logits, const int32_t* draft_ids, int32_t batch,
                           int32_t q_len, int32_t vocab, int32_t* accept_len, int32_t* bonus_ids,
                           int32_t* argmax_ids, const int32_t* kv_lens_in, int32_t* kv_lens_out,
                           void* workspace, size_t workspace_bytes, void* stream);

const char* sv_status_string(sv_status s);
const char* sv_last_error(void);

/* Library version as major*10000 + minor*100 + patch. */
int32_t sv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SV_H_ */
