// Paged causal GQA of a speculative verify block on gfx950 (fp16 or FP8 KV).
//
// One workgroup owns one (key chunk, KV head, request, row tile). All q_len x G
// rows of the KV head's query group ("packed rows": the verify positions
// folded with the G query heads that share the KV head) are processed
// together, so every K/V byte read from HBM is used by every row of the group
// in registers.
//
// Matrix-core mapping (wave64, v_mfma 16x16):
//   S^T = K . Q^T   with 16x16x32 f16: M = 16 tokens, N = 16 rows, K = 32 channels.
//                    A = K rows loaded straight from the page (lane = token),
//                    B = Q fragments, loaded once into each wave's registers.
//   O^T = V^T . P^T with 16x16x16 f16: M = 16 channels, N = 16 rows, K = 16 tokens.
//                    B = P^T is the S^T accumulator converted in place: the
//                    lane that holds a row's scores also holds its softmax
//                    state and its O accumulators, so the online-softmax
//                    rescale needs no cross-lane traffic.
//                    A = V^T: for fp16 KV read from LDS by the transposing
//                    ds_read_b64_tr_b16 (block j is channels 16j .. 16j+15);
//                    for FP8 KV interleaved bytewise in registers and
//                    converted (block j = 4bb + c is channels
//                    64bb + 4*lane16 + c).
// The reduction order inside one MFMA is the hardware's; only the pairing of
// A and B slots is relied on, plus the accumulator layout
// (lane l holds rows 4*(l/16)+i, column l%16).
//
// The chunk's 16-token steps are dealt round-robin to the 4 waves of the
// workgroup. Each wave keeps one or two steps of K/V in flight in a private
// LDS ring while it computes the previous one. At the end the waves' (m, l, O)
// are combined through LDS and the workgroup writes either the final fp16
// rows (request fits one chunk) or an fp32 partial (o normalised, lse) for
// the merge kernel. A workgroup holds at most 48 rows; a KV head with more is
// covered by several workgroups (row tiles) that read the same keys, placed
// on the same XCD so that the later reads are mostly served by its L2.
#include <type_traits>

#include "verify_frag.h"

namespace sv {

template <int RB, bool FP8, int DEPTH>
struct Smem {
  static constexpr int QBYTES = RB * 8 * kWave * 16;
  static constexpr int OBYTES = RB * 16 * kRowStride * 4;
  // a private DEPTH-step ring per wave
  static constexpr int RBYTES = kWavesPerGroup * DEPTH * (FP8 ? kStage8 : kRingStage);
  // Q fragments in their own array (so reading them never waits for the
  // ring's DMAs); the ring and, after the main loop, the combine buffer
  // share the second array.
  static constexpr int BIG = RBYTES > OBYTES ? RBYTES : OBYTES;
};

template <int RB, bool FP8, int DEPTH, bool WIN, bool CLAIM, int CP>
__global__ __launch_bounds__(kThreads, 1) void verify_attn_kernel(AttnArgs a) {
  static_assert(DEPTH == 1 || DEPTH == 2, "one or two steps in flight");
  static_assert(!CLAIM || (!FP8 && DEPTH == 1 && !WIN), "claimed work: fp16 KV, one step in flight, full attention");
  using SM = Smem<RB, FP8, DEPTH>;
  constexpr int NTS = kWavesPerGroup;  // waves that split the chunk's steps
  // K/V cache policy CP: two steps in flight is the launch whose row tiles
  // share the keys (the later ones read them from L2), which keeps the default
  // policy; with one row tile every K/V byte is read once.
  static_assert(DEPTH == 1 || CP == kCacheDefault, "row tiles that share keys keep them in L2");
  __shared__ __attribute__((aligned(1024))) unsigned char qsm[SM::QBYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char bigsm[SM::BIG];
  __shared__ float s_m[NTS][RB * 16];
  __shared__ float s_l[NTS][RB * 16];
  __shared__ int s_flag;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int ts = wave;
  // Workgroup -> (key chunk, KV head, request, row tile). With n row tiles
  // the n workgroups that share a (chunk, KV head, request) get ids 8 apart
  // in one group of 8n, i.e. the same XCD at about the same time (ids go
  // round-robin over the 8 XCDs), so the later readers of each K/V byte
  // mostly find it in that XCD's L2.
  int unit = blockIdx.x, rblk = 0;
  if (a.row_blocks > 1) {
    const int r = blockIdx.x >> 3;
    rblk = r % a.row_blocks;
    unit = ((r / a.row_blocks) << 3) | (blockIdx.x & 7);
    if (unit >= a.units) return;
  }
  // Units are numbered split-major: every (KV head, request) of chunk 0,
  // then chunk 1, ... Consecutive ids (which go to consecutive XCDs) then
  // differ in head and request rather than in chunk, so ragged batches spread
  // evenly over the XCDs. For 2..64 requests ordered_unit takes the full
  // chunks in that order, then the last partial chunks, longest first.
  int split, g, b;
  if (CLAIM || a.balanced) {
    // S (a multiple of 8) workgroups per (request, KV head) group: group
    // (unit / 8) mod (B * Hkv), so each group's workgroups sit on all 8 XCDs
    // and the faster XCDs can claim more of its keys (or, with balanced
    // static chunks, get longer ones). `split` is the workgroup's partial
    // slot; its XCD is split mod 8.
    const int grp = unit >> 3, n_grp = a.batch * a.num_kv_heads;
    g = (grp % n_grp) % a.num_kv_heads;
    b = (grp % n_grp) / a.num_kv_heads;
    split = (grp / n_grp) * 8 + (unit & 7);
  } else if (a.batch > 1 && a.batch <= kWave) {
    if (!ordered_unit<WIN>(a, unit, lane, unit == 0 && rblk == 0 && tid < kWave, &split, &b, &g)) return;
  } else {
    const int hb = unit % (a.num_kv_heads * a.batch);
    split = unit / (a.num_kv_heads * a.batch);
    g = hb % a.num_kv_heads;
    b = hb / a.num_kv_heads;
  }
  const int row0 = rblk * RB * 16;  // first row (of the KV head's q_len*G) of this workgroup
  int flag_bits = 0;
  // the request's block: q_len rows from packed row rstart
  int q_len = a.q_len, rstart = b * a.q_len;
  if (a.q_start) {
    q_len = block_rows(a.q_start, b, a.batch, a.q_len, &rstart, &flag_bits);
    if (q_len == 0) {
      if (flag_bits && tid == 0 && a.flags) atomicOr(a.flags, flag_bits);
      return;
    }
  }
  const int G = a.group, R = q_len * G, Hq = a.num_q_heads;
  if (row0 >= R) return;  // a narrow block leaves the last row tiles empty
  const size_t split_stride = (size_t)a.batch * a.q_len * Hq;  // rows of one split's partials

  // Q fragments of the workgroup's rows, in MFMA B-operand order: loaded into
  // registers first (they depend on no length), so that their latency
  // overlaps the length, page and first K/V loads; they go to LDS once the
  // first DMAs are out.
  constexpr int kQPer = RB * 8 * kWave / kThreads;
  u32x4 qv[kQPer];
#pragma unroll
  for (int k = 0; k < kQPer; ++k) {
    const int idx = tid + k * kThreads;
    const int frag = idx / kWave, ln = idx % kWave;
    const int rb = frag / 8, s = frag % 8;
    const int r = row0 + rb * 16 + (ln & 15);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r < R) {
      const int i = r / G, j = r % G;
      // channel map of the score MFMA's k-step s: fp16 KV 32s + 8*(lane/16);
      // FP8 KV 64*(s/2) + 16*(lane/16) + 8*(s%2) (two k-steps per scale block)
      const int d0 = FP8 ? 64 * (s >> 1) + 16 * (ln >> 4) + 8 * (s & 1) : 32 * s + 8 * (ln >> 4);
      const _Float16* src = a.q + ((size_t)(rstart + i) * Hq + g * G + j) * kHeadDim + d0;
      v = *reinterpret_cast<const u32x4*>(src);
    }
    qv[k] = v;
  }

  const int raw_kv_v = a.kv_lens[b];
  // claimed work: this wave's counter of the head, and its first ticket (of
  // its second segment, or of its first when the cache is too short for a
  // static one), which does not depend on the length either
  const int n_ctr = claim_counters(a.num_splits, a.batch * a.num_kv_heads);
  const int cidx = (ts + NTS * (split >> 3)) % n_ctr;
  int32_t* const ctr = CLAIM ? a.counters + ((b * a.num_kv_heads + g) * n_ctr + cidx) * kCounterStride : nullptr;
  // pool grain of ticket t of this wave's counter (for valid tickets only:
  // see `mine` below, which bounds t before the product is formed)
  auto grain_of = [&](int t) { return cidx + t * n_ctr; };
  int first_ticket = -1;
  if constexpr (CLAIM) {
    int t = 0;
    if (lane == 0) t = atomicAdd(ctr, 1);
    first_ticket = __builtin_amdgcn_readfirstlane(t);
  }
  const int raw_kv = __builtin_amdgcn_readfirstlane(raw_kv_v);
  const int kv = clamp_kv_len(raw_kv, a.max_kv_len, a.max_pages, a.page_size, &flag_bits);
  if (raw_kv < q_len) flag_bits |= 0x2;
  const int L = kv - q_len;
  const int W = a.window, S = a.sink;
  // Key chunks tile the block's live 16-token steps (all steps from position
  // 0, or with a sliding window the sink steps then the window steps):
  // chunk `split` holds steps [split*cs, split*cs + n_steps).
  int n_sink = 0, w0 = 0;
  const int total = WIN ? live_steps(kv, L, W, S, &n_sink, &w0) : (kv > 0 ? (kv + kStep - 1) / kStep : 0);
  const int cs = a.chunk / kStep;
  const int n_chunks = total > 0 ? (total + cs - 1) / cs : 1;
  // (every slot of a balanced plan writes its partial, an empty one too)
  if (!CLAIM && !a.balanced && split >= n_chunks) return;  // whole group: nothing of this request here
  const bool direct = !CLAIM && !a.balanced && (n_chunks == 1);
  int k_base = split * cs;
  int n_steps = min(total - k_base, cs) > 0 ? min(total - k_base, cs) : 0;
  if (!CLAIM && a.balanced) {
    k_base = xcd_chunk_start(total, split, a.num_splits);
    n_steps = xcd_chunk_start(total, split + 1, a.num_splits) - k_base;
  }
  auto live_t0 = [&](int j) {
    const int k = k_base + j;
    if constexpr (!WIN) return kStep * k;
    return k < n_sink ? kStep * k : w0 + kStep * (k - n_sink);
  };
  if (tid == 0) s_flag = 0;

  const int P = a.page_size, Hkv = a.num_kv_heads;
  const _Float16* kpool = static_cast<const _Float16*>(a.k_pages);
  const _Float16* vpool = static_cast<const _Float16*>(a.v_pages);
  const uint8_t* kpool8 = static_cast<const uint8_t*>(a.k_pages);
  const uint8_t* vpool8 = static_cast<const uint8_t*>(a.v_pages);
  const int32_t* ptab = a.page_table + (size_t)b * a.max_pages;
  // cache row ((page, KV head, slot); the pool holds fewer than 2^32 rows)
  // of position t whose page id is pid
  auto row_of = [&](int pid, int t) -> uint32_t {
    if (pid < 0 || pid >= a.num_pages) {
      flag_bits |= 0x4;
      pid = 0;
    }
    return ((uint32_t)pid * (uint32_t)Hkv + (uint32_t)g) * (uint32_t)P + (uint32_t)(t % P);
  };
  // Claimed work: this wave's first segment (the static one, or a first
  // grain when the cache is too short for one) and the ticket of the next.
  int c_f = 0, c_pool0 = 0, c_ngr = 0, seg_base = 0, seg_nb = 0, ticket1 = -1;
  // the grains this wave's counter deals: tickets 0 .. n_mine-1 are valid.
  // Comparing the ticket itself keeps a counter that did not start at zero
  // (any value) from forming an overflowing grain index.
  int n_mine = 0;
  auto mine = [&](int t) { return t >= 0 && t < n_mine; };
  // grains this wave took from its counter: added to the group's tally at
  // the end, which the merge checks against the grain count (a counter that
  // started above zero skips grains yet ends at the clean value)
  int n_claimed = 0;
  if constexpr (CLAIM) {
    claim_layout(total, a.num_splits, &c_f, &c_pool0, &c_ngr);
    n_mine = counter_grains(c_ngr, cidx, n_ctr);
    auto claim = [&]() {
      int t = 0;
      if (lane == 0) t = atomicAdd(ctr, 1);
      return __builtin_amdgcn_readfirstlane(t);
    };
    if (c_f > 0) {
      seg_base = (split * NTS + ts) * c_f;
      seg_nb = c_f;
      ticket1 = first_ticket;
    } else {
      const int t0c = first_ticket;
      if (mine(t0c)) {  // (a counter that did not start at 0 can give anything)
        seg_base = c_pool0 + grain_of(t0c) * kGrain;
        seg_nb = min(kGrain, total - seg_base);
        ticket1 = claim();
        ++n_claimed;
      }
    }
  }
  const int my_steps = CLAIM ? seg_nb : (n_steps > ts ? (n_steps - ts + NTS - 1) / NTS : 0);
  // page id of each of the wave's steps bstart .. bstart+63, one per lane
  // Lane kl of the wave finds the cache row ((page, KV head, slot); the pool
  // holds fewer than 2^32 rows) of the first token of the wave's step
  // bstart + kl, once per batch of 64 steps; a step's DMAs then take it with
  // one readlane.
  auto step_rows = [&](int bstart) {
    uint32_t row = 0;
    const int kl = bstart + lane;
    if (kl < my_steps) {
      const int t = CLAIM ? kStep * (seg_base + kl) : live_t0(ts + kl * NTS);
      row = row_of(ptab[t / P], t);
    }
    return row;
  };
  auto tok_row = [&](uint32_t rows, int kk) {
    return (size_t)(uint32_t)__builtin_amdgcn_readlane((int)rows, kk);
  };
  constexpr int kStageBytes = FP8 ? kStage8 : kRingStage;
  char* const ring = reinterpret_cast<char*>(bigsm) + wave * DEPTH * kStageBytes;
  // The first steps' DMAs go out before Q is staged, so the two latencies
  // overlap (Q lives in its own array; the ring is the wave's own). Step
  // indices past the batch are clamped to its last step.
  uint32_t rows_first = 0;
  if (my_steps > 0) {
    rows_first = step_rows(0);
    const int nb0 = min(kWave, my_steps);
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const size_t tr = tok_row(rows_first, min(d, nb0 - 1));
      char* stage = ring + d * kStageBytes;
      if constexpr (FP8) {
        dma_k8<CP>(kpool8 + tr * kHeadDim, a.k_scales + tr * 4, a.v_scales + tr * 4, stage, lane);
        dma_v8<CP>(vpool8 + tr * kHeadDim, stage, lane);
      } else {
        dma_k<0, 8, CP>(kpool + tr * kHeadDim, stage, lane);
        dma_v<0, 8, CP>(vpool + tr * kHeadDim, stage + 8192, lane);
      }
    }
  }

  // the Q fragments (loaded above) into LDS
  u32x4* qlds = reinterpret_cast<u32x4*>(qsm);
#pragma unroll
  for (int k = 0; k < kQPer; ++k) qlds[tid + k * kThreads] = qv[k];
  __syncthreads();

  WaveState<RB> ws;
  ws.c = a.scale_log2;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    ws.m[rb] = -INFINITY;
    ws.l[rb] = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) ws.o[rb][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  const u32x4* qf = qlds;
  const int rowbase = 0;               // first row of the wave, local to the workgroup
  const int growbase = row0 + rowbase;  // the same row in the KV head's numbering
  // the keys each of this lane's rows sees: row r (block row i = r/G, at
  // position L + i) sees t <= L + i and, with a window, t > L + i - W or t < S;
  // padding rows see every key
  RowMask<RB, WIN> mk;
  mk.sink = S;
  int lmin = INT32_MAX, lmax = INT32_MIN;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = growbase + rb * 16 + (lane & 15);
    mk.lim[rb] = r < R ? min(L + r / G + 1, kv) : kv;
    mk.lo[rb] = r < R ? L + r / G + 1 - W : INT32_MIN;
    lmin = min(lmin, mk.lim[rb]);
    lmax = max(lmax, mk.lo[rb]);
  }
  // across the wave (every lane takes part): the smallest limit, the largest lower edge
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    lmin = min(lmin, __shfl_xor(lmin, o));
    lmax = max(lmax, __shfl_xor(lmax, o));
  }
  mk.lim_min = __builtin_amdgcn_readfirstlane(lmin);
  mk.lo_max = __builtin_amdgcn_readfirstlane(lmax);
  if constexpr (FP8) {
    // ---- FP8: each wave owns its token steps and a private one-step ring ----
    // (same schedule as the fp16 ring below; half-steps are K bytes + both
    // scale sets (5 operations) and V bytes (4 operations): the V half-step
    // (4) is newer than a K read, the next K half-step (5) than a V read)
    const uint32_t ring_lds = lds_addr(ring);
    u32x4 qa[RB][8];  // the wave's Q fragments, in registers for the whole loop
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
      ring_read8<63, 1024>(qa[rb], lds_addr(qf) + (uint32_t)(rb * 8 * kWave + lane) * 16u);
    for (int bstart = 0; bstart < my_steps; bstart += kWave) {
      const uint32_t rows = bstart == 0 ? rows_first : step_rows(bstart);
      const int nb = min(kWave, my_steps - bstart);
      auto step_t0 = [&](int kk) { return live_t0(ts + (bstart + kk) * NTS); };
      auto issue_k = [&](int kk, int stg) {
        const size_t tr = tok_row(rows, kk);
        dma_k8<CP>(kpool8 + tr * kHeadDim, a.k_scales + tr * 4, a.v_scales + tr * 4, ring + stg * kStage8, lane);
      };
      auto issue_v = [&](int kk, int stg) {
        dma_v8<CP>(vpool8 + tok_row(rows, kk) * kHeadDim, ring + stg * kStage8, lane);
      };
      if (bstart > 0) {  // (the first batch's first steps were issued before Q staging)
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
          issue_k(min(d, nb - 1), d);
          issue_v(min(d, nb - 1), d);
        }
      }
      // before a K read the newer operations are V(k) and, with two steps
      // in flight, K(k+1), V(k+1): 4 or 13; before a V read K(k+1) and, with
      // two, V(k+1), K(k+2): 5 or 14
      constexpr int kWaitK = DEPTH == 1 ? 4 : 13, kWaitV = DEPTH == 1 ? 5 : 14;
      // Software pipeline as in the fp16 loop: step k's PV runs while step
      // k+1's softmax is computed (same read order, so the same waits).
      auto sbase = [&](int kk) { return ring_lds + (kk & (DEPTH - 1)) * kStage8; };
      half4_t pr[RB];
      u32x4 sv[2];  // V scales of the step whose PV is next
      {
        KFrag8 kf;
        ring_read_k8<kWaitK>(kf, sbase(0) + k8_lane_off(lane), sbase(0) + 8192 + 32 * (lane >> 4));
        issue_k(min(DEPTH, nb - 1), 0);
        float x0[RB][4], p0[RB][4];
        scores8_mfma<RB>(kf, qa, x0);
        softmax_step<RB>(x0, ws, p0, lane, step_t0(0), mk);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          pr[rb] = half4_t{(_Float16)p0[rb][0], (_Float16)p0[rb][1], (_Float16)p0[rb][2], (_Float16)p0[rb][3]};
        sv[0] = kf.sv[0];
        sv[1] = kf.sv[1];
      }
      auto body = [&](int kk, auto masked) {
        constexpr bool MASKED = decltype(masked)::value;
        const int t0 = step_t0(kk);
        VFrag8 vf;
        ring_read_v8<kWaitV>(vf, sbase(kk) + 4096 + v8_lane_off(lane));
        issue_v(min(kk + DEPTH, nb - 1), kk & (DEPTH - 1));
        KFrag8 kf;
        ring_read_k8<kWaitK>(kf, sbase(kk + 1) + k8_lane_off(lane), sbase(kk + 1) + 8192 + 32 * (lane >> 4));
        issue_k(min(kk + 1 + DEPTH, nb - 1), (kk + 1) & (DEPTH - 1));
        float x[RB][4], lmx[RB], alpha[RB], lsum[RB];
        scores8_mfma<RB>(kf, qa, x);
        // (a step before the wave's last of the batch ends below kv_len)
        step_pv8<RB, false>(vf, sv, pr, ws, lane, t0, kv);
        sv[0] = kf.sv[0];
        sv[1] = kf.sv[1];
        bool any;
        if constexpr (MASKED) any = mask_check<RB>(x, lmx, ws, mk, lane, step_t0(kk + 1));
        else any = max_check<RB>(x, lmx, ws);
        softmax_p<RB>(x, ws, lsum, pr);
        pin_softmax<RB>(pr, lsum);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) alpha[rb] = 1.f;
        if (any) {
          move_ref<RB>(lmx, ws, alpha);
          softmax_p<RB>(x, ws, lsum, pr);
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) ws.l[rb] = ws.l[rb] * alpha[rb] + lsum[rb];
        if (any) rescale_o<RB>(ws, alpha);
      };
      // full attention: masking only on the wave's last steps (as in the
      // fp16 loop below)
      int kk = 0, clean = 0;
      if constexpr (!WIN) {
        const int span = mk.lim_min - kStep - step_t0(1);
        clean = span < 0 ? 0 : min(nb - 1, span / (kStep * NTS) + 1);
      }
      for (; kk < clean; ++kk) body(kk, std::false_type{});
      for (; kk + 1 < nb; ++kk) body(kk, std::true_type{});
      {
        VFrag8 vf;
        ring_read_v8<kWaitV>(vf, sbase(nb - 1) + 4096 + v8_lane_off(lane));
        step_pv8<RB>(vf, sv, pr, ws, lane, step_t0(nb - 1), kv);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
  } else {
    // ---- each wave owns its token steps and a private one-step LDS ring ----
    // The wave's Q fragments stay in registers for the whole loop (32 per
    // row block): re-reading them from LDS at every step made up 24 of the
    // step's 40 KB of LDS reads.
    u32x4 qa[RB][8];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
      ring_read8<63, 1024>(qa[rb], lds_addr(qf) + (uint32_t)(rb * 8 * kWave + lane) * 16u);
    if constexpr (CLAIM) {
      // Segments of consecutive steps (the static one, then claimed grains)
      // run back to back through the one-step ring: during the first step
      // of a segment that has a successor, the successor's page ids and the
      // ticket of the segment after it are loaded, so the DMAs run on across
      // segment ends without draining. A segment with a successor has at
      // least 4 steps (only the last grain is shorter), so those rows are
      // in registers before the step two from the end issues the first DMA
      // of the successor.
      const uint32_t ring_lds = lds_addr(ring);
      constexpr int kWait = 8;
      int base = seg_base, nb = my_steps, kk = 0;
      uint32_t rows = rows_first;
      int nbase = 0, nnb = 0;  // the successor (nnb 0: none)
      if (mine(ticket1)) {
        nbase = c_pool0 + grain_of(ticket1) * kGrain;
        nnb = min(kGrain, total - nbase);
        ++n_claimed;
      }
      uint32_t nrows = 0;
      int tnext = -1;
      // cache row of step j of the stream, counted from the current
      // segment's first step; past the stream's end the last step again
      auto tgt = [&](int j) -> size_t {
        if (j < nb) return tok_row(rows, j);
        if (nnb > 0) return tok_row(nrows, min(j - nb, nnb - 1));
        return tok_row(rows, nb - 1);
      };
      if (nb > 0) {
        half4_t pb[RB];
        {
          KFrag kf;
          ring_read8<kWait, 64>(kf.k, ring_lds + k_lane_off(lane));
          dma_k<0, 8, CP>(kpool + tgt(1) * kHeadDim, ring, lane);
          step_scores<RB>(kf, qa, ws, pb, lane, kStep * base, mk);
        }
        for (;;) {
          if (kk + 1 >= nb && nnb == 0) break;  // step kk is the wave's last
          const bool first = kk == 0 && nnb > 0;
          const int t0 = kStep * (base + kk);
          const int t1 = kk + 1 < nb ? t0 + kStep : kStep * nbase;
          VFrag vf;
          ring_read_vt<kWait>(vf, ring_lds + 8192 + v_lane_off(lane), lane);
          // The successor's page ids and the next ticket, as plain vector
          // loads the compiler does not wait for: the wait that follows 16
          // DMAs later (below) completes them without draining the ring.
          int pid_n = 0, tk = 0;
          if (first) {
            const int32_t* pp = ptab + kStep * (nbase + min(lane, nnb - 1)) / P;
            asm volatile("global_load_dword %0, %1, off" : "+v"(pid_n) : "v"(pp) : "memory");
            if (lane == 0) {
              const int one = 1;
              asm volatile("global_atomic_add %0, %1, %2, off sc0" : "+v"(tk) : "v"(ctr), "v"(one) : "memory");
            }
          }
          __builtin_amdgcn_sched_barrier(0);
          dma_v<0, 8, CP>(vpool + tgt(kk + 1) * kHeadDim, ring + 8192, lane);
          KFrag kf;
          // (two more operations are newer than K's DMAs after a first step)
          if (first)
            ring_read8_acc<kWait + 2, 64>(kf.k, ring_lds + k_lane_off(lane));
          else
            ring_read8_acc<kWait, 64>(kf.k, ring_lds + k_lane_off(lane));
          dma_k<0, 8, CP>(kpool + tgt(kk + 2) * kHeadDim, ring, lane);
          float x[RB][4], lmx[RB], alpha[RB], lsum[RB];
          scores_mfma<RB>(kf, qa, x);
          // (only the stream's last step can end above kv_len)
          step_pv<RB, false>(vf, pb, ws, lane, t0, kv);
          const bool any = mask_check<RB, WIN, false>(x, lmx, ws, mk, lane, t1);
          softmax_p<RB>(x, ws, lsum, pb);
          pin_softmax<RB>(pb, lsum);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) alpha[rb] = 1.f;
          if (any) {
            move_ref<RB>(lmx, ws, alpha);
            softmax_p<RB>(x, ws, lsum, pb);
          }
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) ws.l[rb] = ws.l[rb] * alpha[rb] + lsum[rb];
          if (any) rescale_o<RB>(ws, alpha);
          __builtin_amdgcn_sched_barrier(0);
          if (first) {
            // exactly 16 DMAs (V and K of one step) were issued after the two
            // loads: this completes them and leaves the DMAs in flight
            asm volatile("s_waitcnt vmcnt(16)" : "+v"(pid_n), "+v"(tk) : : "memory");
            nrows = row_of(pid_n, kStep * (nbase + min(lane, nnb - 1)));
            tnext = __builtin_amdgcn_readfirstlane(tk);
          }
          if (++kk == nb) {
            base = nbase;
            nb = nnb;
            rows = nrows;
            kk = 0;
            if (mine(tnext)) {
              nbase = c_pool0 + grain_of(tnext) * kGrain;
              nnb = min(kGrain, total - nbase);
              ++n_claimed;
            } else {
              nnb = 0;
            }
            tnext = -1;
          }
        }
        VFrag vf;
        ring_read_vt<kWait>(vf, ring_lds + 8192 + v_lane_off(lane), lane);
        step_pv<RB>(vf, pb, ws, lane, kStep * (base + kk), kv);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      // the group's tally of grains taken (word 1 of its first counter's line)
      if (lane == 0 && n_claimed > 0)
        atomicAdd(a.counters + (b * a.num_kv_heads + g) * n_ctr * kCounterStride + 1, n_claimed);
    } else
    for (int bstart = 0; bstart < my_steps; bstart += kWave) {
      const uint32_t rows = bstart == 0 ? rows_first : step_rows(bstart);
      const int nb = min(kWave, my_steps - bstart);
      auto step_t0 = [&](int kk) { return live_t0(ts + (bstart + kk) * NTS); };
      auto step_base = [&](int kk, const _Float16* pool) { return pool + tok_row(rows, kk) * kHeadDim; };
      // DEPTH steps in flight per wave in its ring, one in registers. Order
      // of DMA issue: K(k+DEPTH) right after K(k) is read, V(k+DEPTH) right
      // after V(k) is read, so before reading a half-step exactly 2*DEPTH-1
      // newer half-steps (8 operations each) may be outstanding. Indices
      // past the batch are clamped to its last step (a duplicate request
      // that hits in cache) to keep that count exact.
      const uint32_t ring_lds = lds_addr(ring);
      if (bstart > 0) {  // (the first batch's first steps were issued before Q staging)
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
          const int kd = min(d, nb - 1);
          dma_k<0, 8, CP>(step_base(kd, kpool), ring + d * kRingStage, lane);
          dma_v<0, 8, CP>(step_base(kd, vpool), ring + d * kRingStage + 8192, lane);
        }
      }
      constexpr int kWait = 8 * (2 * DEPTH - 1);
      auto stage = [&](int kk) { return (kk & (DEPTH - 1)) * kRingStage; };
      // Software pipeline: step k's PV runs while step k+1's softmax is
      // computed. Read order K(0), V(0), K(1), V(1), ... and the DMA after
      // each read are those of the plain loop, so the waits are the same.
      half4_t pb[RB];
      {
        KFrag kf;
        ring_read8<kWait, 64>(kf.k, ring_lds + stage(0) + k_lane_off(lane));
        dma_k<0, 8, CP>(step_base(min(DEPTH, nb - 1), kpool), ring + stage(0), lane);
        step_scores<RB>(kf, qa, ws, pb, lane, step_t0(0), mk);
      }
      auto body = [&](int kk, auto masked) {
        constexpr bool MASKED = decltype(masked)::value;
        const int t0 = step_t0(kk);
        const int st = stage(kk), st1 = stage(kk + 1);
        VFrag vf;
        ring_read_vt<kWait>(vf, ring_lds + st + 8192 + v_lane_off(lane), lane);
        dma_v<0, 8, CP>(step_base(min(kk + DEPTH, nb - 1), vpool), ring + st + 8192, lane);
        KFrag kf;
        ring_read8_acc<kWait, 64>(kf.k, ring_lds + st1 + k_lane_off(lane));
        dma_k<0, 8, CP>(step_base(min(kk + 1 + DEPTH, nb - 1), kpool), ring + st1, lane);
        float x[RB][4], lmx[RB], alpha[RB], lsum[RB];
        scores_mfma<RB>(kf, qa, x);
        // (a step before the wave's last of the batch ends below kv_len)
        step_pv<RB, false>(vf, pb, ws, lane, t0, kv);
        // (masking without the skip test, and the softmax kept ahead of the
        // rare branch: both keep the softmax in the block of the step's
        // matrix ops, where the scheduler interleaves the two; the FP8 loop
        // above, whose vector work already fills that time, keeps the test,
        // which measured faster there)
        bool any;
        if constexpr (MASKED) any = mask_check<RB, WIN, false>(x, lmx, ws, mk, lane, step_t0(kk + 1));
        else any = max_check<RB>(x, lmx, ws);
        softmax_p<RB>(x, ws, lsum, pb);
        pin_softmax<RB>(pb, lsum);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) alpha[rb] = 1.f;
        if (any) {
          move_ref<RB>(lmx, ws, alpha);
          softmax_p<RB>(x, ws, lsum, pb);
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) ws.l[rb] = ws.l[rb] * alpha[rb] + lsum[rb];
        if (any) rescale_o<RB>(ws, alpha);
      };
      // Full attention: only the wave's last steps (the causal diagonal and
      // the tail) can need masking; the iterations before them (whose next
      // step ends at or below every row's limit) run without it.
      int kk = 0, clean = 0;
      if constexpr (!WIN) {
        const int span = mk.lim_min - kStep - step_t0(1);
        clean = span < 0 ? 0 : min(nb - 1, span / (kStep * NTS) + 1);
      }
      for (; kk < clean; ++kk) body(kk, std::false_type{});
      for (; kk + 1 < nb; ++kk) body(kk, std::true_type{});
      {
        VFrag vf;
        ring_read_vt<kWait>(vf, ring_lds + stage(nb - 1) + 8192 + v_lane_off(lane), lane);
        step_pv<RB>(vf, pb, ws, lane, step_t0(nb - 1), kv);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
  }

  // ---- combine the waves of each row group --------------------------------
  const int lo = lane & 15, hi = lane >> 4;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float lr = ws.l[rb];
    lr += __shfl_xor(lr, 16);
    lr += __shfl_xor(lr, 32);
    if (hi == 0) {
      s_m[ts][rowbase + rb * 16 + lo] = ws.m[rb];
      s_l[ts][rowbase + rb * 16 + lo] = lr;
    }
  }
  if (flag_bits) atomicOr(&s_flag, flag_bits);
  __syncthreads();  // every wave is past its main loop: Q and ring space may be reused

  float lse_row[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = rowbase + rb * 16 + lo;
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < NTS; ++k) M = fmaxf(M, s_m[k][row]);
    const float Mref = (M == -INFINITY) ? 0.f : M;
    float Ls = 0.f;
#pragma unroll
    for (int k = 0; k < NTS; ++k) Ls += s_l[k][row] * exp2_fast(s_m[k][row] - Mref);
    const float f = Ls > 0.f ? exp2_fast(ws.m[rb] - Mref) / Ls : 0.f;
    lse_row[rb] = Ls > 0.f ? (Mref + log2f(Ls)) * kLn2 : -INFINITY;
#pragma unroll
    for (int j = 0; j < 16; ++j) ws.o[rb][j] *= f;
  }

  float* obuf = reinterpret_cast<float*>(bigsm);
  // Round r: wave w adds its quarter (w + r) mod 4 of the channels into the
  // buffer (round 0 writes it), so every round has all four waves at work on
  // disjoint quarters; each wave issues its quarter's LDS reads before the
  // adds and writes.
  static_assert(NTS == 4, "four waves, four channel quarters");
  auto put = [&](auto qc, bool add) {
    constexpr int Q = decltype(qc)::value;
    constexpr int N = RB * 4;  // float4 pieces of one quarter per lane
    float4 val[N];
    float4* dst[N];
    int n = 0;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float* rowp = obuf + (rowbase + rb * 16 + lo) * kRowStride;
      // O^T block j of lane (hi, lo) holds channel rows 4*hi + i of row lo:
      // fp16 KV block j is channels 16j + 4*hi + i (blocks 8h + 2i and
      // 8h + 2i + 1 fill channels of quarter 2h + i/2);
      // FP8 KV block j = 4bb + c is channels 64bb + 4*(4*hi+i) + c (blocks
      // 8h .. 8h + 3 of quarter 2h, blocks 8h + 4 .. 8h + 7 of quarter 2h + 1)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (FP8) {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              if (2 * h + e == Q) {
                const int j = 8 * h + 4 * e;
                val[n] = make_float4(ws.o[rb][j][i], ws.o[rb][j + 1][i], ws.o[rb][j + 2][i], ws.o[rb][j + 3][i]);
                dst[n++] = reinterpret_cast<float4*>(rowp + 64 * Q + 16 * hi + 4 * i);
              }
            }
          } else {
            if (2 * h + i / 2 == Q) {
#pragma unroll
              for (int e = 0; e < 2; ++e) {
                const int j = 8 * h + 2 * i + e;
                val[n] = make_float4(ws.o[rb][j][0], ws.o[rb][j][1], ws.o[rb][j][2], ws.o[rb][j][3]);
                dst[n++] = reinterpret_cast<float4*>(rowp + 16 * j + 4 * hi);
              }
            }
          }
        }
      }
    }
    if (add) {
      float4 old[N];
#pragma unroll
      for (int k = 0; k < N; ++k) old[k] = *dst[k];
#pragma unroll
      for (int k = 0; k < N; ++k)
        *dst[k] = make_float4(old[k].x + val[k].x, old[k].y + val[k].y, old[k].z + val[k].z, old[k].w + val[k].w);
    } else {
#pragma unroll
      for (int k = 0; k < N; ++k) *dst[k] = val[k];
    }
  };
  for (int r = 0; r < NTS; ++r) {
    const int q = (ts + r) & 3;
    const bool add = r > 0;
    if (q == 0) put(std::integral_constant<int, 0>{}, add);
    else if (q == 1) put(std::integral_constant<int, 1>{}, add);
    else if (q == 2) put(std::integral_constant<int, 2>{}, add);
    else put(std::integral_constant<int, 3>{}, add);
    __syncthreads();
  }

  // lse of each row (one writer per row)
  if (ts == 0 && hi == 0) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int r = growbase + rb * 16 + lo;
      if (r < R) {
        const int i = r / G, j = r % G;
        const size_t orow = (size_t)(rstart + i) * Hq + g * G + j;
        if (direct) {
          if (a.out_lse) a.out_lse[orow] = lse_row[rb];
        } else {
          a.part_lse[split * split_stride + orow] = lse_row[rb];
        }
      }
    }
  }
  // rows out: 32 threads per row, 8 channels per thread
  const int rows_here = min(R - row0, RB * 16);
  for (int lr = tid / 32; lr < rows_here; lr += kThreads / 32) {
    const int r = row0 + lr;
    const int d0 = (tid % 32) * 8;
    const float* src = obuf + lr * kRowStride + d0;
    const float4 v0 = *reinterpret_cast<const float4*>(src);
    const float4 v1 = *reinterpret_cast<const float4*>(src + 4);
    const int i = r / G, j = r % G;
    const size_t orow = (size_t)(rstart + i) * Hq + g * G + j;
    if (direct) {
      half8_t hv = {(_Float16)v0.x, (_Float16)v0.y, (_Float16)v0.z, (_Float16)v0.w,
                    (_Float16)v1.x, (_Float16)v1.y, (_Float16)v1.z, (_Float16)v1.w};
      *reinterpret_cast<half8_t*>(a.out + orow * kHeadDim + d0) = hv;
    } else {
      float* dst = a.part_o + (split * split_stride + orow) * kHeadDim + d0;
      reinterpret_cast<float4*>(dst)[0] = v0;
      reinterpret_cast<float4*>(dst)[1] = v1;
    }
  }
  if (tid == 0 && s_flag && a.flags) atomicOr(a.flags, s_flag);
}

template <bool FP8, int DEPTH, bool WIN, int CP>
void launch_rb(const AttnArgs& a, int rb, dim3 grid, hipStream_t s) {
  const dim3 block(kThreads);
  if (rb == 1 && DEPTH == 1) hipLaunchKernelGGL((verify_attn_kernel<1, FP8, 1, WIN, false, CP>), grid, block, 0, s, a);
  else if (rb == 2) hipLaunchKernelGGL((verify_attn_kernel<2, FP8, DEPTH, WIN, false, CP>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((verify_attn_kernel<3, FP8, DEPTH, WIN, false, CP>), grid, block, 0, s, a);
}

// claimed work: fp16 KV, full attention, one row tile, blocks of one width;
// taken for long requests only (at least 32K keys per KV head), whose keys
// are read once
void launch_claim(const AttnArgs& a, int rb, hipStream_t s) {
  const dim3 grid(a.units), block(kThreads);
  constexpr int CP = kCacheStream;
  if (rb == 1) hipLaunchKernelGGL((verify_attn_kernel<1, false, 1, false, true, CP>), grid, block, 0, s, a);
  else if (rb == 2) hipLaunchKernelGGL((verify_attn_kernel<2, false, 1, false, true, CP>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((verify_attn_kernel<3, false, 1, false, true, CP>), grid, block, 0, s, a);
}

template <bool FP8, bool WIN>
void launch_depth(const AttnArgs& a, int rb, bool stream_once, hipStream_t s) {
  // one workgroup per unit; with n row tiles, 8n ids per 8 units, and the
  // workgroups on the same keys (rb is then 2 or 3) keep two steps in flight
  if (a.row_blocks > 1)
    launch_rb<FP8, 2, WIN, kCacheDefault>(a, rb, dim3(a.row_blocks * ((a.units + 7) / 8 * 8)), s);
  else if (stream_once)
    launch_rb<FP8, 1, WIN, kCacheStream>(a, rb, dim3(a.units), s);
  else
    launch_rb<FP8, 1, WIN, kCacheDefault>(a, rb, dim3(a.units), s);
}

void launch_verify_attention(const AttnArgs& a, int rb, bool fp8, bool claim, bool stream_once, hipStream_t s) {
  const bool win = a.window > 0;
  if (claim) {
    launch_claim(a, rb, s);
  } else if (fp8) {
    if (win) launch_depth<true, true>(a, rb, stream_once, s);
    else launch_depth<true, false>(a, rb, stream_once, s);
  } else {
    if (win) launch_depth<false, true>(a, rb, stream_once, s);
    else launch_depth<false, false>(a, rb, stream_once, s);
  }
}

}  // namespace sv
