// Paged causal GQA of a speculative verify block with 49 to 96 rows per KV
// head (a 16-token block over 6 query heads per KV head is 96 rows), fp16 KV,
// one workgroup per (key chunk, KV head, request). Taken for large passes
// (every K/V byte read once, non-temporally); verify_attn_kernel covers the
// rest, with two workgroups of 48 rows that share the keys through L2 for
// such blocks.
//
// The four waves are two row halves times two step parities. Round q holds
// steps 2q and 2q + 1 of the chunk; wave (h, p) computes the scores of step
// 2q + p for rows 48h .. 48h+47 (RB row blocks of 16), and accumulates
// O^T for the same rows but only channels 128p .. 128p+127, over both steps
// of every round: the two waves of a row half hand each other their P^T
// fragments through LDS, and each runs the PV of the round's two steps as one
// 16x16x32 matrix op per (row block, channel block). K-slots 0..3 of lane
// group g are step 2q's tokens 4g..4g+3 and slots 4..7 step 2q+1's, in both
// operands, so every lane's fragments keep the layout of the 16-token step
// (the matrix op sums over the k-slots in any order).
//
// The two waves of a row half share one online-softmax reference per row:
// each publishes its lanes' maxima of its step (4 tokens a lane), and in the
// next round each lane tests its own maximum with the partner's of the same
// lane, so both waves see the same values and take the same decision (the
// lazy rule of verify_attn_kernel); their P^T fragments are then at one
// reference, and their O^T halves and sums need no rescale when combined. Pipeline: the scores of round q, the
// reference and P of round q - 1, and the PV of round q - 2 run in round q.
// K and V pass through rings that all four waves share (K: 3 rounds, V: 5),
// two rounds in flight; each wave issues the copies of one half-step (K or V
// of its parity's step) two rounds ahead, and one barrier per round hands
// stages between the copies and the readers.
#include <type_traits>

#include "verify_frag.h"

namespace sv {

constexpr int kRowsKRounds = 3, kRowsVRounds = 5;     // 48 KB of K and 80 KB of V in LDS
constexpr int kRowsRound = 2 * 8192;                  // K (or V) of a round's two steps
constexpr int kRowsMaxSteps = kRowsMaxChunk / kStep;  // steps per chunk: cache rows held in LDS

namespace {

__device__ __forceinline__ uint32_t lds_read_u32(uint32_t addr) {
  uint32_t v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
  return v;
}

// V^T fragments of one step for channel blocks 8p .. 8p+7 (addr includes the
// 256p bytes of the half), as ring_read_vt.
template <int VMCNT>
__device__ __forceinline__ void ring_read_vt_half(u32x2 (&v)[8], uint32_t addr, int lane) {
  const uint32_t r32 = 32u * (uint32_t)((lane >> 2) & 3);
  const uint32_t b0 = addr + (0u ^ r32), b1 = addr + (32u ^ r32), b2 = addr + (64u ^ r32), b3 = addr + (96u ^ r32);
  asm volatile(
      "s_waitcnt vmcnt(%12)\n\t"
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %9\n\t"
      "ds_read_b64_tr_b16 %2, %10\n\t"
      "ds_read_b64_tr_b16 %3, %11\n\t"
      "ds_read_b64_tr_b16 %4, %8 offset:128\n\t"
      "ds_read_b64_tr_b16 %5, %9 offset:128\n\t"
      "ds_read_b64_tr_b16 %6, %10 offset:128\n\t"
      "ds_read_b64_tr_b16 %7, %11 offset:128\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
      : "v"(b0), "v"(b1), "v"(b2), "v"(b3), "n"(VMCNT)
      : "memory");
}

// The same for two steps (addresses a and b) with one wait.
template <int VMCNT>
__device__ __forceinline__ void ring_read_vt_pair(u32x2 (&va)[8], u32x2 (&vb)[8], uint32_t a, uint32_t b, int lane) {
  const uint32_t r32 = 32u * (uint32_t)((lane >> 2) & 3);
  const uint32_t a0 = a + (0u ^ r32), a1 = a + (32u ^ r32), a2 = a + (64u ^ r32), a3 = a + (96u ^ r32);
  const uint32_t b0 = b + (0u ^ r32), b1 = b + (32u ^ r32), b2 = b + (64u ^ r32), b3 = b + (96u ^ r32);
  asm volatile(
      "s_waitcnt vmcnt(%24)\n\t"
      "ds_read_b64_tr_b16 %0, %16\n\t"
      "ds_read_b64_tr_b16 %1, %17\n\t"
      "ds_read_b64_tr_b16 %2, %18\n\t"
      "ds_read_b64_tr_b16 %3, %19\n\t"
      "ds_read_b64_tr_b16 %4, %16 offset:128\n\t"
      "ds_read_b64_tr_b16 %5, %17 offset:128\n\t"
      "ds_read_b64_tr_b16 %6, %18 offset:128\n\t"
      "ds_read_b64_tr_b16 %7, %19 offset:128\n\t"
      "ds_read_b64_tr_b16 %8, %20\n\t"
      "ds_read_b64_tr_b16 %9, %21\n\t"
      "ds_read_b64_tr_b16 %10, %22\n\t"
      "ds_read_b64_tr_b16 %11, %23\n\t"
      "ds_read_b64_tr_b16 %12, %20 offset:128\n\t"
      "ds_read_b64_tr_b16 %13, %21 offset:128\n\t"
      "ds_read_b64_tr_b16 %14, %22 offset:128\n\t"
      "ds_read_b64_tr_b16 %15, %23 offset:128\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(va[0]), "=&v"(va[1]), "=&v"(va[2]), "=&v"(va[3]), "=&v"(va[4]), "=&v"(va[5]), "=&v"(va[6]),
        "=&v"(va[7]), "=&v"(vb[0]), "=&v"(vb[1]), "=&v"(vb[2]), "=&v"(vb[3]), "=&v"(vb[4]), "=&v"(vb[5]),
        "=&v"(vb[6]), "=&v"(vb[7])
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3), "v"(b0), "v"(b1), "v"(b2), "v"(b3), "n"(VMCNT)
      : "memory");
}

// Keys at or past kv_len may be poison in a page's unused slots: clear the V
// values of those tokens (their weight is 0, but 0 * NaN is NaN).
__device__ __forceinline__ void clear_tail(u32x2 (&v)[8], int lane, int t0, int kv) {
  if (t0 + kStep <= kv) return;
  const int tok = t0 + 4 * (lane >> 4);
  const uint32_t m0 = (tok + 0 < kv ? 0x0000ffffu : 0u) | (tok + 1 < kv ? 0xffff0000u : 0u);
  const uint32_t m1 = (tok + 2 < kv ? 0x0000ffffu : 0u) | (tok + 3 < kv ? 0xffff0000u : 0u);
#pragma unroll
  for (int cb = 0; cb < 8; ++cb) {
    v[cb].x &= m0;
    v[cb].y &= m1;
  }
}

// The copies of one half-step, K (is_v false: dma_k's layout) or V (dma_v's),
// with the lane offsets selected rather than branched on.
template <int CP>
__device__ __forceinline__ void dma_half(const _Float16* base, char* ring, int lane, bool is_v) {
  const __amdgpu_buffer_rsrc_t r = half_step_rsrc(base);
  uint32_t ek, ok, ev, ov;
  k_copy_offsets(lane, &ek, &ok);
  v_copy_offsets(lane, &ev, &ov);
  const uint32_t even = is_v ? ev : ek, odd = is_v ? ov : ok;
  dma_block<0, CP>(r, ring, even);
  dma_block<1, CP>(r, ring, odd);
  dma_block<2, CP>(r, ring, even);
  dma_block<3, CP>(r, ring, odd);
  dma_block<4, CP>(r, ring, even);
  dma_block<5, CP>(r, ring, odd);
  dma_block<6, CP>(r, ring, even);
  dma_block<7, CP>(r, ring, odd);
}

// O^T += V^T . P^T over a round's two steps (A, B) for one channel half.
template <int RB>
__device__ __forceinline__ void pair_pv(const u32x2 (&va)[8], const u32x2 (&vb)[8], const half4_t (&pa)[RB],
                                        const half4_t (&pb)[RB], floatx4 (&o)[RB][8]) {
  u32x4 bop[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const u32x2 x = __builtin_bit_cast(u32x2, pa[rb]), y = __builtin_bit_cast(u32x2, pb[rb]);
    bop[rb] = u32x4{x.x, x.y, y.x, y.y};
  }
#pragma unroll
  for (int cb = 0; cb < 8; ++cb) {
    const u32x4 aop = {va[cb].x, va[cb].y, vb[cb].x, vb[cb].y};
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) o[rb][cb] = mfma_16x16x32(aop, bop[rb], o[rb][cb]);
  }
}

}  // namespace

template <int RB, bool WIN>
__global__ __launch_bounds__(kThreads, 1) void verify_rows_kernel(AttnArgs a) {
  static_assert(RB == 2 || RB == 3, "row halves of 32 or 48 rows");
  static_assert(kWavesPerGroup == 4, "two row halves times two step parities");
  constexpr int HR = RB * 16;  // rows per half
  constexpr int KR = kRowsKRounds, VR = kRowsVRounds;
  // at round r (after its barrier) round r + 2 is issued into the K stage of
  // round r - 1 and the V stage of round r - 3, both read before barrier r
  static_assert(KR == 3 && VR == 5, "two rounds in flight");
  constexpr int CP = kCacheStream;  // (a large pass, each K/V byte read by one workgroup)
  __shared__ __attribute__((aligned(1024))) unsigned char ring[(KR + VR) * kRowsRound];
  __shared__ uint32_t s_rows[kRowsMaxSteps];
  __shared__ float s_lm[2][kWavesPerGroup][RB][kWave];    // lane maxima of a round's steps (by round parity)
  __shared__ u32x2 s_p[2][kWavesPerGroup][RB][kWave];     // P^T fragments of a round's steps (by round parity)
  __shared__ float s_l[kWavesPerGroup][HR];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int h = wave & 1, p = wave >> 1;  // row half, step parity (and channel half)
  const int partner = wave ^ 2;           // the other parity of the same row half
  // workgroup -> (key chunk, KV head, request), as in verify_attn_kernel
  const int unit = blockIdx.x;
  int split, g, b;
  if (a.batch > 1 && a.batch <= kWave) {
    if (!ordered_unit<WIN>(a, unit, lane, unit == 0 && tid < kWave, &split, &b, &g)) return;
  } else {
    const int hb = unit % (a.num_kv_heads * a.batch);
    split = unit / (a.num_kv_heads * a.batch);
    g = hb % a.num_kv_heads;
    b = hb / a.num_kv_heads;
  }
  int flag_bits = 0;
  int q_len = a.q_len, rstart = b * a.q_len;
  if (a.q_start) {
    q_len = block_rows(a.q_start, b, a.batch, a.q_len, &rstart, &flag_bits);
    if (q_len == 0) {
      if (flag_bits && tid == 0 && a.flags) atomicOr(a.flags, flag_bits);
      return;
    }
  }
  const int G = a.group, R = q_len * G, Hq = a.num_q_heads;
  const size_t split_stride = (size_t)a.batch * a.q_len * Hq;
  const int hrow = h * HR;  // the wave's first row (of the KV head's q_len*G, at most 2*HR)

  // the wave's Q fragments (score matrix op k-step s: channels 32s + 8*(lane/16))
  u32x4 qa[RB][8];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = hrow + rb * 16 + (lane & 15);
    const _Float16* src = a.q;
    if (r < R) src = a.q + ((size_t)(rstart + r / G) * Hq + g * G + r % G) * kHeadDim + 8 * (lane >> 4);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (r < R) v = *reinterpret_cast<const u32x4*>(src + 32 * s);
      qa[rb][s] = v;
    }
  }

  const int raw_kv = __builtin_amdgcn_readfirstlane(a.kv_lens[b]);
  const int kv = clamp_kv_len(raw_kv, a.max_kv_len, a.max_pages, a.page_size, &flag_bits);
  if (raw_kv < q_len) flag_bits |= 0x2;
  const int L = kv - q_len;
  const int W = a.window, S = a.sink;
  int n_sink = 0, w0 = 0;
  const int total = WIN ? live_steps(kv, L, W, S, &n_sink, &w0) : (kv > 0 ? (kv + kStep - 1) / kStep : 0);
  const int cs = a.chunk / kStep;
  const int n_chunks = total > 0 ? (total + cs - 1) / cs : 1;
  if (split >= n_chunks) return;  // whole group: nothing of this request here
  const bool direct = n_chunks == 1;
  const int k_base = __builtin_amdgcn_readfirstlane(split * cs);
  const int n = __builtin_amdgcn_readfirstlane(min(total - k_base, cs) > 0 ? min(total - k_base, cs) : 0);
  auto live_t0 = [&](int j) {
    const int k = k_base + j;
    if constexpr (!WIN) return kStep * k;
    return k < n_sink ? kStep * k : w0 + kStep * (k - n_sink);
  };

  // cache row ((page, KV head, slot); the pool holds fewer than 2^32 rows) of
  // the first token of each of the chunk's steps
  const int P = a.page_size, Hkv = a.num_kv_heads;
  const int32_t* ptab = a.page_table + (size_t)b * a.max_pages;
  for (int s = tid; s < n; s += kThreads) {
    const int t = live_t0(s);
    int pid = ptab[t / P];
    if (pid < 0 || pid >= a.num_pages) {
      flag_bits |= 0x4;
      pid = 0;
    }
    s_rows[s] = ((uint32_t)pid * (uint32_t)Hkv + (uint32_t)g) * (uint32_t)P + (uint32_t)(t % P);
  }

  // the keys each of this lane's rows sees (as in verify_attn_kernel)
  RowMask<RB, WIN> mk;
  mk.sink = S;
  int lmin = INT32_MAX, lmax = INT32_MIN;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = hrow + rb * 16 + (lane & 15);
    mk.lim[rb] = r < R ? min(L + r / G + 1, kv) : kv;
    mk.lo[rb] = r < R ? L + r / G + 1 - W : INT32_MIN;
    lmin = min(lmin, mk.lim[rb]);
    lmax = max(lmax, mk.lo[rb]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    lmin = min(lmin, __shfl_xor(lmin, o));
    lmax = max(lmax, __shfl_xor(lmax, o));
  }
  mk.lim_min = __builtin_amdgcn_readfirstlane(lmin);
  mk.lo_max = __builtin_amdgcn_readfirstlane(lmax);
  // (also completes the Q loads, so no later wait on them drains the DMAs)
  __syncthreads();

  const _Float16* kpool = static_cast<const _Float16*>(a.k_pages);
  const _Float16* vpool = static_cast<const _Float16*>(a.v_pages);
  const uint32_t ring_lds = lds_addr(ring), rows_lds = lds_addr(s_rows);
  // Round q's steps 2q and 2q + 1: K in K stage q mod KR, V in V stage q mod
  // VR (8 KB per step). Wave (h, p) issues the copies of half-step (h, p) of
  // round q: K (h = 0) or V (h = 1) of step 2q + p, 8 operations.
  auto issues = [&](int q) { return q >= 0 && 2 * q + p < n; };
  const _Float16* const half_pool = h == 0 ? kpool : vpool;
  const int half_stage0 = h == 0 ? 0 : KR;
  const int half_stages = h == 0 ? KR : VR;
  auto issue_step = [&](int q, int j) {
    const size_t tr = (size_t)__builtin_amdgcn_readfirstlane((int)lds_read_u32(rows_lds + 4u * (uint32_t)j));
    char* const rg = reinterpret_cast<char*>(ring);
    dma_half<CP>(half_pool + tr * kHeadDim, rg + (half_stage0 + q % half_stages) * kRowsRound + p * 8192, lane,
                 h != 0);
  };
  auto issue = [&](int q) { issue_step(q, 2 * q + p); };
  const int rounds = (n + 1) / 2;
  // Barrier r (one per round, r = 0 .. rounds + 1) is passed once every
  // wave's copies of round r have landed; after it, round r + 2 is issued.
  for (int q = 0; q < 2; ++q)
    if (issues(q)) issue(q);
  auto round_barrier = [&](int r) {
    // this wave's copies of round r have landed (those of round r + 1 may be
    // out, 8 operations; near the end there are none, so wait for all)
    if (issues(r + 1)) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    // (and this wave's LDS writes of the row maxima and P^T are done, its
    // LDS reads of the partner's returned)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (issues(r + 2)) issue(r + 2);
  };
  // Steady rounds: every wave has round r + 1 out, and round r + 2 is always
  // issued, its step clamped to the chunk's last (a re-fetch of that step
  // into a stage no later round reads), so the wait count is exact without
  // a branch.
  auto steady_barrier = [&](int r) {
    asm volatile("s_waitcnt vmcnt(8)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    issue_step(r + 2, min(2 * (r + 2) + p, n - 1));
  };
  // LDS addresses of step j's K and V
  auto k_of = [&](int j) { return ring_lds + (uint32_t)(((j >> 1) % KR) * kRowsRound + (j & 1) * 8192); };
  auto v_of = [&](int j) { return ring_lds + (uint32_t)((KR + (j >> 1) % VR) * kRowsRound + (j & 1) * 8192); };
  const uint32_t vlo = v_lane_off(lane) + 256u * (uint32_t)p;

  floatx4 o[RB][8];
  float m[RB], l[RB];
  const float c = a.scale_log2;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m[rb] = -INFINITY;
    l[rb] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) o[rb][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  const int lo = lane & 15, hi = lane >> 4;
  float x[RB][4];    // raw scores of this wave's step of the previous round
  float lown[RB];    // and each lane's maximum of them
  half4_t pown[RB];  // this wave's P^T of the round before that (at the shared reference)
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    lown[rb] = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) x[rb][i] = -INFINITY;
  }

  // The shared reference and P^T of this wave's step of round q, from its
  // raw scores x, its lane maxima lown and the partner's lane maxima lpar of
  // the same lanes (the same rows). The partner calls this with the two
  // maxima swapped, so both see the same values and take the same decisions.
  // Common case: no lane's pair exceeds the reference by more than kLazyLog2
  // and nothing moves; otherwise the row's maximum over its four lanes
  // becomes its reference, and O and l are rescaled.
  auto shared_softmax = [&](int q, const float (&lpar)[RB]) {
    float pm[RB], lsum[RB];
    half4_t pnew[RB];
    bool bump = false;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      pm[rb] = fmaxf(lown[rb], lpar[rb]);
      bump = bump | (pm[rb] * c > m[rb] + kLazyLog2);
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float ref = (m[rb] == -INFINITY) ? 0.f : m[rb];
      float pv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pv[i] = exp2_fast(__builtin_fmaf(x[rb][i], c, -ref));
      lsum[rb] = (pv[0] + pv[1]) + (pv[2] + pv[3]);
      pnew[rb] = half4_t{(_Float16)pv[0], (_Float16)pv[1], (_Float16)pv[2], (_Float16)pv[3]};
    }
    pin_softmax<RB>(pnew, lsum);
    if (__any(bump)) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        float mx = pm[rb];
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        mx *= c;
        const bool bb = mx > m[rb] + kLazyLog2;
        const float mnew = bb ? mx : m[rb];
        const float alpha = bb ? exp2_fast(m[rb] - mnew) : 1.f;  // m = -inf -> 0
        m[rb] = mnew;
        l[rb] *= alpha;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) scale_acc(o[rb][jj], alpha);
        const float ref = (m[rb] == -INFINITY) ? 0.f : m[rb];
        float pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pv[i] = exp2_fast(__builtin_fmaf(x[rb][i], c, -ref));
        lsum[rb] = (pv[0] + pv[1]) + (pv[2] + pv[3]);
        pnew[rb] = half4_t{(_Float16)pv[0], (_Float16)pv[1], (_Float16)pv[2], (_Float16)pv[3]};
      }
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      l[rb] += lsum[rb];
      pown[rb] = pnew[rb];
      s_p[q & 1][wave][rb][lane] = __builtin_bit_cast(u32x2, pnew[rb]);
    }
  };
  // this wave's step of round r: scores in xn, lane maxima published
  auto publish_max = [&](int r, const float (&xn)[RB][4]) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float mx = fmaxf(fmaxf(xn[rb][0], xn[rb][1]), fmaxf(xn[rb][2], xn[rb][3]));
      s_lm[r & 1][wave][rb][lane] = mx;
      lown[rb] = mx;
#pragma unroll
      for (int i = 0; i < 4; ++i) x[rb][i] = xn[rb][i];
    }
  };

  // A round in general form: any round, any step count (the pipeline's
  // first two and last three rounds).
  auto general = [&](int r) {
    round_barrier(r);
    const int k = 2 * r + p;  // this wave's step of round r
    // (1) PV of round r - 2 (both steps, this wave's channel half)
    if (r >= 2) {
      const int q = r - 2, kA = 2 * q, kB = 2 * q + 1;
      half4_t pother[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) pother[rb] = __builtin_bit_cast(half4_t, s_p[q & 1][partner][rb][lane]);
      u32x2 va[8], vb[8];
      ring_read_vt_half<63>(va, v_of(kA) + vlo, lane);
      clear_tail(va, lane, live_t0(kA), kv);
      if (kB < n) {
        ring_read_vt_half<63>(vb, v_of(kB) + vlo, lane);
        clear_tail(vb, lane, live_t0(kB), kv);
      } else {
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) vb[cb] = u32x2{0u, 0u};
      }
      if (p == 0) pair_pv<RB>(va, vb, pown, pother, o);
      else pair_pv<RB>(va, vb, pother, pown, o);
    }
    // (2) the shared reference and P^T of round r - 1
    if (r >= 1 && r <= rounds) {
      float lpar[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) lpar[rb] = s_lm[(r - 1) & 1][partner][rb][lane];
      shared_softmax(r - 1, lpar);
    }
    // (3) scores of round r
    if (r < rounds) {
      float xn[RB][4];
      if (k < n) {
        KFrag kf;
        ring_read8<63, 64>(kf.k, k_of(k) + k_lane_off(lane));
        scores_mfma<RB>(kf, qa, xn);
        apply_mask<RB, WIN>(xn, mk, lane, live_t0(k));
      } else {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int i = 0; i < 4; ++i) xn[rb][i] = -INFINITY;
      }
      publish_max(r, xn);
    }
  };

  // A steady round (2 <= r < rounds - 1): this wave's step exists, both steps
  // of round r - 2 exist and end below kv, so the round is one basic block
  // apart from the rare reference move: the partner's P^T and lane maxima
  // (read first, their latency under the ring reads), the ring reads, the
  // score matrix ops of round r and the PV matrix ops of round r - 2, the
  // softmax of round r - 1 beside them, then the masking and lane maxima of
  // round r.
  auto steady = [&](int r, auto masked) {
    constexpr bool MASKED = decltype(masked)::value;
    steady_barrier(r);
    const int k = 2 * r + p, q2 = r - 2, q1 = r - 1;
    half4_t pother[RB];
    float lpar[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      pother[rb] = __builtin_bit_cast(half4_t, s_p[q2 & 1][partner][rb][lane]);
      lpar[rb] = s_lm[q1 & 1][partner][rb][lane];
    }
    KFrag kf;
    ring_read8<63, 64>(kf.k, k_of(k) + k_lane_off(lane));
    u32x2 va[8], vb[8];
    ring_read_vt_pair<63>(va, vb, v_of(2 * q2) + vlo, v_of(2 * q2 + 1) + vlo, lane);
    half4_t pa[RB], pbb[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      pa[rb] = p == 0 ? pown[rb] : pother[rb];
      pbb[rb] = p == 0 ? pother[rb] : pown[rb];
    }
    float xn[RB][4];
    scores_mfma<RB>(kf, qa, xn);
    pair_pv<RB>(va, vb, pa, pbb, o);
    shared_softmax(q1, lpar);
    if constexpr (MASKED) apply_mask<RB, WIN, false>(xn, mk, lane, live_t0(k));
    publish_max(r, xn);
  };
  const int steady_end = rounds - 1;  // rounds 2 .. steady_end - 1 are steady
  int r = 0;
  for (; r < 2 && r < rounds + 2; ++r) general(r);
  // full attention: the steady rounds whose step ends at or below every
  // row's limit run without masking
  int clean = r;
  if constexpr (!WIN) {
    const int span = mk.lim_min - kStep - kStep * (k_base + p);
    clean = span < 0 ? r : max(r, min(steady_end, span / (2 * kStep) + 1));
  }
  for (; r < clean; ++r) steady(r, std::false_type{});
  for (; r < steady_end; ++r) steady(r, std::true_type{});
  for (; r < rounds + 2; ++r) general(r);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- the two waves of a row half: sums, then each writes its channel half
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float lr = l[rb];
    lr += __shfl_xor(lr, 16);
    lr += __shfl_xor(lr, 32);
    if (hi == 0) s_l[wave][rb * 16 + lo] = lr;
  }
  __syncthreads();
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = hrow + rb * 16 + lo;
    const float Ls = s_l[wave][rb * 16 + lo] + s_l[partner][rb * 16 + lo];
    const float Mref = (m[rb] == -INFINITY) ? 0.f : m[rb];
    const float f = Ls > 0.f ? 1.f / Ls : 0.f;
    const float lse = Ls > 0.f ? (Mref + log2f(Ls)) * kLn2 : -INFINITY;
    if (r < R) {
      const size_t orow = (size_t)(rstart + r / G) * Hq + g * G + r % G;
      if (p == 0 && hi == 0) {
        if (direct) {
          if (a.out_lse) a.out_lse[orow] = lse;
        } else {
          a.part_lse[split * split_stride + orow] = lse;
        }
      }
      // accumulator j of lane (hi, lo) holds channels 16 (8p + j) + 4 hi .. +3 of row lo
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int ch = 16 * (8 * p + j) + 4 * hi;
        const floatx4 v = o[rb][j];
        if (direct) {
          half4_t hv = {(_Float16)(v[0] * f), (_Float16)(v[1] * f), (_Float16)(v[2] * f), (_Float16)(v[3] * f)};
          *reinterpret_cast<half4_t*>(a.out + orow * kHeadDim + ch) = hv;
        } else {
          float* dst = a.part_o + (split * split_stride + orow) * kHeadDim + ch;
          *reinterpret_cast<float4*>(dst) = make_float4(v[0] * f, v[1] * f, v[2] * f, v[3] * f);
        }
      }
    }
  }
  if (flag_bits && a.flags) atomicOr(a.flags, flag_bits);
}

void launch_verify_rows(const AttnArgs& a, int rb, hipStream_t s) {
  const dim3 grid(a.units), block(kThreads);
  if (a.window > 0) {
    if (rb == 2) hipLaunchKernelGGL((verify_rows_kernel<2, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((verify_rows_kernel<3, true>), grid, block, 0, s, a);
  } else {
    if (rb == 2) hipLaunchKernelGGL((verify_rows_kernel<2, false>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((verify_rows_kernel<3, false>), grid, block, 0, s, a);
  }
}

}  // namespace sv
