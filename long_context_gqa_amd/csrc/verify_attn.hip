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

#include "sv_common.h"

namespace sv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

namespace {

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLazyLog2 = 8.f;  // largest p = 256 between rescales

__device__ __forceinline__ floatx4 mfma_16x16x32(const u32x4& a, const u32x4& b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ floatx4 mfma_16x16x16(uint32_t a0, uint32_t a1, const half4_t& b,
                                                 floatx4 c) {
  u32x2 av = {a0, a1};
  return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(half4_t, av), b, c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// K and V of one 16-token step held by a wave: 8 x 16 B of each per lane.
struct KFrag {
  u32x4 k[8];  // k[s]: token lane%16, channels 32s + 8*(lane/16) .. +8
};
struct VFrag {
  u32x2 v[16];  // v[cb]: channel 16cb + lane%16 of tokens 4*(lane/16) + 0..3 (the PV A operand)
};

// Multiply one accumulator tuple by a per-lane factor in place. Done in
// inline asm on the accumulation registers themselves, so the compiler does
// not keep shadow copies of all accumulators in ordinary registers for the
// (rarely taken) rescale branch.
__device__ __forceinline__ void scale_acc(floatx4& acc, float f) {
  float e0 = acc[0], e1 = acc[1], e2 = acc[2], e3 = acc[3];
  float t;
  asm volatile(
      "v_accvgpr_read_b32 %4, %0\n\t"
      "v_mul_f32 %4, %5, %4\n\t"
      "v_accvgpr_write_b32 %0, %4\n\t"
      "v_accvgpr_read_b32 %4, %1\n\t"
      "v_mul_f32 %4, %5, %4\n\t"
      "v_accvgpr_write_b32 %1, %4\n\t"
      "v_accvgpr_read_b32 %4, %2\n\t"
      "v_mul_f32 %4, %5, %4\n\t"
      "v_accvgpr_write_b32 %2, %4\n\t"
      "v_accvgpr_read_b32 %4, %3\n\t"
      "v_mul_f32 %4, %5, %4\n\t"
      "v_accvgpr_write_b32 %3, %4"
      : "+a"(e0), "+a"(e1), "+a"(e2), "+a"(e3), "=&v"(t)
      : "v"(f));
  acc = floatx4{e0, e1, e2, e3};
}

template <int RB>
struct WaveState {
  floatx4 o[RB][16];  // O^T accumulators: block j, rows of this lane
  float m[RB];        // reference (log2 units, >= every score seen - 8) of row lane%16
  float l[RB];        // this lane's share of the running sum
};

// The keys each of a lane's rows sees: t < lim (causal and tail limit) and,
// with a sliding window (WIN), t >= lo or t < sink (the leading sink
// positions). Full attention compiles without the window terms.
template <int RB, bool WIN>
struct RowMask {
  int lim[RB];
  int lo[RB];
  int sink;
  int lim_min;  // smallest lim over the wave's rows (wave-uniform)
  int lo_max;   // largest lo over the wave's rows (wave-uniform)
};

// Masking of one step's scores (lane holds tokens t0 + 4*(lane/16) + i of row
// lane%16 in each row block), without branches.
template <int RB, bool WIN>
__device__ __forceinline__ void apply_mask(float (&x)[RB][4], const RowMask<RB, WIN>& mk, int lane, int t0) {
  // a step wholly below every row's limit (and, with a window, above every
  // row's lower edge) needs no masking: a wave-uniform test
  if (t0 + kStep <= mk.lim_min && (!WIN || t0 >= mk.lo_max)) return;
  const int tok = t0 + 4 * (lane >> 4);
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = tok + i;
      if constexpr (WIN)
        x[rb][i] = (t >= mk.lim[rb] || (t < mk.lo[rb] && t >= mk.sink)) ? -INFINITY : x[rb][i];
      else
        x[rb][i] = t >= mk.lim[rb] ? -INFINITY : x[rb][i];
    }
}

// Online-softmax update of one step from the scaled scores x (log2 units):
// masking, the lazy reference, the running sum, and p.
template <int RB, bool WIN>
__device__ __forceinline__ void softmax_step(float (&x)[RB][4], WaveState<RB>& ws, float (&p)[RB][4],
                                             int lane, int t0, const RowMask<RB, WIN>& mk) {
  apply_mask<RB>(x, mk, lane, t0);
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float mx = fmaxf(fmaxf(x[rb][0], x[rb][1]), fmaxf(x[rb][2], x[rb][3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // Lazy reference: the row's reference m only moves when the tile max
    // exceeds it by more than kLazyLog2, so p = 2^(x - m) <= 2^kLazyLog2 stays
    // well inside fp16 and the O/l rescale (64*RB accumulators) is rare.
    // Numerator and denominator share the reference, so the result is the
    // same softmax.
    const bool bump = mx > ws.m[rb] + kLazyLog2;
    if (__any(bump)) {
      const float mnew = bump ? mx : ws.m[rb];
      const float alpha = bump ? exp2_fast(ws.m[rb] - mnew) : 1.f;  // m = -inf -> 0
      ws.l[rb] *= alpha;
#pragma unroll
      for (int j = 0; j < 16; ++j) scale_acc(ws.o[rb][j], alpha);
      ws.m[rb] = mnew;
    }
    const float ref = (ws.m[rb] == -INFINITY) ? 0.f : ws.m[rb];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[rb][i] = exp2_fast(x[rb][i] - ref);
    ws.l[rb] += (p[rb][0] + p[rb][1]) + (p[rb][2] + p[rb][3]);
  }
}

// The scaled scores of one fp16 step: per row block, the 8 k-steps of the
// score matrix ops on the K fragments and the wave's Q fragments (held in
// registers for the whole loop), in two independent chains.
template <int RB>
__device__ __forceinline__ void scores_mfma(const KFrag& kf, const u32x4 (&qa)[RB][8], float scale_log2,
                                            float (&x)[RB][4]) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    floatx4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 8; s += 2) {
      a0 = mfma_16x16x32(kf.k[s], qa[rb][s], a0);
      a1 = mfma_16x16x32(kf.k[s + 1], qa[rb][s + 1], a1);
    }
    const floatx4 acc = a0 + a1;
#pragma unroll
    for (int i = 0; i < 4; ++i) x[rb][i] = acc[i] * scale_log2;
  }
}

// Scores of one fp16 step and the fp16 P^T fragments.
template <int RB, bool WIN>
__device__ __forceinline__ void step_scores(const KFrag& kf, const u32x4 (&qa)[RB][8], WaveState<RB>& ws,
                                            half4_t (&pb)[RB], int lane, int t0, const RowMask<RB, WIN>& mk,
                                            float scale_log2) {
  float x[RB][4];
  scores_mfma<RB>(kf, qa, scale_log2, x);
  float p[RB][4];
  softmax_step<RB>(x, ws, p, lane, t0, mk);
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
    pb[rb] = half4_t{(_Float16)p[rb][0], (_Float16)p[rb][1], (_Float16)p[rb][2], (_Float16)p[rb][3]};
}

// The pieces of one step for the software-pipelined fp16 loop, where the PV
// matrix ops of step k are issued right after the score matrix ops of step
// k+1, and the softmax of k+1 fills their shadow:
//   scores_mfma   the scaled scores of step k+1 (Q fragments in registers);
//   mask_check    causal/tail masking without branches (per-row limits are
//                 computed once), each lane's own max, and whether any lane
//                 needs its row's reference moved;
//   move_ref      (rare) the row max across the row's four lanes and the new
//                 reference; alpha is the factor O and l must take;
//   softmax_p     p at the current reference, its sum, and the fp16 P^T
//                 fragments (computed before the branch, so they overlap the
//                 matrix ops; redone after a move);
//   rescale_o     (rare) O *= alpha, after step k's PV was accumulated at the
//                 old reference.
template <int RB, bool WIN>
__device__ __forceinline__ bool mask_check(float (&x)[RB][4], float (&lmx)[RB], const WaveState<RB>& ws,
                                           const RowMask<RB, WIN>& mk, int lane, int t0) {
  apply_mask<RB>(x, mk, lane, t0);
  bool bump = false;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    lmx[rb] = fmaxf(fmaxf(x[rb][0], x[rb][1]), fmaxf(x[rb][2], x[rb][3]));
    bump = bump || (lmx[rb] > ws.m[rb] + kLazyLog2);
  }
  return __any(bump);
}

template <int RB>
__device__ __forceinline__ void move_ref(const float (&lmx)[RB], WaveState<RB>& ws, float (&alpha)[RB]) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float mx = lmx[rb];
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const bool bump = mx > ws.m[rb] + kLazyLog2;
    const float mnew = bump ? mx : ws.m[rb];
    alpha[rb] = bump ? exp2_fast(ws.m[rb] - mnew) : 1.f;  // m = -inf -> 0
    ws.m[rb] = mnew;
  }
}

template <int RB>
__device__ __forceinline__ void softmax_p(const float (&x)[RB][4], const WaveState<RB>& ws, float (&lsum)[RB],
                                          half4_t (&pb)[RB]) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float ref = (ws.m[rb] == -INFINITY) ? 0.f : ws.m[rb];
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = exp2_fast(x[rb][i] - ref);
    lsum[rb] = (p[0] + p[1]) + (p[2] + p[3]);
    pb[rb] = half4_t{(_Float16)p[0], (_Float16)p[1], (_Float16)p[2], (_Float16)p[3]};
  }
}

template <int RB>
__device__ __forceinline__ void rescale_o(WaveState<RB>& ws, const float (&alpha)[RB]) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int j = 0; j < 16; ++j) scale_acc(ws.o[rb][j], alpha[rb]);
}

// ---- FP8 E4M3 steps -------------------------------------------------------
//
// E4M3 bytes become fp16 with the packed hardware conversion at scale 1.0:
// every finite E4M3 value is an fp16 value (subnormals included), so the
// conversion is exact; the per-block scales are applied outside the MFMAs in
// fp32. Lanes see the pair (byte 0, byte 1) with word_sel false and (byte 2,
// byte 3) with word_sel true, low byte in the low half.
__device__ __forceinline__ uint32_t e4m3x2_lo(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
}
__device__ __forceinline__ uint32_t e4m3x2_hi(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true));
}
// Interleave two words bytewise: {a.0, b.0, a.1, b.1} and {a.2, b.2, a.3, b.3}
// (v_perm: selectors 0-3 take the second operand's bytes, 4-7 the first's).
__device__ __forceinline__ uint32_t zip_lo(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05010400u); }
__device__ __forceinline__ uint32_t zip_hi(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07030602u); }

// One FP8 step held by a wave.
//   k[b]  : token lane%16, bytes 64b + 16*(lane/16) .. +16 (the 64-channel scale
//           block b; MFMA k-steps 2b and 2b+1 take its halves)
//   v[4e+bb]: token 4*(lane/16)+e, bytes 64bb + 4*(lane%16) .. +4
//   sk[], sv[]: fp16 scales of tokens 4*(lane/16)+i, blocks 0..3 (i-major)
struct KFrag8 {
  u32x4 k[4];
  u32x4 sk[2];
  u32x4 sv[2];
};
struct VFrag8 {
  uint32_t v[16];
};

__device__ __forceinline__ float half_at(const u32x4 (&h)[2], int idx) {
  const uint32_t w = h[idx >> 3][(idx >> 1) & 3];
  const uint16_t bits = (idx & 1) ? (uint16_t)(w >> 16) : (uint16_t)(w & 0xFFFFu);
  return (float)__builtin_bit_cast(_Float16, bits);
}

// O^T += V^T . P^T for one FP8 step: MFMA block j = 4*bb + c holds channels
// 64*bb + 4*(lane%16) + c, all inside scale block bb, so the V scale is folded
// into P^T once per block group and V is used exactly. P^T arrives in fp16
// (as for fp16 KV); each token pair's P is multiplied by its pair of V scales
// with one packed fp16 multiply.
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
template <int RB, bool MASK = true>
__device__ __forceinline__ void step_pv8(VFrag8& vf, const u32x4 (&sv)[2], const half4_t (&ph)[RB],
                                         WaveState<RB>& ws, int lane, int t0, int kv) {
  const int hi = lane >> 4;
  // V scales of tokens (0, 1) and (2, 3) of the lane's group, per block bb,
  // as half pairs: the scale of token i, block bb is half 4i + bb of sv
  // (dword 2i + bb/2, low half for even bb)
  uint32_t s01[4], s23[4];
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) {
    const uint32_t sel = (bb & 1) ? 0x07060302u : 0x05040100u;
    const int d = bb >> 1;
    s01[bb] = __builtin_amdgcn_perm(sv[0][2 + d], sv[0][d], sel);
    s23[bb] = __builtin_amdgcn_perm(sv[1][2 + d], sv[1][d], sel);
  }
  // Keys at or past kv_len: weight 0; their (poison) scales must not enter
  // and their bytes may decode to NaN (0 * NaN is NaN), so clear both.
  if (MASK && t0 + kStep > kv) {
    const int tok = t0 + 4 * hi;
    const uint32_t m01 = (tok + 0 < kv ? 0x0000ffffu : 0u) | (tok + 1 < kv ? 0xffff0000u : 0u);
    const uint32_t m23 = (tok + 2 < kv ? 0x0000ffffu : 0u) | (tok + 3 < kv ? 0xffff0000u : 0u);
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
      s01[bb] &= m01;
      s23[bb] &= m23;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (tok + i >= kv) {
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) vf.v[4 * i + bb] = 0u;
      }
  }
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) {
    half4_t pb[RB];
    const half2_t a01 = __builtin_bit_cast(half2_t, s01[bb]), a23 = __builtin_bit_cast(half2_t, s23[bb]);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const half2_t q01 = half2_t{ph[rb][0], ph[rb][1]} * a01;
      const half2_t q23 = half2_t{ph[rb][2], ph[rb][3]} * a23;
      pb[rb] = half4_t{q01[0], q01[1], q23[0], q23[1]};
    }
    // tokens (0, 1) and (2, 3) of the lane's group, byte c of block bb, as
    // fp16 pairs: A operand halves of channel 64*bb + 4*(lane%16) + c
    const uint32_t z01l = zip_lo(vf.v[bb], vf.v[4 + bb]), z01h = zip_hi(vf.v[bb], vf.v[4 + bb]);
    const uint32_t z23l = zip_lo(vf.v[8 + bb], vf.v[12 + bb]), z23h = zip_hi(vf.v[8 + bb], vf.v[12 + bb]);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t w01 = c < 2 ? z01l : z01h, w23 = c < 2 ? z23l : z23h;
      const uint32_t a0 = (c & 1) ? e4m3x2_hi(w01) : e4m3x2_lo(w01);
      const uint32_t a1 = (c & 1) ? e4m3x2_hi(w23) : e4m3x2_lo(w23);
      const int j = 4 * bb + c;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) ws.o[rb][j] = mfma_16x16x16(a0, a1, pb[rb], ws.o[rb][j]);
    }
  }
}

// O^T += V^T . P^T for one step: matrix op cb covers channels 16cb..16cb+15,
// and its accumulator holds channels 16cb + 4*(lane/16) + i of row lane%16.
template <int RB, bool MASK = true>
__device__ __forceinline__ void step_pv(VFrag& vf, const half4_t (&pb)[RB], WaveState<RB>& ws,
                                        int lane, int t0, int kv) {
  // Keys at or past kv_len may be poison in the page's unused slots; their
  // weight is exactly 0 but 0 * NaN is NaN, so clear those V values.
  if (MASK && t0 + kStep > kv) {
    const int tok = t0 + 4 * (lane >> 4);
    const uint32_t m0 = (tok + 0 < kv ? 0x0000ffffu : 0u) | (tok + 1 < kv ? 0xffff0000u : 0u);
    const uint32_t m1 = (tok + 2 < kv ? 0x0000ffffu : 0u) | (tok + 3 < kv ? 0xffff0000u : 0u);
#pragma unroll
    for (int cb = 0; cb < 16; ++cb) {
      vf.v[cb].x &= m0;
      vf.v[cb].y &= m1;
    }
  }
#pragma unroll
  for (int cb = 0; cb < 16; ++cb)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) ws.o[rb][cb] = mfma_16x16x16(vf.v[cb].x, vf.v[cb].y, pb[rb], ws.o[rb][cb]);
}

}  // namespace

// LDS addresses are 32-bit; the ring is read with inline-asm ds_read_b128 so
// that the compiler does not drain every outstanding DMA before each read
// (it cannot tell which DMA a read depends on); the waits are explicit.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) char*)(p));
}

#define SV_GP(p) ((__attribute__((address_space(1))) void*)(p))
#define SV_LP(p) ((__attribute__((address_space(3))) void*)(p))

// Outputs are early-clobber: a destination must not share a register with
// the address, which later reads of the same block still use while earlier
// ones may already have returned.
// Eight 16-byte reads at addr, addr + STRIDE, ..., addr + 7*STRIDE after
// waiting until at most VMCNT of this wave's vector-memory operations (the
// newer half-steps) are outstanding, i.e. until the block's own DMA has
// landed.
template <int VMCNT, int STRIDE>
__device__ __forceinline__ void ring_read8(u32x4 (&d)[8], uint32_t addr) {
  asm volatile(
      "s_waitcnt vmcnt(%9)\n\t"
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %8 offset:%10\n\t"
      "ds_read_b128 %2, %8 offset:%11\n\t"
      "ds_read_b128 %3, %8 offset:%12\n\t"
      "ds_read_b128 %4, %8 offset:%13\n\t"
      "ds_read_b128 %5, %8 offset:%14\n\t"
      "ds_read_b128 %6, %8 offset:%15\n\t"
      "ds_read_b128 %7, %8 offset:%16\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(d[0]), "=&v"(d[1]), "=&v"(d[2]), "=&v"(d[3]), "=&v"(d[4]), "=&v"(d[5]), "=&v"(d[6]), "=&v"(d[7])
      : "v"(addr), "n"(VMCNT), "n"(STRIDE), "n"(2 * STRIDE), "n"(3 * STRIDE), "n"(4 * STRIDE),
        "n"(5 * STRIDE), "n"(6 * STRIDE), "n"(7 * STRIDE)
      : "memory");
}

// Direct HBM -> LDS copies of 1 KB blocks [B0, B1) of one half-step; block j
// is tokens 2j and 2j+1 of the (page, KV head) run, read contiguously (lane l
// lands at ring + j*1024 + 16*l). V is stored as is: token t, 16-byte chunk c
// at t*512 + 16c. K's chunks are permuted inside each token row: chunk c of
// token t sits at position c ^ (t & 3), so that the MFMA operand reads (lane =
// token t, chunk 4s + lane/16) of 16 lanes spread over the LDS banks.
template <int B0, int B1>
__device__ __forceinline__ void dma_k(const _Float16* kb, char* ring, int lane) {
#pragma unroll
  for (int j = B0; j < B1; ++j) {
    const int t = 2 * j + (lane >> 5);
    const int c = (lane & 31) ^ (t & 3);
    __builtin_amdgcn_global_load_lds(SV_GP(kb + t * kHeadDim + 8 * c), SV_LP(ring + j * 1024), 16, 0, 0);
  }
}
template <int B0, int B1>
__device__ __forceinline__ void dma_v(const _Float16* vb, char* ring, int lane) {
#pragma unroll
  for (int j = B0; j < B1; ++j) {
    const int t = 2 * j + (lane >> 5);
    const int c = (lane & 31) ^ (2 * (t & 3));
    __builtin_amdgcn_global_load_lds(SV_GP(vb + t * kHeadDim + 8 * c), SV_LP(ring + j * 1024), 16, 0, 0);
  }
}
// The same read into accumulation registers: for fragments that only feed
// matrix ops (which read A/B operands from them), keeping them out of the
// ordinary register file.
template <int VMCNT, int STRIDE>
__device__ __forceinline__ void ring_read8_acc(u32x4 (&d)[8], uint32_t addr) {
  asm volatile(
      "s_waitcnt vmcnt(%9)\n\t"
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %8 offset:%10\n\t"
      "ds_read_b128 %2, %8 offset:%11\n\t"
      "ds_read_b128 %3, %8 offset:%12\n\t"
      "ds_read_b128 %4, %8 offset:%13\n\t"
      "ds_read_b128 %5, %8 offset:%14\n\t"
      "ds_read_b128 %6, %8 offset:%15\n\t"
      "ds_read_b128 %7, %8 offset:%16\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&a"(d[0]), "=&a"(d[1]), "=&a"(d[2]), "=&a"(d[3]), "=&a"(d[4]), "=&a"(d[5]), "=&a"(d[6]), "=&a"(d[7])
      : "v"(addr), "n"(VMCNT), "n"(STRIDE), "n"(2 * STRIDE), "n"(3 * STRIDE), "n"(4 * STRIDE),
        "n"(5 * STRIDE), "n"(6 * STRIDE), "n"(7 * STRIDE)
      : "memory");
}
// Per-lane ring offsets of the operand reads. K: lane (token l%16, group
// l/16) reads k-step s at k_lane_off + 64*s.
__device__ __forceinline__ uint32_t k_lane_off(int lane) {
  const int t = lane & 15, g = lane >> 4;
  return t * 512 + 16 * (g ^ (t & 3));
}

// V^T fragments of one step by transposing LDS reads. ds_read_b64_tr_b16
// works on groups of 16 lanes: lane i of a group receives, as its element r,
// the 16-bit element i%4 of the 8 bytes that lane 4r + i/4 of the group
// addresses (pinned with a probe on the GPU). Lane 4r + q of group g
// addresses token 4g + r, channels 16cb + 4q .. +3, so lane i receives
// channel 16cb + i of tokens 4g + 0..3: the A operand of the PV matrix op.
// V rows are stored with the 32-byte window of channel block cb of token t at
// window cb ^ (t & 3) (dma_v), so a group's four rows fall in different
// banks; window cb ^ r = 4*(cb/4) + ((cb%4) ^ r) gives four per-lane bases
// (cb%4 = 0..3) and an immediate offset of 128*(cb/4). VMCNT as in
// ring_read8.
__device__ __forceinline__ uint32_t v_lane_off(int lane) {
  const int g = lane >> 4, r = (lane >> 2) & 3, q = lane & 3;
  return (4 * g + r) * 512 + 8 * q;
}
template <int VMCNT>
__device__ __forceinline__ void ring_read_vt(VFrag& f, uint32_t addr, int lane) {
  const uint32_t r32 = 32u * (uint32_t)((lane >> 2) & 3);
  const uint32_t b0 = addr + (0u ^ r32), b1 = addr + (32u ^ r32), b2 = addr + (64u ^ r32), b3 = addr + (96u ^ r32);
  asm volatile(
      "s_waitcnt vmcnt(%20)\n\t"
      "ds_read_b64_tr_b16 %0, %16\n\t"
      "ds_read_b64_tr_b16 %1, %17\n\t"
      "ds_read_b64_tr_b16 %2, %18\n\t"
      "ds_read_b64_tr_b16 %3, %19\n\t"
      "ds_read_b64_tr_b16 %4, %16 offset:128\n\t"
      "ds_read_b64_tr_b16 %5, %17 offset:128\n\t"
      "ds_read_b64_tr_b16 %6, %18 offset:128\n\t"
      "ds_read_b64_tr_b16 %7, %19 offset:128\n\t"
      "ds_read_b64_tr_b16 %8, %16 offset:256\n\t"
      "ds_read_b64_tr_b16 %9, %17 offset:256\n\t"
      "ds_read_b64_tr_b16 %10, %18 offset:256\n\t"
      "ds_read_b64_tr_b16 %11, %19 offset:256\n\t"
      "ds_read_b64_tr_b16 %12, %16 offset:384\n\t"
      "ds_read_b64_tr_b16 %13, %17 offset:384\n\t"
      "ds_read_b64_tr_b16 %14, %18 offset:384\n\t"
      "ds_read_b64_tr_b16 %15, %19 offset:384\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(f.v[0]), "=&v"(f.v[1]), "=&v"(f.v[2]), "=&v"(f.v[3]), "=&v"(f.v[4]), "=&v"(f.v[5]),
        "=&v"(f.v[6]), "=&v"(f.v[7]), "=&v"(f.v[8]), "=&v"(f.v[9]), "=&v"(f.v[10]), "=&v"(f.v[11]),
        "=&v"(f.v[12]), "=&v"(f.v[13]), "=&v"(f.v[14]), "=&v"(f.v[15])
      : "v"(b0), "v"(b1), "v"(b2), "v"(b3), "n"(VMCNT)
      : "memory");
}

// FP8 ring stage: K bytes (4 KB), V bytes (4 KB), the step's K and V scales
// (2 x 128 B, padded to 256).
constexpr int kStage8 = 8448;

// K half-step of an FP8 step: 4 blocks of 1 KB, block j = tokens 4j..4j+3
// read contiguously, chunk c (16 bytes) of token t at position c ^ (t & 3);
// plus one 256-byte block holding the 16 tokens' K scales (lanes 0..31) and
// V scales (lanes 32..63).
__device__ __forceinline__ void dma_k8(const uint8_t* kb, const _Float16* ksb, const _Float16* vsb,
                                       char* stage, int lane) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = 4 * j + (lane >> 4);
    const int c = (lane & 15) ^ (t & 3);
    __builtin_amdgcn_global_load_lds(SV_GP(kb + t * kHeadDim + 16 * c), SV_LP(stage + j * 1024), 16, 0, 0);
  }
  const _Float16* ssrc = lane < 32 ? ksb + 2 * lane : vsb + 2 * (lane - 32);
  __builtin_amdgcn_global_load_lds(SV_GP(ssrc), SV_LP(stage + 8192), 4, 0, 0);
}
// V half-step of an FP8 step: the 4 KB of 16 tokens copied as is.
__device__ __forceinline__ void dma_v8(const uint8_t* vb, char* stage, int lane) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
    __builtin_amdgcn_global_load_lds(SV_GP(vb + (j * kWave + lane) * 16), SV_LP(stage + 4096 + j * 1024), 16,
                                     0, 0);
}
// Per-lane offsets: K block bk (bytes 64bk + 16*(l/16) of token l%16) at
// k8_lane_off + 64*bk; V dword 4e+bb (bytes 64bb + 4*(l%16) of token
// 4*(l/16)+e) at v8_lane_off + 64*(4e+bb).
__device__ __forceinline__ uint32_t k8_lane_off(int lane) {
  const int t = lane & 15, g = lane >> 4;
  return t * 256 + 16 * (g ^ (t & 3));
}
__device__ __forceinline__ uint32_t v8_lane_off(int lane) { return (lane >> 4) * 1024 + (lane & 15) * 4; }

template <int VMCNT>
__device__ __forceinline__ void ring_read_k8(KFrag8& f, uint32_t addr_lane, uint32_t addr_scale) {
  asm volatile(
      "s_waitcnt vmcnt(%10)\n\t"
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %8 offset:64\n\t"
      "ds_read_b128 %2, %8 offset:128\n\t"
      "ds_read_b128 %3, %8 offset:192\n\t"
      "ds_read_b128 %4, %9\n\t"
      "ds_read_b128 %5, %9 offset:16\n\t"
      "ds_read_b128 %6, %9 offset:128\n\t"
      "ds_read_b128 %7, %9 offset:144\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(f.k[0]), "=&v"(f.k[1]), "=&v"(f.k[2]), "=&v"(f.k[3]), "=&v"(f.sk[0]), "=&v"(f.sk[1]),
        "=&v"(f.sv[0]), "=&v"(f.sv[1])
      : "v"(addr_lane), "v"(addr_scale), "n"(VMCNT)
      : "memory");
}

template <int VMCNT>
__device__ __forceinline__ void ring_read_v8(VFrag8& f, uint32_t addr) {
  asm volatile(
      "s_waitcnt vmcnt(%17)\n\t"
      "ds_read_b32 %0, %16\n\t"
      "ds_read_b32 %1, %16 offset:64\n\t"
      "ds_read_b32 %2, %16 offset:128\n\t"
      "ds_read_b32 %3, %16 offset:192\n\t"
      "ds_read_b32 %4, %16 offset:256\n\t"
      "ds_read_b32 %5, %16 offset:320\n\t"
      "ds_read_b32 %6, %16 offset:384\n\t"
      "ds_read_b32 %7, %16 offset:448\n\t"
      "ds_read_b32 %8, %16 offset:512\n\t"
      "ds_read_b32 %9, %16 offset:576\n\t"
      "ds_read_b32 %10, %16 offset:640\n\t"
      "ds_read_b32 %11, %16 offset:704\n\t"
      "ds_read_b32 %12, %16 offset:768\n\t"
      "ds_read_b32 %13, %16 offset:832\n\t"
      "ds_read_b32 %14, %16 offset:896\n\t"
      "ds_read_b32 %15, %16 offset:960\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(f.v[0]), "=&v"(f.v[1]), "=&v"(f.v[2]), "=&v"(f.v[3]), "=&v"(f.v[4]), "=&v"(f.v[5]),
        "=&v"(f.v[6]), "=&v"(f.v[7]), "=&v"(f.v[8]), "=&v"(f.v[9]), "=&v"(f.v[10]), "=&v"(f.v[11]),
        "=&v"(f.v[12]), "=&v"(f.v[13]), "=&v"(f.v[14]), "=&v"(f.v[15])
      : "v"(addr), "n"(VMCNT)
      : "memory");
}

// The scaled scores of one FP8 step: per 64-channel block, two matrix ops
// on the converted K and the wave's Q fragments (in registers), one
// accumulator per (row block, scale block) so the block scales are applied
// after all matrix ops are issued: S = sum_b scale_b * partial_b, one
// multiply and three fused multiply-adds per score, the softmax scale applied
// once at the end.
template <int RB>
__device__ __forceinline__ void scores8_mfma(const KFrag8& kf, const u32x4 (&qa)[RB][8], float scale_log2,
                                             float (&x)[RB][4]) {
  u32x4 kc[8];
#pragma unroll
  for (int bk = 0; bk < 4; ++bk) {
    kc[2 * bk] = u32x4{e4m3x2_lo(kf.k[bk][0]), e4m3x2_hi(kf.k[bk][0]), e4m3x2_lo(kf.k[bk][1]),
                       e4m3x2_hi(kf.k[bk][1])};
    kc[2 * bk + 1] = u32x4{e4m3x2_lo(kf.k[bk][2]), e4m3x2_hi(kf.k[bk][2]), e4m3x2_lo(kf.k[bk][3]),
                           e4m3x2_hi(kf.k[bk][3])};
  }
  floatx4 acc[RB][4];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int bk = 0; bk < 4; ++bk) {
      acc[rb][bk] = mfma_16x16x32(kc[2 * bk], qa[rb][2 * bk], floatx4{0.f, 0.f, 0.f, 0.f});
      acc[rb][bk] = mfma_16x16x32(kc[2 * bk + 1], qa[rb][2 * bk + 1], acc[rb][bk]);
    }
  }
  float fk[4][4];  // [token i][block]
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int bk = 0; bk < 4; ++bk) fk[i][bk] = half_at(kf.sk, 4 * i + bk);
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float t = fk[i][0] * acc[rb][0][i];
      t = __builtin_fmaf(fk[i][1], acc[rb][1][i], t);
      t = __builtin_fmaf(fk[i][2], acc[rb][2][i], t);
      t = __builtin_fmaf(fk[i][3], acc[rb][3][i], t);
      x[rb][i] = t * scale_log2;
    }
}

constexpr int kRingStage = 16384;  // K (8 KB) + V (8 KB) of one step
// DEPTH steps in flight per wave in its private ring. One (64 KB per CU over
// the four waves) saturates HBM when every workgroup streams its own keys; a
// second step measured slower there. When several workgroups (row tiles)
// read the same keys (more than 48 rows per KV head) they share one HBM
// stream, and two steps each keep as many HBM bytes in flight as one step
// does unshared.

// Dispatch order for a batch of 2..64 requests (one request per lane of the
// wave; every wave computes the same answer): item u of the grid is the
// u-th of all full chunks in split-major order, then the partial last
// chunks, longest first, then nothing. Workgroups start in item order, so
// the uneven pieces of a ragged batch go last and the largest of them
// first (longest-processing-time order); a uniform batch keeps the
// split-major order. A request with rows but no visible key keeps one
// (empty) chunk, which writes its rows and flags; a request without rows (a
// width of 0, or a bad one) has none, so item 0 reports the bad widths.
// Returns false for an item without work.
template <bool WIN>
__device__ bool ordered_unit(const AttnArgs& a, int u, int lane, bool report, int* split, int* b, int* g) {
  const int cs = a.chunk / kStep, Hkv = a.num_kv_heads;
  int tb = 0;          // this lane's request: live 16-token steps
  bool rows = false;   // ... and whether it has rows
  if (lane < a.batch) {
    int fl = 0, st = 0;
    const int q = a.q_start ? block_rows(a.q_start, lane, a.batch, a.q_len, &st, &fl) : a.q_len;
    if (report && (fl & 0x8) && a.flags) atomicOr(a.flags, 0x8);
    fl = 0;
    const int kv = clamp_kv_len(a.kv_lens[lane], a.max_kv_len, a.max_pages, a.page_size, &fl);
    rows = q > 0;
    if (rows) {
      int ns, w0;
      tb = WIN ? live_steps(kv, kv - q, a.window, a.sink, &ns, &w0) : (kv + kStep - 1) / kStep;
    }
  }
  // full chunks, and the last (partial or empty) chunk if any: its length
  const int full = tb / cs, part = tb % cs;
  const bool has_part = part > 0 || (rows && tb == 0);
  int i = u;
  for (int s = 0;; ++s) {
    const uint64_t m = __ballot(full > s);
    if (!m) break;
    const int n = __popcll(m) * Hkv;
    if (i < n) {
      const int j = i / Hkv;
      const int rank = __popcll(m & ((1ull << lane) - 1ull));
      *split = s;
      *b = __builtin_ctzll(__ballot(full > s && rank == j));
      *g = i % Hkv;
      return true;
    }
    i -= n;
  }
  const uint64_t pm = __ballot(has_part);
  if (i >= __popcll(pm) * Hkv) return false;
  int rank = 0;  // among the last chunks: longer first, then lower request
  for (int o = 0; o < a.batch; ++o) {
    const int po = __shfl(part, o);
    const bool ho = (pm >> o) & 1ull;
    rank += (ho && (po > part || (po == part && o < lane))) ? 1 : 0;
  }
  const int bb = __builtin_ctzll(__ballot(has_part && rank == i / Hkv));
  *b = bb;
  *g = i % Hkv;
  *split = __shfl(full, bb);
  return true;
}

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

template <int RB, bool FP8, int DEPTH, bool WIN, bool CLAIM>
__global__ __launch_bounds__(kThreads, 1) void verify_attn_kernel(AttnArgs a) {
  static_assert(DEPTH == 1 || DEPTH == 2, "one or two steps in flight");
  static_assert(!CLAIM || (!FP8 && DEPTH == 1 && !WIN), "claimed work: fp16 KV, one step in flight, full attention");
  using SM = Smem<RB, FP8, DEPTH>;
  constexpr int NTS = kWavesPerGroup;  // waves that split the chunk's steps
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
        dma_k8(kpool8 + tr * kHeadDim, a.k_scales + tr * 4, a.v_scales + tr * 4, stage, lane);
        dma_v8(vpool8 + tr * kHeadDim, stage, lane);
      } else {
        dma_k<0, 8>(kpool + tr * kHeadDim, stage, lane);
        dma_v<0, 8>(vpool + tr * kHeadDim, stage + 8192, lane);
      }
    }
  }

  // the Q fragments (loaded above) into LDS
  u32x4* qlds = reinterpret_cast<u32x4*>(qsm);
#pragma unroll
  for (int k = 0; k < kQPer; ++k) qlds[tid + k * kThreads] = qv[k];
  __syncthreads();

  WaveState<RB> ws;
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
        dma_k8(kpool8 + tr * kHeadDim, a.k_scales + tr * 4, a.v_scales + tr * 4, ring + stg * kStage8, lane);
      };
      auto issue_v = [&](int kk, int stg) {
        dma_v8(vpool8 + tok_row(rows, kk) * kHeadDim, ring + stg * kStage8, lane);
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
        scores8_mfma<RB>(kf, qa, a.scale_log2, x0);
        softmax_step<RB>(x0, ws, p0, lane, step_t0(0), mk);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          pr[rb] = half4_t{(_Float16)p0[rb][0], (_Float16)p0[rb][1], (_Float16)p0[rb][2], (_Float16)p0[rb][3]};
        sv[0] = kf.sv[0];
        sv[1] = kf.sv[1];
      }
      for (int kk = 0; kk + 1 < nb; ++kk) {
        const int t0 = step_t0(kk);
        VFrag8 vf;
        ring_read_v8<kWaitV>(vf, sbase(kk) + 4096 + v8_lane_off(lane));
        issue_v(min(kk + DEPTH, nb - 1), kk & (DEPTH - 1));
        KFrag8 kf;
        ring_read_k8<kWaitK>(kf, sbase(kk + 1) + k8_lane_off(lane), sbase(kk + 1) + 8192 + 32 * (lane >> 4));
        issue_k(min(kk + 1 + DEPTH, nb - 1), (kk + 1) & (DEPTH - 1));
        float x[RB][4], lmx[RB], alpha[RB], lsum[RB];
        scores8_mfma<RB>(kf, qa, a.scale_log2, x);
        // (a step before the wave's last of the batch ends below kv_len)
        step_pv8<RB, false>(vf, sv, pr, ws, lane, t0, kv);
        sv[0] = kf.sv[0];
        sv[1] = kf.sv[1];
        const bool any = mask_check<RB>(x, lmx, ws, mk, lane, step_t0(kk + 1));
        softmax_p<RB>(x, ws, lsum, pr);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) alpha[rb] = 1.f;
        if (any) {
          move_ref<RB>(lmx, ws, alpha);
          softmax_p<RB>(x, ws, lsum, pr);
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) ws.l[rb] = ws.l[rb] * alpha[rb] + lsum[rb];
        if (any) rescale_o<RB>(ws, alpha);
      }
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
          dma_k<0, 8>(kpool + tgt(1) * kHeadDim, ring, lane);
          step_scores<RB>(kf, qa, ws, pb, lane, kStep * base, mk, a.scale_log2);
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
          dma_v<0, 8>(vpool + tgt(kk + 1) * kHeadDim, ring + 8192, lane);
          KFrag kf;
          // (two more operations are newer than K's DMAs after a first step)
          if (first)
            ring_read8_acc<kWait + 2, 64>(kf.k, ring_lds + k_lane_off(lane));
          else
            ring_read8_acc<kWait, 64>(kf.k, ring_lds + k_lane_off(lane));
          dma_k<0, 8>(kpool + tgt(kk + 2) * kHeadDim, ring, lane);
          float x[RB][4], lmx[RB], alpha[RB], lsum[RB];
          scores_mfma<RB>(kf, qa, a.scale_log2, x);
          // (only the stream's last step can end above kv_len)
          step_pv<RB, false>(vf, pb, ws, lane, t0, kv);
          const bool any = mask_check<RB>(x, lmx, ws, mk, lane, t1);
          softmax_p<RB>(x, ws, lsum, pb);
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
          dma_k<0, 8>(step_base(kd, kpool), ring + d * kRingStage, lane);
          dma_v<0, 8>(step_base(kd, vpool), ring + d * kRingStage + 8192, lane);
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
        dma_k<0, 8>(step_base(min(DEPTH, nb - 1), kpool), ring + stage(0), lane);
        step_scores<RB>(kf, qa, ws, pb, lane, step_t0(0), mk, a.scale_log2);
      }
      for (int kk = 0; kk + 1 < nb; ++kk) {
        const int t0 = step_t0(kk);
        const int st = stage(kk), st1 = stage(kk + 1);
        VFrag vf;
        ring_read_vt<kWait>(vf, ring_lds + st + 8192 + v_lane_off(lane), lane);
        dma_v<0, 8>(step_base(min(kk + DEPTH, nb - 1), vpool), ring + st + 8192, lane);
        KFrag kf;
        ring_read8_acc<kWait, 64>(kf.k, ring_lds + st1 + k_lane_off(lane));
        dma_k<0, 8>(step_base(min(kk + 1 + DEPTH, nb - 1), kpool), ring + st1, lane);
        float x[RB][4], lmx[RB], alpha[RB], lsum[RB];
        scores_mfma<RB>(kf, qa, a.scale_log2, x);
        // (a step before the wave's last of the batch ends below kv_len)
        step_pv<RB, false>(vf, pb, ws, lane, t0, kv);
        const bool any = mask_check<RB>(x, lmx, ws, mk, lane, step_t0(kk + 1));
        softmax_p<RB>(x, ws, lsum, pb);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) alpha[rb] = 1.f;
        if (any) {
          move_ref<RB>(lmx, ws, alpha);
          softmax_p<RB>(x, ws, lsum, pb);
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) ws.l[rb] = ws.l[rb] * alpha[rb] + lsum[rb];
        if (any) rescale_o<RB>(ws, alpha);
      }
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

template <bool FP8, int DEPTH, bool WIN>
void launch_rb(const AttnArgs& a, int rb, dim3 grid, hipStream_t s) {
  const dim3 block(kThreads);
  if (rb == 1 && DEPTH == 1) hipLaunchKernelGGL((verify_attn_kernel<1, FP8, 1, WIN, false>), grid, block, 0, s, a);
  else if (rb == 2) hipLaunchKernelGGL((verify_attn_kernel<2, FP8, DEPTH, WIN, false>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((verify_attn_kernel<3, FP8, DEPTH, WIN, false>), grid, block, 0, s, a);
}

// claimed work: fp16 KV, full attention, one row tile, blocks of one width
void launch_claim(const AttnArgs& a, int rb, hipStream_t s) {
  const dim3 grid(a.units), block(kThreads);
  if (rb == 1) hipLaunchKernelGGL((verify_attn_kernel<1, false, 1, false, true>), grid, block, 0, s, a);
  else if (rb == 2) hipLaunchKernelGGL((verify_attn_kernel<2, false, 1, false, true>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((verify_attn_kernel<3, false, 1, false, true>), grid, block, 0, s, a);
}

template <bool FP8, bool WIN>
void launch_depth(const AttnArgs& a, int rb, hipStream_t s) {
  // one workgroup per unit; with n row tiles, 8n ids per 8 units, and the
  // workgroups on the same keys (rb is then 2 or 3) keep two steps in flight
  if (a.row_blocks > 1)
    launch_rb<FP8, 2, WIN>(a, rb, dim3(a.row_blocks * ((a.units + 7) / 8 * 8)), s);
  else
    launch_rb<FP8, 1, WIN>(a, rb, dim3(a.units), s);
}

void launch_verify_attention(const AttnArgs& a, int rb, bool fp8, bool claim, hipStream_t s) {
  const bool win = a.window > 0;
  if (claim) {
    launch_claim(a, rb, s);
  } else if (fp8) {
    if (win) launch_depth<true, true>(a, rb, s);
    else launch_depth<true, false>(a, rb, s);
  } else {
    if (win) launch_depth<false, true>(a, rb, s);
    else launch_depth<false, false>(a, rb, s);
  }
}

}  // namespace sv
