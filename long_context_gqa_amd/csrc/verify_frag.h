// Device building blocks of the verify-attention kernels (internal header):
// matrix-op wrappers and fragment layouts, the online-softmax pieces, masking,
// the HBM -> LDS copies of K/V steps and their operand reads, and the
// dispatch order of batched requests. Included by verify_attn.hip and
// verify_rows.hip; the layouts are described where each piece is defined.
#pragma once

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
  float c;            // sm_scale * log2(e): a raw score q.k times c is in log2 units
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
// SKIP: test first whether the step needs masking at all (a branch, which
// also ends the scheduling region there); without it the selects always run.
template <int RB, bool WIN, bool SKIP = true>
__device__ __forceinline__ void apply_mask(float (&x)[RB][4], const RowMask<RB, WIN>& mk, int lane, int t0) {
  // a step wholly below every row's limit (and, with a window, above every
  // row's lower edge) needs no masking: a wave-uniform test
  if (SKIP && t0 + kStep <= mk.lim_min && (!WIN || t0 >= mk.lo_max)) return;
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

// Online-softmax update of one step from the raw scores x (q.k; x * c is in
// log2 units): masking, the lazy reference, the running sum, and p. The max
// is taken on raw scores (scaling by c > 0, rounded, keeps the order).
template <int RB, bool WIN>
__device__ __forceinline__ void softmax_step(float (&x)[RB][4], WaveState<RB>& ws, float (&p)[RB][4],
                                             int lane, int t0, const RowMask<RB, WIN>& mk) {
  apply_mask<RB>(x, mk, lane, t0);
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float mx = fmaxf(fmaxf(x[rb][0], x[rb][1]), fmaxf(x[rb][2], x[rb][3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    mx *= ws.c;
    // Lazy reference: the row's reference m only moves when the tile max
    // exceeds it by more than kLazyLog2, so p = 2^(x c - m) <= 2^kLazyLog2
    // stays well inside fp16 and the O/l rescale (64*RB accumulators) is
    // rare. Numerator and denominator share the reference, so the result is
    // the same softmax.
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
    for (int i = 0; i < 4; ++i) p[rb][i] = exp2_fast(__builtin_fmaf(x[rb][i], ws.c, -ref));
    ws.l[rb] += (p[rb][0] + p[rb][1]) + (p[rb][2] + p[rb][3]);
  }
}

// The raw scores of one fp16 step: per row block, the 8 k-steps of the
// score matrix ops on the K fragments and the wave's Q fragments (held in
// registers for the whole loop), one accumulation chain per row block (the
// row blocks' chains interleave).
template <int RB>
__device__ __forceinline__ void scores_mfma(const KFrag& kf, const u32x4 (&qa)[RB][8], float (&x)[RB][4]) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 8; ++s) acc = mfma_16x16x32(kf.k[s], qa[rb][s], acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[rb][i] = acc[i];
  }
}

// Scores of one fp16 step and the fp16 P^T fragments.
template <int RB, bool WIN>
__device__ __forceinline__ void step_scores(const KFrag& kf, const u32x4 (&qa)[RB][8], WaveState<RB>& ws,
                                            half4_t (&pb)[RB], int lane, int t0, const RowMask<RB, WIN>& mk) {
  float x[RB][4];
  scores_mfma<RB>(kf, qa, x);
  float p[RB][4];
  softmax_step<RB>(x, ws, p, lane, t0, mk);
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
    pb[rb] = half4_t{(_Float16)p[rb][0], (_Float16)p[rb][1], (_Float16)p[rb][2], (_Float16)p[rb][3]};
}

// The pieces of one step for the software-pipelined fp16 loop, where the PV
// matrix ops of step k are issued right after the score matrix ops of step
// k+1, and the softmax of k+1 fills their shadow:
//   scores_mfma   the raw scores of step k+1 (Q fragments in registers);
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
// (max_check: the same for a step that needs no masking)
template <int RB>
__device__ __forceinline__ bool max_check(const float (&x)[RB][4], float (&lmx)[RB], const WaveState<RB>& ws) {
  bool bump = false;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    lmx[rb] = fmaxf(fmaxf(x[rb][0], x[rb][1]), fmaxf(x[rb][2], x[rb][3]));
    bump = bump | (lmx[rb] * ws.c > ws.m[rb] + kLazyLog2);
  }
  return __any(bump);
}
template <int RB, bool WIN, bool SKIP = true>
__device__ __forceinline__ bool mask_check(float (&x)[RB][4], float (&lmx)[RB], const WaveState<RB>& ws,
                                           const RowMask<RB, WIN>& mk, int lane, int t0) {
  apply_mask<RB, WIN, SKIP>(x, mk, lane, t0);
  return max_check<RB>(x, lmx, ws);
}

template <int RB>
__device__ __forceinline__ void move_ref(const float (&lmx)[RB], WaveState<RB>& ws, float (&alpha)[RB]) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float mx = lmx[rb];
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    mx *= ws.c;
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
    for (int i = 0; i < 4; ++i) p[i] = exp2_fast(__builtin_fmaf(x[rb][i], ws.c, -ref));
    lsum[rb] = (p[0] + p[1]) + (p[2] + p[3]);
    pb[rb] = half4_t{(_Float16)p[0], (_Float16)p[1], (_Float16)p[2], (_Float16)p[3]};
  }
}

// Keeps the common case's softmax (p at the current reference, computed
// before the rare branch that moves the reference and redoes it) where it
// is: otherwise the compiler sinks it past that branch into the common path,
// a basic block of its own, out of reach of the matrix ops of the same step
// that it could be scheduled beside.
template <int RB>
__device__ __forceinline__ void pin_softmax(half4_t (&pb)[RB], float (&lsum)[RB]) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) asm volatile("" : "+v"(pb[rb]), "+v"(lsum[rb]));
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
// The copies go through a buffer resource made per half-step (scalar
// instructions: base = the half-step's first byte, 8 KB long; 4 KB for FP8
// bytes) with a 32-bit
// per-lane offset, which the instruction takes as is, so a step's 16 DMAs
// cost no vector address arithmetic (a 64-bit add each as global loads).
// Block j's offset is 1024 j plus a per-lane part that depends only on the
// parity of j (the swizzle). The instruction's offset field (12 bits) is
// added to both the source and the LDS address, its scalar offset to the
// source only (pinned with a probe on the GPU); so block j takes (j & 3) *
// 1024 in the offset field, from j = 4 on 4096 more in the scalar offset,
// and is given the LDS base ring + (j & 4) * 1024. A lane offset outside the
// resource's range would read zeros instead of faulting.
//
// Cache policy of the copies (the instruction's cache-policy field): a pass
// whose keys one workgroup each reads, and that is large (kStreamOnceBytes),
// goes non-temporal (kCacheStream, the nt bit), the rest with the default
// policy. On MI355X a page gather in this kernel's order (random 8 KB pages,
// 16 KB per wave step, one step in flight) streams at 6.95 TB/s with the nt
// bit against 6.16 TB/s without it (a standalone probe; the scope bits
// sc0/sc1 change nothing). Where several row tiles read the same keys (the
// later ones from L2), nt costs more than it gains: the lines leave L2
// before the second reader comes.
constexpr int kCacheDefault = 0;
constexpr int kCacheStream = 2;  // nt
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer access (gfx9 family)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t half_step_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 8192, kRsrcWord3);
}
template <int J, int CP>
__device__ __forceinline__ void dma_block(__amdgpu_buffer_rsrc_t r, char* ring, uint32_t lane_off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, SV_LP(ring + (J & 4) * 1024), 16, lane_off, J >= 4 ? 4096 : 0,
                                           (J & 3) * 1024, CP);
}
// Per-lane byte offsets of the copies of the blocks with even and odd index
// j (lane l copies 16-byte chunk c = l % 32 of token t = 2j + l / 32). K: the
// chunk lands at chunk c ^ (t & 3); V: at c ^ 2 (t & 3).
__device__ __forceinline__ void k_copy_offsets(int lane, uint32_t* even, uint32_t* odd) {
  const uint32_t h = (uint32_t)lane >> 5, c = (uint32_t)lane & 31u;
  *even = h * 512u + 16u * (c ^ h);
  *odd = h * 512u + 16u * (c ^ (2u + h));
}
__device__ __forceinline__ void v_copy_offsets(int lane, uint32_t* even, uint32_t* odd) {
  const uint32_t h = (uint32_t)lane >> 5, c = (uint32_t)lane & 31u;
  *even = h * 512u + 16u * (c ^ (2u * h));
  *odd = h * 512u + 16u * (c ^ (4u + 2u * h));
}
template <int B0, int B1, int CP>
__device__ __forceinline__ void dma_k(const _Float16* kb, char* ring, int lane) {
  const __amdgpu_buffer_rsrc_t r = half_step_rsrc(kb);
  uint32_t even, odd;
  k_copy_offsets(lane, &even, &odd);
  if constexpr (B0 <= 0 && 0 < B1) dma_block<0, CP>(r, ring, even);
  if constexpr (B0 <= 1 && 1 < B1) dma_block<1, CP>(r, ring, odd);
  if constexpr (B0 <= 2 && 2 < B1) dma_block<2, CP>(r, ring, even);
  if constexpr (B0 <= 3 && 3 < B1) dma_block<3, CP>(r, ring, odd);
  if constexpr (B0 <= 4 && 4 < B1) dma_block<4, CP>(r, ring, even);
  if constexpr (B0 <= 5 && 5 < B1) dma_block<5, CP>(r, ring, odd);
  if constexpr (B0 <= 6 && 6 < B1) dma_block<6, CP>(r, ring, even);
  if constexpr (B0 <= 7 && 7 < B1) dma_block<7, CP>(r, ring, odd);
}
template <int B0, int B1, int CP>
__device__ __forceinline__ void dma_v(const _Float16* vb, char* ring, int lane) {
  const __amdgpu_buffer_rsrc_t r = half_step_rsrc(vb);
  uint32_t even, odd;
  v_copy_offsets(lane, &even, &odd);
  if constexpr (B0 <= 0 && 0 < B1) dma_block<0, CP>(r, ring, even);
  if constexpr (B0 <= 1 && 1 < B1) dma_block<1, CP>(r, ring, odd);
  if constexpr (B0 <= 2 && 2 < B1) dma_block<2, CP>(r, ring, even);
  if constexpr (B0 <= 3 && 3 < B1) dma_block<3, CP>(r, ring, odd);
  if constexpr (B0 <= 4 && 4 < B1) dma_block<4, CP>(r, ring, even);
  if constexpr (B0 <= 5 && 5 < B1) dma_block<5, CP>(r, ring, odd);
  if constexpr (B0 <= 6 && 6 < B1) dma_block<6, CP>(r, ring, even);
  if constexpr (B0 <= 7 && 7 < B1) dma_block<7, CP>(r, ring, odd);
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
template <int CP>
__device__ __forceinline__ void dma_k8(const uint8_t* kb, const _Float16* ksb, const _Float16* vsb,
                                       char* stage, int lane) {
  // (a buffer resource over the 4 KB, as for fp16: token t = 4j + l/16,
  // whose t & 3 does not depend on j, so one lane offset serves all blocks)
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(kb), (short)0, 4096,
                                                                     kRsrcWord3);
  const uint32_t g = (uint32_t)lane >> 4;
  const uint32_t off = g * 256u + 16u * (((uint32_t)lane & 15u) ^ (g & 3u));
  dma_block<0, CP>(r, stage, off);
  dma_block<1, CP>(r, stage, off);
  dma_block<2, CP>(r, stage, off);
  dma_block<3, CP>(r, stage, off);
  const _Float16* ssrc = lane < 32 ? ksb + 2 * lane : vsb + 2 * (lane - 32);
  __builtin_amdgcn_global_load_lds(SV_GP(ssrc), SV_LP(stage + 8192), 4, 0, CP);
}
// V half-step of an FP8 step: the 4 KB of 16 tokens copied as is.
template <int CP>
__device__ __forceinline__ void dma_v8(const uint8_t* vb, char* stage, int lane) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(vb), (short)0, 4096,
                                                                     kRsrcWord3);
  const uint32_t off = (uint32_t)lane * 16u;
  dma_block<0, CP>(r, stage + 4096, off);
  dma_block<1, CP>(r, stage + 4096, off);
  dma_block<2, CP>(r, stage + 4096, off);
  dma_block<3, CP>(r, stage + 4096, off);
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

// The raw scores of one FP8 step: per 64-channel block, two matrix ops on
// the converted K and the wave's Q fragments (in registers), one accumulator
// per (row block, scale block) so the block scales are applied after all
// matrix ops are issued: S = sum_b scale_b * partial_b, one multiply and
// three fused multiply-adds per score (the softmax scale enters with the
// exponent).
template <int RB>
__device__ __forceinline__ void scores8_mfma(const KFrag8& kf, const u32x4 (&qa)[RB][8], float (&x)[RB][4]) {
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
      x[rb][i] = __builtin_fmaf(fk[i][3], acc[rb][3][i], t);
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

}  // namespace sv
