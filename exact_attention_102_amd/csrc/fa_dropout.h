// fa_dropout.h -- dropout on the attention probabilities, fused into the forward,
// dK/dV and dQ kernels.
//
// Dropout is one of the elementwise passes over the N x N matrix that unfused
// attention spends its time in ("ELI5: FlashAttention", standard-attention
// highlights); fused, its mask never exists in memory.  The keep decision of score
// element (b, h, i, j) is a pure function of its coordinates, so every kernel
// recomputes exactly the decisions the forward made:
//   generator  Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel Random
//              Numbers: As Easy as 1, 2, 3", SC '11): ten rounds over four 32-bit
//              words; a round multiplies word 0 by 0xD2511F53 and word 2 by
//              0xCD9E8D57 (64-bit products) and outputs (hi1 ^ w1 ^ k0, lo1,
//              hi0 ^ w3 ^ k1, lo0); the key advances by (0x9E3779B9, 0xBB67AE85)
//              between rounds.
//   key        (seed low 32 bits, seed high 32 bits)
//   counter    (j / 8, i, b * H + h, offset)
//   draws      the 128-bit output read as eight 16-bit draws; key j uses draw
//              j % 8, found in half (j % 2) of word (j % 8) / 2, low half first
//   keep       draw >= t, t = floor(p * 2^16) (at most 2^16 - 1); kept values are
//              scaled by 2^16 / (2^16 - t), the reciprocal of the keep probability.
// In the forward and dQ kernels a lane holds one query and aligned groups of eight
// keys, so one call yields the lane's eight decisions.  In the dK/dV kernel a lane
// holds one key and groups of eight queries: each of the eight lanes of a key
// group makes the call of one query, and an 8 x 8 transpose of the 16-bit draws
// across those lanes hands every lane the draws of its own key.
#pragma once
#include "fa_device.h"

namespace fa {

// Per-launch dropout constants, identical in every lane.
struct DropCtx {
  unsigned k0, k1;   // Philox key
  unsigned bh;       // third counter word: flat head index b * H + h
  unsigned offset;   // fourth counter word
  unsigned t;        // 16-bit threshold, 1 .. 65535
};

__device__ __forceinline__ u32x4 philox4x32_10(unsigned c0, unsigned c1, unsigned c2, unsigned c3, unsigned k0,
                                               unsigned k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    const unsigned long long p0 = (unsigned long long)c0 * 0xD2511F53u;
    const unsigned long long p1 = (unsigned long long)c2 * 0xCD9E8D57u;
    // three-input XORs in one v_bitop3_b32 each (truth table 0x96 = a ^ b ^ c)
    const unsigned n0 = __builtin_amdgcn_bitop3_b32((unsigned)(p1 >> 32), c1, k0, 0x96);
    const unsigned n2 = __builtin_amdgcn_bitop3_b32((unsigned)(p0 >> 32), c3, k1, 0x96);
    c1 = (unsigned)p1;
    c3 = (unsigned)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  u32x4 r;
  r[0] = c0;
  r[1] = c1;
  r[2] = c2;
  r[3] = c3;
  return r;
}

// The eight draws of query i for keys 8 * kgroup .. 8 * kgroup + 7.
__device__ __forceinline__ u32x4 drop_draws(const DropCtx& dc, int kgroup, int i) {
  return philox4x32_10((unsigned)kgroup, (unsigned)i, dc.bh, dc.offset, dc.k0, dc.k1);
}

// AND mask for a dword of two packed bf16 values whose draws are the two halves of w.
__device__ __forceinline__ unsigned keep_bits2(unsigned w, unsigned t) {
  return ((w & 0xffffu) >= t ? 0x0000ffffu : 0u) | ((w >> 16) >= t ? 0xffff0000u : 0u);
}

// Zeroes the dropped entries of eight packed bf16 values (element e <-> draw e).
__device__ __forceinline__ bf16x8 drop_mask8(bf16x8 x, const u32x4& w, unsigned t) {
  u32x4 u = __builtin_bit_cast(u32x4, x);
#pragma unroll
  for (int m = 0; m < 4; ++m) u[m] &= keep_bits2(w[m], t);
  return __builtin_bit_cast(bf16x8, u);
}

// Keep decision of draw e (compile-time after unrolling).
__device__ __forceinline__ bool drop_keep(const u32x4& w, int e, unsigned t) {
  const unsigned x = w[e >> 1];
  return ((e & 1) ? (x >> 16) : (x & 0xffffu)) >= t;
}

// Lane t of every aligned group of eight lanes holds row t of an 8 x 8 matrix of
// 16-bit values (element u in half u % 2 of dword u / 2); returns column t.
// Three exchange stages swap the off-diagonal 4 x 4, 2 x 2 and 1 x 1 blocks with
// the partner lane t ^ 4 (ds_swizzle, xor mode), t ^ 2 and t ^ 1 (DPP quad
// permutes).  Every lane of the wave must be active.
__device__ __forceinline__ u32x4 transpose8_b16(u32x4 w, int lane) {
  {
    const bool hi = lane & 4;
    const int s0 = (int)(hi ? w[0] : w[2]), s1 = (int)(hi ? w[1] : w[3]);
    const unsigned r0 = (unsigned)__builtin_amdgcn_ds_swizzle(s0, 0x101F);  // and 0x1f, or 0, xor 4
    const unsigned r1 = (unsigned)__builtin_amdgcn_ds_swizzle(s1, 0x101F);
    if (hi) {
      w[0] = r0;
      w[1] = r1;
    } else {
      w[2] = r0;
      w[3] = r1;
    }
  }
  {
    const bool hi = lane & 2;
    const int s0 = (int)(hi ? w[0] : w[1]), s1 = (int)(hi ? w[2] : w[3]);
    const unsigned r0 = (unsigned)__builtin_amdgcn_mov_dpp(s0, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
    const unsigned r1 = (unsigned)__builtin_amdgcn_mov_dpp(s1, 0x4E, 0xF, 0xF, false);
    if (hi) {
      w[0] = r0;
      w[2] = r1;
    } else {
      w[1] = r0;
      w[3] = r1;
    }
  }
  {
    const bool hi = lane & 1;
    const int s0 = (int)(hi ? ((w[0] & 0xffffu) | (w[1] << 16)) : ((w[0] >> 16) | (w[1] & 0xffff0000u)));
    const int s1 = (int)(hi ? ((w[2] & 0xffffu) | (w[3] << 16)) : ((w[2] >> 16) | (w[3] & 0xffff0000u)));
    const unsigned r0 = (unsigned)__builtin_amdgcn_mov_dpp(s0, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
    const unsigned r1 = (unsigned)__builtin_amdgcn_mov_dpp(s1, 0xB1, 0xF, 0xF, false);
    if (hi) {
      w[0] = (w[0] & 0xffff0000u) | (r0 & 0xffffu);
      w[1] = (w[1] & 0xffff0000u) | (r0 >> 16);
      w[2] = (w[2] & 0xffff0000u) | (r1 & 0xffffu);
      w[3] = (w[3] & 0xffff0000u) | (r1 >> 16);
    } else {
      w[0] = (w[0] & 0xffffu) | (r0 << 16);
      w[1] = (w[1] & 0xffffu) | (r0 & 0xffff0000u);
      w[2] = (w[2] & 0xffffu) | (r1 << 16);
      w[3] = (w[3] & 0xffffu) | (r1 & 0xffff0000u);
    }
  }
  return w;
}

}  // namespace fa
