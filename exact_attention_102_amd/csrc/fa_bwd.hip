// fa_bwd.hip -- fused attention backward for gfx950, in both designs compared in
// "Potential algorithmic improvements for backward pass" (flash-attention issue
// 1172): the 5-GEMM form whose dK/dV kernel also adds dQ with fp32 atomics, and the
// atomic-free 7-GEMM form (a dK/dV kernel, then a dQ kernel that walks the keys in
// the forward's direction).  Both recompute S and P from Q, K and the saved
// log-sum-exp ("ELI5: FlashAttention", recomputation).
//
// Notation per (query i, key j): P_ij = exp2(S_ij * c - lse_i * log2 e) with
// c = scale * log2 e; dP = dO V^T; dS = P * (dP - delta_i) where delta_i =
// sum_k dO_ik O_ik (the preprocess kernel); dV = P^T dO; dK = scale * dS^T Q;
// dQ = scale * dS K.
//
// Kernels: preprocess_kernel (delta, dq zeroing); dkdv_kernel (one 32-key block per
// wave; both designs, every head dim, dropout); dkdv_wide_kernel (two 32-key blocks
// per wave, so each Q/dO fragment read from LDS feeds two MFMAs; both designs, head
// dims 64, 96, 128, no dropout); dq_kernel (the 7-GEMM dQ pass).
//
// DROP: dropout on P (fa_dropout.h).  With M the keep mask and s the keep scale,
// the forward used Pd = P * M * s, so dV = Pd^T dO and dP = (dO V^T) * M * s, while
// dS = P * (dP - delta_i) keeps its form: delta_i = rowsum(Pd * dO V^T) =
// rowsum(dO * O) is still what the preprocess kernel computes.  The kernels redraw
// the forward's mask from the same counters.
#include "fa_device.h"
#include "fa_dropout.h"
#include "fa_launch.h"

namespace fa {

__device__ __forceinline__ float bf16_bits_to_f32(unsigned short h) {
  return __builtin_bit_cast(float, ((unsigned)h) << 16);
}

// ---------------------------------------------------------------------------
// delta_i = sum_k dO_ik * O_ik; optionally zero dq.  D / 8 threads per row, each
// reading one 16-byte chunk of dO and two of O (chunks past the head dim hd add
// nothing and are not cleared), then a shuffle reduction.
template <int D>
__global__ __launch_bounds__(256) void preprocess_kernel(PreArgs a) {
  constexpr int TPR = D / 8;
  constexpr int RPB = 256 / TPR;
  const int tid = threadIdx.x;
  const int row = blockIdx.x * RPB + tid / TPR;
  const int c = tid % TPR;
  float acc = 0.f;
  if (row < a.rows && c * 8 < a.hd) {
    const int bh = row / a.N, n = row % a.N;
    const size_t obase = head_base(a.vo, bh, a.H) + (size_t)n * a.vo.sn + c * 8;
    const u32x4 dv = *(const u32x4*)(a.dout + head_base(a.vdo, bh, a.H) + (size_t)n * a.vdo.sn + c * 8);
    const f32x4 o0 = *(const f32x4*)(a.o + obase);
    const f32x4 o1 = *(const f32x4*)(a.o + obase + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const unsigned w = dv[e];
      const float lo = bf16_bits_to_f32((unsigned short)(w & 0xffffu));
      const float hi = bf16_bits_to_f32((unsigned short)(w >> 16));
      const float oa = (e < 2) ? o0[2 * e] : o1[2 * e - 4];
      const float ob = (e < 2) ? o0[2 * e + 1] : o1[2 * e - 3];
      acc = fmaf(lo, oa, acc);
      acc = fmaf(hi, ob, acc);
    }
    if (a.dq) {
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      float* dqp = a.dq + head_base(a.vdq, bh, a.H) + (size_t)n * a.vdq.sn + c * 8;
      *(f32x4*)dqp = z;
      *(f32x4*)(dqp + 4) = z;
    }
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, TPR);
  if (row < a.rows && c == 0) a.delta[row] = acc;
}

int launch_preprocess(const PreArgs& a, int d, hipStream_t stream) {
  // head dims 96 and 192 run on the 128- and 256-wide row kernels, 288..384 on the 512-wide one
  // (a.hd masks the rest)
  const int kd = d == 96 ? 128 : (d == 192 ? 256 : (d > 256 ? 512 : d));
  const int rpb = 256 / (kd / 8);
  const int blocks = (a.rows + rpb - 1) / rpb;
  switch (kd) {
    case 64: hipLaunchKernelGGL(preprocess_kernel<64>, dim3(blocks), dim3(256), 0, stream, a); break;
    case 128: hipLaunchKernelGGL(preprocess_kernel<128>, dim3(blocks), dim3(256), 0, stream, a); break;
    case 256: hipLaunchKernelGGL(preprocess_kernel<256>, dim3(blocks), dim3(256), 0, stream, a); break;
    case 512: hipLaunchKernelGGL(preprocess_kernel<512>, dim3(blocks), dim3(256), 0, stream, a); break;
    default: return -1;
  }
  return 0;
}

// ---------------------------------------------------------------------------
// Per-row statistics of a query tile in LDS: lse * log2(e) (+inf past the end, so
// that P = 0 there) and delta (0 past the end).
template <int BQ, int NT>
struct RowStager {
  float raw;
  int q;
  // Issues the load only; nothing reads it until store(), which runs after the
  // tile's wait (wait_tile), so the load never makes the wave wait for the
  // direct-to-LDS prefetch issued after it.
  __device__ __forceinline__ void load(const float* lse, const float* delta, int q0, int N, int tid) {
    const int r = tid < BQ ? tid : tid - BQ;
    q = q0 + r;
    const float* src = tid < BQ ? lse : delta;
    raw = tid < 2 * BQ ? src[min(q, N - 1)] : 0.f;
  }
  __device__ __forceinline__ void store(LDS float* dst, int N, int tid) {
    asm volatile("" : "+v"(raw));  // keeps every use of the loaded value after this point
    if (tid < BQ) {
      dst[tid] = q < N ? raw * kLog2e : INFINITY;
    } else if (tid < 2 * BQ) {
      dst[tid] = q < N ? raw : 0.f;
    }
  }
};

// ---------------------------------------------------------------------------
// dK/dV kernel.  One workgroup owns BK = 32 * NW keys of one (batch, head), each
// wave 32 of them (one key per lane column of the MFMA C layout).  It walks the
// query tiles (BQ rows of Q and dO, plus their lse and delta) through
// double-buffered LDS, the Q/dO rows arriving by direct-to-LDS loads one tile
// ahead.  Per 32-query block:
//   S  = Q K^T,  dP = dO V^T          A = Q / dO row fragments (LDS),
//                                      B = K^T / V^T (registers, or LDS: KVL)
//   P, dS                              elementwise, in registers
//   dV^T += dO^T P,  dK^T += Q^T dS    A = transposed LDS reads, B = P / dS
// ATOMIC (the 5-GEMM design): each wave also writes its dS^T block to LDS; after a
// barrier the workgroup computes dQ_tile = dS K over all BK keys (waves split the
// (query block, d block) pairs) and adds it to dq with fp32 atomics, one atomic
// per dq element per workgroup and query tile.
// KVL: 0 keeps each wave's K and V fragments in registers; 1 reads both from the
// workgroup's K and V tiles in LDS (large d); 2 (atomic shapes) reads K from the LDS
// tile the dQ product needs anyway and keeps only V in registers.
// D: LDS tile width (64, 128, 256); DV <= D (a multiple of 32): the head-dim columns
// computed (96 and 192 run on 128- and 256-wide tiles without the zero columns' products).
template <int D, int DV, int BQ, int NW, bool CAUSAL, bool ATOMIC, int KVL, bool DROP>
struct DkdvMath {
  static constexpr bool K_LDS = KVL != 0;
  static constexpr bool V_LDS = KVL == 1;
  // K tile: plain row fragments (K_LDS) and/or transposed reads (atomic dQ product)
  static constexpr int KMODE = ATOMIC ? (K_LDS ? kBoth : kColOnly) : kRowOnly;
  static constexpr int BK = 32 * NW;
  static constexpr int QBN = BQ / 32;
  static constexpr int DB = DV / 32;
  static constexpr int KK = DV / 16;
  // LDS fragment reads issued ahead of their MFMAs (needs registers the d = 256 and
  // the 8-wave atomic shapes do not have; those keep short scheduling fences)
  static constexpr bool kReadAhead = D <= 128 && !(ATOMIC && NW > 4);
  // Software pipelining across the tile's query blocks (see tile()): measured faster
  // only for two d = 64 shapes (8-wave dK/dV +8%, 4-wave atomic +15%); the 4-wave
  // dK/dV loses 17%, the d = 128 shapes 7-14%, and the 8-wave atomic shapes run out
  // of registers.
  static constexpr bool kPipe =
      !DROP && QBN >= 2 && D == 64 && DV == 64 && (ATOMIC ? NW == 4 : NW == 8);
  // S and dP as vector-register MFMAs (mfma32v_*) where the dK/dV accumulators live in
  // the accumulation registers: workgroups of at most 4 waves (one wave per SIMD)
  static constexpr bool kVgprSP = NW <= 4;
  // dS between the dV products (one wave per SIMD, 7-GEMM): 1-2% faster at d = 192 and
  // 256, level or slower at d = 96 (fewer dV products to hide the arithmetic under)
  static constexpr bool kSplitDS = kVgprSP && !ATOMIC && D >= 192;

  __device__ __forceinline__ static void tile(const LDS char* qtl, const LDS char* dotl, const LDS float* stats,
                                              const LDS char* ktile, const LDS char* vtile, LDS char* dst,
                                              const bf16x8* kf, const bf16x8* vf, f32x16 (&dk)[DB],
                                              f32x16 (&dv)[DB], float* dqh, int q0, int k0, int kw, int key, int N,
                                              float c, float scale, const RowOffsets<D, kBoth>& fr,
                                              const ColOffsets<D, kBoth>& fc, const RowOffsets<D, KMODE>& pk,
                                              const RowOffsets<D, kRowOnly>& pv, int wave, int g, int l32,
                                              int lane, const DropCtx& dc, float ks) {
    const LDS float* l2t = stats;
    const LDS float* dlt = stats + BQ;
    // Pipelined path (kPipe shapes): every query block of the tile is inside the
    // sequence and below the causal diagonal for all of this wave's keys (no mask).
    // The S / dP products of block qb + 1 are issued between the exp / dS arithmetic
    // of block qb, so the wave overlaps its own VALU work with its MFMAs.
    if constexpr (kPipe) {
      if (q0 + BQ <= N && (!CAUSAL || q0 >= kw + 31)) {
        f32x16 sc = zero16(), dpc = zero16();
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          bf16x8 kb, vb;
          if constexpr (K_LDS) {
            kb = pk.row(ktile, wave * 32, kk);
          } else {
            kb = kf[kk];
          }
          if constexpr (V_LDS) {
            vb = pv.row(vtile, wave * 32, kk);
          } else {
            vb = vf[kk];
          }
          sc = mfma32(fr.row(qtl, 0, kk), kb, sc);
          dpc = mfma32(fr.row(dotl, 0, kk), vb, dpc);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int qb = 0; qb < QBN; ++qb) {
          float l2[16], dl[16];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
              const int r = qb * 32 + 16 * h + 8 * g + 4 * hf;
              const f32x4 lv = *(const LDS f32x4*)(l2t + r);
              const f32x4 dd = *(const LDS f32x4*)(dlt + r);
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                l2[8 * h + 4 * hf + e] = lv[e];
                dl[8 * h + 4 * hf + e] = dd[e];
              }
            }
          }
          f32x16 sn = zero16(), dpn = zero16();
          if (qb + 1 < QBN) {
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
              bf16x8 kb, vb;
              if constexpr (K_LDS) {
                kb = pk.row(ktile, wave * 32, kk);
              } else {
                kb = kf[kk];
              }
              if constexpr (V_LDS) {
                vb = pv.row(vtile, wave * 32, kk);
              } else {
                vb = vf[kk];
              }
              sn = mfma32(fr.row(qtl, (qb + 1) * 32, kk), kb, sn);
              dpn = mfma32(fr.row(dotl, (qb + 1) * 32, kk), vb, dpn);
            }
          }
          f32x16 p, ds;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float pv_ = exp2_hw(fmaf(sc[r], c, -l2[r]));
            p[r] = pv_;
            ds[r] = pv_ * (dpc[r] - dl[r]);
          }
          const bf16x8 pb0 = pack8(p, 0), pb1 = pack8(p, 8);
          bf16x8 sb0 = pack8(ds, 0), sb1 = pack8(ds, 8);
          if (qb + 1 < QBN) {
            // stats reads, then each of the 2 KK products with its fragment read and a
            // share of the exp / dS arithmetic
            __builtin_amdgcn_sched_group_barrier(0x100, 8 + 4, 0);
#pragma unroll
            for (int i = 0; i < 2 * KK; ++i) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
              __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            dv[db] = mfma32(fc.col(dotl, qb * 32, db), pb0, dv[db]);
            dv[db] = mfma32(fc.col(dotl, qb * 32 + 16, db), pb1, dv[db]);
            dk[db] = mfma32(fc.col(qtl, qb * 32, db), sb0, dk[db]);
            dk[db] = mfma32(fc.col(qtl, qb * 32 + 16, db), sb1, dk[db]);
            if constexpr (!kReadAhead) fence_every<2>(db);
          }
          if constexpr (kReadAhead) {
            __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
            for (int db = 0; db < DB - 1; ++db) {
              __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
              __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
          }
          if constexpr (ATOMIC) {
            if (!CAUSAL && key >= N) {
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                sb0[e] = (__bf16)0.f;
                sb1[e] = (__bf16)0.f;
              }
            }
            *(LDS bf16x8*)(dst + tile_off<BQ, kBoth>(wave * 32 + l32, qb * 32 + 8 * g)) = sb0;
            *(LDS bf16x8*)(dst + tile_off<BQ, kBoth>(wave * 32 + l32, qb * 32 + 16 + 8 * g)) = sb1;
          }
          __builtin_amdgcn_sched_barrier(0);
          sc = sn;
          dpc = dpn;
        }
        return;
      }
    }
#pragma unroll
    for (int qb = 0; qb < QBN; ++qb) {
      const int qbase = q0 + qb * 32;
      // Scheduling fences between the phases keep the live register set to one
      // phase's operands (otherwise every LDS read of the tile is hoisted up front).
      __builtin_amdgcn_sched_barrier(0);
      // Blocks wholly past the end (padding rows, P = 0), or wholly above the causal
      // diagonal for this wave's keys, contribute nothing.
      if (qbase < N && (!CAUSAL || qbase + 31 >= kw)) {
        // draws of this lane's key for queries qbase + 16 h + 8 g + (0..7): lane t of
        // each 8-lane key group draws query ... + t for the whole group, then transpose
        u32x4 dr[DROP ? 2 : 1];
        if constexpr (DROP) {
#pragma unroll
          for (int h = 0; h < 2; ++h)
            dr[h] = transpose8_b16(drop_draws(dc, (kw >> 3) + (l32 >> 3), qbase + 16 * h + 8 * g + (l32 & 7)), lane);
        }
        f32x16 s, dp;
        if constexpr (kVgprSP) {
          // S and dP in vector registers (see the wide kernel); fragment reads two k-steps
          // ahead through three rotating slots
          bf16x8 qa[3], da[3], kb[3], vb[3];
          auto ld = [&](int kk) {
            qa[kk % 3] = fr.row(qtl, qb * 32, kk);
            da[kk % 3] = fr.row(dotl, qb * 32, kk);
            if constexpr (K_LDS) {
              kb[kk % 3] = pk.row(ktile, wave * 32, kk);
            } else {
              kb[kk % 3] = kf[kk];
            }
            if constexpr (V_LDS) {
              vb[kk % 3] = pv.row(vtile, wave * 32, kk);
            } else {
              vb[kk % 3] = vf[kk];
            }
          };
          ld(0);
          ld(1);
#pragma unroll
          for (int kk = 0; kk < KK; ++kk) {
            if (kk + 2 < KK) ld(kk + 2);
            const int sl = kk % 3;
            mfma32v_kstep(kk, KK, s, dp, qa[sl], kb[sl], da[sl], vb[sl]);
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
          s = zero16();
          dp = zero16();
#pragma unroll
          for (int kk = 0; kk < KK; ++kk) {
            bf16x8 kb, vb;
            if constexpr (K_LDS) {
              kb = pk.row(ktile, wave * 32, kk);
            } else {
              kb = kf[kk];
            }
            if constexpr (V_LDS) {
              vb = pv.row(vtile, wave * 32, kk);
            } else {
              vb = vf[kk];
            }
            s = mfma32(fr.row(qtl, qb * 32, kk), kb, s);
            dp = mfma32(fr.row(dotl, qb * 32, kk), vb, dp);
            if constexpr (!kReadAhead) fence_every<4>(kk);
          }
          // Interleave: fragment reads run two k-steps ahead of their MFMAs, so LDS
          // latency hides under the previous products instead of stalling the wave.
          if constexpr (kReadAhead) {
            constexpr int RPS = 2 + K_LDS + V_LDS;  // row-fragment reads per k-step
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * RPS, 0);
#pragma unroll
            for (int kk = 0; kk < KK - 2; ++kk) {
              __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
              __builtin_amdgcn_sched_group_barrier(0x100, RPS, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        // register 8h + e <-> query row qb*32 + 16h + 8g + e of the tile
        float l2[16], dl[16];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            const int r = qb * 32 + 16 * h + 8 * g + 4 * hf;
            const f32x4 lv = *(const LDS f32x4*)(l2t + r);
            const f32x4 dd = *(const LDS f32x4*)(dlt + r);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              l2[8 * h + 4 * hf + e] = lv[e];
              dl[8 * h + 4 * hf + e] = dd[e];
            }
          }
        }
        // Queries past the end have lse2 = +inf, hence P = 0.  Keys past the end only
        // feed their own dK/dV columns, which are never stored -- except through dS in
        // the atomic dQ product, where their dS^T rows are written as zeros below.
        // Under the causal mask, key > query covers them as well.
        // causal: scores of keys after the query are -inf (P = 0), in a pass of its own
        // that only diagonal blocks take (the empty asm keeps it a branch)
        if (CAUSAL && qbase < kw + 31) {
          asm volatile("");
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int q = qbase + 16 * (r >> 3) + 8 * g + (r & 7);
            if (key > q) s[r] = -INFINITY;
          }
        }
        f32x16 p, ds;
        bf16x8 pb0, pb1, sb0, sb1;
        if constexpr (kSplitDS) {
          // P first; the dS arithmetic then runs between the dV products (they need only
          // P), whose results go to the accumulation registers, so the wave overlaps it
          // with its own MFMAs; the dK products follow
#pragma unroll
          for (int r = 0; r < 16; ++r) p[r] = exp2_hw(fmaf(s[r], c, -l2[r]));
          pb0 = pack8(p, 0);
          pb1 = pack8(p, 8);
          if constexpr (DROP) {  // dV takes Pd = P * M * s; s is applied when dV is stored
            pb0 = drop_mask8(pb0, dr[0], dc.t);
            pb1 = drop_mask8(pb1, dr[1], dc.t);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            dv[db] = mfma32(fc.col(dotl, qb * 32, db), pb0, dv[db]);
            dv[db] = mfma32(fc.col(dotl, qb * 32 + 16, db), pb1, dv[db]);
#pragma unroll
            for (int r = db * 16 / DB; r < (db + 1) * 16 / DB; ++r) {
              float dpv = dp[r];
              if constexpr (DROP) dpv = drop_keep(dr[r >> 3], r & 7, dc.t) ? dpv * ks : 0.f;
              ds[r] = p[r] * (dpv - dl[r]);
            }
            fence_every<1>(db);
          }
          sb0 = pack8(ds, 0);
          sb1 = pack8(ds, 8);
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            dk[db] = mfma32(fc.col(qtl, qb * 32, db), sb0, dk[db]);
            dk[db] = mfma32(fc.col(qtl, qb * 32 + 16, db), sb1, dk[db]);
            fence_every<2>(db);
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float pv = exp2_hw(fmaf(s[r], c, -l2[r]));
            p[r] = pv;
            float dpv = dp[r];
            if constexpr (DROP) dpv = drop_keep(dr[r >> 3], r & 7, dc.t) ? dpv * ks : 0.f;
            ds[r] = pv * (dpv - dl[r]);
          }
          pb0 = pack8(p, 0);
          pb1 = pack8(p, 8);
          if constexpr (DROP) {  // dV takes Pd = P * M * s; s is applied when dV is stored
            pb0 = drop_mask8(pb0, dr[0], dc.t);
            pb1 = drop_mask8(pb1, dr[1], dc.t);
          }
          sb0 = pack8(ds, 0);
          sb1 = pack8(ds, 8);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            dv[db] = mfma32(fc.col(dotl, qb * 32, db), pb0, dv[db]);
            dv[db] = mfma32(fc.col(dotl, qb * 32 + 16, db), pb1, dv[db]);
            dk[db] = mfma32(fc.col(qtl, qb * 32, db), sb0, dk[db]);
            dk[db] = mfma32(fc.col(qtl, qb * 32 + 16, db), sb1, dk[db]);
            if constexpr (!kReadAhead) fence_every<2>(db);
          }
          // transposed reads (8 per d block) run one d block ahead of their 4 MFMAs
          if constexpr (kReadAhead) {
            __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
            for (int db = 0; db < DB - 1; ++db) {
              __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
              __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
          }
        }
        if constexpr (ATOMIC) {
          if (!CAUSAL && key >= N) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              sb0[e] = (__bf16)0.f;
              sb1[e] = (__bf16)0.f;
            }
          }
          *(LDS bf16x8*)(dst + tile_off<BQ, kBoth>(wave * 32 + l32, qb * 32 + 8 * g)) = sb0;
          *(LDS bf16x8*)(dst + tile_off<BQ, kBoth>(wave * 32 + l32, qb * 32 + 16 + 8 * g)) = sb1;
        }
      } else if constexpr (ATOMIC) {
        bf16x8 z;
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] = (__bf16)0.f;
        *(LDS bf16x8*)(dst + tile_off<BQ, kBoth>(wave * 32 + l32, qb * 32 + 8 * g)) = z;
        *(LDS bf16x8*)(dst + tile_off<BQ, kBoth>(wave * 32 + l32, qb * 32 + 16 + 8 * g)) = z;
      }
    }
  }

  // 5-GEMM: dQ_tile = dS K over the workgroup's BK keys (its dS^T blocks in LDS,
  // written by tile() of the previous query tile and made visible by the barrier
  // that ended it), one fp32 atomic per dq element per workgroup.  Running it one
  // tile late lets the atomics drain under the next tile's products instead of
  // holding up the end-of-tile wait.
  __device__ __forceinline__ static void atomic_dq(const LDS char* dst, const LDS char* ktile, float* dqh, int q0,
                                                   int N, float scale, int wave, int g, int l32, int lane) {
    {
      for (int t = wave; t < QBN * DB; t += NW) {
        const int qb = t / DB, db = t % DB;
        f32x16 acc = zero16();
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
          acc = mfma32(ColOffsets<BQ, kBoth>::col_dyn(dst, ks * 16, qb, lane),
                       ColOffsets<D, KMODE>::col_dyn(ktile, ks * 16, db, lane), acc);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int q = q0 + qb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          if (q < N) unsafeAtomicAdd(dqh + (size_t)q * DV + db * 32 + l32, acc[r] * scale);
        }
      }
    }
  }
};

// DEFER (atomic only): the dQ product and atomics of a query tile run at the start
// of the next tile, from a second dS^T buffer, instead of behind an extra barrier.
template <int D, int DV, int BQ, int NW, bool CAUSAL, bool ATOMIC, int KVL, bool DEFER, bool DROP>
__global__ __launch_bounds__(NW * 64, 1) void dkdv_kernel(BwdArgs a) {
  using M = DkdvMath<D, DV, BQ, NW, CAUSAL, ATOMIC, KVL, DROP>;
  constexpr int BK = M::BK, DB = M::DB, KK = M::KK;
  constexpr bool K_LDS = M::K_LDS, V_LDS = M::V_LDS;
  constexpr int NT = NW * 64;
  constexpr int QTILE = BQ * D * 2;
  constexpr int KT_BYTES = (ATOMIC || K_LDS) ? BK * D * 2 : 16;
  constexpr int VT_BYTES = V_LDS ? BK * D * 2 : 16;
  constexpr int DST_BYTES = ATOMIC ? BK * BQ * 2 : 16;
  __shared__ __attribute__((aligned(1024))) char q0s[QTILE];
  __shared__ __attribute__((aligned(1024))) char d0s[QTILE];
  __shared__ __attribute__((aligned(1024))) char q1s[QTILE];
  __shared__ __attribute__((aligned(1024))) char d1s[QTILE];
  __shared__ __attribute__((aligned(16))) float st0s[2 * BQ];
  __shared__ __attribute__((aligned(16))) float st1s[2 * BQ];
  __shared__ __attribute__((aligned(1024))) char kts[KT_BYTES];
  __shared__ __attribute__((aligned(1024))) char vts[VT_BYTES];
  __shared__ __attribute__((aligned(1024))) char dsts[DST_BYTES];
  __shared__ __attribute__((aligned(1024))) char dsts1[DEFER ? DST_BYTES : 16];  // dS^T of alternate query tiles
  LDS char* qbuf0 = (LDS char*)q0s;
  LDS char* dbuf0 = (LDS char*)d0s;
  LDS char* qbuf1 = (LDS char*)q1s;
  LDS char* dbuf1 = (LDS char*)d1s;
  LDS float* st0 = (LDS float*)st0s;
  LDS float* st1 = (LDS float*)st1s;
  LDS char* ktile = (LDS char*)kts;
  LDS char* vtile = (LDS char*)vts;
  LDS char* dst0 = (LDS char*)dsts;
  LDS char* dst1 = (LDS char*)dsts1;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const int N = a.N;
  const int nkt = (N + BK - 1) / BK;
  int bh, kt;
  if (CAUSAL) {
    causal_order(blockIdx.x, a.B * a.H, nkt, false, bh, kt);  // low key tiles see the most queries
  } else {
    const int item = xcd_remap(blockIdx.x, a.B * a.H * nkt);
    bh = item / nkt;
    kt = item % nkt;
  }
  const __bf16* Qh = a.q + head_base(a.vq, bh, a.H);
  const __bf16* Kh = a.k + head_base(a.vk, bh, a.H);
  const __bf16* Vh = a.v + head_base(a.vv, bh, a.H);
  const __bf16* dOh = a.dout + head_base(a.vdo, bh, a.H);
  const float* lseh = a.lse + (size_t)bh * N;
  const float* delh = a.delta + (size_t)bh * N;
  // the atomic dq is a contiguous [B, H, N, DV] accumulator (all DV columns; past the
  // head dim they receive zeros, since K is zero there)
  float* dqh = ATOMIC ? a.dq + (size_t)bh * N * DV : nullptr;
  const int hd = a.hd;  // columns hd .. D-1 are zero padding
  const float c = a.scale * kLog2e;
  const DropCtx dc{a.drop_k0, a.drop_k1, (unsigned)bh, a.drop_offset, a.drop_t};
  const float ks = a.drop_scale;

  const int k0 = kt * BK;
  const int kw = k0 + wave * 32;
  const int key = kw + l32;
  const int nqt = (N + BQ - 1) / BQ;
  const int qt0 = CAUSAL ? k0 / BQ : 0;
  constexpr int KMODE = M::KMODE;
  // Q, dO: row fragments and transposed reads; one copier serves both (their row
  // pitches are equal)
  TileDMA<BQ, D, NW, kBoth> qdma;
  qdma.init(wave, lane, a.vq.sn, hd);
  qdma.issue(Qh, qt0 * BQ, N, qbuf0, wave, lane);
  qdma.issue(dOh, qt0 * BQ, N, dbuf0, wave, lane);
  if constexpr (ATOMIC || K_LDS) {
    TileDMA<BK, D, NW, KMODE> kd;
    kd.init(wave, lane, a.vk.sn, hd);
    kd.issue(Kh, k0, N, ktile, wave, lane);
  }
  if constexpr (V_LDS) {
    TileDMA<BK, D, NW, kRowOnly> vd;
    vd.init(wave, lane, a.vv.sn, hd);
    vd.issue(Vh, k0, N, vtile, wave, lane);
  }
  RowStager<BQ, NT> srow;
  srow.load(lseh, delh, qt0 * BQ, N, tid);
  srow.store(st0, N, tid);

  bf16x8 kf[K_LDS ? 1 : KK], vf[V_LDS ? 1 : KK];
  {
    const int krow_g = min(key, N - 1);  // keys past the end are masked (P = 0) and never stored
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      if constexpr (!K_LDS) kf[kk] = load_row_chunk(Kh + (size_t)krow_g * a.vk.sn, 2 * kk + g, hd >> 3);
      if constexpr (!V_LDS) vf[kk] = load_row_chunk(Vh + (size_t)krow_g * a.vv.sn, 2 * kk + g, hd >> 3);
    }
  }
  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dk[db] = zero16();
    dv[db] = zero16();
  }
  RowOffsets<D, kBoth> fr;
  fr.init(lane);
  ColOffsets<D, kBoth> fc;
  fc.init(lane);
  RowOffsets<D, KMODE> pk;
  RowOffsets<D, kRowOnly> pv;
  if constexpr (K_LDS) pk.init(lane, true);
  if constexpr (V_LDS) pv.init(lane, true);

  wait_tile();
  __syncthreads();
  for (int it = qt0; it < nqt; it += 2) {
    fr.refresh();
    fc.refresh();
    if constexpr (K_LDS) pk.refresh();
    if constexpr (V_LDS) pv.refresh();
    qdma.refresh();
    if (it + 1 < nqt) {
      qdma.issue(Qh, (it + 1) * BQ, N, qbuf1, wave, lane);
      qdma.issue(dOh, (it + 1) * BQ, N, dbuf1, wave, lane);
      srow.load(lseh, delh, (it + 1) * BQ, N, tid);
    }
    if constexpr (ATOMIC && DEFER) {
      if (it > qt0) M::atomic_dq(dst1, ktile, dqh, (it - 1) * BQ, N, a.scale, wave, g, l32, lane);
    }
    M::tile(qbuf0, dbuf0, st0, ktile, vtile, dst0, kf, vf, dk, dv, dqh, it * BQ, k0, kw, key, N, c, a.scale, fr, fc,
            pk, pv, wave, g, l32, lane, dc, ks);
    if constexpr (ATOMIC && !DEFER) {
      __syncthreads();
      M::atomic_dq(dst0, ktile, dqh, it * BQ, N, a.scale, wave, g, l32, lane);
    }
    wait_tile();
    if (it + 1 < nqt) srow.store(st1, N, tid);
    __syncthreads();
    if (it + 1 >= nqt) break;
    fr.refresh();
    fc.refresh();
    if constexpr (K_LDS) pk.refresh();
    if constexpr (V_LDS) pv.refresh();
    qdma.refresh();
    if (it + 2 < nqt) {
      qdma.issue(Qh, (it + 2) * BQ, N, qbuf0, wave, lane);
      qdma.issue(dOh, (it + 2) * BQ, N, dbuf0, wave, lane);
      srow.load(lseh, delh, (it + 2) * BQ, N, tid);
    }
    if constexpr (ATOMIC && DEFER) M::atomic_dq(dst0, ktile, dqh, it * BQ, N, a.scale, wave, g, l32, lane);
    M::tile(qbuf1, dbuf1, st1, ktile, vtile, DEFER ? dst1 : dst0, kf, vf, dk, dv, dqh, (it + 1) * BQ, k0, kw, key, N,
            c, a.scale, fr, fc, pk, pv, wave, g, l32, lane, dc, ks);
    if constexpr (ATOMIC && !DEFER) {
      __syncthreads();
      M::atomic_dq(dst0, ktile, dqh, (it + 1) * BQ, N, a.scale, wave, g, l32, lane);
    }
    wait_tile();
    if (it + 2 < nqt) srow.store(st0, N, tid);
    __syncthreads();
  }
  if constexpr (ATOMIC && DEFER) {  // dQ of the last query tile (its dS^T buffer alternates with the tile's parity)
    const int last = nqt - 1;
    M::atomic_dq(((last - qt0) & 1) ? dst1 : dst0, ktile, dqh, last * BQ, N, a.scale, wave, g, l32, lane);
  }

  if (key < N) {
    float* dkr = a.dk + head_base(a.vdk, bh, a.H) + (size_t)key * a.vdk.sn;
    float* dvr = a.dv + head_base(a.vdv, bh, a.H) + (size_t)key * a.vdv.sn;
    const float vs = DROP ? ks : 1.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int col = db * 32 + 8 * a4 + 4 * g;
        const f32x4 kv = {dk[db][4 * a4] * a.scale, dk[db][4 * a4 + 1] * a.scale, dk[db][4 * a4 + 2] * a.scale,
                          dk[db][4 * a4 + 3] * a.scale};
        const f32x4 vv = {dv[db][4 * a4] * vs, dv[db][4 * a4 + 1] * vs, dv[db][4 * a4 + 2] * vs,
                          dv[db][4 * a4 + 3] * vs};
        if (col < hd) {
          *(f32x4*)(dkr + col) = kv;
          *(f32x4*)(dvr + col) = vv;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Wide dK/dV kernel (both designs): each wave owns two 32-key blocks (64 keys), so
// every Q / dO row fragment and every transposed dO^T / Q^T fragment it reads from
// LDS feeds two MFMAs, one per key block (the kernel above feeds one).  The dK^T and
// dV^T accumulators of both blocks (4 D/32 fp32 x16 per lane) fill the accumulation
// registers at d = 128, so one wave runs per SIMD.  K comes from the workgroup's K
// tile in LDS (row fragments), V from registers.  Per 32-query block:
//   S_b = Q K_b^T,  dP_b = dO V_b^T       (b = 0, 1; Q / dO fragments shared)
//   P_b, dS_b                              elementwise, in registers
//   dV_b^T += dO^T P_b,  dK_b^T += Q^T dS_b  (dO^T / Q^T fragments shared)
// ATOMIC (the 5-GEMM design): each wave also writes its dS^T blocks to LDS, and at
// the start of the next query tile the workgroup computes dQ_tile = dS K over its
// BK = 64 NW keys (K by transposed reads of the same K tile) and adds it to dq with
// one fp32 atomic per dq element, as the kernel above does with its deferred form.
// D: LDS tile width; DV <= D (a multiple of 32): the head-dim columns computed (96 on
// 128-wide tiles, where the accumulators take 192 of the 256 accumulation registers).
template <int D, int DV, int BQ, int NW, bool CAUSAL, bool ATOMIC>
struct DkdvWideMath {
  static constexpr int BK = 64 * NW;
  static constexpr int QBN = BQ / 32;
  static constexpr int DB = DV / 32;
  static constexpr int KK = DV / 16;
  // the K tile serves row fragments (S) and, for the dQ product, transposed reads
  static constexpr int KMODE = ATOMIC ? kBoth : kRowOnly;

  __device__ __forceinline__ static void tile(const LDS char* qtl, const LDS char* dotl, const LDS float* stats,
                                              const LDS char* ktile, LDS char* dst, const bf16x8 (&vf)[2][KK],
                                              f32x16 (&dk)[2][DB], f32x16 (&dv)[2][DB], int q0, int kw, int key,
                                              int N, float c, const RowOffsets<D, kBoth>& fr,
                                              const ColOffsets<D, kBoth>& fc, const RowOffsets<D, KMODE>& pk,
                                              int wave, int g, int l32) {
    const LDS float* l2t = stats;
    const LDS float* dlt = stats + BQ;
#pragma unroll
    for (int qb = 0; qb < QBN; ++qb) {
      const int qbase = q0 + qb * 32;
      __builtin_amdgcn_sched_barrier(0);
      // blocks past the end (P = 0), or above the causal diagonal for all 64 keys,
      // contribute nothing; a block above the diagonal for the second key block
      // only is computed with P = 0 there
      if (qbase < N && (!CAUSAL || qbase + 31 >= kw)) {
        // S of both key blocks first (Q fragments shared), then P; then dP (dO fragments
        // shared) and dS.  Only one of S and dP is live at a time, which keeps both out
        // of the accumulation registers the dK/dV accumulators fill.
        // S and dP land in vector registers (mfma32v_*): the elementwise work reads them
        // there, and the dK/dV accumulators keep the accumulation registers to themselves.
        // The fragment reads run two k-steps ahead through three rotating slots.
        f32x16 p[2];
        {
          bf16x8 qa[3], k0f[3], k1f[3];
          auto ld = [&](int kk) {
            qa[kk % 3] = fr.row(qtl, qb * 32, kk);
            k0f[kk % 3] = pk.row(ktile, wave * 64, kk);
            k1f[kk % 3] = pk.row(ktile, wave * 64 + 32, kk);
          };
          ld(0);
          ld(1);
#pragma unroll
          for (int kk = 0; kk < KK; ++kk) {
            if (kk + 2 < KK) ld(kk + 2);
            const int sl = kk % 3;
            mfma32v_kstep(kk, KK, p[0], p[1], qa[sl], k0f[sl], qa[sl], k1f[sl]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        // register 8h + e <-> query row qb*32 + 16h + 8g + e of the tile
        float l2[16];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            const f32x4 lv = *(const LDS f32x4*)(l2t + qb * 32 + 16 * h + 8 * g + 4 * hf);
#pragma unroll
            for (int e = 0; e < 4; ++e) l2[8 * h + 4 * hf + e] = lv[e];
          }
        }
        // Queries past the end have lse2 = +inf (P = 0); keys past the end feed only
        // their own dK/dV columns, which are never stored.
        bf16x8 pb[2][2], sb[2][2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const int kb = key + 32 * b;
          // causal: scores of keys after the query are -inf (P = 0), in a pass of its own
          // that only diagonal blocks take (the empty asm keeps it a branch)
          if (CAUSAL && qbase < kw + 32 * b + 31) {
            asm volatile("");
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int q = qbase + 16 * (r >> 3) + 8 * g + (r & 7);
              if (kb > q) p[b][r] = -INFINITY;
            }
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) p[b][r] = exp2_hw(fmaf(p[b][r], c, -l2[r]));
          pb[b][0] = pack8(p[b], 0);
          pb[b][1] = pack8(p[b], 8);
        }
        __builtin_amdgcn_sched_barrier(0);
        f32x16 dp[2];
        {
          bf16x8 da[3];
          da[0] = fr.row(dotl, qb * 32, 0);
          da[1] = fr.row(dotl, qb * 32, 1);
#pragma unroll
          for (int kk = 0; kk < KK; ++kk) {
            if (kk + 2 < KK) da[(kk + 2) % 3] = fr.row(dotl, qb * 32, kk + 2);
            const int sl = kk % 3;
            mfma32v_kstep(kk, KK, dp[0], dp[1], da[sl], vf[0][kk], da[sl], vf[1][kk]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        float dl[16];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            const f32x4 dd = *(const LDS f32x4*)(dlt + qb * 32 + 16 * h + 8 * g + 4 * hf);
#pragma unroll
            for (int e = 0; e < 4; ++e) dl[8 * h + 4 * hf + e] = dd[e];
          }
        }
        if constexpr (!ATOMIC) {
          // dV products (they need only P), with the dS arithmetic between them (the VALU
          // work of one wave overlaps its own MFMAs when their results go to the
          // accumulation registers), then the dK products.  Transposed reads run one d
          // block ahead of their MFMAs.
          {
            bf16x8 o[2][2];
            o[0][0] = fc.col(dotl, qb * 32, 0);
            o[0][1] = fc.col(dotl, qb * 32 + 16, 0);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
              if (db + 1 < DB) {
                o[(db + 1) & 1][0] = fc.col(dotl, qb * 32, db + 1);
                o[(db + 1) & 1][1] = fc.col(dotl, qb * 32 + 16, db + 1);
              }
#pragma unroll
              for (int b = 0; b < 2; ++b) {
                dv[b][db] = mfma32(o[db & 1][0], pb[b][0], dv[b][db]);
                dv[b][db] = mfma32(o[db & 1][1], pb[b][1], dv[b][db]);
              }
              // this d block's share of the four 8-element halves of dS
#pragma unroll
              for (int hh = db * 4 / DB; hh < (db + 1) * 4 / DB; ++hh) {
                const int b = hh >> 1, h = hh & 1;
                bf16x8 v;
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = (__bf16)(p[b][8 * h + e] * (dp[b][8 * h + e] - dl[8 * h + e]));
                sb[b][h] = v;
              }
              __builtin_amdgcn_sched_barrier(0);
            }
          }
          {
            bf16x8 t[2][2];
            t[0][0] = fc.col(qtl, qb * 32, 0);
            t[0][1] = fc.col(qtl, qb * 32 + 16, 0);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
              if (db + 1 < DB) {
                t[(db + 1) & 1][0] = fc.col(qtl, qb * 32, db + 1);
                t[(db + 1) & 1][1] = fc.col(qtl, qb * 32 + 16, db + 1);
              }
#pragma unroll
              for (int b = 0; b < 2; ++b) {
                dk[b][db] = mfma32(t[db & 1][0], sb[b][0], dk[b][db]);
                dk[b][db] = mfma32(t[db & 1][1], sb[b][1], dk[b][db]);
              }
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        } else {
          // dS first, then the dV and dK products of each d block together (with the
          // dQ product's registers, the order above spills in this kernel)
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            f32x16 ds;
#pragma unroll
            for (int r = 0; r < 16; ++r) ds[r] = p[b][r] * (dp[b][r] - dl[r]);
            sb[b][0] = pack8(ds, 0);
            sb[b][1] = pack8(ds, 8);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const bf16x8 o0 = fc.col(dotl, qb * 32, db);
            const bf16x8 o1 = fc.col(dotl, qb * 32 + 16, db);
            const bf16x8 t0 = fc.col(qtl, qb * 32, db);
            const bf16x8 t1 = fc.col(qtl, qb * 32 + 16, db);
#pragma unroll
            for (int b = 0; b < 2; ++b) {
              dv[b][db] = mfma32(o0, pb[b][0], dv[b][db]);
              dv[b][db] = mfma32(o1, pb[b][1], dv[b][db]);
              dk[b][db] = mfma32(t0, sb[b][0], dk[b][db]);
              dk[b][db] = mfma32(t1, sb[b][1], dk[b][db]);
            }
          }
          // transposed reads (8 per d block) run one d block ahead of their 8 MFMAs
          __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
          for (int db = 0; db < DB - 1; ++db) {
            __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
        }
        if constexpr (ATOMIC) {
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            // keys past the end: K rows there are clamped copies, so their dS must not reach dQ
            // (under the causal mask they are above the diagonal, dS = 0 already)
            if (!CAUSAL && key + 32 * b >= N) {
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                sb[b][0][e] = (__bf16)0.f;
                sb[b][1][e] = (__bf16)0.f;
              }
            }
            const int krow = wave * 64 + 32 * b + l32;
            *(LDS bf16x8*)(dst + tile_off<BQ, kBoth>(krow, qb * 32 + 8 * g)) = sb[b][0];
            *(LDS bf16x8*)(dst + tile_off<BQ, kBoth>(krow, qb * 32 + 16 + 8 * g)) = sb[b][1];
          }
        }
      } else if constexpr (ATOMIC) {
        bf16x8 z;
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] = (__bf16)0.f;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const int krow = wave * 64 + 32 * b + l32;
          *(LDS bf16x8*)(dst + tile_off<BQ, kBoth>(krow, qb * 32 + 8 * g)) = z;
          *(LDS bf16x8*)(dst + tile_off<BQ, kBoth>(krow, qb * 32 + 16 + 8 * g)) = z;
        }
      }
    }
  }

  // When the (query block, d block) pairs split evenly over the waves, every wave
  // issues exactly kAtomics atomic instructions per dQ product (none is skipped: rows
  // past the end fall outside the buffer range below and the hardware drops them),
  // and the kernel issues one product per query tile, so the end-of-tile wait can
  // leave them in flight: vmcnt retires in issue order, and the tile copies were
  // issued before them.
  static constexpr bool kEvenSplit = (QBN * DB) % NW == 0;
  static constexpr int kPerWave = (QBN * DB + NW - 1) / NW;  // (qb, db) pairs per wave (at most)
  static constexpr int kAtomics = 16 * kPerWave;
  static_assert(!ATOMIC || !kEvenSplit || kAtomics < 64, "vmcnt holds at most 63");

  // dQ_tile = dS K over the workgroup's BK keys (its dS^T blocks in LDS, written by
  // tile() of the previous query tile and made visible by the barrier that ended it),
  // one fp32 atomic per dq element; the waves split the (query block, d block) pairs.
  // The adds are buffer atomics over the head's N x DV accumulator.  The whole row
  // offset of every add sits in the vector offset (plus an immediate of at most
  // 3 DV * 4 bytes): the buffer range check covers the vector and immediate offsets
  // but not the scalar one, and it is what drops the adds of rows past the end
  // ((N + 32) * DV * 4 fits 32 bits; the launcher checks).
  __device__ __forceinline__ static void atomic_dq(const LDS char* dst, const LDS char* ktile, float* dqh, int q0,
                                                   int N, float scale, int wave, int g, int l32, int lane) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(dqh, (short)0, (int)((unsigned)N * (unsigned)(DV * 4)), 0x00020000);
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int t = wave + i * NW;
      if (!kEvenSplit && t >= QBN * DB) break;
      const int qb = t / DB, db = t % DB;
      f32x16 acc = zero16();
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        acc = mfma32(ColOffsets<BQ, kBoth>::col_dyn(dst, ks * 16, qb, lane),
                     ColOffsets<D, kBoth>::col_dyn(ktile, ks * 16, db, lane), acc);
      }
      // register r holds row q0 + 32 qb + 4 g + 8 (r / 4) + r % 4, column 32 db + l32
      const unsigned off = ((unsigned)(q0 + qb * 32 + 4 * g) * DV + db * 32 + l32) * 4u;
      static_assert(3 * DV * 4 < 4096, "the row step r % 4 must fit the 12-bit immediate offset");
#pragma unroll
      for (int r = 0; r < 16; ++r)
        __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(acc[r] * scale, rs,
                                                        off + (unsigned)(8 * (r >> 2) + (r & 3)) * (DV * 4), 0, 0);
    }
  }

  // End of a query tile: the tile copies issued at its start must have landed.  With
  // `atomics` true the last kAtomics vector-memory instructions of this wave are the
  // dQ atomics issued after those copies (and after the statistics load, which the
  // compiler waits for itself), and they may stay outstanding.
  __device__ __forceinline__ static void end_tile_wait(bool atomics) {
    if constexpr (ATOMIC && kEvenSplit) {
      if (atomics) {
        __builtin_amdgcn_s_waitcnt(vmcnt_wait(kAtomics));
        return;
      }
    }
    wait_tile();
  }
};

template <int D, int DV, int BQ, int NW, bool CAUSAL, bool ATOMIC>
__global__ __launch_bounds__(NW * 64, 1) void dkdv_wide_kernel(BwdArgs a) {
  using M = DkdvWideMath<D, DV, BQ, NW, CAUSAL, ATOMIC>;
  constexpr int BK = M::BK, DB = M::DB, KK = M::KK;
  constexpr int KMODE = M::KMODE;
  constexpr int DST_BYTES = ATOMIC ? BK * BQ * 2 : 16;
  constexpr int NT = NW * 64;
  constexpr int QTILE = BQ * D * 2;
  __shared__ __attribute__((aligned(1024))) char q0s[QTILE];
  __shared__ __attribute__((aligned(1024))) char d0s[QTILE];
  __shared__ __attribute__((aligned(1024))) char q1s[QTILE];
  __shared__ __attribute__((aligned(1024))) char d1s[QTILE];
  __shared__ __attribute__((aligned(16))) float st0s[2 * BQ];
  __shared__ __attribute__((aligned(16))) float st1s[2 * BQ];
  __shared__ __attribute__((aligned(1024))) char kts[BK * D * 2];
  // dS^T of alternate query tiles (the dQ product runs one tile late)
  __shared__ __attribute__((aligned(1024))) char dsts0[DST_BYTES];
  __shared__ __attribute__((aligned(1024))) char dsts1[DST_BYTES];
  LDS char* dst0 = (LDS char*)dsts0;
  LDS char* dst1 = (LDS char*)dsts1;
  LDS char* qbuf0 = (LDS char*)q0s;
  LDS char* dbuf0 = (LDS char*)d0s;
  LDS char* qbuf1 = (LDS char*)q1s;
  LDS char* dbuf1 = (LDS char*)d1s;
  LDS float* st0 = (LDS float*)st0s;
  LDS float* st1 = (LDS float*)st1s;
  LDS char* ktile = (LDS char*)kts;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const int N = a.N;
  const int nkt = (N + BK - 1) / BK;
  int bh, kt;
  if (CAUSAL) {
    causal_order(blockIdx.x, a.B * a.H, nkt, false, bh, kt);  // low key tiles see the most queries
  } else {
    const int item = xcd_remap(blockIdx.x, a.B * a.H * nkt);
    bh = item / nkt;
    kt = item % nkt;
  }
  const __bf16* Qh = a.q + head_base(a.vq, bh, a.H);
  const __bf16* Kh = a.k + head_base(a.vk, bh, a.H);
  const __bf16* Vh = a.v + head_base(a.vv, bh, a.H);
  const __bf16* dOh = a.dout + head_base(a.vdo, bh, a.H);
  const float* lseh = a.lse + (size_t)bh * N;
  const float* delh = a.delta + (size_t)bh * N;
  // the atomic dq is a contiguous [B, H, N, DV] accumulator (columns past the head dim
  // receive zeros, since K is zero there)
  float* dqh = ATOMIC ? a.dq + (size_t)bh * N * DV : nullptr;
  const int hd = a.hd;  // columns hd .. D-1 are zero padding
  const float c = a.scale * kLog2e;

  const int k0 = kt * BK;
  const int kw = k0 + wave * 64;  // the wave's keys: kw + l32 (block 0), kw + 32 + l32 (block 1)
  const int key = kw + l32;
  const int nqt = (N + BQ - 1) / BQ;
  const int qt0 = CAUSAL ? k0 / BQ : 0;
  // Q, dO: row fragments and transposed reads; one copier serves both (equal row pitches)
  TileDMA<BQ, D, NW, kBoth> qdma;
  qdma.init(wave, lane, a.vq.sn, hd);
  qdma.issue(Qh, qt0 * BQ, N, qbuf0, wave, lane);
  qdma.issue(dOh, qt0 * BQ, N, dbuf0, wave, lane);
  {
    TileDMA<BK, D, NW, KMODE> kd;
    kd.init(wave, lane, a.vk.sn, hd);
    kd.issue(Kh, k0, N, ktile, wave, lane);
  }
  RowStager<BQ, NT> srow;
  srow.load(lseh, delh, qt0 * BQ, N, tid);
  srow.store(st0, N, tid);

  bf16x8 vf[2][KK];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int vrow = min(key + 32 * b, N - 1);  // keys past the end are never stored
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) vf[b][kk] = load_row_chunk(Vh + (size_t)vrow * a.vv.sn, 2 * kk + g, hd >> 3);
  }
  f32x16 dk[2][DB], dv[2][DB];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      dk[b][db] = zero16();
      dv[b][db] = zero16();
    }
  }
  RowOffsets<D, kBoth> fr;
  fr.init(lane);
  ColOffsets<D, kBoth> fc;
  fc.init(lane);
  RowOffsets<D, KMODE> pk;
  pk.init(lane, true);
  if constexpr (ATOMIC && M::kEvenSplit) {
    // the first query tile's dQ product reads this buffer before any tile wrote it:
    // zeros, so that product adds 0 (it keeps every tile's atomic count equal)
    bf16x8 z;
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] = (__bf16)0.f;
    for (int i = tid; i < DST_BYTES / 16; i += NT) *(LDS bf16x8*)(dst1 + 16 * i) = z;
  }

  wait_tile();
  __syncthreads();
  for (int it = qt0; it < nqt; it += 2) {
    fr.refresh();
    fc.refresh();
    pk.refresh();
    qdma.refresh();
    if (it + 1 < nqt) {
      qdma.issue(Qh, (it + 1) * BQ, N, qbuf1, wave, lane);
      qdma.issue(dOh, (it + 1) * BQ, N, dbuf1, wave, lane);
    }
    // ATOMIC: the statistics load and store run on every path (past the last tile they
    // read a clamped row and fill the unused buffer), so the compiler's own wait for the
    // load can count the atomics issued after it instead of waiting for them
    if (ATOMIC || it + 1 < nqt) srow.load(lseh, delh, (it + 1) * BQ, N, tid);
    if constexpr (ATOMIC) {
      if constexpr (M::kEvenSplit) {  // at the first tile: the zeroed buffer, added to valid rows
        M::atomic_dq(dst1, ktile, dqh, (it > qt0 ? it - 1 : it) * BQ, N, a.scale, wave, g, l32, lane);
      } else if (it > qt0) {
        M::atomic_dq(dst1, ktile, dqh, (it - 1) * BQ, N, a.scale, wave, g, l32, lane);
      }
    }
    M::tile(qbuf0, dbuf0, st0, ktile, dst0, vf, dk, dv, it * BQ, kw, key, N, c, fr, fc, pk, wave, g, l32);
    M::end_tile_wait(ATOMIC);
    if (ATOMIC || it + 1 < nqt) srow.store(st1, N, tid);
    __syncthreads();
    if (it + 1 >= nqt) break;
    fr.refresh();
    fc.refresh();
    pk.refresh();
    qdma.refresh();
    if (it + 2 < nqt) {
      qdma.issue(Qh, (it + 2) * BQ, N, qbuf0, wave, lane);
      qdma.issue(dOh, (it + 2) * BQ, N, dbuf0, wave, lane);
    }
    if (ATOMIC || it + 2 < nqt) srow.load(lseh, delh, (it + 2) * BQ, N, tid);
    if constexpr (ATOMIC) M::atomic_dq(dst0, ktile, dqh, it * BQ, N, a.scale, wave, g, l32, lane);
    M::tile(qbuf1, dbuf1, st1, ktile, dst1, vf, dk, dv, (it + 1) * BQ, kw, key, N, c, fr, fc, pk, wave, g, l32);
    M::end_tile_wait(ATOMIC);
    if (ATOMIC || it + 2 < nqt) srow.store(st0, N, tid);
    __syncthreads();
  }
  if constexpr (ATOMIC) {  // dQ of the last query tile (its dS^T buffer alternates with the tile's parity)
    const int last = nqt - 1;
    M::atomic_dq(((last - qt0) & 1) ? dst1 : dst0, ktile, dqh, last * BQ, N, a.scale, wave, g, l32, lane);
  }

  // dK and dV through LDS as whole rows, each wave staging its blocks in its quarter of the
  // K tile (free once every wave is past the last dQ product, which reads it)
  if constexpr (ATOMIC) __syncthreads();
  constexpr int kRegion = BK * D * 2 / NW;
  LDS char* region = ktile + wave * kRegion;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int kb0 = kw + 32 * b;
    store_tile_rows<DB, kRegion>(dk[b], a.scale, region, a.dk + head_base(a.vdk, bh, a.H) + (size_t)kb0 * a.vdk.sn,
                                 a.vdk.sn, N - kb0, hd, lane);
    store_tile_rows<DB, kRegion>(dv[b], 1.f, region, a.dv + head_base(a.vdv, bh, a.H) + (size_t)kb0 * a.vdv.sn,
                                 a.vdv.sn, N - kb0, hd, lane);
  }
}

// ---------------------------------------------------------------------------
// dQ kernel of the 7-GEMM design: one workgroup owns BR = 32 * NW queries, each
// wave 32 (one per lane column), and walks the key/value tiles in the forward's
// direction, the tiles arriving by direct-to-LDS loads one tile ahead.  Per tile:
//   S^T = K Q^T,  dP^T = V dO^T     A = K / V row fragments (LDS), B = Q^T / dO^T
//   P^T, dS^T                        one lse and one delta per lane
//   dQ^T += K^T dS^T                 A = transposed reads of the K tile
// No atomics: each dq element is written once, so results are reproducible bit
// for bit (issue 1172: the 7-GEMM form is deterministic).
// VSP: S and dP as vector-register MFMAs (mfma32v_*), for the one-wave-per-SIMD shapes.
template <int D, int DV, int BC, bool CAUSAL, bool DROP, bool VSP = false>
struct DqMath {
  static constexpr int KB = BC / 32;
  static constexpr int DB = DV / 32;
  static constexpr int KK = DV / 16;
  __device__ __forceinline__ static void step(const LDS char* kt, const LDS char* vt, const bf16x8 (&qf)[KK],
                                              const bf16x8 (&dof)[KK], f32x16 (&dq)[DB], float lse2, float dl,
                                              int k0, int q_w, int qi, int N, float c,
                                              const RowOffsets<D, kBoth>& fkr, const ColOffsets<D, kBoth>& fkc,
                                              const RowOffsets<D, kRowOnly>& fvr, int g, const DropCtx& dc,
                                              float ks) {
    const bool need_mask = (k0 + BC > N) || (CAUSAL && k0 + BC - 1 > q_w);
    // draws of keys k0 + 32 kb + 16 h + 8 g + (0..7) for this lane's query
    u32x4 dr[DROP ? 2 * KB : 1];
    if constexpr (DROP) {
#pragma unroll
      for (int i = 0; i < 2 * KB; ++i) dr[i] = drop_draws(dc, ((k0 + 8 * g) >> 3) + 2 * i, qi);
    }
    bf16x8 dsb[2 * KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      f32x16 s, dp;
      if constexpr (VSP) {
        // S and dP in vector registers (the dQ accumulators hold the accumulation
        // registers at one wave per SIMD); K and V fragment reads two k-steps ahead
        bf16x8 ka[3], va[3];
        auto ld = [&](int kk) {
          ka[kk % 3] = fkr.row(kt, kb * 32, kk);
          va[kk % 3] = fvr.row(vt, kb * 32, kk);
        };
        ld(0);
        ld(1);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          if (kk + 2 < KK) ld(kk + 2);
          mfma32v_kstep(kk, KK, s, dp, ka[kk % 3], qf[kk], va[kk % 3], dof[kk]);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
        s = zero16();
        dp = zero16();
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          s = mfma32(fkr.row(kt, kb * 32, kk), qf[kk], s);
          dp = mfma32(fvr.row(vt, kb * 32, kk), dof[kk], dp);
          fence_every<4>(kk);
        }
      }
      // keys past the end, and (causal) keys after the query, score -inf (P = 0).  A
      // pass of its own, taken only on tiles that need it; the empty asm statement
      // keeps it a branch (speculated, it becomes per-element selects on every tile).
      if (need_mask) {
        asm volatile("");
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kidx = k0 + kb * 32 + 16 * (r >> 3) + 8 * g + (r & 7);
          if (kidx >= N || (CAUSAL && kidx > qi)) s[r] = -INFINITY;
        }
      }
      f32x16 ds;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = exp2_hw(fmaf(s[r], c, -lse2));
        float dpv = dp[r];
        if constexpr (DROP) dpv = drop_keep(dr[2 * kb + (r >> 3)], r & 7, dc.t) ? dpv * ks : 0.f;
        ds[r] = pv * (dpv - dl);
      }
      dsb[2 * kb] = pack8(ds, 0);
      dsb[2 * kb + 1] = pack8(ds, 8);
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int ks = 0; ks < 2 * KB; ++ks) dq[db] = mfma32(fkc.col(kt, ks * 16, db), dsb[ks], dq[db]);
    }
  }
};

template <int D, int DV, int BC, int NW, int OCC, bool CAUSAL, bool DROP>
__global__ __launch_bounds__(NW * 64, OCC) void dq_kernel(BwdArgs a) {
  using M = DqMath<D, DV, BC, CAUSAL, DROP, OCC == 1 && DV <= 352>;
  constexpr int BR = 32 * NW;
  constexpr int TILE = BC * D * 2;
  constexpr int DB = M::DB, KK = M::KK;
  // K, V double-buffered; one array where dQ is staged through it at the end
  LDS char *kbuf0, *vbuf0, *kbuf1, *vbuf1;
  if constexpr (OCC >= 2) {
    __shared__ __attribute__((aligned(1024))) char tiles_s[4 * TILE];
    kbuf0 = (LDS char*)tiles_s;
    vbuf0 = kbuf0 + TILE;
    kbuf1 = kbuf0 + 2 * TILE;
    vbuf1 = kbuf0 + 3 * TILE;
  } else {
    __shared__ __attribute__((aligned(1024))) char k0s[TILE];
    __shared__ __attribute__((aligned(1024))) char v0s[TILE];
    __shared__ __attribute__((aligned(1024))) char k1s[TILE];
    __shared__ __attribute__((aligned(1024))) char v1s[TILE];
    kbuf0 = (LDS char*)k0s;
    vbuf0 = (LDS char*)v0s;
    kbuf1 = (LDS char*)k1s;
    vbuf1 = (LDS char*)v1s;
  }

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const int N = a.N;
  const int nqt = (N + BR - 1) / BR;
  int bh, qt;
  if (CAUSAL) {
    causal_order(blockIdx.x, a.B * a.H, nqt, true, bh, qt);
  } else {
    const int item = xcd_remap(blockIdx.x, a.B * a.H * nqt);
    bh = item / nqt;
    qt = item % nqt;
  }
  const __bf16* Qh = a.q + head_base(a.vq, bh, a.H);
  const __bf16* Kh = a.k + head_base(a.vk, bh, a.H);
  const __bf16* Vh = a.v + head_base(a.vv, bh, a.H);
  const __bf16* dOh = a.dout + head_base(a.vdo, bh, a.H);
  const int hd = a.hd;  // columns hd .. D-1 are zero padding
  const float c = a.scale * kLog2e;
  const DropCtx dc{a.drop_k0, a.drop_k1, (unsigned)bh, a.drop_offset, a.drop_t};

  const int q_wg = qt * BR;
  const int q_w = q_wg + wave * 32;
  const int qi = q_w + l32;
  const int q_last = min(N, q_wg + BR) - 1;
  const int kv_end = CAUSAL ? q_last + 1 : N;
  const int nkt = (kv_end + BC - 1) / BC;
  TileDMA<BC, D, NW, kBoth> kdma;     // K: row fragments and transposed reads
  TileDMA<BC, D, NW, kRowOnly> vdma;  // V: row fragments only
  kdma.init(wave, lane, a.vk.sn, hd);
  vdma.init(wave, lane, a.vv.sn, hd);
  kdma.issue(Kh, 0, N, kbuf0, wave, lane);
  vdma.issue(Vh, 0, N, vbuf0, wave, lane);

  const int qrow = min(qi, N - 1);  // rows past the end get lse = +inf (P = 0) and are never stored
  bf16x8 qf[KK], dof[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    qf[kk] = load_row_chunk(Qh + (size_t)qrow * a.vq.sn, 2 * kk + g, hd >> 3);
    dof[kk] = load_row_chunk(dOh + (size_t)qrow * a.vdo.sn, 2 * kk + g, hd >> 3);
  }
  const float lse2 = qi < N ? a.lse[(size_t)bh * N + qi] * kLog2e : INFINITY;
  float dl;
  if (a.o) {
    // delta of the lane's row, sum_k dO_ik O_ik, from the dO chunks already in registers
    // (lane half g holds columns 16 kk + 8 g .. + 7) and the same columns of O
    const float* orow = a.o + head_base(a.vo, bh, a.H) + (size_t)qrow * a.vo.sn;
    float acc = 0.f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int ch = 2 * kk + g;
      if (ch < (hd >> 3)) {
        const f32x4 o0 = *(const f32x4*)(orow + 8 * ch);
        const f32x4 o1 = *(const f32x4*)(orow + 8 * ch + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc = fmaf((float)dof[kk][e], o0[e], acc);
          acc = fmaf((float)dof[kk][4 + e], o1[e], acc);
        }
      }
    }
    acc = half_swap_sum(acc);
    dl = qi < N ? acc : 0.f;
    if (g == 0 && qi < N) a.delta_out[(size_t)bh * N + qi] = acc;
  } else {
    dl = qi < N ? a.delta[(size_t)bh * N + qi] : 0.f;
  }
  f32x16 dq[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dq[db] = zero16();
  RowOffsets<D, kBoth> fkr;
  fkr.init(lane);
  ColOffsets<D, kBoth> fkc;
  fkc.init(lane);
  RowOffsets<D, kRowOnly> fvr;
  fvr.init(lane);

  wait_tile();
  __syncthreads();
  for (int j = 0; j < nkt; j += 2) {
    fkr.refresh();
    fkc.refresh();
    fvr.refresh();
    kdma.refresh();
    vdma.refresh();
    if (j + 1 < nkt) {
      kdma.issue(Kh, (j + 1) * BC, N, kbuf1, wave, lane);
      vdma.issue(Vh, (j + 1) * BC, N, vbuf1, wave, lane);
    }
    // waves wholly past the end (padding rows) or below this key tile's diagonal skip the tile
    if (q_w < N && (!CAUSAL || j * BC <= q_w + 31))
      M::step(kbuf0, vbuf0, qf, dof, dq, lse2, dl, j * BC, q_w, qi, N, c, fkr, fkc, fvr, g, dc, a.drop_scale);
    wait_tile();
    __syncthreads();
    if (j + 1 >= nkt) break;
    fkr.refresh();
    fkc.refresh();
    fvr.refresh();
    kdma.refresh();
    vdma.refresh();
    if (j + 2 < nkt) {
      kdma.issue(Kh, (j + 2) * BC, N, kbuf0, wave, lane);
      vdma.issue(Vh, (j + 2) * BC, N, vbuf0, wave, lane);
    }
    if (q_w < N && (!CAUSAL || (j + 1) * BC <= q_w + 31))
      M::step(kbuf1, vbuf1, qf, dof, dq, lse2, dl, (j + 1) * BC, q_w, qi, N, c, fkr, fkc, fvr, g, dc, a.drop_scale);
    wait_tile();
    __syncthreads();
  }

  if constexpr (OCC >= 2) {
    // dQ through LDS as whole rows (the tiles are free: every wave passed the last barrier)
    constexpr int kRegion = (4 * TILE / NW) & ~1023;
    store_tile_rows<DB, kRegion>(dq, a.scale, kbuf0 + wave * kRegion,
                                 a.dq + head_base(a.vdq, bh, a.H) + (size_t)q_w * a.vdq.sn, a.vdq.sn, N - q_w, hd,
                                 lane);
  } else if (qi < N) {
    float* dqr = a.dq + head_base(a.vdq, bh, a.H) + (size_t)qi * a.vdq.sn;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int col = db * 32 + 8 * a4 + 4 * g;
        const f32x4 val = {dq[db][4 * a4] * a.scale, dq[db][4 * a4 + 1] * a.scale, dq[db][4 * a4 + 2] * a.scale,
                           dq[db][4 * a4 + 3] * a.scale};
        if (col < hd) *(f32x4*)(dqr + col) = val;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dK/dV for head dims above 256 (tiles D = 384 wide, DV = 288 .. 384 computed columns).
// For 32 keys per wave, the dK^T/dV^T accumulators of all DV columns (DV registers per
// lane) plus the K and V fragments of the S = Q K^T and dP = dO V^T products (DV / 4
// each) exceed the register file, and K/V tiles in LDS next to the double-buffered Q/dO
// tiles exceed 160 KB.  So each workgroup accumulates one window of WIN = 128 columns
// (three workgroups per key tile): it recomputes S and dP over the full DV contraction (K
// and V in registers) and runs the dV/dK products, the stores and, ATOMIC (5-GEMM), the
// dQ product only for its window.  S and dP are therefore computed once per window -- the
// recompute-for-capacity trade that issue 1172 describes for large head dims, where the
// accumulators no longer fit (192-column windows, two per key tile, spill 90-340
// registers).  ATOMIC: dQ[:, window] = dS K[:, window] with the window's K columns in an
// LDS tile, one fp32 atomic per dq element and window.
template <int D, int DV, int WIN, int BQ, int NW, bool CAUSAL, bool ATOMIC>
__global__ __launch_bounds__(NW * 64, 1) void dkdv_split_kernel(BwdArgs a) {
  constexpr int BK = 32 * NW, QBN = BQ / 32, KK = DV / 16, DBW = WIN / 32;
  constexpr int NSPLIT = (DV + WIN - 1) / WIN;
  constexpr int NT = NW * 64;
  constexpr int QTILE = BQ * D * 2;
  constexpr int KW_BYTES = ATOMIC ? BK * WIN * 2 : 16;
  constexpr int DST_BYTES = ATOMIC ? BK * BQ * 2 : 16;
  static_assert(WIN % 128 == 0 && D == 384, "column windows are multiples of 128 on 384-wide tiles");
  // Q tiles in slots 0-1 and dO tiles in slots 2-3 of one array, the statistics of the two
  // query tiles in one array: buffers are picked by computed offsets, never through a table
  // of LDS pointers (which hides the accesses from the compiler's LDS allocation)
  __shared__ __attribute__((aligned(1024))) char qds[4 * QTILE];
  __shared__ __attribute__((aligned(16))) float sts[4 * BQ];
  __shared__ __attribute__((aligned(1024))) char kws[KW_BYTES];
  __shared__ __attribute__((aligned(1024))) char dsts[DST_BYTES];
  auto qbuf = [&](int i) { return (LDS char*)qds + i * QTILE; };
  auto dbuf = [&](int i) { return (LDS char*)qds + (2 + i) * QTILE; };
  auto stb = [&](int i) { return (LDS float*)sts + i * 2 * BQ; };
  LDS char* const kwin = (LDS char*)kws;
  LDS char* const dst = (LDS char*)dsts;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const int N = a.N;
  const int nkt = (N + BK - 1) / BK;
  const int split = blockIdx.x % NSPLIT;
  int bh, kt;
  if (CAUSAL) {
    causal_order(blockIdx.x / NSPLIT, a.B * a.H, nkt, false, bh, kt);
  } else {
    const int item = xcd_remap(blockIdx.x / NSPLIT, a.B * a.H * nkt);
    bh = item / nkt;
    kt = item % nkt;
  }
  const int c0 = split * WIN;                       // the window's first column
  const int dbv = min(DBW, (DV - c0) / 32);         // 32-column blocks of the window inside DV
  const __bf16* Qh = a.q + head_base(a.vq, bh, a.H);
  const __bf16* Kh = a.k + head_base(a.vk, bh, a.H);
  const __bf16* Vh = a.v + head_base(a.vv, bh, a.H);
  const __bf16* dOh = a.dout + head_base(a.vdo, bh, a.H);
  const float* lseh = a.lse + (size_t)bh * N;
  const float* delh = a.delta + (size_t)bh * N;
  float* dqh = ATOMIC ? a.dq + (size_t)bh * N * DV : nullptr;
  const int hd = a.hd;
  const float c = a.scale * kLog2e;

  const int k0 = kt * BK;
  const int kw = k0 + wave * 32;
  const int key = kw + l32;
  const int nqt = (N + BQ - 1) / BQ;
  const int qt0 = CAUSAL ? k0 / BQ : 0;
  TileDMA<BQ, D, NW, kBoth> qdma;
  qdma.init(wave, lane, a.vq.sn, hd);
  qdma.issue(Qh, qt0 * BQ, N, qbuf(0), wave, lane);
  qdma.issue(dOh, qt0 * BQ, N, dbuf(0), wave, lane);
  if constexpr (ATOMIC) {  // the window's K columns of the workgroup's keys (transposed reads)
    TileDMA<BK, WIN, NW, kColOnly> kd;
    kd.init(wave, lane, a.vk.sn, min(WIN, hd - c0));
    kd.issue(Kh + c0, k0, N, kwin, wave, lane);
  }
  RowStager<BQ, NT> srow;
  srow.load(lseh, delh, qt0 * BQ, N, tid);
  srow.store(stb(0), N, tid);

  bf16x8 kf[KK], vf[KK];
  {
    const int krow = min(key, N - 1);  // keys past the end: masked below, never stored
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      kf[kk] = load_row_chunk(Kh + (size_t)krow * a.vk.sn, 2 * kk + g, hd >> 3);
      vf[kk] = load_row_chunk(Vh + (size_t)krow * a.vv.sn, 2 * kk + g, hd >> 3);
    }
  }
  f32x16 dk[DBW], dv[DBW];
#pragma unroll
  for (int db = 0; db < DBW; ++db) {
    dk[db] = zero16();
    dv[db] = zero16();
  }
  RowOffsets<D, kBoth> fr;
  fr.init(lane);
  ColOffsets<D, kBoth> fc;
  fc.init(lane, c0 / 32);

  wait_tile();
  __syncthreads();
  for (int it = qt0; it < nqt; ++it) {
    const int cur = (it - qt0) & 1;
    fr.refresh();
    fc.refresh();
    qdma.refresh();
    if (it + 1 < nqt) {
      qdma.issue(Qh, (it + 1) * BQ, N, qbuf(cur ^ 1), wave, lane);
      qdma.issue(dOh, (it + 1) * BQ, N, dbuf(cur ^ 1), wave, lane);
      srow.load(lseh, delh, (it + 1) * BQ, N, tid);
    }
    const LDS char* qtl = qbuf(cur);
    const LDS char* dotl = dbuf(cur);
    const LDS float* l2t = stb(cur);
    const LDS float* dlt = stb(cur) + BQ;
    const int q0 = it * BQ;
#pragma unroll
    for (int qb = 0; qb < QBN; ++qb) {
      const int qbase = q0 + qb * 32;
      __builtin_amdgcn_sched_barrier(0);
      bf16x8 sb0, sb1;
      if (qbase < N && (!CAUSAL || qbase + 31 >= kw)) {
        // S and dP in vector registers (mfma32v_*; up to DV = 320, above that the extra
        // vector registers spill); Q and dO fragment reads two k-steps ahead
        f32x16 sc, dp;
        if constexpr (DV > 320) {
          sc = zero16();
          dp = zero16();
#pragma unroll
          for (int kk = 0; kk < KK; ++kk) {
            sc = mfma32(fr.row(qtl, qb * 32, kk), kf[kk], sc);
            dp = mfma32(fr.row(dotl, qb * 32, kk), vf[kk], dp);
            fence_every<4>(kk);
          }
        } else {
          bf16x8 qa[3], da[3];
          auto ld = [&](int kk) {
            qa[kk % 3] = fr.row(qtl, qb * 32, kk);
            da[kk % 3] = fr.row(dotl, qb * 32, kk);
          };
          ld(0);
          ld(1);
#pragma unroll
          for (int kk = 0; kk < KK; ++kk) {
            if (kk + 2 < KK) ld(kk + 2);
            mfma32v_kstep(kk, KK, sc, dp, qa[kk % 3], kf[kk], da[kk % 3], vf[kk]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        float l2[16], dl[16];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            const int r = qb * 32 + 16 * h + 8 * g + 4 * hf;
            const f32x4 lv = *(const LDS f32x4*)(l2t + r);
            const f32x4 dd = *(const LDS f32x4*)(dlt + r);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              l2[8 * h + 4 * hf + e] = lv[e];
              dl[8 * h + 4 * hf + e] = dd[e];
            }
          }
        }
        // queries past the end have lse2 = +inf (P = 0); causal: keys after the query score -inf
        if (CAUSAL && qbase < kw + 31) {
          asm volatile("");
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int q = qbase + 16 * (r >> 3) + 8 * g + (r & 7);
            if (key > q) sc[r] = -INFINITY;
          }
        }
        f32x16 p, ds;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = exp2_hw(fmaf(sc[r], c, -l2[r]));
          p[r] = pv;
          ds[r] = pv * (dp[r] - dl[r]);
        }
        const bf16x8 pb0 = pack8(p, 0), pb1 = pack8(p, 8);
        sb0 = pack8(ds, 0);
        sb1 = pack8(ds, 8);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int db = 0; db < DBW; ++db) {
          if (db < dbv) {
            dv[db] = mfma32(fc.col(dotl, qb * 32, db), pb0, dv[db]);
            dv[db] = mfma32(fc.col(dotl, qb * 32 + 16, db), pb1, dv[db]);
            dk[db] = mfma32(fc.col(qtl, qb * 32, db), sb0, dk[db]);
            dk[db] = mfma32(fc.col(qtl, qb * 32 + 16, db), sb1, dk[db]);
          }
          fence_every<2>(db);
        }
        if (!CAUSAL && key >= N) {  // clamped key rows must not reach dQ
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            sb0[e] = (__bf16)0.f;
            sb1[e] = (__bf16)0.f;
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          sb0[e] = (__bf16)0.f;
          sb1[e] = (__bf16)0.f;
        }
      }
      if constexpr (ATOMIC) {
        *(LDS bf16x8*)(dst + tile_off<BQ, kBoth>(wave * 32 + l32, qb * 32 + 8 * g)) = sb0;
        *(LDS bf16x8*)(dst + tile_off<BQ, kBoth>(wave * 32 + l32, qb * 32 + 16 + 8 * g)) = sb1;
      }
    }
    if constexpr (ATOMIC) {
      // dQ[q0 .., window] = dS K[keys, window]: the waves split the (query block, d block) pairs
      __syncthreads();
      for (int t = wave; t < QBN * DBW; t += NW) {
        const int qb = t / DBW, db = t % DBW;
        if (db >= dbv) continue;
        f32x16 acc = zero16();
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
          acc = mfma32(ColOffsets<BQ, kBoth>::col_dyn(dst, ks * 16, qb, lane),
                       ColOffsets<WIN, kColOnly>::col_dyn(kwin, ks * 16, db, lane), acc);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int q = q0 + qb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          if (q < N) unsafeAtomicAdd(dqh + (size_t)q * DV + c0 + db * 32 + l32, acc[r] * a.scale);
        }
      }
    }
    wait_tile();
    if (it + 1 < nqt) srow.store(stb(cur ^ 1), N, tid);
    __syncthreads();
    // The last dK/dV products sit in a branch (db < dbv) at the end of the body; on the
    // loop-exit path the compiler leaves 10 of the 12 wait states between that MFMA and the
    // first read of its accumulators (the register copies it places at the loop exit, ahead
    // of anything written after the loop).  Eight more at the end of every iteration.
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7");
    __builtin_amdgcn_sched_barrier(0);
  }

  if (key < N) {
    float* dkr = a.dk + head_base(a.vdk, bh, a.H) + (size_t)key * a.vdk.sn;
    float* dvr = a.dv + head_base(a.vdv, bh, a.H) + (size_t)key * a.vdv.sn;
#pragma unroll
    for (int db = 0; db < DBW; ++db) {
      if (db >= dbv) continue;
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int col = c0 + db * 32 + 8 * a4 + 4 * g;
        const f32x4 kv = {dk[db][4 * a4] * a.scale, dk[db][4 * a4 + 1] * a.scale, dk[db][4 * a4 + 2] * a.scale,
                          dk[db][4 * a4 + 3] * a.scale};
        const f32x4 vv = {dv[db][4 * a4], dv[db][4 * a4 + 1], dv[db][4 * a4 + 2], dv[db][4 * a4 + 3]};
        if (col < hd) {
          *(f32x4*)(dkr + col) = kv;
          *(f32x4*)(dvr + col) = vv;
        }
      }
    }
  }
}

template <int D, int DV, int WIN, int BQ, int NW, bool ATOMIC>
static int launch_dkdv_split(const BwdArgs& a, bool causal, hipStream_t stream) {
  constexpr int BK = 32 * NW, NSPLIT = (DV + WIN - 1) / WIN;
  const int nkt = (a.N + BK - 1) / BK;
  const long long blocks = (long long)a.B * a.H * nkt * NSPLIT;
  if (blocks <= 0 || blocks > 0x7fffffff) return -1;
  if (a.drop_t != 0) return -1;
  if (causal) {
    hipLaunchKernelGGL((dkdv_split_kernel<D, DV, WIN, BQ, NW, true, ATOMIC>), dim3((unsigned)blocks), dim3(NW * 64), 0,
                       stream, a);
  } else {
    hipLaunchKernelGGL((dkdv_split_kernel<D, DV, WIN, BQ, NW, false, ATOMIC>), dim3((unsigned)blocks), dim3(NW * 64),
                       0, stream, a);
  }
  return 0;
}

// ---------------------------------------------------------------------------
template <int D, int DV, int BQ, int NW, bool ATOMIC, int KVL, bool DEFER = false, bool DROP = false>
static int launch_dkdv(const BwdArgs& a, bool causal, hipStream_t stream) {
  constexpr int BK = 32 * NW;
  const int nkt = (a.N + BK - 1) / BK;
  const long long blocks = (long long)a.B * a.H * nkt;
  if (blocks <= 0 || blocks > 0x7fffffff) return -1;
  if ((a.drop_t != 0) != DROP) return -1;
  if (causal) {
    hipLaunchKernelGGL((dkdv_kernel<D, DV, BQ, NW, true, ATOMIC, KVL, DEFER, DROP>), dim3((unsigned)blocks),
                       dim3(NW * 64), 0, stream, a);
  } else {
    hipLaunchKernelGGL((dkdv_kernel<D, DV, BQ, NW, false, ATOMIC, KVL, DEFER, DROP>), dim3((unsigned)blocks),
                       dim3(NW * 64), 0, stream, a);
  }
  return 0;
}

template <int D, int DV, int BQ, int NW, bool ATOMIC>
static int launch_dkdv_wide(const BwdArgs& a, bool causal, hipStream_t stream) {
  constexpr int BK = 64 * NW;
  const int nkt = (a.N + BK - 1) / BK;
  const long long blocks = (long long)a.B * a.H * nkt;
  if (blocks <= 0 || blocks > 0x7fffffff) return -1;
  if (a.drop_t != 0) return -1;
  // the atomic dQ product addresses a head's accumulator (plus 32 rows past its end)
  // with 32-bit buffer offsets; heads beyond that take the 8-wave kernel
  if (ATOMIC && ((long long)a.N + 32) * DV * 4 > 0xffffffffLL)
    return launch_dkdv<D, DV, DV == 64 ? 64 : 32, 8, true, 2, true>(a, causal, stream);
  if (causal) {
    hipLaunchKernelGGL((dkdv_wide_kernel<D, DV, BQ, NW, true, ATOMIC>), dim3((unsigned)blocks), dim3(NW * 64), 0, stream,
                       a);
  } else {
    hipLaunchKernelGGL((dkdv_wide_kernel<D, DV, BQ, NW, false, ATOMIC>), dim3((unsigned)blocks), dim3(NW * 64), 0, stream,
                       a);
  }
  return 0;
}

template <int D, int DV, int BC, int NW, int OCC, bool DROP = false>
static int launch_dq(const BwdArgs& a, bool causal, hipStream_t stream) {
  constexpr int BR = 32 * NW;
  const int nqt = (a.N + BR - 1) / BR;
  const long long blocks = (long long)a.B * a.H * nqt;
  if (blocks <= 0 || blocks > 0x7fffffff) return -1;
  if ((a.drop_t != 0) != DROP) return -1;
  if (causal) {
    hipLaunchKernelGGL((dq_kernel<D, DV, BC, NW, OCC, true, DROP>), dim3((unsigned)blocks), dim3(NW * 64), 0, stream, a);
  } else {
    hipLaunchKernelGGL((dq_kernel<D, DV, BC, NW, OCC, false, DROP>), dim3((unsigned)blocks), dim3(NW * 64), 0, stream,
                       a);
  }
  return 0;
}

// where K and V are read from (the KVL argument): registers, LDS tiles, or K from LDS
#define FA_KVL_NAME_false " kv_regs"
#define FA_KVL_NAME_true " kv_lds"
#define FA_KVL_NAME_0 " kv_regs"
#define FA_KVL_NAME_1 " kv_lds"
#define FA_KVL_NAME_2 " k_lds"
#define DKDV_CFG(D, BQ, NW, KVL) \
  { D, 32 * (NW), BQ, NW, "dkdv d" #D " Bk32x" #NW " Bq" #BQ FA_KVL_NAME_##KVL, &launch_dkdv<D, D, BQ, NW, false, KVL> }
#define DKDVA_CFG(D, BQ, NW, KVL)                                                                        \
  {                                                                                                        \
    D, 32 * (NW), BQ, NW, "dkdv+atomic-dq d" #D " Bk32x" #NW " Bq" #BQ FA_KVL_NAME_##KVL,                   \
        &launch_dkdv<D, D, BQ, NW, true, KVL>                                                              \
  }
#define DKDVAD_CFG(D, BQ, NW, KVL)                                                                       \
  {                                                                                                        \
    D, 32 * (NW), BQ, NW, "dkdv+atomic-dq d" #D " Bk32x" #NW " Bq" #BQ FA_KVL_NAME_##KVL " deferred",         \
        &launch_dkdv<D, D, BQ, NW, true, KVL, true>                                                        \
  }
// K read from the LDS tile of the dQ product, V in registers (KVL = 2)
#define DKDVADK_CFG(D, BQ, NW)                                                                           \
  {                                                                                                        \
    D, 32 * (NW), BQ, NW, "dkdv+atomic-dq d" #D " Bk32x" #NW " Bq" #BQ " k_lds deferred",                 \
        &launch_dkdv<D, D, BQ, NW, true, 2, true>                                                          \
  }
#define DKDVADK_CFGV(D, DV, BQ, NW)                                                                      \
  {                                                                                                        \
    DV, 32 * (NW), BQ, NW, "dkdv+atomic-dq d" #DV " (tiles " #D ") Bk32x" #NW " Bq" #BQ " k_lds deferred", \
        &launch_dkdv<D, DV, BQ, NW, true, 2, true>                                                         \
  }
#define DKDVK_CFG(D, BQ, NW) \
  { D, 32 * (NW), BQ, NW, "dkdv d" #D " Bk32x" #NW " Bq" #BQ " k_lds", &launch_dkdv<D, D, BQ, NW, false, 2> }
#define DKDVK_CFGV(D, DV, BQ, NW)                                                                        \
  {                                                                                                        \
    DV, 32 * (NW), BQ, NW, "dkdv d" #DV " (tiles " #D ") Bk32x" #NW " Bq" #BQ " k_lds",                  \
        &launch_dkdv<D, DV, BQ, NW, false, 2>                                                              \
  }
// two 32-key blocks per wave (dkdv_wide_kernel), K read from LDS
#define DKDVW_CFG(D, BQ, NW) \
  { D, 64 * (NW), BQ, NW, "dkdv d" #D " Bk64x" #NW " Bq" #BQ " k_lds wide", &launch_dkdv_wide<D, D, BQ, NW, false> }
#define DKDVAW_CFG(D, BQ, NW)                                                                             \
  {                                                                                                        \
    D, 64 * (NW), BQ, NW, "dkdv+atomic-dq d" #D " Bk64x" #NW " Bq" #BQ " k_lds deferred wide",            \
        &launch_dkdv_wide<D, D, BQ, NW, true>                                                              \
  }
#define DKDVW_CFGV(D, DV, BQ, NW)                                                                        \
  {                                                                                                        \
    DV, 64 * (NW), BQ, NW, "dkdv d" #DV " (tiles " #D ") Bk64x" #NW " Bq" #BQ " k_lds wide",             \
        &launch_dkdv_wide<D, DV, BQ, NW, false>                                                            \
  }
#define DKDVAW_CFGV(D, DV, BQ, NW)                                                                       \
  {                                                                                                        \
    DV, 64 * (NW), BQ, NW, "dkdv+atomic-dq d" #DV " (tiles " #D ") Bk64x" #NW " Bq" #BQ " k_lds deferred wide", \
        &launch_dkdv_wide<D, DV, BQ, NW, true>                                                             \
  }
#define DQ_CFG(D, BC, NW, OCC) \
  { D, 32 * (NW), BC, NW, "dq d" #D " Bq32x" #NW " Bc" #BC " occ" #OCC, &launch_dq<D, D, BC, NW, OCC> }
// head dim DV on D-wide tiles (the table's key is DV)
#define DKDV_CFGV(D, DV, BQ, NW, KVL)                                                                   \
  {                                                                                                        \
    DV, 32 * (NW), BQ, NW, "dkdv d" #DV " (tiles " #D ") Bk32x" #NW " Bq" #BQ FA_KVL_NAME_##KVL,            \
        &launch_dkdv<D, DV, BQ, NW, false, KVL>                                                            \
  }
#define DKDVA_CFGV(D, DV, BQ, NW, KVL)                                                                  \
  {                                                                                                        \
    DV, 32 * (NW), BQ, NW, "dkdv+atomic-dq d" #DV " (tiles " #D ") Bk32x" #NW " Bq" #BQ FA_KVL_NAME_##KVL,  \
        &launch_dkdv<D, DV, BQ, NW, true, KVL>                                                             \
  }
#define DQ_CFGV(D, DV, BC, NW, OCC)                                                                     \
  {                                                                                                        \
    DV, 32 * (NW), BC, NW, "dq d" #DV " (tiles " #D ") Bq32x" #NW " Bc" #BC " occ" #OCC,                 \
        &launch_dq<D, DV, BC, NW, OCC>                                                                     \
  }
#define DKDV_DROP_CFG(D, DV, BQ, NW, KVL)                                                               \
  {                                                                                                        \
    DV, 32 * (NW), BQ, NW, "dkdv+dropout d" #DV " Bk32x" #NW " Bq" #BQ FA_KVL_NAME_##KVL,                    \
        &launch_dkdv<D, DV, BQ, NW, false, KVL, false, true>                                               \
  }
#define DKDVA_DROP_CFG(D, DV, BQ, NW, KVL, DEF)                                                         \
  {                                                                                                        \
    DV, 32 * (NW), BQ, NW, "dkdv+atomic-dq+dropout d" #DV " Bk32x" #NW " Bq" #BQ FA_KVL_NAME_##KVL " defer" #DEF, \
        &launch_dkdv<D, DV, BQ, NW, true, KVL, DEF, true>                                                  \
  }
// head dims above 256: 384-wide tiles, three 128-column windows per key tile
#define DKDVS_CFG(DV)                                                                                    \
  {                                                                                                        \
    DV, 128, 32, 4, "dkdv d" #DV " (tiles 384) Bk32x4 Bq32 kv_regs split128", &launch_dkdv_split<384, DV, 128, 32, 4, false> \
  }
#define DKDVAS_CFG(DV)                                                                                   \
  {                                                                                                        \
    DV, 128, 32, 4, "dkdv+atomic-dq d" #DV " (tiles 384) Bk32x4 Bq32 kv_regs split128",                   \
        &launch_dkdv_split<384, DV, 128, 32, 4, true>                                                      \
  }
#define DQ_DROP_CFG(D, DV, BC, NW, OCC)                                                                 \
  {                                                                                                        \
    DV, 32 * (NW), BC, NW, "dq+dropout d" #DV " Bq32x" #NW " Bc" #BC " occ" #OCC,                         \
        &launch_dq<D, DV, BC, NW, OCC, true>                                                               \
  }

const BwdConfig* dkdv_configs(int* count) {
  static const BwdConfig table[] = {
      DKDV_CFG(64, 64, 4, false),  DKDV_CFG(64, 32, 4, false),  DKDV_CFG(64, 64, 8, false),
      DKDV_CFG(128, 64, 4, false), DKDV_CFG(128, 32, 4, false), DKDV_CFG(128, 32, 4, true),
      DKDV_CFG(128, 64, 4, true),  DKDV_CFG(128, 32, 2, true),
      DKDV_CFG(256, 32, 2, true),
      DKDVK_CFG(128, 64, 4), DKDVK_CFG(256, 32, 4),
      DKDV_CFGV(128, 96, 64, 4, false), DKDV_CFGV(128, 96, 64, 4, true), DKDV_CFGV(256, 192, 32, 2, true),
      DKDVK_CFGV(128, 96, 64, 4), DKDVK_CFGV(256, 192, 32, 4),
      DKDVW_CFG(64, 64, 4),  DKDVW_CFG(64, 32, 4),  DKDVW_CFG(128, 64, 4), DKDVW_CFG(128, 32, 4),
      DKDVW_CFGV(128, 96, 64, 4), DKDVW_CFGV(128, 96, 32, 4),
      // non-power-of-two workgroups: 160-224 keys (5-7 waves), 320 keys at d = 64
      DKDVK_CFG(128, 32, 5), DKDVK_CFG(128, 32, 6), DKDV_CFG(64, 64, 5, false), DKDV_CFG(64, 64, 6, false),
      DKDV_CFG(64, 64, 7, false), DKDV_CFG(64, 32, 10, false),
      DKDVS_CFG(288), DKDVS_CFG(320), DKDVS_CFG(352), DKDVS_CFG(384),
  };
  *count = (int)(sizeof(table) / sizeof(table[0]));
  return table;
}

const BwdConfig* dkdv_atomic_configs(int* count) {
  static const BwdConfig table[] = {
      DKDVA_CFG(64, 64, 4, false),  DKDVA_CFG(64, 32, 4, false),  DKDVA_CFG(64, 64, 8, false),
      DKDVAD_CFG(64, 64, 8, false),
      DKDVA_CFG(128, 64, 4, false), DKDVA_CFG(128, 32, 4, false), DKDVAD_CFG(128, 64, 4, false),
      DKDVA_CFG(256, 32, 2, true),
      DKDVADK_CFG(64, 64, 8), DKDVADK_CFG(128, 32, 8), DKDVADK_CFG(256, 32, 4),
      DKDVA_CFGV(128, 96, 64, 4, false), DKDVA_CFGV(256, 192, 32, 2, true),
      DKDVADK_CFGV(128, 96, 32, 8), DKDVADK_CFGV(256, 192, 32, 4),
      DKDVAW_CFG(64, 64, 4),  DKDVAW_CFG(64, 32, 4),  DKDVAW_CFG(128, 32, 4), DKDVAW_CFGV(128, 96, 32, 4),
      // non-power-of-two workgroups: 160-224 keys (5-7 waves)
      DKDVADK_CFG(128, 32, 5), DKDVADK_CFG(128, 32, 6), DKDVADK_CFG(64, 64, 5), DKDVADK_CFG(64, 64, 6),
      DKDVADK_CFG(64, 64, 7),
      DKDVAS_CFG(288), DKDVAS_CFG(320), DKDVAS_CFG(352), DKDVAS_CFG(384),
  };
  *count = (int)(sizeof(table) / sizeof(table[0]));
  return table;
}

const BwdConfig* dq_configs(int* count) {
  static const BwdConfig table[] = {
      DQ_CFG(64, 64, 4, 2),  DQ_CFG(64, 128, 4, 2), DQ_CFG(64, 64, 8, 2),
      DQ_CFG(128, 64, 4, 2), DQ_CFG(128, 32, 4, 2), DQ_CFG(128, 64, 8, 2),
      DQ_CFG(256, 32, 4, 1), DQ_CFG(256, 64, 4, 1),
      DQ_CFGV(128, 96, 64, 4, 2), DQ_CFGV(128, 96, 64, 8, 2), DQ_CFGV(256, 192, 32, 4, 1),
      // non-power-of-two workgroups: 160-224 query rows (5-7 waves)
      DQ_CFG(128, 64, 5, 2), DQ_CFG(128, 64, 6, 2), DQ_CFG(128, 64, 7, 2), DQ_CFG(64, 64, 5, 2),
      DQ_CFG(64, 64, 6, 2),
      DQ_CFGV(384, 288, 32, 4, 1), DQ_CFGV(384, 320, 32, 4, 1), DQ_CFGV(384, 352, 32, 4, 1),
      DQ_CFGV(384, 384, 32, 4, 1),
  };
  *count = (int)(sizeof(table) / sizeof(table[0]));
  return table;
}

// Dropout: the non-causal default shape of each head dim.
const BwdConfig* dkdv_dropout_configs(int* count) {
  static const BwdConfig table[] = {
      DKDV_DROP_CFG(64, 64, 64, 8, false), DKDV_DROP_CFG(128, 128, 64, 4, false), DKDV_DROP_CFG(256, 256, 32, 4, 2),
      DKDV_DROP_CFG(128, 96, 64, 4, 2),    DKDV_DROP_CFG(256, 192, 32, 4, 2),
  };
  *count = (int)(sizeof(table) / sizeof(table[0]));
  return table;
}

const BwdConfig* dkdv_atomic_dropout_configs(int* count) {
  static const BwdConfig table[] = {
      DKDVA_DROP_CFG(64, 64, 64, 8, 2, true),  DKDVA_DROP_CFG(128, 128, 32, 8, 2, true),
      DKDVA_DROP_CFG(256, 256, 32, 4, 2, true), DKDVA_DROP_CFG(128, 96, 32, 8, 2, true),
      DKDVA_DROP_CFG(256, 192, 32, 4, 2, true),
  };
  *count = (int)(sizeof(table) / sizeof(table[0]));
  return table;
}

const BwdConfig* dq_dropout_configs(int* count) {
  static const BwdConfig table[] = {
      DQ_DROP_CFG(64, 64, 64, 4, 2), DQ_DROP_CFG(128, 128, 64, 8, 2), DQ_DROP_CFG(256, 256, 32, 4, 1),
      DQ_DROP_CFG(128, 96, 64, 8, 2), DQ_DROP_CFG(256, 192, 32, 4, 1),
  };
  *count = (int)(sizeof(table) / sizeof(table[0]));
  return table;
}

}  // namespace fa
