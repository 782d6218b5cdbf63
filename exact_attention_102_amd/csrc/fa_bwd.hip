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
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

__device__ __forceinline__ float bf16_bits_to_f32(unsigned short h) {
  return __builtin_bit_cast(float, ((unsigned)h) << 16);
}

// ---------------------------------------------------------------------------
// delta_i = sum_k dO_ik * O_ik; optionally zero dq.  D / 8 threads per row, each
// reading one 16-byte chunk of dO and two of O, then a shuffle reduction.
template <int D>
__global__ __launch_bounds__(256) void preprocess_kernel(PreArgs a) {
  constexpr int TPR = D / 8;
  constexpr int RPB = 256 / TPR;
  const int tid = threadIdx.x;
  const int row = blockIdx.x * RPB + tid / TPR;
  const int c = tid % TPR;
  float acc = 0.f;
  if (row < a.rows) {
    const size_t base = (size_t)row * D + c * 8;
    const u32x4 dv = *(const u32x4*)(a.dout + base);
    const f32x4 o0 = *(const f32x4*)(a.o + base);
    const f32x4 o1 = *(const f32x4*)(a.o + base + 4);
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
      *(f32x4*)(a.dq + base) = z;
      *(f32x4*)(a.dq + base + 4) = z;
    }
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, TPR);
  if (row < a.rows && c == 0) a.delta[row] = acc;
}

int launch_preprocess(const PreArgs& a, int d, hipStream_t stream) {
  const int rpb = 256 / (d / 8);
  const int blocks = (a.rows + rpb - 1) / rpb;
  switch (d) {
    case 64: hipLaunchKernelGGL(preprocess_kernel<64>, dim3(blocks), dim3(256), 0, stream, a); break;
    case 128: hipLaunchKernelGGL(preprocess_kernel<128>, dim3(blocks), dim3(256), 0, stream, a); break;
    case 256: hipLaunchKernelGGL(preprocess_kernel<256>, dim3(blocks), dim3(256), 0, stream, a); break;
    default: return -1;
  }
  return 0;
}

// ---------------------------------------------------------------------------
// Per-row statistics of a query tile in LDS: lse * log2(e) (+inf past the end, so
// that P = 0 there) and delta (0 past the end).
template <int BQ, int NT>
struct RowStager {
  float v;
  __device__ __forceinline__ void load(const float* lse, const float* delta, int q0, int N, int tid) {
    v = 0.f;
    if (tid < BQ) {
      const int q = q0 + tid;
      v = q < N ? lse[q] * kLog2e : INFINITY;
    } else if (tid < 2 * BQ) {
      const int q = q0 + tid - BQ;
      v = q < N ? delta[q] : 0.f;
    }
  }
  __device__ __forceinline__ void store(LDS float* dst, int tid) const {
    if (tid < 2 * BQ) dst[tid] = v;
  }
};

// ---------------------------------------------------------------------------
// dK/dV kernel.  One workgroup owns BK = 32 * NW keys of one (batch, head), each
// wave 32 of them (one key per lane column of the MFMA C layout).  It walks the
// query tiles (BQ rows of Q and dO, plus their lse and delta) through
// double-buffered LDS.  Per 32-query block:
//   S  = Q K^T,  dP = dO V^T          A = Q / dO row fragments (LDS),
//                                      B = K^T / V^T (registers or LDS)
//   P, dS                              elementwise, in registers
//   dV^T += dO^T P,  dK^T += Q^T dS    A = transposed LDS reads, B = P / dS
// ATOMIC (the 5-GEMM design): each wave also writes its dS^T block to LDS; after a
// barrier the workgroup computes dQ_tile = dS K over all BK keys (waves split the
// (query block, d block) pairs) and adds it to dq with fp32 atomics, one atomic
// per dq element per workgroup and query tile.
// KV_LDS keeps the workgroup's K and V in LDS instead of registers (large d).
template <int D, int BQ, int NW, bool CAUSAL, bool ATOMIC, bool KV_LDS>
__global__ __launch_bounds__(NW * 64) void dkdv_kernel(BwdArgs a) {
  constexpr int BK = 32 * NW;
  constexpr int NT = NW * 64;
  constexpr int QTILE = BQ * D * 2;
  constexpr int STAGE = 2 * QTILE + 2 * BQ * 4;
  constexpr int QBN = BQ / 32;
  constexpr int DB = D / 32;
  constexpr int KK = D / 16;
  constexpr int KT_BYTES = (ATOMIC || KV_LDS) ? BK * D * 2 : 0;
  constexpr int VT_BYTES = KV_LDS ? BK * D * 2 : 0;
  constexpr int DST_BYTES = ATOMIC ? BK * BQ * 2 : 0;
  __shared__ __attribute__((aligned(1024))) char smem_raw[2 * STAGE + KT_BYTES + VT_BYTES + DST_BYTES];
  LDS char* smem = (LDS char*)smem_raw;
  LDS char* ktile = smem + 2 * STAGE;
  LDS char* vtile = ktile + KT_BYTES;
  LDS char* dst = vtile + VT_BYTES;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int N = a.N;
  const int nkt = (N + BK - 1) / BK;
  const int item = xcd_remap(blockIdx.x, a.B * a.H * nkt);
  const int bh = item / nkt;
  const int kt = item % nkt;  // causal: low key tiles see the most queries and come first
  const size_t head = (size_t)bh * N * D;
  const __bf16* Qh = a.q + head;
  const __bf16* Kh = a.k + head;
  const __bf16* Vh = a.v + head;
  const __bf16* dOh = a.dout + head;
  const float* lseh = a.lse + (size_t)bh * N;
  const float* delh = a.delta + (size_t)bh * N;
  const float c = a.scale * kLog2e;

  const int k0 = kt * BK;
  const int kw = k0 + wave * 32;
  const int key = kw + l32;

  if constexpr (ATOMIC || KV_LDS) {
    TileStager<BK, D, NT> st;
    st.load(Kh, k0, N, tid);
    st.store(ktile, tid);
    if constexpr (KV_LDS) {
      st.load(Vh, k0, N, tid);
      st.store(vtile, tid);
    }
  }
  bf16x8 kf[KV_LDS ? 1 : KK], vf[KV_LDS ? 1 : KK];
  if constexpr (!KV_LDS) {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      if (key < N) {
        kf[kk] = *(const bf16x8*)(Kh + (size_t)key * D + kk * 16 + g * 8);
        vf[kk] = *(const bf16x8*)(Vh + (size_t)key * D + kk * 16 + g * 8);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          kf[kk][e] = (__bf16)0.f;
          vf[kk][e] = (__bf16)0.f;
        }
      }
    }
  }

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dk[db] = zero16();
    dv[db] = zero16();
  }

  const int nqt = (N + BQ - 1) / BQ;
  const int qt0 = CAUSAL ? k0 / BQ : 0;
  const int qrow = pi_row(l32);

  TileStager<BQ, D, NT> sq, sdo;
  RowStager<BQ, NT> srow;
  sq.load(Qh, qt0 * BQ, N, tid);
  sdo.load(dOh, qt0 * BQ, N, tid);
  srow.load(lseh, delh, qt0 * BQ, N, tid);
  sq.store(smem, tid);
  sdo.store(smem + QTILE, tid);
  srow.store((LDS float*)(smem + 2 * QTILE), tid);
  __syncthreads();

  for (int it = qt0; it < nqt; ++it) {
    const int buf = (it - qt0) & 1;
    const LDS char* qtl = smem + buf * STAGE;
    const LDS char* dotl = qtl + QTILE;
    const LDS float* l2t = (const LDS float*)(qtl + 2 * QTILE);
    const LDS float* dlt = l2t + BQ;
    const bool more = it + 1 < nqt;
    if (more) {
      sq.load(Qh, (it + 1) * BQ, N, tid);
      sdo.load(dOh, (it + 1) * BQ, N, tid);
      srow.load(lseh, delh, (it + 1) * BQ, N, tid);
    }
    const int q0 = it * BQ;
#pragma unroll
    for (int qb = 0; qb < QBN; ++qb) {
      const int qbase = q0 + qb * 32;
      const bool active = !CAUSAL || qbase + 31 >= kw;
      if (active) {
        f32x16 s = zero16(), dp = zero16();
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const bf16x8 qa = row_frag<D>(qtl, qb * 32 + qrow, kk * 16 + g * 8);
          const bf16x8 da = row_frag<D>(dotl, qb * 32 + qrow, kk * 16 + g * 8);
          bf16x8 kb, vb;
          if constexpr (KV_LDS) {
            kb = row_frag<D>(ktile, wave * 32 + l32, kk * 16 + g * 8);
            vb = row_frag<D>(vtile, wave * 32 + l32, kk * 16 + g * 8);
          } else {
            kb = kf[kk];
            vb = vf[kk];
          }
          s = mfma32(qa, kb, s);
          dp = mfma32(da, vb, dp);
        }
        // register 8h + e <-> query row qb*32 + 16h + 8g + e of the tile
        float l2[16], dl[16];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int r = qb * 32 + 16 * h + 8 * g + 4 * half;
            const f32x4 lv = *(const LDS f32x4*)(l2t + r);
            const f32x4 dd = *(const LDS f32x4*)(dlt + r);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              l2[8 * h + 4 * half + e] = lv[e];
              dl[8 * h + 4 * half + e] = dd[e];
            }
          }
        }
        const bool need_mask = (k0 + BK > N) || (CAUSAL && qbase < kw + 31);
        f32x16 p, ds;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float pv = exp2_hw(fmaf(s[r], c, -l2[r]));
          if (need_mask) {
            const int q = qbase + 16 * (r >> 3) + 8 * g + (r & 7);
            if (key >= N || (CAUSAL && key > q)) pv = 0.f;
          }
          p[r] = pv;
          ds[r] = pv * (dp[r] - dl[r]);
        }
        const bf16x8 pb0 = pack8(p, 0), pb1 = pack8(p, 8);
        const bf16x8 sb0 = pack8(ds, 0), sb1 = pack8(ds, 8);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          dv[db] = mfma32(col_frag<D>(dotl, qb * 32, db * 32, lane), pb0, dv[db]);
          dv[db] = mfma32(col_frag<D>(dotl, qb * 32 + 16, db * 32, lane), pb1, dv[db]);
          dk[db] = mfma32(col_frag<D>(qtl, qb * 32, db * 32, lane), sb0, dk[db]);
          dk[db] = mfma32(col_frag<D>(qtl, qb * 32 + 16, db * 32, lane), sb1, dk[db]);
        }
        if constexpr (ATOMIC) {
          *(LDS bf16x8*)(dst + tile_off<BQ>(wave * 32 + l32, qb * 32 + 8 * g)) = sb0;
          *(LDS bf16x8*)(dst + tile_off<BQ>(wave * 32 + l32, qb * 32 + 16 + 8 * g)) = sb1;
        }
      } else if constexpr (ATOMIC) {
        bf16x8 z;
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] = (__bf16)0.f;
        *(LDS bf16x8*)(dst + tile_off<BQ>(wave * 32 + l32, qb * 32 + 8 * g)) = z;
        *(LDS bf16x8*)(dst + tile_off<BQ>(wave * 32 + l32, qb * 32 + 16 + 8 * g)) = z;
      }
    }
    if constexpr (ATOMIC) {
      __syncthreads();
      float* dqh = a.dq + head;
      for (int t = wave; t < QBN * DB; t += NW) {
        const int qb = t / DB, db = t % DB;
        f32x16 acc = zero16();
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
          acc = mfma32(col_frag<BQ>(dst, ks * 16, qb * 32, lane), col_frag<D>(ktile, ks * 16, db * 32, lane), acc);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int q = q0 + qb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          if (q < N) unsafeAtomicAdd(dqh + (size_t)q * D + db * 32 + l32, acc[r] * a.scale);
        }
      }
    }
    if (more) {
      LDS char* nxt = smem + (buf ^ 1) * STAGE;
      sq.store(nxt, tid);
      sdo.store(nxt + QTILE, tid);
      srow.store((LDS float*)(nxt + 2 * QTILE), tid);
    }
    __syncthreads();
  }

  if (key < N) {
    float* dkr = a.dk + head + (size_t)key * D;
    float* dvr = a.dv + head + (size_t)key * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int col = db * 32 + 8 * a4 + 4 * g;
        const f32x4 kv = {dk[db][4 * a4] * a.scale, dk[db][4 * a4 + 1] * a.scale, dk[db][4 * a4 + 2] * a.scale,
                          dk[db][4 * a4 + 3] * a.scale};
        const f32x4 vv = {dv[db][4 * a4], dv[db][4 * a4 + 1], dv[db][4 * a4 + 2], dv[db][4 * a4 + 3]};
        *(f32x4*)(dkr + col) = kv;
        *(f32x4*)(dvr + col) = vv;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dQ kernel of the 7-GEMM design: one workgroup owns BR = 32 * NW queries, each
// wave 32 (one per lane column), and walks the key/value tiles in the forward's
// direction.  Per tile:
//   S^T = K Q^T,  dP^T = V dO^T     A = K / V row fragments (LDS), B = Q^T / dO^T
//   P^T, dS^T                        one lse and one delta per lane
//   dQ^T += K^T dS^T                 A = transposed reads of the K tile
// No atomics: each dq element is written once, so results are reproducible bit
// for bit ("Potential algorithmic improvements...": the 7-GEMM form is
// deterministic).
template <int D, int BC, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) void dq_kernel(BwdArgs a) {
  constexpr int BR = 32 * NW;
  constexpr int NT = NW * 64;
  constexpr int TILE = BC * D * 2;
  constexpr int KB = BC / 32;
  constexpr int DB = D / 32;
  constexpr int KK = D / 16;
  __shared__ __attribute__((aligned(1024))) char smem_raw[4 * TILE];
  LDS char* smem = (LDS char*)smem_raw;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int N = a.N;
  const int nqt = (N + BR - 1) / BR;
  const int item = xcd_remap(blockIdx.x, a.B * a.H * nqt);
  const int bh = item / nqt;
  const int qt = CAUSAL ? nqt - 1 - item % nqt : item % nqt;
  const size_t head = (size_t)bh * N * D;
  const __bf16* Qh = a.q + head;
  const __bf16* Kh = a.k + head;
  const __bf16* Vh = a.v + head;
  const __bf16* dOh = a.dout + head;
  const float c = a.scale * kLog2e;

  const int q_wg = qt * BR;
  const int q_w = q_wg + wave * 32;
  const int qi = q_w + l32;

  bf16x8 qf[KK], dof[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    if (qi < N) {
      qf[kk] = *(const bf16x8*)(Qh + (size_t)qi * D + kk * 16 + g * 8);
      dof[kk] = *(const bf16x8*)(dOh + (size_t)qi * D + kk * 16 + g * 8);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        qf[kk][e] = (__bf16)0.f;
        dof[kk][e] = (__bf16)0.f;
      }
    }
  }
  const float lse2 = qi < N ? a.lse[(size_t)bh * N + qi] * kLog2e : INFINITY;
  const float dl = qi < N ? a.delta[(size_t)bh * N + qi] : 0.f;

  f32x16 dq[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dq[db] = zero16();

  const int q_last = min(N, q_wg + BR) - 1;
  const int kv_end = CAUSAL ? q_last + 1 : N;
  const int nkt = (kv_end + BC - 1) / BC;
  const int krow = pi_row(l32);

  TileStager<BC, D, NT> sk, sv;
  sk.load(Kh, 0, N, tid);
  sv.load(Vh, 0, N, tid);
  sk.store(smem, tid);
  sv.store(smem + TILE, tid);
  __syncthreads();

  for (int j = 0; j < nkt; ++j) {
    const LDS char* kt = smem + (j & 1) * 2 * TILE;
    const LDS char* vt = kt + TILE;
    const bool more = j + 1 < nkt;
    if (more) {
      sk.load(Kh, (j + 1) * BC, N, tid);
      sv.load(Vh, (j + 1) * BC, N, tid);
    }
    const int k0 = j * BC;
    const bool active = !CAUSAL || k0 <= q_w + 31;
    if (active) {
      const bool need_mask = (k0 + BC > N) || (CAUSAL && k0 + BC - 1 > q_w);
      bf16x8 dsb[2 * KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        f32x16 s = zero16(), dp = zero16();
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const bf16x8 ka = row_frag<D>(kt, kb * 32 + krow, kk * 16 + g * 8);
          const bf16x8 va = row_frag<D>(vt, kb * 32 + krow, kk * 16 + g * 8);
          s = mfma32(ka, qf[kk], s);
          dp = mfma32(va, dof[kk], dp);
        }
        f32x16 ds;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float pv = exp2_hw(fmaf(s[r], c, -lse2));
          if (need_mask) {
            const int kidx = k0 + kb * 32 + 16 * (r >> 3) + 8 * g + (r & 7);
            if (kidx >= N || (CAUSAL && kidx > qi)) pv = 0.f;
          }
          ds[r] = pv * (dp[r] - dl);
        }
        dsb[2 * kb] = pack8(ds, 0);
        dsb[2 * kb + 1] = pack8(ds, 8);
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int ks = 0; ks < 2 * KB; ++ks) {
          dq[db] = mfma32(col_frag<D>(kt, ks * 16, db * 32, lane), dsb[ks], dq[db]);
        }
      }
    }
    if (more) {
      LDS char* nt = smem + ((j + 1) & 1) * 2 * TILE;
      sk.store(nt, tid);
      sv.store(nt + TILE, tid);
    }
    __syncthreads();
  }

  if (qi < N) {
    float* dqr = a.dq + head + (size_t)qi * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const f32x4 val = {dq[db][4 * a4] * a.scale, dq[db][4 * a4 + 1] * a.scale, dq[db][4 * a4 + 2] * a.scale,
                           dq[db][4 * a4 + 3] * a.scale};
        *(f32x4*)(dqr + db * 32 + 8 * a4 + 4 * g) = val;
      }
    }
  }
}

// ---------------------------------------------------------------------------
template <int D, int BQ, int NW, bool ATOMIC, bool KV_LDS>
static int launch_dkdv(const BwdArgs& a, bool causal, hipStream_t stream) {
  constexpr int BK = 32 * NW;
  const int nkt = (a.N + BK - 1) / BK;
  const long long blocks = (long long)a.B * a.H * nkt;
  if (blocks <= 0 || blocks > 0x7fffffff) return -1;
  if (causal) {
    hipLaunchKernelGGL((dkdv_kernel<D, BQ, NW, true, ATOMIC, KV_LDS>), dim3((unsigned)blocks), dim3(NW * 64), 0,
                       stream, a);
  } else {
    hipLaunchKernelGGL((dkdv_kernel<D, BQ, NW, false, ATOMIC, KV_LDS>), dim3((unsigned)blocks), dim3(NW * 64), 0,
                       stream, a);
  }
  return 0;
}

template <int D, int BC, int NW>
static int launch_dq(const BwdArgs& a, bool causal, hipStream_t stream) {
  constexpr int BR = 32 * NW;
  const int nqt = (a.N + BR - 1) / BR;
  const long long blocks = (long long)a.B * a.H * nqt;
  if (blocks <= 0 || blocks > 0x7fffffff) return -1;
  if (causal) {
    hipLaunchKernelGGL((dq_kernel<D, BC, NW, true>), dim3((unsigned)blocks), dim3(NW * 64), 0, stream, a);
  } else {
    hipLaunchKernelGGL((dq_kernel<D, BC, NW, false>), dim3((unsigned)blocks), dim3(NW * 64), 0, stream, a);
  }
  return 0;
}

#define DKDV_CFG(D, BQ, NW, KVL) \
  { D, 32 * (NW), BQ, NW, "dkdv d" #D " Bk32x" #NW " Bq" #BQ " kv_lds" #KVL, &launch_dkdv<D, BQ, NW, false, KVL> }
#define DKDVA_CFG(D, BQ, NW, KVL) \
  { D, 32 * (NW), BQ, NW, "dkdv+atomic-dq d" #D " Bk32x" #NW " Bq" #BQ " kv_lds" #KVL, &launch_dkdv<D, BQ, NW, true, KVL> }
#define DQ_CFG(D, BC, NW) \
  { D, 32 * (NW), BC, NW, "dq d" #D " Bq32x" #NW " Bc" #BC, &launch_dq<D, BC, NW> }

const BwdConfig* dkdv_configs(int* count) {
  static const BwdConfig table[] = {
      DKDV_CFG(64, 32, 4, false),  DKDV_CFG(64, 64, 4, false),
      DKDV_CFG(128, 32, 4, false), DKDV_CFG(128, 64, 4, false),
      DKDV_CFG(256, 32, 2, true),
  };
  *count = (int)(sizeof(table) / sizeof(table[0]));
  return table;
}

const BwdConfig* dkdv_atomic_configs(int* count) {
  static const BwdConfig table[] = {
      DKDVA_CFG(64, 32, 4, false), DKDVA_CFG(64, 64, 4, false),
      DKDVA_CFG(128, 32, 4, false), DKDVA_CFG(128, 64, 4, false),
      DKDVA_CFG(256, 32, 2, true),
  };
  *count = (int)(sizeof(table) / sizeof(table[0]));
  return table;
}

const BwdConfig* dq_configs(int* count) {
  static const BwdConfig table[] = {
      DQ_CFG(64, 64, 4),  DQ_CFG(64, 128, 4),
      DQ_CFG(128, 32, 4), DQ_CFG(128, 64, 4),
      DQ_CFG(256, 32, 4),
  };
  *count = (int)(sizeof(table) / sizeof(table[0]));
  return table;
}

}  // namespace fa
