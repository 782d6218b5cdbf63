// fa_fwd.hip -- fused attention forward for gfx950.
//
// One workgroup owns BR = 32 * NW query rows of one (batch, head); each of its NW
// waves owns 32 of them, one per MFMA lane column.  The workgroup walks the
// key/value tiles (BC keys each) through double-buffered LDS ("ELI5:
// FlashAttention": tiling and kernel fusion -- S and P live only in registers), and
// keeps, per query row, the running maximum m and running exp-sum l of the online
// softmax (same page, the m(x)/l(x) statistics).  Per tile:
//   S^T = K Q^T          MFMA, A = K row fragments from LDS, B = Q^T in registers
//   mask, row max        in-lane over 16 keys per 32-key block + one half swap
//   P^T = exp2(S^T * c - m)   c = scale * log2(e) folded into one FMA
//   O^T += V^T P^T       MFMA, A = V^T via transposed LDS reads, B = P^T from
//                        the S^T accumulators (bf16, round-to-nearest-even)
// The transposed orientation (keys down the MFMA rows, one query per lane column)
// keeps every row statistic in-lane.  K/V tiles move HBM -> LDS by direct-to-LDS
// loads issued one tile ahead, so no registers stage them.
//
// Rescaling is lazy: m only moves (and O, l are rescaled by exp2(m_old - m_new))
// when some row's tile maximum exceeds its running m by more than kRescaleSlack
// (in log2 units).  Otherwise P is computed against the stale m, so P <= 2^slack;
// the result is unchanged in exact arithmetic because O and l carry the same
// factor and the final O / l cancels it, and lse uses the m actually applied.
// Two row sums are kept: l of the fp32 P (for lse) and l~ of the bf16-rounded P
// that the PV product actually consumes (one v_dot2c_f32_bf16 per pair).  O is
// divided by l~, so a row whose softmax is one-hot returns exactly that V row
// even when its dominant P is not a power of two; lse = ln(2) * (m + log2 l).
//
// DROP: dropout on P (fa_dropout.h).  The statistics m, l, l~ and lse stay those of
// the undropped P; the bf16 P^T fed to the PV product has its dropped entries
// zeroed, and the final O / l~ is multiplied by the keep scale.  The draws of a
// tile depend only on indices, so they are made before the tile's products.
#include "fa_device.h"
#include "fa_dropout.h"
#include "fa_launch.h"

namespace fa {

constexpr float kRescaleSlack = 8.0f;
// OPT: largest per-lane partial sum of P (over the lane's keys of one tile) accepted
// against a stale running maximum; P itself then stays at most 2^12.
constexpr float kOptLimit = 4096.0f;

// D: width of the LDS tiles (64, 128, 256); DV <= D, a multiple of 32: the head-dim
// columns actually computed (96 and 192 run on 128- and 256-wide tiles and skip the
// products of the zero columns).
template <int D, int DV, int BC, bool CAUSAL, bool DROP, bool OPT = false>
struct FwdTileMath {
  static constexpr int KB = BC / 32;  // 32-key blocks per tile
  static constexpr int DB = DV / 32;  // 32-wide blocks of the computed head dim
  static constexpr int KK = DV / 16;  // k-steps of Q K^T
  static constexpr int kAhead = 3;
  static constexpr int kAheadV = 3;
  // O accumulators in accumulation registers: the one-wave-per-SIMD shapes (d >= 192).
  // Under the causal mask these waves also run the tiles past their diagonal (fully
  // masked: P = 0, O unchanged) instead of branching around them: at the join of a
  // skipped and a computed tile the compiler copies all of O out of and back into the
  // accumulation registers every tile.
  static constexpr bool kAgprO = DV >= 192;
  // Software pipelining for these one-wave-per-SIMD shapes (optimistic statistics, no
  // dropout): the scores of tile j + 1 are computed before the P V product of tile j, and
  // their exp2 work runs between that product's MFMAs -- a wave overlaps its own VALU work
  // with MFMAs whose results go to the accumulation registers.  A/B against the plain
  // loop: 4-6% faster at d = 256 and 384 (32-key tiles); at d = 192 the 32-key tiles lost
  // 15-20% (the 64-key tiles gained 7-11% but stay slower than 32-key plain), so d = 192
  // keeps the plain loop.
  static constexpr bool kPipe = kAgprO && OPT && !DROP && KB <= 2 && DV >= 256;

  // One K/V tile for one wave: 32 queries (one per lane column) x BC keys.
  __device__ __forceinline__ static void step(const LDS char* kt, const LDS char* vt, const bf16x8 (&qf)[KK],
                                              f32x16 (&o)[DB], float& m_run, float& l_run, float& lb_run, int k0,
                                              int q_w, int qi, int N, float c, const RowOffsets<D, kRowOnly>& fk,
                                              const ColOffsets<D, kColOnly>& fv, int g, const DropCtx& dc,
                                              bool first) {
    // draws of keys k0 + 32 kb + 16 h + 8 g + (0..7) for this lane's query
    u32x4 dr[DROP ? 2 * KB : 1];
    if constexpr (DROP) {
#pragma unroll
      for (int ks = 0; ks < 2 * KB; ++ks) dr[ks] = drop_draws(dc, ((k0 + 8 * g) >> 3) + 2 * ks, qi);
    }
    f32x16 s[KB];
    if constexpr (kAgprO && KB <= 2) {
      // S in vector registers (mfma32v_*; O holds the accumulation registers); K
      // fragment reads two k-steps ahead through three rotating slots
      bf16x8 ka[3][KB];
      auto ld = [&](int kk) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) ka[kk % 3][kb] = fk.row(kt, kb * 32, kk);
      };
      ld(0);
      ld(1);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        if (kk + 2 < KK) ld(kk + 2);
        if constexpr (KB == 2)
          mfma32v_kstep(kk, KK, s[0], s[1], ka[kk % 3][0], qf[kk], ka[kk % 3][1], qf[kk]);
        else
          mfma32v_kstep1(kk, KK, s[0], ka[kk % 3][0], qf[kk]);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) s[kb] = zero16();
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) s[kb] = mfma32(fk.row(kt, kb * 32, kk), qf[kk], s[kb]);
      }
      // K fragment reads run kAhead k-steps ahead of their MFMAs (LDS latency hides
      // under the previous k-steps' products)
      __builtin_amdgcn_sched_group_barrier(0x100, KB * kAhead, 0);
#pragma unroll
      for (int kk = 0; kk < KK - kAhead; ++kk) {
        __builtin_amdgcn_sched_group_barrier(0x008, KB, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, KB, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, KB * kAhead, 0);
    }
    // keys past the end, and (causal) keys after the query, score -inf
    if ((k0 + BC > N) || (CAUSAL && k0 + BC - 1 > q_w)) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + kb * 32 + 16 * (r >> 3) + 8 * g + (r & 7);
          if (key >= N || (CAUSAL && key > qi)) s[kb][r] = -INFINITY;
        }
      }
    }
    bf16x8 pb[2 * KB];
    float rs = 0.f, rb = 0.f;
    // OPT (optimistic statistics): after the first tile, P is computed against the running m
    // without first taking the tile's row maximum; only if some lane's partial sum of P
    // leaves (0, kOptLimit] (an element above the limit, an overflow, or a NaN) does the wave
    // take the maximum and rescale, then recompute P.  The scores stay in s until that test.
    if (OPT && !first) {
      const float nm = -m_run;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float p8[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            p8[e] = exp2_hw(fmaf(s[kb][8 * h + e], c, nm));
            rs += p8[e];
          }
          bf16x8 b;
#pragma unroll
          for (int e = 0; e < 8; ++e) b[e] = (__bf16)p8[e];
          pb[2 * kb + h] = b;
        }
      }
      if (__builtin_amdgcn_ballot_w64(!(rs <= kOptLimit)) == 0) goto have_p;
    }
    {
      float mx = s[0][0];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int r = (kb == 0 ? 1 : 0); r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      }
      mx = half_swap_max(mx) * c;
      // Tile 0 holds key 0 <= every query, so m_run is finite after the first tile.
      const bool grow = OPT ? mx > m_run : mx > m_run + kRescaleSlack;
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
        const float m_new = grow ? mx : m_run;
        const float alpha = exp2_hw(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
        lb_run *= alpha;
        if constexpr (kAgprO) {
          // O lives in accumulation registers (one wave per SIMD): scale it in place.  With
          // plain multiplies the compiler copies all of O into vector registers at the top of
          // every tile, whether or not the tile rescales.
#pragma unroll
          for (int db = 0; db < DB; ++db) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              float x = o[db][r], t;
              asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                           : "+a"(x), "=&v"(t)
                           : "v"(alpha));
              o[db][r] = x;
            }
          }
          asm volatile("s_nop 2");  // accumulation-register writes before the next MFMA reads them
        } else {
#pragma unroll
          for (int db = 0; db < DB; ++db) {
#pragma unroll
            for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
          }
        }
      }
      const float nm = -m_run;
      rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = exp2_hw(fmaf(s[kb][r], c, nm));
          s[kb][r] = p;
          rs += p;
        }
        pb[2 * kb] = pack8(s[kb], 0);
        pb[2 * kb + 1] = pack8(s[kb], 8);
      }
    }
  have_p:
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      rb = sum_bf16x8(pb[2 * kb], rb);
      rb = sum_bf16x8(pb[2 * kb + 1], rb);
      if constexpr (DROP) {
        pb[2 * kb] = drop_mask8(pb[2 * kb], dr[2 * kb], dc.t);
        pb[2 * kb + 1] = drop_mask8(pb[2 * kb + 1], dr[2 * kb + 1], dc.t);
      }
    }
    l_run += rs;
    lb_run += rb;
#pragma unroll
    for (int ks = 0; ks < 2 * KB; ++ks) {
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] = mfma32(fv.col(vt, ks * 16, db), pb[ks], o[db]);
    }
    // transposed V reads (two per MFMA) run kAheadV MFMAs ahead
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kAheadV, 0);
#pragma unroll
    for (int i = 0; i < 2 * KB * DB - kAheadV; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kAheadV, 0);
  }

  // ---- pipelined path (kPipe) ----
  // S = K Q^T of one tile in vector registers, then the mask of keys past the end and
  // (causal) keys after the query
  __device__ __forceinline__ static void scores(const LDS char* kt, const bf16x8 (&qf)[KK], f32x16 (&s)[KB], int k0,
                                                int q_w, int qi, int N, const RowOffsets<D, kRowOnly>& fk, int g) {
    bf16x8 ka[3][KB];
    auto ld = [&](int kk) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) ka[kk % 3][kb] = fk.row(kt, kb * 32, kk);
    };
    ld(0);
    ld(1);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      if (kk + 2 < KK) ld(kk + 2);
      if constexpr (KB == 2)
        mfma32v_kstep(kk, KK, s[0], s[1], ka[kk % 3][0], qf[kk], ka[kk % 3][1], qf[kk]);
      else
        mfma32v_kstep1(kk, KK, s[0], ka[kk % 3][0], qf[kk]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if ((k0 + BC > N) || (CAUSAL && k0 + BC - 1 > q_w)) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + kb * 32 + 16 * (r >> 3) + 8 * g + (r & 7);
          if (key >= N || (CAUSAL && key > qi)) s[kb][r] = -INFINITY;
        }
      }
    }
  }
  // Exact statistics of a tile: its row maximum; when that exceeds the running one, O and
  // the sums are scaled by exp2(m_old - m_new) in place (FIRST: nothing accumulated yet);
  // then P against the maximum into the bf16 operand, its sums into rs, rb.
  template <bool FIRST>
  __device__ __forceinline__ static void exact_p(const f32x16 (&s)[KB], float c, float& m_run, float& l_run,
                                                 float& lb_run, f32x16 (&o)[DB], bf16x8 (&pb)[2 * KB], float& rs,
                                                 float& rb) {
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int r = (kb == 0 ? 1 : 0); r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    }
    mx = half_swap_max(mx) * c;
    const bool grow = mx > m_run;  // m_run = -inf before the first tile
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float m_new = grow ? mx : m_run;
      const float alpha = exp2_hw(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
      lb_run *= alpha;
      if constexpr (!FIRST) {
        // the P V MFMAs that last wrote O may still run: 12 wait states before reading it
        asm volatile("s_nop 7\n\ts_nop 4");
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float x = o[db][r], t;
            asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                         : "+a"(x), "=&v"(t)
                         : "v"(alpha));
            o[db][r] = x;
          }
        }
        asm volatile("s_nop 2");  // accumulation-register writes before the next MFMA reads them
      }
    }
    const float nm = -m_run;
    rs = 0.f;
    rb = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        bf16x8 b;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = exp2_hw(fmaf(s[kb][8 * h + e], c, nm));
          rs += p;
          b[e] = (__bf16)p;
        }
        pb[2 * kb + h] = b;
        rb = sum_bf16x8(b, rb);
      }
    }
  }
  // O += V^T P^T of the current tile (pb), with the optimistic P of the next tile (scores
  // sn against the running maximum, -nm) formed between the MFMAs into pbn, rsn, rbn.
  // NEXT false: the product alone (the last tile).
  template <bool NEXT>
  __device__ __forceinline__ static void pv(const LDS char* vt, const bf16x8 (&pb)[2 * KB], f32x16 (&o)[DB],
                                            const f32x16 (&sn)[KB], float c, float nm, bf16x8 (&pbn)[2 * KB],
                                            float& rsn, float& rbn, const ColOffsets<D, kColOnly>& fv) {
    constexpr int NPV = 2 * KB * DB, NEL = 16 * KB, R = kAheadV + 1;
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    bf16x8 vq[R];
#pragma unroll
    for (int i = 0; i < kAheadV && i < NPV; ++i) vq[i] = fv.col(vt, (i / DB) * 16, i % DB);
    rsn = 0.f;
    rbn = 0.f;
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      if (i + kAheadV < NPV) vq[(i + kAheadV) % R] = fv.col(vt, ((i + kAheadV) / DB) * 16, (i + kAheadV) % DB);
      o[i % DB] = mfma32(vq[i % R], pb[i / DB], o[i % DB]);
      if constexpr (NEXT) {
        // element pairs [i NEL / (2 NPV), (i + 1) NEL / (2 NPV)) of the next tile
#pragma unroll
        for (int pr = i * (NEL / 2) / NPV; pr < (i + 1) * (NEL / 2) / NPV; ++pr) {
          const int e = 2 * pr, kb = e >> 4, r = e & 15;
          const float p0 = exp2_hw(fmaf(sn[kb][r], c, nm));
          const float p1 = exp2_hw(fmaf(sn[kb][r + 1], c, nm));
          rsn += p0;
          rsn += p1;
          const bf16x2 b2 = {(__bf16)p0, (__bf16)p1};
          rbn = __builtin_amdgcn_fdot2_f32_bf16(b2, ones, rbn, false);
          pbn[e >> 3][r & 7] = b2[0];
          pbn[e >> 3][(r & 7) + 1] = b2[1];
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
};

// OCC: waves per SIMD the register allocation must allow (2 lets a second wave's
// MFMAs overlap this wave's softmax; d = 256 needs the whole register file).
template <int D, int DV, int BC, int NW, int OCC, bool CAUSAL, bool DROP, bool OPT>
__global__ __launch_bounds__(NW * 64, OCC) void fwd_kernel(FwdArgs a) {
  using M = FwdTileMath<D, DV, BC, CAUSAL, DROP, OPT>;
  constexpr int BR = 32 * NW;
  constexpr int TILE = BC * D * 2;  // bytes of one K or V tile
  constexpr int DB = M::DB, KK = M::KK, KB = M::KB;
  // K, V double-buffered; one array where the output is staged through it at the end
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
  const int hd = a.hd;  // columns hd .. D-1 are zero padding
  const float c = a.scale * kLog2e;
  const DropCtx dc{a.drop_k0, a.drop_k1, (unsigned)bh, a.drop_offset, a.drop_t};

  const int q_wg = qt * BR;
  const int q_w = q_wg + wave * 32;
  const int qi = q_w + l32;
  const int q_last = min(N, q_wg + BR) - 1;
  const int kv_end = CAUSAL ? q_last + 1 : N;
  const int nkt = (kv_end + BC - 1) / BC;
  TileDMA<BC, D, NW, kRowOnly> kdma;  // K: row fragments only
  TileDMA<BC, D, NW, kColOnly> vdma;  // V: transposed fragments only
  kdma.init(wave, lane, a.vk.sn, hd);
  vdma.init(wave, lane, a.vv.sn, hd);
  kdma.issue(Kh, 0, N, kbuf0, wave, lane);
  vdma.issue(Vh, 0, N, vbuf0, wave, lane);

  bf16x8 qf[KK];
  const int qrow = min(qi, N - 1);  // rows past the end duplicate the last row; never stored
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) qf[kk] = load_row_chunk(Qh + (size_t)qrow * a.vq.sn, 2 * kk + g, hd >> 3);

  float m_run = -INFINITY, l_run = 0.f, lb_run = 0.f;
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = zero16();
  RowOffsets<D, kRowOnly> fk;
  fk.init(lane);
  ColOffsets<D, kColOnly> fv;
  fv.init(lane);

  if constexpr (M::kPipe) {
    // Pipelined: K runs two tiles ahead, V one.  In iteration j the wave computes the scores
    // of tile j + 1 and the P V product of tile j (K_{j+1} and V_j resident, K_{j+2} and
    // V_{j+1} in flight).  Tile j's slots are k/v buffer j % 2.
    if (nkt > 1) kdma.issue(Kh, BC, N, kbuf1, wave, lane);
    wait_tile();
    __syncthreads();
    f32x16 s[KB];
    bf16x8 pb[2 * KB];
    float rs, rb;
    M::scores(kbuf0, qf, s, 0, q_w, qi, N, fk, g);
    M::template exact_p<true>(s, c, m_run, l_run, lb_run, o, pb, rs, rb);
    l_run += rs;
    lb_run += rb;
    // one iteration: kn/vc the slots of K_{j+1} and V_j, kf the slot K_{j+2} goes to (K_j's),
    // vn the slot V_{j+1} goes to (V_{j-1}'s)
    auto iter = [&](int j, const LDS char* kn, const LDS char* vc, LDS char* kf, LDS char* vn) {
      fk.refresh();
      fv.refresh();
      kdma.refresh();
      vdma.refresh();
      wait_tile();      // K_{j+1}, V_j landed
      __syncthreads();  // and every wave is past its reads of K_j and V_{j-1}
      vdma.issue(Vh, (j + 1) * BC, N, vn, wave, lane);
      if (j + 2 < nkt) kdma.issue(Kh, (j + 2) * BC, N, kf, wave, lane);
      f32x16 sn[KB];
      M::scores(kn, qf, sn, (j + 1) * BC, q_w, qi, N, fk, g);
      bf16x8 pbn[2 * KB];
      float rsn, rbn;
      M::template pv<true>(vc, pb, o, sn, c, -m_run, pbn, rsn, rbn, fv);
      if (__builtin_amdgcn_ballot_w64(!(rsn <= kOptLimit)) != 0)
        M::template exact_p<false>(sn, c, m_run, l_run, lb_run, o, pbn, rsn, rbn);
      l_run += rsn;
      lb_run += rbn;
#pragma unroll
      for (int i = 0; i < 2 * KB; ++i) pb[i] = pbn[i];
    };
    int j = 0;
    for (; j + 2 < nkt; j += 2) {
      iter(j, kbuf1, vbuf0, kbuf0, vbuf1);
      iter(j + 1, kbuf0, vbuf1, kbuf1, vbuf0);
    }
    if (j + 1 < nkt) {
      iter(j, kbuf1, vbuf0, kbuf0, vbuf1);
      ++j;
    }
    // the last tile's P V product (V_{nkt-1} in buffer (nkt - 1) % 2)
    wait_tile();
    __syncthreads();
    f32x16 sdummy[KB];
    bf16x8 pdummy[2 * KB];
    float r0, r1;
    M::template pv<false>((j & 1) ? vbuf1 : vbuf0, pb, o, sdummy, c, 0.f, pdummy, r0, r1, fv);
    wait_tile();
    __syncthreads();
  } else {
    wait_tile();
    __syncthreads();
    for (int j = 0; j < nkt; j += 2) {
      fk.refresh();
      fv.refresh();
      kdma.refresh();
      vdma.refresh();
      if (j + 1 < nkt) {
        kdma.issue(Kh, (j + 1) * BC, N, kbuf1, wave, lane);
        vdma.issue(Vh, (j + 1) * BC, N, vbuf1, wave, lane);
      }
      if (!CAUSAL || M::kAgprO || j * BC <= q_w + 31)
        M::step(kbuf0, vbuf0, qf, o, m_run, l_run, lb_run, j * BC, q_w, qi, N, c, fk, fv, g, dc, j == 0);
      wait_tile();
      __syncthreads();
      if (j + 1 >= nkt) break;
      fk.refresh();
      fv.refresh();
      kdma.refresh();
      vdma.refresh();
      if (j + 2 < nkt) {
        kdma.issue(Kh, (j + 2) * BC, N, kbuf0, wave, lane);
        vdma.issue(Vh, (j + 2) * BC, N, vbuf0, wave, lane);
      }
      if (!CAUSAL || M::kAgprO || (j + 1) * BC <= q_w + 31)
        M::step(kbuf1, vbuf1, qf, o, m_run, l_run, lb_run, (j + 1) * BC, q_w, qi, N, c, fk, fv, g, dc, false);
      wait_tile();
      __syncthreads();
    }
  }

  const float lt = half_swap_sum(l_run);
  const float inv = (DROP ? a.drop_scale : 1.f) / half_swap_sum(lb_run);
  if constexpr (OCC >= 2) {
    // O through LDS as whole rows (the tiles are free: every wave passed the last barrier).
    // The one-wave-per-SIMD shapes store directly: the staging's extra registers cost
    // them more than the wider stores gain.
    constexpr int kRegion = (4 * TILE / NW) & ~1023;
    store_tile_rows<DB, kRegion>(o, inv, kbuf0 + wave * kRegion,
                                 a.o + head_base(a.vo, bh, a.H) + (size_t)q_w * a.vo.sn, a.vo.sn, N - q_w, hd, lane);
  } else if (qi < N) {
    float* orow = a.o + head_base(a.vo, bh, a.H) + (size_t)qi * a.vo.sn;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int col = db * 32 + 8 * a4 + 4 * g;
        const f32x4 val = {o[db][4 * a4] * inv, o[db][4 * a4 + 1] * inv, o[db][4 * a4 + 2] * inv,
                           o[db][4 * a4 + 3] * inv};
        if (col < hd) *(f32x4*)(orow + col) = val;
      }
    }
  }
  if (qi < N && g == 0) a.lse[(size_t)bh * N + qi] = (m_run + log2f(lt)) * kLn2;
}

template <int D, int DV, int BC, int NW, int OCC, bool DROP = false, bool OPT = false>
static int launch_fwd(const FwdArgs& a, bool causal, hipStream_t stream) {
  constexpr int BR = 32 * NW;
  const int nqt = (a.N + BR - 1) / BR;
  const long long blocks = (long long)a.B * a.H * nqt;
  if (blocks <= 0 || blocks > 0x7fffffff) return -1;
  if ((a.drop_t != 0) != DROP) return -1;
  if (causal) {
    hipLaunchKernelGGL((fwd_kernel<D, DV, BC, NW, OCC, true, DROP, OPT>), dim3((unsigned)blocks), dim3(NW * 64), 0, stream,
                       a);
  } else {
    hipLaunchKernelGGL((fwd_kernel<D, DV, BC, NW, OCC, false, DROP, OPT>), dim3((unsigned)blocks), dim3(NW * 64), 0, stream,
                       a);
  }
  return 0;
}

#define FWD_CFG(D, BC, NW, OCC) \
  { D, 32 * (NW), BC, NW, "fwd d" #D " Br32x" #NW " Bc" #BC " occ" #OCC, &launch_fwd<D, D, BC, NW, OCC> }
// head dim DV on D-wide tiles (the table's key is DV)
#define FWD_CFGV(D, DV, BC, NW, OCC)                                                                    \
  {                                                                                                       \
    DV, 32 * (NW), BC, NW, "fwd d" #DV " (tiles " #D ") Br32x" #NW " Bc" #BC " occ" #OCC,               \
        &launch_fwd<D, DV, BC, NW, OCC>                                                                   \
  }
// optimistic statistics (OPT): the tile's row maximum is taken only when P leaves its bound
#define FWD_CFGO(D, BC, NW, OCC) \
  { D, 32 * (NW), BC, NW, "fwd d" #D " Br32x" #NW " Bc" #BC " occ" #OCC " opt", &launch_fwd<D, D, BC, NW, OCC, false, true> }
#define FWD_CFGVO(D, DV, BC, NW, OCC)                                                                   \
  {                                                                                                       \
    DV, 32 * (NW), BC, NW, "fwd d" #DV " (tiles " #D ") Br32x" #NW " Bc" #BC " occ" #OCC " opt",        \
        &launch_fwd<D, DV, BC, NW, OCC, false, true>                                                      \
  }
#define FWD_DROP_CFG(D, DV, BC, NW, OCC)                                                                \
  {                                                                                                       \
    DV, 32 * (NW), BC, NW, "fwd+dropout d" #DV " Br32x" #NW " Bc" #BC " occ" #OCC,                     \
        &launch_fwd<D, DV, BC, NW, OCC, true>                                                             \
  }

// Host-side table (function-local so that only the host pass materialises it).
const FwdConfig* fwd_configs(int* count) {
  static const FwdConfig table[] = {
      FWD_CFG(64, 64, 4, 2),   FWD_CFG(64, 128, 4, 2),  FWD_CFG(64, 64, 8, 2),  FWD_CFG(64, 128, 8, 2),
      FWD_CFG(128, 64, 4, 2),  FWD_CFG(128, 32, 4, 2),  FWD_CFG(128, 64, 8, 2), FWD_CFG(128, 128, 4, 1),
      FWD_CFG(256, 32, 4, 1),  FWD_CFG(256, 64, 4, 1),
      FWD_CFGV(128, 96, 64, 4, 2), FWD_CFGV(128, 96, 64, 8, 2), FWD_CFGV(256, 192, 32, 4, 1),
      FWD_CFGV(256, 192, 64, 4, 1),
      FWD_CFG(128, 32, 4, 3),  FWD_CFG(64, 64, 4, 3),  FWD_CFG(64, 32, 4, 4), FWD_CFGV(128, 96, 32, 4, 3),
      FWD_CFGO(128, 32, 4, 3), FWD_CFGO(64, 64, 4, 3), FWD_CFGO(64, 64, 8, 2), FWD_CFGO(256, 32, 4, 1),
      FWD_CFGVO(128, 96, 32, 4, 3), FWD_CFGVO(128, 96, 64, 8, 2), FWD_CFGVO(256, 192, 64, 4, 1),
      FWD_CFGVO(256, 192, 32, 4, 1), FWD_CFGO(128, 64, 4, 2),
      // non-power-of-two workgroups (160, 192, 224 query rows) and the ceil(M / 4d) seed of the
      // block-size rule (M = 160 KB of LDS: 160 keys per tile at d = 128, 320 at d = 64)
      FWD_CFGO(128, 32, 5, 2), FWD_CFGO(128, 32, 6, 2), FWD_CFGO(128, 32, 7, 2), FWD_CFGO(128, 160, 4, 1),
      FWD_CFG(64, 320, 2, 1),
      // head dims above 256 on 384-wide tiles
      FWD_CFGVO(384, 288, 32, 4, 1), FWD_CFGVO(384, 320, 32, 4, 1), FWD_CFGVO(384, 352, 32, 4, 1),
      FWD_CFGVO(384, 384, 32, 4, 1),
      // eight waves over 256 query rows: each K/V tile copied once for twice the rows
      FWD_CFGO(128, 64, 8, 2),
  };
  *count = (int)(sizeof(table) / sizeof(table[0]));
  return table;
}

const FwdConfig* fwd_dropout_configs(int* count) {
  static const FwdConfig table[] = {
      FWD_DROP_CFG(64, 64, 64, 8, 2),   FWD_DROP_CFG(128, 128, 64, 8, 2), FWD_DROP_CFG(256, 256, 32, 4, 1),
      FWD_DROP_CFG(128, 96, 64, 4, 2),  FWD_DROP_CFG(256, 192, 32, 4, 1),
  };
  *count = (int)(sizeof(table) / sizeof(table[0]));
  return table;
}

}  // namespace fa
