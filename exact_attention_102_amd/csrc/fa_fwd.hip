// fa_fwd.hip -- fused attention forward for gfx950.
//
// One workgroup owns BR = 32 * QB * NW query rows of one (batch, head); each of
// its NW waves owns 32 * QB of them.  The workgroup walks the key/value tiles
// (BC keys each) through double-buffered LDS ("ELI5: FlashAttention": tiling and
// kernel fusion -- S and P live only in registers), and keeps, per query row,
// the running maximum m and running exp-sum l of the online softmax (same page,
// the m(x)/l(x) statistics).  Per tile:
//   S^T = K Q^T          MFMA, A = K row fragments from LDS, B = Q^T in registers
//   mask, row max        in-lane over 16 keys per 32-key block + one half swap
//   P^T = exp2(S^T * c - m)   c = scale * log2(e) folded into one FMA
//   O^T += V^T P^T       MFMA, A = V^T via transposed LDS reads, B = P^T from
//                        the S^T accumulators (bf16, round-to-nearest-even)
// The transposed orientation (keys down the MFMA rows, one query per lane
// column) keeps every row statistic in-lane.  The epilogue writes O = O^T / l in
// fp32 and lse = ln(2) * (m + log2 l).
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

template <int D, int BC, int NW, int QB, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) void fwd_kernel(FwdArgs a) {
  constexpr int BR = 32 * QB * NW;
  constexpr int NT = NW * 64;
  constexpr int TILE = BC * D * 2;  // bytes of one K or V tile
  constexpr int KB = BC / 32;       // 32-key blocks per tile
  constexpr int DB = D / 32;        // 32-wide blocks of the head dim
  constexpr int KK = D / 16;        // k-steps of Q K^T
  __shared__ __attribute__((aligned(1024))) char smem_raw[4 * TILE];
  LDS char* smem = (LDS char*)smem_raw;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int N = a.N;
  const int nqt = (N + BR - 1) / BR;
  const int item = xcd_remap(blockIdx.x, a.B * a.H * nqt);
  const int bh = item / nqt;
  const int qt = CAUSAL ? nqt - 1 - item % nqt : item % nqt;  // causal: heavy tiles first
  const size_t head = (size_t)bh * N * D;
  const __bf16* Qh = a.q + head;
  const __bf16* Kh = a.k + head;
  const __bf16* Vh = a.v + head;
  const float c = a.scale * kLog2e;

  const int q_wg = qt * BR;
  const int q_w = q_wg + wave * 32 * QB;

  bf16x8 qf[QB][KK];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qi = q_w + qb * 32 + l32;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      if (qi < N) {
        qf[qb][kk] = *(const bf16x8*)(Qh + (size_t)qi * D + kk * 16 + g * 8);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[qb][kk][e] = (__bf16)0.f;
      }
    }
  }

  float m_run[QB], l_run[QB];
  f32x16 o[QB][DB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[qb][db] = zero16();
  }

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
    const bool active = !CAUSAL || k0 <= q_w + 32 * QB - 1;
    if (active) {
      f32x16 s[QB][KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb][kb] = zero16();
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const bf16x8 ka = row_frag<D>(kt, kb * 32 + krow, kk * 16 + g * 8);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) s[qb][kb] = mfma32(ka, qf[qb][kk], s[qb][kb]);
        }
      }
      const bool need_mask = (k0 + BC > N) || (CAUSAL && k0 + BC - 1 > q_w);
      if (need_mask) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const int qi = q_w + qb * 32 + l32;
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = k0 + kb * 32 + 16 * (r >> 3) + 8 * g + (r & 7);
              if (key >= N || (CAUSAL && key > qi)) s[qb][kb][r] = -INFINITY;
            }
          }
        }
      }
      bf16x8 pb[QB][2 * KB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[qb][kb][r]);
        }
        mx = half_swap_max(mx);
        const float m_new = fmaxf(m_run[qb], mx * c);
        const float alpha = exp2_hw(m_run[qb] - m_new);
        m_run[qb] = m_new;
        const float nm = -m_new;
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = exp2_hw(fmaf(s[qb][kb][r], c, nm));
            s[qb][kb][r] = p;
            rs += p;
          }
          pb[qb][2 * kb] = pack8(s[qb][kb], 0);
          pb[qb][2 * kb + 1] = pack8(s[qb][kb], 8);
        }
        l_run[qb] = l_run[qb] * alpha + rs;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
          for (int r = 0; r < 16; ++r) o[qb][db][r] *= alpha;
        }
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int ks = 0; ks < 2 * KB; ++ks) {
          const bf16x8 va = col_frag<D>(vt, ks * 16, db * 32, lane);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) o[qb][db] = mfma32(va, pb[qb][ks], o[qb][db]);
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

  float* Oh = a.o + head;
  float* Lh = a.lse + (size_t)bh * N;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = half_swap_sum(l_run[qb]);
    const float inv = 1.f / lt;
    const int qi = q_w + qb * 32 + l32;
    if (qi < N) {
      float* orow = Oh + (size_t)qi * D;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const f32x4 val = {o[qb][db][4 * a4] * inv, o[qb][db][4 * a4 + 1] * inv, o[qb][db][4 * a4 + 2] * inv,
                             o[qb][db][4 * a4 + 3] * inv};
          *(f32x4*)(orow + db * 32 + 8 * a4 + 4 * g) = val;
        }
      }
      if (g == 0) Lh[qi] = (m_run[qb] + log2f(lt)) * kLn2;
    }
  }
}

template <int D, int BC, int NW, int QB>
static int launch_fwd(const FwdArgs& a, bool causal, hipStream_t stream) {
  constexpr int BR = 32 * QB * NW;
  const int nqt = (a.N + BR - 1) / BR;
  const long long blocks = (long long)a.B * a.H * nqt;
  if (blocks <= 0 || blocks > 0x7fffffff) return -1;
  if (causal) {
    hipLaunchKernelGGL((fwd_kernel<D, BC, NW, QB, true>), dim3((unsigned)blocks), dim3(NW * 64), 0, stream, a);
  } else {
    hipLaunchKernelGGL((fwd_kernel<D, BC, NW, QB, false>), dim3((unsigned)blocks), dim3(NW * 64), 0, stream, a);
  }
  return 0;
}

#define FWD_CFG(D, BC, NW, QB) \
  { D, 32 * (QB) * (NW), BC, NW, "fwd d" #D " Br" #QB "x32x" #NW " Bc" #BC, &launch_fwd<D, BC, NW, QB> }

// Host-side table (function-local so that only the host pass materialises it).
const FwdConfig* fwd_configs(int* count) {
  static const FwdConfig table[] = {
      FWD_CFG(64, 64, 4, 1),  FWD_CFG(64, 128, 4, 1), FWD_CFG(64, 64, 4, 2),
      FWD_CFG(128, 64, 4, 1), FWD_CFG(128, 32, 4, 2), FWD_CFG(128, 128, 4, 1),
      FWD_CFG(256, 32, 4, 1),
  };
  *count = (int)(sizeof(table) / sizeof(table[0]));
  return table;
}

}  // namespace fa
