// probe_atomic_dq.hip -- measures the ceiling that the 5-GEMM backward's dQ
// accumulation runs into: the atomic pattern of the dK/dV kernel with fused dQ
// ("Potential algorithmic improvements for backward pass", flash-attention issue
// 1172: the 5-GEMM design adds dQ with atomics), with none of its math.
//
// One workgroup per (head, key tile of BK = 32 * NW keys), as in the kernel; for
// each query tile of BQ rows its waves split the (32-query block, 32-column block)
// pairs and each lane adds 16 fp32 values with global atomics (rows
// q0 + 32 qb + 8 (r / 4) + 4 g + r % 4, column 32 db + l % 32: the MFMA C layout the
// kernel adds from).  Every dQ element receives N / BK adds.  A second variant
// writes the same values with plain stores into per-key-tile partial buffers
// ([N / BK] x [B, H, N, d], the payload of a two-stage reduction), for comparison.
// The result of the atomic run is checked (every element must equal N / BK).
//
//   probe_atomic_dq [B H N d]      (default 4 16 2048 128; d in {64, 128, 256})
// prints one JSON line per variant.  Built by exact_attention_102_amd/build.py.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <vector>

#define CHECK(x)                                                                   \
  do {                                                                             \
    hipError_t e_ = (x);                                                           \
    if (e_ != hipSuccess) {                                                        \
      std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      std::exit(1);                                                                \
    }                                                                              \
  } while (0)

template <int D, int BQ, int NW, bool ATOMIC>
__global__ __launch_bounds__(NW * 64) void dq_pattern(float* dq, int N, int nkt) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 5, l32 = lane & 31;
  const int bh = blockIdx.x / nkt, kt = blockIdx.x % nkt;
  const size_t head = (size_t)bh * N * D;
  // atomic: all key tiles add into dq; plain: key tile kt writes its own partial copy
  float* dst = ATOMIC ? dq + head : dq + (size_t)kt * gridDim.x / nkt * N * D + head;
  constexpr int QBN = BQ / 32, DB = D / 32;
  const int nqt = N / BQ;
  for (int it = 0; it < nqt; ++it) {
    const int q0 = it * BQ;
    for (int t = wave; t < QBN * DB; t += NW) {
      const int qb = t / DB, db = t % DB;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int q = q0 + qb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
        float* p = dst + (size_t)q * D + db * 32 + l32;
        if (ATOMIC) {
          unsafeAtomicAdd(p, 1.0f);
        } else {
          *p = 1.0f;
        }
      }
    }
  }
}

template <int D, int BQ, int NW>
void run(int B, int H, int N) {
  const int BK = 32 * NW;
  const int nkt = N / BK;
  const size_t elems = (size_t)B * H * N * D;
  float* dq = nullptr;
  float* part = nullptr;
  CHECK(hipMalloc(&dq, elems * 4));
  CHECK(hipMalloc(&part, elems * 4 * nkt));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  const dim3 grid(B * H * nkt), block(NW * 64);
  for (int variant = 0; variant < 2; ++variant) {
    float best = 1e30f;
    for (int rep = 0; rep < 6; ++rep) {
      if (variant == 0) CHECK(hipMemset(dq, 0, elems * 4));
      CHECK(hipEventRecord(e0));
      if (variant == 0) {
        hipLaunchKernelGGL((dq_pattern<D, BQ, NW, true>), grid, block, 0, 0, dq, N, nkt);
      } else {
        hipLaunchKernelGGL((dq_pattern<D, BQ, NW, false>), grid, block, 0, 0, part, N, nkt);
      }
      CHECK(hipGetLastError());
      CHECK(hipEventRecord(e1));
      CHECK(hipEventSynchronize(e1));
      float ms = 0.f;
      CHECK(hipEventElapsedTime(&ms, e0, e1));
      if (rep > 0 && ms < best) best = ms;  // the first run warms up
    }
    size_t wrong = 0;
    if (variant == 0) {
      std::vector<float> h(elems);
      CHECK(hipMemcpy(h.data(), dq, elems * 4, hipMemcpyDeviceToHost));
      for (size_t i = 0; i < elems; ++i) wrong += (h[i] != (float)nkt);
    }
    const double ops = (double)elems * nkt;
    std::printf("{\"probe\": \"%s\", \"B\": %d, \"H\": %d, \"N\": %d, \"d\": %d, \"BK\": %d, \"BQ\": %d, "
                "\"values_per_element\": %d, \"ms\": %.4f, \"G_per_s\": %.1f, \"payload_TB_per_s\": %.3f, "
                "\"wrong\": %zu}\n",
                variant == 0 ? "fp32 atomic add" : "plain fp32 store to partials", B, H, N, D, BK, BQ, nkt, best,
                ops / best / 1e6, ops * 4 / best / 1e9, wrong);
    std::fflush(stdout);
  }
  CHECK(hipFree(dq));
  CHECK(hipFree(part));
}

int main(int argc, char** argv) {
  int B = 4, H = 16, N = 2048, d = 128;
  if (argc == 5) {
    B = std::atoi(argv[1]);
    H = std::atoi(argv[2]);
    N = std::atoi(argv[3]);
    d = std::atoi(argv[4]);
  }
  // tile shapes of the default atomic configurations: d64 Bk256 Bq64, d128 Bk128 Bq64, d256 Bk64 Bq32
  const int bk = d == 64 ? 256 : (d == 128 ? 128 : 64), bq = d == 256 ? 32 : 64;
  if (B <= 0 || H <= 0 || N <= 0 || (d != 64 && d != 128 && d != 256) || N % bk != 0 || N % bq != 0) {
    std::printf("usage: probe_atomic_dq B H N d  (d in {64,128,256}, N a multiple of %d)\n", bk);
    return 2;
  }
  if (d == 64) run<64, 64, 8>(B, H, N);
  if (d == 128) run<128, 64, 4>(B, H, N);
  if (d == 256) run<256, 32, 2>(B, H, N);
  return 0;
}
