// probe_atomic_dq.hip -- measures the ceiling that the 5-GEMM backward's dQ
// accumulation runs into: the atomic pattern of the dK/dV kernel with fused dQ
// ("Potential algorithmic improvements for backward pass", flash-attention issue
// 1172: the 5-GEMM design adds dQ with atomics), with none of its math.
//
// The pattern is that of the default d <= 128 atomic kernel (two 32-key blocks per
// wave): one workgroup of 4 waves per (head, key tile of BK = 256 keys); for each
// query tile of BQ = 32 rows the 4 waves split the (32-query block, 32-column block)
// pairs (d / 32 of them) and each lane adds 16 fp32 values (rows
// q0 + 8 (r / 4) + 4 g + r % 4, column 32 db + l % 32: the MFMA C layout the kernel
// adds from).  Every dQ element receives N / BK adds of 1.0; the result is checked.
//
// Variants (one JSON line each):
//   buffer aux=A   buffer atomics over the head's accumulator (the kernel's form) with
//                  cache-policy bits A (gfx950: 1 = sc0, 2 = nt, 16 = sc1)
//   global scope=S global atomics at memory scope S (workgroup, agent)
//   plain stores   the same values written into per-key-tile partial buffers
//   rows of 64     buffer atomics, each instruction one row of 64 consecutive columns
//                  (the kernel's instructions cover two rows of 32)
// and two work mappings: "xcd" keeps every key tile of a head on one XCD (the
// kernel's mapping; workgroup x runs on XCD x % 8), "spread" puts a head's key
// tiles on different XCDs.  A variant whose adds were performed in a per-XCD L2
// would lose updates under "spread" (wrong > 0) and run faster under "xcd".
//
//   probe_atomic_dq [B H N d]      (default 4 16 2048 128; d in {64, 128, 256})
// Built by exact_attention_102_amd/build.py.
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

constexpr int NW = 4, BK = 256, BQ = 32;

// Workgroups are dispatched round-robin over the 8 XCDs; this gives XCD x a
// contiguous range of work items (whole heads when the count divides evenly).
__device__ int xcd_item(int x, int total) {
  const int q = total >> 3, r = total & 7;
  const int xcd = x & 7, local = x >> 3;
  return (xcd < r) ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}

// KIND: 0 buffer atomic (cache policy AUX), 1 global atomic workgroup scope,
// 2 global atomic agent scope, 3 plain stores into per-key-tile partials, 4 buffer
// atomics with each instruction covering one row of 64 consecutive columns.
template <int D, int KIND, int AUX>
__global__ __launch_bounds__(NW * 64) void dq_pattern(float* dq, int N, int nkt, int spread) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 5, l32 = lane & 31;
  const int total = gridDim.x;
  const int item = spread ? (int)blockIdx.x : xcd_item(blockIdx.x, total);
  const int bh = item / nkt, kt = item % nkt;
  const size_t head = (size_t)bh * N * D;
  float* dst = KIND == 3 ? dq + (size_t)kt * (total / nkt) * N * D + head : dq + head;
  constexpr int DB = D / 32;
  const int nqt = N / BQ;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(dst, (short)0, (int)((unsigned)N * (unsigned)(D * 4)), 0x00020000);
  for (int it = 0; it < nqt; ++it) {
    const int q0 = it * BQ;
    if constexpr (KIND == 4) {
      // the same adds with one row of 64 consecutive columns per instruction: wave w
      // takes rows w * 8 .. w * 8 + 7 of the query tile, lane l column 64 p + l
#pragma unroll
      for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int pcol = 0; pcol < DB / 2; ++pcol) {
          const unsigned o = ((unsigned)(q0 + wave * 8 + i) * D + pcol * 64 + lane) * 4u;
          __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(1.0f, rs, o, 0, AUX);
        }
      }
      continue;
    }
    for (int db = wave; db < DB; db += NW) {
      const unsigned off = ((unsigned)(q0 + 4 * g) * D + db * 32 + l32) * 4u;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const unsigned o = off + (unsigned)(8 * (r >> 2) + (r & 3)) * (D * 4);
        if constexpr (KIND == 0) {
          __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(1.0f, rs, o, 0, AUX);
        } else if constexpr (KIND == 1) {
          __hip_atomic_fetch_add(dst + o / 4, 1.0f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        } else if constexpr (KIND == 2) {
          __hip_atomic_fetch_add(dst + o / 4, 1.0f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
          dst[o / 4] = 1.0f;
        }
      }
    }
  }
}

template <int D, int KIND, int AUX>
void run(const char* name, int B, int H, int N, int spread, float* dq, float* part, std::vector<float>& h) {
  const int nkt = N / BK;
  const size_t elems = (size_t)B * H * N * D;
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  const dim3 grid(B * H * nkt), block(NW * 64);
  float best = 1e30f;
  float* buf = KIND == 3 ? part : dq;
  for (int rep = 0; rep < 6; ++rep) {
    if (KIND != 3) CHECK(hipMemset(dq, 0, elems * 4));
    CHECK(hipEventRecord(e0));
    hipLaunchKernelGGL((dq_pattern<D, KIND, AUX>), grid, block, 0, 0, buf, N, nkt, spread);
    CHECK(hipGetLastError());
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    if (rep > 0 && ms < best) best = ms;  // the first run warms up
  }
  size_t wrong = 0;
  if (KIND != 3) {
    CHECK(hipMemcpy(h.data(), dq, elems * 4, hipMemcpyDeviceToHost));
    for (size_t i = 0; i < elems; ++i) wrong += (h[i] != (float)nkt);
  }
  const double ops = (double)elems * nkt;
  std::printf("{\"probe\": \"%s\", \"mapping\": \"%s\", \"B\": %d, \"H\": %d, \"N\": %d, \"d\": %d, \"BK\": %d, "
              "\"BQ\": %d, \"values_per_element\": %d, \"ms\": %.4f, \"G_per_s\": %.1f, \"payload_TB_per_s\": %.3f, "
              "\"wrong\": %zu}\n",
              name, spread ? "spread" : "xcd", B, H, N, D, BK, BQ, nkt, best, ops / best / 1e6, ops * 4 / best / 1e9,
              wrong);
  std::fflush(stdout);
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
}

template <int D>
void run_all(int B, int H, int N) {
  const int nkt = N / BK;
  const size_t elems = (size_t)B * H * N * D;
  float* dq = nullptr;
  float* part = nullptr;
  CHECK(hipMalloc(&dq, elems * 4));
  CHECK(hipMalloc(&part, elems * 4 * nkt));
  std::vector<float> h(elems);
  for (int spread = 0; spread < 2; ++spread) {
    run<D, 0, 0>("buffer aux=0", B, H, N, spread, dq, part, h);
    run<D, 0, 2>("buffer aux=2 (nt)", B, H, N, spread, dq, part, h);
    run<D, 0, 16>("buffer aux=16 (sc1)", B, H, N, spread, dq, part, h);
    run<D, 1, 0>("global scope=workgroup", B, H, N, spread, dq, part, h);
    run<D, 2, 0>("global scope=agent", B, H, N, spread, dq, part, h);
    run<D, 4, 0>("buffer rows of 64 columns", B, H, N, spread, dq, part, h);
  }
  run<D, 3, 0>("plain stores to partials", B, H, N, 0, dq, part, h);
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
  if (B <= 0 || H <= 0 || N <= 0 || (d != 64 && d != 128 && d != 256) || N % BK != 0) {
    std::printf("usage: probe_atomic_dq B H N d  (d in {64,128,256}, N a multiple of %d)\n", BK);
    return 2;
  }
  if (d == 64) run_all<64>(B, H, N);
  if (d == 128) run_all<128>(B, H, N);
  if (d == 256) run_all<256>(B, H, N);
  return 0;
}
