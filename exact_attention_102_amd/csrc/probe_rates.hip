// probe_rates.hip -- issue rates of the units the fused kernels lean on, for the
// roofline's secondary ceilings: the matmul-to-exp ratio that "Potential
// algorithmic improvements for backward pass" (flash-attention issue 1172)
// singles out, and the LDS fragment reads that feed every MFMA.
//
//   mfma     v_mfma_f32_32x32x16_bf16 on register operands, four independent
//            accumulator chains per wave, two waves per SIMD      -> TFLOP/s
//   exp      v_exp_f32, eight independent chains per lane (the negation rides on
//            the instruction's source modifier, so each step is one exp)
//                                                                  -> T lane-ops/s
//   fma      v_fma_f32, eight independent chains per lane          -> T lane-ops/s
//   lds_row  ds_read_b128 row fragments through the kernels' row-only swizzle
//   lds_tr   ds_read_b64_tr_b16 transposed fragments through the column swizzle
//                                                                  -> TB/s, B/clk/CU
// Every workgroup writes only its own output words; LDS reads stay inside the
// workgroup's 64 KB array.  Best of 5 timed launches after one warm-up (HIP
// events).  Prints one JSON line per rate.  Built by exact_attention_102_amd/build.py.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

#include "fa_device.h"

using namespace fa;

#define CHECK(x)                                                                   \
  do {                                                                             \
    hipError_t e_ = (x);                                                           \
    if (e_ != hipSuccess) {                                                        \
      std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      std::exit(1);                                                                \
    }                                                                              \
  } while (0)

constexpr int kThreads = 256;  // 4 waves per workgroup

__global__ __launch_bounds__(kThreads, 2) void mfma_rate(float* out, int iters) {
  const int tid = threadIdx.x;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (float)((tid + e) & 7));
    b[e] = (__bf16)(0.001f * (float)((tid * 3 + e) & 7));
  }
  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = zero16();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = mfma32(a, b, acc[i]);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[i][r];
  out[blockIdx.x * kThreads + tid] = s;
}

__global__ __launch_bounds__(kThreads) void exp_rate(float* out, int iters) {
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = 0.25f + 0.01f * (float)((threadIdx.x + i) & 15);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = __builtin_amdgcn_exp2f(-x[i]);  // stays in (0.5, 1]
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += x[i];
  out[blockIdx.x * kThreads + threadIdx.x] = s;
}

__global__ __launch_bounds__(kThreads) void fma_rate(float* out, int iters) {
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = 0.5f + 0.01f * (float)((threadIdx.x + i) & 15);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = fmaf(x[i], 0.999f, 0.001f);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += x[i];
  out[blockIdx.x * kThreads + threadIdx.x] = s;
}

// MODE 0: row fragments (kRowOnly swizzle); MODE 1: transposed fragments (kColOnly).
// Each wave reads its own 16 KB 64 x 128 tile of the 64 KB array.
template <int MODE>
__global__ __launch_bounds__(kThreads, 2) void lds_rate(unsigned* out, int iters) {
  __shared__ __attribute__((aligned(1024))) char lds[65536];
  for (int i = threadIdx.x; i < 65536 / 16; i += kThreads) ((LDS u32x4*)lds)[i] = u32x4{(unsigned)i, 1u, 2u, 3u};
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const LDS char* tile = (const LDS char*)lds + wave * 16384;
  RowOffsets<128, kRowOnly> fr;
  fr.init(lane);
  ColOffsets<128, kColOnly> fc;
  fc.init(lane);
  unsigned acc = 0;
  for (int it = 0; it < iters; ++it) {
    fr.refresh();
    fc.refresh();
    if constexpr (MODE == 0) {
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {  // rows 0..63 of the tile, all 16 chunks
        const u32x4 v = __builtin_bit_cast(u32x4, fr.row(tile, 32 * (it & 1), kk));
        acc ^= v[0] ^ v[3];
      }
    } else {
#pragma unroll
      for (int db = 0; db < 4; ++db) {  // rows r0 .. r0 + 15 (r0 <= 48), all 128 columns
        const u32x4 v = __builtin_bit_cast(u32x4, fc.col(tile, 16 * (it & 3), db));
        acc ^= v[0] ^ v[3];
      }
    }
  }
  out[blockIdx.x * kThreads + threadIdx.x] = acc;
}

template <typename F>
float best_ms(F launch) {
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  launch();
  CHECK(hipGetLastError());
  CHECK(hipDeviceSynchronize());
  float best = 1e30f;
  for (int rep = 0; rep < 5; ++rep) {
    CHECK(hipEventRecord(e0));
    launch();
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    if (ms < best) best = ms;
  }
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  return best;
}

int main() {
  hipDeviceProp_t prop;
  CHECK(hipGetDeviceProperties(&prop, 0));
  const int cus = prop.multiProcessorCount;
  const double clk_ghz = 2.4;  // MI355X peak engine clock, for bytes per clock
  const int blocks = cus * 2;   // two 4-wave workgroups per CU: two waves per SIMD
  float* fout = nullptr;
  unsigned* uout = nullptr;
  CHECK(hipMalloc(&fout, (size_t)blocks * 4 * kThreads * sizeof(float)));
  CHECK(hipMalloc(&uout, (size_t)blocks * 4 * kThreads * sizeof(unsigned)));
  const int waves = blocks * (kThreads / 64);

  const int mi = 4000;
  const float t_mfma = best_ms([&] { hipLaunchKernelGGL(mfma_rate, dim3(blocks), dim3(kThreads), 0, 0, fout, mi); });
  const double mfma_tf = (double)waves * mi * 4 * 32768.0 / (t_mfma * 1e-3) / 1e12;
  std::printf("{\"rate\": \"mfma_32x32x16_bf16_registers\", \"cus\": %d, \"ms\": %.4f, \"TFLOP_per_s\": %.1f}\n", cus,
              t_mfma, mfma_tf);

  const int xi = 20000, vb = blocks * 4;  // eight waves per SIMD for the VALU rates
  const float t_exp = best_ms([&] { hipLaunchKernelGGL(exp_rate, dim3(vb), dim3(kThreads), 0, 0, fout, xi); });
  const double exp_t = (double)vb * kThreads * xi * 8 / (t_exp * 1e-3) / 1e12;
  std::printf("{\"rate\": \"v_exp_f32\", \"ms\": %.4f, \"T_lane_ops_per_s\": %.2f, \"lanes_per_clk_per_cu\": %.1f}\n",
              t_exp, exp_t, exp_t * 1e12 / (cus * clk_ghz * 1e9));
  const float t_fma = best_ms([&] { hipLaunchKernelGGL(fma_rate, dim3(vb), dim3(kThreads), 0, 0, fout, xi); });
  const double fma_t = (double)vb * kThreads * xi * 8 / (t_fma * 1e-3) / 1e12;
  std::printf("{\"rate\": \"v_fma_f32\", \"ms\": %.4f, \"T_lane_ops_per_s\": %.2f, \"lanes_per_clk_per_cu\": %.1f}\n",
              t_fma, fma_t, fma_t * 1e12 / (cus * clk_ghz * 1e9));
  std::printf("{\"rate\": \"matmul_to_exp\", \"mfma_flop_per_exp\": %.0f}\n", mfma_tf / exp_t);

  const int li = 4000;
  const float t_row = best_ms([&] { hipLaunchKernelGGL(lds_rate<0>, dim3(blocks), dim3(kThreads), 0, 0, uout, li); });
  const double row_b = (double)waves * li * 8 * 1024;
  std::printf("{\"rate\": \"lds_ds_read_b128_row_fragments\", \"ms\": %.4f, \"TB_per_s\": %.2f, \"B_per_clk_per_cu\": "
              "%.0f}\n", t_row, row_b / (t_row * 1e-3) / 1e12, row_b / (t_row * 1e-3) / (cus * clk_ghz * 1e9));
  const float t_tr = best_ms([&] { hipLaunchKernelGGL(lds_rate<1>, dim3(blocks), dim3(kThreads), 0, 0, uout, li); });
  const double tr_b = (double)waves * li * 4 * 1024;
  std::printf("{\"rate\": \"lds_ds_read_b64_tr_b16_transposed\", \"ms\": %.4f, \"TB_per_s\": %.2f, "
              "\"B_per_clk_per_cu\": %.0f}\n", t_tr, tr_b / (t_tr * 1e-3) / 1e12,
              tr_b / (t_tr * 1e-3) / (cus * clk_ghz * 1e9));
  CHECK(hipFree(fout));
  CHECK(hipFree(uout));
  return 0;
}
