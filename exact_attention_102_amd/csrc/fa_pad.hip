// fa_pad.hip -- layout adapters of the general entry points (fa_fwd_general,
// fa_bwd_general): any head dimension 1..256 and any row/head/batch strides.
//
// The fused kernels are built for head dims 64, 96, 128, 192 and 256 and read
// strided views in place when rows are 16-byte aligned and d is a multiple of 8.
// Any other general call gathers each strided [B, H, N, d] view into a contiguous
// [B, H, N, Dp] workspace buffer, Dp the next built head dim, with the columns
// d .. Dp-1 set to zero, runs the fused kernels at Dp, and scatters the first d
// columns of the results back into the caller's views.  Zero columns leave
// every score q.k unchanged (so P, the softmax statistics and lse are exact), add
// zero columns to O and dV, and add nothing to dQ and dK in the first d columns.
// Both adapters are memory-bound and linear in N, against the fused kernels'
// quadratic work.  Each thread moves one 16-byte chunk of a padded row (8 bf16 or
// 4 fp32 values): one vector access where the chunk is whole and 16-byte aligned in
// the view, element accesses otherwise (ragged d, odd strides).
#include <cstdint>

#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kPadThreads = 256;
constexpr long long kPadMaxBlocks = 16384;

typedef unsigned u32x4v __attribute__((ext_vector_type(4)));

// element offset in a view of flat row `row` of a [B, H, N] grid
__device__ __forceinline__ long long view_row(int row, int H, int N, const View& s) {
  const int n = row % N;
  const int bh = row / N;
  return (long long)(bh / H) * s.sb + (long long)(bh % H) * s.sh + (long long)n * s.sn;
}

// T: element type; E: elements per 16-byte chunk; cpr: chunks per padded row (dp / E)
template <typename T, int E>
__global__ void gather_kernel(const T* __restrict__ src, View s, T* __restrict__ dst, int H, int N, int d, int cpr,
                              long long total_chunks) {
  const long long step = (long long)gridDim.x * blockDim.x;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < total_chunks; i += step) {
    const int row = (int)(i / cpr);
    const int c0 = (int)(i - (long long)row * cpr) * E;
    const T* sp = src + view_row(row, H, N, s) + c0;
    u32x4v v;
    if (c0 + E <= d && (reinterpret_cast<uintptr_t>(sp) & 15u) == 0) {
      v = *reinterpret_cast<const u32x4v*>(sp);
    } else {
      T tmp[E];
#pragma unroll
      for (int e = 0; e < E; ++e) tmp[e] = (c0 + e < d) ? sp[e] : T(0);
      __builtin_memcpy(&v, tmp, 16);
    }
    *reinterpret_cast<u32x4v*>(dst + i * E) = v;
  }
}

template <typename T, int E>
__global__ void scatter_kernel(const T* __restrict__ src, T* __restrict__ dst, View s, int H, int N, int d, int cpr,
                               long long total_chunks) {
  const long long step = (long long)gridDim.x * blockDim.x;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < total_chunks; i += step) {
    const int row = (int)(i / cpr);
    const int c0 = (int)(i - (long long)row * cpr) * E;
    if (c0 >= d) continue;
    T* dp = dst + view_row(row, H, N, s) + c0;
    const u32x4v v = *reinterpret_cast<const u32x4v*>(src + i * E);
    if (c0 + E <= d && (reinterpret_cast<uintptr_t>(dp) & 15u) == 0) {
      *reinterpret_cast<u32x4v*>(dp) = v;
    } else {
      T tmp[E];
      __builtin_memcpy(tmp, &v, 16);
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (c0 + e < d) dp[e] = tmp[e];
    }
  }
}

unsigned pad_blocks(long long total) {
  const long long b = (total + kPadThreads - 1) / kPadThreads;
  return (unsigned)(b < 1 ? 1 : (b > kPadMaxBlocks ? kPadMaxBlocks : b));
}

}  // namespace

// dp (the padded row, 64, 96, 128, 192 or 256 elements) is a whole number of chunks.
void launch_gather_bf16(const void* src, View s, void* dst, int B, int H, int N, int d, int dp, hipStream_t st) {
  const int cpr = dp / 8;
  const long long total = (long long)B * H * N * cpr;
  hipLaunchKernelGGL((gather_kernel<unsigned short, 8>), dim3(pad_blocks(total)), dim3(kPadThreads), 0, st,
                     static_cast<const unsigned short*>(src), s, static_cast<unsigned short*>(dst), H, N, d, cpr, total);
}

void launch_gather_f32(const float* src, View s, float* dst, int B, int H, int N, int d, int dp, hipStream_t st) {
  const int cpr = dp / 4;
  const long long total = (long long)B * H * N * cpr;
  hipLaunchKernelGGL((gather_kernel<float, 4>), dim3(pad_blocks(total)), dim3(kPadThreads), 0, st, src, s, dst, H, N,
                     d, cpr, total);
}

void launch_scatter_f32(const float* src, float* dst, View s, int B, int H, int N, int d, int dp, hipStream_t st) {
  const int cpr = dp / 4;
  const long long total = (long long)B * H * N * cpr;
  hipLaunchKernelGGL((scatter_kernel<float, 4>), dim3(pad_blocks(total)), dim3(kPadThreads), 0, st, src, dst, s, H,
                     N, d, cpr, total);
}

}  // namespace fa
