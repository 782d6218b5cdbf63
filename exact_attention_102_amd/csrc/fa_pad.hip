// fa_pad.hip -- layout adapters of the general entry points (fa_fwd_general,
// fa_bwd_general): any head dimension 1..256 and any row/head/batch strides.
//
// The fused kernels are built for head dims 64, 128 and 256 on contiguous
// [B, H, N, d] tensors.  A general call gathers each strided [B, H, N, d] view into
// a contiguous [B, H, N, Dp] workspace buffer, Dp the next built head dim, with the
// columns d .. Dp-1 set to zero, runs the fused kernels at Dp, and scatters the
// first d columns of the results back into the caller's views.  Zero columns leave
// every score q.k unchanged (so P, the softmax statistics and lse are exact), add
// zero columns to O and dV, and add nothing to dQ and dK in the first d columns.
// Both adapters are memory-bound and linear in N, against the fused kernels'
// quadratic work.
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kPadThreads = 256;
constexpr long long kPadMaxBlocks = 8192;

// (b, h, n) of flat row index `row` of a [B, H, N] grid, as an element offset in a view
__device__ __forceinline__ long long view_row(long long row, int H, int N, const View& s) {
  const long long n = row % N;
  const long long bh = row / N;
  return (bh / H) * s.sb + (bh % H) * s.sh + n * s.sn;
}

template <typename T>
__global__ void gather_kernel(const T* __restrict__ src, View s, T* __restrict__ dst, int H, int N, int d, int dp,
                              long long total) {
  const long long step = (long long)gridDim.x * blockDim.x;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += step) {
    const int c = (int)(i % dp);
    const long long row = i / dp;
    T v = T(0);
    if (c < d) v = src[view_row(row, H, N, s) + c];
    dst[i] = v;
  }
}

template <typename T>
__global__ void scatter_kernel(const T* __restrict__ src, T* __restrict__ dst, View s, int H, int N, int d, int dp,
                               long long total) {
  const long long step = (long long)gridDim.x * blockDim.x;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += step) {
    const int c = (int)(i % d);
    const long long row = i / d;
    dst[view_row(row, H, N, s) + c] = src[row * dp + c];
  }
}

unsigned pad_blocks(long long total) {
  const long long b = (total + kPadThreads - 1) / kPadThreads;
  return (unsigned)(b < 1 ? 1 : (b > kPadMaxBlocks ? kPadMaxBlocks : b));
}

}  // namespace

void launch_gather_bf16(const void* src, View s, void* dst, int B, int H, int N, int d, int dp, hipStream_t st) {
  const long long total = (long long)B * H * N * dp;
  hipLaunchKernelGGL(gather_kernel<unsigned short>, dim3(pad_blocks(total)), dim3(kPadThreads), 0, st,
                     static_cast<const unsigned short*>(src), s, static_cast<unsigned short*>(dst), H, N, d, dp,
                     total);
}

void launch_gather_f32(const float* src, View s, float* dst, int B, int H, int N, int d, int dp, hipStream_t st) {
  const long long total = (long long)B * H * N * dp;
  hipLaunchKernelGGL(gather_kernel<float>, dim3(pad_blocks(total)), dim3(kPadThreads), 0, st, src, s, dst, H, N, d,
                     dp, total);
}

void launch_scatter_f32(const float* src, float* dst, View s, int B, int H, int N, int d, int dp, hipStream_t st) {
  const long long total = (long long)B * H * N * d;
  hipLaunchKernelGGL(scatter_kernel<float>, dim3(pad_blocks(total)), dim3(kPadThreads), 0, st, src, dst, s, H, N, d,
                     dp, total);
}

}  // namespace fa
