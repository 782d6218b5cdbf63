// fa_launch.h -- host/device argument blocks and the per-pass tile-configuration
// tables that the C ABI (fa_api.cpp) dispatches through.
#pragma once
#include <hip/hip_runtime.h>

namespace fa {

// Element strides of a [B, H, N, *] tensor (the head dim is contiguous): element
// (b, h, n, i) is at base[b * sb + h * sh + n * sn + i].
struct View {
  long long sb, sh, sn;
};

// Every tensor is passed as a base pointer plus a View; hd is the tensors' head
// dim.  The kernels are built for D = 64, 96, 128, 192, 256 >= hd: columns hd .. D-1 read as
// zeros (the tile copies and register loads fetch nothing there) and are never
// written, so the result is the attention of the hd columns (zero columns change
// no score).  Row starts are 16-byte aligned and hd is a multiple of 8.
__device__ __forceinline__ size_t head_base(const View& v, int bh, int H) {
  return (size_t)(bh / H) * (size_t)v.sb + (size_t)(bh % H) * (size_t)v.sh;
}

struct FwdArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  float* o;
  float* lse;
  int B, H, N;
  float scale;
  // dropout on P (fa_dropout.h); drop_t == 0 means none
  unsigned drop_k0 = 0, drop_k1 = 0, drop_offset = 0, drop_t = 0;
  float drop_scale = 1.f;
  View vq{}, vk{}, vv{}, vo{};
  int hd = 0;
};

struct BwdArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* dout;
  const float* lse;
  const float* delta;
  float* dq;
  float* dk;
  float* dv;
  int B, H, N;
  float scale;
  unsigned drop_k0 = 0, drop_k1 = 0, drop_offset = 0, drop_t = 0;
  float drop_scale = 1.f;
  View vq{}, vk{}, vv{}, vdo{}, vdq{}, vdk{}, vdv{};  // vdo.sn == vq.sn (one tile copier serves both)
  int hd = 0;
  // dQ kernel only: with o set, it computes delta itself from O and dO (no preprocess
  // launch) and writes it to delta_out for the dK/dV kernel that runs after it
  const float* o = nullptr;
  View vo{};
  float* delta_out = nullptr;
};

struct PreArgs {
  const float* o;
  const __bf16* dout;
  float* delta;
  float* dq;  // zeroed when non-null
  int rows;   // B * H * N
  int H = 0, N = 0, hd = 0;
  View vo{}, vdo{}, vdq{};
};

typedef int (*FwdLaunch)(const FwdArgs&, bool causal, hipStream_t);
typedef int (*BwdLaunch)(const BwdArgs&, bool causal, hipStream_t);

struct FwdConfig {
  int d;
  int rows;   // query rows per workgroup
  int cols;   // keys per LDS tile
  int waves;
  const char* name;
  FwdLaunch launch;
};

struct BwdConfig {
  int d;
  int rows;   // rows owned per workgroup (keys for dK/dV, queries for dQ)
  int cols;   // rows per LDS tile along the traversal
  int waves;
  const char* name;
  BwdLaunch launch;
};

const FwdConfig* fwd_configs(int* count);
const BwdConfig* dkdv_configs(int* count);         // 7-GEMM dK/dV (no dQ)
const BwdConfig* dkdv_atomic_configs(int* count);  // 5-GEMM dK/dV with fp32-atomic dQ
const BwdConfig* dq_configs(int* count);           // 7-GEMM dQ
// The same passes with dropout on P: one configuration per head dim each.
const FwdConfig* fwd_dropout_configs(int* count);
const BwdConfig* dkdv_dropout_configs(int* count);
const BwdConfig* dkdv_atomic_dropout_configs(int* count);
const BwdConfig* dq_dropout_configs(int* count);

int launch_preprocess(const PreArgs& a, int d, hipStream_t stream);

// General-entry layout adapters (fa_pad.hip): strided [B,H,N,d] view <-> contiguous
// [B,H,N,dp] buffer; gathers zero-fill columns d .. dp-1.
void launch_gather_bf16(const void* src, View s, void* dst, int B, int H, int N, int d, int dp, hipStream_t st);
void launch_gather_f32(const float* src, View s, float* dst, int B, int H, int N, int d, int dp, hipStream_t st);
void launch_scatter_f32(const float* src, float* dst, View s, int B, int H, int N, int d, int dp, hipStream_t st);

}  // namespace fa
