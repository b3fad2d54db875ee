// fp32 grouped expert FFN: plain one-thread-per-output kernels with fp32 FMA
// accumulation, for fp32 layers (small correctness-grade shapes); the bf16
// path runs on the matrix cores (grouped_gemm_bf16.hip).
// [DWDP README "Executor Module"; modelexpress refit test, FusedMoEModel:
//  w13 = gate rows [0, I) then up rows [I, 2I) of each expert slot]
#include <math.h>

#include "moe_internal.h"

namespace moe {
namespace {

// Expert owning packed row p: the e with offsets[e] <= p < offsets[e+1].
__device__ __forceinline__ int owner_group(const int32_t* offsets, int E, int p) {
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= p) lo = mid; else hi = mid;
  }
  return lo;
}

__global__ __launch_bounds__(256) void ffn_gate_up_f32_kernel(
    const float* __restrict__ x, const int32_t* __restrict__ gather, const int32_t* __restrict__ offsets,
    const float* __restrict__ w13, int P, int H, int E, int I, float* __restrict__ h) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)P * I) return;
  const int p = (int)(idx / I);
  const int n = (int)(idx - (int64_t)p * I);
  int e = 0;
  if (offsets != nullptr) {
    if (p >= offsets[E]) return;
    e = owner_group(offsets, E, p);
  }
  const int64_t tok = gather ? (int64_t)gather[p] : (int64_t)p;
  const float* xr = x + tok * H;
  const float* wg = w13 + ((int64_t)e * 2 * I + n) * H;
  const float* wu = w13 + ((int64_t)e * 2 * I + I + n) * H;
  float g = 0.f, u = 0.f;
  for (int k = 0; k < H; ++k) {
    g = fmaf(xr[k], wg[k], g);
    u = fmaf(xr[k], wu[k], u);
  }
  h[(int64_t)p * I + n] = g / (1.0f + expf(-g)) * u;
}

__global__ __launch_bounds__(256) void ffn_down_f32_kernel(
    const float* __restrict__ h, const int32_t* __restrict__ offsets, const float* __restrict__ w2, int P, int H,
    int E, int I, float* __restrict__ y) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)P * H) return;
  const int p = (int)(idx / H);
  const int c = (int)(idx - (int64_t)p * H);
  int e = 0;
  if (offsets != nullptr) {
    if (p >= offsets[E]) return;
    e = owner_group(offsets, E, p);
  }
  const float* hr = h + (int64_t)p * I;
  const float* wr = w2 + ((int64_t)e * H + c) * I;
  float acc = 0.f;
  for (int i = 0; i < I; ++i) acc = fmaf(hr[i], wr[i], acc);
  y[(int64_t)p * H + c] = acc;
}

}  // namespace

hipError_t launch_ffn_gate_up_f32(const float* x, const int32_t* gather, const int32_t* offsets, const float* w13,
                                  int P, int H, int E, int I, float* h, hipStream_t s) {
  const int64_t n = (int64_t)P * I;
  if (n == 0) return hipSuccess;
  profile_begin("ffn_gate_up_f32", s);
  hipLaunchKernelGGL(ffn_gate_up_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, x, gather,
                     offsets, w13, P, H, E, I, h);
  profile_end(s);
  return hipGetLastError();
}

hipError_t launch_ffn_down_f32(const float* h, const int32_t* offsets, const float* w2, int P, int H, int E, int I,
                               float* y, hipStream_t s) {
  const int64_t n = (int64_t)P * H;
  if (n == 0) return hipSuccess;
  profile_begin("ffn_down_f32", s);
  hipLaunchKernelGGL(ffn_down_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, h, offsets, w2, P, H,
                     E, I, y);
  profile_end(s);
  return hipGetLastError();
}

}  // namespace moe
