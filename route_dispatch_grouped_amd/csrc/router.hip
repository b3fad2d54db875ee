// Router kernels: fp32 logits (the bf16 logits GEMM is an epilogue of the
// grouped MFMA GEMM) and the wavefront top-k with softmax / renormalisation.
// [DWDP README "Router Module": router logits, routing probabilities, top-k
//  expert indices, normalized routing weights; diffulex.moe "diffulex.moe.topk"]
#include <math.h>

#include "moe_internal.h"
#include "topk_wave.h"

namespace moe {
namespace {

// fp32 router logits (+ the shared-expert gate logit as row E): one wave per
// (token, router row).  Each lane multiplies 4 consecutive hidden elements per
// pass (16-byte loads, H % 4 == 0) and the wave sums its 64 partial dot
// products.
__global__ __launch_bounds__(256) void router_logits_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ wr, const float* __restrict__ bias,
    const float* __restrict__ gate, int T, int H, int E, float* __restrict__ logits,
    float* __restrict__ gate_logit) {
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  const int C = E + (gate != nullptr ? 1 : 0);
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= (int64_t)T * C) return;
  const int t = (int)(item / C);
  const int c = (int)(item - (int64_t)t * C);
  const float* xr = x + (int64_t)t * H;
  const float* w = (c < E) ? wr + (int64_t)c * H : gate;
  float acc = 0.f;
  for (int h = 4 * lane; h < H; h += 256) {
    const f32x4_t a = *reinterpret_cast<const f32x4_t*>(xr + h);
    const f32x4_t b = *reinterpret_cast<const f32x4_t*>(w + h);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = fmaf(a[i], b[i], acc);
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) acc += __shfl_xor(acc, d, 64);
  if (lane == 0) {
    if (c < E) logits[(int64_t)t * E + c] = acc + (bias ? bias[c] : 0.f);
    else gate_logit[t] = acc;
  }
}

// One wavefront per token (topk_row).
template <int VPL>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                   int renorm, int32_t* __restrict__ ids,
                                                   float* __restrict__ weights, float* __restrict__ probs,
                                                   int n_group, int topk_group) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  topk_row<VPL>(logits + (int64_t)t * E, E, k, renorm, ids + (int64_t)t * k, weights + (int64_t)t * k,
                probs ? probs + (int64_t)t * E : nullptr, lane, nullptr, n_group, topk_group);
}

// Router logits for a handful of tokens (decode batches), bf16: workgroup
// (r, b) computes row r of the router weight (r == E: the shared-expert gate
// vector) against tokens [16b, 16b + 16).  Each thread owns 8 consecutive
// hidden elements per pass (16-byte loads) and one fp32 partial dot product
// per token; the exact bf16 products are summed in fp32, then across the wave
// (DPP) and across the four waves (LDS).  The weight row is read once; the
// token rows, 4 KB each at H = 2048, come from L2 for all but the first row.
constexpr int kSmallT = 16;

__device__ __forceinline__ void bf16x8_to_f32(const uint4 v, float (&f)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

__global__ __launch_bounds__(256) void router_small_t_bf16_kernel(const uint16_t* __restrict__ x,
                                                                  const uint16_t* __restrict__ wr,
                                                                  const float* __restrict__ bias,
                                                                  const uint16_t* __restrict__ gate, int T, int H,
                                                                  int E, float* __restrict__ logits,
                                                                  float* __restrict__ gate_logit) {
  const int r = blockIdx.x;
  const int t0 = blockIdx.y * kSmallT;
  const int nt = min(kSmallT, T - t0);
  const uint16_t* w = (r < E) ? wr + (int64_t)r * H : gate;
  float acc[kSmallT];
#pragma unroll
  for (int tt = 0; tt < kSmallT; ++tt) acc[tt] = 0.f;
  for (int h = threadIdx.x * 8; h < H; h += 256 * 8) {
    // every load of the pass is issued before the first FMA (rows past the
    // batch re-read its last row and are never stored)
    uint4 xv[kSmallT];
#pragma unroll
    for (int tt = 0; tt < kSmallT; ++tt)
      xv[tt] = *reinterpret_cast<const uint4*>(x + (int64_t)(t0 + min(tt, nt - 1)) * H + h);
    float wf[8];
    bf16x8_to_f32(*reinterpret_cast<const uint4*>(w + h), wf);
#pragma unroll
    for (int tt = 0; tt < kSmallT; ++tt) {
      float xf[8];
      bf16x8_to_f32(xv[tt], xf);
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[tt] = fmaf(xf[c], wf[c], acc[tt]);
    }
  }
  __shared__ float red[4][kSmallT];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int tt = 0; tt < kSmallT; ++tt) {
    const float v = wave_sum(acc[tt]);
    if (lane == 0) red[wave][tt] = v;
  }
  __syncthreads();
  if ((int)threadIdx.x < nt) {
    const int tt = threadIdx.x;
    const float v = (red[0][tt] + red[1][tt]) + (red[2][tt] + red[3][tt]);
    if (r < E) logits[(int64_t)(t0 + tt) * E + r] = v + (bias ? bias[r] : 0.f);
    else gate_logit[t0 + tt] = v;
  }
}

}  // namespace

hipError_t launch_router_small_t_bf16(const uint16_t* x, const uint16_t* wr, const float* bias, const uint16_t* gate,
                                      int T, int H, int E, float* logits, float* gate_logit, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 grid((unsigned)(E + (gate ? 1 : 0)), (unsigned)((T + kSmallT - 1) / kSmallT));
  profile_begin("router_logits_bf16", s);
  hipLaunchKernelGGL(router_small_t_bf16_kernel, grid, dim3(256), 0, s, x, wr, bias, gate, T, H, E, logits,
                     gate_logit);
  profile_end(s);
  return hipGetLastError();
}

hipError_t launch_router_logits_f32(const float* x, const float* wr, const float* bias, const float* gate,
                                    int T, int H, int E, float* logits, float* gate_logit, hipStream_t s) {
  const int64_t n = (int64_t)T * (E + (gate ? 1 : 0));
  if (n == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((n + 3) / 4);  // four waves per workgroup, one per (token, row)
  profile_begin("router_logits_f32", s);
  hipLaunchKernelGGL(router_logits_f32_kernel, dim3(blocks), dim3(256), 0, s, x, wr, bias, gate, T, H, E,
                     logits, gate_logit);
  profile_end(s);
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int T, int E, int k, int renormalize, int32_t* ids, float* weights,
                       float* probs, hipStream_t s, int n_group, int topk_group) {
  if (T == 0) return hipSuccess;
  const dim3 grid((T + 3) / 4), block(256);
  profile_begin(n_group > 1 ? "router_topk_grouped" : "router_topk", s);
#define MOE_TOPK(VPL)                                                                                          \
  hipLaunchKernelGGL(topk_kernel<VPL>, grid, block, 0, s, logits, T, E, k, renormalize, ids, weights, probs,  \
                     n_group, topk_group)
  if (E <= 64) MOE_TOPK(1);
  else if (E <= 128) MOE_TOPK(2);
  else if (E <= 256) MOE_TOPK(4);
  else MOE_TOPK(8);
#undef MOE_TOPK
  profile_end(s);
  return hipGetLastError();
}

}  // namespace moe
