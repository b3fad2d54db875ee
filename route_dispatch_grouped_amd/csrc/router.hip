// Router kernels: fp32 logits (the bf16 logits GEMM is an epilogue of the
// grouped MFMA GEMM) and the wavefront top-k with softmax / renormalisation.
// [DWDP README "Router Module": router logits, routing probabilities, top-k
//  expert indices, normalized routing weights; diffulex.moe "diffulex.moe.topk"]
#include <math.h>

#include "moe_internal.h"

namespace moe {
namespace {

// One thread per (token, column); column E is the shared expert's gate vector.
__global__ __launch_bounds__(256) void router_logits_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ wr, const float* __restrict__ bias,
    const float* __restrict__ gate, int T, int H, int E, float* __restrict__ logits,
    float* __restrict__ gate_logit) {
  const int C = E + (gate != nullptr ? 1 : 0);
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)T * C) return;
  const int t = (int)(idx / C);
  const int c = (int)(idx - (int64_t)t * C);
  const float* xr = x + (int64_t)t * H;
  const float* w = (c < E) ? wr + (int64_t)c * H : gate;
  float acc = 0.f;
  for (int h = 0; h < H; ++h) acc = fmaf(xr[h], w[h], acc);
  if (c < E) logits[(int64_t)t * E + c] = acc + (bias ? bias[c] : 0.f);
  else gate_logit[t] = acc;
}

// Order-preserving map float -> uint32 (larger float -> larger key), after
// -0.0 has been folded onto +0.0.  NaN is not a supported input.
__device__ __forceinline__ uint32_t order_key(float f) {
  if (f == 0.f) f = 0.f;
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float order_value(uint32_t o) {
  const uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __uint_as_float(u);
}

// One step of a max-reduction through a DPP lane permutation (within 16-lane rows).
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_max_step(uint64_t v) {
  const int hi = (int)(v >> 32), lo = (int)(v & 0xFFFFFFFFu);
  const uint32_t ohi = (uint32_t)__builtin_amdgcn_update_dpp(hi, hi, CTRL, 0xF, 0xF, false);
  const uint32_t olo = (uint32_t)__builtin_amdgcn_update_dpp(lo, lo, CTRL, 0xF, 0xF, false);
  const uint64_t o = ((uint64_t)ohi << 32) | olo;
  return o > v ? o : v;
}

// Wave-wide maximum of a 64-bit key, returned wave-uniform: DPP exchanges
// (xor 1, xor 2, half-row mirror, row mirror) leave every lane of a 16-lane
// row holding the row maximum; the four row maxima are then read out with
// readlane.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = dpp_max_step<0xB1>(v);   // quad_perm(1,0,3,2)
  v = dpp_max_step<0x4E>(v);   // quad_perm(2,3,0,1)
  v = dpp_max_step<0x141>(v);  // row_half_mirror
  v = dpp_max_step<0x140>(v);  // row_mirror
  uint64_t best = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(v >> 32), 16 * r);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(v & 0xFFFFFFFFu), 16 * r);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    best = o > best ? o : best;
  }
  return best;
}

template <int CTRL>
__device__ __forceinline__ float dpp_add_step(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, 0xF, 0xF,
                                                         false));
}

// Wave-wide float sum, wave-uniform (same exchange pattern as wave_max_u64).
__device__ __forceinline__ float wave_sum(float v) {
  v = dpp_add_step<0xB1>(v);
  v = dpp_add_step<0x4E>(v);
  v = dpp_add_step<0x141>(v);
  v = dpp_add_step<0x140>(v);
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) s += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16 * r));
  return s;
}

// One wavefront per token.  Lane l holds the logits of experts l, l+64, ...
// k rounds of a wave-wide max over the 64-bit key (value key << 32 | ~id): the
// larger logit wins, and on equal logits the lower expert id has the larger
// ~id and wins.  Winner j is kept by lane j % 64 in slot j / 64.
template <int VPL>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                   int renorm, int32_t* __restrict__ ids,
                                                   float* __restrict__ weights, float* __restrict__ probs) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + (int64_t)t * E;

  float v[VPL];
  uint32_t key[VPL];
  uint32_t avail = 0;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + 64 * i;
    if (e < E) {
      v[i] = row[e];
      key[i] = order_key(v[i]);
      avail |= 1u << i;
    } else {
      v[i] = -INFINITY;
      key[i] = 0;
    }
  }

  int my_id[VPL];
  float my_val[VPL];
#pragma unroll
  for (int c = 0; c < VPL; ++c) {
    my_id[c] = 0;
    my_val[c] = 0.f;
    const int jn = min(64, k - 64 * c);
    for (int jj = 0; jj < jn; ++jj) {
      uint64_t best = 0;
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        if ((avail >> i) & 1u) {
          const uint64_t kk = ((uint64_t)key[i] << 32) | (uint32_t)(~(uint32_t)(lane + 64 * i));
          best = kk > best ? kk : best;
        }
      }
      best = wave_max_u64(best);
      const int id = (int)(~(uint32_t)(best & 0xFFFFFFFFu));
      if ((id & 63) == lane) avail &= ~(1u << (id >> 6));
      if (jj == lane) {
        my_id[c] = id;
        my_val[c] = order_value((uint32_t)(best >> 32));
      }
    }
  }

  const float m = __shfl(my_val[0], 0, 64);  // largest logit
  float s_sel = 0.f, s_all = 0.f;
#pragma unroll
  for (int c = 0; c < VPL; ++c)
    if (64 * c + lane < k) s_sel += expf(my_val[c] - m);
  s_sel = wave_sum(s_sel);
  if (!renorm || probs != nullptr) {
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (lane + 64 * i < E) s_all += expf(v[i] - m);
    s_all = wave_sum(s_all);
  }
  const float denom = renorm ? s_sel : s_all;
#pragma unroll
  for (int c = 0; c < VPL; ++c) {
    const int j = 64 * c + lane;
    if (j < k) {
      ids[(int64_t)t * k + j] = my_id[c];
      weights[(int64_t)t * k + j] = expf(my_val[c] - m) / denom;
    }
  }
  if (probs != nullptr) {
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = lane + 64 * i;
      if (e < E) probs[(int64_t)t * E + e] = expf(v[i] - m) / s_all;
    }
  }
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
    float wf[8];
    bf16x8_to_f32(*reinterpret_cast<const uint4*>(w + h), wf);
#pragma unroll
    for (int tt = 0; tt < kSmallT; ++tt) {
      if (tt < nt) {
        float xf[8];
        bf16x8_to_f32(*reinterpret_cast<const uint4*>(x + (int64_t)(t0 + tt) * H + h), xf);
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[tt] = fmaf(xf[c], wf[c], acc[tt]);
      }
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
  const unsigned blocks = (unsigned)((n + 255) / 256);
  profile_begin("router_logits_f32", s);
  hipLaunchKernelGGL(router_logits_f32_kernel, dim3(blocks), dim3(256), 0, s, x, wr, bias, gate, T, H, E,
                     logits, gate_logit);
  profile_end(s);
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int T, int E, int k, int renormalize, int32_t* ids, float* weights,
                       float* probs, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 grid((T + 3) / 4), block(256);
  profile_begin("router_topk", s);
  if (E <= 64) hipLaunchKernelGGL(topk_kernel<1>, grid, block, 0, s, logits, T, E, k, renormalize, ids, weights, probs);
  else if (E <= 128) hipLaunchKernelGGL(topk_kernel<2>, grid, block, 0, s, logits, T, E, k, renormalize, ids, weights, probs);
  else if (E <= 256) hipLaunchKernelGGL(topk_kernel<4>, grid, block, 0, s, logits, T, E, k, renormalize, ids, weights, probs);
  else hipLaunchKernelGGL(topk_kernel<8>, grid, block, 0, s, logits, T, E, k, renormalize, ids, weights, probs);
  profile_end(s);
  return hipGetLastError();
}

}  // namespace moe
