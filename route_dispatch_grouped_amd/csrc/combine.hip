// Weighted combine back to token order through the inverse permutation.
// [DWDP README "Merger Module": restore token-major assignment order,
//  accumulate the top-k expert outputs, apply the routing weights]
//   out[t] = sum_j w[t,j] * y[inv[t*k+j]]  (ascending j, fp32)
//            (+ sigmoid(gate[t]) * shared[t])
// One workgroup per token; each thread owns groups of 4 consecutive columns
// (16-byte loads), so every packed row is read once, fully coalesced.
#include <math.h>

#include "moe_internal.h"

namespace moe {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// KC = assignments gathered per pass (k is processed in passes of KC); CPT =
// 16-byte column groups per thread.  Every load of a pass is issued before the
// first add, so a thread keeps KC * CPT row reads in flight.
template <int KC, int CPT>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y, const int32_t* __restrict__ inv,
                                                      const float* __restrict__ w, const float* __restrict__ shared,
                                                      const float* __restrict__ sgl, int H, int k, int out_bf16,
                                                      void* __restrict__ out) {
  const int t = blockIdx.x;
  const int H4 = H >> 2;
  float gate = 1.f;
  if (shared != nullptr && sgl != nullptr) gate = 1.0f / (1.0f + expf(-sgl[t]));
  for (int cbase = 0; cbase < H4; cbase += CPT * (int)blockDim.x) {
    f32x4_t acc[CPT];
    int col[CPT];
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      acc[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      col[q] = cbase + threadIdx.x + q * blockDim.x;
    }
    for (int j0 = 0; j0 < k; j0 += KC) {
      int64_t row[KC];
      float wj[KC];
#pragma unroll
      for (int j = 0; j < KC; ++j) {
        const bool live = j0 + j < k;
        row[j] = live ? (int64_t)inv[(int64_t)t * k + j0 + j] * H4 : 0;
        wj[j] = live ? w[(int64_t)t * k + j0 + j] : 0.f;
      }
      f32x4_t v[KC][CPT];
#pragma unroll
      for (int j = 0; j < KC; ++j)
#pragma unroll
        for (int q = 0; q < CPT; ++q)
          v[j][q] = (j0 + j < k && col[q] < H4) ? reinterpret_cast<const f32x4_t*>(y)[row[j] + col[q]]
                                                  : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < KC; ++j)
        if (j0 + j < k)
#pragma unroll
          for (int q = 0; q < CPT; ++q) acc[q] += wj[j] * v[j][q];
    }
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int c = col[q];
      if (c >= H4) continue;
      f32x4_t a = acc[q];
      if (shared != nullptr) {
        const f32x4_t sv = reinterpret_cast<const f32x4_t*>(shared + (int64_t)t * H)[c];
        a += gate * sv;
      }
      if (out_bf16) {
        uint2 o;
        o.x = bf16_rne(a[0]) | (bf16_rne(a[1]) << 16);
        o.y = bf16_rne(a[2]) | (bf16_rne(a[3]) << 16);
        reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + (int64_t)t * H)[c] = o;
      } else {
        reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(out) + (int64_t)t * H)[c] = a;
      }
    }
  }
}

}  // namespace

hipError_t launch_combine(const float* y, const int32_t* inv, const float* w, const float* shared,
                          const float* shared_gate_logit, int T, int H, int k, int out_bf16, void* out,
                          hipStream_t s) {
  if (T == 0) return hipSuccess;
  // 16-byte column groups: up to 256 threads, each owning CPT groups
  const int H4 = H / 4;
  int threads = H4 > 256 ? 256 : ((H4 + 63) / 64) * 64;
  const int cpt = (H4 + threads - 1) / threads;
  profile_begin("combine", s);
  if (cpt <= 1)
    hipLaunchKernelGGL((combine_kernel<8, 1>), dim3(T), dim3(threads), 0, s, y, inv, w, shared, shared_gate_logit,
                       H, k, out_bf16, out);
  else if (cpt <= 2)
    hipLaunchKernelGGL((combine_kernel<8, 2>), dim3(T), dim3(threads), 0, s, y, inv, w, shared, shared_gate_logit,
                       H, k, out_bf16, out);
  else  // wider rows take several passes of 4 groups per thread
    hipLaunchKernelGGL((combine_kernel<4, 4>), dim3(T), dim3(threads), 0, s, y, inv, w, shared, shared_gate_logit,
                       H, k, out_bf16, out);
  profile_end(s);
  return hipGetLastError();
}

}  // namespace moe
