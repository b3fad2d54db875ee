// Weighted combine back to token order through the inverse permutation.
// [DWDP README "Merger Module": restore token-major assignment order,
//  accumulate the top-k expert outputs, apply the routing weights]
//   out[t] = sum_j w[t,j] * y[inv[t*k+j]]  (ascending j, fp32)
//            (+ sigmoid(gate[t]) * shared[t])
// One workgroup per token; each thread owns 4 consecutive columns (16-byte
// loads), so every packed row is read once, fully coalesced.
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

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y, const int32_t* __restrict__ inv,
                                                      const float* __restrict__ w, const float* __restrict__ shared,
                                                      const float* __restrict__ sgl, int H, int k, int out_bf16,
                                                      void* __restrict__ out) {
  const int t = blockIdx.x;
  const int H4 = H >> 2;
  float gate = 1.f;
  if (shared != nullptr && sgl != nullptr) gate = 1.0f / (1.0f + expf(-sgl[t]));
  for (int c = threadIdx.x; c < H4; c += blockDim.x) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const int64_t p = inv[(int64_t)t * k + j];
      const float wj = w[(int64_t)t * k + j];
      const f32x4_t v = reinterpret_cast<const f32x4_t*>(y + p * H)[c];
      acc += wj * v;
    }
    if (shared != nullptr) {
      const f32x4_t v = reinterpret_cast<const f32x4_t*>(shared + (int64_t)t * H)[c];
      acc += gate * v;
    }
    if (out_bf16) {
      uint2 o;
      o.x = bf16_rne(acc[0]) | (bf16_rne(acc[1]) << 16);
      o.y = bf16_rne(acc[2]) | (bf16_rne(acc[3]) << 16);
      reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + (int64_t)t * H)[c] = o;
    } else {
      reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(out) + (int64_t)t * H)[c] = acc;
    }
  }
}

}  // namespace

hipError_t launch_combine(const float* y, const int32_t* inv, const float* w, const float* shared,
                          const float* shared_gate_logit, int T, int H, int k, int out_bf16, void* out,
                          hipStream_t s) {
  if (T == 0) return hipSuccess;
  int threads = H / 4;
  if (threads > 256) threads = 256;
  threads = ((threads + 63) / 64) * 64;
  profile_begin("combine", s);
  hipLaunchKernelGGL(combine_kernel, dim3(T), dim3(threads), 0, s, y, inv, w, shared, shared_gate_logit, H, k,
                     out_bf16, out);
  profile_end(s);
  return hipGetLastError();
}

}  // namespace moe
