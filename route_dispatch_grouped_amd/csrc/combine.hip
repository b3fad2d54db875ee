// Weighted combine back to token order through the inverse permutation.
// [DWDP README "Merger Module": restore token-major assignment order,
//  accumulate the top-k expert outputs, apply the routing weights]
//   out[t] = sum_j w[t,j] * y[inv[t*k+j]]  (ascending j, fp32)
//            (+ sigmoid(gate[t]) * shared[t])
// y and shared are fp32 or bf16 (widened exactly); the sum is fp32 either way.
// One workgroup per token; each thread owns groups of VEC consecutive columns
// (one 16-byte load per packed row: 4 fp32 or 8 bf16 values), so every packed
// row is read once, fully coalesced.
#include <math.h>

#include "moe_internal.h"

namespace moe {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// 16 bytes of y -> VEC floats
template <bool YB>
__device__ __forceinline__ void widen(const u32x4_t& raw, float (&v)[YB ? 8 : 4]) {
  if constexpr (YB) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(raw[i] << 16);
      v[2 * i + 1] = __uint_as_float(raw[i] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(raw[i]);
  }
}

// KC = assignments gathered per pass (k is processed in passes of KC); CPT =
// column groups per thread; YB = y and shared stored as bf16.  Every load of a
// pass is issued before the first add, so a thread keeps KC * CPT row reads
// in flight.
template <int KC, int CPT, bool YB>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ y_, const int32_t* __restrict__ inv,
                                                      const float* __restrict__ w, const void* __restrict__ shared_,
                                                      const float* __restrict__ sgl, int H, int k, int out_bf16,
                                                      void* __restrict__ out) {
  constexpr int VEC = YB ? 8 : 4;  // columns per 16-byte group
  const u32x4_t* y = static_cast<const u32x4_t*>(y_);
  const int t = blockIdx.x;
  const int HV = H / VEC;
  float gate = 1.f;
  if (shared_ != nullptr && sgl != nullptr) gate = 1.0f / (1.0f + expf(-sgl[t]));
  for (int cbase = 0; cbase < HV; cbase += CPT * (int)blockDim.x) {
    float acc[CPT][VEC];
    int col[CPT];
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
#pragma unroll
      for (int c = 0; c < VEC; ++c) acc[q][c] = 0.f;
      col[q] = cbase + threadIdx.x + q * blockDim.x;
    }
    for (int j0 = 0; j0 < k; j0 += KC) {
      int64_t row[KC];
      float wj[KC];
#pragma unroll
      for (int j = 0; j < KC; ++j) {
        const bool live = j0 + j < k;
        row[j] = live ? (int64_t)inv[(int64_t)t * k + j0 + j] * HV : 0;
        wj[j] = live ? w[(int64_t)t * k + j0 + j] : 0.f;
      }
      u32x4_t raw[KC][CPT];
#pragma unroll
      for (int j = 0; j < KC; ++j)
#pragma unroll
        for (int q = 0; q < CPT; ++q)
          raw[j][q] = (j0 + j < k && col[q] < HV) ? y[row[j] + col[q]] : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < KC; ++j)
        if (j0 + j < k)
#pragma unroll
          for (int q = 0; q < CPT; ++q) {
            float v[VEC];
            widen<YB>(raw[j][q], v);
#pragma unroll
            for (int c = 0; c < VEC; ++c) acc[q][c] += wj[j] * v[c];
          }
    }
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int cg = col[q];
      if (cg >= HV) continue;
      float a[VEC];
#pragma unroll
      for (int c = 0; c < VEC; ++c) a[c] = acc[q][c];
      if (shared_ != nullptr) {
        float sv[VEC];
        widen<YB>(static_cast<const u32x4_t*>(shared_)[(int64_t)t * HV + cg], sv);
#pragma unroll
        for (int c = 0; c < VEC; ++c) a[c] += gate * sv[c];
      }
      if (out_bf16) {
        uint32_t o[VEC / 2];
#pragma unroll
        for (int c = 0; c < VEC / 2; ++c) o[c] = bf16_rne(a[2 * c]) | (bf16_rne(a[2 * c + 1]) << 16);
        uint16_t* orow = static_cast<uint16_t*>(out) + (int64_t)t * H + (int64_t)cg * VEC;
        if constexpr (YB) {
          *reinterpret_cast<u32x4_t*>(orow) = u32x4_t{o[0], o[1], o[2], o[3]};
        } else {
          *reinterpret_cast<uint2*>(orow) = uint2{o[0], o[1]};
        }
      } else {
        f32x4_t* orow = reinterpret_cast<f32x4_t*>(static_cast<float*>(out) + (int64_t)t * H + (int64_t)cg * VEC);
#pragma unroll
        for (int c = 0; c < VEC / 4; ++c) orow[c] = f32x4_t{a[4 * c], a[4 * c + 1], a[4 * c + 2], a[4 * c + 3]};
      }
    }
  }
}

template <bool YB>
void launch_typed(const void* y, const int32_t* inv, const float* w, const void* shared,
                  const float* shared_gate_logit, int T, int H, int k, int out_bf16, void* out, hipStream_t s) {
  // 16-byte column groups: up to 256 threads, each owning CPT groups
  const int HV = H / (YB ? 8 : 4);
  const int threads = HV > 256 ? 256 : ((HV + 63) / 64) * 64;
  const int cpt = (HV + threads - 1) / threads;
  if (cpt <= 1)
    hipLaunchKernelGGL((combine_kernel<8, 1, YB>), dim3(T), dim3(threads), 0, s, y, inv, w, shared,
                       shared_gate_logit, H, k, out_bf16, out);
  else if (cpt <= 2)
    hipLaunchKernelGGL((combine_kernel<8, 2, YB>), dim3(T), dim3(threads), 0, s, y, inv, w, shared,
                       shared_gate_logit, H, k, out_bf16, out);
  else  // wider rows take several passes of 4 groups per thread
    hipLaunchKernelGGL((combine_kernel<4, 4, YB>), dim3(T), dim3(threads), 0, s, y, inv, w, shared,
                       shared_gate_logit, H, k, out_bf16, out);
}

}  // namespace

hipError_t launch_combine(const void* y, int y_bf16, const int32_t* inv, const float* w, const void* shared,
                          const float* shared_gate_logit, int T, int H, int k, int out_bf16, void* out,
                          hipStream_t s) {
  if (T == 0) return hipSuccess;
  profile_begin("combine", s);
  if (y_bf16)
    launch_typed<true>(y, inv, w, shared, shared_gate_logit, T, H, k, out_bf16, out, s);
  else
    launch_typed<false>(y, inv, w, shared, shared_gate_logit, T, H, k, out_bf16, out, s);
  profile_end(s);
  return hipGetLastError();
}

}  // namespace moe
