// Weighted combine back to token order through the inverse permutation.
// [DWDP README "Merger Module": restore token-major assignment order,
//  accumulate the top-k expert outputs, apply the routing weights]
//   out[t] = sum_j w[t,j] * y[inv[t*k+j]]  (ascending j, fp32)
//            (+ sigmoid(gate[t]) * shared[t])
// y is fp32, bf16, or fp16 with a power-of-two exponent per (row, 64 columns)
// (every format widened exactly); shared is fp32, or bf16 with bf16 y; the sum
// is fp32 in every case.  One workgroup per token (for small batches, one
// wave per 64 column groups of a token); each thread owns groups of
// VEC consecutive columns (one 16-byte load per packed row: 4 fp32 or 8
// 16-bit values), so every packed row is read once, fully coalesced.
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

// 16 bytes of y -> VEC floats (MODE: YFormat)
template <int MODE>
__device__ __forceinline__ void widen(const u32x4_t& raw, float (&v)[MODE == Y_F32 ? 4 : 8]) {
  if constexpr (MODE == Y_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(raw[i] << 16);
      v[2 * i + 1] = __uint_as_float(raw[i] & 0xFFFF0000u);
    }
  } else if constexpr (MODE == Y_F16S) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(raw[i] & 0xFFFFu));
      v[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(raw[i] >> 16));
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(raw[i]);
  }
}

// KC = assignments gathered per pass (k is processed in passes of KC); CPT =
// column groups per thread; MODE = format of y (YFormat).  Every load of a
// pass is issued before the first add, so a thread keeps KC * CPT row reads
// in flight.  With Y_F16S the routing weight of a row is scaled by the
// segment's 2^-k once, so every value enters as w * 2^-k * fp16.
template <int KC, int CPT, int MODE>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ y_,
                                                      const int32_t* __restrict__ y_scale,
                                                      const int32_t* __restrict__ inv,
                                                      const float* __restrict__ w, const void* __restrict__ shared_,
                                                      const float* __restrict__ sgl, int H, int k, int out_bf16,
                                                      void* __restrict__ out) {
  constexpr bool YB = MODE == Y_BF16;  // shared is bf16 too
  constexpr int VEC = (MODE == Y_F32) ? 4 : 8;  // columns per 16-byte group
  const u32x4_t* y = static_cast<const u32x4_t*>(y_);
  const int t = blockIdx.x;
  const int HV = H / VEC;
  float gate = 1.f;
  if (shared_ != nullptr && sgl != nullptr) gate = 1.0f / (1.0f + expf(-sgl[t]));
  // gridDim.y workgroups share a token's columns (small batches), one pass each
  const int step = CPT * (int)blockDim.x;
  for (int cbase = (int)blockIdx.y * step; cbase < HV; cbase += step * (int)gridDim.y) {
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
      int sc[KC][CPT];
#pragma unroll
      for (int j = 0; j < KC; ++j)
#pragma unroll
        for (int q = 0; q < CPT; ++q) {
          const bool ok = j0 + j < k && col[q] < HV;
          raw[j][q] = ok ? y[row[j] + col[q]] : u32x4_t{0u, 0u, 0u, 0u};
          if constexpr (MODE == Y_F16S)  // row[j] / HV = packed row; 8 groups per 64-column segment
            sc[j][q] = ok ? y_scale[(row[j] / HV) * (H / 64) + col[q] / 8] : 0;
        }
#pragma unroll
      for (int j = 0; j < KC; ++j)
        if (j0 + j < k)
#pragma unroll
          for (int q = 0; q < CPT; ++q) {
            float v[VEC];
            widen<MODE>(raw[j][q], v);
            const float wv = (MODE == Y_F16S) ? ldexpf(wj[j], -sc[j][q]) : wj[j];
#pragma unroll
            for (int c = 0; c < VEC; ++c) acc[q][c] += wv * v[c];
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
        if constexpr (YB) {
          widen<Y_BF16>(static_cast<const u32x4_t*>(shared_)[(int64_t)t * HV + cg], sv);
        } else {  // fp32, VEC / 4 groups of 4
#pragma unroll
          for (int h = 0; h < VEC / 4; ++h) {
            float s4[4];
            widen<Y_F32>(static_cast<const u32x4_t*>(shared_)[((int64_t)t * H + (int64_t)cg * VEC) / 4 + h], s4);
#pragma unroll
            for (int c = 0; c < 4; ++c) sv[4 * h + c] = s4[c];
          }
        }
#pragma unroll
        for (int c = 0; c < VEC; ++c) a[c] += gate * sv[c];
      }
      if (out_bf16) {
        uint32_t o[VEC / 2];
#pragma unroll
        for (int c = 0; c < VEC / 2; ++c) o[c] = bf16_rne(a[2 * c]) | (bf16_rne(a[2 * c + 1]) << 16);
        uint16_t* orow = static_cast<uint16_t*>(out) + (int64_t)t * H + (int64_t)cg * VEC;
        if constexpr (VEC == 8) {
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

template <int MODE>
void launch_typed(const void* y, const int32_t* ys, const int32_t* inv, const float* w, const void* shared,
                  const float* shared_gate_logit, int T, int H, int k, int out_bf16, void* out, hipStream_t s) {
  // 16-byte column groups: up to 256 threads, each owning CPT groups
  const int HV = H / (MODE == Y_F32 ? 4 : 8);
  if (T < 256 && HV > 64) {
    // few tokens: one wave per 64 column groups, so the chip has work and each
    // workgroup is done after one round of loads
    const dim3 grid((unsigned)T, (unsigned)((HV + 63) / 64));
    hipLaunchKernelGGL((combine_kernel<8, 1, MODE>), grid, dim3(64), 0, s, y, ys, inv, w, shared, shared_gate_logit, H,
                       k, out_bf16, out);
    return;
  }
  const int threads = HV > 256 ? 256 : ((HV + 63) / 64) * 64;
  const int cpt = (HV + threads - 1) / threads;
  if (cpt <= 1)
    hipLaunchKernelGGL((combine_kernel<8, 1, MODE>), dim3(T), dim3(threads), 0, s, y, ys, inv, w, shared,
                       shared_gate_logit, H, k, out_bf16, out);
  else if (cpt <= 2)
    hipLaunchKernelGGL((combine_kernel<8, 2, MODE>), dim3(T), dim3(threads), 0, s, y, ys, inv, w, shared,
                       shared_gate_logit, H, k, out_bf16, out);
  else  // wider rows take several passes of 4 groups per thread
    hipLaunchKernelGGL((combine_kernel<4, 4, MODE>), dim3(T), dim3(threads), 0, s, y, ys, inv, w, shared,
                       shared_gate_logit, H, k, out_bf16, out);
}

}  // namespace

hipError_t launch_combine(const void* y, int y_format, const int32_t* y_scale, const int32_t* inv, const float* w,
                          const void* shared, const float* shared_gate_logit, int T, int H, int k, int out_bf16,
                          void* out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (y_format == Y_F16S && (H % 64 != 0 || y_scale == nullptr)) return hipErrorInvalidValue;
  profile_begin("combine", s);
  if (y_format == Y_BF16)
    launch_typed<Y_BF16>(y, nullptr, inv, w, shared, shared_gate_logit, T, H, k, out_bf16, out, s);
  else if (y_format == Y_F16S)
    launch_typed<Y_F16S>(y, y_scale, inv, w, shared, shared_gate_logit, T, H, k, out_bf16, out, s);
  else
    launch_typed<Y_F32>(y, nullptr, inv, w, shared, shared_gate_logit, T, H, k, out_bf16, out, s);
  profile_end(s);
  return hipGetLastError();
}

}  // namespace moe
