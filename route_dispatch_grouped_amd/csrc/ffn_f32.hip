// fp32 grouped expert FFN (fp32 layers: small, correctness-grade shapes; the
// bf16 path runs on the matrix cores in grouped_gemm_bf16.hip).
// [DWDP README "Executor Module"; modelexpress refit test, FusedMoEModel:
//  w13 = gate rows [0, I) then up rows [I, 2I) of each expert slot]
//
// One kernel for both projections: a tile is 32 packed rows x 64 output
// columns (gate/up: 64 h columns, i.e. the 64 matching gate rows and 64 up
// rows of the expert's w13), K in steps of 32 staged through LDS with 16-byte
// coalesced loads (gathered token rows for gate/up).  Each thread owns 2 rows
// x 4 columns and accumulates over k in ascending order with fp32 FMA, so
// every output is the same sequence of roundings as a plain dot product.
// The tile list is derived from expert_offsets inside each workgroup: expert
// e contributes ceil(rows_e / 32) m-tiles, in expert order.
#include <math.h>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kBM = 32;
constexpr int kBN = 64;
constexpr int kBK = 32;
constexpr int kThreadsF = 256;

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Expert, first row and rows of m-tile `tile`: the experts' tile counts
// ceil(rows / kBM) scanned in LDS.  Returns false (for the whole workgroup)
// when the tile is past the last one.
__device__ bool find_tile(const int32_t* __restrict__ offsets, int E, int P, int tile, int* s_scan, int& e_out,
                          int& m0, int& rows) {
  const int tid = threadIdx.x;
  if (offsets == nullptr) {
    e_out = 0;
    m0 = tile * kBM;
    rows = min(kBM, P - m0);
    return m0 < P;
  }
  // s_scan[e + 1] = tiles of experts 0..e (E <= MOE_MAX_GROUPS_INTERNAL = 2 per thread)
  int c[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int e = 2 * tid + i;
    c[i] = (e < E) ? (offsets[e + 1] - offsets[e] + kBM - 1) / kBM : 0;
  }
  s_scan[tid + 1] = c[0] + c[1];
  if (tid == 0) s_scan[0] = 0;
  __syncthreads();
  // inclusive scan of the 256 pair sums (Hillis-Steele: read, barrier, add, barrier)
  for (int d = 1; d < kThreadsF; d <<= 1) {
    const int v = (tid + 1 > d) ? s_scan[tid + 1 - d] : 0;
    __syncthreads();
    s_scan[tid + 1] += v;
    __syncthreads();
  }
  // s_scan[j] = tiles of experts [0, 2j); the expert of `tile`: scan pairs,
  // then the member of the pair
  const int total = s_scan[kThreadsF];
  if (tile >= total) return false;
  int lo = 0, hi = kThreadsF;  // largest j with s_scan[j] <= tile
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_scan[mid] <= tile) lo = mid; else hi = mid;
  }
  int e = 2 * lo;
  int t0 = s_scan[lo];
  const int c0 = (offsets[e + 1] - offsets[e] + kBM - 1) / kBM;
  if (tile - t0 >= c0) {
    t0 += c0;
    e += 1;
  }
  e_out = e;
  m0 = offsets[e] + (tile - t0) * kBM;
  rows = min(kBM, offsets[e + 1] - m0);
  return true;
}

// SWIGLU: out[p, c] = silu(x_p . wg_c) * (x_p . wu_c), c < N = I, with
// wg_c = W[e][c], wu_c = W[e][up_row0 + c]; otherwise out[p, c] = a_p . W[e][c]
// (c < N).  A rows have K values (K % 8 == 0); W groups are w_stride apart.
template <bool SWIGLU>
__global__ __launch_bounds__(kThreadsF) void ffn_f32_tiled_kernel(
    const float* __restrict__ A, const int32_t* __restrict__ gather, const int32_t* __restrict__ offsets,
    const float* __restrict__ W, int P, int K, int N, int E, int64_t w_stride, int up_row0,
    float* __restrict__ out) {
  constexpr int NW = SWIGLU ? 2 : 1;
  __shared__ int s_scan[kThreadsF + 1];
  __shared__ float s_a[kBK][kBM + 1];
  __shared__ float s_w[NW][kBK][kBN + 4];

  const int tid = threadIdx.x;
  int e, m0, rows;
  if (!find_tile(offsets, E, P, blockIdx.x, s_scan, e, m0, rows)) return;
  const int n0 = blockIdx.y * kBN;
  const float* __restrict__ We = W + (int64_t)e * w_stride;

  // load assignments: A row tid / 8 (32 rows), 4 k from (tid % 8) * 4;
  // W rows tid / 8 and tid / 8 + 32 (64 columns), same k
  const int lr = tid >> 3, lk = (tid & 7) * 4;
  const int64_t arow = (lr < rows) ? (gather ? (int64_t)gather[m0 + lr] : (int64_t)(m0 + lr)) : -1;
  int wrow[2][2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = n0 + lr + 32 * h;
    wrow[0][h] = (c < N) ? c : -1;
    wrow[1][h] = (c < N) ? up_row0 + c : -1;
  }
  // compute assignment: rows 2 ty, 2 ty + 1; columns 4 tx .. 4 tx + 3
  const int ty = tid >> 4, tx = tid & 15;
  float acc[NW][2][4];
#pragma unroll
  for (int m = 0; m < NW; ++m)
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[m][r][c] = 0.f;

  for (int k0 = 0; k0 < K; k0 += kBK) {
    const bool kin = k0 + lk < K;  // K % 4 == 0: a 4-wide chunk is wholly in or out
    f32x4_t av = {0.f, 0.f, 0.f, 0.f};
    if (arow >= 0 && kin) av = *reinterpret_cast<const f32x4_t*>(A + arow * K + k0 + lk);
#pragma unroll
    for (int i = 0; i < 4; ++i) s_a[lk + i][lr] = av[i];
#pragma unroll
    for (int m = 0; m < NW; ++m)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f32x4_t wv = {0.f, 0.f, 0.f, 0.f};
        if (wrow[m][h] >= 0 && kin) wv = *reinterpret_cast<const f32x4_t*>(We + (int64_t)wrow[m][h] * K + k0 + lk);
#pragma unroll
        for (int i = 0; i < 4; ++i) s_w[m][lk + i][lr + 32 * h] = wv[i];
      }
    __syncthreads();
    const int kn = min(kBK, K - k0);
    for (int k = 0; k < kn; ++k) {
      const float a0 = s_a[k][2 * ty], a1 = s_a[k][2 * ty + 1];
#pragma unroll
      for (int m = 0; m < NW; ++m) {
        const f32x4_t b = *reinterpret_cast<const f32x4_t*>(&s_w[m][k][4 * tx]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          acc[m][0][c] = fmaf(a0, b[c], acc[m][0][c]);
          acc[m][1][c] = fmaf(a1, b[c], acc[m][1][c]);
        }
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int row = 2 * ty + r;
    if (row >= rows) continue;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int col = n0 + 4 * tx + c;
      if (col >= N) continue;
      float v;
      if (SWIGLU) {
        const float g = acc[0][r][c];
        v = g / (1.0f + expf(-g)) * acc[NW - 1][r][c];
      } else {
        v = acc[0][r][c];
      }
      out[(int64_t)(m0 + row) * N + col] = v;
    }
  }
}

hipError_t launch_tiled(bool swiglu, const float* A, const int32_t* gather, const int32_t* offsets, const float* W,
                        int P, int K, int N, int E, int64_t w_stride, int up_row0, float* out, hipStream_t s) {
  int64_t ub = ((int64_t)P + kBM - 1) / kBM;
  if (offsets) ub += (E < P ? E : P);
  const dim3 grid((unsigned)ub, (unsigned)((N + kBN - 1) / kBN));
  if (swiglu)
    hipLaunchKernelGGL(ffn_f32_tiled_kernel<true>, grid, dim3(kThreadsF), 0, s, A, gather, offsets, W, P, K, N, E,
                       w_stride, up_row0, out);
  else
    hipLaunchKernelGGL(ffn_f32_tiled_kernel<false>, grid, dim3(kThreadsF), 0, s, A, gather, offsets, W, P, K, N, E,
                       w_stride, up_row0, out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ffn_gate_up_f32(const float* x, const int32_t* gather, const int32_t* offsets, const float* w13,
                                  int P, int H, int E, int I, float* h, hipStream_t s) {
  if ((int64_t)P * I == 0) return hipSuccess;
  if (E > MOE_MAX_GROUPS_INTERNAL) return hipErrorInvalidValue;
  profile_begin("ffn_gate_up_f32", s);
  const hipError_t e = launch_tiled(true, x, gather, offsets, w13, P, H, I, E, (int64_t)2 * I * H, I, h, s);
  profile_end(s);
  return e;
}

hipError_t launch_ffn_down_f32(const float* h, const int32_t* offsets, const float* w2, int P, int H, int E, int I,
                               float* y, hipStream_t s) {
  if ((int64_t)P * H == 0) return hipSuccess;
  if (E > MOE_MAX_GROUPS_INTERNAL) return hipErrorInvalidValue;
  profile_begin("ffn_down_f32", s);
  const hipError_t e = launch_tiled(false, h, nullptr, offsets, w2, P, I, H, E, (int64_t)H * I, 0, y, s);
  profile_end(s);
  return e;
}

}  // namespace moe
