// K-blocked copies of expert weights (MOE_DTYPE_BF16_KB32 layers).
// [DWDP README "Executor Module"; modelexpress refit test: w13 [E, 2I, H],
//  w2 [E, H, I]]
//
// dst[g][b][r][i] = src[g][r][32 b + i] (zero past k): a K step of 32 of any
// block of consecutive rows is one contiguous run, so the grouped GEMMs' DMA
// instructions fetch whole 128-byte lines.
#include "moe_internal.h"

namespace moe {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// One thread per 16-byte chunk of dst (8 elements, a quarter of a row's
// block), in dst order: writes are contiguous, each group of 4 threads reads
// 64 contiguous bytes of one source row.
__global__ __launch_bounds__(256) void pack_kb32_kernel(const u32x4_t* __restrict__ src, u32x4_t* __restrict__ dst,
                                                        int64_t G, int64_t R, int64_t K) {
  const int64_t KB = (K + kKBlock - 1) / kKBlock;
  const int64_t n = G * KB * R * 4;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t c = i & 3;
    const int64_t rb = i >> 2;  // (g * KB + b) * R + r
    const int64_t r = rb % R;
    const int64_t gb = rb / R;
    const int64_t b = gb % KB;
    const int64_t g = gb / KB;
    const int64_t k0 = b * kKBlock + c * 8;
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (k0 < K) v = src[((g * R + r) * K + k0) / 8];
    dst[i] = v;
  }
}

}  // namespace

hipError_t launch_pack_kb32(const void* src, void* dst, int64_t G, int64_t R, int64_t K, hipStream_t s) {
  const int64_t n = G * ((K + kKBlock - 1) / kKBlock) * R * 4;
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(pack_kb32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, static_cast<const u32x4_t*>(src),
                     static_cast<u32x4_t*>(dst), G, R, K);
  return hipGetLastError();
}

}  // namespace moe
