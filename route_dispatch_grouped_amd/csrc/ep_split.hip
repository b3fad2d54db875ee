// Expert-parallel routing table: the P = T*k token-major assignments split
// into the ones whose expert lies in this rank's range [start, end) and the
// rest, each bucket keeping assignment order.
// [metrale_model_layers ep_dispatch.rs: build_ep_routing_table, EpRoutingTable]
//
// A stable compaction in two launches over segments of kEpSeg assignments
// (one workgroup of 256 threads, 4 consecutive assignments per thread):
//   1. count  local assignments per segment -> seg_count[u]
//   2. split  every workgroup adds up seg_count[0..u) itself (a few hundred
//             values at most), scans its segment's flags in LDS, and writes
//             local entry a at base + rank and remote entry a at a - (locals
//             before a).  Workgroup 0 writes counts = {local, remote}.
// No atomics: the result does not depend on timing.
//
// Also the per-rank send counts of the expert-major packed order when G ranks
// own contiguous expert ranges (each rank's local_expert_start/end as in
// ep_dispatch.rs): differences of the dispatch plan's expert offsets at the
// range boundaries.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kEpSeg = 1024;
constexpr int kEpThreads = 256;

__device__ __forceinline__ bool ep_local(int32_t id, uint32_t start, uint32_t end) {
  const uint32_t e = (uint32_t)id;  // expert ids are unsigned on the page; negative int32 = large u32
  return e >= start && e < end;
}

__device__ __forceinline__ int block_excl_scan(int v, int* s_wsum, int& total) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  if (lane == 63) s_wsum[w] = incl;
  __syncthreads();
  int base = 0;
  total = 0;
#pragma unroll
  for (int q = 0; q < kEpThreads / 64; ++q) {
    if (q < w) base += s_wsum[q];
    total += s_wsum[q];
  }
  return base + incl - v;
}

__global__ __launch_bounds__(kEpThreads) void ep_count_kernel(const int32_t* __restrict__ ids, int P, uint32_t start,
                                                              uint32_t end, int32_t* __restrict__ seg_count) {
  __shared__ int s_wsum[kEpThreads / 64];
  const int a0 = blockIdx.x * kEpSeg + threadIdx.x * 4;
  int c = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (a0 + i < P && ep_local(ids[a0 + i], start, end)) ++c;
  int total;
  (void)block_excl_scan(c, s_wsum, total);
  if (threadIdx.x == 0) seg_count[blockIdx.x] = total;
}

__global__ __launch_bounds__(kEpThreads) void ep_split_kernel(
    const int32_t* __restrict__ ids, const float* __restrict__ w, int P, int k, uint32_t start, uint32_t end,
    const int32_t* __restrict__ seg_count, int U, int32_t* __restrict__ l_tok, int32_t* __restrict__ l_eid,
    float* __restrict__ l_w, int32_t* __restrict__ r_tok, int32_t* __restrict__ r_eid, float* __restrict__ r_w,
    int32_t* __restrict__ counts) {
  __shared__ int s_wsum[kEpThreads / 64];
  __shared__ int s_base[2];
  // locals before this segment (and, for workgroup 0, the grand total)
  {
    const int lim = (blockIdx.x == 0) ? U : (int)blockIdx.x;
    int v = 0;
    for (int u = threadIdx.x; u < lim; u += kEpThreads) v += seg_count[u];
    int total;
    (void)block_excl_scan(v, s_wsum, total);
    if (threadIdx.x == 0) s_base[0] = total;
    __syncthreads();
  }
  const int seg_base = (blockIdx.x == 0) ? 0 : s_base[0];
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    counts[0] = s_base[0];
    counts[1] = P - s_base[0];
  }
  __syncthreads();  // s_wsum is reused below
  const int a0 = blockIdx.x * kEpSeg + threadIdx.x * 4;
  int32_t id[4];
  bool loc[4];
  int c = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    id[i] = (a0 + i < P) ? ids[a0 + i] : 0;
    loc[i] = a0 + i < P && ep_local(id[i], start, end);
    c += loc[i] ? 1 : 0;
  }
  int seg_total;
  int rank = block_excl_scan(c, s_wsum, seg_total);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int a = a0 + i;
    if (a >= P) break;
    const int before = seg_base + rank;  // locals before assignment a
    const int tok = a / k;
    if (loc[i]) {
      l_tok[before] = tok;
      l_eid[before] = id[i];
      l_w[before] = w[a];
      ++rank;
    } else {
      const int pos = a - before;
      r_tok[pos] = tok;
      r_eid[pos] = id[i];
      r_w[pos] = w[a];
    }
  }
}

// Per-rank send counts of the expert-major packed order for G expert-parallel
// ranks with contiguous expert ranges: rank r owns [r*E/G, (r+1)*E/G) (floor),
// so its segment of the packed order starts at offsets[r*E/G] and holds
// offsets[(r+1)*E/G] - offsets[r*E/G] rows.  Thread r < G writes counts[r] and
// starts[r]; thread G writes starts[G] = offsets[E].
__global__ __launch_bounds__(256) void ep_rank_counts_kernel(const int32_t* __restrict__ offsets, int E, int G,
                                                             int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ starts) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r > G) return;
  if (r == G) {
    if (starts != nullptr) starts[G] = offsets[E];
    return;
  }
  const int lo = (int)(((int64_t)r * E) / G);
  const int hi = (int)(((int64_t)(r + 1) * E) / G);
  counts[r] = offsets[hi] - offsets[lo];
  if (starts != nullptr) starts[r] = offsets[lo];
}

}  // namespace

size_t ep_split_scratch_bytes(int64_t P) { return (size_t)((P + kEpSeg - 1) / kEpSeg) * sizeof(int32_t); }

hipError_t launch_ep_rank_counts(const int32_t* offsets, int E, int G, int32_t* counts, int32_t* starts,
                                 hipStream_t s) {
  profile_begin("ep_rank_counts", s);
  hipLaunchKernelGGL(ep_rank_counts_kernel, dim3((G + 1 + 255) / 256), dim3(256), 0, s, offsets, E, G, counts,
                     starts);
  profile_end(s);
  return hipGetLastError();
}

hipError_t launch_ep_split(const int32_t* ids, const float* w, int T, int k, int64_t start, int64_t end,
                           int32_t* l_tok, int32_t* l_eid, float* l_w, int32_t* r_tok, int32_t* r_eid, float* r_w,
                           int32_t* counts, void* scratch, hipStream_t s) {
  const int P = T * k;
  // [start, end) clipped to the u32 range of expert ids
  const uint32_t st = (uint32_t)(start < 0 ? 0 : (start > 0xFFFFFFFFll ? 0xFFFFFFFFll : start));
  const uint32_t en = (uint32_t)(end < 0 ? 0 : (end > 0xFFFFFFFFll ? 0xFFFFFFFFll : end));
  const int U = (P + kEpSeg - 1) / kEpSeg;
  int32_t* seg_count = static_cast<int32_t*>(scratch);
  profile_begin("ep_routing_table", s);
  if (U > 0)
    hipLaunchKernelGGL(ep_count_kernel, dim3(U), dim3(kEpThreads), 0, s, ids, P, st, en, seg_count);
  hipLaunchKernelGGL(ep_split_kernel, dim3(U > 0 ? U : 1), dim3(kEpThreads), 0, s, ids, w, P, k, st, en, seg_count,
                     U, l_tok, l_eid, l_w, r_tok, r_eid, r_w, counts);
  profile_end(s);
  return hipGetLastError();
}

}  // namespace moe
