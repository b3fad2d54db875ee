// Dispatch plan: a deterministic counting sort of the token-major assignments
// by expert id.  [DWDP README "Dispatcher Module": per-expert counts, expert
// offsets, token permutation, inverse permutation, packed token indices and
// packed routing weights; metrale ep_dispatch.rs: assignments a = t*k + j are
// kept in the order given]
//
// For P <= kDispatchSmallP one workgroup does all of it in LDS
// (dispatch_small_kernel).  Otherwise the P = T*k assignments are cut into
// segments of kDispatchSegment (128) consecutive indices, one wavefront per
// segment.
//   1. hist    each wave counts its segment per expert in LDS and writes
//              cnt[e][u] (expert-major, U = number of segments).
//   2. scan    one wave per expert: an exclusive scan of cnt[e][0..U) into
//              base[e][u]; the total -> counts[e].
//   3. scatter every workgroup scans the expert totals into offsets (the first
//              one writes them out, offsets[E] = P); each wave stages
//              offsets[e] + base[e][u] for every expert in LDS, then re-reads
//              its segment 64 assignments at a time, in
//              index order.  Lanes holding the same expert id find each other
//              with ballots; a lane's rank among them plus the wave's running
//              count for that expert plus the staged base is the assignment's
//              position p.  Equal ids therefore keep index order (stability),
//              and no position depends on the timing of atomics.
#include <mutex>

#include "moe_internal.h"
#include "topk_wave.h"

namespace moe {
namespace {

constexpr int kSeg = kDispatchSegment;  // assignments per wave
constexpr int kMaxE = MOE_MAX_GROUPS_INTERNAL;

__global__ __launch_bounds__(256) void dispatch_hist_kernel(const int32_t* __restrict__ ids, int P, int E, int U,
                                                            int32_t* __restrict__ cnt) {
  __shared__ int h[4][kMaxE];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int u = blockIdx.x * 4 + w;
  for (int e = lane; e < E; e += 64) h[w][e] = 0;
  __syncthreads();
  if (u < U) {
    int id[kSeg / 64];
#pragma unroll
    for (int r = 0; r < kSeg / 64; ++r) {
      const int a = u * kSeg + r * 64 + lane;
      id[r] = (a < P) ? ids[a] : -1;
    }
#pragma unroll
    for (int r = 0; r < kSeg / 64; ++r)
      if ((unsigned)id[r] < (unsigned)E) atomicAdd(&h[w][id[r]], 1);  // ids outside [0, E) are a caller error
  }
  __syncthreads();
  if (u < U)
    for (int e = lane; e < E; e += 64) cnt[(int64_t)e * U + u] = h[w][e];
}

// Top-k of the tokens of one dispatch segment, then that segment's expert
// histogram, for k dividing the segment size: workgroup u owns assignments
// [u*kSeg, (u+1)*kSeg), i.e. tokens [u*kSeg/k, (u+1)*kSeg/k).  Its 16 waves
// select those tokens' top-k with topk_row (the same ids and weights as the
// router's top-k kernel; the ids also go to LDS), then the workgroup counts
// the segment's ids in LDS and writes cnt[e][u] exactly as
// dispatch_hist_kernel does, which saves that launch.
template <int VPL>
__global__ __launch_bounds__(1024) void topk_hist_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                         int renorm, int32_t* __restrict__ ids,
                                                         float* __restrict__ weights, int U,
                                                         int32_t* __restrict__ cnt) {
  __shared__ int s_ids[kSeg];
  __shared__ int h[kMaxE];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int u = blockIdx.x;
  const int tpw = kSeg / k;  // tokens per segment
  const int t0 = u * tpw;
  for (int e = threadIdx.x; e < E; e += blockDim.x) h[e] = 0;
  for (int j = w; j < tpw; j += (int)(blockDim.x >> 6)) {
    const int t = t0 + j;
    if (t >= T) break;  // wave-uniform
    topk_row<VPL>(logits + (int64_t)t * E, E, k, renorm, ids + (int64_t)t * k, weights + (int64_t)t * k, nullptr,
                  lane, s_ids + j * k);
  }
  __syncthreads();
  const int a = u * kSeg + (int)threadIdx.x;
  if (threadIdx.x < kSeg && a < T * k) atomicAdd(&h[s_ids[threadIdx.x]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[(int64_t)e * U + u] = h[e];
}

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  return v;
}

// One wave per expert (4 per workgroup): exclusive scan of cnt[e][0..U) into
// base[e][u] (VPL consecutive segments per lane, all loads of a lane issued
// before any store) and the expert total into counts[e].  Workgroup 0 also
// zeroes `zero_ints` (the tile counters of the grouped GEMMs that follow).
template <int VPL>
__global__ __launch_bounds__(256) void dispatch_scan_kernel(const int32_t* __restrict__ cnt,
                                                            int32_t* __restrict__ base, int U, int E,
                                                            int32_t* __restrict__ counts, int* zero_ints,
                                                            int n_zero) {
  if (zero_ints != nullptr && blockIdx.x == 0 && (int)threadIdx.x < n_zero) zero_ints[threadIdx.x] = 0;
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= E) return;
  const int32_t* src = cnt + (int64_t)e * U;
  int32_t* dst = base + (int64_t)e * U;
  int carry = 0;
  for (int u0 = 0; u0 < U; u0 += 64 * VPL) {
    int v[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int u = u0 + lane * VPL + i;
      v[i] = (u < U) ? src[u] : 0;
    }
    int sum = 0;
#pragma unroll
    for (int i = 0; i < VPL; ++i) sum += v[i];
    const int incl = wave_incl_scan(sum, lane);
    int run = carry + incl - sum;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int u = u0 + lane * VPL + i;
      if (u < U) dst[u] = run;
      run += v[i];
    }
    carry += __shfl(incl, 63, 64);
  }
  if (lane == 0) counts[e] = carry;
}

__global__ __launch_bounds__(256) void dispatch_scatter_kernel(
    const int32_t* __restrict__ ids, const float* __restrict__ wts, int P, int k, int E, int U,
    const int32_t* __restrict__ base, const int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv, int32_t* __restrict__ packed_ids,
    float* __restrict__ packed_w) {
  __shared__ int pos0[4][kMaxE];  // offsets[e] + base[e][u], advanced as the wave places assignments
  __shared__ int off[kMaxE];      // expert offsets: exclusive scan of counts
  __shared__ int wsum[4];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int u = blockIdx.x * 4 + w;
  int id[kSeg / 64];
#pragma unroll
  for (int r = 0; r < kSeg / 64; ++r) {
    const int a = u * kSeg + r * 64 + lane;
    id[r] = (u < U && a < P) ? ids[a] : -1;
  }
  // every workgroup scans the E <= 512 expert totals itself (two per thread)
  {
    const int e0 = 2 * threadIdx.x, e1 = e0 + 1;
    const int c0 = (e0 < E) ? counts[e0] : 0;
    const int c1 = (e1 < E) ? counts[e1] : 0;
    const int incl = wave_incl_scan(c0 + c1, lane);
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    int b = 0;
    for (int q = 0; q < w; ++q) b += wsum[q];
    const int ex = b + incl - (c0 + c1);
    if (e0 < E) off[e0] = ex;
    if (e1 < E) off[e1] = ex + c0;
    if (blockIdx.x == 0) {
      if (e0 < E) offsets[e0] = ex;
      if (e1 < E) offsets[e1] = ex + c0;
      if (threadIdx.x == 0) offsets[E] = P;
    }
    __syncthreads();
  }
  if (u >= U) return;  // no workgroup barrier below: the waves are independent
  for (int e = lane; e < E; e += 64) pos0[w][e] = off[e] + base[(int64_t)e * U + u];
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes land before its reads below
  __builtin_amdgcn_wave_barrier();
  const uint64_t lt_mask = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
#pragma unroll
  for (int r = 0; r < kSeg / 64; ++r) {
    const int a = u * kSeg + r * 64 + lane;
    const bool valid = (unsigned)id[r] < (unsigned)E;
    const int my = valid ? id[r] : -1;
    uint64_t todo = __ballot(valid);
    uint64_t peers = 0;
    while (todo) {
      const int leader = __builtin_ctzll(todo);
      const int lid = __builtin_amdgcn_readlane(my, leader);
      const uint64_t m = __ballot(my == lid);
      if (my == lid) peers = m;
      todo &= ~m;
    }
    int pos = 0;
    if (valid) pos = pos0[w][my] + __popcll(peers & lt_mask);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
    if (valid && lane == __builtin_ctzll(peers)) pos0[w][my] += __popcll(peers);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
    if (valid) {
      perm[pos] = a;
      inv[a] = pos;
      packed_ids[pos] = a / k;
      if (packed_w != nullptr) packed_w[pos] = wts[a];
    }
  }
}

// Whole plan in one workgroup for P <= kDispatchSmallP (decode batches):
// the same three steps as above with the 16 waves as the segments and every
// intermediate in LDS.  Wave w owns the contiguous chunk [w*C, (w+1)*C) of
// the assignments, C = ceil(P / 16).  The per-wave counters take 16 * E ints
// of dynamic LDS (only what E needs, so that these launches fit next to a
// streaming GEMM's workgroup on a CU).
constexpr int kSmallWaves = 16;

__device__ __forceinline__ void dispatch_small_body(const int32_t* __restrict__ ids, const float* __restrict__ wts,
                                                    int P, int k, int E, int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
                                                    int32_t* __restrict__ inv, int32_t* __restrict__ packed_ids,
                                                    float* __restrict__ packed_w, int* zero_ints, int n_zero,
                                                    int* cnt) {
  // cnt[q * E + e]: per-wave counts, then per-wave running positions
  __shared__ int wsum[kSmallWaves];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  if (zero_ints != nullptr && tid < n_zero) zero_ints[tid] = 0;
  for (int i = tid; i < kSmallWaves * E; i += 1024) cnt[i] = 0;
  __syncthreads();
  const int C = (P + kSmallWaves - 1) / kSmallWaves;
  const int a0 = w * C;
  const int a1 = min(P, a0 + C);
  for (int a = a0 + lane; a < a1; a += 64) {
    const int e = ids[a];
    if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[w * E + e], 1);  // ids outside [0, E) are a caller error
  }
  __syncthreads();
  // per expert: running sum over the waves (cnt[w][e] <- count of waves < w)
  // and the total; then an exclusive scan of the totals over the experts
  int tot = 0;
  if (tid < E) {
#pragma unroll
    for (int q = 0; q < kSmallWaves; ++q) {
      const int c = cnt[q * E + tid];
      cnt[q * E + tid] = tot;
      tot += c;
    }
  }
  const int incl = wave_incl_scan(tot, lane);
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int base = 0;
  for (int q = 0; q < w; ++q) base += wsum[q];
  if (tid < E) {
    const int off = base + incl - tot;
    counts[tid] = tot;
    offsets[tid] = off;
#pragma unroll
    for (int q = 0; q < kSmallWaves; ++q) cnt[q * E + tid] += off;
  }
  if (tid == 0) offsets[E] = P;
  __syncthreads();
  // stable placement, 64 assignments at a time in index order
  const uint64_t lt_mask = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
  for (int r0 = a0; r0 < a1; r0 += 64) {
    const int a = r0 + lane;
    const bool valid = a < a1 && (unsigned)ids[a] < (unsigned)E;
    const int my = valid ? ids[a] : -1;
    uint64_t todo = __ballot(valid);
    uint64_t peers = 0;
    while (todo) {
      const int leader = __builtin_ctzll(todo);
      const int lid = __builtin_amdgcn_readlane(my, leader);
      const uint64_t m = __ballot(my == lid);
      if (my == lid) peers = m;
      todo &= ~m;
    }
    int pos = 0;
    if (valid) pos = cnt[w * E + my] + __popcll(peers & lt_mask);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
    if (valid && lane == __builtin_ctzll(peers)) cnt[w * E + my] += __popcll(peers);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
    if (valid) {
      perm[pos] = a;
      inv[a] = pos;
      packed_ids[pos] = a / k;
      if (packed_w != nullptr) packed_w[pos] = wts[a];
    }
  }
}


__global__ __launch_bounds__(1024) void dispatch_small_kernel(const int32_t* __restrict__ ids,
                                                              const float* __restrict__ wts, int P, int k, int E,
                                                              int32_t* __restrict__ counts,
                                                              int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ perm, int32_t* __restrict__ inv,
                                                              int32_t* __restrict__ packed_ids,
                                                              float* __restrict__ packed_w, int* zero_ints,
                                                              int n_zero) {
  extern __shared__ int dyn_lds[];  // [16 * E]
  dispatch_small_body(ids, wts, P, k, E, counts, offsets, perm, inv, packed_ids, packed_w, zero_ints, n_zero,
                      dyn_lds);
}

// Decode batches: top-k of every token (one wave per token, the same
// wave-level selection and weights as the router's top-k kernel, so the ids
// and weights are identical bit for bit), then, after a workgroup barrier,
// the whole plan as in dispatch_small_kernel, reading the ids from LDS.
// One launch instead of two on the latency-bound path from the logits to the
// expert GEMMs.
template <int VPL>
__global__ __launch_bounds__(1024) void topk_dispatch_small_kernel(const float* __restrict__ logits, int T, int E,
                                                                   int k, int renorm, int32_t* __restrict__ ids,
                                                                   float* __restrict__ weights,
                                                                   int32_t* __restrict__ counts,
                                                                   int32_t* __restrict__ offsets,
                                                                   int32_t* __restrict__ perm,
                                                                   int32_t* __restrict__ inv,
                                                                   int32_t* __restrict__ packed_ids, int* zero_ints,
                                                                   int n_zero) {
  // the ids also go to LDS, where the plan reads them (no global round trip)
  extern __shared__ int dyn_lds[];  // [16 * E] counters, then [T * k] ids
  int32_t* s_ids = dyn_lds + kSmallWaves * E;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  for (int t = w; t < T; t += kSmallWaves)
    topk_row<VPL>(logits + (int64_t)t * E, E, k, renorm, ids + (int64_t)t * k, weights + (int64_t)t * k, nullptr,
                  lane, s_ids + t * k);
  __syncthreads();
  dispatch_small_body(s_ids, nullptr, T * k, k, E, counts, offsets, perm, inv, packed_ids, nullptr, zero_ints,
                      n_zero, dyn_lds);
}

}  // namespace

hipError_t launch_topk_dispatch_small(const float* logits, int T, int E, int k, int renorm, int32_t* ids,
                                      float* weights, int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                                      int32_t* packed_ids, hipStream_t s, int* zero_ints, int n_zero) {
  if (T == 0) return hipSuccess;
  const size_t lds = (size_t)(kSmallWaves * E + T * k) * sizeof(int);
  profile_begin("topk_dispatch_small", s);
  if (E <= 64)
    hipLaunchKernelGGL(topk_dispatch_small_kernel<1>, dim3(1), dim3(1024), lds, s, logits, T, E, k, renorm, ids,
                       weights, counts, offsets, perm, inv, packed_ids, zero_ints, n_zero);
  else if (E <= 128)
    hipLaunchKernelGGL(topk_dispatch_small_kernel<2>, dim3(1), dim3(1024), lds, s, logits, T, E, k, renorm, ids,
                       weights, counts, offsets, perm, inv, packed_ids, zero_ints, n_zero);
  else if (E <= 256)
    hipLaunchKernelGGL(topk_dispatch_small_kernel<4>, dim3(1), dim3(1024), lds, s, logits, T, E, k, renorm, ids,
                       weights, counts, offsets, perm, inv, packed_ids, zero_ints, n_zero);
  else
    hipLaunchKernelGGL(topk_dispatch_small_kernel<8>, dim3(1), dim3(1024), lds, s, logits, T, E, k, renorm, ids,
                       weights, counts, offsets, perm, inv, packed_ids, zero_ints, n_zero);
  profile_end(s);
  return hipGetLastError();
}

// Scratch of the dispatch plan for callers that cannot allocate: a fixed
// device array of kDispatchStaticScratchBytes, one copy per GPU, alive until
// the process ends.  Host code never passes the array's name to a kernel (on
// the host it is only a stand-in for the symbol); it passes the device address
// that hipGetSymbolAddress returns, looked up once per device with that device
// current.  Every call on a GPU shares that GPU's copy: calls that overlap in
// time on one GPU race on it.  The plan writes every (expert, segment) count
// and base it later reads, so nothing in it needs clearing between calls.
__device__ __align__(256) unsigned char scratch[kDispatchStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t dispatch_static_scratch(void** out) {
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

size_t dispatch_scratch_bytes(int64_t P, int64_t E) {
  const int64_t U = (P + kSeg - 1) / kSeg;
  return (size_t)(2 * U * E * (int64_t)sizeof(int32_t));  // counts, then bases
}

bool dispatch_takes_hist(int T, int k) {
  const int64_t P = (int64_t)T * k;
  return P > kDispatchSmallP && kSeg % k == 0;
}

hipError_t launch_topk_hist(const float* logits, int T, int E, int k, int renorm, int32_t* ids, float* weights,
                            void* scratch, hipStream_t s) {
  if (!dispatch_takes_hist(T, k)) return hipErrorInvalidValue;
  const int P = T * k;
  const int U = (P + kSeg - 1) / kSeg;
  int32_t* cnt = static_cast<int32_t*>(scratch);
  profile_begin("router_topk_hist", s);
#define MOE_TOPK_HIST(VPL) \
  hipLaunchKernelGGL(topk_hist_kernel<VPL>, dim3(U), dim3(1024), 0, s, logits, T, E, k, renorm, ids, weights, U, cnt)
  if (E <= 64) MOE_TOPK_HIST(1);
  else if (E <= 128) MOE_TOPK_HIST(2);
  else if (E <= 256) MOE_TOPK_HIST(4);
  else MOE_TOPK_HIST(8);
#undef MOE_TOPK_HIST
  profile_end(s);
  return hipGetLastError();
}

hipError_t launch_dispatch(const int32_t* ids, const float* w, int T, int k, int E, int32_t* counts,
                           int32_t* offsets, int32_t* perm, int32_t* inv, int32_t* packed_ids, float* packed_w,
                           void* scratch, hipStream_t s, int* zero_ints, int n_zero, bool have_hist) {
  const int P = T * k;
  if (P == 0) return hipSuccess;
  if (have_hist && !dispatch_takes_hist(T, k)) return hipErrorInvalidValue;
  if (P <= kDispatchSmallP) {
    profile_begin("dispatch_small", s);
    hipLaunchKernelGGL(dispatch_small_kernel, dim3(1), dim3(1024), (size_t)kSmallWaves * E * sizeof(int), s, ids, w,
                       P, k, E, counts, offsets, perm, inv, packed_ids, packed_w, zero_ints, n_zero);
    profile_end(s);
    return hipGetLastError();
  }
  const int U = (P + kSeg - 1) / kSeg;
  int32_t* cnt = reinterpret_cast<int32_t*>(scratch);
  int32_t* base = cnt + (int64_t)U * E;
  const unsigned blocks = (unsigned)((U + 3) / 4);
  if (!have_hist) {
    profile_begin("dispatch_hist", s);
    hipLaunchKernelGGL(dispatch_hist_kernel, dim3(blocks), dim3(256), 0, s, ids, P, E, U, cnt);
    profile_end(s);
  }
  profile_begin("dispatch_scan", s);
  const dim3 sgrid((unsigned)((E + 3) / 4));
  if (U <= 64)
    hipLaunchKernelGGL(dispatch_scan_kernel<1>, sgrid, dim3(256), 0, s, cnt, base, U, E, counts, zero_ints, n_zero);
  else if (U <= 256)
    hipLaunchKernelGGL(dispatch_scan_kernel<4>, sgrid, dim3(256), 0, s, cnt, base, U, E, counts, zero_ints, n_zero);
  else
    hipLaunchKernelGGL(dispatch_scan_kernel<16>, sgrid, dim3(256), 0, s, cnt, base, U, E, counts, zero_ints,
                       n_zero);
  profile_end(s);
  profile_begin("dispatch_scatter", s);
  hipLaunchKernelGGL(dispatch_scatter_kernel, dim3(blocks), dim3(256), 0, s, ids, w, P, k, E, U, base, counts,
                     offsets, perm, inv, packed_ids, packed_w);
  profile_end(s);
  return hipGetLastError();
}

}  // namespace moe
