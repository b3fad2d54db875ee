// Grouped bf16 GEMM on gfx950 matrix cores (v_mfma_f32_16x16x32_bf16), fp32
// accumulate, with three epilogues:
//   EPI_SWIGLU  gate/up projection of the experts: each tile multiplies the same
//               gathered rows by matching gate and up weight rows of the fused
//               w13 buffer (gate rows first, then up rows, as FusedMoEModel in
//               the modelexpress refit test lays them out) and writes
//               h = silu(g) * u as bf16.               [DWDP README "Executor Module"]
//   EPI_F32     down projection y = W2[e] h, fp32 out.  [DWDP README "Executor Module"]
//   EPI_ROUTER  router logits x Wr^T (+ bias) with an optional extra weight row
//               (the shared expert's gate vector).      [DWDP README "Router Module"]
//
// Scheduling: the packed rows of each group (expert) form expert-major execution
// ranges [offsets[g], offsets[g+1]) ([DWDP README "Scheduler Module"]).  Every
// range is cut into BM-row m-tiles; m-tiles x n-blocks form a linear tile list,
// expert-major.  The grid is persistent; each workgroup derives the tile list
// itself from `offsets` (a block-wide scan in LDS), so no host sync and no
// separate schedule kernel is needed.  Tiles are handed out XCD-aware: MI355X
// places workgroup b on XCD b % 8, so XCD x owns the contiguous tile range
// [x*per, (x+1)*per) and its 4 MB L2 sees all n-blocks of an m-tile and all
// m-tiles of an expert close together in time.
//
// Tile: BM rows x (4 waves x 64 B-rows); BK = 64.  The A tile (gathered
// activation rows, shared by the 4 waves) is staged through LDS, double
// buffered, with a 16-byte-chunk XOR swizzle (chunk c of row r sits at c ^ (r & 7))
// so that both the row-wise stores and the fragment loads are bank-conflict
// free.  B rows belong to exactly one wave, so each wave loads its B fragments
// straight from global memory into registers, one stage ahead.
//
// Rows past the end of a group are computed on a clamped (valid) row and never
// stored; 16-row sub-tiles that lie wholly past the end skip their MFMAs, so a
// ragged last tile costs MFMA time in proportion to its real rows.
#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int BK = 64;
constexpr int kMaxGroups = MOE_MAX_GROUPS_INTERNAL;
constexpr int kXcds = 8;

__device__ __forceinline__ u32x4_t ldg16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <int BM, int EPI>
__global__ __launch_bounds__(kThreads) void grouped_gemm_bf16_kernel(GemmArgs p) {
  constexpr int MSUB = BM / 16;
  constexpr int A_SLOTS = (BM * 8 + kThreads - 1) / kThreads;  // 16-byte A chunks per thread
  constexpr int BN_OUT = (EPI == EPI_SWIGLU) ? 128 : 256;      // output columns per tile

  __shared__ u32x4_t sA[2][BM * 8];
  __shared__ int s_off[kMaxGroups + 1];
  __shared__ int s_tb[kMaxGroups + 1];
  __shared__ int s_wsum[kThreads / 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = p.G;

  // ---- tile schedule: m-tiles per group, exclusive scan -----------------
  if (p.offsets) {
    for (int g = tid; g <= G; g += kThreads) s_off[g] = p.offsets[g];
  } else if (tid == 0) {
    s_off[0] = 0;
    s_off[1] = p.M;
  }
  __syncthreads();
  {
    const int g0 = 2 * tid, g1 = 2 * tid + 1;
    const int t0 = (g0 < G) ? (s_off[g0 + 1] - s_off[g0] + BM - 1) / BM : 0;
    const int t1 = (g1 < G) ? (s_off[g1 + 1] - s_off[g1] + BM - 1) / BM : 0;
    const int sum = t0 + t1;
    int incl = sum;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d, 64);
      if (lane >= d) incl += v;
    }
    if (lane == 63) s_wsum[wave] = incl;
    __syncthreads();
    int wbase = 0;
    for (int w = 0; w < wave; ++w) wbase += s_wsum[w];
    const int excl = wbase + incl - sum;
    if (g0 < G) s_tb[g0] = excl;
    if (g1 < G) s_tb[g1] = excl + t0;
    if (tid == 0) {
      int tot = 0;
      for (int w = 0; w < kThreads / 64; ++w) tot += s_wsum[w];
      s_tb[G] = tot;
    }
  }
  __syncthreads();

  const int total_m = s_tb[G];
  const int nblk = (p.N + BN_OUT - 1) / BN_OUT;
  const int total = total_m * nblk;
  const int xcd = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;
  const int nslots = gridDim.x / kXcds;
  const int per = (total + kXcds - 1) / kXcds;
  const int t_begin = xcd * per;
  const int t_end = min(total, t_begin + per);
  const int KT = p.K / BK;

  for (int t = t_begin + slot; t < t_end; t += nslots) {
    const int mt = t / nblk;
    const int nb = t - mt * nblk;
    int lo = 0, hi = G;  // s_tb[lo] <= mt < s_tb[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_tb[mid] <= mt) lo = mid; else hi = mid;
    }
    const int g = __builtin_amdgcn_readfirstlane(lo);
    const int m0 = __builtin_amdgcn_readfirstlane(s_off[g] + (mt - s_tb[g]) * BM);
    const int rows = __builtin_amdgcn_readfirstlane(min(BM, s_off[g + 1] - m0));
    const int msub_live = (rows + 15) >> 4;
    const int n0 = nb * BN_OUT;
    const uint16_t* Bg = p.B + (int64_t)g * p.b_group_stride;

    // A source rows (gathered), one 16-byte chunk per slot
    const int a_chunk = tid & 7;
    const uint16_t* a_src[A_SLOTS];
    int a_row[A_SLOTS];
#pragma unroll
    for (int i = 0; i < A_SLOTS; ++i) {
      const int r = (tid >> 3) + 32 * i;
      a_row[i] = r;
      const int rr = min(r, rows - 1);
      const int64_t grow = p.gather ? (int64_t)p.gather[m0 + rr] : (int64_t)(m0 + rr);
      a_src[i] = p.A + grow * p.K + a_chunk * 8;
    }

    // B fragment rows of this wave: 4 sub-tiles of 16 rows
    const uint16_t* b_src[4];
    bool sub_live[4];
    int wave_col0;
    if (EPI == EPI_SWIGLU) wave_col0 = n0 + 32 * wave;
    else wave_col0 = n0 + 64 * wave;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int col0, brow;
      if (EPI == EPI_SWIGLU) {
        col0 = wave_col0 + 16 * (j & 1);
        const int c = min(col0 + (lane & 15), p.N - 1);
        brow = (j < 2) ? c : p.up_row0 + c;
      } else {
        col0 = wave_col0 + 16 * j;
        brow = min(col0 + (lane & 15), p.N - 1);
      }
      sub_live[j] = col0 < p.N;
      const uint16_t* rp = Bg + (int64_t)brow * p.K;
      if (EPI == EPI_ROUTER && p.b_extra != nullptr && brow == p.N - 1) rp = p.b_extra;
      b_src[j] = rp + (lane >> 4) * 8;
    }
    const bool wave_live = wave_col0 < p.N;

    f32x4_t acc[MSUB][4];
#pragma unroll
    for (int i = 0; i < MSUB; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    u32x4_t a_reg[A_SLOTS];
    u32x4_t b_cur[4][2], b_nxt[4][2];

#pragma unroll
    for (int i = 0; i < A_SLOTS; ++i)
      if (a_row[i] < BM) a_reg[i] = ldg16(a_src[i]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) b_cur[j][kk] = ldg16(b_src[j] + kk * 32);
#pragma unroll
    for (int i = 0; i < A_SLOTS; ++i)
      if (a_row[i] < BM) sA[0][a_row[i] * 8 + (a_chunk ^ (a_row[i] & 7))] = a_reg[i];
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
      const int buf = kt & 1;
      const bool more = kt + 1 < KT;
      if (more) {
        const int ko = (kt + 1) * BK;
#pragma unroll
        for (int i = 0; i < A_SLOTS; ++i)
          if (a_row[i] < BM) a_reg[i] = ldg16(a_src[i] + ko);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) b_nxt[j][kk] = ldg16(b_src[j] + ko + kk * 32);
      }
      if (wave_live) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
          for (int i = 0; i < MSUB; ++i) {
            if (i < msub_live) {
              const int row = 16 * i + (lane & 15);
              const int chunk = kk * 4 + (lane >> 4);
              const bf16x8_t a = __builtin_bit_cast(bf16x8_t, sA[buf][row * 8 + (chunk ^ (row & 7))]);
#pragma unroll
              for (int j = 0; j < 4; ++j)
                if (sub_live[j])
                  acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                      a, __builtin_bit_cast(bf16x8_t, b_cur[j][kk]), acc[i][j], 0, 0, 0);
            }
          }
        }
      }
      if (more) {
#pragma unroll
        for (int i = 0; i < A_SLOTS; ++i)
          if (a_row[i] < BM) sA[buf ^ 1][a_row[i] * 8 + (a_chunk ^ (a_row[i] & 7))] = a_reg[i];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) b_cur[j][kk] = b_nxt[j][kk];
      }
      __syncthreads();
    }

    // ---- epilogue.  C fragment: lane holds column (lane & 15), rows 4*(lane>>4)+r
    if (wave_live) {
#pragma unroll
      for (int i = 0; i < MSUB; ++i) {
        if (i >= msub_live) continue;
        if (EPI == EPI_SWIGLU) {
          uint16_t* out = reinterpret_cast<uint16_t*>(p.out);
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int col = wave_col0 + 16 * jj + (lane & 15);
            if (col >= p.N) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int row = 16 * i + 4 * (lane >> 4) + r;
              if (row < rows) {
                const float gv = acc[i][jj][r];
                const float uv = acc[i][jj + 2][r];
                const float h = gv / (1.0f + __expf(-gv)) * uv;
                out[(int64_t)(m0 + row) * p.ldo + col] = f32_to_bf16_rne(h);
              }
            }
          }
        } else {
          float* out = reinterpret_cast<float*>(p.out);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int col = wave_col0 + 16 * j + (lane & 15);
            if (col >= p.N) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int row = 16 * i + 4 * (lane >> 4) + r;
              if (row < rows) {
                float v = acc[i][j][r];
                if (EPI == EPI_ROUTER) {
                  if (p.b_extra != nullptr && col == p.N - 1) {
                    p.extra_out[m0 + row] = v;
                    continue;
                  }
                  if (p.bias) v += p.bias[col];
                }
                out[(int64_t)(m0 + row) * p.ldo + col] = v;
              }
            }
          }
        }
      }
    }
  }
}

// Resident workgroups per CU for one instantiation (the persistent grid must
// fit in one wave of residency, or the static tile split would serialise).
template <int BM, int EPI>
int resident_blocks_per_cu() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, grouped_gemm_bf16_kernel<BM, EPI>, kThreads, 0) !=
            hipSuccess || n < 1)
      n = 1;
    cached[dev] = n;
  }
  return cached[dev];
}

template <int BM, int EPI>
hipError_t launch_bm(const GemmArgs& a, hipStream_t s, const char* name, int max_occupancy) {
  int occupancy = resident_blocks_per_cu<BM, EPI>();
  if (occupancy > max_occupancy) occupancy = max_occupancy;
  constexpr int BN_OUT = (EPI == EPI_SWIGLU) ? 128 : 256;
  const int64_t nblk = (a.N + BN_OUT - 1) / BN_OUT;
  int64_t ub_m = (a.M + BM - 1) / BM;
  if (a.offsets) ub_m += (a.G < a.M ? a.G : a.M);
  const int64_t ub = ub_m * nblk;
  int64_t grid = (int64_t)device_cu_count() * occupancy;
  if (ub < grid) grid = ub;
  grid = ((grid + kXcds - 1) / kXcds) * kXcds;
  if (grid < kXcds) grid = kXcds;
  profile_begin(name, s);
  hipLaunchKernelGGL((grouped_gemm_bf16_kernel<BM, EPI>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  profile_end(s);
  return hipGetLastError();
}

template <int EPI>
hipError_t launch_epi(const GemmArgs& a, hipStream_t s, const char* name) {
  // rows per group on average decides the m-tile height
  const int64_t groups = a.offsets ? (a.G < a.M ? a.G : a.M) : 1;
  const int64_t avg = groups > 0 ? (a.M + groups - 1) / groups : a.M;
  if (avg <= 16) return launch_bm<16, EPI>(a, s, name, 4);
  if (avg <= 32) return launch_bm<32, EPI>(a, s, name, 4);
  if (avg <= 64) return launch_bm<64, EPI>(a, s, name, 2);
  return launch_bm<128, EPI>(a, s, name, 1);
}

}  // namespace

hipError_t launch_grouped_gemm_bf16(const GemmArgs& a, GemmEpilogue epi, hipStream_t s, const char* name) {
  if (a.M <= 0) return hipSuccess;
  switch (epi) {
    case EPI_SWIGLU: return launch_epi<EPI_SWIGLU>(a, s, name);
    case EPI_F32: return launch_epi<EPI_F32>(a, s, name);
    case EPI_ROUTER: return launch_bm<32, EPI_ROUTER>(a, s, name, 4);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
