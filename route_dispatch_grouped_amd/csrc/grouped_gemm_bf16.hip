// Grouped bf16 GEMM on gfx950 matrix cores (v_mfma_f32_16x16x32_bf16), fp32
// accumulate, with three epilogues:
//   EPI_SWIGLU  gate/up projection of the experts: each tile multiplies the same
//               gathered rows by matching gate and up weight rows of the fused
//               w13 buffer (gate rows first, then up rows, as FusedMoEModel in
//               the modelexpress refit test lays them out) and writes
//               h = silu(g) * u as bf16.               [DWDP README "Executor Module"]
//   EPI_F32     down projection y = W2[e] h, fp32 out.  [DWDP README "Executor Module"]
//   EPI_BF16    the same, y rounded once to bf16 (RNE).
//   EPI_F16S    the same, y as fp16 with a power-of-two scale per (row, 64
//               columns) (256-row kernels only).
//   EPI_ROUTER  router logits x Wr^T (+ bias).          [DWDP README "Router Module"]
//
// Scheduling: the packed rows of each group (expert) form expert-major execution
// ranges [offsets[g], offsets[g+1]) ([DWDP README "Scheduler Module"]).  Every
// range is cut into BM-row m-tiles; m-tiles x n-blocks form a linear tile list,
// expert-major, n-block fastest.  The grid is persistent; each workgroup derives
// the tile list itself from `offsets` (a block-wide scan in LDS), so no host
// sync and no separate schedule kernel is needed.  Tiles are handed out
// XCD-aware: MI355X places workgroup b on XCD b % 8, so XCD x owns the
// contiguous tile range [x*per, (x+1)*per) and its 4 MB L2 serves all n-blocks
// of an m-tile and all m-tiles of an expert close together in time.
//
// Kernels, by rows per group on average: up to 16 the streaming kernel
// (decode batches, a pure weight stream), 17-95 the BM-row kernel described
// next, from 96 the 256-row tiles of the 8-wave pipelined kernel (or of the
// plain 256-row kernel for K loops the pipelined one does not take); each is
// described at its definition.
//
// BM-row kernel.  Tile: BM rows x 256 weight rows (EPI_SWIGLU: 128 gate + the matching 128 up
// rows; otherwise 256 output columns), BK = 64 (128 bytes per row); K needs
// only to be a multiple of 8 (16-byte chunks): chunks past K read zeros.  Both
// operands stream through an NS-stage LDS ring filled by direct global->LDS
// DMA (buffer_load_dwordx4 ... lds): no staging registers, NS-1 K-steps in
// flight.  Each stage is its own __shared__ object, so the compiler tracks the
// DMA of each stage separately and waits only for the stage being read.  One
// workgroup barrier per K-step: each wave first waits for its own DMA of the
// stage, the barrier then publishes the whole stage and also proves that every
// wave has finished reading the buffer the next DMA will overwrite.
//
// LDS layout: row r of a tile holds eight 16-byte chunks; chunk c sits at
// position c ^ (r & 7), so the row-wise DMA writes and the fragment reads (16
// rows, one chunk column) are both bank-conflict free.  The DMA writes lane l
// of an instruction to slot base + l; each lane therefore fetches the global
// chunk that belongs at its slot.
//
// Wave w computes all BM rows against its 64 weight rows (EPI_SWIGLU: gate
// rows 32w..32w+31 and the same up rows, so gate and up of one h column meet
// in the same lane of the accumulators).  Rows past the end of a group read a
// clamped (valid) row and are never stored; 16-row sub-tiles wholly past the
// end skip their MFMAs (a straight-line K loop per live sub-tile count).
#include <atomic>
#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int BK = 64;
constexpr int kBRows = 256;
constexpr int kMaxGroups = MOE_MAX_GROUPS_INTERNAL;
constexpr int kXcds = 8;
constexpr int kBufferWord3 = 0x00020000;  // raw buffer resource, 32-bit data

// BR weight rows per tile: 256 (EPI_SWIGLU: 128 gate + 128 up), or 128 for
// narrow outputs (the router of up to 128 experts), which halves the stage
// and leaves LDS for a deeper ring.
template <int BM, int BR = kBRows>
struct Tile {
  static constexpr int MSUB = BM / 16;
  static constexpr int NJ = BR / 64;                       // 16-column weight sub-tiles per wave
  static constexpr int STAGE_BYTES = (BM + BR) * BK * 2;
  static constexpr int NS = (BR == kBRows) ? ((BM >= 64) ? 3 : 4)   // LDS ring depth
                                           : ((144 * 1024 / STAGE_BYTES) < 8 ? (144 * 1024 / STAGE_BYTES) : 8);
  static constexpr int SLOTS = (BM + BR) * 8;              // 16-byte slots per stage
  static constexpr int A_INSTR = BM / 8;                   // wave-instructions (64 slots each)
  static constexpr int B_INSTR = BR / 8;
  static constexpr int A_MAX = (A_INSTR + 3) / 4;          // per wave
  static constexpr int A_MIN = A_INSTR / 4;
  static constexpr int B_PER = B_INSTR / 4;                // per wave
  // outstanding DMA instructions allowed while waiting for the oldest stage
  static constexpr int VM_WAIT = (NS - 2) * (A_MIN + B_PER);
  static_assert(NS >= 3 && VM_WAIT < 64, "ring depth");
};

// two values rounded to bf16 (nearest even), the first in the low half (the
// lower address): one v_cvt_pk_bf16_f32, which gives the bits of the integer
// rounding u + 0x7FFF + ((u >> 16) & 1) for every finite input
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) { return static_cast<uint16_t>(pack_bf16x2(f, 0.f)); }

// Exponent k that brings a segment whose largest magnitude is m into
// [2^14, 2^15) (0 for an all-zero segment; below the normal range the
// smallest normal's k is used, and Inf/NaN keep their value).
__device__ __forceinline__ int f16s_exponent(float m) {
  const uint32_t eb = (__float_as_uint(m) >> 23) & 0xFFu;
  if (m == 0.f) return 0;
  const int e = (eb == 0) ? -126 : (int)eb - 127;
  return 14 - e;
}

// two values rounded to fp16 (nearest even; one v_cvt_pk_f16_f32), the first
// in the low half
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}

// silu(g) * u = g * u / (1 + e^-g), with the hardware reciprocal (about 1 ulp)
// instead of an IEEE division: the result is rounded to bf16 right after.
// e^-g overflowing to +inf gives exactly 0, the limit of silu at -inf.
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * u * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

// s_waitcnt immediates (gfx9 encoding: vmcnt bits [3:0] and [15:14], expcnt
// [6:4], lgkmcnt [11:8]); issued through the builtin so that the compiler's
// own wait tracking sees them.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// All of this wave's LDS reads are complete, then a workgroup barrier.  The
// barrier itself is an asm statement with a memory clobber so that no LDS
// access moves across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt((0xF) | (0x3 << 14) | (0x7 << 4));  // lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
}

// Per-tile DMA addressing: byte offsets of every slot this lane fetches.
// a_cb / b_cb: byte offset of the lane's chunk inside a stage row; with
// ktail (K not a multiple of BK) chunks at or past the end of a row are
// fetched through an offset past the buffer (zeros).
template <int BM, int BR>
struct DmaPlan {
  uint32_t a_off[Tile<BM, BR>::A_MAX];
  uint32_t b_off[Tile<BM, BR>::B_PER];
  uint32_t a_cb[Tile<BM, BR>::A_MAX];
  uint32_t b_cb[Tile<BM, BR>::B_PER];
  uint32_t row_bytes;
  bool ktail;
};

// Byte offset of the 16-byte chunk at byte cb of a stage row of row r, for an
// operand whose element (r, k) sits at row_pitch * r + blk_pitch * (k / 32) +
// 2 * (k % 32) (row-major: row_pitch = 2K, blk_pitch = 64).  The stage's own
// K offset goes separately into the DMA's scalar offset (stage_off).
__device__ __forceinline__ uint32_t chunk_off(int r, uint32_t cb, uint32_t row_pitch, uint32_t blk_pitch) {
  return (uint32_t)r * row_pitch + (cb >> 6) * blk_pitch + (cb & 63u);
}
// Scalar offset of the stage starting at logical byte kbytes of a row (a
// multiple of 64).
__device__ __forceinline__ int stage_off(int kbytes, uint32_t blk_pitch) { return (kbytes >> 6) * (int)blk_pitch; }

// Raw buffer resource (gfx9 V#): 48-bit base, stride 0, size in bytes; loads
// past `bytes` return zero instead of faulting.
__device__ __forceinline__ u32x4_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4_t{(uint32_t)a, (uint32_t)(a >> 32) & 0xFFFFu, bytes, (uint32_t)kBufferWord3};
}

// One 16-byte-per-lane DMA from global (buffer + voff + soff) to LDS: lane l
// lands at lds_dst + 16*l.  Issued as inline asm so that the compiler neither
// tracks nor waits for it: the K loop waits with explicit vmcnt counts.  The
// instruction has no register result, so nothing can be overwritten in flight.
__device__ __forceinline__ void dma16(const u32x4_t* lds_dst, u32x4_t rsrc, uint32_t voff, int soff) {
  const uint32_t m0v =
      (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const void*)lds_dst);
  uint32_t saved;  // m0 is restored, so the compiler's own use of it is unaffected
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, %4 offen lds\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(m0v), "v"(voff), "s"(rsrc), "s"(soff)
      : "memory");
}

// One 4-byte-per-lane DMA from global to LDS: lane l lands at lds_dst + 4*l.
__device__ __forceinline__ void dma4(const int* lds_dst, u32x4_t rsrc, uint32_t voff, int soff) {
  const uint32_t m0v = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const void*)lds_dst);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
      "buffer_load_dword %2, %3, %4 offen lds\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(m0v), "v"(voff), "s"(rsrc), "s"(soff)
      : "memory");
}

template <int BM, int BR>
__device__ __forceinline__ void issue_stage(u32x4_t* buf, const DmaPlan<BM, BR>& d, u32x4_t ra, u32x4_t rb,
                                            int wave, int kbytes, uint32_t b_blk) {
  using C = Tile<BM, BR>;
#pragma unroll
  for (int qi = 0; qi < C::A_MAX; ++qi) {
    const int q = qi * 4 + wave;
    uint32_t v = d.a_off[qi];
    if (d.ktail && d.a_cb[qi] + (uint32_t)kbytes >= d.row_bytes) v = 0x80000000u;
    if (qi < C::A_MIN || q < C::A_INSTR) dma16(buf + q * 64, ra, v, kbytes);
  }
#pragma unroll
  for (int qi = 0; qi < C::B_PER; ++qi) {
    const int q = qi * 4 + wave;
    uint32_t v = d.b_off[qi];
    if (d.ktail && d.b_cb[qi] + (uint32_t)kbytes >= d.row_bytes) v = 0x80000000u;
    dma16(buf + BM * 8 + q * 64, rb, v, stage_off(kbytes, b_blk));
  }
}

// One K-step from one stage: LIVE row sub-tiles x NJ weight sub-tiles x 2 k32.
template <int BM, int NJ, int LIVE>
__device__ __forceinline__ void mma_stage(f32x4_t (&acc)[BM / 16][NJ], const u32x4_t* __restrict__ buf,
                                          const int (&brow)[NJ], int lane) {
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int sw = (kk * 4 + (lane >> 4)) ^ (lane & 7);
    bf16x8_t b[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) b[j] = __builtin_bit_cast(bf16x8_t, buf[BM * 8 + (brow[j] + (lane & 15)) * 8 + sw]);
#pragma unroll
    for (int i = 0; i < LIVE; ++i) {
      const bf16x8_t a = __builtin_bit_cast(bf16x8_t, buf[(16 * i + (lane & 15)) * 8 + sw]);
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[j], acc[i][j], 0, 0, 0);
    }
  }
}

// K loop over an NS-stage ring (stage s at ring + s * SLOTS); the loop body is
// unrolled NS times so that every stage buffer has a static role.
template <int BM, int BR, int NJ, int LIVE>
__device__ __forceinline__ void kloop(f32x4_t (&acc)[BM / 16][NJ], u32x4_t* ring, const DmaPlan<BM, BR>& d,
                                      u32x4_t ra, u32x4_t rb, int wave, int lane, int KT, int kbase, bool wave_live,
                                      const int (&brow)[NJ], uint32_t b_blk) {
  using C = Tile<BM, BR>;
  static_assert(NJ == C::NJ, "weight sub-tiles per wave");
  constexpr int NS = C::NS;
  // prologue: stages 0 .. NS-2 in flight (kbase: byte offset of this tile's K range)
#pragma unroll
  for (int st = 0; st < NS - 1; ++st)
    if (st < KT) issue_stage<BM, BR>(ring + st * C::SLOTS, d, ra, rb, wave, kbase + st * BK * 2, b_blk);
  for (int kt0 = 0; kt0 < KT; kt0 += NS) {
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int kt = kt0 + u;
      if (kt >= KT) break;
      // wait for this wave's DMA of stage kt (later stages may stay in flight)
      if (kt + NS - 2 < KT) wait_vmcnt<C::VM_WAIT>();
      else wait_vmcnt<0>();
      lds_barrier();
      if (kt + NS - 1 < KT)
        issue_stage<BM, BR>(ring + ((u + NS - 1) % NS) * C::SLOTS, d, ra, rb, wave, kbase + (kt + NS - 1) * BK * 2,
                            b_blk);
      if (wave_live) mma_stage<BM, NJ, LIVE>(acc, ring + u * C::SLOTS, brow, lane);
    }
  }
}

// Tile schedule shared by every workgroup: s_off <- offsets (E+1), s_tb[g] <-
// first m-tile of group g (exclusive scan of ceil(rows/BM)), s_tb[G] = total.
template <int BM, int NT = kThreads>
__device__ __forceinline__ void build_schedule(const GemmArgs& p, int* s_off, int* s_tb, int* s_wsum, int tid,
                                               int lane, int wave) {
  const int G = p.G;
  if (p.offsets) {
    for (int g = tid; g <= G; g += NT) s_off[g] = p.offsets[g];
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
    for (int dd = 1; dd < 64; dd <<= 1) {
      const int v = __shfl_up(incl, dd, 64);
      if (lane >= dd) incl += v;
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
      for (int w = 0; w < NT / 64; ++w) tot += s_wsum[w];
      s_tb[G] = tot;
    }
  }
  __syncthreads();

}

// Tile t -> (group g, first packed row m0, rows in the tile, n-block nb).
// The tiles of group g occupy [s_tb[g]*nblk, s_tb[g+1]*nblk) of the tile list.
// Inside a group they are numbered in chunks of kChunkM m-tiles, and inside a
// chunk the m-tile index runs fastest: the tiles that read one weight block
// are handed out back to back, and the tiles that read one block of activation
// rows are at most kChunkM apart, close enough in time for the XCD's L2 to
// serve both reuses.
constexpr int kChunkM = 4;

struct TileCoord {
  int g, m0, rows, nb;
};

template <int BM>
__device__ __forceinline__ TileCoord tile_coord(int t, int nblk, int G, const int* s_tb, const int* s_off) {
  const int mt = t / nblk;
  int lo = 0, hi = G;  // s_tb[lo] <= mt < s_tb[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_tb[mid] <= mt) lo = mid; else hi = mid;
  }
  const int mbase = s_tb[lo];
  const int mcount = s_tb[lo + 1] - mbase;
  const int local = t - mbase * nblk;
  const int c = local / (kChunkM * nblk);
  const int rem = local - c * kChunkM * nblk;
  const int cs = min(kChunkM, mcount - c * kChunkM);
  const int nb = rem / cs;
  const int mi = c * kChunkM + (rem - nb * cs);
  TileCoord tc;
  tc.g = __builtin_amdgcn_readfirstlane(lo);
  tc.m0 = __builtin_amdgcn_readfirstlane(s_off[lo] + mi * BM);
  tc.rows = __builtin_amdgcn_readfirstlane(min(BM, s_off[lo + 1] - tc.m0));
  tc.nb = __builtin_amdgcn_readfirstlane(nb);
  return tc;
}

template <int BM, int EPI, int BR>
__global__ __launch_bounds__(kThreads) void grouped_gemm_bf16_kernel(GemmArgs p) {
  using C = Tile<BM, BR>;
  constexpr int MSUB = C::MSUB;
  constexpr int NJ = C::NJ;
  static_assert(EPI != EPI_SWIGLU || BR == kBRows, "the SwiGLU tile pairs 128 gate with 128 up rows");
  constexpr int BN_OUT = (EPI == EPI_SWIGLU) ? 128 : BR;  // output columns per tile

  __shared__ u32x4_t ring[C::NS * C::SLOTS];
  __shared__ int s_off[kMaxGroups + 1];
  __shared__ int s_tb[kMaxGroups + 1];
  __shared__ int s_wsum[kThreads / 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = p.G;

  build_schedule<BM>(p, s_off, s_tb, s_wsum, tid, lane, wave);

  const int total_m = s_tb[G];
  const int nblk = (p.N + BN_OUT - 1) / BN_OUT;
  // split-K: the K range is cut into p.ksplit chunks of KTc stages; tile t
  // covers (m-tile, n-block) t % total_mn and chunk t / total_mn
  const int ksplit = (EPI != EPI_ROUTER && p.partial != nullptr && p.ksplit > 1) ? p.ksplit : 1;
  const int total_mn = total_m * nblk;
  const int total = total_mn * ksplit;
  const int xcd = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;
  const int nslots = gridDim.x / kXcds;
  const int per = (total + kXcds - 1) / kXcds;
  const int t_begin = xcd * per;
  const int t_end = min(total, t_begin + per);
  const int KT_all = (p.K + BK - 1) / BK;  // the last stage may be partly past K
  const int KTc = (KT_all + ksplit - 1) / ksplit;
  const uint32_t row_bytes = (uint32_t)p.K * 2u;

  // weight rows of this wave inside the BR-row B tile (sub-tile bases)
  int brow[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j)
    brow[j] = (EPI == EPI_SWIGLU) ? ((j < 2) ? 32 * wave + 16 * j : 128 + 32 * wave + 16 * (j - 2))
                                  : (BR / 4) * wave + 16 * j;

  for (int t = t_begin + slot; t < t_end; t += nslots) {
    const int kc = __builtin_amdgcn_readfirstlane(t / total_mn);
    const TileCoord tc = tile_coord<BM>(t - kc * total_mn, nblk, G, s_tb, s_off);
    const int g = tc.g, m0 = tc.m0, rows = tc.rows, nb = tc.nb;
    const int msub_live = (rows + 15) >> 4;
    const int KT = min(KTc, KT_all - kc * KTc);
    const int kbase = kc * KTc * BK * 2;
    const int n0 = nb * BN_OUT;
    const uint16_t* Bg = p.B + (int64_t)g * p.b_group_stride;

    // DMA plan of this lane: slot s = q*64 + lane holds row s/8, chunk (s%8)^(row%8)
    DmaPlan<BM, BR> d;
#pragma unroll
    for (int qi = 0; qi < C::A_MAX; ++qi) {
      const int q = qi * 4 + wave;
      const int r = min(q * 8 + (lane >> 3), BM - 1);
      const int c = (lane & 7) ^ (r & 7);
      const int rr = min(r, rows - 1);
      const int grow = p.gather ? p.gather[m0 + rr] : (m0 + rr);
      d.a_off[qi] = (uint32_t)grow * row_bytes + (uint32_t)c * 16u;
      d.a_cb[qi] = (uint32_t)c * 16u;
    }
#pragma unroll
    for (int qi = 0; qi < C::B_PER; ++qi) {
      const int q = qi * 4 + wave;
      const int r = q * 8 + (lane >> 3);  // B tile row
      const int c = (lane & 7) ^ (r & 7);
      // weight rows past N (a ragged last column block, or experts past E in
      // the router) fetch through an offset past the buffer: zeros, no traffic
      const int col = (EPI == EPI_SWIGLU) ? n0 + (r & 127) : n0 + r;
      const int wr = (EPI == EPI_SWIGLU && r >= 128) ? p.up_row0 + col : col;
      d.b_off[qi] = (col < p.N) ? chunk_off(wr, (uint32_t)c * 16u, p.b_row_pitch, p.b_blk_pitch) : 0x80000000u;
      d.b_cb[qi] = (uint32_t)c * 16u;
    }
    d.row_bytes = row_bytes;
    d.ktail = (p.K % BK) != 0;
    const u32x4_t ra = make_rsrc(p.A, (uint32_t)p.a_rows * row_bytes);
    const u32x4_t rb = make_rsrc(Bg, p.b_group_bytes);

    const int wave_col0 = (EPI == EPI_SWIGLU) ? n0 + 32 * wave : n0 + (BR / 4) * wave;
    const bool wave_live = wave_col0 < p.N;

    f32x4_t acc[MSUB][NJ];
#pragma unroll
    for (int i = 0; i < MSUB; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    switch (msub_live) {
#define MOE_LIVE_CASE(n)                                                                                      \
  case n:                                                                                                     \
    if (n <= MSUB)                                                                                            \
      kloop<BM, BR, NJ, (n <= MSUB ? n : MSUB)>(acc, ring, d, ra, rb, wave, lane, KT, kbase, wave_live, brow,   \
                                                p.b_blk_pitch);                                                  \
    break;
      MOE_LIVE_CASE(1) MOE_LIVE_CASE(2) MOE_LIVE_CASE(3) MOE_LIVE_CASE(4)
      MOE_LIVE_CASE(5) MOE_LIVE_CASE(6) MOE_LIVE_CASE(7) MOE_LIVE_CASE(8)
#undef MOE_LIVE_CASE
      default: break;
    }
    // every wave is done reading the ring before the next tile's DMA starts
    lds_barrier();

    // ---- epilogue.  C fragment: lane holds column (lane & 15), rows 4*(lane>>4)+r
    if (wave_live && ksplit > 1) {
      // raw fp32 sums of this K chunk: partial[kc][row][col] (SwiGLU: gate
      // columns [0, N), up columns [N, 2N))
      const int ldp = (EPI == EPI_SWIGLU) ? 2 * p.N : p.N;
      float* part = p.partial + (int64_t)kc * p.M * ldp;
#pragma unroll
      for (int i = 0; i < MSUB; ++i) {
        if (i >= msub_live) continue;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          int col;
          if (EPI == EPI_SWIGLU) {
            const int c0 = wave_col0 + 16 * (j & 1) + (lane & 15);
            if (c0 >= p.N) continue;
            col = (j < 2) ? c0 : p.N + c0;
          } else {
            col = wave_col0 + 16 * j + (lane & 15);
            if (col >= p.N) continue;
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = 16 * i + 4 * (lane >> 4) + r;
            if (row < rows) part[(int64_t)(m0 + row) * ldp + col] = acc[i][j][r];
          }
        }
      }
    } else if (wave_live) {
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
                const float h = silu_mul(gv, uv);
                out[(int64_t)(m0 + row) * p.ldo + col] = f32_to_bf16_rne(h);
              }
            }
          }
        } else if (EPI == EPI_BF16) {
          uint16_t* out = reinterpret_cast<uint16_t*>(p.out);
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            const int col = wave_col0 + 16 * j + (lane & 15);
            if (col >= p.N) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int row = 16 * i + 4 * (lane >> 4) + r;
              if (row < rows) out[(int64_t)(m0 + row) * p.ldo + col] = f32_to_bf16_rne(acc[i][j][r]);
            }
          }
        } else {
          float* out = reinterpret_cast<float*>(p.out);
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            const int col = wave_col0 + 16 * j + (lane & 15);
            if (col >= p.N) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int row = 16 * i + 4 * (lane >> 4) + r;
              if (row < rows) {
                float v = acc[i][j][r];
                if (EPI == EPI_ROUTER && p.bias) v += p.bias[col];
                out[(int64_t)(m0 + row) * p.ldo + col] = v;
              }
            }
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Streaming variant for groups of at most 16 rows on average (decode
// batches).  There the GEMM is a pure weight stream, so the tile is shaped for
// HBM rather than for operand reuse:
//   * a tile is BM rows x 64 weight rows (EPI_SWIGLU: 32 gate rows and the
//     matching 32 up rows, 32 h columns; otherwise 64 output columns), and a
//     stage covers 256 k, i.e. 512 contiguous bytes of every row.  A read-only
//     probe of the two orders on MI355X: 128-byte pieces of 256 rows per stage
//     (the large-tile kernels' K walk) stream HBM at about 4.1 TB/s with one
//     workgroup per CU, 512-byte pieces of 64 rows at about 6.1 TB/s, the rate
//     of a contiguous read.
//   * wave w owns weight rows 16w..16w+15 of the tile.  With EPI_SWIGLU those
//     are 8 gate rows and the same 8 up rows, so a 16x16 accumulator holds
//     gate in its columns 0-7 and up in columns 8-15; one lane exchange pairs
//     them for the SwiGLU epilogue.
//   * each workgroup runs through its units (tile, K chunk) as one software
//     pipeline over a 3-stage ring: the DMA of sequence stage g + 2 is issued
//     while stage g is computed, across unit boundaries, so the stream never
//     drains between tiles.
//   * vmcnt: every stage is exactly SD DMA instructions per wave and every
//     epilogue exactly SS stores per wave (masked lanes store through an
//     offset past the buffer, which the hardware drops), so each wait is an
//     exact count of what was issued after the stage it needs.
//   * LDS: row r of a stage holds 32 chunks of 16 bytes, chunk c at position
//     c ^ (r & 15); the fragment reads (16 rows, one chunk column) then touch
//     16 distinct 4-bank groups.
//   * K need not be a multiple of 256: chunks past the end of a row are
//     fetched through an offset past the buffer (zeros).
//   * the gathered row indices are staged in LDS up front (dynamic LDS of M
//     ints, none without a gather), so that building the DMA plan of the next
//     unit issues no vector load (which would make the compiler wait for
//     every DMA in flight).
constexpr int kStreamBR = 64;          // weight rows per tile
constexpr int kStreamCH = 32;          // 16-byte chunks per row per stage (256 k)
constexpr int kStreamNS = 3;           // ring depth

template <int BM>
struct StreamTile {
  static constexpr int MSUB = BM / 16;
  static constexpr int SLOTS = (BM + kStreamBR) * kStreamCH;  // 16-byte slots per stage
  static constexpr int A_PER = BM * kStreamCH / 64 / 4;       // DMA instructions per wave (A rows)
  static constexpr int B_PER = kStreamBR * kStreamCH / 64 / 4;
  static constexpr int SD = A_PER + B_PER;                    // per wave per stage
  static constexpr int SS = 4 * MSUB;                         // epilogue stores per wave
  // packed rows whose gathered indices fit in LDS next to the ring
  static constexpr int MAX_ROWS = (BM == 16) ? 8192 : 2048;
  static_assert(SD + 2 * SS < 64, "vmcnt");
};

struct StreamUnit {
  int g, m0, rows, n0, kc, KT;
};

template <int BM>
struct StreamPlan {
  uint32_t a_off[StreamTile<BM>::A_PER];
  uint32_t b_off[StreamTile<BM>::B_PER];
  uint32_t a_cb[StreamTile<BM>::A_PER];  // byte offset of the lane's chunk inside a stage row
  uint32_t b_cb[StreamTile<BM>::B_PER];
  u32x4_t rb;
};

template <int BM, int EPI>
__device__ __forceinline__ StreamUnit stream_unit(int t, int total_mn, int nblk, int G, const int* s_tb,
                                                  const int* s_off, int KTc, int KT_all) {
  constexpr int BN_OUT = (EPI == EPI_SWIGLU) ? kStreamBR / 2 : kStreamBR;
  StreamUnit u;
  u.kc = __builtin_amdgcn_readfirstlane(t / total_mn);
  const TileCoord tc = tile_coord<BM>(t - u.kc * total_mn, nblk, G, s_tb, s_off);
  u.g = tc.g;
  u.m0 = tc.m0;
  u.rows = tc.rows;
  u.n0 = tc.nb * BN_OUT;
  u.KT = __builtin_amdgcn_readfirstlane(min(KTc, KT_all - u.kc * KTc));
  return u;
}

template <int BM, int EPI>
__device__ __forceinline__ void stream_plan(StreamPlan<BM>& d, const GemmArgs& p, const int* s_gidx,
                                            const StreamUnit& u, int wave, int lane, uint32_t row_bytes) {
  using C = StreamTile<BM>;
#pragma unroll
  for (int qi = 0; qi < C::A_PER; ++qi) {
    const int r = 2 * (qi * 4 + wave) + (lane >> 5);  // A row of the tile
    const int c = (lane & 31) ^ (r & 15);
    d.a_cb[qi] = (uint32_t)c * 16u;
    if (r < u.rows) {
      const int grow = p.gather ? s_gidx[u.m0 + r] : (u.m0 + r);
      d.a_off[qi] = (uint32_t)grow * row_bytes + (uint32_t)c * 16u;
    } else {
      d.a_off[qi] = 0x80000000u;
    }
  }
#pragma unroll
  for (int qi = 0; qi < C::B_PER; ++qi) {
    const int rb = 2 * (qi * 4 + wave) + (lane >> 5);  // weight row of the tile
    const int c = (lane & 31) ^ (rb & 15);
    d.b_cb[qi] = (uint32_t)c * 16u;
    int col, wr;
    if (EPI == EPI_SWIGLU) {
      col = u.n0 + 8 * (rb >> 4) + (rb & 7);
      wr = (rb & 8) ? p.up_row0 + col : col;
    } else {
      col = u.n0 + rb;
      wr = col;
    }
    d.b_off[qi] = (col < p.N) ? chunk_off(wr, (uint32_t)c * 16u, p.b_row_pitch, p.b_blk_pitch) : 0x80000000u;
  }
  d.rb = make_rsrc(p.B + (int64_t)u.g * p.b_group_stride, p.b_group_bytes);
}

template <int BM>
__device__ __forceinline__ void stream_issue(u32x4_t* buf, const StreamPlan<BM>& d, u32x4_t ra, int wave, int kbytes,
                                             uint32_t row_bytes, bool ktail, uint32_t b_blk) {
  using C = StreamTile<BM>;
#pragma unroll
  for (int qi = 0; qi < C::A_PER; ++qi) {
    uint32_t v = d.a_off[qi];
    if (ktail && d.a_cb[qi] + (uint32_t)kbytes >= row_bytes) v = 0x80000000u;
    dma16(buf + (qi * 4 + wave) * 64, ra, v, kbytes);
  }
#pragma unroll
  for (int qi = 0; qi < C::B_PER; ++qi) {
    uint32_t v = d.b_off[qi];
    if (ktail && d.b_cb[qi] + (uint32_t)kbytes >= row_bytes) v = 0x80000000u;
    dma16(buf + BM * kStreamCH + (qi * 4 + wave) * 64, d.rb, v, stage_off(kbytes, b_blk));
  }
}

template <int BM, int LIVE>
__device__ __forceinline__ void stream_mma(f32x4_t (&acc)[BM / 16], const u32x4_t* __restrict__ buf, int wave,
                                           int lane) {
#pragma unroll
  for (int kk = 0; kk < kStreamCH / 4; ++kk) {
    const int pos = (kk * 4 + (lane >> 4)) ^ (lane & 15);
    const bf16x8_t b =
        __builtin_bit_cast(bf16x8_t, buf[(BM + 16 * wave + (lane & 15)) * kStreamCH + pos]);
#pragma unroll
    for (int i = 0; i < LIVE; ++i) {
      const bf16x8_t a = __builtin_bit_cast(bf16x8_t, buf[(16 * i + (lane & 15)) * kStreamCH + pos]);
      acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[i], 0, 0, 0);
    }
  }
}

template <int BM, int EPI>
__global__ __launch_bounds__(kThreads) void grouped_gemm_bf16_stream_kernel(GemmArgs p) {
  using C = StreamTile<BM>;
  constexpr int MSUB = C::MSUB;
  constexpr int BN_OUT = (EPI == EPI_SWIGLU) ? kStreamBR / 2 : kStreamBR;
  static_assert(EPI != EPI_ROUTER, "the router has its own kernels");

  __shared__ u32x4_t ring[kStreamNS * C::SLOTS];
  __shared__ int s_off[kMaxGroups + 1];
  __shared__ int s_tb[kMaxGroups + 1];
  __shared__ int s_wsum[kThreads / 64];
  extern __shared__ int s_gidx[];  // [M] with a gather; the host keeps M <= MAX_ROWS

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = p.G;
  if (p.gather)
    for (int i = tid; i < p.M; i += kThreads) s_gidx[i] = p.gather[i];
  build_schedule<BM>(p, s_off, s_tb, s_wsum, tid, lane, wave);  // ends with a barrier

  const int nblk = (p.N + BN_OUT - 1) / BN_OUT;
  const int ksplit = (p.partial != nullptr && p.ksplit > 1) ? p.ksplit : 1;
  const int total_mn = s_tb[G] * nblk;
  const int total = total_mn * ksplit;
  const int xcd = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;
  const int nslots = gridDim.x / kXcds;
  const int per = (total + kXcds - 1) / kXcds;
  const int t_end = min(total, xcd * per + per);
  const uint32_t row_bytes = (uint32_t)p.K * 2u;
  const int KT_all = (p.K + 8 * kStreamCH - 1) / (8 * kStreamCH);
  const int KTc = (KT_all + ksplit - 1) / ksplit;
  const bool ktail = (p.K % (8 * kStreamCH)) != 0;
  constexpr int kStageBytes = kStreamCH * 16;

  int t_dma = xcd * per + slot;
  if (t_dma >= t_end) return;
  int t_cmp = t_dma;

  const u32x4_t ra = make_rsrc(p.A, (uint32_t)p.a_rows * row_bytes);
  // output: the fp32 partial planes of a split K, else y / h
  const int ldp = (EPI == EPI_SWIGLU) ? 2 * p.N : p.N;
  const size_t out_bytes = (ksplit > 1) ? (size_t)ksplit * p.M * ldp * 4
                                        : (size_t)p.M * p.ldo * ((EPI == EPI_F32) ? 4 : 2);
  const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
      (ksplit > 1) ? static_cast<void*>(p.partial) : p.out, (short)0, (int)out_bytes, kBufferWord3);

  // DMA side: unit t_dma, its next stage kt_dma, its plan
  StreamUnit ud = stream_unit<BM, EPI>(t_dma, total_mn, nblk, G, s_tb, s_off, KTc, KT_all);
  StreamPlan<BM> dp;
  stream_plan<BM, EPI>(dp, p, s_gidx, ud, wave, lane, row_bytes);
  int kt_dma = 0;
  bool dma_live = true;
  int dma_slot = 0;
  int issued = 0;  // stages issued so far (sequence numbers 0 .. issued-1)

  auto issue_next = [&]() {
    stream_issue<BM>(ring + dma_slot * C::SLOTS, dp, ra, wave, (ud.kc * KTc + kt_dma) * kStageBytes, row_bytes,
                     ktail, p.b_blk_pitch);
    ++issued;
    dma_slot = (dma_slot + 1 == kStreamNS) ? 0 : dma_slot + 1;
    if (++kt_dma == ud.KT) {
      kt_dma = 0;
      t_dma += nslots;
      dma_live = t_dma < t_end;
      if (dma_live) {
        ud = stream_unit<BM, EPI>(t_dma, total_mn, nblk, G, s_tb, s_off, KTc, KT_all);
        stream_plan<BM, EPI>(dp, p, s_gidx, ud, wave, lane, row_bytes);
      }
    }
  };

#pragma unroll
  for (int s = 0; s < kStreamNS - 1; ++s)
    if (dma_live) issue_next();

  StreamUnit uc = stream_unit<BM, EPI>(t_cmp, total_mn, nblk, G, s_tb, s_off, KTc, KT_all);
  int kt_cmp = 0;
  int cmp_slot = 0;
  int seq = 0;
  int ends = 0;  // epilogues of the last two iterations (issued after the stage being waited for)
  f32x4_t acc[MSUB];
#pragma unroll
  for (int i = 0; i < MSUB; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  while (true) {
    // wait for the DMA of stage `seq`: later stages and later epilogue stores may stay in flight
    const int n_dma = issued - (seq + 1);  // 0 or 1
    const int n_epi = (ends & 1) + (ends >> 1);
    switch (n_dma * 3 + n_epi) {
      case 0: wait_vmcnt<0>(); break;
      case 1: wait_vmcnt<C::SS>(); break;
      case 2: wait_vmcnt<2 * C::SS>(); break;
      case 3: wait_vmcnt<C::SD>(); break;
      case 4: wait_vmcnt<C::SD + C::SS>(); break;
      default: wait_vmcnt<C::SD + 2 * C::SS>(); break;
    }
    lds_barrier();  // the stage is complete for every wave; the slot the next DMA overwrites is free
    if (dma_live) issue_next();
    const u32x4_t* buf = ring + cmp_slot * C::SLOTS;
    const int live = (uc.rows + 15) >> 4;
    if (MSUB == 1 || live >= MSUB) stream_mma<BM, MSUB>(acc, buf, wave, lane);
    else stream_mma<BM, 1>(acc, buf, wave, lane);
    cmp_slot = (cmp_slot + 1 == kStreamNS) ? 0 : cmp_slot + 1;
    ++seq;
    const bool end = ++kt_cmp == uc.KT;
    if (end) {
      // ---- epilogue: exactly SS stores per wave.  Lane: column (lane & 15)
      // of the wave's 16 weight rows, rows 4 * (lane >> 4) + r of each sub-tile.
      const int cl = lane & 15;
#pragma unroll
      for (int i = 0; i < MSUB; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * i + 4 * (lane >> 4) + r;
          const bool row_ok = row < uc.rows;
          const float v = acc[i][r];
          if (EPI == EPI_SWIGLU) {
            const float other = __shfl_xor(v, 8, 64);  // up for gate lanes, gate for up lanes
            const int col = uc.n0 + 8 * wave + (cl & 7);
            const bool ok = row_ok && col < p.N;
            if (ksplit > 1) {
              const int pc = (cl < 8) ? col : p.N + col;
              const uint32_t off =
                  ok ? (uint32_t)((((int64_t)uc.kc * p.M + uc.m0 + row) * ldp + pc) * 4) : 0x80000000u;
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), ro, (int)off, 0, 0);
            } else {
              const uint32_t off =
                  (ok && cl < 8) ? (uint32_t)(((int64_t)(uc.m0 + row) * p.ldo + col) * 2) : 0x80000000u;
              __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_rne(silu_mul(v, other)), ro, (int)off, 0, 0);
            }
          } else {
            const int col = uc.n0 + 16 * wave + cl;
            const bool ok = row_ok && col < p.N;
            if (ksplit > 1) {
              const uint32_t off =
                  ok ? (uint32_t)((((int64_t)uc.kc * p.M + uc.m0 + row) * ldp + col) * 4) : 0x80000000u;
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), ro, (int)off, 0, 0);
            } else if (EPI == EPI_BF16) {
              const uint32_t off = ok ? (uint32_t)(((int64_t)(uc.m0 + row) * p.ldo + col) * 2) : 0x80000000u;
              __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_rne(v), ro, (int)off, 0, 0);
            } else {
              const uint32_t off = ok ? (uint32_t)(((int64_t)(uc.m0 + row) * p.ldo + col) * 4) : 0x80000000u;
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), ro, (int)off, 0, 0);
            }
          }
        }
        acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
      t_cmp += nslots;
      if (t_cmp >= t_end) break;
      uc = stream_unit<BM, EPI>(t_cmp, total_mn, nblk, G, s_tb, s_off, KTc, KT_all);
      kt_cmp = 0;
    }
    ends = ((ends << 1) | (end ? 1 : 0)) & 3;
  }
}

// ---------------------------------------------------------------------------
// Large-group variant (groups of hundreds of rows, e.g. prefill): 256 x 256
// tiles, BK = 32 per stage, a 4-stage ring (32 KB per stage), 2 x 2 waves of
// 128 x 128 computed with v_mfma_f32_32x32x16_bf16 (4 x 4 sub-tiles of 32 x 32;
// wave row wm owns the tile's 32-row sub-tiles wm, wm+2, wm+4, wm+6).
// On gfx950 the 32x32x16 shape sustains about 1.5x the rate of 16x16x32 and
// does so at one wave per SIMD.  Per stage a wave issues 16 fragment reads for
// 32 MFMAs, and the CU streams 64 KB per 2 x 256 x 256 x 64 flops, about 31
// bytes per clock at the MFMA rate, below the ~52 B/clk/CU that the
// L2 -> LDS DMA path sustains.  The plain kernel takes K in whole stages (a
// multiple of 32); the pipelined one below also pads K to whole groups of
// four stages.
//
// LDS layout: a row holds four 16-byte chunks (64 bytes); chunk c of row r sits
// at position c ^ ((r >> 2) & 3).  For the 32-row fragment reads (lane l: row
// l & 31, chunk 2h + (l >> 5)) this is the placement that gfx950's LDS serves
// without bank conflicts: measured with the SQ_LDS_BANK_CONFLICT counter on a
// read-only probe, where XOR patterns built from r & 3, (r >> 1) & 3 or
// ((r >> 1) ^ (r >> 3)) & 3 all cost 4 extra cycles per ds_read_b128.
//
// The MFMA operands are swapped (weight fragment first), so the accumulator
// holds the transpose: lane l owns output row (l & 31) of a 32 x 32 sub-tile
// and the columns 8g + 4*(l >> 5) + {0..3}, g = 0..3 (value 4g + c).  The
// epilogue therefore writes 8 (h, bf16) or 16 (y, fp32) contiguous bytes per
// lane and group.
typedef float f32x16_t __attribute__((ext_vector_type(16)));

struct Big {
  static constexpr int BM = 256;
  static constexpr int KB = 32;                   // k elements per stage
  static constexpr int A_SLOTS = 256 * 4;         // 16-byte slots of the A tile
  static constexpr int SLOTS = 2 * A_SLOTS;       // A tile then B tile
  static constexpr int PER_WAVE = 8;              // DMA instructions per wave per stage
};

__device__ __forceinline__ int big_swz(int r) { return (r >> 2) & 3; }

struct BigPlan {
  uint32_t a_off[4];
  uint32_t b_off[4];
};

__device__ __forceinline__ void big_issue(u32x4_t* buf, const BigPlan& d, u32x4_t ra, u32x4_t rb, int wave,
                                          int kbytes, uint32_t b_blk) {
#pragma unroll
  for (int qi = 0; qi < 4; ++qi) dma16(buf + (qi * 4 + wave) * 64, ra, d.a_off[qi], kbytes);
#pragma unroll
  for (int qi = 0; qi < 4; ++qi)
    dma16(buf + Big::A_SLOTS + (qi * 4 + wave) * 64, rb, d.b_off[qi], stage_off(kbytes, b_blk));
}

// Byte position of this lane's 16-byte chunk inside a 64-byte stage row.  A
// lane fetches chunk (lane & 3) ^ big_swz(r) of row r = 16 q + (lane >> 2),
// and big_swz(r) = (lane >> 4) & 3 for every q, so the chunk depends on the
// lane only.
__device__ __forceinline__ uint32_t big_chunk_bytes(int lane) {
  return (uint32_t)(((lane & 3) ^ ((lane >> 4) & 3)) * 16);
}

// The plan of the stage at byte offset kbytes of a row in a K loop padded to
// whole groups of four stages (K possibly ending inside a stage): chunks at
// or past the end of the row fetch through an offset past the buffer, which
// lands zeros in LDS and moves no data.  Unpadded loops use the plan as is
// (no copy: a copied plan changes the register allocation of the hot loop).
__device__ __forceinline__ BigPlan stage_plan(const BigPlan& d, uint32_t cb, int kbytes, uint32_t row_bytes) {
  BigPlan m;
  const bool dead = cb + (uint32_t)kbytes >= row_bytes;
#pragma unroll
  for (int qi = 0; qi < 4; ++qi) {
    m.a_off[qi] = dead ? 0x80000000u : d.a_off[qi];
    m.b_off[qi] = dead ? 0x80000000u : d.b_off[qi];
  }
  return m;
}

// Fragments of one stage for one wave: [k16 half][sub-tile].
struct BigFrags {
  bf16x8_t a[2][4];
  bf16x8_t b[2][4];
};

// Slot offset of weight sub-tile j from the wave's first weight row (the
// SwiGLU tile holds 2 gate sub-tiles, then the matching up rows 128 further on).
template <int EPI>
__device__ __forceinline__ constexpr int big_b_off(int j) {
  return (EPI == EPI_SWIGLU) ? ((j < 2) ? 128 * j : 512 + 128 * (j - 2)) : 128 * j;
}

template <int EPI, int LIVE>
__device__ __forceinline__ void big_read(BigFrags& f, const u32x4_t* __restrict__ buf, const int (&a_slot)[2],
                                         const int (&b_slot)[2]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int j = 0; j < 4; ++j) f.b[h][j] = __builtin_bit_cast(bf16x8_t, buf[b_slot[h] + big_b_off<EPI>(j)]);
#pragma unroll
    for (int i = 0; i < LIVE; ++i) f.a[h][i] = __builtin_bit_cast(bf16x8_t, buf[a_slot[h] + 256 * i]);
  }
}

// Waits until this wave's DMA of stage `st` has landed, given that stages up
// to `issued - 1` have been issued (each later stage may stay in flight).
__device__ __forceinline__ void big_wait(int st, int issued) {
  const int later = issued - 1 - st;
  if (later >= 2) wait_vmcnt<2 * Big::PER_WAVE>();
  else if (later == 1) wait_vmcnt<Big::PER_WAVE>();
  else wait_vmcnt<0>();
}

// One K-step for a wave with LIVE >= 1 live row sub-tiles: the 8 * LIVE MFMAs
// of stage `cur` are issued in 2 * LIVE groups of four (k16 half h, row
// sub-tile i); after each group come that group's share of the 8 DMA
// instructions of stage kt+4 and of the next stage's fragment reads.  Issue is
// in order, so a long run of DMA or LDS instructions would hold the MFMA pipe
// idle while the texture and LDS queues drain; spreading them keeps the pipe
// fed.  The reads (weight fragments of h = 0 and 1, then row fragments of
// h = 0 and 1) all go out in the first half of the step, so that they have
// landed by the next barrier.  Scheduling barriers pin this order.
template <int EPI, int LIVE>
__device__ __forceinline__ void big_step(f32x16_t (&acc)[4][4], const BigFrags& cur, BigFrags& nxt,
                                         u32x4_t* refill, const u32x4_t* __restrict__ next_buf, bool dma, int kbytes,
                                         const BigPlan& d, u32x4_t ra, u32x4_t rb, int wave,
                                         const int (&a_slot)[2], const int (&b_slot)[2], uint32_t b_blk) {
  static_assert(LIVE >= 1 && LIVE <= 4, "live row sub-tiles");
  constexpr int NG = 2 * LIVE;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int h = g / LIVE, i = g % LIVE;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.b[h][j], cur.a[h][i], acc[i][j], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    if (dma) {
#pragma unroll
      for (int q = (g * 8) / NG; q < ((g + 1) * 8) / NG; ++q) {
        if (q < 4) dma16(refill + (q * 4 + wave) * 64, ra, d.a_off[q], kbytes);
        else dma16(refill + Big::A_SLOTS + ((q - 4) * 4 + wave) * 64, rb, d.b_off[q - 4], stage_off(kbytes, b_blk));
      }
    }
    // read chunk c (0, 1: weight fragments of h = c; 2, 3: row fragments of
    // h = c - 2) goes out with group (c * NG) / 8
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if ((c * NG) / 8 != g) continue;
      if (c < 2) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          nxt.b[c][jj] = __builtin_bit_cast(bf16x8_t, next_buf[b_slot[c] + big_b_off<EPI>(jj)]);
      } else {
#pragma unroll
        for (int ii = 0; ii < LIVE; ++ii)
          nxt.a[c - 2][ii] = __builtin_bit_cast(bf16x8_t, next_buf[a_slot[c - 2] + 256 * ii]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// K loop: a 4-deep LDS ring filled by DMA three stages ahead and two register
// sets of fragments.  Step kt: wait for stage kt+1 and barrier (which also
// proves every wave has read stage kt out of LDS), refill that buffer with
// stage kt+4, read stage kt+1's fragments into the spare register set, and run
// stage kt's MFMAs, which hide the latency of those reads.  The last step
// reads a stale (in-bounds) buffer that is never used, so every path reaches
// the MFMAs with the same, fully waited, fragment reads.
template <int EPI, int LIVE>
__device__ __forceinline__ void big_kloop(f32x16_t (&acc)[4][4], u32x4_t* s0, u32x4_t* s1, u32x4_t* s2,
                                          u32x4_t* s3, const BigPlan& d, u32x4_t ra, u32x4_t rb, int wave, int KT,
                                          const int (&a_slot)[2], const int (&b_slot)[2], uint32_t b_blk) {
  u32x4_t* bufs[4] = {s0, s1, s2, s3};
  int issued = 0;
#pragma unroll
  for (int st = 0; st < 3; ++st)
    if (st < KT) {
      big_issue(bufs[st], d, ra, rb, wave, st * Big::KB * 2, b_blk);
      ++issued;
    }
  big_wait(0, issued);
  lds_barrier();
  if (3 < KT) {
    big_issue(s3, d, ra, rb, wave, 3 * Big::KB * 2, b_blk);
    ++issued;
  }
  BigFrags fx, fy;
  big_read<EPI, LIVE>(fx, s0, a_slot, b_slot);
  for (int kt0 = 0; kt0 < KT; kt0 += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int kt = kt0 + u;
      if (kt >= KT) break;
      BigFrags& cur = (u & 1) ? fy : fx;
      BigFrags& nxt = (u & 1) ? fx : fy;
      big_wait(kt + 1, issued);
      lds_barrier();
      const bool dma = kt + 4 < KT;
      if constexpr (LIVE >= 1) {
        big_step<EPI, LIVE>(acc, cur, nxt, bufs[u], bufs[(u + 1) & 3], dma, (kt + 4) * Big::KB * 2, d, ra, rb,
                            wave, a_slot, b_slot, b_blk);
      } else {
        if (dma) big_issue(bufs[u], d, ra, rb, wave, (kt + 4) * Big::KB * 2, b_blk);
      }
      if (dma) ++issued;
    }
  }
}

template <int EPI>
__global__ __launch_bounds__(kThreads) void grouped_gemm_bf16_big_kernel(GemmArgs p) {
  constexpr int BM = Big::BM;
  constexpr int BN_OUT = (EPI == EPI_SWIGLU) ? 128 : 256;

  __shared__ u32x4_t st0[Big::SLOTS];
  __shared__ u32x4_t st1[Big::SLOTS];
  __shared__ u32x4_t st2[Big::SLOTS];
  __shared__ u32x4_t st3[Big::SLOTS];
  __shared__ int s_off[kMaxGroups + 1];
  __shared__ int s_tb[kMaxGroups + 1];
  __shared__ int s_wsum[kThreads / 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int G = p.G;
  build_schedule<BM>(p, s_off, s_tb, s_wsum, tid, lane, wave);

  const int total_m = s_tb[G];
  const int nblk = (p.N + BN_OUT - 1) / BN_OUT;
  const int total = total_m * nblk;
  const int xcd = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;
  const int nslots = gridDim.x / kXcds;
  const int per = (total + kXcds - 1) / kXcds;
  const int t_begin = xcd * per;
  const int t_end = min(total, t_begin + per);
  const int KT = p.K / Big::KB;
  const uint32_t row_bytes = (uint32_t)p.K * 2u;

  // fragment slots: lane reads row (l & 31) of a 32-row sub-tile, chunk
  // 2h + (l >> 5) of the stage for k16 half h
  const int rin = lane & 31;
  int a_slot[2], b_slot[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int pos = (2 * h + (lane >> 5)) ^ big_swz(rin);
    a_slot[h] = (32 * wm + rin) * 4 + pos;
    b_slot[h] = Big::A_SLOTS + (((EPI == EPI_SWIGLU) ? 64 : 128) * wn + rin) * 4 + pos;
  }

  // Tile loop.  With p.tile_counter the tiles of this XCD's range are handed
  // out dynamically: a free workgroup takes the next tile in list order, which
  // balances ragged tiles and keeps neighbouring tiles close in time.  The grab
  // for the following tile is issued after the K loop (no DMA in flight then)
  // and consumed after the epilogue, which hides its latency; grabbing any
  // earlier lets tiles start out of list order, and the weight and row blocks
  // that neighbouring tiles share then drop out of L2 between their uses.
  __shared__ int s_grab;
  int t_local = slot;
  if (p.tile_counter) {
    if (tid == 0) s_grab = atomicAdd(&p.tile_counter[xcd], 1);
    __syncthreads();
    t_local = s_grab;
  }
  while (t_begin + t_local < t_end) {
    const int t = t_begin + t_local;
    int next_grab = 0;
    const TileCoord tc = tile_coord<BM>(t, nblk, G, s_tb, s_off);
    const int g = tc.g, m0 = tc.m0, rows = tc.rows, nb = tc.nb;
    const int n0 = nb * BN_OUT;
    const uint16_t* Bg = p.B + (int64_t)g * p.b_group_stride;

    // DMA plan: slot s = q*64 + lane holds row s/4 (16 rows per instruction)
    BigPlan d;
#pragma unroll
    for (int qi = 0; qi < 4; ++qi) {
      const int q = qi * 4 + wave;
      const int r = q * 16 + (lane >> 2);
      const int c = (lane & 3) ^ big_swz(r);
      if (r < rows) {
        const int grow = p.gather ? p.gather[m0 + r] : (m0 + r);
        d.a_off[qi] = (uint32_t)grow * row_bytes + (uint32_t)c * 16u;
      } else {
        d.a_off[qi] = 0x80000000u;  // past the buffer: reads zero, moves no data
      }
      int wr;
      if (EPI == EPI_SWIGLU) {
        const int col = min(n0 + (r & 127), p.N - 1);
        wr = (r < 128) ? col : p.up_row0 + col;
      } else {
        wr = min(n0 + r, p.N - 1);
      }
      d.b_off[qi] = chunk_off(wr, (uint32_t)c * 16u, p.b_row_pitch, p.b_blk_pitch);
    }
    const u32x4_t ra = make_rsrc(p.A, (uint32_t)p.a_rows * row_bytes);
    const u32x4_t rb = make_rsrc(Bg, p.b_group_bytes);

    f32x16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x16_t{};

    // 32-row sub-tiles of the tile alternate between the two wave rows, so a
    // ragged tile keeps both halves of the SIMDs busy
    const int units = (rows + 31) >> 5;
    const int live = __builtin_amdgcn_readfirstlane(min(4, (units - wm + 1) >> 1));
    switch (live) {
#define MOE_BIG_CASE(n) \
  case n: big_kloop<EPI, n>(acc, st0, st1, st2, st3, d, ra, rb, wave, KT, a_slot, b_slot, p.b_blk_pitch); break;
      MOE_BIG_CASE(0) MOE_BIG_CASE(1) MOE_BIG_CASE(2) MOE_BIG_CASE(3) MOE_BIG_CASE(4)
#undef MOE_BIG_CASE
      default: break;
    }
    if (p.tile_counter && tid == 0) next_grab = atomicAdd(&p.tile_counter[xcd], 1);

    // ---- epilogue: lane owns row (l & 31) and columns 8g + 4*(l>>5) + {0..3}
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i >= live) break;
      const int row = 32 * (2 * i + wm) + rin;
      if (row >= rows) continue;
      if (EPI == EPI_SWIGLU) {
        uint16_t* out = reinterpret_cast<uint16_t*>(p.out) + (int64_t)(m0 + row) * p.ldo;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const int col = n0 + 64 * wn + 32 * j + 8 * gq + 4 * (lane >> 5);
            if (col >= p.N) continue;
            uint32_t hb[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const float gv = acc[i][j][4 * gq + c];
              const float uv = acc[i][j + 2][4 * gq + c];
              hb[c] = f32_to_bf16_rne(silu_mul(gv, uv));
            }
            uint2 v;
            v.x = hb[0] | (hb[1] << 16);
            v.y = hb[2] | (hb[3] << 16);
            *reinterpret_cast<uint2*>(out + col) = v;
          }
        }
      } else if (EPI == EPI_F16S) {
        // as in the pipelined kernel: per 64-column segment of the row, one
        // exponent (from this lane's 32 values and those of lane ^ 32, which
        // holds the same row) and 64 scaled fp16 values; N % 64 == 0, so a
        // segment is live or dead as a whole
        uint16_t* out = reinterpret_cast<uint16_t*>(p.out) + (int64_t)(m0 + row) * p.ldo;
        const int64_t nseg = p.ldo / kF16SegCols;
#pragma unroll
        for (int sg = 0; sg < 2; ++sg) {
          float m = 0.f;
#pragma unroll
          for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(acc[i][2 * sg + jj][e]));
          m = fmaxf(m, __shfl_xor(m, 32, 64));
          const int kx = f16s_exponent(m);
          const int seg_col = n0 + 128 * wn + 64 * sg;
          if (seg_col >= p.N) continue;
          if (lane < 32) p.scale_out[(int64_t)(m0 + row) * nseg + seg_col / kF16SegCols] = kx;
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int j = 2 * sg + jj;
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
              const int col = n0 + 128 * wn + 32 * j + 8 * gq + 4 * (lane >> 5);
              uint2 v;
              v.x = pack_f16x2(ldexpf(acc[i][j][4 * gq], kx), ldexpf(acc[i][j][4 * gq + 1], kx));
              v.y = pack_f16x2(ldexpf(acc[i][j][4 * gq + 2], kx), ldexpf(acc[i][j][4 * gq + 3], kx));
              *reinterpret_cast<uint2*>(out + col) = v;
            }
          }
        }
      } else if (EPI == EPI_BF16) {
        uint16_t* out = reinterpret_cast<uint16_t*>(p.out) + (int64_t)(m0 + row) * p.ldo;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const int col = n0 + 128 * wn + 32 * j + 8 * gq + 4 * (lane >> 5);
            if (col >= p.N) continue;
            uint2 v;
            v.x = pack_bf16x2(acc[i][j][4 * gq], acc[i][j][4 * gq + 1]);
            v.y = pack_bf16x2(acc[i][j][4 * gq + 2], acc[i][j][4 * gq + 3]);
            *reinterpret_cast<uint2*>(out + col) = v;
          }
        }
      } else {
        float* out = reinterpret_cast<float*>(p.out) + (int64_t)(m0 + row) * p.ldo;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const int col = n0 + 128 * wn + 32 * j + 8 * gq + 4 * (lane >> 5);
            if (col >= p.N) continue;
            *reinterpret_cast<f32x4_t*>(out + col) =
                f32x4_t{acc[i][j][4 * gq], acc[i][j][4 * gq + 1], acc[i][j][4 * gq + 2], acc[i][j][4 * gq + 3]};
          }
        }
      }
    }
    if (p.tile_counter && tid == 0) s_grab = next_grab;
    lds_barrier();  // also: every wave is done with the ring before the next tile's DMA
    t_local = p.tile_counter ? s_grab : t_local + nslots;
  }
}

// ---------------------------------------------------------------------------
// Pipelined variant of the large-group kernel (same tiles, ring, fragments and
// MFMA schedule) for K loops of at least 8 stages, a multiple of 4.  The ring
// never drains between tiles: the last four K steps of a tile fill the ring
// with stages 0..3 of the workgroup's next tile, so that tile's first DMA
// latency and the epilogue stores of the current tile overlap.
//
//  * Tiles are assigned statically (round robin inside the XCD's range), so
//    the next tile is known without a memory round trip.
//  * The next tile's gathered row indices are fetched by a 4-byte DMA into LDS
//    at step KT-8 and read back at step KT-4, after the barrier that follows
//    the wait which covers that DMA; the compiler therefore never has to wait
//    for a global load while stage DMAs are in flight.
//  * vmcnt retires in issue order.  Every stage is 8 DMA instructions per
//    wave; the epilogue issues exactly kEpiStores buffer stores per wave (rows
//    and columns outside the output get an offset past the buffer, which the
//    hardware drops), so each wait below is an exact count of the operations
//    issued after the stage it needs (an extra index DMA only makes a wait
//    stricter).  Counts above 63 are clamped: vmcnt cannot exceed 63, so once
//    more than 63 operations follow a stage, that stage has retired.
template <int N>
__device__ __forceinline__ void wait_vmcnt_clamped() {
  wait_vmcnt<(N > 63 ? 63 : N)>();
}

struct PipeNext {
  bool has;
  int g, m0, rows, n0;
};

// ---------------------------------------------------------------- 8-wave pipelined kernel
// Used for large groups (at least 96 rows per group on average: the prefill
// workloads).  256x256 output tiles (EPI_SWIGLU: 128 h columns, i.e. 128 gate
// rows and the matching 128 up rows of w13), persistent workgroups of eight
// waves, two per SIMD: with one wave per SIMD every stall of the single
// instruction stream (a DMA waiting for room in the texture queues, an LDS
// read, a barrier) leaves the matrix core idle; with two, the SIMD issues the
// other wave's MFMAs meanwhile.  MI355X sustains the same MFMA rate with one
// or two waves per SIMD, and its LDS serves about 200 B/clk to eight waves
// against about 115 B/clk to four.
//
// K loop: 32-wide K stages (A 256 rows and B 256 rows x 64 bytes, 32 KB)
// through a 4-stage LDS ring filled by direct global->LDS DMA three stages
// ahead, one barrier per stage.  The ring never drains between tiles: the
// last four steps of a tile fill it with the workgroup's next tile, whose
// gathered row indices arrive in LDS by a 4-byte DMA four steps earlier.
// Rows past a group's end fetch through an out-of-range offset (zeros in LDS,
// no data moved) and are never stored.  A K loop not a multiple of four
// stages (PAD) is padded with chunks that read zeros.  Chunk c of row r sits
// at 16-byte position c ^ ((r >> 2) & 3) of the row's 64 bytes, which the
// 32x32x16 fragment reads take without bank conflicts.
//
// Wave w (SIMD w % 4) has wm = w / 4 and wn = w % 4: it owns row sub-tiles
// wm, wm + 2, wm + 4, wm + 6 of 32 rows (so both waves of a SIMD lose rows
// alike in a partly filled tile; sub-tiles wholly past the group's end skip
// their MFMAs) and weight sub-tiles of 32 rows: for EPI_SWIGLU the gate rows
// 32 wn .. 32 wn + 31 and the same up rows (h columns 32 wn ..), otherwise
// output columns 64 wn .. 64 wn + 63 (one 64-column segment of the fp16 +
// exponent layout).  Accumulators: 4 x 2 32x32 blocks, 128 fp32 per lane.
// Each stage is 32 DMA instructions, four per wave (two A, two B); the
// epilogue issues a fixed number of stores per wave, so every vmcnt wait is
// an exact count of the operations issued after the stage it needs.
constexpr int kThreads8 = 512;

struct P8 {
  static constexpr int PER_WAVE = 4;  // DMA instructions per wave per stage
};

struct Plan8 {
  uint32_t a_off[2];
  uint32_t b_off[2];
};

template <int EPI>
struct Pipe8Epi {
  // 16-byte stores per wave per tile: EPI_SWIGLU 2 per row sub-tile, EPI_F16S
  // 4 and one exponent, EPI_BF16 4, EPI_F32 8
  static constexpr int kStores = (EPI == EPI_SWIGLU) ? 8 : (EPI == EPI_F16S) ? 20 : (EPI == EPI_BF16) ? 16 : 32;
};

// Column groups g (even) and g + 1 of a row, each four 16-bit values (two
// dwords) held by lanes l (columns 8g + 0..3, 8(g+1) + 0..3) and l ^ 32
// (columns 8g + 4..7, 8(g+1) + 4..7): one swap of the upper half of the first
// with the lower half of the second (v_permlane32_swap) leaves lane l < 32
// with the 8 columns of group g and lane l + 32 with those of group g + 1, in
// column order, as one 16-byte store each.
__device__ __forceinline__ u32x4_t pair_columns(uint32_t g_lo, uint32_t g_hi, uint32_t h_lo, uint32_t h_hi) {
  const auto x = __builtin_amdgcn_permlane32_swap(g_lo, h_lo, false, false);
  const auto y = __builtin_amdgcn_permlane32_swap(g_hi, h_hi, false, false);
  return u32x4_t{(uint32_t)x[0], (uint32_t)y[0], (uint32_t)x[1], (uint32_t)y[1]};
}

// a_blk / b_blk: block pitches of A and B (64 for row-major operands).
__device__ __forceinline__ void p8_issue(u32x4_t* buf, const Plan8& d, u32x4_t ra, u32x4_t rb, int wave,
                                         int kbytes, uint32_t a_blk, uint32_t b_blk) {
#pragma unroll
  for (int qi = 0; qi < 2; ++qi) dma16(buf + (qi * 8 + wave) * 64, ra, d.a_off[qi], stage_off(kbytes, a_blk));
#pragma unroll
  for (int qi = 0; qi < 2; ++qi)
    dma16(buf + Big::A_SLOTS + (qi * 8 + wave) * 64, rb, d.b_off[qi], stage_off(kbytes, b_blk));
}

// As stage_plan: chunks at or past the end of a row read zeros (padded K loops).
__device__ __forceinline__ Plan8 p8_stage_plan(const Plan8& d, uint32_t cb, int kbytes, uint32_t row_bytes) {
  Plan8 m;
  const bool dead = cb + (uint32_t)kbytes >= row_bytes;
#pragma unroll
  for (int qi = 0; qi < 2; ++qi) {
    m.a_off[qi] = dead ? 0x80000000u : d.a_off[qi];
    m.b_off[qi] = dead ? 0x80000000u : d.b_off[qi];
  }
  return m;
}

// DMA plan of a tile: instruction q = 8 qi + wave covers tile rows 16 q ..
// 16 q + 15; lane l fetches chunk (l & 3) ^ swz of row 16 q + (l >> 2).  A rows
// past the tile's rows fetch through an out-of-range offset (zeros, no data
// moved); weight rows past N are clamped to the last one (never stored).
// Gathered row indices come from `gidx` (LDS, the next tile) or from global
// memory (`from_global`, the first tile).
template <int EPI>
__device__ __forceinline__ void p8_plan(Plan8& d, const GemmArgs& p, const int* gidx, bool from_global, int rows,
                                        int m0, int n0, int wave, int lane, uint32_t row_bytes) {
#pragma unroll
  for (int qi = 0; qi < 2; ++qi) {
    const int q = qi * 8 + wave;
    const int r = q * 16 + (lane >> 2);
    const int c = (lane & 3) ^ big_swz(r);
    if (r < rows) {
      const int grow = p.gather ? (from_global ? p.gather[m0 + r] : gidx[r]) : (m0 + r);
      d.a_off[qi] = chunk_off(grow, (uint32_t)c * 16u, p.a_row_pitch, p.a_blk_pitch);
    } else {
      d.a_off[qi] = 0x80000000u;
    }
    int wr;
    if (EPI == EPI_SWIGLU) {
      const int col = min(n0 + (r & 127), p.N - 1);
      wr = (r < 128) ? col : p.up_row0 + col;
    } else {
      wr = min(n0 + r, p.N - 1);
    }
    d.b_off[qi] = chunk_off(wr, (uint32_t)c * 16u, p.b_row_pitch, p.b_blk_pitch);
  }
}

struct Frags8 {
  bf16x8_t a[2][4];
  bf16x8_t b[2][2];
};

// Slot offset of weight sub-tile j from the wave's first weight row.
template <int EPI>
__device__ __forceinline__ constexpr int p8_b_off(int j) {
  return (EPI == EPI_SWIGLU) ? 512 * j : 128 * j;
}

template <int EPI, int LIVE>
__device__ __forceinline__ void p8_read(Frags8& f, const u32x4_t* __restrict__ buf, const int (&a_slot)[2],
                                        const int (&b_slot)[2]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int j = 0; j < 2; ++j) f.b[h][j] = __builtin_bit_cast(bf16x8_t, buf[b_slot[h] + p8_b_off<EPI>(j)]);
#pragma unroll
    for (int i = 0; i < LIVE; ++i) f.a[h][i] = __builtin_bit_cast(bf16x8_t, buf[a_slot[h] + 256 * i]);
  }
}

// One K step of a wave with LIVE >= 1 live row sub-tiles: 4 LIVE MFMAs in
// 2 LIVE groups of two (k16 half h, row sub-tile i), the wave's 4 DMA
// instructions of stage kt+4 spread over the groups.  One register set of
// fragments: once the last MFMA of half h has issued, half h's fragments of
// the next stage are read into the same registers (the other wave of the SIMD
// keeps the matrix core busy while they arrive).
template <int EPI, int LIVE>
__device__ __forceinline__ void p8_step(f32x16_t (&acc)[4][2], Frags8& f, u32x4_t* refill,
                                        const u32x4_t* __restrict__ next_buf, bool dma, int kbytes, const Plan8& d,
                                        u32x4_t ra, u32x4_t rb, int wave, const int (&a_slot)[2],
                                        const int (&b_slot)[2], uint32_t a_blk, uint32_t b_blk) {
  static_assert(LIVE >= 1 && LIVE <= 4, "live row sub-tiles");
  constexpr int NG = 2 * LIVE;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int h = g / LIVE, i = g % LIVE;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[h][j], f.a[h][i], acc[i][j], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    if (dma) {
#pragma unroll
      for (int q = (g * 4) / NG; q < ((g + 1) * 4) / NG; ++q) {
        if (q < 2) dma16(refill + (q * 8 + wave) * 64, ra, d.a_off[q], stage_off(kbytes, a_blk));
        else dma16(refill + Big::A_SLOTS + ((q - 2) * 8 + wave) * 64, rb, d.b_off[q - 2], stage_off(kbytes, b_blk));
      }
    }
    if (i == LIVE - 1) {
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
        f.b[h][jj] = __builtin_bit_cast(bf16x8_t, next_buf[b_slot[h] + p8_b_off<EPI>(jj)]);
#pragma unroll
      for (int ii = 0; ii < LIVE; ++ii)
        f.a[h][ii] = __builtin_bit_cast(bf16x8_t, next_buf[a_slot[h] + 256 * ii]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One tile's K loop.  On entry stages 0..3 of this tile are in flight (or
// landed); `after_epi` says whether the previous tile's epilogue stores were
// issued after them.  Step kt waits for this wave's DMA of stage kt+1, meets
// the other waves at the barrier (which publishes the stage and proves that
// every wave has read stage kt's buffer), refills that buffer with stage
// kt+4 and computes stage kt.  With nx.has the last four steps issue the next
// tile's stages 0..3 instead, from the plan built at step KT-4 out of the row
// indices that waves 0..3 (64 rows each) staged into s_gidx at step KT-8.
template <int EPI, int LIVE, bool PAD>
__device__ __forceinline__ void pipe8_kloop(f32x16_t (&acc)[4][2], u32x4_t* s0, u32x4_t* s1, u32x4_t* s2,
                                            u32x4_t* s3, int* s_gidx, const GemmArgs& p, const Plan8& d,
                                            u32x4_t ra, u32x4_t rb, Plan8& dn, u32x4_t rbn, const PipeNext& nx,
                                            bool after_epi, int wave, int lane, int KT, uint32_t row_bytes,
                                            const int (&a_slot)[2], const int (&b_slot)[2]) {
  constexpr int S = Pipe8Epi<EPI>::kStores;
  constexpr int PW = P8::PER_WAVE;
  u32x4_t* bufs[4] = {s0, s1, s2, s3};
  if (after_epi) wait_vmcnt_clamped<3 * PW + S>();
  else wait_vmcnt<3 * PW>();
  lds_barrier();
  Frags8 f;
  if constexpr (LIVE > 0) p8_read<EPI, LIVE>(f, s0, a_slot, b_slot);
  for (int kt0 = 0; kt0 < KT; kt0 += 4) {
    const bool last = kt0 + 4 == KT;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int kt = kt0 + u;
#define MOE_P8_STEP(PL) \
  p8_step<EPI, LIVE>(acc, f, bufs[u], bufs[(u + 1) & 3], dma, kbytes, PL, ra, rbs, wave, a_slot, b_slot, \
                     p.a_blk_pitch, p.b_blk_pitch)
      if (last && !nx.has) {
        if (u == 0) wait_vmcnt<2 * PW>();
        else if (u == 1) wait_vmcnt<PW>();
        else wait_vmcnt<0>();
      } else if (kt0 == 0 && u < 3 && after_epi) {
        wait_vmcnt_clamped<2 * PW + S>();
      } else {
        wait_vmcnt<2 * PW>();
      }
      lds_barrier();
      if (u == 0 && kt0 + 8 == KT && nx.has && p.gather && wave < 4) {
        const int r = 64 * wave + lane;
        const uint32_t voff = (r < nx.rows) ? (uint32_t)(nx.m0 + r) * 4u : 0x80000000u;
        dma4(s_gidx + 64 * wave, make_rsrc(p.gather, (uint32_t)p.M * 4u), voff, 0);
      }
      if (u == 0 && last && nx.has) p8_plan<EPI>(dn, p, s_gidx, false, nx.rows, nx.m0, nx.n0, wave, lane, row_bytes);
      bool dma;
      int kbytes;
      if (!last) {
        dma = true;
        kbytes = (kt + 4) * Big::KB * 2;
      } else {
        dma = nx.has;
        kbytes = u * Big::KB * 2;
      }
      Plan8 dd;
#pragma unroll
      for (int qi = 0; qi < 2; ++qi) {
        dd.a_off[qi] = last ? dn.a_off[qi] : d.a_off[qi];
        dd.b_off[qi] = last ? dn.b_off[qi] : d.b_off[qi];
      }
      const u32x4_t rbs = last ? rbn : rb;
      if constexpr (PAD) {
        const Plan8 dk = p8_stage_plan(dd, big_chunk_bytes(lane), kbytes, row_bytes);
        if constexpr (LIVE >= 1) {
          MOE_P8_STEP(dk);
        } else {
          if (dma) p8_issue(bufs[u], dk, ra, rbs, wave, kbytes, p.a_blk_pitch, p.b_blk_pitch);
        }
      } else {
        if constexpr (LIVE >= 1) {
          MOE_P8_STEP(dd);
        } else {
          if (dma) p8_issue(bufs[u], dd, ra, rbs, wave, kbytes, p.a_blk_pitch, p.b_blk_pitch);
        }
      }
    }
  }
}

// Epilogue of the 8-wave kernel: exactly Pipe8Epi<EPI>::kStores buffer
// stores per wave, 16 bytes per lane (rows past the tile and columns past N go
// to an offset past the buffer, which stores nothing), so that the K loop's
// vmcnt waits stay exact counts.  Lane l (row 32 (2i + wm) + (l & 31)) holds
// columns 8g + 4 (l >> 5) + 0..3 of each 32-column block; pair_columns gives
// each lane 8 consecutive columns of its row.
//
// EPI_F16S: a wave's 64 columns of a row are 128 bytes, one whole line of y.
// The fp16 values go through the wave's own LDS block (`stage`: 16 rows of
// 128 bytes, 144 bytes apart, so that neither the 8-byte writes of 16 rows nor
// the 16-byte reads of 8 rows pile onto a few banks), so that each of the 16
// value stores writes 8 whole rows' 128 bytes instead of 32 rows' 32-byte
// pieces: the same bytes in a quarter of the write requests (down 254 -> 237
// us measured for the store pattern alone).
constexpr int kStageRow = 9;                   // 16-byte units per staged row

// Orders a wave's LDS accesses around an exchange between its lanes: what a
// lane wrote before is visible to every lane of the wave after (the compiler
// may not keep an earlier read of the same address, nor move accesses across).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
constexpr int kStageWave = 16 * kStageRow;     // 16-byte units per wave

template <int EPI>
__device__ __forceinline__ void p8_epilogue(const f32x16_t (&acc)[4][2], const GemmArgs& p,
                                            __amdgpu_buffer_rsrc_t ro, int rows, int m0, int n0, int wm, int wn,
                                            int lane, u32x4_t* __restrict__ stage) {
  const int rin = lane & 31;
  const int hi = lane >> 5;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 32 * (2 * i + wm) + rin;
    const bool row_ok = row < rows;
    if (EPI == EPI_SWIGLU) {
      uint32_t hb[4][2];
#pragma unroll
      for (int gq = 0; gq < 4; ++gq)
#pragma unroll
        for (int c = 0; c < 2; ++c)
          hb[gq][c] = pack_bf16x2(silu_mul(acc[i][0][4 * gq + 2 * c], acc[i][1][4 * gq + 2 * c]),
                                  silu_mul(acc[i][0][4 * gq + 2 * c + 1], acc[i][1][4 * gq + 2 * c + 1]));
#pragma unroll
      for (int gp = 0; gp < 4; gp += 2) {
        const u32x4_t v = pair_columns(hb[gp][0], hb[gp][1], hb[gp + 1][0], hb[gp + 1][1]);
        const int col = n0 + 32 * wn + 8 * (gp + hi);
        // row-major h, or K-blocked [N/32][M][32] for a down projection that reads it so
        const int64_t e = p.out_kblocked ? ((int64_t)(col >> 5) * p.M + (m0 + row)) * 32 + (col & 31)
                                         : (int64_t)(m0 + row) * p.ldo + col;
        const uint32_t off = (row_ok && col < p.N) ? (uint32_t)(e * 2) : 0x80000000u;
        __builtin_amdgcn_raw_buffer_store_b128(v, ro, (int)off, 0, 0);
      }
    } else if (EPI == EPI_F16S) {
      // this wave's 64 columns are one segment: this lane's 32 values and
      // the 32 of lane ^ 32, which holds the same row
      const int nseg = (int)(p.ldo / kF16SegCols);
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          p.scale_out, (short)0, (int)((size_t)p.M * nseg * 4), kBufferWord3);
      float m = 0.f;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(acc[i][j][e]));
      m = fmaxf(m, __shfl_xor(m, 32, 64));
      const int kx = f16s_exponent(m);
      const int seg_col = n0 + 64 * wn;
      const uint32_t soff = (row_ok && seg_col < p.N && lane < 32)
                                ? (uint32_t)(((int64_t)(m0 + row) * nseg + seg_col / kF16SegCols) * 4)
                                : 0x80000000u;
      __builtin_amdgcn_raw_buffer_store_b32((uint32_t)kx, rs, (int)soff, 0, 0);
      // this lane's row in the block (rows kStageRow 16-byte units apart)
      uint2* const st8 = reinterpret_cast<uint2*>(stage + (rin & 15) * kStageRow) + hi;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        // rows 16 half .. 16 half + 15 of the sub-tile into the block: this
        // lane's 8-byte pieces, columns 32j + 8gq + 4hi .. +3 of its row, are
        // the (hi)-th halves of 16-byte groups 4j + gq
        if ((rin >> 4) == half) {
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq)
              st8[2 * (4 * j + gq)] =
                  uint2{pack_f16x2(ldexpf(acc[i][j][4 * gq], kx), ldexpf(acc[i][j][4 * gq + 1], kx)),
                        pack_f16x2(ldexpf(acc[i][j][4 * gq + 2], kx), ldexpf(acc[i][j][4 * gq + 3], kx))};
        }
        // and out again, 8 rows x 8 groups per store (the lanes read what
        // other lanes wrote: a wave-level fence on both sides)
        wave_sync();
#pragma unroll
        for (int s8 = 0; s8 < 2; ++s8) {
          const int r = 8 * s8 + (lane >> 3);
          const int g = lane & 7;
          const u32x4_t v = stage[r * kStageRow + g];
          const int orow = 32 * (2 * i + wm) + 16 * half + r;
          const int col = seg_col + 8 * g;
          const uint32_t off =
              (orow < rows && col < p.N) ? (uint32_t)(((int64_t)(m0 + orow) * p.ldo + col) * 2) : 0x80000000u;
          __builtin_amdgcn_raw_buffer_store_b128(v, ro, (int)off, 0, 0);
        }
        wave_sync();
      }
    } else if (EPI == EPI_BF16) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        uint32_t hv[4][2];
#pragma unroll
        for (int gq = 0; gq < 4; ++gq)
#pragma unroll
          for (int c = 0; c < 2; ++c) hv[gq][c] = pack_bf16x2(acc[i][j][4 * gq + 2 * c], acc[i][j][4 * gq + 2 * c + 1]);
#pragma unroll
        for (int gp = 0; gp < 4; gp += 2) {
          const u32x4_t v = pair_columns(hv[gp][0], hv[gp][1], hv[gp + 1][0], hv[gp + 1][1]);
          const int col = n0 + 64 * wn + 32 * j + 8 * (gp + hi);
          const uint32_t off =
              (row_ok && col < p.N) ? (uint32_t)(((int64_t)(m0 + row) * p.ldo + col) * 2) : 0x80000000u;
          __builtin_amdgcn_raw_buffer_store_b128(v, ro, (int)off, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int col = n0 + 64 * wn + 32 * j + 8 * gq + 4 * hi;
          typedef float f32x4b_t __attribute__((ext_vector_type(4)));
          const f32x4b_t v = {acc[i][j][4 * gq], acc[i][j][4 * gq + 1], acc[i][j][4 * gq + 2],
                              acc[i][j][4 * gq + 3]};
          const uint32_t off =
              (row_ok && col < p.N) ? (uint32_t)(((int64_t)(m0 + row) * p.ldo + col) * 4) : 0x80000000u;
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), ro, (int)off, 0, 0);
        }
      }
    }
  }
}

#undef MOE_P8_STEP

// ---------------------------------------------------------------- 8-wave kernel, A in whole lines
// For a row-major A and K a multiple of 128 (the gathered token rows of
// gate/up; h or dense rows elsewhere) A is fetched in 128-byte row pieces
// that cover two consecutive stages: one whole-line request per row and two
// stages instead of two half-line requests.  The A halves of slots 2j and
// 2j + 1 form pair slot j (tile rows 0..127 in slot 2j, rows 128..255 in slot
// 2j + 1, 128 bytes per row), shared by stages 4m + 2j and 4m + 2j + 1.  A pair
// slot is free once both of its stages have been read, at the barrier of the
// second: odd steps kt fetch A for stages kt + 3 and kt + 4 (two and three
// steps ahead), and every step fetches B for stage kt + 4 into its own slot,
// as in the 8-wave kernel above.  Chunk c (16 bytes: k 8c .. 8c + 7 of the
// pair) of row r sits at position c ^ ((r >> 1) & 7) of the row's 128 bytes,
// so the 32x32x16 fragment reads of 16 lanes (16 rows, one chunk) cover 16
// distinct 16-byte bank groups.
//
// Per wave, even steps issue 2 DMA instructions (B) and odd steps 6 (4 A,
// then 2 B).  The wait before step kt needs this wave's last instruction of
// stage kt + 1: for even kt the B of step kt - 3 (8 instructions issued since),
// for odd kt the last A of step kt - 2 (4 since).
struct Plan8A {
  uint32_t a_off[4];
  uint32_t b_off[2];
};

__device__ __forceinline__ int ap_swz(int r) { return (r >> 1) & 7; }

// DMA plan of a tile.  A: instruction q = 8 qi + wave covers tile rows 8q ..
// 8q + 7; lane l fetches chunk (l & 7) ^ ap_swz(r) of row r = 8q + (l >> 3)
// (rows past the tile read zeros through an out-of-range offset).  B: as in
// p8_plan.
template <int EPI>
__device__ __forceinline__ void p8a_plan(Plan8A& d, const GemmArgs& p, const int* gidx, bool from_global, int rows,
                                         int m0, int n0, int wave, int lane) {
#pragma unroll
  for (int qi = 0; qi < 4; ++qi) {
    const int r = (qi * 8 + wave) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ap_swz(r);
    if (r < rows) {
      const int grow = p.gather ? (from_global ? p.gather[m0 + r] : gidx[r]) : (m0 + r);
      d.a_off[qi] = (uint32_t)grow * p.a_row_pitch + (uint32_t)c * 16u;
    } else {
      d.a_off[qi] = 0x80000000u;
    }
  }
#pragma unroll
  for (int qi = 0; qi < 2; ++qi) {
    const int q = qi * 8 + wave;
    const int r = q * 16 + (lane >> 2);
    const int c = (lane & 3) ^ big_swz(r);
    int wr;
    if (EPI == EPI_SWIGLU) {
      const int col = min(n0 + (r & 127), p.N - 1);
      wr = (r < 128) ? col : p.up_row0 + col;
    } else {
      wr = min(n0 + r, p.N - 1);
    }
    d.b_off[qi] = chunk_off(wr, (uint32_t)c * 16u, p.b_row_pitch, p.b_blk_pitch);
  }
}

// DMA instruction q of step U (kt % 4): for odd U, q < 4 are the A pair
// (stages kt + 3, kt + 4 into pair slot U / 2), the rest B of stage kt + 4
// into slot U.  a_kbytes: byte offset of the pair in a row; b_kbytes: of the
// B stage.
template <int U>
__device__ __forceinline__ void p8a_dma(int q, u32x4_t* const (&bufs)[4], const Plan8A& d, u32x4_t ra, u32x4_t rb,
                                        int wave, int a_kbytes, int b_kbytes, uint32_t b_blk) {
  constexpr int NA = (U & 1) ? 4 : 0;
  if (q < NA) {
    dma16(bufs[(U >> 1) * 2 + (q >> 1)] + ((q & 1) * 8 + wave) * 64, ra, d.a_off[q], a_kbytes);
  } else {
    const int qb = q - NA;
    dma16(bufs[U] + Big::A_SLOTS + (qb * 8 + wave) * 64, rb, d.b_off[qb], stage_off(b_kbytes, b_blk));
  }
}

template <int U>
__device__ __forceinline__ void p8a_issue(u32x4_t* const (&bufs)[4], const Plan8A& d, u32x4_t ra, u32x4_t rb,
                                          int wave, int a_kbytes, int b_kbytes, uint32_t b_blk) {
  constexpr int NQ = (U & 1) ? 6 : 2;
#pragma unroll
  for (int q = 0; q < NQ; ++q) p8a_dma<U>(q, bufs, d, ra, rb, wave, a_kbytes, b_kbytes, b_blk);
}

// Fragments of the stage held in slot U: B from slot U, A from pair slot
// U / 2 at half U % 2.  a_idx[h]: this lane's A chunk of k16 half h in the
// first stage of a pair (row sub-tiles i and i + 2 share it, in slots 2j and
// 2j + 1); the second stage's chunk is 4 positions further, i.e. position
// bit 2 flipped.
template <int EPI, int LIVE, int U>
__device__ __forceinline__ void p8a_read_half(Frags8& f, int h, u32x4_t* const (&bufs)[4], const int (&a_idx)[2],
                                              const int (&b_slot)[2]) {
  constexpr int S = U & 1, J = U >> 1;
#pragma unroll
  for (int j = 0; j < 2; ++j) f.b[h][j] = __builtin_bit_cast(bf16x8_t, bufs[U][b_slot[h] + p8_b_off<EPI>(j)]);
  const int ai = a_idx[h] ^ (4 * S);
#pragma unroll
  for (int i = 0; i < LIVE; ++i) f.a[h][i] = __builtin_bit_cast(bf16x8_t, bufs[2 * J + (i >> 1)][ai + 512 * (i & 1)]);
}

// One K step (slot U = kt % 4) of a wave with LIVE >= 1 live row sub-tiles:
// as p8_step, with this step's DMA instructions spread over the MFMA groups
// and the next stage's fragments read from slot (U + 1) % 4.
template <int EPI, int LIVE, int U>
__device__ __forceinline__ void p8a_step(f32x16_t (&acc)[4][2], Frags8& f, u32x4_t* const (&bufs)[4], bool dma,
                                         int a_kbytes, int b_kbytes, const Plan8A& d, u32x4_t ra, u32x4_t rb,
                                         int wave, const int (&a_idx)[2], const int (&b_slot)[2],
                                         uint32_t b_blk) {
  static_assert(LIVE >= 1 && LIVE <= 4, "live row sub-tiles");
  constexpr int NG = 2 * LIVE;
  constexpr int NQ = (U & 1) ? 6 : 2;
  constexpr int UN = (U + 1) & 3;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int h = g / LIVE, i = g % LIVE;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[h][j], f.a[h][i], acc[i][j], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    if (dma) {
#pragma unroll
      for (int q = (g * NQ) / NG; q < ((g + 1) * NQ) / NG; ++q)
        p8a_dma<U>(q, bufs, d, ra, rb, wave, a_kbytes, b_kbytes, b_blk);
    }
    if (i == LIVE - 1) p8a_read_half<EPI, LIVE, UN>(f, h, bufs, a_idx, b_slot);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Step kt = kt0 + U of a tile's K loop: the wait, the barrier, the next
// tile's row indices (step KT - 8) and plan (step KT - 4), and the step.
// LAST: one of the last four steps, whose DMAs fetch the next tile's stages
// 0..3 (plan dn, weights rbn) if there is one.  The last four steps are
// separate code so that the plan of each step's DMAs is known without a
// select between two plans.
template <int EPI, int LIVE, int U, bool LAST>
__device__ __forceinline__ void p8a_kstep(f32x16_t (&acc)[4][2], Frags8& f, u32x4_t* const (&bufs)[4], int* s_gidx,
                                          const GemmArgs& p, const Plan8A& d, u32x4_t ra, u32x4_t rb, Plan8A& dn,
                                          u32x4_t rbn, const PipeNext& nx, bool after_epi, int wave, int lane,
                                          int KT, int kt0, const int (&a_idx)[2], const int (&b_slot)[2]) {
  constexpr int S = Pipe8Epi<EPI>::kStores;
  constexpr int W = (U & 1) ? 4 : 8;
  const int kt = kt0 + U;
  if (LAST && !nx.has) {
    // nothing is issued in the last four steps: stage KT - 3 has 8
    // instructions after it, stage KT - 2 (its A at step KT - 5) 2, stage
    // KT - 1 none
    if (U == 0) wait_vmcnt<8>();
    else if (U == 1) wait_vmcnt<2>();
    else wait_vmcnt<0>();
  } else if (kt0 == 0 && U < 3 && after_epi) {
    wait_vmcnt_clamped<W + S>();
  } else {
    wait_vmcnt<W>();
  }
  lds_barrier();
  if (!LAST && U == 0 && kt0 + 8 == KT && nx.has && p.gather && wave < 4) {
    const int r = 64 * wave + lane;
    const uint32_t voff = (r < nx.rows) ? (uint32_t)(nx.m0 + r) * 4u : 0x80000000u;
    dma4(s_gidx + 64 * wave, make_rsrc(p.gather, (uint32_t)p.M * 4u), voff, 0);
  }
  if (LAST && U == 0 && nx.has) p8a_plan<EPI>(dn, p, s_gidx, false, nx.rows, nx.m0, nx.n0, wave, lane);
  const bool dma = LAST ? nx.has : true;
  const int a_kbytes = LAST ? (U - 1) * Big::KB * 2 : (kt + 3) * Big::KB * 2;
  const int b_kbytes = LAST ? U * Big::KB * 2 : (kt + 4) * Big::KB * 2;
  const Plan8A& dd = LAST ? dn : d;
  const u32x4_t rbs = LAST ? rbn : rb;
  if constexpr (LIVE >= 1) {
    p8a_step<EPI, LIVE, U>(acc, f, bufs, dma, a_kbytes, b_kbytes, dd, ra, rbs, wave, a_idx, b_slot, p.b_blk_pitch);
  } else {
    if (dma) p8a_issue<U>(bufs, dd, ra, rbs, wave, a_kbytes, b_kbytes, p.b_blk_pitch);
  }
}

// One tile's K loop.  On entry stages 0..3 of this tile are in flight (or
// landed), issued in step order: B0 | A(0,1) B1 | B2 | A(2,3) B3, so 10
// instructions follow stage 0's last (plus the previous tile's epilogue
// stores when `after_epi`).
template <int EPI, int LIVE>
__device__ __forceinline__ void pipe8a_kloop(f32x16_t (&acc)[4][2], u32x4_t* const (&bufs)[4], int* s_gidx,
                                             const GemmArgs& p, const Plan8A& d, u32x4_t ra, u32x4_t rb,
                                             Plan8A& dn, u32x4_t rbn, const PipeNext& nx, bool after_epi, int wave,
                                             int lane, int KT, const int (&a_idx)[2], const int (&b_slot)[2]) {
  constexpr int S = Pipe8Epi<EPI>::kStores;
  if (after_epi) wait_vmcnt_clamped<10 + S>();
  else wait_vmcnt<10>();
  lds_barrier();
  Frags8 f;
  if constexpr (LIVE > 0) {
    p8a_read_half<EPI, LIVE, 0>(f, 0, bufs, a_idx, b_slot);
    p8a_read_half<EPI, LIVE, 0>(f, 1, bufs, a_idx, b_slot);
  }
#define MOE_P8A_STEP(U, LAST)                                                                                     \
  p8a_kstep<EPI, LIVE, U, LAST>(acc, f, bufs, s_gidx, p, d, ra, rb, dn, rbn, nx, after_epi, wave, lane, KT, kt0, \
                                a_idx, b_slot)
  int kt0 = 0;
  for (; kt0 + 4 < KT; kt0 += 4) {
    MOE_P8A_STEP(0, false);
    MOE_P8A_STEP(1, false);
    MOE_P8A_STEP(2, false);
    MOE_P8A_STEP(3, false);
  }
  MOE_P8A_STEP(0, true);
  MOE_P8A_STEP(1, true);
  MOE_P8A_STEP(2, true);
  MOE_P8A_STEP(3, true);
#undef MOE_P8A_STEP
}

template <int EPI, bool PAD, bool AP>
__global__ __launch_bounds__(kThreads8) void grouped_gemm_bf16_pipe8_kernel(GemmArgs p) {
  static_assert(!(PAD && AP), "whole-line A needs K a multiple of 128");
  using PlanT = std::conditional_t<AP, Plan8A, Plan8>;
  constexpr int BM = Big::BM;
  constexpr int BN_OUT = (EPI == EPI_SWIGLU) ? 128 : 256;

  __shared__ u32x4_t st0[Big::SLOTS];
  __shared__ u32x4_t st1[Big::SLOTS];
  __shared__ u32x4_t st2[Big::SLOTS];
  __shared__ u32x4_t st3[Big::SLOTS];
  __shared__ int s_off[kMaxGroups + 1];
  __shared__ int s_tb[kMaxGroups + 1];
  __shared__ int s_wsum[kThreads8 / 64];
  __shared__ int s_gidx[BM];
  __shared__ u32x4_t s_stage[(EPI == EPI_F16S) ? 8 * kStageWave : 1];  // the epilogue's rows per wave

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int G = p.G;
  build_schedule<BM, kThreads8>(p, s_off, s_tb, s_wsum, tid, lane, wave);

  const int total_m = s_tb[G];
  const int nblk = (p.N + BN_OUT - 1) / BN_OUT;
  const int total = total_m * nblk;
  const int xcd = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;
  const int nslots = gridDim.x / kXcds;
  const int per = (total + kXcds - 1) / kXcds;
  const int t_begin = xcd * per;
  const int t_end = min(total, t_begin + per);
  const int KT = PAD ? ((p.K + Big::KB - 1) / Big::KB + 3) & ~3 : p.K / Big::KB;
  const uint32_t row_bytes = (uint32_t)p.K * 2u;
  int t = t_begin + slot;
  if (t >= t_end) return;  // whole workgroup, after the last barrier it takes part in

  const int rin = lane & 31;
  int a_slot[2], b_slot[2];
  int a_idx[2];  // whole-line A: k16 half h of a pair's first stage
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int pos = (2 * h + (lane >> 5)) ^ big_swz(rin);
    a_slot[h] = (32 * wm + rin) * 4 + pos;
    b_slot[h] = Big::A_SLOTS + (((EPI == EPI_SWIGLU) ? 32 : 64) * wn + rin) * 4 + pos;
    a_idx[h] = (32 * wm + rin) * 8 + ((2 * h + (lane >> 5)) ^ ap_swz(32 * wm + rin));
  }
  u32x4_t* const bufs[4] = {st0, st1, st2, st3};
  const u32x4_t ra = make_rsrc(p.A, (uint32_t)p.a_rows * row_bytes);
  const uint32_t b_bytes = p.b_group_bytes;
  const size_t out_elt = (EPI == EPI_F32) ? 4 : 2;
  const __amdgpu_buffer_rsrc_t ro =
      __builtin_amdgcn_make_buffer_rsrc(p.out, (short)0, (int)((size_t)p.M * p.ldo * out_elt), kBufferWord3);

  TileCoord tc = tile_coord<BM>(t, nblk, G, s_tb, s_off);
  PlanT d;
  if constexpr (AP) p8a_plan<EPI>(d, p, nullptr, true, tc.rows, tc.m0, tc.nb * BN_OUT, wave, lane);
  else p8_plan<EPI>(d, p, nullptr, true, tc.rows, tc.m0, tc.nb * BN_OUT, wave, lane, row_bytes);
  u32x4_t rb = make_rsrc(p.B + (int64_t)tc.g * p.b_group_stride, b_bytes);
  if constexpr (AP) {
    // step order: B0 | A(0,1) B1 | B2 | A(2,3) B3
    p8a_issue<0>(bufs, d, ra, rb, wave, 0, 0, p.b_blk_pitch);
    p8a_issue<1>(bufs, d, ra, rb, wave, 0, 1 * Big::KB * 2, p.b_blk_pitch);
    p8a_issue<2>(bufs, d, ra, rb, wave, 0, 2 * Big::KB * 2, p.b_blk_pitch);
    p8a_issue<3>(bufs, d, ra, rb, wave, 2 * Big::KB * 2, 3 * Big::KB * 2, p.b_blk_pitch);
  } else if constexpr (PAD) {
    const uint32_t cb = big_chunk_bytes(lane);
    p8_issue(st0, p8_stage_plan(d, cb, 0, row_bytes), ra, rb, wave, 0, p.a_blk_pitch, p.b_blk_pitch);
    p8_issue(st1, p8_stage_plan(d, cb, 1 * Big::KB * 2, row_bytes), ra, rb, wave, 1 * Big::KB * 2, p.a_blk_pitch, p.b_blk_pitch);
    p8_issue(st2, p8_stage_plan(d, cb, 2 * Big::KB * 2, row_bytes), ra, rb, wave, 2 * Big::KB * 2, p.a_blk_pitch, p.b_blk_pitch);
    p8_issue(st3, p8_stage_plan(d, cb, 3 * Big::KB * 2, row_bytes), ra, rb, wave, 3 * Big::KB * 2, p.a_blk_pitch, p.b_blk_pitch);
  } else {
    p8_issue(st0, d, ra, rb, wave, 0, p.a_blk_pitch, p.b_blk_pitch);
    p8_issue(st1, d, ra, rb, wave, 1 * Big::KB * 2, p.a_blk_pitch, p.b_blk_pitch);
    p8_issue(st2, d, ra, rb, wave, 2 * Big::KB * 2, p.a_blk_pitch, p.b_blk_pitch);
    p8_issue(st3, d, ra, rb, wave, 3 * Big::KB * 2, p.a_blk_pitch, p.b_blk_pitch);
  }

  bool after_epi = false;
  while (true) {
    const int m0 = tc.m0, rows = tc.rows, n0 = tc.nb * BN_OUT;
    PipeNext nx;
    const int tn = t + nslots;
    nx.has = tn < t_end;
    TileCoord tcn = tc;
    if (nx.has) tcn = tile_coord<BM>(tn, nblk, G, s_tb, s_off);
    nx.g = tcn.g;
    nx.m0 = tcn.m0;
    nx.rows = tcn.rows;
    nx.n0 = tcn.nb * BN_OUT;
    const u32x4_t rbn = make_rsrc(p.B + (int64_t)tcn.g * p.b_group_stride, b_bytes);
    PlanT dn = d;

    f32x16_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};

    const int units = (rows + 31) >> 5;
    const int live = __builtin_amdgcn_readfirstlane(min(4, (units - wm + 1) >> 1));
    switch (live) {
#define MOE_PIPE8_CASE(n)                                                                                        \
  case n:                                                                                                        \
    if constexpr (AP)                                                                                            \
      pipe8a_kloop<EPI, n>(acc, bufs, s_gidx, p, d, ra, rb, dn, rbn, nx, after_epi, wave, lane, KT, a_idx,      \
                           b_slot);                                                                              \
    else                                                                                                         \
      pipe8_kloop<EPI, n, PAD>(acc, st0, st1, st2, st3, s_gidx, p, d, ra, rb, dn, rbn, nx, after_epi, wave,     \
                               lane, KT, row_bytes, a_slot, b_slot);                                             \
    break;
      MOE_PIPE8_CASE(0) MOE_PIPE8_CASE(1) MOE_PIPE8_CASE(2) MOE_PIPE8_CASE(3) MOE_PIPE8_CASE(4)
#undef MOE_PIPE8_CASE
      default: break;
    }

    p8_epilogue<EPI>(acc, p, ro, rows, m0, n0, wm, wn, lane, s_stage + kStageWave * wave);
    if (!nx.has) break;
    t = tn;
    tc = tcn;
    d = dn;
    rb = rbn;
    after_epi = true;
  }
}

// Split-K reduction: the chunks' fp32 partial sums added in chunk order (so
// the result does not depend on timing), then the epilogue of the unsplit
// kernel: SwiGLU to bf16 h, or y in fp32 or bf16.  One thread per 4 columns
// of a row.
template <int EPI>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ partial, int ksplit, int M,
                                                            int N, void* __restrict__ out, int64_t ldo) {
  const int ldp = (EPI == EPI_SWIGLU) ? 2 * N : N;
  const int n4 = N >> 2;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)M * n4) return;
  const int row = (int)(idx / n4);
  const int col = (int)(idx - (int64_t)row * n4) * 4;
  const int64_t plane = (int64_t)M * ldp;
  const float* src = partial + (int64_t)row * ldp + col;
  f32x4_t a = *reinterpret_cast<const f32x4_t*>(src);
  for (int s = 1; s < ksplit; ++s) a += *reinterpret_cast<const f32x4_t*>(src + s * plane);
  if (EPI == EPI_SWIGLU) {
    f32x4_t u = *reinterpret_cast<const f32x4_t*>(src + N);
    for (int s = 1; s < ksplit; ++s) u += *reinterpret_cast<const f32x4_t*>(src + N + s * plane);
    uint32_t hb[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) hb[c] = f32_to_bf16_rne(silu_mul(a[c], u[c]));
    uint2 v;
    v.x = hb[0] | (hb[1] << 16);
    v.y = hb[2] | (hb[3] << 16);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + row * ldo + col) = v;
  } else if (EPI == EPI_BF16) {
    uint2 v;
    v.x = pack_bf16x2(a[0], a[1]);
    v.y = pack_bf16x2(a[2], a[3]);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + row * ldo + col) = v;
  } else {
    *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(out) + row * ldo + col) = a;
  }
}

// Shared-expert gate logits x . g (one wave per token, fp32 accumulation of
// exact bf16 products).
__global__ __launch_bounds__(256) void gate_logit_bf16_kernel(const uint16_t* __restrict__ x,
                                                              const uint16_t* __restrict__ g, int T, int H,
                                                              float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float acc = 0.f;
  for (int h = lane; h < H; h += 64) {
    const float xv = __uint_as_float((uint32_t)x[(int64_t)t * H + h] << 16);
    const float gv = __uint_as_float((uint32_t)g[h] << 16);
    acc = fmaf(xv, gv, acc);
  }
#pragma unroll
  for (int dd = 32; dd >= 1; dd >>= 1) acc += __shfl_xor(acc, dd, 64);
  if (lane == 0) out[t] = acc;
}

__global__ void zero_ints_kernel(int* p, int n) {
  if ((int)threadIdx.x < n) p[threadIdx.x] = 0;
}

// Workgroups of `kernel` (kThreads threads, no dynamic LDS) that fit on one
// CU, queried once per device and kept in `cache`.
template <typename Kern>
int occupancy_per_cu(std::atomic<int> (&cache)[64], Kern kernel) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, kThreads, 0) != hipSuccess || n < 1) n = 1;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Resident workgroups per CU for one instantiation (the persistent grid must
// fit in one wave of residency, or the static tile split would serialise).
template <int BM, int EPI, int BR>
int resident_blocks_per_cu() {
  static std::atomic<int> cache[64];
  return occupancy_per_cu(cache, grouped_gemm_bf16_kernel<BM, EPI, BR>);
}

// m-tile height the grouped GEMM picks for M rows in `groups` groups (0: the
// 256-row kernels).  From 96 rows per group on average the 256-row tiles win
// even when half their rows are padding: a weight block is read once per
// m-tile, and with 128-row tiles a group of 100-150 rows already needs two.
int pick_bm(int64_t M, int64_t groups) {
  const int64_t avg = groups > 0 ? (M + groups - 1) / groups : M;
  if (avg <= 16) return 16;
  if (avg <= 32) return 32;
  if (avg <= 64) return 64;
  if (avg < 96) return 128;
  return 0;
}

// Split-K for the weight-streaming regime (small m-tiles): with few
// (m-tile, n-block) tiles the chip is not filled and each CU streams a long
// weight panel alone; cutting K gives about kSplitTarget tiles, every chunk at
// least kSplitMinStages K stages (shorter chunks are all DMA prologue).
// Decided from the shapes and the tile upper bound only; the constants are
// the best of a sweep on the Qwen1.5-MoE decode shape.
constexpr int64_t kSplitTarget = 256;
constexpr int64_t kSplitMinStages = 8;

// The streaming kernel (16-row groups, up to StreamTile<16>::MAX_ROWS packed
// rows) pipelines its units, so it only needs about two units per CU, each
// at least kStreamMinStages stages of 256 k.
constexpr int64_t kStreamSplitTarget = 512;
constexpr int64_t kStreamMinStages = 2;

bool uses_stream(int64_t M, int64_t groups) { return pick_bm(M, groups) == 16 && M <= StreamTile<16>::MAX_ROWS; }

int ksplit_for(int64_t M, int64_t G, bool grouped, int64_t N, int64_t K, GemmEpilogue epi) {
  if (epi == EPI_ROUTER || M <= 0) return 1;
  const int64_t groups = grouped ? (G < M ? G : M) : 1;
  const int bm = pick_bm(M, groups);
  if (bm == 0) return 1;
  if (uses_stream(M, groups)) {
    const int64_t bn = (epi == EPI_SWIGLU) ? kStreamBR / 2 : kStreamBR;
    const int64_t tiles = ((M + 15) / 16 + (grouped ? groups : 0)) * ((N + bn - 1) / bn);
    const int64_t KT = (K + 8 * kStreamCH - 1) / (8 * kStreamCH);
    int64_t ks = (kStreamSplitTarget + tiles - 1) / tiles;
    if (ks > KT / kStreamMinStages) ks = KT / kStreamMinStages;
    if (ks <= 1) return 1;
    const int64_t ktc = (KT + ks - 1) / ks;
    ks = (KT + ktc - 1) / ktc;
    const int64_t ldp = (epi == EPI_SWIGLU) ? 2 * N : N;
    if (ks * M * ldp * 4 > ((int64_t)1 << 31) - 1) return 1;  // 32-bit store offsets
    return (int)ks;
  }
  const int64_t bn = (epi == EPI_SWIGLU) ? 128 : 256;
  const int64_t tiles = ((M + bm - 1) / bm + (grouped ? groups : 0)) * ((N + bn - 1) / bn);
  const int64_t KT = (K + BK - 1) / BK;
  int64_t ks = (kSplitTarget + tiles - 1) / tiles;
  if (ks > KT / kSplitMinStages) ks = KT / kSplitMinStages;
  if (ks <= 1) return 1;
  const int64_t ktc = (KT + ks - 1) / ks;
  return (int)((KT + ktc - 1) / ktc);  // no empty chunk
}

template <int BM, int EPI, int BR = kBRows>
hipError_t launch_bm(const GemmArgs& a_in, hipStream_t s, const char* name) {
  constexpr int BN_OUT = (EPI == EPI_SWIGLU) ? 128 : BR;
  GemmArgs a = a_in;
  a.ksplit = (a.partial != nullptr) ? ksplit_for(a.M, a.G, a.offsets != nullptr, a.N, a.K, (GemmEpilogue)EPI) : 1;
  const int64_t nblk = (a.N + BN_OUT - 1) / BN_OUT;
  int64_t ub_m = (a.M + BM - 1) / BM;
  if (a.offsets) ub_m += (a.G < a.M ? a.G : a.M);
  const int64_t ub = ub_m * nblk * a.ksplit;
  int64_t grid = (int64_t)device_cu_count() * resident_blocks_per_cu<BM, EPI, BR>();
  if (ub < grid) grid = ub;
  grid = ((grid + kXcds - 1) / kXcds) * kXcds;
  if (grid < kXcds) grid = kXcds;
  profile_begin(name, s);
  hipLaunchKernelGGL((grouped_gemm_bf16_kernel<BM, EPI, BR>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  if (EPI != EPI_ROUTER && a.ksplit > 1) {
    const int64_t n = (int64_t)a.M * (a.N / 4);
    hipLaunchKernelGGL((splitk_reduce_kernel<EPI>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a.partial,
                       a.ksplit, a.M, a.N, a.out, a.ldo);
  }
  profile_end(s);
  return hipGetLastError();
}

template <int BM, int EPI>
int resident_stream_per_cu() {
  static std::atomic<int> cache[64];
  return occupancy_per_cu(cache, grouped_gemm_bf16_stream_kernel<BM, EPI>);
}

template <int BM, int EPI>
hipError_t launch_stream(const GemmArgs& a_in, hipStream_t s, const char* name) {
  constexpr int BN_OUT = (EPI == EPI_SWIGLU) ? kStreamBR / 2 : kStreamBR;
  GemmArgs a = a_in;
  a.ksplit = (a.partial != nullptr) ? ksplit_for(a.M, a.G, a.offsets != nullptr, a.N, a.K, (GemmEpilogue)EPI) : 1;
  const int64_t nblk = (a.N + BN_OUT - 1) / BN_OUT;
  int64_t ub_m = (a.M + BM - 1) / BM;
  if (a.offsets) ub_m += (a.G < a.M ? a.G : a.M);
  const int64_t ub = ub_m * nblk * a.ksplit;
  int64_t grid = (int64_t)device_cu_count() * resident_stream_per_cu<BM, EPI>();
  if (ub < grid) grid = ub;
  grid = ((grid + kXcds - 1) / kXcds) * kXcds;
  if (grid < kXcds) grid = kXcds;
  profile_begin(name, s);
  const size_t lds = a.gather ? (size_t)a.M * sizeof(int) : 0;
  hipLaunchKernelGGL((grouped_gemm_bf16_stream_kernel<BM, EPI>), dim3((unsigned)grid), dim3(kThreads), lds, s, a);
  if (a.ksplit > 1) {
    const int64_t n = (int64_t)a.M * (a.N / 4);
    hipLaunchKernelGGL((splitk_reduce_kernel<EPI>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a.partial,
                       a.ksplit, a.M, a.N, a.out, a.ldo);
  }
  profile_end(s);
  return hipGetLastError();
}

template <int EPI>
int resident_big_per_cu() {
  static std::atomic<int> cache[64];
  return occupancy_per_cu(cache, grouped_gemm_bf16_big_kernel<EPI>);
}

template <int EPI>
hipError_t launch_big(const GemmArgs& a, hipStream_t s, const char* name) {
  constexpr int BN_OUT = (EPI == EPI_SWIGLU) ? 128 : 256;
  if (a.K % Big::KB != 0) return hipErrorInvalidValue;  // whole 32-wide stages only
  const int64_t nblk = (a.N + BN_OUT - 1) / BN_OUT;
  int64_t ub_m = (a.M + Big::BM - 1) / Big::BM;
  if (a.offsets) ub_m += (a.G < a.M ? a.G : a.M);
  const int64_t ub = ub_m * nblk;
  int64_t grid = (int64_t)device_cu_count() * resident_big_per_cu<EPI>();
  if (ub < grid) grid = ub;
  grid = ((grid + kXcds - 1) / kXcds) * kXcds;
  if (grid < kXcds) grid = kXcds;
  profile_begin(name, s);
  hipLaunchKernelGGL((grouped_gemm_bf16_big_kernel<EPI>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  profile_end(s);
  return hipGetLastError();
}

template <int EPI>
hipError_t launch_pipe(const GemmArgs& a, hipStream_t s, const char* name) {
  constexpr int BN_OUT = (EPI == EPI_SWIGLU) ? 128 : 256;
  const int64_t nblk = (a.N + BN_OUT - 1) / BN_OUT;
  int64_t ub_m = (a.M + Big::BM - 1) / Big::BM;
  if (a.offsets) ub_m += (a.G < a.M ? a.G : a.M);
  const int64_t ub = ub_m * nblk;
  int64_t grid = (int64_t)device_cu_count();
  if (ub < grid) grid = ub;
  grid = ((grid + kXcds - 1) / kXcds) * kXcds;
  if (grid < kXcds) grid = kXcds;
  // A row-major (gathered or plain rows, not K-blocked) with whole groups of
  // four stages: A in whole 128-byte lines (not under the fp16 + exponent
  // epilogue, whose LDS staging leaves no registers for the larger plan)
  constexpr bool kWholeLineA = EPI != EPI_F16S;
  const bool a_rows = a.a_row_pitch == (uint32_t)a.K * 2u && a.a_blk_pitch == 64u;
  profile_begin(name, s);
  if (a.K % (4 * Big::KB) != 0) {
    hipLaunchKernelGGL((grouped_gemm_bf16_pipe8_kernel<EPI, true, false>), dim3((unsigned)grid), dim3(kThreads8), 0,
                       s, a);
  } else if (kWholeLineA && a_rows) {
    hipLaunchKernelGGL((grouped_gemm_bf16_pipe8_kernel<EPI, false, kWholeLineA>), dim3((unsigned)grid),
                       dim3(kThreads8), 0, s, a);
  } else {
    hipLaunchKernelGGL((grouped_gemm_bf16_pipe8_kernel<EPI, false, false>), dim3((unsigned)grid), dim3(kThreads8), 0,
                       s, a);
  }
  profile_end(s);
  return hipGetLastError();
}

// The pipelined 256-row kernel runs K loops in whole groups of four 32-wide
// stages, padding with chunks that read zeros; it takes a K loop when the
// padding adds at most a third to it, and with gathered rows only from 8
// stages on (the next tile's row indices are staged at step KT - 8, four
// steps before its first DMA).  K not a multiple of 32 (H or I a multiple of
// 8 or 16 only) runs here whenever it can, whatever the padding: the plain
// 256-row kernel needs whole stages.
bool pipe_fits(const GemmArgs& a) {
  const int64_t KT = (a.K + Big::KB - 1) / Big::KB;
  const int64_t KTp = (KT + 3) & ~(int64_t)3;
  const int64_t min_stages = a.gather ? 8 : 4;
  if (a.K % Big::KB != 0) return KTp >= min_stages;
  if (3 * KTp > 4 * KT) return false;
  return KTp >= min_stages;
}

template <int EPI>
hipError_t launch_epi(const GemmArgs& a, hipStream_t s, const char* name) {
  // rows per group on average decides the m-tile height
  const int64_t groups = a.offsets ? (a.G < a.M ? a.G : a.M) : 1;
  if (uses_stream(a.M, groups)) return launch_stream<16, EPI>(a, s, name);
  switch (pick_bm(a.M, groups)) {
    case 16: return launch_bm<16, EPI>(a, s, name);
    case 32: return launch_bm<32, EPI>(a, s, name);
    case 64: return launch_bm<64, EPI>(a, s, name);
    case 128: return launch_bm<128, EPI>(a, s, name);
    default: break;
  }
  if (pipe_fits(a)) return launch_pipe<EPI>(a, s, name);
  // a short K loop that is not whole 32-wide stages, with gathered rows
  // (hidden size a multiple of 8 only): 128-row tiles, which mask any K tail
  if (a.K % Big::KB != 0) return launch_bm<128, EPI>(a, s, name);
  return launch_big<EPI>(a, s, name);
}

}  // namespace

hipError_t launch_zero_ints(int* p, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_ints_kernel, dim3(1), dim3(64), 0, s, p, n);
  return hipGetLastError();
}

bool grouped_gemm_uses_counter(const GemmArgs& a) {
  return pick_bm(a.M, a.offsets ? (a.G < a.M ? a.G : a.M) : 1) == 0;
}

int grouped_gemm_ksplit(int64_t M, int64_t G, bool grouped, int64_t N, int64_t K, GemmEpilogue epi) {
  return ksplit_for(M, G, grouped, N, K, epi);
}

size_t grouped_gemm_partial_bytes(int64_t M, int64_t G, bool grouped, int64_t N, int64_t K, GemmEpilogue epi) {
  const int ks = ksplit_for(M, G, grouped, N, K, epi);
  if (ks <= 1) return 0;
  const int64_t ldp = (epi == EPI_SWIGLU) ? 2 * N : N;
  return (size_t)ks * (size_t)M * (size_t)ldp * sizeof(float);
}

bool grouped_gemm_has_f16s(const GemmArgs& a) {
  const int64_t groups = a.offsets ? (a.G < a.M ? a.G : a.M) : 1;
  return a.M > 0 && pick_bm(a.M, groups) == 0;
}

bool grouped_gemm_runs_pipe8(const GemmArgs& a, GemmEpilogue epi) {
  if (epi == EPI_ROUTER || a.M <= 0) return false;
  const int64_t groups = a.offsets ? (a.G < a.M ? a.G : a.M) : 1;
  if (pick_bm(a.M, groups) != 0) return false;
  return pipe_fits(a);
}

hipError_t launch_grouped_gemm_bf16(const GemmArgs& a_in, GemmEpilogue epi, hipStream_t s, const char* name) {
  if (a_in.M <= 0) return hipSuccess;
  // operand layouts: row-major unless given
  GemmArgs a = a_in;
  const int b_rows_total = (epi == EPI_SWIGLU) ? 2 * a.up_row0 : a.N;
  if (a.b_row_pitch == 0) {
    a.b_row_pitch = (uint32_t)a.K * 2u;
    a.b_blk_pitch = 64u;
  }
  if (a.b_group_bytes == 0) a.b_group_bytes = (uint32_t)b_rows_total * (uint32_t)a.K * 2u;
  if (a.a_row_pitch == 0) {
    a.a_row_pitch = (uint32_t)a.K * 2u;
    a.a_blk_pitch = 64u;
  }
  // a K-blocked A (not gathered) or a K-blocked h output: the pipelined kernel only
  const bool a_blocked = a.a_row_pitch != (uint32_t)a.K * 2u || a.a_blk_pitch != 64u;
  if ((a_blocked || a.out_kblocked) && !grouped_gemm_runs_pipe8(a, epi)) return hipErrorInvalidValue;
  if (a_blocked && a.gather != nullptr) return hipErrorInvalidValue;
  if (a.out_kblocked && (epi != EPI_SWIGLU || a.N % kKBlock != 0 || a.ldo != a.N)) return hipErrorInvalidValue;
  if (epi == EPI_F16S) {
    if (!grouped_gemm_has_f16s(a) || a.scale_out == nullptr || a.N % kF16SegCols != 0 || a.ldo % kF16SegCols != 0)
      return hipErrorInvalidValue;
    if (pipe_fits(a)) return launch_pipe<EPI_F16S>(a, s, name);
    return launch_big<EPI_F16S>(a, s, name);
  }
  switch (epi) {
    case EPI_SWIGLU: return launch_epi<EPI_SWIGLU>(a, s, name);
    case EPI_F32: return launch_epi<EPI_F32>(a, s, name);
    case EPI_BF16: return launch_epi<EPI_BF16>(a, s, name);
    case EPI_ROUTER: {
      // up to 128 experts: 128-row weight tiles, half the stage, a deeper ring
      hipError_t e = (a.N <= 128) ? launch_bm<32, EPI_ROUTER, 128>(a, s, name) : launch_bm<32, EPI_ROUTER>(a, s, name);
      if (e != hipSuccess || a.b_extra == nullptr) return e;
      profile_begin("router_gate_logit_bf16", s);
      hipLaunchKernelGGL(gate_logit_bf16_kernel, dim3((a.M + 3) / 4), dim3(256), 0, s, a.A, a.b_extra, a.M, a.K,
                         a.extra_out);
      profile_end(s);
      return hipGetLastError();
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
