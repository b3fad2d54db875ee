// Internal declarations shared by the HIP translation units of libmoe_mi355x.
// Nothing here is part of the C ABI (include/moe.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#define MOE_MAX_GROUPS_INTERNAL 512

namespace moe {

// Launch record for optional per-kernel timing (see moe_profile_enable).
void profile_begin(const char* name, hipStream_t s);
void profile_end(hipStream_t s);

// Number of compute units of the current device (cached per device).
int device_cu_count();

// ---------------------------------------------------------------- GEMM (bf16)
// Epilogue of the grouped MFMA GEMM.
enum GemmEpilogue {
  EPI_SWIGLU = 0,  // paired gate/up rows -> h = silu(g) * u, stored bf16
  EPI_F32 = 1,     // plain fp32 store
  EPI_ROUTER = 2,  // fp32 logits (+ bias), extra column -> gate logit
  EPI_BF16 = 3,    // plain store rounded once to bf16 (RNE)
  EPI_F16S = 4,    // fp16 scaled by a power of two per (row, 64 columns); 256-row pipelined kernel only
};

// EPI_F16S layout: value (r, c) is stored as fp16(y * 2^k) with k =
// scale_out[r * (ldo / 64) + c / 64], chosen from the segment's largest |y|
// so that it lands in [2^14, 2^15): fp16 keeps 11 significant bits (about 8x
// finer than bf16) with no overflow, and takes half the bytes of fp32.
constexpr int kF16SegCols = 64;

struct GemmArgs {
  const uint16_t* A;        // bf16 activations, rows of length K
  const int32_t* gather;    // A row of packed row p is gather[p] (NULL: row p)
  const int32_t* offsets;   // [G+1] packed row ranges of the groups (NULL: one group of M rows)
  int M;                    // total packed rows (upper bound of offsets[G])
  int a_rows;               // rows of A (bounds the DMA: reads past it return 0)
  int G;                    // groups (experts)
  const uint16_t* B;        // bf16 weights, per group `b_rows` rows of length K
  int64_t b_group_stride;   // elements between groups of B
  const uint16_t* b_extra;  // EPI_ROUTER: shared-expert gate vector [K] (NULL: none)
  int K;                    // reduction length, multiple of 64
  int N;                    // output columns (EPI_SWIGLU: I, the h width)
  int up_row0;              // EPI_SWIGLU: first up row inside a group (= I)
  void* out;                // EPI_SWIGLU: bf16 h; EPI_F32: f32; EPI_BF16: bf16; EPI_ROUTER: f32 logits
  int64_t ldo;              // output row stride in elements
  const float* bias;        // EPI_ROUTER: per-column bias or NULL
  float* extra_out;         // EPI_ROUTER: x . b_extra per row, when b_extra != NULL
  int32_t* scale_out;       // EPI_F16S: per (row, 64-column segment) exponents, [M, ldo / 64]
  int* tile_counter;        // large-group kernel: 8 zeroed ints (per-XCD tile grabs) or NULL
  float* partial;           // split-K scratch of grouped_gemm_partial_bytes() bytes, or NULL (no split)
  int ksplit;               // set by launch_grouped_gemm_bf16 (callers leave it 0)
  // Byte layout of a group of B: element (r, k) at b_row_pitch * r +
  // b_blk_pitch * (k / 32) + 2 * (k % 32).  Row-major [rows][K]: (2K, 64);
  // K-blocked [ceil(K/32)][rows][32] (kb32_bytes): (64, 64 * rows).  0: row-major.
  uint32_t b_row_pitch, b_blk_pitch;
  uint32_t b_group_bytes;   // bytes one group's B occupies (0: rows * 2K)
  // The same for A (rows not gathered): only the pipelined kernel reads a
  // K-blocked A, the h that its own gate/up epilogue wrote K-blocked.  0: row-major.
  uint32_t a_row_pitch, a_blk_pitch;
  int out_kblocked;         // EPI_SWIGLU on the pipelined kernel: h written K-blocked [I/32][M][32]
};

// Bytes of a K-blocked matrix of `rows` rows of length K: ceil(K/32) blocks of
// rows x 32 elements, the tail block zero-padded.
constexpr int kKBlock = 32;
inline size_t kb32_bytes(int64_t rows, int64_t K) { return (size_t)((K + kKBlock - 1) / kKBlock) * rows * kKBlock * 2; }
// True when the grouped GEMM for `a` (epilogue epi) runs the 8-wave pipelined
// kernel: the only kernel that reads a K-blocked A or writes a K-blocked h.
bool grouped_gemm_runs_pipe8(const GemmArgs& a, GemmEpilogue epi);

constexpr int kTileCounterInts = 8;
// True when the grouped GEMM for `a` runs the large-group kernel (which uses
// a.tile_counter when given).
bool grouped_gemm_uses_counter(const GemmArgs& a);
// True when `a` runs on a 256-row kernel (plain or pipelined), the kernels
// with the EPI_F16S epilogue.
bool grouped_gemm_has_f16s(const GemmArgs& a);
hipError_t launch_zero_ints(int* p, int n, hipStream_t s);

hipError_t launch_grouped_gemm_bf16(const GemmArgs& a, GemmEpilogue epi, hipStream_t s, const char* name);

// Split-K factor the bf16 grouped GEMM uses for a problem of M packed rows in
// G groups, N output columns and reduction length K (1: no split; the
// router epilogue never splits), and the bytes of fp32 partial sums it then
// needs in GemmArgs::partial (0 without a split).  Both depend on the shapes
// only.
int grouped_gemm_ksplit(int64_t M, int64_t G, bool grouped, int64_t N, int64_t K, GemmEpilogue epi);
size_t grouped_gemm_partial_bytes(int64_t M, int64_t G, bool grouped, int64_t N, int64_t K, GemmEpilogue epi);

// Router logits (+ shared-gate logit when gate != NULL) for T <= kRouterSmallT
// bf16 tokens, without the GEMM tiling.
constexpr int kRouterSmallT = 64;
hipError_t launch_router_small_t_bf16(const uint16_t* x, const uint16_t* wr, const float* bias, const uint16_t* gate,
                                      int T, int H, int E, float* logits, float* gate_logit, hipStream_t s);

// ---------------------------------------------------------------- fp32 path
hipError_t launch_router_logits_f32(const float* x, const float* wr, const float* bias,
                                    const float* gate, int T, int H, int E,
                                    float* logits, float* gate_logit, hipStream_t s);
hipError_t launch_ffn_gate_up_f32(const float* x, const int32_t* gather, const int32_t* offsets,
                                  const float* w13, int P, int H, int E, int I,
                                  float* h, hipStream_t s);
hipError_t launch_ffn_down_f32(const float* h, const int32_t* offsets, const float* w2,
                               int P, int H, int E, int I, float* y, hipStream_t s);

// ---------------------------------------------------------------- router top-k
// n_group > 1: group-limited selection (n_group <= 64 divides E; topk_group
// groups kept; k <= topk_group * E / n_group).
hipError_t launch_topk(const float* logits, int T, int E, int k, int renormalize,
                       int32_t* ids, float* weights, float* probs, hipStream_t s,
                       int n_group = 1, int topk_group = 1);

// ---------------------------------------------------------------- EP routing table
size_t ep_split_scratch_bytes(int64_t P);
hipError_t launch_ep_split(const int32_t* ids, const float* w, int T, int k, int64_t start, int64_t end,
                           int32_t* l_tok, int32_t* l_eid, float* l_w, int32_t* r_tok, int32_t* r_eid, float* r_w,
                           int32_t* counts, void* scratch, hipStream_t s);
// counts[r] / starts[r]: rows of rank r's experts [r*E/G, (r+1)*E/G) in the
// expert-major order and where they start; starts[G] = offsets[E] (starts may
// be NULL).
hipError_t launch_ep_rank_counts(const int32_t* offsets, int E, int G, int32_t* counts, int32_t* starts,
                                 hipStream_t s);

// ---------------------------------------------------------------- dispatch
constexpr int kDispatchSegment = 128;  // assignments per wave-segment
constexpr int kDispatchSmallP = 4096;  // up to this many assignments: one workgroup, all in LDS
size_t dispatch_scratch_bytes(int64_t P, int64_t E);
// Size of the library's fixed dispatch scratch (see dispatch_static_scratch).
constexpr size_t kDispatchStaticScratchBytes = (size_t)8 << 20;
// Device address of the current device's fixed dispatch scratch of
// kDispatchStaticScratchBytes (looked up on the device's first call, then
// kept): the workspace of moe_dispatch_plan_noalloc.
hipError_t dispatch_static_scratch(void** out);
// have_hist: the segment histogram is already in the scratch (written by
// launch_topk_hist), so the histogram launch is skipped.
hipError_t launch_dispatch(const int32_t* ids, const float* w, int T, int k, int E,
                           int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                           int32_t* packed_ids, float* packed_w, void* scratch, hipStream_t s,
                           int* zero_ints = nullptr, int n_zero = 0, bool have_hist = false);
// True when launch_dispatch(T, k) runs the segmented passes and k divides a
// segment, so that launch_topk_hist can stand in for the top-k and the
// histogram.
bool dispatch_takes_hist(int T, int k);
// The router's top-k (ids and weights, no probabilities) fused with the
// dispatch histogram written into `scratch` (the dispatch scratch of the same
// T, k, E).
hipError_t launch_topk_hist(const float* logits, int T, int E, int k, int renorm, int32_t* ids, float* weights,
                            void* scratch, hipStream_t s);

// Top-k of T <= kTopkDispatchSmallT tokens fused with the one-workgroup plan
// (T*k <= kDispatchSmallP): the same ids, weights and plan as launch_topk
// followed by launch_dispatch.
constexpr int kTopkDispatchSmallT = 64;
hipError_t launch_topk_dispatch_small(const float* logits, int T, int E, int k, int renorm, int32_t* ids,
                                      float* weights, int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                                      int32_t* packed_ids, hipStream_t s, int* zero_ints, int n_zero);

// ---------------------------------------------------------------- weights
// K-blocked copy of G row-major [R, K] bf16 matrices (K a multiple of 8):
// dst[g][b][r][i] = src[g][r][32 b + i], zero past K; kb32_bytes(R, K) per group.
hipError_t launch_pack_kb32(const void* src, void* dst, int64_t G, int64_t R, int64_t K, hipStream_t s);

// ---------------------------------------------------------------- combine
// y [P,H]: fp32 (y_format 0), bf16 (1), or fp16 with the EPI_F16S
// exponents y_scale [P, H/64] (2).  shared [T,H] (or NULL): fp32, or bf16
// when y_format is 1.
enum YFormat { Y_F32 = 0, Y_BF16 = 1, Y_F16S = 2 };
hipError_t launch_combine(const void* y, int y_format, const int32_t* y_scale, const int32_t* inv, const float* w,
                          const void* shared, const float* shared_gate_logit,
                          int T, int H, int k, int out_bf16, void* out, hipStream_t s);

}  // namespace moe
