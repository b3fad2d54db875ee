// C ABI of the MoE layer forward: host-side argument checks, workspace
// carving and launch sequencing.  Every check runs before anything is
// enqueued, so a failed call leaves the stream untouched.
//
// Pipeline ([DWDP README "Runtime Integration Layer"]):
//   router (logits GEMM -> top-k/softmax) -> dispatch plan (hist -> scan ->
//   scatter) -> [shared expert gate/up -> down] -> experts gate/up+SwiGLU ->
//   experts down -> combine.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "moe.h"
#include "moe_internal.h"

namespace {

thread_local std::string g_last_error;

moe_status fail(moe_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

moe_status succeed() {
  g_last_error.clear();
  return MOE_OK;
}

moe_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return succeed();
  return fail(MOE_ERR_HIP, std::string(where) + ": " + hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr size_t kAlign = 256;
size_t align_up(size_t n) { return (n + kAlign - 1) / kAlign * kAlign; }

size_t dtype_size(int dtype) { return dtype == MOE_DTYPE_BF16 ? 2 : 4; }

// Common size checks; returns MOE_OK or an error with the message set.
moe_status check_sizes(int64_t T, int64_t H, int64_t E, int64_t k, int dtype, bool need_h) {
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "num_tokens is negative");
  if (E < 1) return fail(MOE_ERR_INVALID_ARG, "num_experts must be >= 1");
  if (E > MOE_MAX_EXPERTS) return fail(MOE_ERR_UNSUPPORTED, "num_experts > 512 is not supported");
  if (k < 1 || k > E) return fail(MOE_ERR_INVALID_ARG, "top_k must be in [1, num_experts]");
  if (T * k >= (int64_t)1 << 31) return fail(MOE_ERR_UNSUPPORTED, "num_tokens * top_k must be < 2^31");
  if (dtype != MOE_DTYPE_F32 && dtype != MOE_DTYPE_BF16) return fail(MOE_ERR_INVALID_ARG, "dtype must be MOE_DTYPE_F32 or MOE_DTYPE_BF16");
  if (need_h) {
    if (H < 1) return fail(MOE_ERR_INVALID_ARG, "hidden_size must be >= 1");
    if (H % 8 != 0) return fail(MOE_ERR_UNSUPPORTED, "hidden_size must be a multiple of 8 (16-byte rows)");
  }
  return MOE_OK;
}

// The bf16 kernels address every operand with 32-bit byte offsets from a
// buffer base (one expert's weights, the activations, h).
// y_elt: bytes per element of the packed expert outputs [T*k, H] (0: none)
moe_status check_buffer_bytes(int64_t T, int64_t H, int64_t k, int64_t I, int dtype, int64_t y_elt = 0) {
  if (dtype != MOE_DTYPE_BF16) return MOE_OK;
  const int64_t lim = ((int64_t)1 << 31) - 1;
  if (T * H * 2 > lim || T * k * I * 2 > lim || 2 * I * H * 2 > lim || T * k * H * y_elt > lim)
    return fail(MOE_ERR_UNSUPPORTED, "a bf16-layer operand exceeds 2 GiB (32-bit buffer offsets)");
  return MOE_OK;
}

moe_status check_inter(int64_t I, int dtype, const char* name) {
  if (I < 1) return fail(MOE_ERR_INVALID_ARG, std::string(name) + " must be >= 1");
  if (dtype == MOE_DTYPE_BF16 && I % 16 != 0) return fail(MOE_ERR_UNSUPPORTED, std::string("bf16 needs ") + name + " % 16 == 0");
  if (dtype == MOE_DTYPE_F32 && I % 16 != 0) return fail(MOE_ERR_UNSUPPORTED, std::string("f32 needs ") + name + " % 16 == 0");
  return MOE_OK;
}

// One expert's K-blocked w13 [2I, H] and w2 [H, I] must each stay under 2 GiB
// (32-bit buffer offsets).
moe_status check_packed_bytes(int64_t H, int64_t I) {
  const size_t lim = ((size_t)1 << 31) - 1;
  if (moe::kb32_bytes(2 * I, H) > lim || moe::kb32_bytes(H, I) > lim)
    return fail(MOE_ERR_UNSUPPORTED, "one expert's packed weights exceed 2 GiB (32-bit buffer offsets)");
  return MOE_OK;
}

#define REQUIRE_PTR(p)                                                       \
  do {                                                                       \
    if ((p) == nullptr) return fail(MOE_ERR_INVALID_ARG, #p " is NULL");     \
  } while (0)
#define REQUIRE_ALIGNED(p)                                                              \
  do {                                                                                  \
    if ((p) != nullptr && !aligned16(p))                                                \
      return fail(MOE_ERR_UNSUPPORTED, #p " is not 16-byte aligned");                   \
  } while (0)
#define RETURN_IF_ERR(x)              \
  do {                                \
    moe_status _st = (x);             \
    if (_st != MOE_OK) return _st;    \
  } while (0)

// -------------------------------------------------------------- workspace
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <class T>
  T* take(size_t count) {
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += align_up(count * sizeof(T));
    return p;
  }
};

struct ForwardLayout {
  float* logits;
  float* gate_logit;
  int32_t* ids;
  float* weights;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
  int32_t* inv;
  int32_t* packed_ids;
  void* dispatch_scratch;
  void* h;
  float* y;  // packed expert outputs, a P*H*4-byte slot: fp32, or fp16 + per-(row, 64 columns) exponents
  void* hs;
  float* ys;
  int* counters;  // tile counters of the four grouped GEMMs (routed, shared)
  float* partial;         // split-K partial sums of the routed GEMMs (they run in order)
  float* partial_shared;  // same for the shared expert, which may run concurrently
  size_t bytes;
};

// Split-K scratch of one FFN (gate/up then down) over P rows in E groups.
size_t ffn_pair_partial_bytes(int64_t P, int64_t H, int64_t E, bool grouped, int64_t I, int dtype) {
  if (dtype != MOE_DTYPE_BF16 || P <= 0 || I <= 0) return 0;
  return std::max(moe::grouped_gemm_partial_bytes(P, E, grouped, I, H, moe::EPI_SWIGLU),
                  moe::grouped_gemm_partial_bytes(P, E, grouped, H, I, moe::EPI_F32));
}


ForwardLayout carve_forward(void* ws, int64_t T, int64_t H, int64_t E, int64_t k, int64_t I, int64_t Is, int dtype) {
  const int64_t P = T * k;
  Carver c(ws);
  ForwardLayout L;
  L.logits = c.take<float>((size_t)(T * E));
  L.gate_logit = c.take<float>((size_t)(Is > 0 ? T : 0));
  L.ids = c.take<int32_t>((size_t)P);
  L.weights = c.take<float>((size_t)P);
  L.counts = c.take<int32_t>((size_t)E);
  L.offsets = c.take<int32_t>((size_t)E + 1);
  L.perm = c.take<int32_t>((size_t)P);
  L.inv = c.take<int32_t>((size_t)P);
  L.packed_ids = c.take<int32_t>((size_t)P);
  L.dispatch_scratch = c.take<char>(moe::dispatch_scratch_bytes(P, E));
  L.h = c.take<char>((size_t)(P * I) * dtype_size(dtype));
  L.y = c.take<float>((size_t)(P * H));
  L.hs = c.take<char>((size_t)(Is > 0 ? T * Is : 0) * dtype_size(dtype));
  L.ys = c.take<float>((size_t)(Is > 0 ? T * H : 0));
  L.counters = c.take<int>(4 * moe::kTileCounterInts);
  L.partial = c.take<float>(ffn_pair_partial_bytes(P, H, E, true, I, dtype) / sizeof(float));
  L.partial_shared = c.take<float>((Is > 0 ? ffn_pair_partial_bytes(T, H, 1, false, Is, dtype) : 0) / sizeof(float));
  L.bytes = c.off;
  return L;
}

// -------------------------------------------------------------- stage launches
moe::GemmArgs gemm_args() {
  moe::GemmArgs a;
  std::memset(&a, 0, sizeof(a));
  return a;
}

// Router logits, then (with_topk) the top-k ids and weights.
hipError_t run_router(const void* x, const void* wr, const float* bias, const void* gate, int T, int H, int E, int k,
                      int renorm, int dtype, float* logits, float* probs, int32_t* ids, float* weights,
                      float* gate_logit, hipStream_t s, bool with_topk = true) {
  hipError_t e;
  if (dtype == MOE_DTYPE_BF16 && T <= moe::kRouterSmallT) {
    e = moe::launch_router_small_t_bf16(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(wr), bias,
                                        static_cast<const uint16_t*>(gate), T, H, E, logits, gate_logit, s);
  } else if (dtype == MOE_DTYPE_BF16) {
    moe::GemmArgs a = gemm_args();
    a.A = static_cast<const uint16_t*>(x);
    a.M = T;
    a.a_rows = T;
    a.G = 1;
    a.B = static_cast<const uint16_t*>(wr);
    a.b_group_stride = 0;
    a.b_extra = static_cast<const uint16_t*>(gate);
    a.K = H;
    a.N = E;
    a.out = logits;
    a.ldo = E;
    a.bias = bias;
    a.extra_out = gate_logit;
    e = moe::launch_grouped_gemm_bf16(a, moe::EPI_ROUTER, s, "router_logits_bf16");
  } else {
    e = moe::launch_router_logits_f32(static_cast<const float*>(x), static_cast<const float*>(wr), bias,
                                      static_cast<const float*>(gate), T, H, E, logits, gate_logit, s);
  }
  if (e != hipSuccess || !with_topk) return e;
  return moe::launch_topk(logits, T, E, k, renorm, ids, weights, probs, s);
}

// counters: 2 * kTileCounterInts zeroed ints (gate/up, down) or NULL.  y is
// bf16 when y_dtype is MOE_DTYPE_BF16 (bf16 layers only), else fp32.
// y_format (moe::YFormat, bf16 layers only for Y_BF16 and Y_F16S): fp32 y,
// bf16 y, or fp16 y with the exponents y_scale [P, H/64].
// packed: w13 / w2 K-blocked (moe_pack_weights), bf16 layers only.
hipError_t run_ffn(const void* x, const int32_t* gather, const int32_t* offsets, const void* w13, const void* w2,
                   int T_rows, int P, int H, int E, int I, int dtype, bool packed, void* h, void* y, int y_format,
                   int32_t* y_scale, hipStream_t s, bool shared, int* counters, float* partial) {
  hipError_t e;
  if (dtype == MOE_DTYPE_BF16) {
    moe::GemmArgs a = gemm_args();
    a.A = static_cast<const uint16_t*>(x);
    a.gather = gather;
    a.offsets = offsets;
    a.M = P;
    a.a_rows = T_rows;
    a.G = E;
    a.B = static_cast<const uint16_t*>(w13);
    a.b_group_stride = (int64_t)2 * I * H;
    a.K = H;
    a.N = I;
    a.up_row0 = I;
    a.out = h;
    a.ldo = I;
    a.tile_counter = counters;
    a.partial = partial;
    if (packed) {
      a.b_group_bytes = (uint32_t)moe::kb32_bytes(2 * I, H);
      a.b_group_stride = (int64_t)a.b_group_bytes / 2;
      a.b_row_pitch = 64;
      a.b_blk_pitch = 64u * (uint32_t)(2 * I);
    }
    moe::GemmArgs b = gemm_args();
    b.A = static_cast<const uint16_t*>(h);
    b.gather = nullptr;
    b.offsets = offsets;
    b.M = P;
    b.a_rows = P;
    b.G = E;
    b.B = static_cast<const uint16_t*>(w2);
    b.b_group_stride = (int64_t)H * I;
    b.K = I;
    b.N = H;
    b.out = y;
    b.ldo = H;
    b.tile_counter = counters ? counters + moe::kTileCounterInts : nullptr;
    b.partial = partial;
    b.scale_out = y_scale;
    const moe::GemmEpilogue epi = (y_format == moe::Y_BF16)   ? moe::EPI_BF16
                                  : (y_format == moe::Y_F16S) ? moe::EPI_F16S
                                                              : moe::EPI_F32;
    if (packed) {
      b.b_group_bytes = (uint32_t)moe::kb32_bytes(H, I);
      b.b_group_stride = (int64_t)b.b_group_bytes / 2;
      b.b_row_pitch = 64;
      b.b_blk_pitch = 64u * (uint32_t)H;
    }
    // h K-blocked ([I/32][P][32]) when both GEMMs run the pipelined kernel:
    // the down projection then fetches whole 128-byte lines of it
    if (I % moe::kKBlock == 0 && moe::grouped_gemm_runs_pipe8(a, moe::EPI_SWIGLU) &&
        moe::grouped_gemm_runs_pipe8(b, epi)) {
      a.out_kblocked = 1;
      b.a_row_pitch = 64;
      b.a_blk_pitch = 64u * (uint32_t)P;
    }
    e = moe::launch_grouped_gemm_bf16(a, moe::EPI_SWIGLU, s, shared ? "shared_gate_up_bf16" : "ffn_gate_up_bf16");
    if (e != hipSuccess) return e;
    return moe::launch_grouped_gemm_bf16(b, epi, s, shared ? "shared_down_bf16" : "ffn_down_bf16");
  }
  e = moe::launch_ffn_gate_up_f32(static_cast<const float*>(x), gather, offsets, static_cast<const float*>(w13), P,
                                  H, E, I, static_cast<float*>(h), s);
  if (e != hipSuccess) return e;
  return moe::launch_ffn_down_f32(static_cast<const float*>(h), offsets, static_cast<const float*>(w2), P, H, E, I,
                                  static_cast<float*>(y), s);
}

// -------------------------------------------------------------- profiling
struct ProfRecord {
  const char* name;
  hipEvent_t start;
  hipEvent_t stop;
};
// Second stream for the shared expert, which depends only on the input and
// runs concurrently with the routed experts: one per (device, caller stream),
// created on first use, default priority, joined back through its own pair of
// events (a pattern that HIP graph capture records as a fork and a join).
// Keying by the caller's stream keeps independent caller streams independent:
// their shared experts neither queue behind each other on one aux stream nor
// share an event, and a graph capture on one caller stream never sees another
// stream's work.  A slot's own mutex covers the enqueue of one forward (its
// events are re-recorded by every forward on that caller stream); the table
// lock is held only for the lookup.
struct AuxSlot {
  int dev = -1;
  hipStream_t caller = nullptr;
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr;
  hipEvent_t join = nullptr;
  bool ok = false;
  std::mutex mu;
};
constexpr int kMaxAuxSlots = 256;
std::mutex g_aux_table_mu;
AuxSlot g_aux_slots[kMaxAuxSlots];
int g_aux_used = 0;

// The aux slot of `caller` on the current device, or nullptr when there is
// none and none can be made: the caller then runs the shared expert on its own
// stream.  A slot is never created while `caller` is being captured into a
// graph (creating streams and events there could invalidate the capture); a
// caller that wants the fork inside a captured graph runs one forward on the
// capture stream before capturing.
AuxSlot* aux_slot(hipStream_t caller) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lk(g_aux_table_mu);
  for (int i = 0; i < g_aux_used; ++i)
    if (g_aux_slots[i].dev == dev && g_aux_slots[i].caller == caller)
      return g_aux_slots[i].ok ? &g_aux_slots[i] : nullptr;
  if (g_aux_used == kMaxAuxSlots) return nullptr;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(caller, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone) return nullptr;
  AuxSlot& a = g_aux_slots[g_aux_used++];
  a.dev = dev;
  a.caller = caller;
  // The join only orders device work after device work (the shared
  // expert's kernels before the combine), so it needs no system-scope
  // fence; the fork keeps it, because the aux stream's first reads may
  // follow a host-to-device copy on the caller's stream.
  a.ok = hipStreamCreateWithFlags(&a.stream, hipStreamNonBlocking) == hipSuccess &&
         hipEventCreateWithFlags(&a.fork, hipEventDisableTiming) == hipSuccess &&
         hipEventCreateWithFlags(&a.join, hipEventDisableTiming | hipEventDisableSystemFence) == hipSuccess;
  return a.ok ? &a : nullptr;
}

// Kernel timing state.  g_prof_on is read without the lock first, so that a
// launch with profiling off takes no process-wide lock.
std::mutex g_prof_mu;
std::atomic<bool> g_prof_on{false};
std::vector<ProfRecord> g_prof;
thread_local int g_prof_open = -1;

}  // namespace

namespace moe {

void profile_begin(const char* name, hipStream_t s) {
  g_prof_open = -1;
  if (!g_prof_on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof_on.load(std::memory_order_relaxed)) return;
  ProfRecord r{name, nullptr, nullptr};
  if (hipEventCreate(&r.start) != hipSuccess) return;
  if (hipEventCreate(&r.stop) != hipSuccess) {
    (void)hipEventDestroy(r.start);
    return;
  }
  (void)hipEventRecord(r.start, s);
  g_prof.push_back(r);
  g_prof_open = (int)g_prof.size() - 1;
}

void profile_end(hipStream_t s) {
  if (g_prof_open < 0) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (g_prof_open < 0 || g_prof_open >= (int)g_prof.size()) return;
  (void)hipEventRecord(g_prof[g_prof_open].stop, s);
  g_prof_open = -1;
}

int device_cu_count() {
  static std::atomic<int> cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace moe

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

const char* moe_last_error_message(void) { return g_last_error.c_str(); }

moe_status moe_router_topk(const void* hidden_states, const void* router_weight, const float* router_bias,
                           const void* shared_gate, int64_t num_tokens, int64_t hidden_size, int64_t num_experts,
                           int64_t top_k, int renormalize, int dtype, float* router_logits, float* routing_probs,
                           int32_t* topk_ids, float* topk_weights, float* shared_gate_logit, void* stream) {
  if (dtype == MOE_DTYPE_BF16_KB32) dtype = MOE_DTYPE_BF16;  // the router weight is row-major either way
  RETURN_IF_ERR(check_sizes(num_tokens, hidden_size, num_experts, top_k, dtype, true));
  RETURN_IF_ERR(check_buffer_bytes(num_tokens, hidden_size, 1, 1, dtype));
  if (num_tokens == 0) return succeed();
  REQUIRE_PTR(hidden_states);
  REQUIRE_PTR(router_weight);
  REQUIRE_PTR(topk_ids);
  REQUIRE_PTR(topk_weights);
  REQUIRE_PTR(router_logits);
  if ((shared_gate == nullptr) != (shared_gate_logit == nullptr))
    return fail(MOE_ERR_INVALID_ARG, "shared_gate and shared_gate_logit must be given together");
  REQUIRE_ALIGNED(hidden_states);
  REQUIRE_ALIGNED(router_weight);
  REQUIRE_ALIGNED(shared_gate);
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(run_router(hidden_states, router_weight, router_bias, shared_gate, (int)num_tokens,
                               (int)hidden_size, (int)num_experts, (int)top_k, renormalize ? 1 : 0, dtype,
                               router_logits, routing_probs, topk_ids, topk_weights, shared_gate_logit, s),
                    "moe_router_topk");
}

size_t moe_dispatch_workspace_size(int64_t num_tokens, int64_t top_k, int64_t num_experts) {
  if (num_tokens < 0 || top_k < 1 || num_experts < 1) return 0;
  return align_up(moe::dispatch_scratch_bytes(num_tokens * top_k, num_experts));
}

moe_status moe_router_topk_grouped(const void* hidden_states, const void* router_weight, const float* router_bias,
                                   int64_t num_tokens, int64_t hidden_size, int64_t num_experts, int64_t top_k,
                                   int64_t n_group, int64_t topk_group, int renormalize, int dtype,
                                   float* router_logits, float* routing_probs, int32_t* topk_ids, float* topk_weights,
                                   void* stream) {
  if (dtype == MOE_DTYPE_BF16_KB32) dtype = MOE_DTYPE_BF16;  // the router weight is row-major either way
  RETURN_IF_ERR(check_sizes(num_tokens, hidden_size, num_experts, top_k, dtype, true));
  RETURN_IF_ERR(check_buffer_bytes(num_tokens, hidden_size, 1, 1, dtype));
  if (n_group < 1 || n_group > 64) return fail(MOE_ERR_INVALID_ARG, "n_group must be in [1, 64]");
  if (num_experts % n_group != 0) return fail(MOE_ERR_INVALID_ARG, "n_group must divide num_experts");
  if (topk_group < 1 || topk_group > n_group) return fail(MOE_ERR_INVALID_ARG, "topk_group must be in [1, n_group]");
  if (top_k > topk_group * (num_experts / n_group))
    return fail(MOE_ERR_INVALID_ARG, "top_k exceeds the experts of topk_group groups");
  if (num_tokens == 0) return succeed();
  REQUIRE_PTR(hidden_states);
  REQUIRE_PTR(router_weight);
  REQUIRE_PTR(topk_ids);
  REQUIRE_PTR(topk_weights);
  REQUIRE_PTR(router_logits);
  REQUIRE_ALIGNED(hidden_states);
  REQUIRE_ALIGNED(router_weight);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int T = (int)num_tokens, E = (int)num_experts, k = (int)top_k;
  hipError_t e = run_router(hidden_states, router_weight, router_bias, nullptr, T, (int)hidden_size, E, k,
                            renormalize ? 1 : 0, dtype, router_logits, nullptr, nullptr, nullptr, nullptr, s, false);
  if (e == hipSuccess)
    e = moe::launch_topk(router_logits, T, E, k, renormalize ? 1 : 0, topk_ids, topk_weights, routing_probs, s,
                         (int)n_group, (int)topk_group);
  return hip_status(e, "moe_router_topk_grouped");
}

moe_status moe_dispatch_plan(const int32_t* topk_ids, const float* topk_weights, int64_t num_tokens, int64_t top_k,
                             int64_t num_experts, int32_t* expert_counts, int32_t* expert_offsets,
                             int32_t* token_permutation, int32_t* inverse_permutation, int32_t* packed_token_indices,
                             float* packed_routing_weights, void* workspace, size_t workspace_bytes, void* stream) {
  RETURN_IF_ERR(check_sizes(num_tokens, 1, num_experts, top_k, MOE_DTYPE_F32, false));
  if (num_tokens == 0) return succeed();
  REQUIRE_PTR(topk_ids);
  REQUIRE_PTR(expert_counts);
  REQUIRE_PTR(expert_offsets);
  REQUIRE_PTR(token_permutation);
  REQUIRE_PTR(inverse_permutation);
  REQUIRE_PTR(packed_token_indices);
  if ((topk_weights == nullptr) != (packed_routing_weights == nullptr))
    return fail(MOE_ERR_INVALID_ARG, "topk_weights and packed_routing_weights must be given together");
  const size_t need = moe_dispatch_workspace_size(num_tokens, top_k, num_experts);
  if (workspace == nullptr || workspace_bytes < need) return fail(MOE_ERR_WORKSPACE, "workspace too small");
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(moe::launch_dispatch(topk_ids, topk_weights, (int)num_tokens, (int)top_k, (int)num_experts,
                                         expert_counts, expert_offsets, token_permutation, inverse_permutation,
                                         packed_token_indices, packed_routing_weights, workspace, s),
                    "moe_dispatch_plan");
}

size_t moe_dispatch_noalloc_max_workspace(void) { return moe::kDispatchStaticScratchBytes; }

moe_status moe_dispatch_plan_noalloc(const int32_t* topk_ids, const float* topk_weights, int64_t num_tokens,
                                     int64_t top_k, int64_t num_experts, int32_t* expert_counts,
                                     int32_t* expert_offsets, int32_t* token_permutation,
                                     int32_t* inverse_permutation, int32_t* packed_token_indices,
                                     float* packed_routing_weights, void* stream) {
  RETURN_IF_ERR(check_sizes(num_tokens, 1, num_experts, top_k, MOE_DTYPE_F32, false));
  if (num_tokens == 0) return succeed();
  REQUIRE_PTR(topk_ids);
  REQUIRE_PTR(expert_counts);
  REQUIRE_PTR(expert_offsets);
  REQUIRE_PTR(token_permutation);
  REQUIRE_PTR(inverse_permutation);
  REQUIRE_PTR(packed_token_indices);
  if ((topk_weights == nullptr) != (packed_routing_weights == nullptr))
    return fail(MOE_ERR_INVALID_ARG, "topk_weights and packed_routing_weights must be given together");
  const size_t need = moe_dispatch_workspace_size(num_tokens, top_k, num_experts);
  if (need > moe::kDispatchStaticScratchBytes)
    return fail(MOE_ERR_UNSUPPORTED, "num_tokens * top_k and num_experts need " + std::to_string(need) +
                                         " bytes of dispatch scratch, above the fixed " +
                                         std::to_string(moe::kDispatchStaticScratchBytes));
  void* scratch = nullptr;
  hipError_t e = moe::dispatch_static_scratch(&scratch);
  if (e != hipSuccess) return hip_status(e, "moe_dispatch_plan_noalloc(scratch)");
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(moe::launch_dispatch(topk_ids, topk_weights, (int)num_tokens, (int)top_k, (int)num_experts,
                                         expert_counts, expert_offsets, token_permutation, inverse_permutation,
                                         packed_token_indices, packed_routing_weights, scratch, s),
                    "moe_dispatch_plan_noalloc");
}

size_t moe_ep_routing_table_workspace_size(int64_t num_tokens, int64_t top_k) {
  if (num_tokens < 0 || top_k < 1) return 0;
  return align_up(moe::ep_split_scratch_bytes(num_tokens * top_k)) + kAlign;
}

moe_status moe_ep_routing_table(const int32_t* gate_indices, int64_t gate_indices_len, const float* gate_weights,
                                int64_t gate_weights_len, int64_t num_tokens, int64_t top_k,
                                int64_t local_expert_start, int64_t local_expert_end,
                                int32_t* local_token_indices, int32_t* local_expert_ids, float* local_weights,
                                int32_t* remote_token_indices, int32_t* remote_expert_ids, float* remote_weights,
                                int32_t* counts, void* workspace, size_t workspace_bytes, void* stream) {
  if (num_tokens < 0) return fail(MOE_ERR_INVALID_ARG, "num_tokens is negative");
  if (top_k < 1) return fail(MOE_ERR_INVALID_ARG, "top_k must be >= 1");
  if (num_tokens * top_k >= (int64_t)1 << 31) return fail(MOE_ERR_UNSUPPORTED, "num_tokens * top_k must be < 2^31");
  if (local_expert_start < 0 || local_expert_end < 0)
    return fail(MOE_ERR_INVALID_ARG, "local expert range bounds must be >= 0");
  const int64_t total = num_tokens * top_k;
  if (gate_indices_len != total) return fail(MOE_ERR_INVALID_ARG, "gate_indices length mismatch");
  if (gate_weights_len != total) return fail(MOE_ERR_INVALID_ARG, "gate_weights length mismatch");
  REQUIRE_PTR(counts);
  if (total > 0) {
    REQUIRE_PTR(gate_indices);
    REQUIRE_PTR(gate_weights);
    REQUIRE_PTR(local_token_indices);
    REQUIRE_PTR(local_expert_ids);
    REQUIRE_PTR(local_weights);
    REQUIRE_PTR(remote_token_indices);
    REQUIRE_PTR(remote_expert_ids);
    REQUIRE_PTR(remote_weights);
  }
  const size_t need = moe_ep_routing_table_workspace_size(num_tokens, top_k);
  if (workspace == nullptr || workspace_bytes < need) return fail(MOE_ERR_WORKSPACE, "workspace too small");
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(moe::launch_ep_split(gate_indices, gate_weights, (int)num_tokens, (int)top_k, local_expert_start,
                                         local_expert_end, local_token_indices, local_expert_ids, local_weights,
                                         remote_token_indices, remote_expert_ids, remote_weights, counts, workspace,
                                         s),
                    "moe_ep_routing_table");
}

moe_status moe_tp_load_expert(const void* src, int proj, int64_t hidden_size, int64_t intermediate_size,
                              int tp_size, int tp_rank, int64_t expert, int64_t local_experts, int dtype,
                              void* dst, void* stream) {
  REQUIRE_PTR(src);
  REQUIRE_PTR(dst);
  if (dtype == MOE_DTYPE_BF16_KB32)
    return fail(MOE_ERR_INVALID_ARG, "the loader writes row-major weights: load with MOE_DTYPE_BF16, then moe_pack_weights");
  if (dtype != MOE_DTYPE_F32 && dtype != MOE_DTYPE_BF16) return fail(MOE_ERR_INVALID_ARG, "unknown dtype");
  if (proj != MOE_PROJ_GATE && proj != MOE_PROJ_UP && proj != MOE_PROJ_DOWN)
    return fail(MOE_ERR_INVALID_ARG, "unknown proj");
  if (hidden_size < 1 || intermediate_size < 1 || local_experts < 1)
    return fail(MOE_ERR_INVALID_ARG, "hidden_size, intermediate_size and local_experts must be >= 1");
  if (tp_size < 1 || tp_rank < 0 || tp_rank >= tp_size)
    return fail(MOE_ERR_INVALID_ARG, "tp_rank must lie in [0, tp_size)");
  if (intermediate_size % tp_size != 0) return fail(MOE_ERR_INVALID_ARG, "tp_size must divide intermediate_size");
  if (expert < 0 || expert >= local_experts) return fail(MOE_ERR_INVALID_ARG, "expert must lie in [0, local_experts)");
  const size_t es = dtype_size(dtype);
  const size_t H = (size_t)hidden_size, I = (size_t)intermediate_size, Ip = I / (size_t)tp_size;
  const size_t r = (size_t)tp_rank, e = (size_t)expert;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const char* sb = static_cast<const char*>(src);
  char* db = static_cast<char*>(dst);
  if (proj == MOE_PROJ_DOWN)  // H rows of Ip columns, taken from rows of I
    return hip_status(hipMemcpy2DAsync(db + e * H * Ip * es, Ip * es, sb + r * Ip * es, I * es, Ip * es, H,
                                       hipMemcpyDefault, s),
                      "moe_tp_load_expert");
  // Ip whole rows of H: one contiguous block on both sides
  const size_t member = (proj == MOE_PROJ_UP) ? 1 : 0;
  return hip_status(hipMemcpyAsync(db + (e * 2 * Ip + member * Ip) * H * es, sb + r * Ip * H * es, Ip * H * es,
                                   hipMemcpyDefault, s),
                    "moe_tp_load_expert");
}

size_t moe_packed_weights_size(int64_t groups, int64_t rows, int64_t k) {
  if (groups < 1 || rows < 1 || k < 1) return 0;
  return (size_t)groups * moe::kb32_bytes(rows, k);
}

moe_status moe_pack_weights(const void* src, void* dst, int64_t groups, int64_t rows, int64_t k, void* stream) {
  REQUIRE_PTR(src);
  REQUIRE_PTR(dst);
  if (groups < 1 || rows < 1 || k < 1) return fail(MOE_ERR_INVALID_ARG, "groups, rows and k must be >= 1");
  if (k % 8 != 0) return fail(MOE_ERR_UNSUPPORTED, "k must be a multiple of 8 (16-byte rows)");
  if (moe::kb32_bytes(rows, k) > ((size_t)1 << 31) - 1)
    return fail(MOE_ERR_UNSUPPORTED, "one group's packed weights exceed 2 GiB (32-bit buffer offsets)");
  REQUIRE_ALIGNED(src);
  REQUIRE_ALIGNED(dst);
  const char* s0 = static_cast<const char*>(src);
  const char* d0 = static_cast<const char*>(dst);
  const size_t src_bytes = (size_t)groups * rows * k * 2, dst_bytes = moe_packed_weights_size(groups, rows, k);
  if (s0 < d0 + dst_bytes && d0 < s0 + src_bytes) return fail(MOE_ERR_INVALID_ARG, "src and dst overlap");
  return hip_status(moe::launch_pack_kb32(src, dst, groups, rows, k, static_cast<hipStream_t>(stream)),
                    "moe_pack_weights");
}

moe_status moe_ep_rank_counts(const int32_t* expert_offsets, int64_t num_experts, int64_t num_ranks,
                              int32_t* send_counts, int32_t* send_offsets, void* stream) {
  REQUIRE_PTR(expert_offsets);
  REQUIRE_PTR(send_counts);
  if (num_experts < 1 || num_experts > MOE_MAX_EXPERTS)
    return fail(MOE_ERR_INVALID_ARG, "num_experts must be in [1, 512]");
  if (num_ranks < 1 || num_ranks > num_experts) return fail(MOE_ERR_INVALID_ARG, "num_ranks must be in [1, num_experts]");
  return hip_status(moe::launch_ep_rank_counts(expert_offsets, (int)num_experts, (int)num_ranks, send_counts,
                                               send_offsets, static_cast<hipStream_t>(stream)),
                    "moe_ep_rank_counts");
}

// Split-K scratch of moe_grouped_ffn; with one expert the offsets may be
// absent (one ungrouped block) or present, and the two can split differently.
size_t grouped_ffn_partial_bytes(int64_t P, int64_t H, int64_t E, int64_t I, int dtype) {
  size_t b = ffn_pair_partial_bytes(P, H, E, true, I, dtype);
  if (E == 1) b = std::max(b, ffn_pair_partial_bytes(P, H, 1, false, I, dtype));
  return b;
}

size_t moe_grouped_ffn_workspace_size(int64_t num_tokens, int64_t hidden_size, int64_t top_k, int64_t num_experts,
                                      int64_t intermediate_size, int dtype) {
  if (dtype == MOE_DTYPE_BF16_KB32) dtype = MOE_DTYPE_BF16;
  if (num_tokens < 0 || hidden_size < 1 || top_k < 1 || num_experts < 1 || intermediate_size < 1) return 0;
  const int64_t P = num_tokens * top_k;
  // tile counters of the two GEMMs, h, then the split-K partial sums
  return kAlign + align_up((size_t)(P * intermediate_size) * dtype_size(dtype)) +
         align_up(grouped_ffn_partial_bytes(P, hidden_size, num_experts, intermediate_size, dtype));
}

moe_status moe_grouped_ffn(const void* hidden_states, const int32_t* packed_token_indices,
                           const int32_t* expert_offsets, const void* w13, const void* w2, int64_t num_tokens,
                           int64_t hidden_size, int64_t num_experts, int64_t top_k, int64_t intermediate_size,
                           int dtype, int expert_out_dtype, void* packed_expert_outputs, void* workspace,
                           size_t workspace_bytes, void* stream) {
  const bool packed = dtype == MOE_DTYPE_BF16_KB32;
  if (packed) dtype = MOE_DTYPE_BF16;
  RETURN_IF_ERR(check_sizes(num_tokens, hidden_size, num_experts, top_k, dtype, true));
  RETURN_IF_ERR(check_inter(intermediate_size, dtype, "intermediate_size"));
  if (packed) RETURN_IF_ERR(check_packed_bytes(hidden_size, intermediate_size));
  if (expert_out_dtype != MOE_DTYPE_F32 && expert_out_dtype != MOE_DTYPE_BF16)
    return fail(MOE_ERR_INVALID_ARG, "expert_out_dtype must be MOE_DTYPE_F32 or MOE_DTYPE_BF16");
  if (expert_out_dtype == MOE_DTYPE_BF16 && dtype != MOE_DTYPE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "bf16 expert outputs need a bf16 layer");
  RETURN_IF_ERR(check_buffer_bytes(num_tokens, hidden_size, top_k, intermediate_size, dtype,
                                   dtype_size(expert_out_dtype)));
  if (num_tokens == 0) return succeed();
  REQUIRE_PTR(hidden_states);
  REQUIRE_PTR(w13);
  REQUIRE_PTR(w2);
  REQUIRE_PTR(packed_expert_outputs);
  if (expert_offsets == nullptr && num_experts != 1)
    return fail(MOE_ERR_INVALID_ARG, "expert_offsets may be NULL only with num_experts == 1");
  if (packed_token_indices == nullptr && top_k != 1)
    return fail(MOE_ERR_INVALID_ARG, "packed_token_indices may be NULL only with top_k == 1");
  REQUIRE_ALIGNED(hidden_states);
  REQUIRE_ALIGNED(w13);
  REQUIRE_ALIGNED(w2);
  REQUIRE_ALIGNED(packed_expert_outputs);
  const size_t need =
      moe_grouped_ffn_workspace_size(num_tokens, hidden_size, top_k, num_experts, intermediate_size, dtype);
  if (workspace == nullptr || workspace_bytes < need) return fail(MOE_ERR_WORKSPACE, "workspace too small");
  REQUIRE_ALIGNED(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int P = (int)(num_tokens * top_k);
  int* counters = static_cast<int*>(workspace);
  void* h = static_cast<char*>(workspace) + kAlign;
  const size_t part_bytes = grouped_ffn_partial_bytes(P, hidden_size, num_experts, intermediate_size, dtype);
  float* partial = part_bytes ? reinterpret_cast<float*>(static_cast<char*>(workspace) + kAlign +
                                                         align_up((size_t)P * intermediate_size * dtype_size(dtype)))
                              : nullptr;
  if (dtype == MOE_DTYPE_BF16) {
    hipError_t ez = moe::launch_zero_ints(counters, 2 * moe::kTileCounterInts, s);
    if (ez != hipSuccess) return hip_status(ez, "moe_grouped_ffn");
  }
  return hip_status(run_ffn(hidden_states, packed_token_indices, expert_offsets, w13, w2, (int)num_tokens, P,
                            (int)hidden_size, (int)num_experts, (int)intermediate_size, dtype, packed, h,
                            packed_expert_outputs, expert_out_dtype == MOE_DTYPE_BF16 ? moe::Y_BF16 : moe::Y_F32,
                            nullptr, s, false,
                            dtype == MOE_DTYPE_BF16 ? counters : nullptr,
                            partial),
                    "moe_grouped_ffn");
}

moe_status moe_combine(const void* packed_expert_outputs, const int32_t* inverse_permutation,
                       const float* topk_weights, const void* shared_output, const float* shared_gate_logit,
                       int64_t num_tokens, int64_t hidden_size, int64_t top_k, int expert_dtype, int out_dtype,
                       void* output, void* stream) {
  if (num_tokens < 0) return fail(MOE_ERR_INVALID_ARG, "num_tokens is negative");
  if (top_k < 1) return fail(MOE_ERR_INVALID_ARG, "top_k must be >= 1");
  if (hidden_size < 1) return fail(MOE_ERR_INVALID_ARG, "hidden_size must be >= 1");
  if (hidden_size % 8 != 0) return fail(MOE_ERR_UNSUPPORTED, "hidden_size % 8 != 0");
  if (expert_dtype != MOE_DTYPE_F32 && expert_dtype != MOE_DTYPE_BF16)
    return fail(MOE_ERR_INVALID_ARG, "expert_dtype must be MOE_DTYPE_F32 or MOE_DTYPE_BF16");
  if (out_dtype != MOE_DTYPE_F32 && out_dtype != MOE_DTYPE_BF16)
    return fail(MOE_ERR_INVALID_ARG, "out_dtype must be MOE_DTYPE_F32 or MOE_DTYPE_BF16");
  if (num_tokens * top_k >= (int64_t)1 << 31) return fail(MOE_ERR_UNSUPPORTED, "num_tokens * top_k must be < 2^31");
  if (num_tokens == 0) return succeed();
  REQUIRE_PTR(packed_expert_outputs);
  REQUIRE_PTR(inverse_permutation);
  REQUIRE_PTR(topk_weights);
  REQUIRE_PTR(output);
  if (shared_gate_logit != nullptr && shared_output == nullptr)
    return fail(MOE_ERR_INVALID_ARG, "shared_gate_logit given without shared_output");
  REQUIRE_ALIGNED(packed_expert_outputs);
  REQUIRE_ALIGNED(shared_output);
  REQUIRE_ALIGNED(output);
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(moe::launch_combine(packed_expert_outputs,
                                        expert_dtype == MOE_DTYPE_BF16 ? moe::Y_BF16 : moe::Y_F32, nullptr,
                                        inverse_permutation,
                                        topk_weights, shared_output, shared_gate_logit, (int)num_tokens,
                                        (int)hidden_size, (int)top_k, out_dtype == MOE_DTYPE_BF16, output, s),
                    "moe_combine");
}

size_t moe_forward_workspace_size(int64_t num_tokens, int64_t hidden_size, int64_t num_experts, int64_t top_k,
                                  int64_t intermediate_size, int64_t shared_intermediate_size, int dtype) {
  if (dtype == MOE_DTYPE_BF16_KB32) dtype = MOE_DTYPE_BF16;
  if (num_tokens < 0 || hidden_size < 1 || num_experts < 1 || top_k < 1 || intermediate_size < 1 ||
      shared_intermediate_size < 0)
    return 0;
  return carve_forward(nullptr, num_tokens, hidden_size, num_experts, top_k, intermediate_size,
                       shared_intermediate_size, dtype)
      .bytes;
}

// True when the forward's down projection stores the packed expert outputs as
// fp16 + one exponent per 64 columns (bf16 layers on the 256-row kernels,
// H a multiple of 64); otherwise they are fp32.  Depends on the shapes only.
static bool forward_y_f16s(int64_t P, int64_t E, int64_t H, int dtype) {
  if (dtype != MOE_DTYPE_BF16 || H % moe::kF16SegCols != 0 || P <= 0) return false;
  static const int32_t grouped = 0;  // any non-NULL offsets: a grouped GEMM
  moe::GemmArgs probe = gemm_args();
  probe.M = (int)P;
  probe.G = (int)E;
  probe.offsets = &grouped;
  return moe::grouped_gemm_has_f16s(probe);
}

moe_status moe_forward(const void* hidden_states, const void* router_weight, const float* router_bias, const void* w13,
                       const void* w2, const void* shared_w13, const void* shared_w2, const void* shared_gate,
                       int64_t num_tokens, int64_t hidden_size, int64_t num_experts, int64_t top_k,
                       int64_t intermediate_size, int64_t shared_intermediate_size, int renormalize, int dtype,
                       int out_dtype, void* output, int32_t* topk_ids_out, float* topk_weights_out,
                       float* router_logits_out, void* workspace, size_t workspace_bytes, void* stream) {
  const bool packed = dtype == MOE_DTYPE_BF16_KB32;
  if (packed) dtype = MOE_DTYPE_BF16;
  RETURN_IF_ERR(check_sizes(num_tokens, hidden_size, num_experts, top_k, dtype, true));
  RETURN_IF_ERR(check_inter(intermediate_size, dtype, "intermediate_size"));
  if (packed) RETURN_IF_ERR(check_packed_bytes(hidden_size, intermediate_size));
  const int nshared = (shared_w13 != nullptr) + (shared_w2 != nullptr) + (shared_gate != nullptr);
  if (nshared != 0 && nshared != 3)
    return fail(MOE_ERR_INVALID_ARG, "shared_w13, shared_w2 and shared_gate must be given together");
  const int64_t Is = nshared ? shared_intermediate_size : 0;
  if (nshared) RETURN_IF_ERR(check_inter(Is, dtype, "shared_intermediate_size"));
  if (nshared && packed) RETURN_IF_ERR(check_packed_bytes(hidden_size, Is));
  // the packed expert outputs take 2 bytes per value when stored as fp16 + exponents
  const int64_t y_elt = forward_y_f16s(num_tokens * top_k, num_experts, hidden_size, dtype) ? 2 : 4;
  RETURN_IF_ERR(check_buffer_bytes(num_tokens, hidden_size, top_k, intermediate_size, dtype, y_elt));
  if (nshared) RETURN_IF_ERR(check_buffer_bytes(num_tokens, hidden_size, 1, Is, dtype, 4));
  if (out_dtype != MOE_DTYPE_F32 && out_dtype != MOE_DTYPE_BF16)
    return fail(MOE_ERR_INVALID_ARG, "out_dtype must be MOE_DTYPE_F32 or MOE_DTYPE_BF16");
  if (num_tokens == 0) return succeed();
  REQUIRE_PTR(hidden_states);
  REQUIRE_PTR(router_weight);
  REQUIRE_PTR(w13);
  REQUIRE_PTR(w2);
  REQUIRE_PTR(output);
  REQUIRE_ALIGNED(hidden_states);
  REQUIRE_ALIGNED(router_weight);
  REQUIRE_ALIGNED(w13);
  REQUIRE_ALIGNED(w2);
  REQUIRE_ALIGNED(shared_w13);
  REQUIRE_ALIGNED(shared_w2);
  REQUIRE_ALIGNED(shared_gate);
  REQUIRE_ALIGNED(output);
  const size_t need = moe_forward_workspace_size(num_tokens, hidden_size, num_experts, top_k, intermediate_size, Is,
                                                 dtype);
  if (workspace == nullptr || workspace_bytes < need) return fail(MOE_ERR_WORKSPACE, "workspace too small");
  REQUIRE_ALIGNED(workspace);

  const int T = (int)num_tokens, H = (int)hidden_size, E = (int)num_experts, k = (int)top_k;
  const int I = (int)intermediate_size;
  const int P = T * k;
  ForwardLayout L = carve_forward(workspace, num_tokens, hidden_size, num_experts, top_k, intermediate_size, Is, dtype);
  float* logits = router_logits_out ? router_logits_out : L.logits;
  int32_t* ids = topk_ids_out ? topk_ids_out : L.ids;
  float* weights = topk_weights_out ? topk_weights_out : L.weights;
  hipStream_t s = static_cast<hipStream_t>(stream);

  hipError_t e = hipSuccess;
  // The shared expert depends only on the input: the aux stream forks before
  // the router, so that its weight streaming overlaps the router, top-k and
  // dispatch (small launches that leave most of the chip idle) and then the
  // routed experts; the join comes before the combine.  The routing launches
  // are enqueued first, so that the host's launch latency delays the shared
  // expert rather than the critical path.
  std::unique_lock<std::mutex> aux_lock;
  AuxSlot* aux = nullptr;
  if (Is) {
    aux = aux_slot(s);
    if (aux != nullptr) {
      aux_lock = std::unique_lock<std::mutex>(aux->mu);
      e = hipEventRecord(aux->fork, s);
      if (e == hipSuccess) e = hipStreamWaitEvent(aux->stream, aux->fork, 0);
      if (e != hipSuccess) return hip_status(e, "moe_forward(fork)");
    }
  }
  // decode batches: top-k and the plan in one single-workgroup launch; large
  // batches with k dividing a dispatch segment: top-k fused with the
  // dispatch histogram
  const bool small = T <= moe::kTopkDispatchSmallT && P <= moe::kDispatchSmallP;
  const bool fused_hist = !small && moe::dispatch_takes_hist(T, k);
  e = run_router(hidden_states, router_weight, router_bias, Is ? shared_gate : nullptr, T, H, E, k,
                 renormalize ? 1 : 0, dtype, logits, nullptr, ids, weights, Is ? L.gate_logit : nullptr, s,
                 !small && !fused_hist);
  if (e == hipSuccess && fused_hist)
    e = moe::launch_topk_hist(logits, T, E, k, renormalize ? 1 : 0, ids, weights, L.dispatch_scratch, s);
  if (e != hipSuccess) return hip_status(e, "moe_forward(router)");
  // the dispatch also zeroes the tile counters of the routed GEMMs
  if (small)
    e = moe::launch_topk_dispatch_small(logits, T, E, k, renormalize ? 1 : 0, ids, weights, L.counts, L.offsets,
                                        L.perm, L.inv, L.packed_ids, s, L.counters, 2 * moe::kTileCounterInts);
  else
    e = moe::launch_dispatch(ids, nullptr, T, k, E, L.counts, L.offsets, L.perm, L.inv, L.packed_ids, nullptr,
                             L.dispatch_scratch, s, L.counters, 2 * moe::kTileCounterInts, fused_hist);
  if (e != hipSuccess) return hip_status(e, "moe_forward(dispatch)");
  if (Is) {
    hipStream_t ss = aux != nullptr ? aux->stream : s;
    int* shared_counters = L.counters + 2 * moe::kTileCounterInts;
    if (dtype == MOE_DTYPE_BF16) {
      moe::GemmArgs probe = gemm_args();
      probe.M = T;
      probe.G = 1;
      if (moe::grouped_gemm_uses_counter(probe)) {
        e = moe::launch_zero_ints(shared_counters, 2 * moe::kTileCounterInts, ss);
        if (e != hipSuccess) return hip_status(e, "moe_forward(shared expert)");
      }
    }
    e = run_ffn(hidden_states, nullptr, nullptr, shared_w13, shared_w2, T, T, H, 1, (int)Is, dtype, packed, L.hs, L.ys,
                moe::Y_F32, nullptr, ss, true, shared_counters, L.partial_shared);
    if (e != hipSuccess) return hip_status(e, "moe_forward(shared expert)");
    if (aux != nullptr) {
      e = hipEventRecord(aux->join, aux->stream);
      if (e != hipSuccess) return hip_status(e, "moe_forward(join)");
    }
  }
  // Large batches (the 256-row down kernels): the packed expert
  // outputs go out as fp16 with a power-of-two scale per (row, 64 columns),
  // half the bytes of fp32 for the down projection to write and the combine
  // to read, with 11 significant bits (bf16 storage would keep 8 and about
  // double the layer's output error).  The exponents follow the values in
  // y's fp32-sized slot.
  int y_format = moe::Y_F32;
  int32_t* y_scale = nullptr;
  if (forward_y_f16s(P, E, H, dtype)) {
    y_format = moe::Y_F16S;
    y_scale = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(L.y) + align_up((size_t)P * H * 2));
  }
  e = run_ffn(hidden_states, L.packed_ids, L.offsets, w13, w2, T, P, H, E, I, dtype, packed, L.h, L.y, y_format,
              y_scale, s,
              false, L.counters, L.partial);
  if (e != hipSuccess) return hip_status(e, "moe_forward(experts)");
  if (aux != nullptr) {
    e = hipStreamWaitEvent(s, aux->join, 0);
    if (e != hipSuccess) return hip_status(e, "moe_forward(join)");
  }
  if (aux_lock.owns_lock()) aux_lock.unlock();
  e = moe::launch_combine(L.y, y_format, y_scale, L.inv, weights, Is ? L.ys : nullptr, Is ? L.gate_logit : nullptr,
                          T, H, k, out_dtype == MOE_DTYPE_BF16, output, s);
  return hip_status(e, "moe_forward(combine)");
}

void moe_profile_enable(int enable) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on.store(enable != 0, std::memory_order_relaxed);
}

int moe_profile_collect(const char** names, double* total_ms, int64_t* launches, int capacity) {
  std::vector<ProfRecord> recs;
  {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    recs.swap(g_prof);
  }
  std::vector<const char*> nm;
  std::vector<double> ms;
  std::vector<int64_t> cnt;
  for (const ProfRecord& r : recs) {
    float t = 0.f;
    if (hipEventSynchronize(r.stop) == hipSuccess && hipEventElapsedTime(&t, r.start, r.stop) == hipSuccess) {
      size_t i = 0;
      while (i < nm.size() && std::strcmp(nm[i], r.name) != 0) ++i;
      if (i == nm.size()) {
        nm.push_back(r.name);
        ms.push_back(0.0);
        cnt.push_back(0);
      }
      ms[i] += t;
      cnt[i] += 1;
    }
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
  }
  for (size_t i = 0; i < nm.size() && (int)i < capacity; ++i) {
    if (names) names[i] = nm[i];
    if (total_ms) total_ms[i] = ms[i];
    if (launches) launches[i] = cnt[i];
  }
  return (int)nm.size();
}

}  // extern "C"
