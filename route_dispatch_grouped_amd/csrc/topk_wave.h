// Wave-level routing primitives shared by the router kernels: an
// order-preserving float key, DPP wave reductions, and the top-k / softmax /
// renormalisation of one token's logits by one wavefront.
// [DWDP README "Router Module": routing probabilities, top-k expert indices,
//  normalized routing weights; diffulex.moe "diffulex.moe.topk"]
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace moe {

// Order-preserving map float -> uint32 (larger float -> larger key), after
// -0.0 has been folded onto +0.0.  NaN is not a supported input.
__device__ __forceinline__ uint32_t order_key(float f) {
  if (f == 0.f) f = 0.f;
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float order_value(uint32_t o) {
  const uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __uint_as_float(u);
}

// One step of a max-reduction through a DPP lane permutation (within 16-lane rows).
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_max_step(uint64_t v) {
  const int hi = (int)(v >> 32), lo = (int)(v & 0xFFFFFFFFu);
  const uint32_t ohi = (uint32_t)__builtin_amdgcn_update_dpp(hi, hi, CTRL, 0xF, 0xF, false);
  const uint32_t olo = (uint32_t)__builtin_amdgcn_update_dpp(lo, lo, CTRL, 0xF, 0xF, false);
  const uint64_t o = ((uint64_t)ohi << 32) | olo;
  return o > v ? o : v;
}

// Wave-wide maximum of a 64-bit key, returned wave-uniform: DPP exchanges
// (xor 1, xor 2, half-row mirror, row mirror) leave every lane of a 16-lane
// row holding the row maximum; the four row maxima are then read out with
// readlane.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = dpp_max_step<0xB1>(v);   // quad_perm(1,0,3,2)
  v = dpp_max_step<0x4E>(v);   // quad_perm(2,3,0,1)
  v = dpp_max_step<0x141>(v);  // row_half_mirror
  v = dpp_max_step<0x140>(v);  // row_mirror
  uint64_t best = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(v >> 32), 16 * r);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(v & 0xFFFFFFFFu), 16 * r);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    best = o > best ? o : best;
  }
  return best;
}

// Wave-wide maximum of a 32-bit key, wave-uniform (same exchange pattern).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4E, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x141, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x140, 0xF, 0xF, false));
  uint32_t best = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) best = max(best, (uint32_t)__builtin_amdgcn_readlane((int)v, 16 * r));
  return best;
}

template <int CTRL>
__device__ __forceinline__ float dpp_add_step(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, 0xF, 0xF,
                                                         false));
}

// Wave-wide float sum, wave-uniform (same exchange pattern as wave_max_u64).
__device__ __forceinline__ float wave_sum(float v) {
  v = dpp_add_step<0xB1>(v);
  v = dpp_add_step<0x4E>(v);
  v = dpp_add_step<0x141>(v);
  v = dpp_add_step<0x140>(v);
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) s += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16 * r));
  return s;
}

// One wavefront selects the top-k of one token's logits row[0..E) (global or
// LDS memory) and writes ids[0..k), weights[0..k) and, when probs != NULL, the
// full softmax probs[0..E).  Lane l holds experts l, l+64, ... (VPL >= E/64).
// k rounds; each takes a wave-wide max of the 32-bit order-preserving key of
// the logits still available, then the lowest expert id holding that key (a
// ballot per slot, slots scanned in id order): the larger logit wins and, on
// equal logits, the lower expert id.  Winner j is kept by lane j % 64 in slot
// j / 64.  Weights:
// exp(l_j - l_max) over the sum of the selected terms (renormalised) or over
// all E terms (the plain softmax probability).
//
// Group-limited selection (n_group > 1; [diffulex.moe "diffulex.moe.topk"]:
// a router with group-limited expert selection): experts form n_group <= 64
// contiguous groups of E / n_group; a group's score is the largest key it
// holds (its largest logit, the lower id on equal logits, so equal group
// scores go to the lower group); the topk_group best groups stay available
// and the k rounds run over their experts only.  The softmax terms still
// cover all E experts.
template <int VPL>
__device__ __forceinline__ void topk_row(const float* row, int E, int k, int renorm, int32_t* __restrict__ ids,
                                         float* __restrict__ weights, float* __restrict__ probs, int lane,
                                         int32_t* ids_copy = nullptr, int n_group = 1, int topk_group = 1) {
  float v[VPL];
  uint32_t key[VPL];
  uint32_t avail = 0;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + 64 * i;
    if (e < E) {
      v[i] = row[e];
      key[i] = order_key(v[i]);
      avail |= 1u << i;
    } else {
      v[i] = -INFINITY;
      key[i] = 0;
    }
  }

  if (n_group > 1 && (E / n_group) <= 16 && ((E / n_group) & (E / n_group - 1)) == 0) {
    // Groups of gs = 1, 2, 4, 8 or 16 experts occupy aligned gs-lane segments
    // of one slot (expert e = lane + 64 i lies in group e / gs = lane / gs +
    // i * 64 / gs), so the first DPP steps of a wave reduction, stopped at the
    // segment size, leave each lane holding its group's largest key.
    const int gs = E / n_group;
    uint32_t gk[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      uint32_t v = ((avail >> i) & 1u) ? key[i] : 0u;
      if (gs >= 2) v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xF, 0xF, false));
      if (gs >= 4) v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4E, 0xF, 0xF, false));
      if (gs >= 8) v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x141, 0xF, 0xF, false));
      if (gs >= 16) v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x140, 0xF, 0xF, false));
      gk[i] = v;
    }
    // topk_group rounds: the largest group score, the lowest group holding it
    // (groups past n_group hold no expert: score 0, below every real one)
    uint64_t kept = 0;
    for (int r = 0; r < topk_group; ++r) {
      uint32_t mine = 0;
#pragma unroll
      for (int i = 0; i < VPL; ++i) mine = max(mine, gk[i]);
      const uint32_t best = wave_max_u32(mine);
      int g = 0;
#pragma unroll
      for (int i = VPL - 1; i >= 0; --i) {
        const uint64_t hit = __ballot(gk[i] == best);
        if (hit != 0) g = __builtin_ctzll(hit) / gs + i * (64 / gs);
      }
      kept |= 1ull << g;
#pragma unroll
      for (int i = 0; i < VPL; ++i)
        if (lane / gs + i * (64 / gs) == g) gk[i] = 0;
    }
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = lane + 64 * i;
      if (e < E && !((kept >> (e / gs)) & 1ull)) avail &= ~(1u << i);
    }
  } else if (n_group > 1) {
    const int gs = E / n_group;
    uint64_t gkey = 0;  // lane g < n_group: group g's score key
    for (int g = 0; g < n_group; ++g) {
      uint64_t best = 0;
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int e = lane + 64 * i;
        if (((avail >> i) & 1u) && e / gs == g) {
          const uint64_t kk = ((uint64_t)key[i] << 32) | (uint32_t)(~(uint32_t)e);
          best = kk > best ? kk : best;
        }
      }
      best = wave_max_u64(best);
      if (lane == g) gkey = best;
    }
    uint64_t kept = 0;  // bit g: group g kept
    bool gfree = lane < n_group;
    for (int r = 0; r < topk_group; ++r) {
      const uint64_t b = wave_max_u64(gfree ? gkey : 0);
      const int gw = __builtin_ctzll(__ballot(gfree && gkey == b));
      kept |= 1ull << gw;
      if (lane == gw) gfree = false;
    }
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = lane + 64 * i;
      if (e < E && !((kept >> (e / gs)) & 1ull)) avail &= ~(1u << i);
    }
  }

  // Each round: the largest available key over the wave (32-bit), then the
  // lowest expert id holding it: slots are scanned in id order (slot i holds
  // ids 64 i .. 64 i + 63), the first slot with a match gives its lowest lane.
  // Key 0 lies below every float's key, so it marks a taken or absent slot.
  int my_id[VPL];
  float my_val[VPL];
#pragma unroll
  for (int c = 0; c < VPL; ++c) {
    my_id[c] = 0;
    my_val[c] = 0.f;
    const int jn = min(64, k - 64 * c);
    for (int jj = 0; jj < jn; ++jj) {
      uint32_t mine = 0;
#pragma unroll
      for (int i = 0; i < VPL; ++i)
        if ((avail >> i) & 1u) mine = max(mine, key[i]);
      const uint32_t best = wave_max_u32(mine);
      int id = 0;
#pragma unroll
      for (int i = VPL - 1; i >= 0; --i) {
        const uint64_t hit = __ballot(((avail >> i) & 1u) && key[i] == best);
        if (hit != 0) id = 64 * i + __builtin_ctzll(hit);
      }
      if ((id & 63) == lane) avail &= ~(1u << (id >> 6));
      if (jj == lane) {
        my_id[c] = id;
        my_val[c] = order_value(best);
      }
    }
  }

  const float m = __shfl(my_val[0], 0, 64);  // largest logit
  float s_sel = 0.f, s_all = 0.f;
#pragma unroll
  for (int c = 0; c < VPL; ++c)
    if (64 * c + lane < k) s_sel += expf(my_val[c] - m);
  s_sel = wave_sum(s_sel);
  if (!renorm || probs != nullptr) {
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (lane + 64 * i < E) s_all += expf(v[i] - m);
    s_all = wave_sum(s_all);
  }
  const float denom = renorm ? s_sel : s_all;
#pragma unroll
  for (int c = 0; c < VPL; ++c) {
    const int j = 64 * c + lane;
    if (j < k) {
      ids[j] = my_id[c];
      if (ids_copy != nullptr) ids_copy[j] = my_id[c];
      weights[j] = expf(my_val[c] - m) / denom;
    }
  }
  if (probs != nullptr) {
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = lane + 64 * i;
      if (e < E) probs[e] = expf(v[i] - m) / s_all;
    }
  }
}

}  // namespace moe
