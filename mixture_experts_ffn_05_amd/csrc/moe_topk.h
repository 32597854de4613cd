// Top-k selection of the router: one wave per token (moe_route.hip,
// moe_scatter.hip).  PLENA_Simulator PR #97, section "C_SET_TOPK_REG": top-k
// softmax generic in the expert count and in k.  Order key: logit descending,
// expert index ascending, NaN lowest; slots are filled in that order.
#pragma once

#include "moe_common.h"

namespace moe {

// Router order of two experts: higher logit first, lower index on ties.
__device__ __forceinline__ bool ranks_before(float v, int e, float bv, int be) {
  return v > bv || (v == bv && e < be);
}

constexpr int kTopkPer = kMaxExperts / kWave;  // logits per lane of one token, at most

// Logits per lane for E experts (a power of two up to kTopkPer), the template
// argument of topk_wave and of the kernels that call it.
inline int topk_per_lane(int E) {
  int q = 1;
  while (q * kWave < E) q <<= 1;
  return q;
}

// One exchange of a wave arg-max through DPP (lanes of one 16-lane row; no LDS):
// take the partner's (key, index) if it ranks first.  CTRL is a DPP control
// that gives every lane a valid partner (quad permutations, row rotations).
template <int CTRL>
__device__ __forceinline__ void argmax_dpp_step(float& bv, int& be) {
  const float ov = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(bv), CTRL, 0xF, 0xF, false));
  const int oe = __builtin_amdgcn_update_dpp(0, be, CTRL, 0xF, 0xF, false);
  if (ranks_before(ov, oe, bv, be)) {
    bv = ov;
    be = oe;
  }
}

// Top-k of one token whose logits a wave holds: lane l holds raw[q], the
// logit of expert l + 64q, for l + 64q < E.  k rounds of a wave arg-max under
// the key (logit descending, index ascending, NaN lowest), then a softmax over
// the k selected logits.  Lane j < k returns the j-th selection in slot order
// (id, weight); the other lanes return id -1.
template <int Q>
__device__ __forceinline__ void topk_wave(const float (&raw)[Q], int E, int k, int& my_id, float& my_w) {
  static_assert(Q >= 1 && Q <= kTopkPer && (Q & (Q - 1)) == 0, "logits per lane: a power of two up to kTopkPer");
  const int lane = lane_id();
  float key[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) key[q] = (raw[q] != raw[q]) ? -INFINITY : raw[q];
  uint32_t taken = 0;
  float my_sel = 0.f;
  my_id = -1;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int e = lane + kWave * q;
      if (e < E && !((taken >> q) & 1u) && ranks_before(key[q], e, bv, be)) {
        bv = key[q];
        be = e;
      }
    }
    // Wave arg-max: inside each 16-lane row by DPP (quad swaps of 1 and 2, then
    // row rotations by 4 and 8), then across rows by two shuffles.  The order is
    // total (indices are unique), so every lane ends with the same winner
    // whatever the exchange pattern.
    argmax_dpp_step<0xB1>(bv, be);   // quad_perm [1,0,3,2]
    argmax_dpp_step<0x4E>(bv, be);   // quad_perm [2,3,0,1]
    argmax_dpp_step<0x124>(bv, be);  // row_ror:4
    argmax_dpp_step<0x128>(bv, be);  // row_ror:8
#pragma unroll
    for (int d = 16; d <= 32; d <<= 1) {
      const float ov = __shfl_xor(bv, d, kWave);
      const int oe = __shfl_xor(be, d, kWave);
      if (ranks_before(ov, oe, bv, be)) {
        bv = ov;
        be = oe;
      }
    }
    // the winner's raw logit (a NaN stays NaN): lane be % 64 holds it in slot be / 64
    float cand = raw[0];
#pragma unroll
    for (int q = 1; q < Q; ++q)
      if ((be >> 6) == q) cand = raw[q];
    const float br = __shfl(cand, be & 63, kWave);
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    if (lane == j) {
      my_id = be;
      my_sel = br;
    }
  }
  const float m = __shfl(my_sel, 0, kWave);
  const float ex = lane < k ? expf(my_sel - m) : 0.f;
  const float s = wave_sum(ex);
  my_w = ex / s;
}

}  // namespace moe
