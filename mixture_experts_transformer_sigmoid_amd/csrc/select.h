// Per-token top-k and gates, one wave per token: "Kimi K2 · Transformer blocks", MoE
// equations E_sel (the k largest biased scores s + b) and G_i (alpha * s_i over the sum of
// the chosen s, the bias left out); "nnterp encyclopedia · kimi_k2", "The mixture of
// experts" (all experts eligible; the gates from the selected sigmoid scores, bias excluded).
// Used by the selection kernels of route.hip.  Every definition lives in an unnamed
// namespace: each source file that includes this gets its own copy.
#pragma once

#include <math.h>

#include <type_traits>

#include "common.h"

namespace moe {
namespace {

// Order key of a candidate: the fp32 score mapped to an unsigned integer that orders as
// the float does (negative values bit-inverted, the sign bit set on the others; -0 first
// made +0, so that the two compare equal as floats do), in the high half, and the
// complement of the expert index in the low half, so that of two equal scores the lower
// index has the larger key.  Every key of a real candidate is nonzero (even a score of
// -inf); 0 marks an expert past E or one already picked.
__device__ __forceinline__ uint64_t select_key(float score, int e) {
  const uint32_t u = __float_as_uint(score + 0.0f);
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)ord << 32) | (uint32_t)(0xffffffffu - (uint32_t)e);
}

// The largest key of the wave, in every lane: within each row of 16 lanes by DPP (swap
// neighbours, then pairs, then mirror the halves of 8 and of 16), across the rows by two
// lane shuffles.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t v) {
  auto step_dpp = [](uint64_t x, auto ctrl) {
    const int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)x, decltype(ctrl)::value, 0xf, 0xf, false);
    const int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(x >> 32), decltype(ctrl)::value, 0xf, 0xf,
                                            false);
    const uint64_t o = ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
    return o > x ? o : x;
  };
  v = step_dpp(v, std::integral_constant<int, 0xb1>{});   // quad_perm [1, 0, 3, 2]
  v = step_dpp(v, std::integral_constant<int, 0x4e>{});   // quad_perm [2, 3, 0, 1]
  v = step_dpp(v, std::integral_constant<int, 0x141>{});  // row_half_mirror
  v = step_dpp(v, std::integral_constant<int, 0x140>{});  // row_mirror
#pragma unroll
  for (int off = 16; off <= 32; off <<= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, off);
    const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), off);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

// Lane l holds experts l, l + 64, ..., l + 64 (EPL - 1).  Scores of experts >= E, and NaN
// scores, must already be -inf.  k rounds of a wave-wide argmax over (score, -index) pick
// the experts in descending score, ties to the lower index (select_key; experts past E are
// never picked); the gates are alpha * s / den with den the fp32 sum of the picked experts'
// sigmoid scores in pick order (0 if den is 0).  Lane j < k writes pick j to idx[j] / w[j]
// (global, or null) and idx_lds[j] (LDS, or null).  No branch depends on the data: each
// round is one key reduction, a read of the winner's sigmoid from its lane, and the
// winner's key cleared in its lane.
template <int EPL>
__device__ __forceinline__ void select_topk(const float (&score)[EPL], const float (&sig)[EPL],
                                            int E, int k, float alpha, int lane, int32_t* idx,
                                            float* w, int32_t* idx_lds) {
  uint64_t key[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    key[i] = e < E ? select_key(score[i], e) : 0ull;
  }
  int sel_idx[kMaxTopK];
  float sel_s[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    sel_idx[j] = 0;
    sel_s[j] = 0.0f;
  }
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    if (j < k) {
      uint64_t m = key[0];
#pragma unroll
      for (int i = 1; i < EPL; ++i) m = key[i] > m ? key[i] : m;
      m = wave_max_key(m);
      // the winner, the same in every lane
      const int e = __builtin_amdgcn_readfirstlane((int)(0xffffffffu - (uint32_t)m));
      const int slot = e >> 6;
      float mine = sig[0];
#pragma unroll
      for (int i = 1; i < EPL; ++i) mine = slot == i ? sig[i] : mine;
      sel_s[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine), e & 63));
      sel_idx[j] = e;
#pragma unroll
      for (int i = 0; i < EPL; ++i) key[i] = key[i] == m ? 0ull : key[i];
    }
  }
  float den = 0.0f;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j)
    if (j < k) den += sel_s[j];
  int my_idx = 0;
  float my_s = 0.0f;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    my_idx = lane == j ? sel_idx[j] : my_idx;
    my_s = lane == j ? sel_s[j] : my_s;
  }
  if (lane < k) {
    if (idx != nullptr) idx[lane] = my_idx;
    if (w != nullptr) w[lane] = den > 0.0f ? alpha * my_s / den : 0.0f;
    if (idx_lds != nullptr) idx_lds[lane] = my_idx;
  }
}

// Experts per lane for E experts: the smallest instantiated EPL >= ceil(E / 64).
inline int select_epl(int E) {
  const int epl = (E + 63) / 64;
  return epl <= 1 ? 1 : epl <= 2 ? 2 : epl <= 4 ? 4 : epl <= 6 ? 6 : epl <= 8 ? 8 : 16;
}

}  // namespace
}  // namespace moe
