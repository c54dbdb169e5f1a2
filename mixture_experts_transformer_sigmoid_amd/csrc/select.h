// Per-token top-k and gates, one wave per token: "Kimi K2 · Transformer blocks", MoE
// equations E_sel (the k largest biased scores s + b) and G_i (alpha * s_i over the sum of
// the chosen s, the bias left out); "nnterp encyclopedia · kimi_k2", "The mixture of
// experts" (all experts eligible; the gates from the selected sigmoid scores, bias excluded).
// Used by the selection kernels of route.hip.  Every definition lives in an unnamed
// namespace: each source file that includes this gets its own copy.
#pragma once

#include <math.h>

#include "common.h"

namespace moe {
namespace {

// Lane l holds experts l, l + 64, ..., l + 64 (EPL - 1).  Scores of experts >= E, and NaN
// scores, must already be -inf.  k rounds of a wave-wide argmax over (score, -index) pick
// the experts in descending score, ties to the lower index; the gates are alpha * s / den
// with den the fp32 sum of the picked experts' sigmoid scores in pick order (0 if den is
// 0).  Lane j < k writes pick j to idx[j] / w[j] (global, or null) and idx_lds[j] (LDS, or
// null).
template <int EPL>
__device__ __forceinline__ void select_topk(const float (&score)[EPL], const float (&sig)[EPL],
                                            int E, int k, float alpha, int lane, int32_t* idx,
                                            float* w, int32_t* idx_lds) {
  uint32_t taken = 0;
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
      float bv = -INFINITY, bs = 0.0f;
      int bi = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        if (e < E && !((taken >> i) & 1u)) {
          if (score[i] > bv || (score[i] == bv && e < bi)) {
            bv = score[i];
            bi = e;
            bs = sig[i];
          }
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oi = __shfl_xor(bi, off);
        const float os = __shfl_xor(bs, off);
        if (ov > bv || (ov == bv && oi < bi)) {
          bv = ov;
          bi = oi;
          bs = os;
        }
      }
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (lane + 64 * i == bi) taken |= 1u << i;
      sel_idx[j] = bi;
      sel_s[j] = bs;
    }
  }
  float den = 0.0f;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j)
    if (j < k) den += sel_s[j];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    if (j < k && lane == j) {
      if (idx != nullptr) idx[j] = sel_idx[j];
      if (w != nullptr) w[j] = den > 0.0f ? alpha * sel_s[j] / den : 0.0f;
      if (idx_lds != nullptr) idx_lds[j] = sel_idx[j];
    }
  }
}

// Experts per lane for E experts: the smallest instantiated EPL >= ceil(E / 64).
inline int select_epl(int E) {
  const int epl = (E + 63) / 64;
  return epl <= 1 ? 1 : epl <= 2 ? 2 : epl <= 4 ? 4 : epl <= 6 ? 6 : epl <= 8 ? 8 : 16;
}

}  // namespace
}  // namespace moe
