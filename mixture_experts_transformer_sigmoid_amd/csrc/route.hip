// Router: z = x W_r^T, s = sigmoid(z), top-k of s + b, gates alpha * s / sum(s).
// "Kimi K2 · Transformer blocks", MoE equations z, s, E_sel, G_i; selection bias and
// bias-free gates as in "nnterp encyclopedia · kimi_k2", "The mixture of experts".
//
// The logits GEMM runs on the bf16 MFMA units without losing fp32 accuracy: each fp32
// router weight is split exactly into three bf16 numbers, w = hi + mid + lo (hi is w
// rounded to bf16, mid the rounded remainder, lo the rest, which fits in bf16's 8
// significant bits), so x W_r^T = x hi^T + x mid^T + x lo^T.  x is bf16, so every
// product is exact in fp32; the three partial logits are accumulated in fp32 by the
// grouped-GEMM kernels (one group, 3E outputs) and added in fp64 by the selection kernel.
// (The split follows the bf16x3 scheme of Henry, Tang and Heinecke, "Leveraging the
// bfloat16 artificial intelligence datatype for higher-precision computations", 2019.)
#include <math.h>

#include "common.h"

namespace moe {
namespace {

// w_split[p][e][j], p = 0 (hi), 1 (mid), 2 (lo)
__global__ __launch_bounds__(256) void router_split_kernel(const float* __restrict__ w_r,
                                                           int64_t n,
                                                           uint16_t* __restrict__ w_split) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const float w = w_r[i];
    const uint32_t hi = f32_to_bf16(w);
    const float r1 = w - bf16_to_f32(hi);
    const uint32_t mid = f32_to_bf16(r1);
    const float r2 = r1 - bf16_to_f32(mid);
    w_split[i] = (uint16_t)hi;
    w_split[n + i] = (uint16_t)mid;
    w_split[2 * n + i] = (uint16_t)f32_to_bf16(r2);
  }
}

// ---------------------------------------------------------------- top-k + gates
// One wave per token.  z = hi + mid + lo partial logits summed in fp64, rounded to fp32.
// Lane l holds experts l, l + 64, ...; k rounds of a wave-wide argmax over (score,
// -index) pick the experts (ties to the lower index, NaN scores treated as -inf); the
// gates use the sigmoid without the bias.
template <int EPL>
__global__ __launch_bounds__(256) void router_select_kernel(const float* __restrict__ z_part,
                                                            const float* __restrict__ bias,
                                                            int64_t T, int E, int k, float alpha,
                                                            float* __restrict__ logits,
                                                            int32_t* __restrict__ topk_idx,
                                                            float* __restrict__ topk_w) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* zp = z_part + t * 3 * E;

  float score[EPL], sig[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    if (e < E) {
      const float z = (float)((double)zp[e] + (double)zp[E + e] + (double)zp[2 * E + e]);
      if (logits != nullptr) logits[t * E + e] = z;
      const float s = 1.0f / (1.0f + expf(-z));
      float v = s + bias[e];
      if (v != v) v = -INFINITY;
      score[i] = v;
      sig[i] = s;
    } else {
      score[i] = -INFINITY;
      sig[i] = 0.0f;
    }
  }
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
      topk_idx[t * k + j] = sel_idx[j];
      topk_w[t * k + j] = den > 0.0f ? alpha * sel_s[j] / den : 0.0f;
    }
  }
}

template <int EPL>
void select_launch(const float* z_part, const float* bias, int64_t T, int E, int k, float alpha,
                   float* logits, int32_t* idx, float* w, hipStream_t s) {
  const unsigned grid = (unsigned)((T + 3) / 4);
  hipLaunchKernelGGL(router_select_kernel<EPL>, dim3(grid), dim3(256), 0, s, z_part, bias, T, E,
                     k, alpha, logits, idx, w);
}

}  // namespace

hipError_t launch_router(const uint16_t* x, const float* w_r, const float* bias, int64_t T, int d,
                         int E, int k, float alpha, uint16_t* w_split, float* z_part,
                         Tile* tiles, int32_t* ntiles, float* logits, int32_t* topk_idx,
                         float* topk_w, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const int64_t n = (int64_t)E * d;
  const int64_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
  hipLaunchKernelGGL(router_split_kernel, dim3((unsigned)blocks), dim3(256), 0, s, w_r, n,
                     w_split);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  err = launch_dense(x, T, d, w_split, 3 * E, DenseOut::kF32, z_part, nullptr, nullptr, tiles,
                     ntiles, s);
  if (err != hipSuccess) return err;
  const int epl = (E + 63) / 64;
  if (epl <= 1)
    select_launch<1>(z_part, bias, T, E, k, alpha, logits, topk_idx, topk_w, s);
  else if (epl <= 2)
    select_launch<2>(z_part, bias, T, E, k, alpha, logits, topk_idx, topk_w, s);
  else if (epl <= 4)
    select_launch<4>(z_part, bias, T, E, k, alpha, logits, topk_idx, topk_w, s);
  else if (epl <= 6)
    select_launch<6>(z_part, bias, T, E, k, alpha, logits, topk_idx, topk_w, s);
  else if (epl <= 8)
    select_launch<8>(z_part, bias, T, E, k, alpha, logits, topk_idx, topk_w, s);
  else
    select_launch<16>(z_part, bias, T, E, k, alpha, logits, topk_idx, topk_w, s);
  return hipGetLastError();
}

}  // namespace moe
