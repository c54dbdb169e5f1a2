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
// For a few tokens (decode) one kernel does the split in registers and cuts K into
// slices instead (router_small_kernel below).
// (The split follows the bf16x3 scheme of Henry, Tang and Heinecke, "Leveraging the
// bfloat16 artificial intelligence datatype for higher-precision computations", 2019.)
#include <math.h>

#include "common.h"

namespace moe {
namespace {

// w_split[p][e][j], p = 0 (hi), 1 (mid), 2 (lo), each part Ep = router_part_rows(E) rows
// of d: rows E .. Ep - 1 are zero, so that every part, and every row of partial logits the
// GEMM writes, is a whole number of 4-float groups
__global__ __launch_bounds__(256) void router_split_kernel(const float* __restrict__ w_r,
                                                           int64_t n, int64_t np_,
                                                           uint16_t* __restrict__ w_split) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < np_;
       i += (int64_t)gridDim.x * 256) {
    const float w = i < n ? w_r[i] : 0.0f;
    const uint32_t hi = f32_to_bf16(w);
    const float r1 = w - bf16_to_f32(hi);
    const uint32_t mid = f32_to_bf16(r1);
    const float r2 = r1 - bf16_to_f32(mid);
    w_split[i] = (uint16_t)hi;
    w_split[np_ + i] = (uint16_t)mid;
    w_split[2 * np_ + i] = (uint16_t)f32_to_bf16(r2);
  }
}

// ---------------------------------------------------------------- logits, few tokens
// For a decode-sized batch the logits GEMM is small (T x E outputs) and its cost is
// reading W_r.  This kernel reads the fp32 router weights once, splits each value into
// its hi, mid and lo bf16 parts in registers (no split pass, no bf16 copy of W_r) and
// accumulates the three partial logits in three fp32 accumulators.  K is cut into
// kRouterKSplit slices (grid z) so that the launch fills the chip; every (slice, part)
// pair writes its own partial, and the selection kernel adds the 3 * kRouterKSplit
// partials of a logit in fp64, in a fixed order (slice by slice, hi, mid, lo).
// Block: 4 waves; wave w owns experts n0 + 16 w .. + 15 (one MFMA fragment), the block
// 16 rows (tokens).  Lane (r, q): expert n0 + 16 w + r, token t0 + r, k 8q .. 8q + 7 of
// each 32-wide step; weights are the MFMA's A operand, tokens its B operand.
#ifndef MOE_ROUTER_KU
#define MOE_ROUTER_KU 4
#endif
constexpr int kRouterKU = MOE_ROUTER_KU;   // k-steps of loads issued before their MFMAs

// The split of two weights at once, each part a packed bf16 pair (first weight in bits
// 0..15), on the hardware round-to-nearest-even conversion (two values per instruction;
// the same rounding as f32_to_bf16).  Each remainder is exact in fp32.
__device__ __forceinline__ void split3x2(float a, float b, uint32_t& H, uint32_t& M,
                                         uint32_t& L) {
  H = pack_bf16x2(a, b);
  const float ra = a - __uint_as_float(H << 16), rb = b - __uint_as_float(H & 0xffff0000u);
  M = pack_bf16x2(ra, rb);
  L = pack_bf16x2(ra - __uint_as_float(M << 16), rb - __uint_as_float(M & 0xffff0000u));
}

__global__ __launch_bounds__(256) void router_small_kernel(const uint16_t* __restrict__ x,
                                                           const float* __restrict__ w_r,
                                                           int64_t T, int d, int E,
                                                           float* __restrict__ z_part) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r = lane & 15, q = lane >> 4;
  const int64_t t0 = (int64_t)blockIdx.x * 16;
  const int n0 = blockIdx.y * 64 + wave * 16;
  const int kz = blockIdx.z, nks = d / 32;
  const int ks0 = (int)((int64_t)nks * kz / kRouterKSplit);
  const int ks1 = (int)((int64_t)nks * (kz + 1) / kRouterKSplit);
  int64_t t = t0 + r;
  if (t > T - 1) t = T - 1;
  int e = n0 + r;
  if (e > E - 1) e = E - 1;
  const float* wrow = w_r + (int64_t)e * d + q * 8;
  const uint16_t* xrow = x + t * d + q * 8;
  f32x4_t acc[3] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f},
                    f32x4_t{0.f, 0.f, 0.f, 0.f}};
  auto step = [&](const u32x4_t (&wv)[2], u32x4_t xv) {
    uint32_t h[4], m[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4_t& w = wv[i >> 1];
      split3x2(__uint_as_float(w[2 * (i & 1)]), __uint_as_float(w[2 * (i & 1) + 1]), h[i], m[i],
               l[i]);
    }
    const u32x4_t H = {h[0], h[1], h[2], h[3]}, Mv = {m[0], m[1], m[2], m[3]},
                  Lv = {l[0], l[1], l[2], l[3]};
    acc[0] = mfma16x16x32(H, xv, acc[0]);
    acc[1] = mfma16x16x32(Mv, xv, acc[1]);
    acc[2] = mfma16x16x32(Lv, xv, acc[2]);
  };
  int ks = ks0;
  for (; ks + kRouterKU <= ks1; ks += kRouterKU) {
    u32x4_t wv[kRouterKU][2], xv[kRouterKU];
#pragma unroll
    for (int u = 0; u < kRouterKU; ++u) {
      const float* wp = wrow + (ks + u) * 32;
      wv[u][0] = *reinterpret_cast<const u32x4_t*>(wp);
      wv[u][1] = *reinterpret_cast<const u32x4_t*>(wp + 4);
      xv[u] = load16(xrow + (ks + u) * 32);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kRouterKU; ++u) step(wv[u], xv[u]);
  }
  for (; ks < ks1; ++ks) {
    const float* wp = wrow + ks * 32;
    const u32x4_t wv[2] = {*reinterpret_cast<const u32x4_t*>(wp),
                           *reinterpret_cast<const u32x4_t*>(wp + 4)};
    step(wv, load16(xrow + ks * 32));
  }
  // lane holds experts n0 + 4q .. + 3 of token t0 + r; partial (slice kz, part p) of a
  // token's logits sits at z_part[t][(3 kz + p) E + e]
  if (t0 + r >= T) return;
  float* zrow = z_part + (t0 + r) * (int64_t)(3 * kRouterKSplit) * E;
#pragma unroll
  for (int p = 0; p < 3; ++p)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ee = n0 + 4 * q + i;
      if (ee < E) zrow[(3 * kz + p) * (int64_t)E + ee] = acc[p][i];
    }
}

// ---------------------------------------------------------------- top-k + gates
// One wave per token.  z = hi + mid + lo partial logits summed in fp64, rounded to fp32.
// Lane l holds experts l, l + 64, ...; k rounds of a wave-wide argmax over (score,
// -index) pick the experts (ties to the lower index, NaN scores treated as -inf); the
// gates use the sigmoid without the bias.
template <int EPL, int PB>
__global__ __launch_bounds__(256) void router_select_kernel(const float* __restrict__ z_part,
                                                            int np, int row_parts, int pstride,
                                                            const float* __restrict__ bias,
                                                            int64_t T, int E, int k, float alpha,
                                                            float* __restrict__ logits,
                                                            int32_t* __restrict__ topk_idx,
                                                            float* __restrict__ topk_w) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* zp = z_part + t * (int64_t)row_parts * pstride;

  // the np partial logits of each expert, added in fp64 in part order.  Loads of PB parts
  // are issued together (the host picks PB >= np where the registers allow, so that the
  // wave waits for one round trip): every load reads an in-range element (part and expert
  // clamped) and the out-of-range ones are dropped afterwards, so that no load sits behind
  // a branch (a guarded load compiles to a branch and a wait per load)
  double zd[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) zd[i] = 0.0;
  for (int p0 = 0; p0 < np; p0 += PB) {
    float v[PB][EPL];
#pragma unroll
    for (int j = 0; j < PB; ++j)
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        v[j][i] = zp[min(p0 + j, np - 1) * pstride + min(lane + 64 * i, E - 1)];
    // all of the batch's loads before the first add (left alone, the compiler interleaves
    // them and keeps only about 32 in flight)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < PB; ++j)
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        zd[i] += (p0 + j < np) ? (double)v[j][i] : 0.0;
  }
  float score[EPL], sig[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    if (e < E) {
      const float z = (float)zd[i];
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

// Parts per batch of loads: every part in one batch (np is at most 24: 3 per K slice, at
// most 8 slices) while the loaded values fit in 144 registers, else batches of 8.
template <int EPL>
void select_launch(const float* z_part, int np, int row_parts, int pstride, const float* bias,
                   int64_t T, int E, int k, float alpha, float* logits, int32_t* idx, float* w,
                   hipStream_t s) {
  const unsigned grid = (unsigned)((T + 3) / 4);
  if (EPL <= 6 && np <= 12)
    hipLaunchKernelGGL((router_select_kernel<EPL, 12>), dim3(grid), dim3(256), 0, s, z_part, np,
                       row_parts, pstride, bias, T, E, k, alpha, logits, idx, w);
  else if (EPL <= 6)
    hipLaunchKernelGGL((router_select_kernel<EPL, 24>), dim3(grid), dim3(256), 0, s, z_part, np,
                       row_parts, pstride, bias, T, E, k, alpha, logits, idx, w);
  else
    hipLaunchKernelGGL((router_select_kernel<EPL, 8>), dim3(grid), dim3(256), 0, s, z_part, np,
                       row_parts, pstride, bias, T, E, k, alpha, logits, idx, w);
}

}  // namespace

hipError_t launch_router(const uint16_t* x, const float* w_r, const float* bias, int64_t T, int d,
                         int E, int k, float alpha, uint16_t* w_split, float* z_part,
                         Tile* tiles, int32_t* ntiles, float* logits, int32_t* topk_idx,
                         float* topk_w, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  hipError_t err;
  int np, row_parts, pstride;
  if (T <= kRouterSmallT) {
    const dim3 grid((unsigned)((T + 15) / 16), (unsigned)((E + 63) / 64), kRouterKSplit);
    hipLaunchKernelGGL(router_small_kernel, grid, dim3(256), 0, s, x, w_r, T, d, E, z_part);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    // the selection adds the 3 * kRouterKSplit partials of each logit in fp64, slice by
    // slice
    np = 3 * kRouterKSplit;
    row_parts = 3 * kRouterKSplit;
    pstride = E;
  } else {
    const int Ep = router_part_rows(E);
    const int64_t n = (int64_t)E * d, np_ = (int64_t)Ep * d;
    const int64_t blocks = (np_ + 255) / 256 < 4096 ? (np_ + 255) / 256 : 4096;
    hipLaunchKernelGGL(router_split_kernel, dim3((unsigned)blocks), dim3(256), 0, s, w_r, n, np_,
                       w_split);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    // K cut into S slices (router_ksplit): every token's row holds S x (hi, mid, lo)
    // partial logits, Ep apart, which the selection adds in fp64 in that order
    const int S = router_ksplit(T, E, d);
    err = launch_dense(x, T, d, w_split, 3 * Ep, DenseOut::kF32, z_part, nullptr, nullptr, tiles,
                       ntiles, s, S);
    if (err != hipSuccess) return err;
    np = 3 * S;
    row_parts = 3 * S;
    pstride = Ep;
  }
  const int epl = (E + 63) / 64;
  if (epl <= 1)
    select_launch<1>(z_part, np, row_parts, pstride, bias, T, E, k, alpha, logits, topk_idx, topk_w, s);
  else if (epl <= 2)
    select_launch<2>(z_part, np, row_parts, pstride, bias, T, E, k, alpha, logits, topk_idx, topk_w, s);
  else if (epl <= 4)
    select_launch<4>(z_part, np, row_parts, pstride, bias, T, E, k, alpha, logits, topk_idx, topk_w, s);
  else if (epl <= 6)
    select_launch<6>(z_part, np, row_parts, pstride, bias, T, E, k, alpha, logits, topk_idx, topk_w, s);
  else if (epl <= 8)
    select_launch<8>(z_part, np, row_parts, pstride, bias, T, E, k, alpha, logits, topk_idx, topk_w, s);
  else
    select_launch<16>(z_part, np, row_parts, pstride, bias, T, E, k, alpha, logits, topk_idx, topk_w, s);
  return hipGetLastError();
}

}  // namespace moe
