// Router: z = x W_r^T (fp32), s = sigmoid(z), top-k of s + b, gates alpha * s / sum(s).
// "Kimi K2 · Transformer blocks", MoE equations z, s, E_sel, G_i; selection bias and
// bias-free gates as in "nnterp encyclopedia · kimi_k2", "The mixture of experts".
#include <math.h>

#include "common.h"

namespace moe {
namespace {

// ---------------------------------------------------------------- logits GEMM
// One workgroup computes a TM x TE block of z.  256 threads as 16 x 16; thread (ty, tx)
// owns tokens ty + 16 i and experts tx + 16 j.  K is walked in chunks of 32 staged in
// LDS as fp32; each chunk's 32 products are summed in fp32 and the chunk sums are added
// in fp64, so z carries ~1e-7 absolute error whatever d is (the top-k decision on
// sigmoid(z) + b needs z well inside 1e-6).
template <int TM, int TE>
__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                            const float* __restrict__ w_r,
                                                            int64_t T, int d, int E,
                                                            float* __restrict__ z) {
  constexpr int KC = 32;
  constexpr int RM = TM / 16, RE = TE / 16;
  __shared__ float xs[KC][TM];
  __shared__ float ws[KC][TE + 4];

  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int64_t t0 = (int64_t)blockIdx.y * TM;
  const int e0 = blockIdx.x * TE;

  double acc[RM][RE];
#pragma unroll
  for (int i = 0; i < RM; ++i)
#pragma unroll
    for (int j = 0; j < RE; ++j) acc[i][j] = 0.0;

  for (int k0 = 0; k0 < d; k0 += KC) {
    // stage x: TM rows x 32 bf16 = TM*4 16-byte pieces
    for (int piece = tid; piece < TM * 4; piece += 256) {
      const int m = piece >> 2, kk = (piece & 3) * 8;
      int64_t t = t0 + m;
      if (t >= T) t = T - 1;
      const u32x4_t v = load16(x + t * d + k0 + kk);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        xs[kk + 2 * q][m] = bf16_to_f32(v[q] & 0xffffu);
        xs[kk + 2 * q + 1][m] = bf16_to_f32(v[q] >> 16);
      }
    }
    // stage W_r: TE rows x 32 fp32 = TE*8 16-byte pieces
    for (int piece = tid; piece < TE * 8; piece += 256) {
      const int e = piece >> 3, kk = (piece & 7) * 4;
      int ee = e0 + e;
      if (ee >= E) ee = E - 1;
      const float4 v = *reinterpret_cast<const float4*>(w_r + (int64_t)ee * d + k0 + kk);
      ws[kk + 0][e] = v.x;
      ws[kk + 1][e] = v.y;
      ws[kk + 2][e] = v.z;
      ws[kk + 3][e] = v.w;
    }
    __syncthreads();
    float part[RM][RE];
#pragma unroll
    for (int i = 0; i < RM; ++i)
#pragma unroll
      for (int j = 0; j < RE; ++j) part[i][j] = 0.0f;
#pragma unroll 8
    for (int kk = 0; kk < KC; ++kk) {
      float xv[RM], wv[RE];
#pragma unroll
      for (int i = 0; i < RM; ++i) xv[i] = xs[kk][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < RE; ++j) wv[j] = ws[kk][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < RM; ++i)
#pragma unroll
        for (int j = 0; j < RE; ++j) part[i][j] = fmaf(xv[i], wv[j], part[i][j]);
    }
#pragma unroll
    for (int i = 0; i < RM; ++i)
#pragma unroll
      for (int j = 0; j < RE; ++j) acc[i][j] += (double)part[i][j];
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < RM; ++i) {
    const int64_t t = t0 + ty + 16 * i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < RE; ++j) {
      const int e = e0 + tx + 16 * j;
      if (e < E) z[t * E + e] = (float)acc[i][j];
    }
  }
}

// ---------------------------------------------------------------- top-k + gates
// One wave per token.  Lane l holds experts l, l + 64, ...; k rounds of a wave-wide
// argmax over (score, -index) pick the experts (ties to the lower index, NaN scores
// treated as -inf); the gates use the sigmoid without the bias.
template <int EPL>
__global__ __launch_bounds__(256) void router_select_kernel(const float* __restrict__ z,
                                                            const float* __restrict__ bias,
                                                            int64_t T, int E, int k, float alpha,
                                                            int32_t* __restrict__ topk_idx,
                                                            float* __restrict__ topk_w) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;

  float score[EPL], sig[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    if (e < E) {
      const float s = 1.0f / (1.0f + expf(-z[t * E + e]));
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
void select_launch(const float* z, const float* bias, int64_t T, int E, int k, float alpha,
                   int32_t* idx, float* w, hipStream_t s) {
  const unsigned grid = (unsigned)((T + 3) / 4);
  hipLaunchKernelGGL(router_select_kernel<EPL>, dim3(grid), dim3(256), 0, s, z, bias, T, E, k,
                     alpha, idx, w);
}

}  // namespace

hipError_t launch_router(const uint16_t* x, const float* w_r, const float* bias, int64_t T, int d,
                         int E, int k, float alpha, float* logits, int32_t* topk_idx,
                         float* topk_w, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (T <= 512) {
    dim3 grid((E + 15) / 16, (unsigned)((T + 31) / 32));
    hipLaunchKernelGGL((router_logits_kernel<32, 16>), grid, dim3(256), 0, s, x, w_r, T, d, E,
                       logits);
  } else {
    dim3 grid((E + 63) / 64, (unsigned)((T + 63) / 64));
    hipLaunchKernelGGL((router_logits_kernel<64, 64>), grid, dim3(256), 0, s, x, w_r, T, d, E,
                       logits);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int epl = (E + 63) / 64;
  if (epl <= 1)
    select_launch<1>(logits, bias, T, E, k, alpha, topk_idx, topk_w, s);
  else if (epl <= 2)
    select_launch<2>(logits, bias, T, E, k, alpha, topk_idx, topk_w, s);
  else if (epl <= 4)
    select_launch<4>(logits, bias, T, E, k, alpha, topk_idx, topk_w, s);
  else if (epl <= 6)
    select_launch<6>(logits, bias, T, E, k, alpha, topk_idx, topk_w, s);
  else if (epl <= 8)
    select_launch<8>(logits, bias, T, E, k, alpha, topk_idx, topk_w, s);
  else
    select_launch<16>(logits, bias, T, E, k, alpha, topk_idx, topk_w, s);
  return hipGetLastError();
}

}  // namespace moe
