// Weighted combine plus the shared expert: out[t] = sum_slot G * E_slot + y_shared[t].
// "Kimi K2 · Transformer blocks", y_routed = sum_i G_i E_i and Delta_ffn = y_routed +
// y_shared; the weighted sum over the k slots in fp32 as in the moe_infer of
// "Kimi K3 · Latent up-projection".  fp32 accumulation in slot order, one bf16 rounding.
//
// Each thread owns 8 consecutive features of one token (32-byte fp32 loads, one 16-byte
// bf16 store);
// a token's k expert rows are gathered through inv_perm.
#include "common.h"

namespace moe {
namespace {

constexpr int kCombineThreads = 256;

template <int KMAX>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    const float* __restrict__ y_routed, const int32_t* __restrict__ inv,
    const float* __restrict__ topk_w, const float* __restrict__ y_shared,
    uint16_t* __restrict__ out, int64_t T, int d, int k) {
  const int nchunk = (d / 8 + kCombineThreads - 1) / kCombineThreads;
  const int64_t t = blockIdx.x / nchunk;
  const int c = ((int)(blockIdx.x % nchunk) * kCombineThreads + threadIdx.x) * 8;
  if (t >= T || c >= d) return;
  const int64_t slots = T * k;
  // all slot indices and weights first, then every row load in flight together
  int32_t p[KMAX];
  float w[KMAX];
#pragma unroll
  for (int s = 0; s < KMAX; ++s) {
    p[s] = -1;
    w[s] = 0.0f;
    if (s < k) {
      p[s] = inv[t * k + s];
      w[s] = topk_w[t * k + s];
    }
  }
  f32x4_t ra[KMAX], rb[KMAX];
#pragma unroll
  for (int s = 0; s < KMAX; ++s) {
    if (p[s] >= 0 && p[s] < slots) {
      const f32x4_t* src = reinterpret_cast<const f32x4_t*>(y_routed + (int64_t)p[s] * d + c);
      ra[s] = src[0];
      rb[s] = src[1];
    } else {
      ra[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      rb[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      w[s] = 0.0f;
    }
  }
  f32x4_t lo = {0.f, 0.f, 0.f, 0.f}, hi = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < KMAX; ++s) {
    if (s >= k) break;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo[i] = fmaf(w[s], ra[s][i], lo[i]);
      hi[i] = fmaf(w[s], rb[s][i], hi[i]);
    }
  }
  if (y_shared != nullptr) {
    const f32x4_t* src = reinterpret_cast<const f32x4_t*>(y_shared + t * d + c);
    lo += src[0];
    hi += src[1];
  }
  u32x4_t o;
  o[0] = f32_to_bf16(lo[0]) | (f32_to_bf16(lo[1]) << 16);
  o[1] = f32_to_bf16(lo[2]) | (f32_to_bf16(lo[3]) << 16);
  o[2] = f32_to_bf16(hi[0]) | (f32_to_bf16(hi[1]) << 16);
  o[3] = f32_to_bf16(hi[2]) | (f32_to_bf16(hi[3]) << 16);
  *reinterpret_cast<u32x4_t*>(out + t * d + c) = o;
}

// Latent variant: u_hat[t] = bf16(RMSNorm(sum_slot G * Y[inv[t, slot]])) with unit gain,
// eps as given ("Kimi K3 · Latent up-projection": the routed sum on the latent width is
// normalised before the up-projection).  One workgroup per token; each thread keeps up
// to CPT 4-wide fp32 chunks of the sum, the sum of squares is reduced in a fixed tree
// order (deterministic), and the row is scaled by 1/sqrt(mean + eps).
template <int KMAX, int CPT>
__global__ __launch_bounds__(kCombineThreads) void combine_rmsnorm_kernel(
    const float* __restrict__ y_routed, const int32_t* __restrict__ inv,
    const float* __restrict__ topk_w, uint16_t* __restrict__ out, int64_t T, int L, int k,
    float eps) {
  __shared__ float wsum[kCombineThreads / 64];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  const int nch = L / 4;
  const int64_t slots = T * k;
  int32_t p[KMAX];
  float w[KMAX];
#pragma unroll
  for (int s = 0; s < KMAX; ++s) {
    p[s] = -1;
    w[s] = 0.0f;
    if (s < k) {
      p[s] = inv[t * k + s];
      w[s] = topk_w[t * k + s];
      if (p[s] < 0 || p[s] >= slots) {
        p[s] = -1;
        w[s] = 0.0f;
      }
    }
  }
  f32x4_t acc[CPT];
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int c = tid + kCombineThreads * j;
    if (c < nch) {
#pragma unroll
      for (int s = 0; s < KMAX; ++s) {
        if (s >= k) break;
        if (p[s] < 0) continue;
        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(y_routed + (int64_t)p[s] * L + 4 * c);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[j][i] = fmaf(w[s], v[i], acc[j][i]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) ss = fmaf(acc[j][i], acc[j][i], ss);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  if ((tid & 63) == 0) wsum[tid >> 6] = ss;
  __syncthreads();
  float tot = 0.0f;
#pragma unroll
  for (int i = 0; i < kCombineThreads / 64; ++i) tot += wsum[i];
  const float scale = 1.0f / sqrtf(tot / (float)L + eps);
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int c = tid + kCombineThreads * j;
    if (c >= nch) continue;
    u32x2_t o;
    o[0] = f32_to_bf16(acc[j][0] * scale) | (f32_to_bf16(acc[j][1] * scale) << 16);
    o[1] = f32_to_bf16(acc[j][2] * scale) | (f32_to_bf16(acc[j][3] * scale) << 16);
    *reinterpret_cast<u32x2_t*>(out + t * L + 4 * c) = o;
  }
}

}  // namespace

hipError_t launch_combine_rmsnorm(const float* y_routed, const int32_t* inv, const float* topk_w,
                                  uint16_t* out, int64_t T, int L, int k, float eps,
                                  hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (L <= 4 * kCombineThreads * 4)
    hipLaunchKernelGGL((combine_rmsnorm_kernel<kMaxTopK, 4>), dim3((unsigned)T),
                       dim3(kCombineThreads), 0, s, y_routed, inv, topk_w, out, T, L, k, eps);
  else
    hipLaunchKernelGGL((combine_rmsnorm_kernel<kMaxTopK, 8>), dim3((unsigned)T),
                       dim3(kCombineThreads), 0, s, y_routed, inv, topk_w, out, T, L, k, eps);
  return hipGetLastError();
}

hipError_t launch_combine(const float* y_routed, const int32_t* inv, const float* topk_w,
                          const float* y_shared, uint16_t* out, int64_t T, int d, int k,
                          hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const int64_t nchunk = (d / 8 + kCombineThreads - 1) / kCombineThreads;
  dim3 grid((unsigned)(nchunk * T));
  hipLaunchKernelGGL(combine_kernel<kMaxTopK>, grid, dim3(kCombineThreads), 0, s, y_routed, inv,
                     topk_w, y_shared, out, T, d, k);
  return hipGetLastError();
}

}  // namespace moe
