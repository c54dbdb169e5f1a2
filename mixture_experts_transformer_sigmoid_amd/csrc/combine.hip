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

}  // namespace

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
