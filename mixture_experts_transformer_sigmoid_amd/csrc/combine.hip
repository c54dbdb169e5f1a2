// Weighted combine plus the shared expert: out[t] = sum_slot G * E_slot + y_shared[t].
// "Kimi K2 · Transformer blocks", y_routed = sum_i G_i E_i and Delta_ffn = y_routed +
// y_shared; the weighted sum over the k slots in fp32 as in the moe_infer of
// "Kimi K3 · Latent up-projection".  fp32 accumulation in slot order, one bf16 rounding.
//
// Each thread owns 8 consecutive features of one token (32-byte fp32 loads, or 24 bytes
// of packed 24-bit floats; one 16-byte bf16 store), a block 1,024 features; a token's k
// expert rows are gathered through inv_perm.
#include "common.h"

namespace moe {
namespace {

constexpr int kCombineThreads = 256;
// combine_kernel: 128 threads, 1,024 features per block (7 blocks per token at d = 7168,
// none idle); at the K2 prefill shape 414 us against 437 us with 256 threads per block
constexpr int kGatherThreads = 128;

// Features c .. c + 7 of expert row `row` (fp32 rows of d, or with Y24 packed 24-bit rows
// of 3 d bytes).
template <bool Y24>
__device__ __forceinline__ void load_y8(const void* y, int64_t row, int d, int c, f32x4_t& a,
                                        f32x4_t& b) {
  if constexpr (Y24) {
    const F24x4* src = reinterpret_cast<const F24x4*>(static_cast<const uint8_t*>(y) +
                                                      (row * d + c) * 3);
    a = unpack_f24x4(src[0]);
    b = unpack_f24x4(src[1]);
  } else {
    const f32x4_t* src = reinterpret_cast<const f32x4_t*>(static_cast<const float*>(y) +
                                                          row * d + c);
    a = src[0];
    b = src[1];
  }
}

template <int KMAX, bool Y24>
__global__ __launch_bounds__(kGatherThreads) void combine_kernel(
    const void* __restrict__ y_routed, const int32_t* __restrict__ inv,
    const float* __restrict__ topk_w, const void* __restrict__ y_shared,
    const uint16_t* __restrict__ residual, uint16_t* __restrict__ out, int64_t T, int d, int k) {
  const int nchunk = (d / 8 + kGatherThreads - 1) / kGatherThreads;
  const int64_t t = blockIdx.x / nchunk;
  const int c = ((int)(blockIdx.x % nchunk) * kGatherThreads + threadIdx.x) * 8;
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
      load_y8<Y24>(y_routed, p[s], d, c, ra[s], rb[s]);
    } else {
      ra[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      rb[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      w[s] = 0.0f;
    }
  }
  // the shared expert's row and the residual are requested before any of the loads above
  // is waited for (issued after the sums, they would cost a second round trip)
  f32x4_t sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
  u32x4_t v = {0u, 0u, 0u, 0u};
  if (y_shared != nullptr) load_y8<Y24>(y_shared, t, d, c, sa, sb);
  if (residual != nullptr) v = load16(residual + t * d + c);
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
    lo += sa;
    hi += sb;
  }
  if (residual != nullptr) {
    // x_{n+1} = x'_n + Delta_ffn, added in fp32 before the one bf16 rounding
    lo[0] += bf16_to_f32(v[0] & 0xffffu);
    lo[1] += bf16_to_f32(v[0] >> 16);
    lo[2] += bf16_to_f32(v[1] & 0xffffu);
    lo[3] += bf16_to_f32(v[1] >> 16);
    hi[0] += bf16_to_f32(v[2] & 0xffffu);
    hi[1] += bf16_to_f32(v[2] >> 16);
    hi[2] += bf16_to_f32(v[3] & 0xffffu);
    hi[3] += bf16_to_f32(v[3] >> 16);
  }
  u32x4_t o;
  o[0] = f32_to_bf16(lo[0]) | (f32_to_bf16(lo[1]) << 16);
  o[1] = f32_to_bf16(lo[2]) | (f32_to_bf16(lo[3]) << 16);
  o[2] = f32_to_bf16(hi[0]) | (f32_to_bf16(hi[1]) << 16);
  o[3] = f32_to_bf16(hi[2]) | (f32_to_bf16(hi[3]) << 16);
  *reinterpret_cast<u32x4_t*>(out + t * d + c) = o;
}

// Latent variant: u_hat[t] = RMSNorm(sum_slot G * Y[inv[t, slot]]) with unit gain, eps as
// given ("Kimi K3 · Latent up-projection": the routed sum on the latent width is
// normalised before the up-projection).  Y holds the routed rows as packed 24-bit floats
// (3 L bytes each).  One workgroup per token; each thread keeps up to CPT 4-wide fp32
// chunks of the sum, the sum of squares is reduced in a fixed tree
// order (deterministic), and the row is scaled by 1/sqrt(mean + eps).  u_hat is the
// up-projection's MFMA operand: rounded to bf16 once (rows of L), or with TWO in two bf16
// parts, [bf16(u_hat) | bf16(rest)] (rows of 2L).
template <int KMAX, int CPT, bool TWO>
__global__ __launch_bounds__(kCombineThreads) void combine_rmsnorm_kernel(
    const void* __restrict__ y_routed, const int32_t* __restrict__ inv,
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
  // every row piece of the token is requested before the first add: loads at clamped
  // in-range addresses (a dropped slot reads row 0 and its value is replaced by 0), so
  // that no load sits behind a branch and waits alone
  f32x4_t v[CPT][KMAX];
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int c = min(tid + kCombineThreads * j, nch - 1);
#pragma unroll
    for (int s = 0; s < KMAX; ++s) {
      const int64_t e = (int64_t)max(p[s], 0) * L + 4 * c;  // first element of the piece
      v[j][s] = unpack_f24x4(
          *reinterpret_cast<const F24x4*>(static_cast<const uint8_t*>(y_routed) + e * 3));
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  f32x4_t acc[CPT];
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KMAX; ++s) {
      // a dropped slot, or one past k (weight 0, index -1), adds fma(0, 0, acc) = acc: the
      // same bits as skipping it
      const bool ok = p[s] >= 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[j][i] = fmaf(w[s], ok ? v[j][s][i] : 0.0f, acc[j][i]);
    }
    if (tid + kCombineThreads * j < nch) {
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
    f32x4_t u;
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = acc[j][i] * scale;
    u32x2_t hi, lo;
    hi[0] = f32_to_bf16(u[0]) | (f32_to_bf16(u[1]) << 16);
    hi[1] = f32_to_bf16(u[2]) | (f32_to_bf16(u[3]) << 16);
    // the remainders are exact in fp32
    lo[0] = f32_to_bf16(u[0] - bf16_to_f32(hi[0] & 0xffffu)) |
            (f32_to_bf16(u[1] - bf16_to_f32(hi[0] >> 16)) << 16);
    lo[1] = f32_to_bf16(u[2] - bf16_to_f32(hi[1] & 0xffffu)) |
            (f32_to_bf16(u[3] - bf16_to_f32(hi[1] >> 16)) << 16);
    if constexpr (TWO) {
      uint16_t* row = out + t * 2 * L;
      *reinterpret_cast<u32x2_t*>(row + 4 * c) = hi;
      *reinterpret_cast<u32x2_t*>(row + L + 4 * c) = lo;
    } else {
      *reinterpret_cast<u32x2_t*>(out + t * L + 4 * c) = hi;
    }
  }
}

}  // namespace

hipError_t launch_combine_rmsnorm(const void* y_routed, const int32_t* inv, const float* topk_w,
                                  uint16_t* out, int64_t T, int L, int k, float eps,
                                  bool two_part, hipStream_t s) {
  if (T <= 0) return hipSuccess;
#define MOE_CRN(CPT, TWO)                                                                   \
  hipLaunchKernelGGL((combine_rmsnorm_kernel<kMaxTopK, CPT, TWO>), dim3((unsigned)T),        \
                     dim3(kCombineThreads), 0, s, y_routed, inv, topk_w, out, T, L, k, eps)
  if (L <= 4 * kCombineThreads * 4) {
    if (two_part) MOE_CRN(4, true);
    else MOE_CRN(4, false);
  } else {
    if (two_part) MOE_CRN(8, true);
    else MOE_CRN(8, false);
  }
#undef MOE_CRN
  return hipGetLastError();
}

hipError_t launch_combine(const void* y_routed, const int32_t* inv, const float* topk_w,
                          const void* y_shared, const uint16_t* residual, uint16_t* out,
                          int64_t T, int d, int k, hipStream_t s, bool y24) {
  if (T <= 0) return hipSuccess;
  const int64_t nchunk = (d / 8 + kGatherThreads - 1) / kGatherThreads;
  dim3 grid((unsigned)(nchunk * T));
  if (y24)
    hipLaunchKernelGGL((combine_kernel<kMaxTopK, true>), grid, dim3(kGatherThreads), 0, s,
                       y_routed, inv, topk_w, y_shared, residual, out, T, d, k);
  else
    hipLaunchKernelGGL((combine_kernel<kMaxTopK, false>), grid, dim3(kGatherThreads), 0, s,
                       y_routed, inv, topk_w, y_shared, residual, out, T, d, k);
  return hipGetLastError();
}

// Pre-MoE RMSNorm: x_ffn[t] = bf16(x'[t] / sqrt(mean(x'[t]^2) + eps) * gain), one
// workgroup per token.  The arithmetic is fp64 (sum of squares in a fixed tree order,
// then the scaling), rounded once to fp32 and then to bf16: the normalised row feeds the
// router, whose top-k decision would turn on a one-ulp difference in any element, and in
// fp64 the result does not depend on the summation order to within bf16 rounding.
// The first kNormVec 8-element pieces of each thread (the whole row up to d = 8192), and
// the gain values that scale them (two 16-byte loads per piece), are requested at once and
// kept in registers for the scaling pass; loads at clamped in-range addresses, so that
// none sits behind a branch.  Wider rows loop over the rest.
constexpr int kNormVec = 4;

__global__ __launch_bounds__(kCombineThreads) void rmsnorm_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ gain, uint16_t* __restrict__ out,
    int d, float eps) {
  __shared__ double wsum[kCombineThreads / 64];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  const uint16_t* row = x + t * d;
  constexpr int kSpan = kCombineThreads * 8;  // elements per pass of the workgroup
  u32x4_t v[kNormVec];
  f32x4_t gv[kNormVec][2];
#pragma unroll
  for (int j = 0; j < kNormVec; ++j) {
    const int c = min(tid * 8 + j * kSpan, d - 8);
    v[j] = load16(row + c);
    gv[j][0] = *reinterpret_cast<const f32x4_t*>(gain + c);
    gv[j][1] = *reinterpret_cast<const f32x4_t*>(gain + c + 4);
  }
  auto sumsq = [](const u32x4_t& w, double acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const double a = bf16_to_f32(w[i] & 0xffffu), b = bf16_to_f32(w[i] >> 16);
      acc = fma(a, a, acc);
      acc = fma(b, b, acc);
    }
    return acc;
  };
  double ss = 0.0;
#pragma unroll
  for (int j = 0; j < kNormVec; ++j)
    if (tid * 8 + j * kSpan < d) ss = sumsq(v[j], ss);
  for (int c = tid * 8 + kNormVec * kSpan; c < d; c += kSpan) ss = sumsq(load16(row + c), ss);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  if ((tid & 63) == 0) wsum[tid >> 6] = ss;
  __syncthreads();
  double tot = 0.0;
#pragma unroll
  for (int i = 0; i < kCombineThreads / 64; ++i) tot += wsum[i];
  const double inv_rms = 1.0 / sqrt(tot / (double)d + (double)eps);
  // element 2i of the piece with gain g[i >> 1][(2i) & 3], element 2i + 1 with the next
  auto scale_store = [&](const u32x4_t& w, const f32x4_t (&g)[2], int c) {
    u32x4_t o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float ga = g[i >> 1][(2 * i) & 3], gb = g[i >> 1][(2 * i + 1) & 3];
      const float a = (float)((double)bf16_to_f32(w[i] & 0xffffu) * inv_rms * (double)ga);
      const float b = (float)((double)bf16_to_f32(w[i] >> 16) * inv_rms * (double)gb);
      o[i] = f32_to_bf16(a) | (f32_to_bf16(b) << 16);
    }
    *reinterpret_cast<u32x4_t*>(out + t * d + c) = o;
  };
#pragma unroll
  for (int j = 0; j < kNormVec; ++j)
    if (tid * 8 + j * kSpan < d) scale_store(v[j], gv[j], tid * 8 + j * kSpan);
  for (int c = tid * 8 + kNormVec * kSpan; c < d; c += kSpan) {
    const f32x4_t g[2] = {*reinterpret_cast<const f32x4_t*>(gain + c),
                          *reinterpret_cast<const f32x4_t*>(gain + c + 4)};
    scale_store(load16(row + c), g, c);
  }
}

hipError_t launch_rmsnorm(const uint16_t* x, const float* gain, uint16_t* out, int64_t T, int d,
                          float eps, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(rmsnorm_kernel, dim3((unsigned)T), dim3(kCombineThreads), 0, s, x, gain, out,
                     d, eps);
  return hipGetLastError();
}

}  // namespace moe
