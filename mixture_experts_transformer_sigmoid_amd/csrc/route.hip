// Router: z = x W_r^T, s = sigmoid(z), top-k of s + b, gates alpha * s / sum(s).
// "Kimi K2 · Transformer blocks", MoE equations z, s, E_sel, G_i; selection bias and
// bias-free gates as in "nnterp encyclopedia · kimi_k2", "The mixture of experts".
//
// The logits GEMM runs on the bf16 MFMA units without losing fp32 accuracy: each fp32
// router weight is split exactly into three bf16 numbers, w = hi + mid + lo (hi is w
// rounded to bf16, mid the rounded remainder, lo the rest, which fits in bf16's 8
// significant bits), so x W_r^T = x hi^T + x mid^T + x lo^T.  x is bf16, so every
// product is exact in fp32.  Above kRouterSmallT tokens the three partial logits are
// accumulated in fp32 by the grouped-GEMM kernels (one group, 3E outputs) and added in
// fp64 by the selection kernel.  For fewer tokens (decode) router_scores_kernel does the
// split in registers, owns whole logits, applies the sigmoid and the bias, and takes the
// top-k and the gates itself: with at most 16 experts one of its workgroups holds every
// logit of its tokens, and with more the last workgroup of a token block to finish (an
// arrival count per block) selects for the block.
// (The split follows the bf16x3 scheme of Henry, Tang and Heinecke, "Leveraging the
// bfloat16 artificial intelligence datatype for higher-precision computations", 2019.)
#include <math.h>

#include <mutex>
#include <unordered_map>

#include "arrival_slots.h"
#include "common.h"
#include "select.h"

namespace moe {
namespace {

// Arrival counts of the small-batch router: kArrivalBlocks counters (one per 16-token
// block) in each of kArrivalSlots slots, per GPU.  They are zero when the library is
// loaded and the last workgroup of each block puts its counter back to zero, so they are
// zero again whenever no router launch is running.  Each workspace is given a slot of its
// own (arrival_slot below), so calls that may overlap, which need their own workspaces,
// never share counters.
constexpr int kArrivalSlots = 1024;
constexpr int kArrivalBlocks = (int)(kRouterSmallT / 16);
__device__ uint32_t g_arrivals[kArrivalSlots * kArrivalBlocks];

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

// ---------------------------------------------------------------- scores, few tokens
// Up to kRouterSmallT tokens the router is a small GEMM (T x E outputs) whose cost is
// reading the fp32 W_r.  One workgroup owns a 16-token x 16-expert tile of z over the whole
// K, so every logit is complete inside it and the sigmoid and the bias follow in its
// epilogue (no partial logits leave the chip).  Its 16 waves take a sixteenth of K each,
// so that a workgroup keeps many loads in flight; each fp32 router weight is split into
// its hi, mid and lo bf16 parts in registers (no split pass, no bf16 copy of W_r), and the
// three partial products accumulate in three fp32 accumulators.  The 48 per-wave partials
// of a logit are then added in fp64 in a fixed order (wave by wave, hi, mid, lo) and
// rounded to fp32.
// Lane (r, q) of a wave: expert e0 + r and token t0 + r, k 8q .. 8q + 7 of each 32-wide
// step; the weights are the MFMA's A operand, the tokens its B operand, so the lane's
// accumulator holds experts e0 + 4q .. + 3 of token t0 + r.
// With a norm (the block entry point), x is the residual stream x': the waves first take
// the sums of squares of the 16 rows (a row's loads in flight at once, fp64, a fixed
// order), and every operand element is then bf16(fp32(x' * (1 / sqrt(mean + eps)) * gain)),
// the value the norm kernel stores; the workgroups of expert tile 0 store those rows as
// x_ffn for the experts.
// Waves per workgroup x k-steps of loads in flight per wave, swept at the K2 shape (d 7168,
// 384 experts; one box; kernel us at T = 16 / 128 / 512, then with the norm at T = 128):
// 16 x 4: 21.7 / 22.8 / 60.0, 37.6; 16 x 7: 21.3 / 22.3 / 62.5, 71.1 (the norm variant
// spills); 8 x 7: 21.0 / 21.8 / 57.8, 43.2; 8 x 14: 21.7 / 22.4 / 63.4, 73.8 (spills);
// 4 x 14: 22.3 / 23.7 / 61.6, 54.0.
#ifndef MOE_ROUTER_WAVES
#define MOE_ROUTER_WAVES 16
#endif
constexpr int kRouterWaves = MOE_ROUTER_WAVES;
// the epilogue's 256 threads each add one (token, expert) logit; the norm takes 16 rows
static_assert(kRouterWaves >= 4 && kRouterWaves <= 16, "router waves per workgroup");
#ifndef MOE_ROUTER_KU
#define MOE_ROUTER_KU 4
#endif
constexpr int kRouterKU = MOE_ROUTER_KU;   // k-steps of loads issued before their MFMAs
// row pieces (8 elements) per lane that the norm prologue requests at once: rows of up to
// 64 x 16 x 8 = 8192 elements in one batch
constexpr int kRouterNormPieces = 16;

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

__device__ __forceinline__ double sumsq8(const u32x4_t& w, double acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const double a = bf16_to_f32(w[i] & 0xffffu), b = bf16_to_f32(w[i] >> 16);
    acc = fma(a, a, acc);
    acc = fma(b, b, acc);
  }
  return acc;
}

// Eight elements of x' normalised with the row's 1/rms and the gain: fp64 products rounded
// to fp32, then to bf16 (nearest-even both times).
__device__ __forceinline__ u32x4_t norm8(const u32x4_t& v, double rinv, const u32x4_t (&g)[2]) {
  u32x4_t o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float ga = __uint_as_float(g[i >> 1][2 * (i & 1)]);
    const float gb = __uint_as_float(g[i >> 1][2 * (i & 1) + 1]);
    const float a = (float)((double)bf16_to_f32(v[i] & 0xffffu) * rinv * (double)ga);
    const float b = (float)((double)bf16_to_f32(v[i] >> 16) * rinv * (double)gb);
    o[i] = f32_to_bf16(a) | (f32_to_bf16(b) << 16);
  }
  return o;
}

// A float another workgroup wrote, read at device scope (not from a cache line that may be
// stale for this CU).
__device__ __forceinline__ float load_device(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The top-k and the gates of each token of the block (one wave per token, select_topk with
// EPL experts per lane).  With one expert tile (gridDim.y == 1, E <= 16) the workgroup holds
// every score of its tokens and selects from LDS; score and sig are then not written.  With
// more, every workgroup writes its scores and sigmoids to score / sig and adds one to its
// block's arrival count in slot `slot` of g_arrivals (a release at device scope); the
// workgroup that brings the count to gridDim.y is the block's last: it acquires, puts the
// count back to zero and selects from score / sig.  Both ways select from the same fp32
// values, so the routing does not depend on which workgroup selects.  No workgroup waits
// for another.
template <bool NORM, int EPL>
__global__ __launch_bounds__(64 * kRouterWaves) void router_scores_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ gain, float eps,
    uint16_t* __restrict__ x_ffn, const float* __restrict__ w_r, const float* __restrict__ bias,
    int64_t T, int d, int E, float* __restrict__ score, float* __restrict__ sig,
    float* __restrict__ logits, int k, float alpha, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, int slot) {
  constexpr bool kCanBeLocal = EPL == 1;
  __shared__ f32x4_t part[kRouterWaves][3][64];
  __shared__ double rinv_s[16];
  __shared__ float sel_sc[16][16], sel_sg[16][16];
  __shared__ uint32_t last_s;
  const bool local = kCanBeLocal && gridDim.y == 1;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r = lane & 15, q = lane >> 4;
  const int64_t t0 = (int64_t)blockIdx.x * 16;
  const int e0 = blockIdx.y * 16;
  if constexpr (NORM) {
    // wave w: rows t0 + w, t0 + w + kRouterWaves, ...; lane l sums pieces l, l + 64, ...
    // (8 elements each), then the 64 partial sums of a row meet in a fixed butterfly order
    const int npc = d / 8;
    for (int i = wave; i < 16; i += kRouterWaves) {
      const uint16_t* row = x + min<int64_t>(t0 + i, T - 1) * d;
      double ss = 0.0;
      for (int c0 = 0; c0 < npc; c0 += 64 * kRouterNormPieces) {
        u32x4_t v[kRouterNormPieces];
#pragma unroll
        for (int u = 0; u < kRouterNormPieces; ++u)
          v[u] = load16(row + 8 * min(c0 + lane + 64 * u, npc - 1));
#pragma unroll
        for (int u = 0; u < kRouterNormPieces; ++u)
          if (c0 + lane + 64 * u < npc) ss = sumsq8(v[u], ss);
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
      if (lane == 0) rinv_s[i] = 1.0 / sqrt(ss / (double)d + (double)eps);
    }
    __syncthreads();
  }
  const int64_t t = min<int64_t>(t0 + r, T - 1);
  const int e = min(e0 + r, E - 1);
  const float* wrow = w_r + (int64_t)e * d + q * 8;
  const uint16_t* xrow = x + t * d + q * 8;
  const float* grow = NORM ? gain + q * 8 : nullptr;
  const double rinv = NORM ? rinv_s[r] : 1.0;
  uint16_t* xo = (NORM && blockIdx.y == 0 && t0 + r < T) ? x_ffn + t * d + q * 8 : nullptr;
  const int nst = d / 32;
  const int s0 = nst * wave / kRouterWaves, s1 = nst * (wave + 1) / kRouterWaves;
  f32x4_t acc[3] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f},
                    f32x4_t{0.f, 0.f, 0.f, 0.f}};
  auto step = [&](const u32x4_t (&wv)[2], u32x4_t xv, const u32x4_t (&gv)[2], int k) {
    if constexpr (NORM) {
      xv = norm8(xv, rinv, gv);
      if (xo != nullptr) *reinterpret_cast<u32x4_t*>(xo + k) = xv;
    }
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
  auto load_step = [&](int st, u32x4_t (&wv)[2], u32x4_t& xv, u32x4_t (&gv)[2]) {
    const float* wp = wrow + st * 32;
    wv[0] = *reinterpret_cast<const u32x4_t*>(wp);
    wv[1] = *reinterpret_cast<const u32x4_t*>(wp + 4);
    xv = load16(xrow + st * 32);
    if constexpr (NORM) {
      gv[0] = *reinterpret_cast<const u32x4_t*>(grow + st * 32);
      gv[1] = *reinterpret_cast<const u32x4_t*>(grow + st * 32 + 4);
    }
  };
  int st = s0;
  for (; st + kRouterKU <= s1; st += kRouterKU) {
    u32x4_t wv[kRouterKU][2], xv[kRouterKU], gv[kRouterKU][2];
#pragma unroll
    for (int u = 0; u < kRouterKU; ++u) load_step(st + u, wv[u], xv[u], gv[u]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kRouterKU; ++u) step(wv[u], xv[u], gv[u], (st + u) * 32);
  }
  for (; st < s1; ++st) {
    u32x4_t wv[2], xv, gv[2];
    load_step(st, wv, xv, gv);
    step(wv, xv, gv, st * 32);
  }
  // the 48 partials of each logit meet in LDS and are added in fp64, wave by wave, hi,
  // mid, lo
#pragma unroll
  for (int p = 0; p < 3; ++p) part[wave][p][lane] = acc[p];
  __syncthreads();
  if (tid < 256) {
    const int i = tid >> 4, jj = tid & 15;   // token t0 + i, expert e0 + jj
    const int src = (jj >> 2) * 16 + i, reg = jj & 3;
    double zd = 0.0;
#pragma unroll
    for (int w = 0; w < kRouterWaves; ++w)
#pragma unroll
      for (int p = 0; p < 3; ++p) zd += (double)part[w][p][src][reg];
    const int64_t tt = t0 + i;
    const int ee = e0 + jj;
    float v = -INFINITY, s = 0.0f;
    if (tt < T && ee < E) {
      const float z = (float)zd;
      if (logits != nullptr) logits[tt * E + ee] = z;
      s = 1.0f / (1.0f + expf(-z));
      v = s + bias[ee];
      if (v != v) v = -INFINITY;
    }
    sel_sc[i][jj] = v;
    sel_sg[i][jj] = s;
  }
  __syncthreads();
  if (kCanBeLocal && local) {
    // lane l holds expert l (lanes from E on: -inf)
    for (int i = wave; i < 16; i += kRouterWaves) {
      const int64_t tt = t0 + i;
      if (tt >= T) break;
      float sc[1] = {lane < E ? sel_sc[i][lane] : -INFINITY};
      float sg[1] = {lane < E ? sel_sg[i][lane] : 0.0f};
      select_topk<1>(sc, sg, E, k, alpha, lane, topk_idx + tt * k, topk_w + tt * k, nullptr);
    }
    return;
  }
  if (wave == 0) {
    // wave 0 writes the tile (lane: experts e0 + (lane & 15) of tokens t0 + (lane >> 4) +
    // 4 j) and counts the workgroup's arrival with a release at device scope (its stores
    // go out of this XCD's L2 first).  The block's last workgroup acquires at device scope
    // before any of its waves reads the other workgroups' scores; the others return.
    const int ee = e0 + (lane & 15);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = (lane >> 4) + 4 * j;
      const int64_t tt = t0 + i;
      if (tt < T && ee < E) {
        score[tt * E + ee] = sel_sc[i][lane & 15];
        sig[tt * E + ee] = sel_sg[i][lane & 15];
      }
    }
    if (lane == 0) {
      uint32_t* cnt = g_arrivals + (int64_t)slot * kArrivalBlocks + blockIdx.x;
      const uint32_t before =
          __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t last = before + 1 == gridDim.y ? 1u : 0u;
      if (last) {
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      last_s = last;
    }
  }
  __syncthreads();
  if (last_s == 0) return;
  // every workgroup of the block has counted, so all of its scores are out (the barrier
  // orders every wave's loads after wave 0's acquire): lane l holds experts l, l + 64, ...
  // (loads at clamped addresses; experts from E on get score -inf)
  for (int i = wave; i < 16; i += kRouterWaves) {
    const int64_t tt = t0 + i;
    if (tt >= T) break;
    float sc[EPL], sg[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = min(lane + 64 * j, E - 1);
      sc[j] = load_device(score + tt * E + e);
      sg[j] = load_device(sig + tt * E + e);
    }
#pragma unroll
    for (int j = 0; j < EPL; ++j)
      if (lane + 64 * j >= E) {
        sc[j] = -INFINITY;
        sg[j] = 0.0f;
      }
    select_topk<EPL>(sc, sg, E, k, alpha, lane, topk_idx + tt * k, topk_w + tt * k, nullptr);
  }
}

// ---------------------------------------------------------------- top-k + gates
// Above kRouterSmallT tokens: z = the np partial logits (hi, mid, lo of each K slice)
// summed in fp64, rounded to fp32; then as above.
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
  select_topk<EPL>(score, sig, E, k, alpha, lane, topk_idx + t * k, topk_w + t * k, nullptr);
}

// Parts per batch of loads: up to 12 parts in one batch while the loaded values fit in
// registers, else batches of 8.
template <int EPL>
void select_launch(const float* z_part, int np, int row_parts, int pstride, const float* bias,
                   int64_t T, int E, int k, float alpha, float* logits, int32_t* idx, float* w,
                   hipStream_t s) {
  const unsigned grid = (unsigned)((T + 3) / 4);
  if (EPL <= 6 && np <= 12)
    hipLaunchKernelGGL((router_select_kernel<EPL, 12>), dim3(grid), dim3(256), 0, s, z_part, np,
                       row_parts, pstride, bias, T, E, k, alpha, logits, idx, w);
  else
    hipLaunchKernelGGL((router_select_kernel<EPL, 8>), dim3(grid), dim3(256), 0, s, z_part, np,
                       row_parts, pstride, bias, T, E, k, alpha, logits, idx, w);
}

// The slot tables, one per GPU, and the lock that serialises them.
std::mutex g_slot_mu;
std::unordered_map<int, ArrivalSlotTable<kArrivalSlots>> g_slot_tables;

// The arrival slot of a workspace on the device of `s`, where the router will run
// (ArrivalSlotTable; pinned when the call is being captured into a graph on `s`).
hipError_t arrival_slot(const void* ws, hipStream_t s, int* slot) {
  hipDevice_t dev = 0;
  hipError_t err = hipStreamGetDevice(s, &dev);
  if (err != hipSuccess) return err;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  err = hipStreamIsCapturing(s, &cap);
  if (err != hipSuccess) return err;
  std::lock_guard<std::mutex> lock(g_slot_mu);
  const int i =
      g_slot_tables[dev].slot(reinterpret_cast<uintptr_t>(ws), cap != hipStreamCaptureStatusNone);
  if (i < 0) return hipErrorOutOfMemory;
  *slot = i;
  return hipSuccess;
}

}  // namespace

void arrival_release(const void* ws) {
  std::lock_guard<std::mutex> lock(g_slot_mu);
  for (auto& t : g_slot_tables) t.second.release(reinterpret_cast<uintptr_t>(ws));
}

hipError_t launch_router_small(const uint16_t* x, const RouterNorm* norm, const float* w_r,
                               const float* bias, int64_t T, int d, int E, int k, float alpha,
                               float* score, float* sig, float* logits, int32_t* idx, float* w,
                               const void* ws, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (T > kRouterSmallT) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((T + 15) / 16), (unsigned)((E + 15) / 16));
  int slot = 0;
  if (grid.y > 1) {
    const hipError_t err = arrival_slot(ws, s, &slot);
    if (err != hipSuccess) return err;
  }
  const float* gain = norm != nullptr ? norm->gain : nullptr;
  const float eps = norm != nullptr ? norm->eps : 0.0f;
  uint16_t* x_ffn = norm != nullptr ? norm->x_ffn : nullptr;
#define MOE_SCORES(NORM, EPL)                                                                  \
  hipLaunchKernelGGL((router_scores_kernel<NORM, EPL>), grid, dim3(64 * kRouterWaves), 0, s, x, \
                     gain, eps, x_ffn, w_r, bias, T, d, E, score, sig, logits, k, alpha, idx, w, \
                     slot)
#define MOE_SCORES_EPL(NORM)             \
  switch (select_epl(E)) {               \
    case 1: MOE_SCORES(NORM, 1); break;  \
    case 2: MOE_SCORES(NORM, 2); break;  \
    case 4: MOE_SCORES(NORM, 4); break;  \
    case 6: MOE_SCORES(NORM, 6); break;  \
    case 8: MOE_SCORES(NORM, 8); break;  \
    default: MOE_SCORES(NORM, 16); break; \
  }
  if (norm != nullptr) {
    MOE_SCORES_EPL(true)
  } else {
    MOE_SCORES_EPL(false)
  }
#undef MOE_SCORES_EPL
#undef MOE_SCORES
  return hipGetLastError();
}

hipError_t launch_router(const uint16_t* x, const float* w_r, const float* bias, int64_t T, int d,
                         int E, int k, float alpha, uint16_t* w_split, float* z_part,
                         Tile* tiles, int32_t* ntiles, float* logits, int32_t* topk_idx,
                         float* topk_w, const void* ws, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  hipError_t err;
  if (T <= kRouterSmallT) {
    // scores [T, E] and sigmoids [T, E] in z_part
    return launch_router_small(x, nullptr, w_r, bias, T, d, E, k, alpha, z_part, z_part + T * E,
                               logits, topk_idx, topk_w, ws, s);
  }
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
  const int np = 3 * S, row_parts = 3 * S, pstride = Ep;
  switch (select_epl(E)) {
    case 1: select_launch<1>(z_part, np, row_parts, pstride, bias, T, E, k, alpha, logits, topk_idx, topk_w, s); break;
    case 2: select_launch<2>(z_part, np, row_parts, pstride, bias, T, E, k, alpha, logits, topk_idx, topk_w, s); break;
    case 4: select_launch<4>(z_part, np, row_parts, pstride, bias, T, E, k, alpha, logits, topk_idx, topk_w, s); break;
    case 6: select_launch<6>(z_part, np, row_parts, pstride, bias, T, E, k, alpha, logits, topk_idx, topk_w, s); break;
    case 8: select_launch<8>(z_part, np, row_parts, pstride, bias, T, E, k, alpha, logits, topk_idx, topk_w, s); break;
    default: select_launch<16>(z_part, np, row_parts, pstride, bias, T, E, k, alpha, logits, topk_idx, topk_w, s); break;
  }
  return hipGetLastError();
}

}  // namespace moe
