// Token permutation: group the T*k (token, slot) pairs by expert.
// "Kimi K3 · Latent up-projection", moe_infer: tokens per expert, the slots sorted by
// expert, each expert's rows a contiguous segment at the running sum of the counts.
//
// Three small launches, all deterministic and with no float work:
//   count   one workgroup per 256 tokens; each wave marks, per expert, which of its 64
//           tokens chose it (a 64-bit LDS mask per expert); hist[b][e] = popcount sum
//   scan    one workgroup: per-expert running sums over the blocks (base[b][e]), the
//           counts, and the exclusive scan over experts (offsets)
//   scatter rebuilds the masks; a slot's row is offsets[e] + base[b][e] + the tokens of
//           earlier waves of the block + popcount(mask & lanes-below): token-ascending
//           order inside every segment, with no sequential loop anywhere.
// Up to 256 tokens (one count block, decode) one workgroup runs the three phases in a
// single launch, and can build the grouped GEMMs' tile list from the new offsets at its
// end: each of those launches costs a few microseconds of latency for far less work.
#include "common.h"
#include "tiles.h"

namespace moe {
namespace {

constexpr int kTokPerBlock = 256;

// Fill the per-wave expert masks of one 256-token block.  Returns in slot_e[] the expert
// of each of this thread's slots, or -1 for a dropped slot (index out of range, or the
// same expert as an earlier slot of the token).
__device__ __forceinline__ void build_masks(const int32_t* __restrict__ topk_idx, int64_t T, int E,
                                            int k, unsigned long long (*masks)[kMaxExperts],
                                            int* slot_e) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int i = tid; i < 4 * E; i += kTokPerBlock) masks[i / E][i % E] = 0ull;
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * kTokPerBlock + tid;
#pragma unroll
  for (int s = 0; s < kMaxTopK; ++s) {
    slot_e[s] = -1;
    if (s < k && t < T) {
      const int e = topk_idx[t * k + s];
      bool ok = (e >= 0 && e < E);
#pragma unroll
      for (int q = 0; q < kMaxTopK; ++q)
        if (q < s && slot_e[q] == e) ok = false;
      if (ok) {
        slot_e[s] = e;
        atomicOr(&masks[wave][e], 1ull << lane);
      }
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(kTokPerBlock) void permute_count_kernel(
    const int32_t* __restrict__ topk_idx, int64_t T, int E, int k, int32_t* __restrict__ hist) {
  __shared__ unsigned long long masks[4][kMaxExperts];
  int slot_e[kMaxTopK];
  build_masks(topk_idx, T, E, k, masks, slot_e);
  for (int e = threadIdx.x; e < E; e += kTokPerBlock) {
    const int c = __popcll(masks[0][e]) + __popcll(masks[1][e]) + __popcll(masks[2][e]) +
                  __popcll(masks[3][e]);
    hist[(int64_t)blockIdx.x * E + e] = c;
  }
}

__global__ __launch_bounds__(1024) void permute_scan_kernel(const int32_t* __restrict__ hist,
                                                            int64_t nblocks, int E,
                                                            int64_t slots,
                                                            int32_t* __restrict__ base,
                                                            int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ perm) {
  __shared__ int32_t sc[kMaxExperts];
  __shared__ int32_t wsum[16];
  const int tid = threadIdx.x;
  int32_t run = 0;
  if (tid < E) {
    // 8 independent loads in flight per step; the running sum follows
    for (int64_t b0 = 0; b0 < nblocks; b0 += 8) {
      int32_t h[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) h[j] = (b0 + j < nblocks) ? hist[(b0 + j) * E + tid] : 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (b0 + j < nblocks) base[(b0 + j) * E + tid] = run;
        run += h[j];
      }
    }
    counts[tid] = run;
  }
  // exclusive scan of run over experts: wave-level inclusive scan, then across waves
  const int lane = tid & 63, wave = tid >> 6;
  int32_t v = (tid < E) ? run : 0;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t o = __shfl_up(v, off);
    if (lane >= off) v += o;
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  if (tid == 0) {
    int32_t acc = 0;
    for (int w = 0; w < 16; ++w) {
      const int32_t x = wsum[w];
      wsum[w] = acc;
      acc += x;
    }
  }
  __syncthreads();
  const int32_t incl = v + wsum[wave];
  if (tid < E) {
    offsets[tid] = incl - run;
    sc[tid] = incl;
  }
  if (tid == E - 1) offsets[E] = incl;
  __syncthreads();
  const int64_t total = sc[E - 1];
  for (int64_t p = total + tid; p < slots; p += 1024) perm[p] = -1;
}

__global__ __launch_bounds__(kTokPerBlock) void permute_scatter_kernel(
    const int32_t* __restrict__ topk_idx, int64_t T, int E, int k,
    const int32_t* __restrict__ base, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
  __shared__ unsigned long long masks[4][kMaxExperts];
  int slot_e[kMaxTopK];
  build_masks(topk_idx, T, E, k, masks, slot_e);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t t = (int64_t)blockIdx.x * kTokPerBlock + tid;
  if (t >= T) return;
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int s = 0; s < kMaxTopK; ++s) {
    if (s >= k) break;
    const int e = slot_e[s];
    const int64_t slot = t * k + s;
    if (e < 0) {
      inv[slot] = -1;
      continue;
    }
    int r = __popcll(masks[wave][e] & below);
    for (int w = 0; w < wave; ++w) r += __popcll(masks[w][e]);
    const int32_t pos = offsets[e] + base[(int64_t)blockIdx.x * E + e] + r;
    perm[pos] = (int32_t)slot;
    inv[slot] = pos;
  }
}

// All three phases for T <= 256 in one workgroup of 1024 threads: the first 256 threads
// (waves 0-3) own one token each, as in the count and scatter blocks, and with a single
// block every base is 0.  The results equal the three-launch path's, element by element.
// With tiles non-null the workgroup then builds the tile list of ts from the offsets.
__global__ __launch_bounds__(1024) void permute_small_kernel(
    const int32_t* __restrict__ topk_idx, int64_t T, int E, int k, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv,
    TileSpec ts, Tile* __restrict__ tiles, int32_t* __restrict__ ntiles) {
  __shared__ unsigned long long masks[4][kMaxExperts];
  __shared__ int32_t soff[kMaxExperts + 1];
  __shared__ int32_t wsum[16];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int i = tid; i < 4 * E; i += 1024) masks[i / E][i % E] = 0ull;
  __syncthreads();
  const bool tok = tid < kTokPerBlock && tid < T;
  int slot_e[kMaxTopK];
#pragma unroll
  for (int s = 0; s < kMaxTopK; ++s) {
    slot_e[s] = -1;
    if (s < k && tok) {
      const int e = topk_idx[(int64_t)tid * k + s];
      bool ok = (e >= 0 && e < E);
#pragma unroll
      for (int q = 0; q < kMaxTopK; ++q)
        if (q < s && slot_e[q] == e) ok = false;
      if (ok) {
        slot_e[s] = e;
        atomicOr(&masks[wave][e], 1ull << lane);
      }
    }
  }
  __syncthreads();
  // counts, then their exclusive scan over experts (wave scans, then across the waves)
  int32_t c = 0;
  if (tid < E)
    c = __popcll(masks[0][tid]) + __popcll(masks[1][tid]) + __popcll(masks[2][tid]) +
        __popcll(masks[3][tid]);
  int32_t v = c;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t o = __shfl_up(v, off);
    if (lane >= off) v += o;
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  if (tid == 0) {
    int32_t acc = 0;
    for (int w = 0; w < 16; ++w) {
      const int32_t x = wsum[w];
      wsum[w] = acc;
      acc += x;
    }
  }
  __syncthreads();
  const int32_t incl = v + wsum[wave];
  if (tid < E) {
    counts[tid] = c;
    offsets[tid] = incl - c;
    soff[tid] = incl - c;
  }
  if (tid == E - 1) {
    offsets[E] = incl;
    soff[E] = incl;
  }
  __syncthreads();
  const int64_t slots = T * k;
  for (int64_t p = soff[E] + tid; p < slots; p += 1024) perm[p] = -1;
  if (tok) {
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s) {
      if (s >= k) break;
      const int e = slot_e[s];
      const int64_t slot = (int64_t)tid * k + s;
      if (e < 0) {
        inv[slot] = -1;
        continue;
      }
      int r = __popcll(masks[wave][e] & below);
      for (int w = 0; w < wave; ++w) r += __popcll(masks[w][e]);
      const int32_t pos = soff[e] + r;
      perm[pos] = (int32_t)slot;
      inv[slot] = pos;
    }
  }
  if (tiles != nullptr)
    build_tiles_block(soff, ts.E, ts.routed_rows, ts.shared_rows, ts.BM, ts.parts, ts.capacity,
                      tiles, ntiles);
}

}  // namespace

int64_t permute_blocks(int64_t T) { return (T + kTokPerBlock - 1) / kTokPerBlock; }

hipError_t launch_permute(const int32_t* topk_idx, int64_t T, int E, int k, int32_t* hist,
                          int32_t* base, int32_t* counts, int32_t* offsets, int32_t* perm,
                          int32_t* inv, hipStream_t s, const TileSpec* ts, Tile* tiles,
                          int32_t* ntiles) {
  if (T <= kTokPerBlock) {
    hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(1024), 0, s, topk_idx, T, E, k, counts,
                       offsets, perm, inv, ts != nullptr ? *ts : TileSpec{},
                       ts != nullptr ? tiles : nullptr, ntiles);
    return hipGetLastError();
  }
  const int64_t nb = permute_blocks(T);
  if (nb > 0) {
    hipLaunchKernelGGL(permute_count_kernel, dim3((unsigned)nb), dim3(kTokPerBlock), 0, s,
                       topk_idx, T, E, k, hist);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(1024), 0, s, hist, nb, E, T * k, base,
                     counts, offsets, perm);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || nb == 0) return err;
  hipLaunchKernelGGL(permute_scatter_kernel, dim3((unsigned)nb), dim3(kTokPerBlock), 0, s,
                     topk_idx, T, E, k, base, offsets, perm, inv);
  err = hipGetLastError();
  if (err != hipSuccess || ts == nullptr) return err;
  hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(1024), 0, s, offsets, *ts, tiles, ntiles);
  return hipGetLastError();
}

}  // namespace moe
