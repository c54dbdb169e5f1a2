// The grouped GEMMs' work list: one entry per row tile of a group (a routed expert's
// segment of the permuted rows, or the shared expert's T rows), built on the device from
// the permutation's offsets.  Used by the GEMM launches and by the permutation launch,
// which can build the list in its own workgroup.  Every definition lives in an unnamed
// namespace: each source file that includes this gets its own copy.
#pragma once

#include "common.h"

namespace moe {
namespace {

// ------------------------------------------------------------------ tile list
// The shared expert's row tiles can be cut into `parts` parts (at most kMaxSharedParts),
// part i placed after the i-th share of the routed experts.  The work list is dealt to the
// 8 XCDs as 8 contiguous runs: with 256-row tiles (prefill) the shared tiles are the
// heaviest work and are spread over all 8 (parts = 8); with 16-row tiles (decode) every
// shared tile reads the whole shared weight matrix, and keeping them together (parts = 1)
// lets them share it in one L2.
constexpr int kMaxSharedParts = 8;

// The list for one set of offsets, built by one workgroup of 1024 threads (every thread
// must call it).  offsets may point to global or LDS memory.
__device__ void build_tiles_block(const int32_t* offsets, int E, int64_t routed_rows,
                                  int64_t shared_rows, int BM, int parts, int64_t capacity,
                                  Tile* __restrict__ tiles, int32_t* __restrict__ ntiles) {
  __shared__ int32_t wsum[16];
  __shared__ int32_t routed_total;
  __shared__ int32_t set_start[kMaxSharedParts + 1];  // routed tiles before expert E*i/P
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int32_t o0 = 0, o1 = 0, n = 0;
  if (tid < E) {
    // clamp: rows must stay inside the grouped block whatever the caller passed
    o0 = min<int64_t>(max(offsets[tid], 0), routed_rows);
    o1 = min<int64_t>(max<int64_t>(offsets[tid + 1], o0), routed_rows);
    n = (o1 - o0 + BM - 1) / BM;
  }
  int32_t v = n;
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
    routed_total = acc;
    // a set with no expert (E = 0 in dense launches, or E < 8) starts after all routed
    // tiles; the first expert of a set overwrites its entry below
    set_start[0] = 0;
    for (int i = 1; i <= parts; ++i) set_start[i] = acc;
  }
  __syncthreads();
  // exclusive prefix of routed tiles before expert tid
  const int32_t before = v + wsum[wave] - n;
  if (tid < E) {
    for (int i = 1; i < parts; ++i)
      if (tid == (int)((int64_t)E * i / parts)) set_start[i] = before;
  }
  __syncthreads();
  // never write past the list, whatever offsets the caller passed (overlapping segments
  // would otherwise multiply the tile count)
  const int64_t ns = (shared_rows + BM - 1) / BM;
  const int32_t R = (int32_t)min<int64_t>(routed_total, capacity - ns);
  // shared tiles placed before routed set s: ns * s / P (parts 0 .. s-1)
  auto shared_before = [&](int s) { return (int32_t)(ns * s / parts); };
  if (tid < E) {
    // the set of expert tid: largest s with E*s/P <= tid
    int s = 0;
    for (int i = 1; i < parts; ++i)
      if (tid >= (int)((int64_t)E * i / parts)) s = i;
    const int32_t start = before + shared_before(s);
    const int32_t cnt = max(0, min(n, R - before));  // routed tiles stop at R
    for (int j = 0; j < cnt; ++j) {
      Tile t;
      t.group = tid;
      t.row_begin = o0 + j * BM;
      t.row_end = min(o0 + (j + 1) * BM, o1);
      t.first = start;
      t.count = cnt;
      t.pad[0] = t.pad[1] = t.pad[2] = 0;
      tiles[start + j] = t;
    }
  }
  // shared part i: tiles ns*i/P .. ns*(i+1)/P of the shared rows, after routed set i
  for (int64_t j = tid; j < ns; j += 1024) {
    int i = 0;
    while (i + 1 < parts && j >= shared_before(i + 1)) ++i;
    const int32_t rs = min(set_start[i + 1], R);  // routed tiles before part i
    const int32_t first = rs + shared_before(i);
    Tile t;
    t.group = E;
    t.row_begin = (int32_t)(routed_rows + j * BM);
    t.row_end = (int32_t)min<int64_t>(routed_rows + (j + 1) * BM, routed_rows + shared_rows);
    t.first = first;
    t.count = shared_before(i + 1) - shared_before(i);
    t.pad[0] = t.pad[1] = t.pad[2] = 0;
    tiles[first + (j - shared_before(i))] = t;
  }
  if (tid == 0) *ntiles = R + (int32_t)ns;
}

__global__ __launch_bounds__(1024) void build_tiles_kernel(const int32_t* __restrict__ offsets,
                                                           TileSpec ts, Tile* __restrict__ tiles,
                                                           int32_t* __restrict__ ntiles) {
  build_tiles_block(offsets, ts.E, ts.routed_rows, ts.shared_rows, ts.BM, ts.parts, ts.capacity,
                    tiles, ntiles);
}

}  // namespace
}  // namespace moe
