// Grouped-GEMM plumbing shared by the bf16 and FP8 expert kernels: the argument block,
// the on-device tile list, the XCD-aware work mapping, row gathering and the epilogues.
// Every definition lives in an unnamed namespace: each source file that includes this
// gets its own copy.
#pragma once

#include "common.h"
#include "tiles.h"

namespace moe {
namespace {

// Epilogue of a GEMM launch.
enum Epi : int {
  kSwiGLU = 0,   // two weight matrices (W1, W3): h = bf16(silu(g) * u) into C
  kF32 = 1,      // fp32 rows into Y (grouped rows) or Ys (the last group's rows)
  kBF16 = 2,     // bf16 rows into C
  kAddBF16 = 3,  // bf16(acc + R[row]) into C, R fp32 with the same layout
  kF24 = 4,      // packed 24-bit float rows (3 N bytes, F24x4 groups) into Y / Ys
};

struct FfnArgs {
  const uint16_t* A;      // gate/up: x [T, K]; down: h [rows, K]
  const int32_t* perm;    // gate/up: slot id of each grouped row
  int64_t routed_rows;    // T*k: rows at or past this index belong to the shared expert
  const uint16_t* B1;     // routed weights [E, N, K] (w1, or w2 for down)
  const uint16_t* B3;     // routed w3 [E, N, K] (gate/up)
  const uint16_t* S1;     // shared weights [N, K] (ws1, or ws2 for down)
  const uint16_t* S3;     // shared ws3 (gate/up)
  uint16_t* C;            // gate/up: h [rows, N] bf16
  float* Y;               // down: y_routed [T*k, N] fp32 (kF24: 3 N bytes per row)
  float* Ys;              // down: y_shared [T, N] fp32 (kF24: 3 N bytes per row)
  const Tile* tiles;
  const int32_t* ntiles;
  int32_t k;              // slots per token (gate/up gather: token = slot / k)
  int32_t N, K, E;
  int32_t ksplit;         // 256-row kernel, fp32 output: K slices (0 or 1: none)
  int32_t ldc;            // row stride of Ys (0: N); slice j writes from column j N
  int32_t wk;             // > 0: A in two bf16 parts ([hi | lo], K = 2 wk) and weight rows
                          // of wk; reduction index k reads weight column k mod wk
  int32_t hsplit;         // gate/up: write h in two bf16 parts, rows [hi | lo] of 2N
  int64_t a_rows;         // rows of A (gate/up: tokens of x)
  const float* R;         // kAddBF16: fp32 rows added before the bf16 store
  // FP8 kernels only: E4M3 codes with the layouts of B1, B3, S1, S3, and their fp32
  // scales, one per 128 x 128 block ([E, N/128, K/128] routed, [N/128, K/128] shared)
  const uint8_t* Q1;
  const uint8_t* Q3;
  const uint8_t* QS1;
  const uint8_t* QS3;
  const float* B1s;
  const float* B3s;
  const float* S1s;
  const float* S3s;
};

// Work item of this workgroup (see the ordering above).  False: nothing to do.
__device__ __forceinline__ bool map_work(const FfnArgs& a, int NB, Tile& tile, int& nb) {
  const int32_t nt = *a.ntiles;
  const int64_t total = (int64_t)nt * NB;
  const int64_t per = (total + 7) / 8;
  const int64_t b = blockIdx.x;
  if (b >= 8 * per) return false;
  const int64_t L = (b & 7) * per + (b >> 3);
  if (L >= total) return false;
  const Tile t0 = a.tiles[L / NB];
  const int64_t local = L - (int64_t)t0.first * NB;
  const int j = (int)(local % t0.count);
  nb = (int)(local / t0.count);
  tile = a.tiles[t0.first + j];
  return true;
}

// Row p of the grouped order -> its activation row.
__device__ __forceinline__ const uint16_t* act_row(const FfnArgs& a, bool gateup, int64_t p) {
  if (!gateup) return a.A + p * a.K;
  int64_t tok;
  if (p < a.routed_rows) {
    int64_t sl = a.perm[p];
    if (sl < 0 || sl >= a.routed_rows) sl = 0;
    tok = sl / a.k;
  } else {
    tok = p - a.routed_rows;
  }
  return a.A + tok * a.K;
}

// Four consecutive h values as bf16 at dst; with lo non-null also their remainders
// bf16(h - bf16(h)) at lo (the remainder is exact in fp32, its rounding leaves h with 16
// significant bits in the two parts).
__device__ __forceinline__ void store_h4(uint16_t* dst, uint16_t* lo, f32x4_t v) {
  u32x2_t packed;
  packed[0] = pack_bf16x2(v[0], v[1]);
  packed[1] = pack_bf16x2(v[2], v[3]);
  *reinterpret_cast<u32x2_t*>(dst) = packed;
  if (lo != nullptr) {
    u32x2_t rest;
    rest[0] = pack_bf16x2(v[0] - __uint_as_float(packed[0] << 16),
                          v[1] - __uint_as_float(packed[0] & 0xffff0000u));
    rest[1] = pack_bf16x2(v[2] - __uint_as_float(packed[1] << 16),
                          v[3] - __uint_as_float(packed[1] & 0xffff0000u));
    *reinterpret_cast<u32x2_t*>(lo) = rest;
  }
}

// h = silu(g) u for four outputs (features nn .. nn + 3) of grouped row p, in one or two
// bf16 parts.
__device__ __forceinline__ void store_gateup(const FfnArgs& a, int64_t p, int nn, f32x4_t g,
                                             f32x4_t u) {
  f32x4_t v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = swiglu_f32(g[i], u[i]);
  if (a.hsplit) {
    uint16_t* row = a.C + p * 2 * a.N;
    store_h4(row + nn, row + a.N + nn, v);
  } else {
    store_h4(a.C + p * a.N + nn, nullptr, v);
  }
}

// Four outputs (features nn .. nn + 3, nn a multiple of 4) of grouped row p as packed
// 24-bit floats: routed rows into Y, the shared expert's into Ys, 3 N bytes per row.
__device__ __forceinline__ void store_f24_row4(const FfnArgs& a, int64_t p, int nn, f32x4_t v) {
  const int64_t N = a.N;
  uint8_t* row = p < a.routed_rows ? reinterpret_cast<uint8_t*>(a.Y) + p * 3 * N
                                   : reinterpret_cast<uint8_t*>(a.Ys) + (p - a.routed_rows) * 3 * N;
  *reinterpret_cast<F24x4*>(row + 3 * nn) = pack_f24x4(v);
}

// Store four consecutive outputs (features nn .. nn+3) of grouped row p.  Every output
// row is a whole number of 4-feature groups: N is a multiple of 64 for every bf16 output
// (d, I and the latent width are), and the fp32 outputs are the down GEMM's (N = d) and
// the router's partial logits, whose parts are padded to a multiple of 4 (checked on the
// host by launch_dense).
template <int EPI>
__device__ __forceinline__ void store4(const FfnArgs& a, int64_t p, int nn, f32x4_t v,
                                       f32x4_t u, int col0 = 0) {
  const int N = a.N;
  if (EPI == kSwiGLU) {
    store_gateup(a, p, nn, v, u);
  } else if (EPI == kF32) {
    float* yrow = p < a.routed_rows ? a.Y + p * N
                                    : a.Ys + (p - a.routed_rows) * (a.ldc ? a.ldc : N) + col0;
    *reinterpret_cast<f32x4_t*>(yrow + nn) = v;
  } else if (EPI == kF24) {
    store_f24_row4(a, p, nn, v);
  } else {
    if (EPI == kAddBF16) v += *reinterpret_cast<const f32x4_t*>(a.R + p * N + nn);
    u32x2_t packed;
    packed[0] = pack_bf16x2(v[0], v[1]);
    packed[1] = pack_bf16x2(v[2], v[3]);
    *reinterpret_cast<u32x2_t*>(a.C + p * N + nn) = packed;
  }
}

// Epilogue of the LDS-tiled kernels (256-row tiles).  Accumulator register j of fragment
// (t, o), lane l, is tile row arow + tstride t + (l & 31) and output
// 32 o + 8 (j >> 2) + 4 (l >> 5) + (j & 3) of the wave's block (first output nbase), so a
// direct store writes 16 bytes into each of 32 rows, and the memory system handles such
// scattered pieces far slower than whole lines.  Instead each wave stages one 32-row
// fragment at a time in its own part of the (by then idle) activation buffers (32 rows of
// its outputs in fp32, the SwiGLU already applied: 16 KiB at most) and reads it back along
// the rows, so that one store instruction covers whole rows: with four fragments 2 x 512 B
// (fp32, 128 outputs) or 4 x 128 B (bf16 h, 64 outputs), with two 4 x 256 B or 8 x 64 B
// (24-bit rows: 4 x 192 B).
//
// Staging layout: row r (0..31) holds FW / 4 pieces of 4 outputs; piece p sits in slot
// r (FW / 4) + (p ^ (r & 7)), so the 8 lanes that the LDS serves together (8 rows, one
// piece, on the write side; one row, 8 pieces, on the read side) hit distinct banks.
template <int EPI>
__device__ __forceinline__ void store_row4(const FfnArgs& a, int64_t p, int nn, f32x4_t v,
                                           int col0) {
  const int N = a.N;
  if constexpr (EPI == kF32) {
    float* yrow = p < a.routed_rows ? a.Y + p * N
                                    : a.Ys + (p - a.routed_rows) * (a.ldc ? a.ldc : N) + col0;
    *reinterpret_cast<f32x4_t*>(yrow + nn) = v;
  } else if constexpr (EPI == kF24) {
    store_f24_row4(a, p, nn, v);
  } else {
    if constexpr (EPI == kAddBF16) v += *reinterpret_cast<const f32x4_t*>(a.R + p * N + nn);
    u32x2_t packed;
    packed[0] = pack_bf16x2(v[0], v[1]);
    packed[1] = pack_bf16x2(v[2], v[3]);
    *reinterpret_cast<u32x2_t*>(a.C + p * N + nn) = packed;
  }
}

// NO: output fragments the wave holds per row fragment (gate/up: the first NO / 2 of W1,
// the rest the same features of W3).  col0: first column of this workgroup's K slice in a
// row of Ys (fp32 output only).
template <int EPI, int NF, int NO = 4>
__device__ __forceinline__ void lds_epilogue(const FfnArgs& a, u32x4_t* stage,
                                             const f32x16_t (&acc)[NF][NO], int arow,
                                             int tstride, const Tile& tile, int nbase,
                                             int col0 = 0) {
  constexpr bool GATEUP = EPI == kSwiGLU;
  constexpr int FO = GATEUP ? NO / 2 : NO;  // 32-output fragments per row
  constexpr int PPR = 8 * FO;         // 16-byte pieces per staged row
  constexpr int RPI = 64 / PPR;       // rows per read-back instruction
  const int lane = threadIdx.x & 63, hl = lane >> 5;
  const int nrows = tile.row_end - tile.row_begin;
  const int rw = lane & 31;
  const int rr = lane / PPR, pr = lane % PPR;  // read side: row within the group, piece
#pragma unroll
  for (int t = 0; t < NF; ++t) {
#pragma unroll
    for (int oo = 0; oo < FO; ++oo)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x16_t& g = acc[t][oo];
        f32x4_t v = {g[4 * q], g[4 * q + 1], g[4 * q + 2], g[4 * q + 3]};
        if constexpr (GATEUP) {
          const f32x16_t& u = acc[t][oo + NO / 2];
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = swiglu_f32(v[i], u[4 * q + i]);
        }
        const int piece = 8 * oo + 2 * q + hl;
        stage[rw * PPR + (piece ^ (rw & 7))] = __builtin_bit_cast(u32x4_t, v);
      }
    // LDS operations of one wave complete in order: the reads below see these writes, and
    // the next fragment's writes come after these reads
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int r = RPI * i + rr;
      const f32x4_t v = __builtin_bit_cast(f32x4_t, stage[r * PPR + (pr ^ (r & 7))]);
      const int m = arow + tstride * t + r;
      const int nn = nbase + 4 * pr;
      if (m < nrows && nn < a.N) {
        if constexpr (GATEUP) {
          const int64_t p = tile.row_begin + m;
          if (a.hsplit) {
            uint16_t* row = a.C + p * 2 * a.N;
            store_h4(row + nn, row + a.N + nn, v);
          } else {
            store_h4(a.C + p * a.N + nn, nullptr, v);
          }
        } else {
          store_row4<EPI>(a, tile.row_begin + m, nn, v, col0);
        }
      }
    }
  }
}

constexpr int kSkinnyBM = 16;
constexpr int kWideBM = 256;
#ifndef MOE_SKINNY_NF
#define MOE_SKINNY_NF 2
#endif
#ifndef MOE_SKINNY_KU
#define MOE_SKINNY_KU 8
#endif
#ifndef MOE_SKINNY_GU_NF
#define MOE_SKINNY_GU_NF 1
#endif
#ifndef MOE_SKINNY_GU_KU
#define MOE_SKINNY_GU_KU 16
#endif
constexpr int kSkinnyNF = MOE_SKINNY_NF;  // skinny: 4 waves x NF fragments = 64 NF features per block
constexpr int kSkinnyKU = MOE_SKINNY_KU;  // skinny: k-steps (of 32) per batch of loads
// gate/up reads two matrices per fragment, so it keeps as many bytes in flight with half
// the fragments; its smaller blocks also shorten the launch's tail (K2 decode: 3.49 against
// 3.54 ms with the down GEMM's 2 x 8)
constexpr int kSkinnyGuNF = MOE_SKINNY_GU_NF;
constexpr int kSkinnyGuKU = MOE_SKINNY_GU_KU;
// bf16 256-row kernel: features of N per workgroup
constexpr int kWideBNGateUp = 128;  // gate/up: 128 features of W1 and the same of W3
constexpr int kWideBNDown = 256;

int64_t max_tiles_for(const FfnShape& sh, int BM) {
  // sum_e ceil(c_e / BM) <= (T*k) / BM + E, plus the shared expert's ceil(T / BM)
  return sh.T * sh.k / BM + sh.E + (sh.shared ? (sh.T + BM - 1) / BM : 0) + 1;
}

// A launch with a single group (a dense projection, or the latent variant's shared expert
// on its own) takes the tall-tile kernel above this many rows.  Below it, the skinny
// kernel's tiles each read the one weight matrix, mostly from L2.
constexpr int64_t kSingleGroupWideRows = 512;

// The 256-row kernels also need the gate/up GEMM's reduction (the model width d) to be at
// least this long.  Their fixed cost per tile (the first two chunks' loads, the staged
// epilogue) is spread over d / 64 chunks; at d = 256 (four chunks) the skinny kernels are
// faster at every batch measured.  Whole layer, 16 experts, top-2, I = 128, back to back,
// skinny against 256-row (two passes on one box, us): bf16 T = 64 26.2-26.7 / 31.5-32.0,
// T = 256 27.0-27.9 / 42.5-42.6, T = 1024 51.4-52.5 / 61.7-62.6; FP8 29.0-29.2 / 30.0-30.4,
// 29.3-29.6 / 33.9-34.7, 48.1 / 52.2-52.7.  From d = 512 on the 256-row kernels win at every
// shape measured, also with 48 workgroups per launch: bf16 d = 512, 8 experts, top-2,
// T = 2048 77.6-78.0 against 119.5-119.7 us skinny; d = 1024, 16 experts, top-4,
// T = 1024 91.5-92.7 against 221.6-222.3; d = 4096, 128 experts, top-8, T = 2048 913.6-926.7
// against 4838-4858; FP8 65.6-66.2 against 79.6-79.8, 79.3-79.4 against 140.6-140.9 and
// 824.3-826.2 against 2314.
constexpr int kWideMinK = 512;

// Average rows per group (routed experts plus the shared expert) decides the kernel: up to
// rows_per_group (decode) -> skinny kernel; more -> the 256-row kernel (bf16 or FP8), if d
// is at least kWideMinK.  Each weight type passes its own crossover, measured with the
// routed experts present; a launch of one group uses kSingleGroupWideRows instead.
bool use_wide(const FfnShape& sh, int rows_per_group) {
  const int64_t rows = sh.T * sh.k + (sh.shared ? sh.T : 0);
  const int64_t groups = sh.E + (sh.shared ? 1 : 0);
  if (groups <= 1) return rows > kSingleGroupWideRows;
  return sh.d >= kWideMinK && rows > (int64_t)rows_per_group * groups;
}

TileSpec tile_spec_for(const FfnShape& sh, int BM) {
  TileSpec t;
  t.E = sh.E;
  t.BM = BM;
  t.parts = BM > kSkinnyBM ? kMaxSharedParts : 1;
  t.routed_rows = sh.T * sh.k;
  t.shared_rows = sh.shared ? sh.T : 0;
  t.capacity = max_tiles_for(sh, BM);
  return t;
}

hipError_t tiles_launch(const FfnShape& sh, const int32_t* offsets, int BM, Tile* tiles,
                        int32_t* ntiles, hipStream_t s) {
  hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(1024), 0, s, offsets,
                     tile_spec_for(sh, BM), tiles, ntiles);
  return hipGetLastError();
}

dim3 grid_for(const FfnShape& sh, int BM, int BN, int N) {
  const int64_t NB = (N + BN - 1) / BN;
  const int64_t total = max_tiles_for(sh, BM) * NB;
  return dim3((unsigned)((total + 7) / 8 * 8));
}

}  // namespace
}  // namespace moe
