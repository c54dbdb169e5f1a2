// Grouped expert GEMMs on FP8 block-scaled weights: the checkpoint form of K2's expert
// weights ("nnterp encyclopedia · kimi_k2", loading a K2 checkpoint: FP8 blocks with
// per-block scales).  Codes are OCP E4M3; one fp32 scale covers a 128 x 128 block of an
// [out, in] matrix; the weight is code value x scale.
//
// Dequantisation is exact.  Every E4M3 value has at most four significant bits, so it
// converts to bf16 without rounding (v_cvt_scalef32_pk_bf16_fp8 with scale 1.0, two
// codes per instruction) and enters the bf16 MFMA as it is.  A weight fragment's 16 or 32
// output features lie in one 128-row block, so across one 128-wide k block all of its
// products share one scale: they are summed into a partial accumulator, and the scale is
// applied to that fp32 partial, acc += s * partial, at the end of the block.  The result
// is the exact dequantised product up to fp32 accumulation, like the bf16 path.
//
// Two kernels: the skinny one (up to 16 rows per tile, weights HBM -> registers) and the
// 256-row one (both operands through LDS).  The work list, work mapping, row gathering and
// epilogues are the bf16 kernels' ones.  In both, one 16-byte piece of a weight row holds
// 16 consecutive k, i.e. two MFMA steps' worth: the lane's first 8 codes feed one step, the
// next 8 the other, and the activation operand follows the same assignment (the MFMA only
// needs A and B to agree on which k each operand slot holds).
#include <type_traits>

#include "grouped.h"

namespace moe {
namespace {

// 16 E4M3 codes (k 0..15 of a lane) -> two operands of 8 bf16 each, exactly.
__device__ __forceinline__ void e4m3x16_to_bf16(u32x4_t q, u32x4_t& lo, u32x4_t& hi) {
#define MOE_CVT(w, sel) \
  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((w), 1.0f, sel))
  lo = u32x4_t{MOE_CVT(q[0], false), MOE_CVT(q[0], true), MOE_CVT(q[1], false),
               MOE_CVT(q[1], true)};
  hi = u32x4_t{MOE_CVT(q[2], false), MOE_CVT(q[2], true), MOE_CVT(q[3], false),
               MOE_CVT(q[3], true)};
#undef MOE_CVT
}

__device__ __forceinline__ u32x4_t load16b(const uint8_t* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

__device__ __forceinline__ void fma4(f32x4_t& acc, float s, f32x4_t part) {
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = fmaf(s, part[i], acc[i]);
}

// ------------------------------------------------------------- skinny FP8 GEMM
// The skinny kernel's shape (<= 16 rows per tile, 4 waves x NF 16-feature strips, weights
// HBM -> registers) on E4M3 weights: a batch is KB 128-k blocks, all of whose weight and
// activation loads are issued before the batch's first MFMA.
template <int NF, int KB, int EPI>
__global__ __launch_bounds__(256) void ffn_skinny_fp8_kernel(const FfnArgs a) {
  constexpr bool GATEUP = EPI == kSwiGLU;
  constexpr int BN = 4 * 16 * NF;
  Tile tile;
  int nb;
  if (!map_work(a, (a.N + BN - 1) / BN, tile, nb)) return;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, q = lane >> 4;
  const int K = a.K, N = a.N, KBLK = K / kFp8Block;

  int64_t p = tile.row_begin + r;
  const bool row_ok = p < tile.row_end;
  if (!row_ok) p = tile.row_end - 1;
  const uint16_t* arow = act_row(a, GATEUP, p) + q * 16;

  const bool is_shared = tile.group >= a.E;
  const int64_t wofs = (int64_t)tile.group * N * K;
  const int64_t sofs = (int64_t)tile.group * (N / kFp8Block) * KBLK;
  const uint8_t* W1 = is_shared ? a.QS1 : a.Q1 + wofs;
  const uint8_t* W3 = GATEUP ? (is_shared ? a.QS3 : a.Q3 + wofs) : nullptr;
  const float* S1 = is_shared ? a.S1s : a.B1s + sofs;
  const float* S3 = GATEUP ? (is_shared ? a.S3s : a.B3s + sofs) : nullptr;

  const int n0 = nb * BN + wave * 16 * NF;
  const uint8_t* w1p[NF];
  const uint8_t* w3p[NF];
  const float* s1p[NF];
  const float* s3p[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    int n = n0 + 16 * f + r;
    if (n > N - 1) n = N - 1;
    int nf = n0 + 16 * f;  // the fragment's first feature: its 16 rows share a block
    if (nf > N - 1) nf = N - 1;
    w1p[f] = W1 + (int64_t)n * K + q * 16;
    w3p[f] = GATEUP ? W3 + (int64_t)n * K + q * 16 : nullptr;
    s1p[f] = S1 + (int64_t)(nf / kFp8Block) * KBLK;
    s3p[f] = GATEUP ? S3 + (int64_t)(nf / kFp8Block) * KBLK : nullptr;
  }

  f32x4_t acc1[NF], acc3[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    acc1[f] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    acc3[f] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // one batch of NB blocks starting at block kb: loads, then MFMAs and scaling
  auto batch = [&](int kb, auto nb_tag) {
    constexpr int NB = decltype(nb_tag)::value;
    u32x4_t w1v[NF][NB][2], w3v[NF][NB][2], av[NB][2][2];
    float s1v[NF][NB], s3v[NF][NB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        const int koff = (kb + b) * kFp8Block + pp * 64;
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          w1v[f][b][pp] = load16b(w1p[f] + koff);
          if (GATEUP) w3v[f][b][pp] = load16b(w3p[f] + koff);
        }
      }
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        const int koff = (kb + b) * kFp8Block + pp * 64;
        av[b][pp][0] = load16(arow + koff);
        av[b][pp][1] = load16(arow + koff + 8);
      }
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        s1v[f][b] = s1p[f][kb + b];
        if (GATEUP) s3v[f][b] = s3p[f][kb + b];
      }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        f32x4_t p1 = f32x4_t{0.f, 0.f, 0.f, 0.f}, p3 = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          u32x4_t lo, hi;
          e4m3x16_to_bf16(w1v[f][b][pp], lo, hi);
          p1 = mfma16x16x32(lo, av[b][pp][0], p1);
          p1 = mfma16x16x32(hi, av[b][pp][1], p1);
          if (GATEUP) {
            e4m3x16_to_bf16(w3v[f][b][pp], lo, hi);
            p3 = mfma16x16x32(lo, av[b][pp][0], p3);
            p3 = mfma16x16x32(hi, av[b][pp][1], p3);
          }
        }
        fma4(acc1[f], s1v[f][b], p1);
        if (GATEUP) fma4(acc3[f], s3v[f][b], p3);
      }
    }
  };
  int kb = 0;
  for (; kb + KB <= KBLK; kb += KB) batch(kb, std::integral_constant<int, KB>{});
  for (; kb < KBLK; ++kb) batch(kb, std::integral_constant<int, 1>{});

  if (!row_ok) return;
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int nn = n0 + 16 * f + 4 * q;
    if (nn < N) store4<EPI>(a, p, nn, acc1[f], acc3[f]);
  }
}

// ------------------------------------------------------------- 256-row FP8 GEMM
// The bf16 256-row kernel's plan on E4M3 codes: tiles of up to 256 rows, so that one pass
// over an expert's weights serves up to 256 of its rows, with both operands moved into LDS
// by direct transfer.  A workgroup computes 256 rows x 128 weight rows (gate/up: 64
// features of W1 and the same 64 of W3; down: 128 features) with eight waves, two per
// SIMD.  Wave (wm, wn) holds row fragments wm and wm + 4 (tile rows 32 wm and 32 wm + 128,
// so that a partly filled tile keeps the waves equally busy) x 2 weight fragments of
// 32 x 32, each with a partial accumulator beside the running one, all in VGPRs.  A
// partial collects one 128-k block (two chunks of 64 k); at the block's end
// acc += s * partial with the block's scale, one VALU op per output, which the SIMD's other
// wave covers with its MFMAs.
//
// Three buffers of each operand: during chunk c the transfers of chunk c + 2 are issued,
// and the barrier before chunk c + 1 waits for all but those.  Activation buffers (256 rows
// x 128 B) use the bf16 kernel's layout.  Weight buffers (128 rows x 64 B of codes, 512
// slots of 16 B): piece p (codes of k 16 p .. 16 p + 15) of row m sits in slot
// 4 m + (p ^ s(m)), with s(m) = ((m >> 1) ^ (m >> 3)) & 1 | (((m >> 2) ^ (m >> 3)) & 1) << 1,
// so that a fragment read (16 rows, one piece) meets distinct 16-byte bank groups.  K
// mapping: in k-pair j (32 k) of a chunk, lane (r, h) reads piece 2 j + h of its weight row;
// the piece's first 8 codes feed MFMA step 2 j, the other 8 step 2 j + 1, and the activation
// operand of step s takes piece 4 (s >> 1) + 2 h + (s & 1), which holds the same k.
constexpr int kF8LdsBM = 256;
constexpr int kF8LdsFeatGateUp = 64;  // features of W1 (and of W3) per workgroup
constexpr int kF8LdsFeatDown = 128;
constexpr int kF8LdsWaves = 8;

struct F8LdsCtx {
  __amdgpu_buffer_rsrc_t act;  // activation rows (x, or the tile's rows of h)
  __amdgpu_buffer_rsrc_t wgt;  // codes of the matrix this wave transfers (gate/up: W1 for
                               // waves 0-3, W3 for waves 4-7)
  uint32_t aoff[4];            // per-lane byte offsets of the wave's 4 activation units
  uint32_t woff;               // per-lane byte offset of the wave's weight unit
  uint32_t aoob, woob;         // wave-uniform offsets past the end of act / wgt
  int wrd[2];                  // slot of the lane's weight piece in k-pair j (fragment 0)
  int ard[4];                  // slot of the lane's activation piece in step s (fragment 0)
  int nc;                      // chunks (even: K is a whole number of 128-k blocks)
};

__device__ __forceinline__ int f8_wswz(int m) {
  return (((m >> 1) ^ (m >> 3)) & 1) | ((((m >> 2) ^ (m >> 3)) & 1) << 1);
}

// Codes 8 i .. 8 i + 7 of a 16-code piece as one bf16 operand, exactly.
__device__ __forceinline__ u32x4_t e4m3x8_to_bf16(u32x4_t q, int i) {
#define MOE_CVT(w, sel) \
  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((w), 1.0f, sel))
  const uint32_t a = i ? q[2] : q[0], b = i ? q[3] : q[1];
  return u32x4_t{MOE_CVT(a, false), MOE_CVT(a, true), MOE_CVT(b, false), MOE_CVT(b, true)};
#undef MOE_CVT
}

// At the top of a chunk: this wave's transfers of the chunk are complete (only the next
// chunk's 5 may still be in flight) and every wave has finished the previous chunk.
__device__ __forceinline__ void f8_sync5() {
  asm volatile("s_waitcnt vmcnt(5) lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Part s (0..2) of this wave's 5 transfers of chunk c: activation units 2 s, 2 s + 1, or
// (s = 2) the weight unit.  Past the last chunk the offsets point past the buffers (zeros,
// no data moved), so every chunk issues the same count.
__device__ __forceinline__ void f8_fetch(const F8LdsCtx& x, u32x4_t* abuf, u32x4_t* wbuf,
                                         int wave, int c, int s) {
  if (s < 2) {
    const uint32_t so = c < x.nc ? (uint32_t)c * 128u : x.aoob;
#pragma unroll
    for (int j = 2 * s; j < 2 * s + 2; ++j)
      dma16(x.act, abuf + (wave * 4 + j) * 64, x.aoff[j], so);
  } else {
    const uint32_t so = c < x.nc ? (uint32_t)c * 64u : x.woob;
    dma16(x.wgt, wbuf + wave * 64, x.woff, so);
  }
}

// One chunk: FIRST starts the block's partials, LAST closes the block (scales sc0, sc1 of
// weight fragments 0 and 1).  WF1: slot distance from weight fragment 0 to fragment 1.
template <int NF, int WF1, bool FIRST, bool LAST>
__device__ __forceinline__ void f8_chunk(const F8LdsCtx& x, const u32x4_t* acur,
                                         const u32x4_t* wcur, u32x4_t* anext2,
                                         u32x4_t* wnext2, int wave, int c, const float* sc0,
                                         const float* sc1, f32x16_t (&acc)[NF > 0 ? NF : 1][2],
                                         f32x16_t (&part)[NF > 0 ? NF : 1][2]) {
  constexpr int NA = NF > 0 ? NF : 1;
  f8_sync5();
  u32x4_t wq[2][2], av[2][NA];
  if constexpr (NF > 0) {
#pragma unroll
    for (int o = 0; o < 2; ++o) wq[0][o] = wcur[x.wrd[0] + WF1 * o];
#pragma unroll
    for (int t = 0; t < NF; ++t) av[0][t] = acur[x.ard[0] + 1024 * t];
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if (s < 3) f8_fetch(x, anext2, wnext2, wave, c + 2, s);
    if constexpr (NF > 0) {
      if (s == 0) {
#pragma unroll
        for (int o = 0; o < 2; ++o) wq[1][o] = wcur[x.wrd[1] + WF1 * o];
      }
      if (s < 3) {
#pragma unroll
        for (int t = 0; t < NF; ++t) av[(s + 1) & 1][t] = acur[x.ard[s + 1] + 1024 * t];
      }
      u32x4_t wb[2];
#pragma unroll
      for (int o = 0; o < 2; ++o) wb[o] = e4m3x8_to_bf16(wq[s >> 1][o], s & 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < NF; ++t)
#pragma unroll
        for (int o = 0; o < 2; ++o)
          part[t][o] = mfma32x32x16(wb[o], av[s & 1][t],
                                    (FIRST && s == 0) ? f32x16_t{} : part[t][o]);
    }
  }
  if constexpr (LAST && NF > 0) {
    const int kb = c >> 1;
    const float s0 = sc0[kb], s1 = sc1[kb];
#pragma unroll
    for (int t = 0; t < NF; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        acc[t][0][e] = fmaf(s0, part[t][0][e], acc[t][0][e]);
        acc[t][1][e] = fmaf(s1, part[t][1][e], acc[t][1][e]);
      }
  }
}

struct F8LdsBufs {
  u32x4_t* A0;
  u32x4_t* A1;
  u32x4_t* A2;
  u32x4_t* W0;
  u32x4_t* W1;
  u32x4_t* W2;
};

template <int EPI, int NF>
__device__ __forceinline__ void f8_lds_tile(const FfnArgs& a, const F8LdsCtx& x,
                                            const F8LdsBufs& b, int wave, int arow,
                                            const Tile& tile, int nbase, const float* sc0,
                                            const float* sc1) {
  constexpr bool GATEUP = EPI == kSwiGLU;
  constexpr int NA = NF > 0 ? NF : 1;
  constexpr int WF1 = GATEUP ? 4 * 64 : 4 * 32;  // gate/up: W3 rows 64 further; down: 32
  f32x16_t acc[NA][2], part[NA][2];
#pragma unroll
  for (int t = 0; t < NA; ++t)
#pragma unroll
    for (int o = 0; o < 2; ++o) {
      acc[t][o] = f32x16_t{};
      part[t][o] = f32x16_t{};
    }
  const int nc = x.nc;
#pragma unroll
  for (int s = 0; s < 3; ++s) f8_fetch(x, b.A0, b.W0, wave, 0, s);
#pragma unroll
  for (int s = 0; s < 3; ++s) f8_fetch(x, b.A1, b.W1, wave, 1, s);
  // chunk mod 3 picks the buffers, chunk mod 2 the place in the block: period 6
  int c = 0;
  for (; c + 6 <= nc; c += 6) {
    f8_chunk<NF, WF1, true, false>(x, b.A0, b.W0, b.A2, b.W2, wave, c, sc0, sc1, acc, part);
    f8_chunk<NF, WF1, false, true>(x, b.A1, b.W1, b.A0, b.W0, wave, c + 1, sc0, sc1, acc, part);
    f8_chunk<NF, WF1, true, false>(x, b.A2, b.W2, b.A1, b.W1, wave, c + 2, sc0, sc1, acc, part);
    f8_chunk<NF, WF1, false, true>(x, b.A0, b.W0, b.A2, b.W2, wave, c + 3, sc0, sc1, acc, part);
    f8_chunk<NF, WF1, true, false>(x, b.A1, b.W1, b.A0, b.W0, wave, c + 4, sc0, sc1, acc, part);
    f8_chunk<NF, WF1, false, true>(x, b.A2, b.W2, b.A1, b.W1, wave, c + 5, sc0, sc1, acc, part);
  }
  // 0, 2 or 4 chunks left
  if (c < nc) {
    f8_chunk<NF, WF1, true, false>(x, b.A0, b.W0, b.A2, b.W2, wave, c, sc0, sc1, acc, part);
    f8_chunk<NF, WF1, false, true>(x, b.A1, b.W1, b.A0, b.W0, wave, c + 1, sc0, sc1, acc, part);
  }
  if (c + 2 < nc) {
    f8_chunk<NF, WF1, true, false>(x, b.A2, b.W2, b.A1, b.W1, wave, c + 2, sc0, sc1, acc, part);
    f8_chunk<NF, WF1, false, true>(x, b.A0, b.W0, b.A2, b.W2, wave, c + 3, sc0, sc1, acc, part);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  lds_barrier();
  // staging: 8 KiB per wave, waves 0-3 in buffer A0, 4-7 in A1
  if constexpr (NF > 0)
    lds_epilogue<EPI, NF, 2>(a, (wave < 4 ? b.A0 : b.A1) + (wave & 3) * 512, acc, arow, 128,
                             tile, nbase);
}

template <int EPI>
__global__ __launch_bounds__(64 * kF8LdsWaves, 1) void ffn_lds_fp8_kernel(const FfnArgs a) {
  constexpr bool GATEUP = EPI == kSwiGLU;
  constexpr int BM = kF8LdsBM;
  constexpr int FEAT = GATEUP ? kF8LdsFeatGateUp : kF8LdsFeatDown;
  constexpr int MAXKB = kFp8MaxK / kFp8Block;
  constexpr int NT = 64 * kF8LdsWaves;
  __shared__ __attribute__((aligned(1024))) u32x4_t A0[BM * 8];
  __shared__ __attribute__((aligned(1024))) u32x4_t A1[BM * 8];
  __shared__ __attribute__((aligned(1024))) u32x4_t A2[BM * 8];
  __shared__ __attribute__((aligned(1024))) u32x4_t W0[512];
  __shared__ __attribute__((aligned(1024))) u32x4_t W1[512];
  __shared__ __attribute__((aligned(1024))) u32x4_t W2[512];
  __shared__ float sc[2 * MAXKB];

  Tile tile;
  int nb;
  if (!map_work(a, (a.N + FEAT - 1) / FEAT, tile, nb)) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int K = a.K, N = a.N, KBLK = K / kFp8Block;
  const int nrows = tile.row_end - tile.row_begin;
  const int f0 = nb * FEAT;

  const bool is_shared = tile.group >= a.E;
  const int64_t wofs = (int64_t)tile.group * N * K;
  const int64_t sofs = (int64_t)tile.group * (N / kFp8Block) * KBLK;
  const uint8_t* Q1 = is_shared ? a.QS1 : a.Q1 + wofs;
  const uint8_t* Q3 = GATEUP ? (is_shared ? a.QS3 : a.Q3 + wofs) : Q1;
  const float* S1 = is_shared ? a.S1s : a.B1s + sofs;
  const float* S3 = GATEUP ? (is_shared ? a.S3s : a.B3s + sofs) : S1;

  // the workgroup's features lie in one 128-feature block row: its scales (gate/up: rows of
  // W1 and W3; down: one row, twice) go to LDS and are read after the first barrier
  {
    const int brow = min(f0, N - 1) / kFp8Block;
    for (int i = tid; i < 2 * KBLK; i += NT) {
      const int row = i / KBLK, kb = i - row * KBLK;
      sc[row * MAXKB + kb] = (row == 0 ? S1 : S3)[(int64_t)brow * KBLK + kb];
    }
  }

  F8LdsCtx x;
  const uint32_t wbytes = (uint32_t)N * (uint32_t)K;  // < 2^32 (checked on the host)
  x.wgt = buffer_rsrc(GATEUP && wave >= 4 ? Q3 : Q1, wbytes);
  const uint16_t* abase = GATEUP ? a.A : a.A + (int64_t)tile.row_begin * K;
  const uint32_t abytes = GATEUP ? (uint32_t)(a.a_rows * K * 2) : (uint32_t)nrows * K * 2u;
  x.act = buffer_rsrc(abase, abytes);
  // activation transfer lane l of unit u = 4 wave + j: row 8 u + (l >> 3), the bf16
  // kernel's layout; rows past the tile's end read past the buffer (zeros; not stored)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int u = wave * 4 + j, m = 8 * u + (lane >> 3);
    const int piece = (lane & 7) ^ (m & 7) ^ (u & 1);
    const int64_t p = tile.row_begin + m;
    x.aoff[j] = p < tile.row_end ? (uint32_t)(act_row(a, GATEUP, p) - abase) * 2u + piece * 16
                                 : abytes;
  }
  // weight transfer lane l of unit u = wave: LDS row m = 16 u + (l >> 2), slot l & 3 holding
  // piece (l & 3) ^ s(m).  Gate/up rows 0..63 are W1 features f0 + m, rows 64..127 the same
  // features of W3; down rows are features f0 + m.  Features past N read past the matrix
  // (zeros; outputs not stored).
  {
    const int m = 16 * wave + (lane >> 2);
    const int f = f0 + (GATEUP ? (m & 63) : m);
    const int piece = (lane & 3) ^ f8_wswz(m);
    x.woff = f < N ? (uint32_t)f * (uint32_t)K + piece * 16 : wbytes;
  }
  x.aoob = abytes;
  x.woob = wbytes;
  const int arow = 32 * wm;
  {
    const int r = lane & 31, h = lane >> 5;
    // weight fragment 0 of this wave: gate/up W1 rows 32 wn (fragment 1: the W3 rows 64
    // further); down rows 64 wn (fragment 1: 32 further)
    const int wrow0 = GATEUP ? 32 * wn : 64 * wn;
#pragma unroll
    for (int j = 0; j < 2; ++j) x.wrd[j] = 4 * (wrow0 + r) + ((2 * j + h) ^ f8_wswz(r));
    const int sig = (r & 7) ^ ((r >> 3) & 1);
#pragma unroll
    for (int s = 0; s < 4; ++s)
      x.ard[s] = 8 * (arow + r) + ((4 * (s >> 1) + 2 * h + (s & 1)) ^ sig);
  }
  x.nc = K / 64;
  const int nbase = f0 + (GATEUP ? 32 : 64) * wn;
  const float* sc0 = sc;
  const float* sc1 = GATEUP ? sc + MAXKB : sc;

  // live row fragments of this wave: tile rows 32 wm .. and 32 wm + 128 ..
  const int nf = (nrows > arow ? 1 : 0) + (nrows > arow + 128 ? 1 : 0);
  const F8LdsBufs bufs{A0, A1, A2, W0, W1, W2};
  switch (nf) {
    case 0: f8_lds_tile<EPI, 0>(a, x, bufs, wave, arow, tile, nbase, sc0, sc1); break;
    case 1: f8_lds_tile<EPI, 1>(a, x, bufs, wave, arow, tile, nbase, sc0, sc1); break;
    default: f8_lds_tile<EPI, 2>(a, x, bufs, wave, arow, tile, nbase, sc0, sc1); break;
  }
}

// Skinny FP8 shapes (NF 16-feature fragments per wave, KB 128-k blocks per load batch).
// A sweep at K2 decode on one box (gate/up, ms): 2x2 1.88, 1x4 1.94, 2x3 1.87, 2x4 2.09,
// 4x2 1.95, 4x1 1.83, 8x1 2.00 (2x4, 4x2 and 8x1 spill).  Down with gate/up 4x1, the layer:
// 2x2 2.83, 4x1 2.78, 4x2 2.79, 8x1 2.79, 2x4 2.84, 1x4 3.05.
#ifndef MOE_F8_GU_NF
#define MOE_F8_GU_NF 4
#endif
#ifndef MOE_F8_GU_KB
#define MOE_F8_GU_KB 1
#endif
constexpr int kSkinnyF8GuNF = MOE_F8_GU_NF;
constexpr int kSkinnyF8GuKB = MOE_F8_GU_KB;
#ifndef MOE_F8_DN_NF
#define MOE_F8_DN_NF 4
#endif
#ifndef MOE_F8_DN_KB
#define MOE_F8_DN_KB 1
#endif
constexpr int kSkinnyF8DnNF = MOE_F8_DN_NF;
constexpr int kSkinnyF8DnKB = MOE_F8_DN_KB;

FfnArgs fp8_args(const FfnShape& sh, const Fp8Weights& w, bool gateup, Tile* tiles,
                 int32_t* ntiles) {
  FfnArgs a{};
  a.Q1 = gateup ? w.w1 : w.w2;
  a.Q3 = gateup ? w.w3 : nullptr;
  a.QS1 = gateup ? w.ws1 : w.ws2;
  a.QS3 = gateup ? w.ws3 : nullptr;
  a.B1s = gateup ? w.w1_scale : w.w2_scale;
  a.B3s = gateup ? w.w3_scale : nullptr;
  a.S1s = gateup ? w.ws1_scale : w.ws2_scale;
  a.S3s = gateup ? w.ws3_scale : nullptr;
  a.tiles = tiles;
  a.ntiles = ntiles;
  a.k = sh.k;
  a.E = sh.E;
  a.routed_rows = sh.T * sh.k;
  return a;
}

}  // namespace

// FP8 weights: the 256-row kernel above 16 rows per group (and from d = 512 on, as with
// bf16 weights).  It converts every weight it reads and applies a scale per 128-k block, so
// the skinny kernel stays ahead longer than with bf16 weights: K2-shape layer, ms, skinny /
// 256-row: T 128 2.78 / 4.06, 256 3.05 / 4.32, 448 3.32 / 4.44, 640 3.71 / 4.53, 1024 5.20 /
// 4.59, 2048 8.65 / 4.95 (at T = 640 there are 15 rows per group, at 1024 24).
#ifndef MOE_F8_WIDE_ROWS
#define MOE_F8_WIDE_ROWS 16
#endif
constexpr int kWideRowsFp8 = MOE_F8_WIDE_ROWS;

TileSpec ffn_tile_spec_fp8(const FfnShape& sh) {
  return tile_spec_for(sh, use_wide(sh, kWideRowsFp8) ? kF8LdsBM : kSkinnyBM);
}

hipError_t launch_gate_up_fp8(const FfnShape& sh, const uint16_t* x, const int32_t* perm,
                              const int32_t* offsets, const Fp8Weights& w, uint16_t* h,
                              Tile* tiles, int32_t* ntiles, hipStream_t s, bool tiles_ready) {
  const bool wide = use_wide(sh, kWideRowsFp8);
  const int BM = wide ? kF8LdsBM : kSkinnyBM;
  if (!tiles_ready) {
    hipError_t err = tiles_launch(sh, offsets, BM, tiles, ntiles, s);
    if (err != hipSuccess) return err;
  }
  FfnArgs a = fp8_args(sh, w, true, tiles, ntiles);
  a.A = x;
  a.a_rows = sh.T;
  a.perm = perm;
  a.C = h;
  a.N = sh.I;
  a.K = sh.d;
  if (wide)
    hipLaunchKernelGGL(ffn_lds_fp8_kernel<kSwiGLU>, grid_for(sh, BM, kF8LdsFeatGateUp, a.N),
                       dim3(64 * kF8LdsWaves), 0, s, a);
  else
    hipLaunchKernelGGL((ffn_skinny_fp8_kernel<kSkinnyF8GuNF, kSkinnyF8GuKB, kSwiGLU>),
                       grid_for(sh, BM, 64 * kSkinnyF8GuNF, a.N), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_down_fp8(const FfnShape& sh, const uint16_t* h, const int32_t* offsets,
                           const Fp8Weights& w, void* y_routed, void* y_shared, Tile* tiles,
                           int32_t* ntiles, hipStream_t s, bool tiles_ready, bool y24) {
  const bool wide = use_wide(sh, kWideRowsFp8);
  const int BM = wide ? kF8LdsBM : kSkinnyBM;
  if (!tiles_ready) {
    hipError_t err = tiles_launch(sh, offsets, BM, tiles, ntiles, s);
    if (err != hipSuccess) return err;
  }
  FfnArgs a = fp8_args(sh, w, false, tiles, ntiles);
  a.A = h;
  a.a_rows = sh.T * sh.k + (sh.shared ? sh.T : 0);
  a.Y = static_cast<float*>(y_routed);
  a.Ys = static_cast<float*>(y_shared);
  a.N = sh.d;
  a.K = sh.I;
  const dim3 gw = grid_for(sh, BM, kF8LdsFeatDown, a.N),
             gs = grid_for(sh, BM, 64 * kSkinnyF8DnNF, a.N);
  if (wide) {
    if (y24)
      hipLaunchKernelGGL(ffn_lds_fp8_kernel<kF24>, gw, dim3(64 * kF8LdsWaves), 0, s, a);
    else
      hipLaunchKernelGGL(ffn_lds_fp8_kernel<kF32>, gw, dim3(64 * kF8LdsWaves), 0, s, a);
  } else {
    if (y24)
      hipLaunchKernelGGL((ffn_skinny_fp8_kernel<kSkinnyF8DnNF, kSkinnyF8DnKB, kF24>), gs,
                         dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((ffn_skinny_fp8_kernel<kSkinnyF8DnNF, kSkinnyF8DnKB, kF32>), gs,
                         dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace moe
