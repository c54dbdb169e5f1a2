// Grouped expert GEMMs on FP8 block-scaled weights: the checkpoint form of K2's expert
// weights ("nnterp encyclopedia · kimi_k2", loading a K2 checkpoint: FP8 blocks with
// per-block scales).  Codes are OCP E4M3; one fp32 scale covers a 128 x 128 block of an
// [out, in] matrix; the weight is code value x scale.
//
// Dequantisation is exact.  Every E4M3 value has at most four significant bits, so it
// converts to bf16 without rounding (v_cvt_scalef32_pk_bf16_fp8 with scale 1.0, two
// codes per instruction) and enters the bf16 MFMA as it is.  A weight fragment's 16
// output features lie in one 128-row block, so across one 128-wide k block all of its
// products share one scale: they are summed into a partial accumulator, and the scale is
// applied to that fp32 partial, acc += s * partial, at the end of the block.  The result
// is the exact dequantised product up to fp32 accumulation, like the bf16 path.
//
// The work list, work mapping, row gathering and epilogues are the bf16 kernels' ones.
// K-mapping of the MFMA operands: one 16-byte load of a weight row holds 16 consecutive
// k, i.e. two 32-k MFMA steps' worth.  Lane group q of a 64-k pair takes k 16q .. 16q+15
// of the pair: the first 8 feed the pair's first MFMA, the next 8 its second; the
// activation operand follows the same assignment (the MFMA only needs A and B to agree).
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

// ------------------------------------------------------------- stream FP8 GEMM
// 128-row tiles: eight waves, each holding all of the tile's rows (8 row fragments) x 32
// outputs (gate/up: 16 features of W1 and the same 16 of W3; down: 32 features), with a
// partial accumulator next to the running one (the scale is applied per 128-k block).
// The tile's activations are staged in LDS in 64-wide k-chunks, double-buffered, k-chunk-
// major with the row XOR-swizzled by the chunk (slot = c * 128 + (m ^ 2c)); one 64-k
// chunk is one FP8 pair, so lane group q reads chunk pieces 2q and 2q + 1.  Weights
// stream HBM -> registers through a ring of F8_RING pairs (16 bytes per lane per
// fragment each).  The block's scales (two rows of K/128) are copied to LDS first.
constexpr int kF8BM = 128;
constexpr int kF8Ring = 4;  // 64-k pairs of weights held in registers per wave (even)

struct F8Ctx {
  __amdgpu_buffer_rsrc_t w1, w3, act;
  uint32_t woff[2];  // byte offset of the lane's weight row + 16 q, per fragment
  uint32_t aoff[2];  // byte offset of the thread's two activation pieces
  int adst;          // LDS element offset of piece 0 (piece 1 sits 64 slots further)
  int npair;         // K / 64
  int sidx[2];       // LDS scale row of fragment 0 and 1
};

template <int EPI, int NL>
__device__ __forceinline__ void f8_loop(const F8Ctx& c_, uint16_t* lds, const float* sc,
                                        f32x4_t (&acc)[8][2]) {
  constexpr bool GATEUP = EPI == kSwiGLU;
  constexpr int BM = kF8BM, BK = 64, NW = 2, D = kF8Ring;
  static_assert(D % 2 == 0 && D >= 2, "ring depth");
  const int lane = threadIdx.x & 63, r = lane & 15, q = lane >> 4;
  const int np = c_.npair;
  u32x4_t W[D][NW], AR[2];
  f32x4_t part[NL][NW];
#pragma unroll
  for (int i = 0; i < NL; ++i)
#pragma unroll
    for (int f = 0; f < NW; ++f) part[i][f] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto load_w = [&](u32x4_t* S, int pr) {
    const uint32_t kb = (uint32_t)(pr < np ? pr : np - 1) * 64;  // past the end: re-read
    S[0] = bload16(c_.w1, c_.woff[0], kb);
    S[1] = bload16(GATEUP ? c_.w3 : c_.w1, c_.woff[1], kb);
  };
  auto load_a = [&](int c) {
    const uint32_t cb = (uint32_t)(c < np ? c : np - 1) * (BK * 2);
    AR[0] = bload16(c_.act, c_.aoff[0], cb);
    AR[1] = bload16(c_.act, c_.aoff[1], cb);
  };
  auto store_a = [&](int buf) {
    *reinterpret_cast<u32x4_t*>(lds + buf * BM * BK + c_.adst) = AR[0];
    *reinterpret_cast<u32x4_t*>(lds + buf * BM * BK + c_.adst + 64 * 8) = AR[1];
  };
  // the pair of chunk c: MFMAs over pieces 2q (low 8 k of the lane) and 2q + 1 (high 8)
  auto mma_pair = [&](int buf, const u32x4_t* S) {
    u32x4_t lo[NW], hi[NW];
#pragma unroll
    for (int f = 0; f < NW; ++f) e4m3x16_to_bf16(S[f], lo[f], hi[f]);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = 2 * q + h;
      const uint16_t* As = lds + buf * BM * BK + (c * BM + (r ^ (2 * c))) * 8;
      u32x4_t G0 = *reinterpret_cast<const u32x4_t*>(As), G1;
#pragma unroll
      for (int g = 0; g < NL; ++g) {
        const u32x4_t cur = (g & 1) ? G1 : G0;
        if (g + 1 < NL) {
          if (g & 1)
            G0 = *reinterpret_cast<const u32x4_t*>(As + 16 * (g + 1) * 8);
          else
            G1 = *reinterpret_cast<const u32x4_t*>(As + 16 * (g + 1) * 8);
        }
        part[g][0] = mfma16x16x32(h ? hi[0] : lo[0], cur, part[g][0]);
        part[g][1] = mfma16x16x32(h ? hi[1] : lo[1], cur, part[g][1]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  // end of a 128-k block: apply its scales to the partials
  auto close_block = [&](int blk) {
    const float s0 = sc[c_.sidx[0] + blk], s1 = sc[c_.sidx[1] + blk];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      fma4(acc[i][0], s0, part[i][0]);
      fma4(acc[i][1], s1, part[i][1]);
      part[i][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      part[i][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  };
  auto next_chunk = [&](int c) {
    store_a((c + 1) & 1);
    load_a(c + 2);
    lds_barrier();
  };
  // chunk cc = c + j of a ring period; ring slot j holds its pair
  auto chunk = [&](int c, int j) {
    const int cc = c + j;
    load_w(W[(j + D - 1) % D], cc + D - 1);
    mma_pair(cc & 1, W[j]);
    if (j & 1) close_block(cc >> 1);
    next_chunk(cc);
  };

  load_a(0);
#pragma unroll
  for (int t = 0; t < D - 1; ++t) load_w(W[t], t);
  store_a(0);
  load_a(1);
  lds_barrier();
  int c = 0;
  // at the top of an iteration W[t] holds pair c + t for t < D - 1; c is even
  for (; c + D <= np; c += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) chunk(c, j);
  }
#pragma unroll
  for (int j = 0; j < D - 1; ++j)
    if (c + j < np) chunk(c, j);
}

template <int EPI>
__global__ __launch_bounds__(512, 1) void ffn_stream_fp8_kernel(const FfnArgs a) {
  constexpr bool GATEUP = EPI == kSwiGLU;
  constexpr int BM = kF8BM, BK = 64, NW = 2, NT = 512;
  constexpr int FEAT_WAVE = GATEUP ? 16 : 32;
  constexpr int FEAT = 8 * FEAT_WAVE;
  constexpr int MAXKB = kFp8MaxK / kFp8Block;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * BM * BK];
  __shared__ float sc[2 * MAXKB];

  Tile tile;
  int nb;
  if (!map_work(a, (a.N + FEAT - 1) / FEAT, tile, nb)) return;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, q = lane >> 4;
  const int K = a.K, N = a.N, KBLK = K / kFp8Block;
  const int nrows = tile.row_end - tile.row_begin;
  const int n_wave = nb * FEAT + wave * FEAT_WAVE;

  const bool is_shared = tile.group >= a.E;
  const int64_t wofs = (int64_t)tile.group * N * K;
  const int64_t sofs = (int64_t)tile.group * (N / kFp8Block) * KBLK;
  const uint8_t* W1 = is_shared ? a.QS1 : a.Q1 + wofs;
  const uint8_t* W3 = GATEUP ? (is_shared ? a.QS3 : a.Q3 + wofs) : nullptr;
  const float* S1 = is_shared ? a.S1s : a.B1s + sofs;
  const float* S3 = GATEUP ? (is_shared ? a.S3s : a.B3s + sofs) : nullptr;

  // the block's scale rows: gate/up: W1's and W3's block row of the block's 128 features;
  // down: the two 128-feature block rows of its 256 features (the second clamped to N)
  {
    const int nb0 = (nb * FEAT) / kFp8Block;
    int nb1 = GATEUP ? nb0 : nb0 + 1;
    if (nb1 > N / kFp8Block - 1) nb1 = N / kFp8Block - 1;
    for (int i = tid; i < 2 * KBLK; i += NT) {
      const int row = i / KBLK, kb = i - row * KBLK;
      sc[row * MAXKB + kb] = GATEUP ? (row == 0 ? S1 : S3)[(int64_t)nb0 * KBLK + kb]
                                    : S1[(int64_t)(row == 0 ? nb0 : nb1) * KBLK + kb];
    }
  }

  F8Ctx ctx;
  const uint32_t wbytes = (uint32_t)N * (uint32_t)K;  // < 2^32 (checked on the host)
  ctx.w1 = buffer_rsrc(W1, wbytes);
  ctx.w3 = buffer_rsrc(GATEUP ? W3 : W1, wbytes);
  const uint16_t* abase = GATEUP ? a.A : a.A + (int64_t)tile.row_begin * K;
  const uint32_t abytes = GATEUP ? (uint32_t)(a.a_rows * K * 2) : (uint32_t)nrows * K * 2u;
  ctx.act = buffer_rsrc(abase, abytes);
#pragma unroll
  for (int f = 0; f < NW; ++f) {
    int n = n_wave + (GATEUP ? 0 : 16 * f) + r;
    if (n > N - 1) n = N - 1;
    ctx.woff[f] = (uint32_t)n * (uint32_t)K + q * 16;
  }
  // fragment scale rows: gate/up f = 0 -> W1 row, f = 1 -> W3 row; down: both fragments
  // of a wave lie in the block row of its 32 features (rows 0 for waves 0..3, 1 for 4..7)
  if (GATEUP) {
    ctx.sidx[0] = 0;
    ctx.sidx[1] = MAXKB;
  } else {
    ctx.sidx[0] = ctx.sidx[1] = (wave >= 4 ? MAXKB : 0);
  }
  // activation pieces of this thread: row (tid >> 3) + 64 i, 16-byte chunk tid & 7
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int m = (tid >> 3) + 64 * i;
    int64_t p = tile.row_begin + m;
    if (p >= tile.row_end) p = tile.row_end - 1;
    ctx.aoff[i] = (uint32_t)(act_row(a, GATEUP, p) - abase) * 2u + (tid & 7) * 16;
  }
  ctx.adst = ((tid & 7) * BM + ((tid >> 3) ^ (2 * (tid & 7)))) * 8;
  ctx.npair = K / 64;

  f32x4_t acc[8][NW];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int f = 0; f < NW; ++f) acc[i][f] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // scale rows are visible to every wave after the loop's first barrier
  if (nrows <= 64)
    f8_loop<EPI, 4>(ctx, lds, sc, acc);
  else
    f8_loop<EPI, 8>(ctx, lds, sc, acc);

#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int m = 16 * i + r;
    if (m >= nrows) continue;
    const int64_t p = tile.row_begin + m;
    if (GATEUP) {
      const int nn = n_wave + 4 * q;
      if (nn < N) store4<EPI>(a, p, nn, acc[i][0], acc[i][1]);
    } else {
#pragma unroll
      for (int f = 0; f < NW; ++f) {
        const int nn = n_wave + 16 * f + 4 * q;
        if (nn < N) store4<EPI>(a, p, nn, acc[i][f], acc[i][f]);
      }
    }
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

// FP8 weights: the 128-row stream kernel above 16 rows per group.  Its tiles are half as
// tall and it converts every weight, so the skinny kernel stays ahead longer: K2-shape layer,
// ms, skinny / 128-row: T 128 2.88 / 3.51, 256 3.16 / 3.80, 448 3.42 / 3.89, 640 3.81 / 3.93.
constexpr int kWideRowsFp8 = 16;

TileSpec ffn_tile_spec_fp8(const FfnShape& sh) {
  return tile_spec_for(sh, use_wide(sh, kWideRowsFp8) ? kF8BM : kSkinnyBM);
}

hipError_t launch_gate_up_fp8(const FfnShape& sh, const uint16_t* x, const int32_t* perm,
                              const int32_t* offsets, const Fp8Weights& w, uint16_t* h,
                              Tile* tiles, int32_t* ntiles, hipStream_t s, bool tiles_ready) {
  const bool wide = use_wide(sh, kWideRowsFp8);
  const int BM = wide ? kF8BM : kSkinnyBM;
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
    hipLaunchKernelGGL(ffn_stream_fp8_kernel<kSwiGLU>, grid_for(sh, BM, kWideBNGateUp, a.N),
                       dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL((ffn_skinny_fp8_kernel<kSkinnyF8GuNF, kSkinnyF8GuKB, kSwiGLU>),
                       grid_for(sh, BM, 64 * kSkinnyF8GuNF, a.N), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_down_fp8(const FfnShape& sh, const uint16_t* h, const int32_t* offsets,
                           const Fp8Weights& w, float* y_routed, float* y_shared, Tile* tiles,
                           int32_t* ntiles, hipStream_t s, bool tiles_ready) {
  const bool wide = use_wide(sh, kWideRowsFp8);
  const int BM = wide ? kF8BM : kSkinnyBM;
  if (!tiles_ready) {
    hipError_t err = tiles_launch(sh, offsets, BM, tiles, ntiles, s);
    if (err != hipSuccess) return err;
  }
  FfnArgs a = fp8_args(sh, w, false, tiles, ntiles);
  a.A = h;
  a.a_rows = sh.T * sh.k + (sh.shared ? sh.T : 0);
  a.Y = y_routed;
  a.Ys = y_shared;
  a.N = sh.d;
  a.K = sh.I;
  if (wide)
    hipLaunchKernelGGL(ffn_stream_fp8_kernel<kF32>, grid_for(sh, BM, kWideBNDown, a.N),
                       dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL((ffn_skinny_fp8_kernel<kSkinnyF8DnNF, kSkinnyF8DnKB, kF32>),
                       grid_for(sh, BM, 64 * kSkinnyF8DnNF, a.N), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
