// Grouped expert GEMMs: gate/up with the SwiGLU product fused in the epilogue, and down.
// "Kimi K2 · Transformer blocks", expert equations g = x W1, u = x W3, a = g sigma(g),
// h = a (.) u, E_i = h W2; the shared expert is the same SwiGLU on every token.
//
// Work is a device-built list of row tiles (expert, rows [begin, end) of the grouped
// order); the shared expert is one more group (index E) whose rows are the T tokens.
// Each row tile is crossed with the n-blocks of the output; the grid is sized for the
// worst case and workgroups past the live count return at once, so no host sync is
// needed to learn the per-expert counts.
//
// Order of the work items: group by group (expert 0 first, the shared expert last),
// inside a group n-block by n-block, and inside an n-block the group's row tiles — so the
// row tiles that read the same weight tile are neighbours, and all n-blocks of an expert
// (which read the same activation rows) come together.  The hardware deals workgroups
// round-robin to the 8 XCDs; workgroup b takes item (b % 8) * ceil(total / 8) + b / 8, so
// each XCD walks one contiguous run of items and an expert's weight and activation
// reuse stays inside one L2.
//
// Two kernels: "skinny" for row tiles of <= 16 rows (decode: a few tokens per expert),
// weights streamed from HBM straight into MFMA registers and activations from L2; and an
// LDS-tiled kernel for 256-row tiles (prefill, and the dense projections), both operands
// staged in LDS and shared by the workgroup's eight waves.
#include "grouped.h"

namespace moe {
namespace {

// ------------------------------------------------------------- skinny GEMM
// Each wave owns NF 16-row strips of the weight matrix (two strips, W1 and W3, per
// fragment for gate/up) and runs them against the tile's <= 16 activation rows over the
// whole K.  Weights go straight from HBM to registers in the MFMA operand layout — each
// lane reads 16 contiguous bytes, four lanes cover 64 contiguous bytes of a weight row.
// All loads of a batch of KU k-steps are issued before the first MFMA of the batch
// (a scheduling barrier keeps the compiler from interleaving them), so a wave keeps
// KU * NF * (2 or 1) KiB of weights in flight.  Activation rows come from L2 (every
// n-block of the expert reads the same few rows).
//
// The MFMA computes C^T = W . A^T: weights as the A operand (16 output features),
// activations as the B operand (16 rows), so a lane ends up with four consecutive
// output features of one row and stores them with one 8-byte (bf16) or 16-byte (fp32)
// write.
//
// TWO: the activation rows are in two bf16 parts [hi | lo] (K = 2 WK) and the weight rows
// have WK elements; reduction index k reads weight column k mod WK.
template <int NF, int KU, int EPI, bool TWO = false>
__global__ __launch_bounds__(256) void ffn_skinny_kernel(const FfnArgs a) {
  constexpr bool GATEUP = EPI == kSwiGLU;
  constexpr int BN = 4 * 16 * NF;
  Tile tile;
  int nb;
  if (!map_work(a, (a.N + BN - 1) / BN, tile, nb)) return;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, q = lane >> 4;
  const int K = a.K, N = a.N;
  const int WK = TWO ? a.wk : K;
  auto wcol = [&](int k) { return TWO && k >= WK ? k - WK : k; };

  int64_t p = tile.row_begin + r;
  const bool row_ok = p < tile.row_end;
  if (!row_ok) p = tile.row_end - 1;
  const uint16_t* arow = act_row(a, GATEUP, p) + q * 8;

  const bool is_shared = tile.group >= a.E;
  const int64_t wofs = (int64_t)tile.group * N * WK;
  const uint16_t* W1 = is_shared ? a.S1 : a.B1 + wofs;
  const uint16_t* W3 = GATEUP ? (is_shared ? a.S3 : a.B3 + wofs) : nullptr;

  const int n0 = nb * BN + wave * 16 * NF;
  const uint16_t* w1p[NF];
  const uint16_t* w3p[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    int n = n0 + 16 * f + r;
    if (n > N - 1) n = N - 1;
    w1p[f] = W1 + (int64_t)n * WK + q * 8;
    w3p[f] = GATEUP ? W3 + (int64_t)n * WK + q * 8 : nullptr;
  }

  f32x4_t acc1[NF], acc3[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    acc1[f] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    acc3[f] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  int k0 = 0;
  for (; k0 + 32 * KU <= K; k0 += 32 * KU) {
    u32x4_t av[KU], b1v[NF][KU], b3v[NF][KU];
#pragma unroll
    for (int u = 0; u < KU; ++u)
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        b1v[f][u] = load16(w1p[f] + wcol(k0 + 32 * u));
        if (GATEUP) b3v[f][u] = load16(w3p[f] + wcol(k0 + 32 * u));
      }
#pragma unroll
    for (int u = 0; u < KU; ++u) av[u] = load16(arow + k0 + 32 * u);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < KU; ++u)
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        acc1[f] = mfma16x16x32(b1v[f][u], av[u], acc1[f]);
        if (GATEUP) acc3[f] = mfma16x16x32(b3v[f][u], av[u], acc3[f]);
      }
  }
  for (; k0 < K; k0 += 32) {
    const u32x4_t av = load16(arow + k0);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      acc1[f] = mfma16x16x32(load16(w1p[f] + wcol(k0)), av, acc1[f]);
      if (GATEUP) acc3[f] = mfma16x16x32(load16(w3p[f] + wcol(k0)), av, acc3[f]);
    }
  }

  if (!row_ok) return;
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int nn = n0 + 16 * f + 4 * q;
    if (nn < N) store4<EPI>(a, p, nn, acc1[f], acc3[f]);
  }
}

// ------------------------------------------------------------- LDS-tiled GEMM
// 256-row tiles x 256 outputs per workgroup (gate/up: 128 features of W1 and the same 128
// of W3; otherwise 256 features).  Eight waves, two per SIMD, each owning 128 rows x 64
// outputs as eight 32 x 32 fp32 accumulator tiles in VGPRs, so every activation fragment
// read from LDS feeds two MFMAs and every weight fragment four; the 32x32x16 MFMA also
// reads half the operand bytes per flop of the 16x16x32 one.  With two waves per SIMD one
// wave's LDS reads and waits overlap the other's MFMAs.  (Four waves, one per SIMD, each
// with a 128 x 128 quarter in 256 accumulator registers, read less LDS per MFMA but hide
// nothing; they measured slower.)
//
// K goes in chunks of 64.  Per chunk a workgroup moves 32 KiB of weights and 32 KiB of
// activations (gate/up: rows of x gathered through perm, each lane's offset naming its
// row), 8 rows x 128 contiguous bytes per wave-wide 16-byte-per-lane transfer, all of them
// straight into LDS (buffer loads that write LDS, no registers):
//   - weights from HBM, three chunk buffers, requested two chunks ahead;
//   - activations (mostly L2 hits), two chunk buffers, requested one chunk ahead, at the
//     start of the chunk before.
// 160 KiB of LDS in all, five separate arrays.  Against activations staged through
// registers this took the prefill layer from 8.70-8.79 to 8.59-8.60 ms and the skewed
// 4,096-token layer from 3.33-3.36 to 3.19-3.20 ms (one box, alternating runs).
//
// LDS layout of a chunk operand (256 rows x 8 pieces of 16 bytes): the 1 KiB unit u holds
// rows 8u .. 8u+7; piece p of row m sits in slot 8 (m & 7) + (p ^ sigma(m)) of its unit,
// sigma(m) = (m & 7) ^ ((m >> 3) & 1).  A load lane fetches whichever piece belongs to its
// slot, so the global reads stay 128 contiguous bytes per row, and an MFMA operand read
// (16 consecutive rows, one piece) touches 16 distinct 16-byte bank groups.
constexpr int kLdsChunkK = 64;
// Eight waves per workgroup (four, one per SIMD, measured slower: see the launch below).
constexpr int kLdsWaves = 8;
constexpr int kLdsUnits = 32 / kLdsWaves;  // 1 KiB transfers per wave and operand (4)
constexpr int kLdsNO = 2;                  // 32-output fragments per wave

struct LdsCtx {
  __amdgpu_buffer_rsrc_t act;  // activation rows (x, or the tile's rows of h)
  __amdgpu_buffer_rsrc_t wgt;  // this wave's weight matrix (gate/up: W1 for the first
                               // half of the waves, W3 for the second)
  uint32_t aoff[kLdsUnits];    // per-lane byte offset of the wave's activation units
  uint32_t woff[2];            // per-lane byte offset of the wave's even / odd weight
                               // units, less the unit stride
  uint32_t wstride;            // bytes between the wave's consecutive weight units (8 rows)
  uint32_t aoob, woob;         // a wave-uniform offset past the end of act / wgt: a load
                               // there returns zeros and moves no data
  int wrd[4];                  // per-lane slot (16 B units) of sub-step kk's piece in the
  int ard[4];                  // wave's first weight / activation row fragment
  int nc;                      // chunks
  int ncw;                     // chunks of a weight row: chunk c reads weight chunk c mod ncw
                               // (ncw < nc only for two-part activations)
};

// Whole-chunk weight move, for the prologue: the wave's weight transfers of chunk c
// (units kLdsUnits wave ..).
__device__ __forceinline__ void lds_fetch_w(const LdsCtx& x, u32x4_t* wgt, int wave, int c) {
  const uint32_t soff = c < x.nc ? (uint32_t)(c >= x.ncw ? c - x.ncw : c) * (kLdsChunkK * 2)
                                  : x.woob;
#pragma unroll
  for (int j = 0; j < kLdsUnits; ++j)
    dma16(x.wgt, wgt + (wave * kLdsUnits + j) * 64, x.woff[j & 1],
          soff + (uint32_t)j * x.wstride);
}

// Sub-step kk reads weight fragment o at slot wrd[kk] + 8 wfrag_row(o) and row fragment t
// (tile rows 64 t + 32 wm ..) at slot ard[kk] + 512 t (the wave-dependent parts are in
// wrd/ard, so the fragment offsets are immediates).
template <bool GATEUP>
__device__ __forceinline__ constexpr int wfrag_row(int o) {
  // gate/up: o = 0 the wave's 32 W1 features, o = 1 the same features of W3 (128 rows
  // further); otherwise 32 o
  return GATEUP ? 128 * o : 32 * o;
}

// Chunk c reads activation buffer Acur and weight buffer Wcur; during it the activations
// of chunk c + 1 go to Anext (sub-steps 0 and 1, half of the wave's units each) and the
// weights of chunk c + 2 to Wnext2 (sub-steps 2 and 3).  All buffers are separate LDS
// arrays, so the compiler can tell which pending transfer an LDS read depends on.  At the
// barrier before chunk c + 1 only the wave's 4 weight transfers of chunk c + 2 may still be
// in flight: the activation transfers of chunk c + 1 were issued before them, and
// transfers complete in order.
__device__ __forceinline__ void lds_sync_chunk() {
  static_assert(kLdsUnits == 4, "the wait below counts the wave's weight transfers");
  asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Half of the wave's activation (weight) transfers of chunk c: units j0 .. j0 + H - 1 of the
// wave's kLdsUnits, H = kLdsUnits / 2.
__device__ __forceinline__ void lds_fetch_a(const LdsCtx& x, u32x4_t* act, int wave, int c,
                                            int j0) {
  const uint32_t soff = c < x.nc ? (uint32_t)c * (kLdsChunkK * 2) : x.aoob;
#pragma unroll
  for (int j = j0; j < j0 + kLdsUnits / 2; ++j)
    dma16(x.act, act + (wave * kLdsUnits + j) * 64, x.aoff[j], soff);
}

__device__ __forceinline__ void lds_fetch_w_half(const LdsCtx& x, u32x4_t* wgt, int wave,
                                                 int c, int j0) {
  const uint32_t soff = c < x.nc ? (uint32_t)(c >= x.ncw ? c - x.ncw : c) * (kLdsChunkK * 2)
                                  : x.woob;
#pragma unroll
  for (int j = j0; j < j0 + kLdsUnits / 2; ++j)
    dma16(x.wgt, wgt + (wave * kLdsUnits + j) * 64, x.woff[j & 1],
          soff + (uint32_t)j * x.wstride);
}

template <bool GATEUP, int NF>
__device__ __forceinline__ void lds_chunk_dma(const LdsCtx& x, const u32x4_t* acur,
                                              u32x4_t* anext, const u32x4_t* wcur,
                                              u32x4_t* wnext2, int wave, int c,
                                              f32x16_t (&acc)[NF > 0 ? NF : 1][kLdsNO]) {
  lds_sync_chunk();
  constexpr int NA = NF > 0 ? NF : 1;
  u32x4_t wv[2][kLdsNO], av[2][NA];
  auto read = [&](int kk, int b) {
#pragma unroll
    for (int o = 0; o < kLdsNO; ++o) wv[b][o] = wcur[x.wrd[kk] + 8 * wfrag_row<GATEUP>(o)];
#pragma unroll
    for (int t = 0; t < NF; ++t) av[b][t] = acur[x.ard[kk] + 512 * t];
  };
  if constexpr (NF > 0) read(0, 0);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    if (kk < 2) lds_fetch_a(x, anext, wave, c + 1, (kLdsUnits / 2) * kk);
    else lds_fetch_w_half(x, wnext2, wave, c + 2, (kLdsUnits / 2) * (kk - 2));
    if constexpr (NF > 0) {
      if (kk < 3) read(kk + 1, (kk + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < NF; ++t)
#pragma unroll
        for (int o = 0; o < kLdsNO; ++o)
          acc[t][o] = mfma32x32x16(wv[kk & 1][o], av[kk & 1][t], acc[t][o]);
    }
  }
}

struct LdsBufs {
  u32x4_t* A;     // activation chunk buffers of even and odd chunks (2048 slots each;
  u32x4_t* A1;    // separate LDS arrays, like the weight buffers)
  u32x4_t* W0;    // weight chunk buffers (named separately so that the compiler can tell
  u32x4_t* W1;    // which transfers a read depends on)
  u32x4_t* W2;
};

// A tile for a wave with NF live row fragments (NF = 0: the wave only moves data): the K
// loop, then the epilogue.  Every wave runs the same loads and barriers whatever its NF.
template <int EPI, int NF>
__device__ __forceinline__ void lds_tile(const FfnArgs& a, const LdsCtx& x, const LdsBufs& b,
                                         int wave, int arow, const Tile& tile, int nbase,
                                         int col0) {
  constexpr bool GATEUP = EPI == kSwiGLU;
  constexpr int NA = NF > 0 ? NF : 1;
  f32x16_t acc[NA][kLdsNO];
#pragma unroll
  for (int t = 0; t < NA; ++t)
#pragma unroll
    for (int o = 0; o < kLdsNO; ++o)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[t][o][e] = 0.f;

  const int nc = x.nc;
  // prologue: activations of chunk 0, then the weights of chunks 0 and 1 (the first
  // barrier leaves only chunk 1's weights in flight)
  lds_fetch_a(x, b.A, wave, 0, 0);
  lds_fetch_a(x, b.A, wave, 0, kLdsUnits / 2);
  lds_fetch_w(x, b.W0, wave, 0);
  lds_fetch_w(x, b.W1, wave, 1);
  // chunk parity picks the activation buffer, chunk mod 3 the weight buffer: period 6
  int c = 0;
  for (; c + 6 <= nc; c += 6) {
    lds_chunk_dma<GATEUP, NF>(x, b.A, b.A1, b.W0, b.W2, wave, c, acc);
    lds_chunk_dma<GATEUP, NF>(x, b.A1, b.A, b.W1, b.W0, wave, c + 1, acc);
    lds_chunk_dma<GATEUP, NF>(x, b.A, b.A1, b.W2, b.W1, wave, c + 2, acc);
    lds_chunk_dma<GATEUP, NF>(x, b.A1, b.A, b.W0, b.W2, wave, c + 3, acc);
    lds_chunk_dma<GATEUP, NF>(x, b.A, b.A1, b.W1, b.W0, wave, c + 4, acc);
    lds_chunk_dma<GATEUP, NF>(x, b.A1, b.A, b.W2, b.W1, wave, c + 5, acc);
  }
  if (c < nc) lds_chunk_dma<GATEUP, NF>(x, b.A, b.A1, b.W0, b.W2, wave, c, acc);
  if (c + 1 < nc) lds_chunk_dma<GATEUP, NF>(x, b.A1, b.A, b.W1, b.W0, wave, c + 1, acc);
  if (c + 2 < nc) lds_chunk_dma<GATEUP, NF>(x, b.A, b.A1, b.W2, b.W1, wave, c + 2, acc);
  if (c + 3 < nc) lds_chunk_dma<GATEUP, NF>(x, b.A1, b.A, b.W0, b.W2, wave, c + 3, acc);
  if (c + 4 < nc) lds_chunk_dma<GATEUP, NF>(x, b.A, b.A1, b.W1, b.W0, wave, c + 4, acc);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  lds_barrier();
  if constexpr (NF > 0) {
    // staging: the first half of the waves in the even buffer, the rest in the odd one
    // (8 KiB per wave)
    constexpr int HW = kLdsWaves / 2, SL = 2048 / HW;
    if (wave < HW)
      lds_epilogue<EPI, NF, kLdsNO>(a, b.A + (wave % HW) * SL, acc, arow, 64, tile, nbase,
                                    col0);
    else
      lds_epilogue<EPI, NF, kLdsNO>(a, b.A1 + (wave % HW) * SL, acc, arow, 64, tile, nbase,
                                    col0);
  }
}

template <int EPI>
__global__ __launch_bounds__(64 * kLdsWaves, 1) void ffn_lds_kernel(const FfnArgs a) {
  constexpr bool GATEUP = EPI == kSwiGLU;
  constexpr int BM = 256;
  constexpr int FEAT = GATEUP ? 128 : 256;  // features of N per workgroup
  __shared__ __attribute__((aligned(1024))) u32x4_t Ab[BM * 8];
  __shared__ __attribute__((aligned(1024))) u32x4_t Ab1[BM * 8];
  __shared__ __attribute__((aligned(1024))) u32x4_t W0[BM * 8];
  __shared__ __attribute__((aligned(1024))) u32x4_t W1[BM * 8];
  __shared__ __attribute__((aligned(1024))) u32x4_t W2[BM * 8];

  // fp32 output only: K cut into ksplit slices, the slices of one n-block adjacent
  const int nks = (EPI == kF32 && a.ksplit > 1) ? a.ksplit : 1;
  Tile tile;
  int nbk;
  if (!map_work(a, ((a.N + FEAT - 1) / FEAT) * nks, tile, nbk)) return;
  const int nb = nbk / nks, ks = nbk - nb * nks;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // wave (wm, wn): rows half wm, outputs part wn (of 4)
  const int wm = wave / (kLdsWaves / 2), wn = wave % (kLdsWaves / 2);
  const int K = a.K, N = a.N;
  const int nrows = tile.row_end - tile.row_begin;
  const int f0 = nb * FEAT;

  // weight row length: K, or half of it for two-part activations ([hi | lo], K = 2 WK; no K
  // slices then)
  const int WK = a.wk > 0 ? a.wk : K;
  const bool is_shared = tile.group >= a.E;
  const int64_t wofs = (int64_t)tile.group * N * WK;
  const uint16_t* Wa = is_shared ? a.S1 : a.B1 + wofs;
  const uint16_t* Wb = GATEUP ? (is_shared ? a.S3 : a.B3 + wofs) : Wa;

  // this slice's chunks c0 .. c1 - 1 of K: its byte offset goes into every row's
  // starting offset (rows past the tile or the matrix keep theirs, past the buffer end)
  const int nct = K / kLdsChunkK;
  const int c0 = nct * ks / nks, c1 = nct * (ks + 1) / nks;
  const uint32_t kofs = (uint32_t)c0 * (kLdsChunkK * 2);

  LdsCtx x;
  // one weight matrix is N*K*2 < 2^32 bytes, and so is x (checked on the host)
  const uint32_t wbytes = (uint32_t)N * (uint32_t)WK * 2u;
  x.wgt = buffer_rsrc(GATEUP && wave >= kLdsWaves / 2 ? Wb : Wa, wbytes);
  const uint16_t* abase = GATEUP ? a.A : a.A + (int64_t)tile.row_begin * K;
  const uint32_t abytes = GATEUP ? (uint32_t)(a.a_rows * K * 2) : (uint32_t)nrows * K * 2u;
  x.act = buffer_rsrc(abase, abytes);
  // transfer lane l of unit u: row 8u + (l >> 3), slot piece l & 7 holding piece
  // (l & 7) ^ sigma(row)
  // rows past the tile's end load nothing (an offset past the buffer reads zeros and
  // moves no data; their outputs are not stored)
#pragma unroll
  for (int j = 0; j < kLdsUnits; ++j) {
    const int u = wave * kLdsUnits + j, m = 8 * u + (lane >> 3);
    const int piece = (lane & 7) ^ (m & 7) ^ (u & 1);
    const int64_t p = tile.row_begin + m;
    x.aoff[j] = p < tile.row_end
                    ? (uint32_t)(act_row(a, GATEUP, p) - abase) * 2u + piece * 16 + kofs
                    : abytes;
  }
  // weight row m of the workgroup: gate/up rows 0..127 are W1 features f0 + m, rows
  // 128..255 the same features of W3; otherwise features f0 + m.  Unit j of the wave:
  // m = 8 (kLdsUnits wave + j) + (lane >> 3), piece (lane & 7) ^ (lane >> 3) ^ (j & 1).
  // Features past N read beyond the matrix and get zeros (their outputs are not stored).
  {
    constexpr int RPW = 8 * kLdsUnits;  // weight rows per wave
    const int n0 = f0 + RPW * (GATEUP ? (wave % (kLdsWaves / 2)) : wave) + (lane >> 3);
#pragma unroll
    for (int e = 0; e < 2; ++e)
      x.woff[e] = (uint32_t)n0 * (uint32_t)WK * 2u + ((lane & 7) ^ (lane >> 3) ^ e) * 16 + kofs;
    x.wstride = 8u * (uint32_t)WK * 2u;
  }
  // the two row halves interleave 32-row fragments (wave wm: tile rows 64 t + 32 wm ..),
  // so a partly filled tile keeps both halves equally busy
  const int arow = 32 * wm;
  // first weight row of this wave's fragments: gate/up W1 rows 32 wn (W3 rows 128 + 32 wn);
  // otherwise 64 wn
  constexpr int OPW = 256 / (kLdsWaves / 2);  // weight rows of the wave's fragments
  const int wrow0 = (GATEUP ? OPW / 2 : OPW) * wn;
  {
    const int r32 = lane & 31, sig = (lane & 7) ^ ((r32 >> 3) & 1);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int rd = (r32 >> 3) * 64 + (lane & 7) * 8 + ((2 * kk + (lane >> 5)) ^ sig);
      x.wrd[kk] = wrow0 * 8 + rd;
      x.ard[kk] = arow * 8 + rd;
    }
  }
  x.nc = c1 - c0;
  x.ncw = WK < K ? WK / kLdsChunkK : x.nc;
  // both buffers are under 2 GiB (checked on the host), so offset + this stays in 32 bits
  x.aoob = abytes;
  x.woob = wbytes;
  // first output feature of this wave's fragments (gate/up: of its W1 and W3 fragments)
  const int nbase = f0 + (GATEUP ? OPW / 2 : OPW) * wn;

  // live 32-row fragments of this wave's half of the tile (wave-uniform)
  const int nf = min(4, max(0, (nrows - arow + 63) / 64));
  const LdsBufs bufs{Ab, Ab1, W0, W1, W2};
  const int col0 = ks * N;  // this slice's columns in a row of Ys
  switch (nf) {
    case 0: lds_tile<EPI, 0>(a, x, bufs, wave, arow, tile, nbase, col0); break;
    case 1: lds_tile<EPI, 1>(a, x, bufs, wave, arow, tile, nbase, col0); break;
    case 2: lds_tile<EPI, 2>(a, x, bufs, wave, arow, tile, nbase, col0); break;
    case 3: lds_tile<EPI, 3>(a, x, bufs, wave, arow, tile, nbase, col0); break;
    default: lds_tile<EPI, 4>(a, x, bufs, wave, arow, tile, nbase, col0); break;
  }
}

}  // namespace

int64_t ffn_max_tiles(const FfnShape& sh) { return max_tiles_for(sh, kSkinnyBM); }

// bf16 weights: the 256-row kernel from 5 rows per group on (and from d = 512 on).  The
// whole K2-shape layer (d 7168, 384 experts, top-8, I 2048) over T = 64..640, each kernel
// forced (one box, two passes, ms): T 64 4.16 skinny / 4.31 256-row, 128 5.25 / 5.25,
// 192 5.55 / 5.55, 224 5.64 / 5.58, 256 5.67 / 5.61, 448 6.14 / 5.83, 640 7.37 / 6.01.
// Switching at 16 rows per group left T = 200..680 up to 18% slow.
constexpr int kWideRowsBf16 = 5;

TileSpec ffn_tile_spec(const FfnShape& sh) {
  return tile_spec_for(sh, use_wide(sh, kWideRowsBf16) ? kWideBM : kSkinnyBM);
}

// Eight waves against four, each forced over the K2-shape layer: prefill gate/up 5.07-5.13
// against 5.22-5.28 ms (alternating runs on one box, three each), down 3.01 against 3.03;
// skewed routing 3.18-3.19 against 3.30-3.33 ms; the latent variant 4.26 against 4.27;
// the router GEMM 144 against 152 us (T = 8192) and 74 against 80 us (T = 4096).
// The 256-row-tile kernel covers 128 (gate/up) or 256 (otherwise) features of N per block.
template <int EPI>
void launch_wide(dim3 grid, hipStream_t s, const FfnArgs& a) {
  hipLaunchKernelGGL(ffn_lds_kernel<EPI>, grid, dim3(64 * kLdsWaves), 0, s, a);
}

hipError_t launch_dense(const uint16_t* A, int64_t rows, int K, const uint16_t* W, int N,
                        DenseOut mode, float* Cf, uint16_t* Cb, const float* R, Tile* tiles,
                        int32_t* ntiles, hipStream_t s, int ksplit, int wk) {
  // the epilogues store whole 4-output groups: an output row must be a multiple of 4
  if ((N & 3) != 0) return hipErrorInvalidValue;
  // two-part activations: K = 2 wk, no K slices
  if (wk > 0 && (K != 2 * wk || ksplit > 1)) return hipErrorInvalidValue;
  // one group (the "shared" slot of the tile list) whose rows are all the rows of A
  const FfnShape sh{rows, K, 0, 0, N, true};
  const bool wide = rows > kSingleGroupWideRows;
  const int BM = wide ? kWideBM : kSkinnyBM;
  hipError_t err = tiles_launch(sh, nullptr, BM, tiles, ntiles, s);
  if (err != hipSuccess) return err;
  FfnArgs a{};
  a.A = A;
  a.a_rows = rows;
  a.routed_rows = 0;
  a.S1 = W;
  a.Ys = Cf;
  a.C = Cb;
  a.R = R;
  a.tiles = tiles;
  a.ntiles = ntiles;
  a.k = 1;
  a.N = N;
  a.K = K;
  a.wk = wk;
  a.E = 0;
  // K slices only on the 256-row kernel's fp32 output, each at least one 64-k chunk
  const int nks = (mode == DenseOut::kF32 && wide && ksplit > 1)
                      ? (ksplit < K / kLdsChunkK ? ksplit : K / kLdsChunkK)
                      : 1;
  a.ksplit = nks;
  a.ldc = nks * N;
  const dim3 gs = grid_for(sh, BM, kWideBNDown, N), gk = grid_for(sh, BM, 64, N),
             gk2 = grid_for(sh, BM, 128, N);
  const bool two = wk > 0;
  switch (mode) {
    case DenseOut::kF32:
      if (wide) launch_wide<kF32>(dim3(gs.x * nks), s, a);
      else if (two) hipLaunchKernelGGL((ffn_skinny_kernel<1, kSkinnyKU, kF32, true>), gk, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((ffn_skinny_kernel<1, kSkinnyKU, kF32>), gk, dim3(256), 0, s, a);
      break;
    case DenseOut::kBF16:
      if (wide) launch_wide<kBF16>(gs, s, a);
      else if (two) hipLaunchKernelGGL((ffn_skinny_kernel<2, kSkinnyKU, kBF16, true>), gk2, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((ffn_skinny_kernel<2, kSkinnyKU, kBF16>), gk2, dim3(256), 0, s, a);
      break;
    case DenseOut::kAddBF16:
      if (wide) launch_wide<kAddBF16>(gs, s, a);
      else if (two) hipLaunchKernelGGL((ffn_skinny_kernel<2, kSkinnyKU, kAddBF16, true>), gk2, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((ffn_skinny_kernel<2, kSkinnyKU, kAddBF16>), gk2, dim3(256), 0, s, a);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_gate_up(const FfnShape& sh, const uint16_t* x, const int32_t* perm,
                          const int32_t* offsets, const uint16_t* w1, const uint16_t* w3,
                          const uint16_t* ws1, const uint16_t* ws3, uint16_t* h, Tile* tiles,
                          int32_t* ntiles, hipStream_t s, bool tiles_ready) {
  const bool wide = use_wide(sh, kWideRowsBf16);
  const int BM = wide ? kWideBM : kSkinnyBM;
  if (!tiles_ready) {
    hipError_t err = tiles_launch(sh, offsets, BM, tiles, ntiles, s);
    if (err != hipSuccess) return err;
  }
  FfnArgs a{};
  a.A = x;
  a.a_rows = sh.T;
  a.perm = perm;
  a.routed_rows = sh.T * sh.k;
  a.B1 = w1;
  a.B3 = w3;
  a.S1 = ws1;
  a.S3 = ws3;
  a.C = h;
  a.tiles = tiles;
  a.ntiles = ntiles;
  a.k = sh.k;
  a.N = sh.I;
  a.K = sh.d;
  a.E = sh.E;
  a.hsplit = sh.hsplit ? 1 : 0;
  if (wide) {
    launch_wide<kSwiGLU>(grid_for(sh, BM, kWideBNGateUp, a.N), s, a);
  } else {
    hipLaunchKernelGGL((ffn_skinny_kernel<kSkinnyGuNF, kSkinnyGuKU, kSwiGLU>),
                       grid_for(sh, BM, 64 * kSkinnyGuNF, a.N), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_down(const FfnShape& sh, const uint16_t* h, const int32_t* offsets,
                       const uint16_t* w2, const uint16_t* ws2, void* y_routed, void* y_shared,
                       Tile* tiles, int32_t* ntiles, hipStream_t s, bool tiles_ready,
                       bool y24) {
  const bool wide = use_wide(sh, kWideRowsBf16);
  const int BM = wide ? kWideBM : kSkinnyBM;
  if (!tiles_ready) {
    hipError_t err = tiles_launch(sh, offsets, BM, tiles, ntiles, s);
    if (err != hipSuccess) return err;
  }
  FfnArgs a{};
  a.A = h;
  a.a_rows = sh.T * sh.k + (sh.shared ? sh.T : 0);
  a.perm = nullptr;
  a.routed_rows = sh.T * sh.k;
  a.B1 = w2;
  a.B3 = nullptr;
  a.S1 = ws2;
  a.S3 = nullptr;
  a.Y = static_cast<float*>(y_routed);
  a.Ys = static_cast<float*>(y_shared);
  a.tiles = tiles;
  a.ntiles = ntiles;
  a.k = sh.k;
  a.N = sh.d;
  // h in two bf16 parts: rows [hi | lo] of 2I, each weight used for both
  a.K = sh.hsplit ? 2 * sh.I : sh.I;
  a.wk = sh.hsplit ? sh.I : 0;
  a.E = sh.E;
  const dim3 gw = grid_for(sh, BM, kWideBNDown, a.N), gs = grid_for(sh, BM, 64 * kSkinnyNF, a.N);
  if (wide) {
    if (y24) launch_wide<kF24>(gw, s, a);
    else launch_wide<kF32>(gw, s, a);
  } else if (sh.hsplit) {
    if (y24)
      hipLaunchKernelGGL((ffn_skinny_kernel<kSkinnyNF, kSkinnyKU, kF24, true>), gs, dim3(256),
                         0, s, a);
    else
      hipLaunchKernelGGL((ffn_skinny_kernel<kSkinnyNF, kSkinnyKU, kF32, true>), gs, dim3(256),
                         0, s, a);
  } else {
    if (y24)
      hipLaunchKernelGGL((ffn_skinny_kernel<kSkinnyNF, kSkinnyKU, kF24>), gs, dim3(256), 0, s,
                         a);
    else
      hipLaunchKernelGGL((ffn_skinny_kernel<kSkinnyNF, kSkinnyKU, kF32>), gs, dim3(256), 0, s,
                         a);
  }
  return hipGetLastError();
}

}  // namespace moe
