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
// Two kernels, both streaming weights from HBM straight into MFMA registers: "skinny"
// for row tiles of <= 16 rows (decode: a few tokens per expert), activations from L2;
// "stream" for 256-row tiles (prefill), activations staged in LDS and shared by the
// workgroup's waves.
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
template <int NF, int KU, int EPI>
__global__ __launch_bounds__(256) void ffn_skinny_kernel(const FfnArgs a) {
  constexpr bool GATEUP = EPI == kSwiGLU;
  constexpr int BN = 4 * 16 * NF;
  Tile tile;
  int nb;
  if (!map_work(a, (a.N + BN - 1) / BN, tile, nb)) return;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, q = lane >> 4;
  const int K = a.K, N = a.N;

  int64_t p = tile.row_begin + r;
  const bool row_ok = p < tile.row_end;
  if (!row_ok) p = tile.row_end - 1;
  const uint16_t* arow = act_row(a, GATEUP, p) + q * 8;

  const bool is_shared = tile.group >= a.E;
  const int64_t wofs = (int64_t)tile.group * N * K;
  const uint16_t* W1 = is_shared ? a.S1 : a.B1 + wofs;
  const uint16_t* W3 = GATEUP ? (is_shared ? a.S3 : a.B3 + wofs) : nullptr;

  const int n0 = nb * BN + wave * 16 * NF;
  const uint16_t* w1p[NF];
  const uint16_t* w3p[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    int n = n0 + 16 * f + r;
    if (n > N - 1) n = N - 1;
    w1p[f] = W1 + (int64_t)n * K + q * 8;
    w3p[f] = GATEUP ? W3 + (int64_t)n * K + q * 8 : nullptr;
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
        b1v[f][u] = load16(w1p[f] + k0 + 32 * u);
        if (GATEUP) b3v[f][u] = load16(w3p[f] + k0 + 32 * u);
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
      acc1[f] = mfma16x16x32(load16(w1p[f] + k0), av, acc1[f]);
      if (GATEUP) acc3[f] = mfma16x16x32(load16(w3p[f] + k0), av, acc3[f]);
    }
  }

  if (!row_ok) return;
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int nn = n0 + 16 * f + 4 * q;
    if (nn < N) store4<EPI>(a, p, nn, acc1[f], acc3[f]);
  }
}

// ------------------------------------------------------------- stream GEMM
// 256-row tiles (prefill: an expert's rows usually fit one tile, so its weights leave HBM
// once).  Eight waves, each owning all of the tile's rows (16 row fragments) x 32 outputs
// (gate/up: 16 features of W1 and the same 16 of W3; down: 32 features), so no two waves
// load the same weights.  Weights stream from HBM straight into MFMA registers, the same
// operand layout as the skinny kernel, through a ring of six k-step register sets: five
// k-steps (10 KiB per wave, 80 KiB per CU) are in flight while one is multiplied.  The
// tile's activation rows are staged in LDS in 64-wide k-chunks, double-buffered, with one
// LDS-only barrier per chunk (it does not drain the weight loads in flight).  Within a
// buffer the 16-byte pieces are stored k-chunk-major with the row index XOR-swizzled by
// the chunk (slot = c * 256 + (m ^ 2c)), so the 16 lanes of an MFMA operand read (16 rows,
// one chunk) and of a chunk write (2 rows x 8 chunks) touch 16 distinct bank groups.  Activation fragments are
// read from LDS one at a time, one fragment ahead of the two MFMAs that use it.
// The main loop is straight-line code: it is instantiated for 4, 8, 12 or 16 live row
// fragments (the tile's rows rounded up to 64: rows past the end cost at most three
// fragments of MFMAs; finer steps measured slower, the extra copies of the loop crowd the
// instruction cache), prefetch indices are clamped instead of guarded, and one ring
// period (RING / 2 chunks) is unrolled per iteration so the register ring is indexed
// statically.  Branches inside the loop would make the compiler's wait-count analysis
// conservative at every join and wait for the prefetched loads too.
// Tuning constants of the stream kernel, measured on MI355X at the K2 prefill shape
// (gate/up, ms): 64-row granules 6.33 vs 128-row 6.95 vs none 6.60; read groups of 1
// fragment 6.33, 2: 6.34, 4: 6.88; without the scheduling barrier 8.40; ring depth 6:
// 6.25, 8: 6.87, 10: 7.47 (spills); weight requests batched two k-steps at a time 6.38.
#ifndef MOE_STREAM_NL_STEP
#define MOE_STREAM_NL_STEP 4      // live row fragments are rounded up to this multiple
#endif
#ifndef MOE_STREAM_GS
#define MOE_STREAM_GS 1           // activation fragments read from LDS per group
#endif
#ifndef MOE_STREAM_SCHED_BARRIER
#define MOE_STREAM_SCHED_BARRIER 1  // keep reads one group ahead of their MFMAs
#endif
#ifndef MOE_STREAM_RING
#define MOE_STREAM_RING 6         // k-steps of weights held in registers per wave (even)
#endif
#ifndef MOE_STREAM_BATCH
#define MOE_STREAM_BATCH 1        // k-steps of weights requested together (1 or 2)
#endif

struct StreamCtx {
  __amdgpu_buffer_rsrc_t w1;   // matrix of weight fragment 0 (and 1 unless gate/up)
  __amdgpu_buffer_rsrc_t w3;   // gate/up: matrix of weight fragment 1
  __amdgpu_buffer_rsrc_t act;  // activation rows (x, or the tile's rows of h)
  uint32_t woff[2];            // byte offset of the lane's row and k lane-group, per fragment
  uint32_t aoff[4];            // byte offset of each activation piece (row start + chunk)
  int adst;                    // LDS offset (elements) of the first activation piece; the
                               // XOR touches bits 1..3 of the row only, so piece i (row
                               // + 64 i) sits 64 i slots further
  int nks, nc;                 // k-steps (32) and chunks (64)
};

template <int EPI, int NL>
__device__ __forceinline__ void stream_loop(const StreamCtx& c_, uint16_t* lds,
                                            f32x4_t (&acc)[16][2]) {
  constexpr bool GATEUP = EPI == kSwiGLU;
  constexpr int BM = 256, BK = 64, NW = 2, NA = 4;
  constexpr int D = MOE_STREAM_RING, P = MOE_STREAM_BATCH;
  static_assert(D % 2 == 0 && D >= 4 && (P == 1 || P == 2), "weight ring shape");
  const int lane = threadIdx.x & 63, r = lane & 15, q = lane >> 4;
  const int nks = c_.nks, nc = c_.nc;
  u32x4_t W[D][NW], AR[NA];

  auto load_w = [&](u32x4_t* S, int ks) {
    const uint32_t kb = (uint32_t)(ks < nks ? ks : nks - 1) * 64;  // past the end: re-read
    S[0] = bload16(c_.w1, c_.woff[0], kb);
    S[1] = bload16(GATEUP ? c_.w3 : c_.w1, c_.woff[1], kb);
  };
  auto load_a = [&](int c) {
    const uint32_t cb = (uint32_t)(c < nc ? c : nc - 1) * (BK * 2);
#pragma unroll
    for (int i = 0; i < NA; ++i) AR[i] = bload16(c_.act, c_.aoff[i], cb);
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NA; ++i)
      *reinterpret_cast<u32x4_t*>(lds + buf * BM * BK + c_.adst + i * 64 * 8) = AR[i];
  };
  // slot of (row m, 8-element k-chunk c) = c * BM + (m ^ 2c): a lane's fragment read is
  // row 16 i + r of chunk c = 4 kk + q, i.e. slot c * BM + 16 i + (r ^ 2c)
  auto mma_step = [&](int buf, int kk, const u32x4_t* S) {
    constexpr int GS = MOE_STREAM_GS;         // fragments per read group
    const int c = 4 * kk + q;
    const uint16_t* As = lds + buf * BM * BK + (c * BM + (r ^ (2 * c))) * 8;
    u32x4_t G0[GS], G1[GS];
#pragma unroll
    for (int j = 0; j < GS; ++j) G0[j] = *reinterpret_cast<const u32x4_t*>(As + 16 * j * 8);
#pragma unroll
    for (int g = 0; g < NL / GS; ++g) {
      u32x4_t* cur = (g & 1) ? G1 : G0;
      u32x4_t* nxt = (g & 1) ? G0 : G1;
      if (g + 1 < NL / GS) {
#pragma unroll
        for (int j = 0; j < GS; ++j)
          nxt[j] = *reinterpret_cast<const u32x4_t*>(As + 16 * (GS * (g + 1) + j) * 8);
      }
#pragma unroll
      for (int j = 0; j < GS; ++j) {
        acc[GS * g + j][0] = mfma16x16x32(S[0], cur[j], acc[GS * g + j][0]);
        acc[GS * g + j][1] = mfma16x16x32(S[1], cur[j], acc[GS * g + j][1]);
      }
      if (MOE_STREAM_SCHED_BARRIER) __builtin_amdgcn_sched_barrier(0);
    }
  };
  // chunk c+1's activations (in AR) go to the other LDS buffer; AR then loads chunk c+2
  auto next_chunk = [&](int c) {
    store_a((c + 1) & 1);
    load_a(c + 2);
    lds_barrier();
  };
  // Chunk j of a ring period (k-steps s = 2c + 2j and s + 1, ring slots t = 2j, t + 1).
  // P = 1: each k-step refills the slot freed just before it, D - 1 k-steps in flight.
  // P = 2: both refills of the chunk are issued together at its start (128 contiguous
  // bytes of every weight row at once), D - 2 k-steps in flight.
  auto chunk = [&](int c, int j) {
    const int t = 2 * j, s = 2 * c + t;
    if (P == 1) {
      load_w(W[(t + D - 1) % D], s + D - 1);
      mma_step((c + j) & 1, 0, W[t]);
      load_w(W[t], s + D);
      mma_step((c + j) & 1, 1, W[t + 1]);
    } else {
      load_w(W[(t + D - 2) % D], s + D - 2);
      load_w(W[(t + D - 1) % D], s + D - 1);
      mma_step((c + j) & 1, 0, W[t]);
      mma_step((c + j) & 1, 1, W[t + 1]);
    }
    next_chunk(c + j);
  };

  load_a(0);
#pragma unroll
  for (int t = 0; t < D - P; ++t) load_w(W[t], t);
  store_a(0);
  load_a(1);
  lds_barrier();
  int c = 0;
  // at the top of an iteration W[t] holds k-step 2c + t for t < D - P
  for (; c + D / 2 <= nc; c += D / 2) {
#pragma unroll
    for (int j = 0; j < D / 2; ++j) chunk(c, j);
  }
#pragma unroll
  for (int j = 0; j < D / 2 - 1; ++j)
    if (c + j < nc) chunk(c, j);
}

// stream_loop instantiated for the smallest multiple of STEP fragments >= nfrag
template <int EPI, int STEP, int NL = STEP>
__device__ __forceinline__ void stream_dispatch(int nfrag, const StreamCtx& ctx, uint16_t* lds,
                                                f32x4_t (&acc)[16][2]) {
  if constexpr (NL >= 16) {
    stream_loop<EPI, 16>(ctx, lds, acc);
  } else {
    if (nfrag <= NL)
      stream_loop<EPI, NL>(ctx, lds, acc);
    else
      stream_dispatch<EPI, STEP, NL + STEP>(nfrag, ctx, lds, acc);
  }
}

template <int EPI>
__global__ __launch_bounds__(512, 1) void ffn_stream_kernel(const FfnArgs a) {
  constexpr bool GATEUP = EPI == kSwiGLU;
  constexpr int BM = 256, BK = 64;
  constexpr int FM = BM / 16;                 // row fragments (every wave has all rows)
  constexpr int NW = 2;                       // weight fragments per wave per k-step
  constexpr int FEAT_WAVE = GATEUP ? 16 : 32; // features of N per wave
  constexpr int FEAT = 8 * FEAT_WAVE;         // features of N per workgroup
  constexpr int NT = 512;                     // threads
  constexpr int NA = BM * BK / 8 / NT;        // 16-byte activation pieces per thread (4)
  static_assert(NA == 4 && FM == 16, "stream tile shape");
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * BM * BK];

  Tile tile;
  int nb;
  if (!map_work(a, (a.N + FEAT - 1) / FEAT, tile, nb)) return;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, q = lane >> 4;
  const int K = a.K, N = a.N;
  const int nrows = tile.row_end - tile.row_begin;
  const int n_wave = nb * FEAT + wave * FEAT_WAVE;

  const bool is_shared = tile.group >= a.E;
  const int64_t wofs = (int64_t)tile.group * N * K;
  const uint16_t* W1 = is_shared ? a.S1 : a.B1 + wofs;
  const uint16_t* W3 = GATEUP ? (is_shared ? a.S3 : a.B3 + wofs) : nullptr;

  StreamCtx ctx;
  // one weight matrix is N*K*2 < 2^32 bytes (checked on the host)
  const uint32_t wbytes = (uint32_t)N * (uint32_t)K * 2u;
  ctx.w1 = buffer_rsrc(W1, wbytes);
  ctx.w3 = buffer_rsrc(GATEUP ? W3 : W1, wbytes);
  // gate/up gathers rows of x (T*K*2 < 2^32 bytes, checked on the host); down reads the
  // tile's own contiguous rows of h
  const uint16_t* abase = GATEUP ? a.A : a.A + (int64_t)tile.row_begin * K;
  const uint32_t abytes = GATEUP ? (uint32_t)(a.a_rows * K * 2) : (uint32_t)nrows * K * 2u;
  ctx.act = buffer_rsrc(abase, abytes);
  // weight fragment f: gate/up: f = 0 -> W1 rows, f = 1 -> the same rows of W3;
  // down: 16 rows each
#pragma unroll
  for (int f = 0; f < NW; ++f) {
    int n = n_wave + (GATEUP ? 0 : 16 * f) + r;
    if (n > N - 1) n = N - 1;
    ctx.woff[f] = ((uint32_t)n * (uint32_t)K + q * 8) * 2u;
  }
  // activation pieces of this thread: row (tid >> 3) + 64 i, 16-byte chunk tid & 7
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int m = (tid >> 3) + (NT / 8) * i;
    int64_t p = tile.row_begin + m;
    if (p >= tile.row_end) p = tile.row_end - 1;
    ctx.aoff[i] = (uint32_t)(act_row(a, GATEUP, p) - abase) * 2u + (tid & 7) * 16;
  }
  ctx.adst = ((tid & 7) * BM + ((tid >> 3) ^ (2 * (tid & 7)))) * 8;
  ctx.nks = K / 32;
  ctx.nc = K / BK;

  f32x4_t acc[FM][NW];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int f = 0; f < NW; ++f) acc[i][f] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // live row fragments rounded up to a multiple of MOE_STREAM_NL_STEP (workgroup-uniform)
  const int nfrag = (nrows + 15) / 16;
  stream_dispatch<EPI, MOE_STREAM_NL_STEP>(nfrag, ctx, lds, acc);

  // epilogue: acc[i][f] of this lane = tile row 16 i + r, features 4 q .. 4 q + 3 of
  // weight fragment f
#pragma unroll
  for (int i = 0; i < FM; ++i) {
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

}  // namespace

int64_t ffn_max_tiles(const FfnShape& sh) { return max_tiles_for(sh, kSkinnyBM); }

// The 256-row-tile kernel covers 128 (gate/up) or 256 (otherwise) features of N per block.
template <int EPI>
void launch_wide(dim3 grid, hipStream_t s, const FfnArgs& a) {
  hipLaunchKernelGGL(ffn_stream_kernel<EPI>, grid, dim3(512), 0, s, a);
}

hipError_t launch_dense(const uint16_t* A, int64_t rows, int K, const uint16_t* W, int N,
                        DenseOut mode, float* Cf, uint16_t* Cb, const float* R, Tile* tiles,
                        int32_t* ntiles, hipStream_t s) {
  // one group (the "shared" slot of the tile list) whose rows are all the rows of A
  const FfnShape sh{rows, K, 0, 0, N, true};
  const bool wide = rows > 512;
  const int BM = wide ? kStreamBM : kSkinnyBM;
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
  a.E = 0;
  const dim3 gs = grid_for(sh, BM, kStreamBNDown, N), gk = grid_for(sh, BM, 64, N),
             gk2 = grid_for(sh, BM, 128, N);
  switch (mode) {
    case DenseOut::kF32:
      if (wide) launch_wide<kF32>(gs, s, a);
      else hipLaunchKernelGGL((ffn_skinny_kernel<1, kSkinnyKU, kF32>), gk, dim3(256), 0, s, a);
      break;
    case DenseOut::kBF16:
      if (wide) launch_wide<kBF16>(gs, s, a);
      else hipLaunchKernelGGL((ffn_skinny_kernel<2, kSkinnyKU, kBF16>), gk2, dim3(256), 0, s, a);
      break;
    case DenseOut::kAddBF16:
      if (wide) launch_wide<kAddBF16>(gs, s, a);
      else hipLaunchKernelGGL((ffn_skinny_kernel<2, kSkinnyKU, kAddBF16>), gk2, dim3(256), 0, s, a);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_gate_up(const FfnShape& sh, const uint16_t* x, const int32_t* perm,
                          const int32_t* offsets, const uint16_t* w1, const uint16_t* w3,
                          const uint16_t* ws1, const uint16_t* ws3, uint16_t* h, Tile* tiles,
                          int32_t* ntiles, hipStream_t s) {
  const bool wide = use_wide(sh);
  const int BM = wide ? kStreamBM : kSkinnyBM;
  hipError_t err = tiles_launch(sh, offsets, BM, tiles, ntiles, s);
  if (err != hipSuccess) return err;
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
  if (wide)
    launch_wide<kSwiGLU>(grid_for(sh, BM, kStreamBNGateUp, a.N), s, a);
  else
    hipLaunchKernelGGL((ffn_skinny_kernel<kSkinnyNF, kSkinnyKU, kSwiGLU>),
                       grid_for(sh, BM, 64 * kSkinnyNF, a.N), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_down(const FfnShape& sh, const uint16_t* h, const int32_t* offsets,
                       const uint16_t* w2, const uint16_t* ws2, float* y_routed,
                       float* y_shared, Tile* tiles, int32_t* ntiles, hipStream_t s) {
  const bool wide = use_wide(sh);
  const int BM = wide ? kStreamBM : kSkinnyBM;
  hipError_t err = tiles_launch(sh, offsets, BM, tiles, ntiles, s);
  if (err != hipSuccess) return err;
  FfnArgs a{};
  a.A = h;
  a.a_rows = sh.T * sh.k + (sh.shared ? sh.T : 0);
  a.perm = nullptr;
  a.routed_rows = sh.T * sh.k;
  a.B1 = w2;
  a.B3 = nullptr;
  a.S1 = ws2;
  a.S3 = nullptr;
  a.Y = y_routed;
  a.Ys = y_shared;
  a.tiles = tiles;
  a.ntiles = ntiles;
  a.k = sh.k;
  a.N = sh.d;
  a.K = sh.I;
  a.E = sh.E;
  if (wide)
    launch_wide<kF32>(grid_for(sh, BM, kStreamBNDown, a.N), s, a);
  else
    hipLaunchKernelGGL((ffn_skinny_kernel<kSkinnyNF, kSkinnyKU, kF32>),
                       grid_for(sh, BM, 64 * kSkinnyNF, a.N), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
