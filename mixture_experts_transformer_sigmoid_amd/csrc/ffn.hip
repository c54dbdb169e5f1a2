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
// a pure weight stream from HBM straight into MFMA registers; "wide" for 128-row tiles
// (prefill), LDS-tiled with a three-deep register prefetch of the next k-chunks.
#include "common.h"

namespace moe {
namespace {

struct FfnArgs {
  const uint16_t* A;      // gate/up: x [T, K]; down: h [rows, K]
  const int32_t* perm;    // gate/up: slot id of each grouped row
  int64_t routed_rows;    // T*k: rows at or past this index belong to the shared expert
  const uint16_t* B1;     // routed weights [E, N, K] (w1, or w2 for down)
  const uint16_t* B3;     // routed w3 [E, N, K] (gate/up)
  const uint16_t* S1;     // shared weights [N, K] (ws1, or ws2 for down)
  const uint16_t* S3;     // shared ws3 (gate/up)
  uint16_t* C;            // gate/up: h [rows, N] bf16
  float* Y;               // down: y_routed [T*k, N] fp32
  float* Ys;              // down: y_shared [T, N] fp32
  const Tile* tiles;
  const int32_t* ntiles;
  int32_t k;              // slots per token (gate/up gather: token = slot / k)
  int32_t N, K, E;
};

// ------------------------------------------------------------------ tile list
__global__ __launch_bounds__(1024) void build_tiles_kernel(const int32_t* __restrict__ offsets,
                                                           int E, int64_t routed_rows,
                                                           int64_t shared_rows, int BM,
                                                           int64_t capacity,
                                                           Tile* __restrict__ tiles,
                                                           int32_t* __restrict__ ntiles) {
  __shared__ int32_t wsum[16];
  __shared__ int32_t routed_total;
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
  }
  __syncthreads();
  // never write past the list, whatever offsets the caller passed (overlapping
  // segments would otherwise multiply the tile count)
  const int64_t ns = (shared_rows + BM - 1) / BM;
  const int32_t R = (int32_t)min<int64_t>(routed_total, capacity - ns);
  const int32_t start = v + wsum[wave] - n;
  const int32_t cnt = max(0, min(n, R - start));
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
  for (int64_t j = tid; j < ns; j += 1024) {
    Tile t;
    t.group = E;
    t.row_begin = (int32_t)(routed_rows + j * BM);
    t.row_end = (int32_t)min<int64_t>(routed_rows + (j + 1) * BM, routed_rows + shared_rows);
    t.first = R;
    t.count = (int32_t)ns;
    t.pad[0] = t.pad[1] = t.pad[2] = 0;
    tiles[R + j] = t;
  }
  if (tid == 0) *ntiles = R + (int32_t)ns;
}

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

__device__ __forceinline__ void store_gateup(uint16_t* dst, f32x4_t g, f32x4_t u) {
  float v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = silu_f32(g[i]) * u[i];
  u32x2_t packed;
  packed[0] = f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
  packed[1] = f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16);
  *reinterpret_cast<u32x2_t*>(dst) = packed;
}

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
template <int NF, int KU, bool GATEUP>
__global__ __launch_bounds__(256) void ffn_skinny_kernel(const FfnArgs a) {
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
  if (GATEUP) {
    uint16_t* crow = a.C + p * N;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int nn = n0 + 16 * f + 4 * q;
      if (nn < N) store_gateup(crow + nn, acc1[f], acc3[f]);
    }
  } else {
    float* yrow = p < a.routed_rows ? a.Y + p * N : a.Ys + (p - a.routed_rows) * N;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int nn = n0 + 16 * f + 4 * q;
      if (nn < N) *reinterpret_cast<f32x4_t*>(yrow + nn) = acc1[f];
    }
  }
}

// --------------------------------------------------------------- wide GEMM
// 128-row tiles.  Four waves as 2 (rows) x 2 (features); each wave owns a 64-row x
// BN/2-feature block (per weight matrix).  K is walked in 64-wide chunks staged in LDS
// (row pitch 144 B: 16 B of padding make the MFMA operand reads and the chunk writes
// bank-conflict free).  Global loads for chunk kt+3 are issued while chunk kt is being
// multiplied, through a ring of three register sets, and chunk kt+1 is written to the
// other LDS buffer at the end of the step: one barrier per chunk.  16-row fragments
// past the tile's last row skip their MFMAs (a wave-uniform branch), so a 108-row
// expert costs 112 rows of MFMA work, not 128.
template <int BN, bool GATEUP>
__global__ __launch_bounds__(256, 2) void ffn_wide_kernel(const FfnArgs a) {
  constexpr int BM = 128, BK = 64;
  constexpr int PITCH = BK + 8;                       // bf16 elements per LDS row
  constexpr int WROWS = GATEUP ? 2 * BN : BN;         // weight rows staged per chunk
  constexpr int NCA = BM * 8 / 256;                   // 16-byte pieces per thread: acts
  constexpr int NCW = WROWS * 8 / 256;                // 16-byte pieces per thread: weights
  constexpr int NC = NCA + NCW;
  constexpr int STAGE = (BM + WROWS) * PITCH;         // bf16 elements per LDS stage
  constexpr int WM = BM / 2, WN = BN / 2, FM = WM / 16, FN = WN / 16;
  static_assert(NCA * 256 == BM * 8 && NCW * 256 == WROWS * 8, "tile / thread mismatch");
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * STAGE];

  Tile tile;
  int nb;
  if (!map_work(a, (a.N + BN - 1) / BN, tile, nb)) return;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, q = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const int K = a.K, N = a.N;
  const int n_base = nb * BN;
  const int nrows = tile.row_end - tile.row_begin;

  const bool is_shared = tile.group >= a.E;
  const int64_t wofs = (int64_t)tile.group * N * K;
  const uint16_t* W1 = is_shared ? a.S1 : a.B1 + wofs;
  const uint16_t* W3 = GATEUP ? (is_shared ? a.S3 : a.B3 + wofs) : nullptr;

  // this thread's 16-byte pieces of a stage: row (tid >> 3) + 32 i, chunk tid & 7
  const int prow = tid >> 3, pch = tid & 7;
  const uint16_t* src[NC];
  int dst[NC];
#pragma unroll
  for (int i = 0; i < NCA; ++i) {
    const int m = prow + 32 * i;
    int64_t p = tile.row_begin + m;
    if (p >= tile.row_end) p = tile.row_end - 1;
    src[i] = act_row(a, GATEUP, p) + pch * 8;
    dst[i] = m * PITCH + pch * 8;
  }
#pragma unroll
  for (int i = 0; i < NCW; ++i) {
    const int wr = prow + 32 * i;
    const bool second = GATEUP && wr >= BN;
    int n = n_base + (second ? wr - BN : wr);
    if (n > N - 1) n = N - 1;
    src[NCA + i] = (second ? W3 : W1) + (int64_t)n * K + pch * 8;
    dst[NCA + i] = (BM + wr) * PITCH + pch * 8;
  }

  f32x4_t acc1[FM][FN], acc3[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int f = 0; f < FN; ++f) {
      acc1[i][f] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      acc3[i][f] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  bool live[FM];
#pragma unroll
  for (int i = 0; i < FM; ++i) live[i] = wm * WM + 16 * i < nrows;

  const int nk = K / BK;
  u32x4_t R0[NC], R1[NC], R2[NC];

#define WIDE_ISSUE(R, kt)                                            \
  _Pragma("unroll") for (int c = 0; c < NC; ++c) R[c] = load16(src[c] + (int64_t)(kt) * BK);
#define WIDE_COMMIT(R, buf)                                          \
  _Pragma("unroll") for (int c = 0; c < NC; ++c)                    \
      *reinterpret_cast<u32x4_t*>(lds + (buf) * STAGE + dst[c]) = R[c];

  auto compute = [&](int buf) {
    const uint16_t* As = lds + buf * STAGE;
    const uint16_t* Ws = As + BM * PITCH;
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      u32x4_t af[FM], w1f[FN], w3f[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *reinterpret_cast<const u32x4_t*>(As + (wm * WM + 16 * i + r) * PITCH + ks * 32 + q * 8);
#pragma unroll
      for (int f = 0; f < FN; ++f) {
        w1f[f] = *reinterpret_cast<const u32x4_t*>(Ws + (wn * WN + 16 * f + r) * PITCH + ks * 32 + q * 8);
        if (GATEUP)
          w3f[f] = *reinterpret_cast<const u32x4_t*>(Ws + (BN + wn * WN + 16 * f + r) * PITCH + ks * 32 + q * 8);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        if (!live[i]) continue;
#pragma unroll
        for (int f = 0; f < FN; ++f) {
          acc1[i][f] = mfma16x16x32(w1f[f], af[i], acc1[i][f]);
          if (GATEUP) acc3[i][f] = mfma16x16x32(w3f[f], af[i], acc3[i][f]);
        }
      }
    }
  };

#define WIDE_STEP(kt, Rfree, Rnext)                                  \
  {                                                                  \
    if ((kt) + 3 < nk) { WIDE_ISSUE(Rfree, (kt) + 3) }               \
    compute((kt) & 1);                                               \
    if ((kt) + 1 < nk) { WIDE_COMMIT(Rnext, ((kt) + 1) & 1) }        \
    __syncthreads();                                                 \
  }

  WIDE_ISSUE(R0, 0)
  if (nk > 1) { WIDE_ISSUE(R1, 1) }
  if (nk > 2) { WIDE_ISSUE(R2, 2) }
  WIDE_COMMIT(R0, 0)
  __syncthreads();
  for (int kt = 0; kt < nk; kt += 3) {
    WIDE_STEP(kt, R0, R1)
    if (kt + 1 < nk) WIDE_STEP(kt + 1, R1, R2)
    if (kt + 2 < nk) WIDE_STEP(kt + 2, R2, R0)
  }
#undef WIDE_STEP
#undef WIDE_COMMIT
#undef WIDE_ISSUE

  // epilogue: fragment (i, f) of this lane = row wm*WM + 16 i + r, features
  // n_base + wn*WN + 16 f + 4 q .. +3
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int m = wm * WM + 16 * i + r;
    if (m >= nrows) continue;
    const int64_t p = tile.row_begin + m;
#pragma unroll
    for (int f = 0; f < FN; ++f) {
      const int nn = n_base + wn * WN + 16 * f + 4 * q;
      if (nn >= N) continue;
      if (GATEUP) {
        store_gateup(a.C + p * N + nn, acc1[i][f], acc3[i][f]);
      } else {
        float* yrow = p < a.routed_rows ? a.Y + p * N : a.Ys + (p - a.routed_rows) * N;
        *reinterpret_cast<f32x4_t*>(yrow + nn) = acc1[i][f];
      }
    }
  }
}

constexpr int kSkinnyBM = 16;
constexpr int kWideBM = 128;
constexpr int kSkinnyNF = 2;       // skinny: 4 waves x 2 fragments = 128 features per block
constexpr int kSkinnyKU = 8;       // skinny: k-steps (of 32) per batch of loads
constexpr int kWideBNGateUp = 64;  // wide: features per block (x2 weight matrices)
constexpr int kWideBNDown = 128;

int64_t max_tiles_for(const FfnShape& sh, int BM) {
  // sum_e ceil(c_e / BM) <= (T*k) / BM + E, plus the shared expert's ceil(T / BM)
  return sh.T * sh.k / BM + sh.E + (sh.shared ? (sh.T + BM - 1) / BM : 0) + 1;
}

// Average rows per routed expert decides the kernel: a few (decode) -> skinny stream;
// many (prefill) -> wide LDS-tiled kernel.
bool use_wide(const FfnShape& sh) { return sh.T * sh.k > (int64_t)16 * sh.E; }

hipError_t tiles_launch(const FfnShape& sh, const int32_t* offsets, int BM, Tile* tiles,
                        int32_t* ntiles, hipStream_t s) {
  hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(1024), 0, s, offsets, sh.E, sh.T * sh.k,
                     sh.shared ? sh.T : (int64_t)0, BM, max_tiles_for(sh, BM), tiles, ntiles);
  return hipGetLastError();
}

dim3 grid_for(const FfnShape& sh, int BM, int BN, int N) {
  const int64_t NB = (N + BN - 1) / BN;
  const int64_t total = max_tiles_for(sh, BM) * NB;
  return dim3((unsigned)((total + 7) / 8 * 8));
}

}  // namespace

int64_t ffn_max_tiles(const FfnShape& sh) { return max_tiles_for(sh, kSkinnyBM); }

hipError_t launch_gate_up(const FfnShape& sh, const uint16_t* x, const int32_t* perm,
                          const int32_t* offsets, const uint16_t* w1, const uint16_t* w3,
                          const uint16_t* ws1, const uint16_t* ws3, uint16_t* h, Tile* tiles,
                          int32_t* ntiles, hipStream_t s) {
  const bool wide = use_wide(sh);
  const int BM = wide ? kWideBM : kSkinnyBM;
  hipError_t err = tiles_launch(sh, offsets, BM, tiles, ntiles, s);
  if (err != hipSuccess) return err;
  FfnArgs a{};
  a.A = x;
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
    hipLaunchKernelGGL((ffn_wide_kernel<kWideBNGateUp, true>),
                       grid_for(sh, BM, kWideBNGateUp, a.N), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((ffn_skinny_kernel<kSkinnyNF, kSkinnyKU, true>),
                       grid_for(sh, BM, 64 * kSkinnyNF, a.N), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_down(const FfnShape& sh, const uint16_t* h, const int32_t* offsets,
                       const uint16_t* w2, const uint16_t* ws2, float* y_routed,
                       float* y_shared, Tile* tiles, int32_t* ntiles, hipStream_t s) {
  const bool wide = use_wide(sh);
  const int BM = wide ? kWideBM : kSkinnyBM;
  hipError_t err = tiles_launch(sh, offsets, BM, tiles, ntiles, s);
  if (err != hipSuccess) return err;
  FfnArgs a{};
  a.A = h;
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
    hipLaunchKernelGGL((ffn_wide_kernel<kWideBNDown, false>),
                       grid_for(sh, BM, kWideBNDown, a.N), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((ffn_skinny_kernel<kSkinnyNF, kSkinnyKU, false>),
                       grid_for(sh, BM, 64 * kSkinnyNF, a.N), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
