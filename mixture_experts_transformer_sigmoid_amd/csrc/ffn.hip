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
// Block -> tile mapping is XCD-aware: the hardware deals workgroups round-robin to the
// 8 XCDs, so workgroup b takes logical tile (b % 8) * ceil(total / 8) + b / 8 and each
// XCD gets one contiguous run of logical tiles — an expert's n-blocks (which share its
// activation rows) and its row tiles (which share weight tiles) stay in one L2.
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
  uint16_t* C;            // gate/up: h [rows, N]; down: y_routed [T*k, N]
  uint16_t* Cs;           // down: y_shared [T, N]
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
  for (int j = 0; j < n && start + j < R; ++j) {
    Tile t;
    t.group = tid;
    t.row_begin = o0 + j * BM;
    t.row_end = min(o0 + (j + 1) * BM, o1);
    t.pad = 0;
    tiles[start + j] = t;
  }
  for (int64_t j = tid; j < ns; j += 1024) {
    Tile t;
    t.group = E;
    t.row_begin = (int32_t)(routed_rows + j * BM);
    t.row_end = (int32_t)min<int64_t>(routed_rows + (j + 1) * BM, routed_rows + shared_rows);
    t.pad = 0;
    tiles[R + j] = t;
  }
  if (tid == 0) *ntiles = R + (int32_t)ns;
}

// ------------------------------------------------------------- skinny GEMM
// For row tiles of at most 16 rows (decode: a few tokens per expert).  The kernel is a
// weight stream: each wave owns NF 16-row strips of the weight matrix (two strips, W1
// and W3, per fragment for gate/up) and runs them against the tile's <= 16 activation
// rows over the whole K.  Weights go straight from HBM to registers in the MFMA
// operand layout — each lane reads 16 contiguous bytes, four lanes cover 64 contiguous
// bytes of a weight row — KU k-steps per batch of loads so that a wave keeps
// KU * NF * (2 or 1) KiB in flight.  Activation rows come from L2 (every n-block of
// the expert reads the same few rows).
//
// The MFMA computes C^T = W . A^T: weights as the A operand (16 output features),
// activations as the B operand (16 rows), so a lane ends up with four consecutive
// output features of one row and stores them as one 8-byte write.
template <int NF, int KU, bool GATEUP>
__global__ __launch_bounds__(256) void ffn_skinny_kernel(const FfnArgs a) {
  constexpr int BN = 4 * 16 * NF;
  const int32_t nt = *a.ntiles;
  const int NB = (a.N + BN - 1) / BN;
  const int64_t total = (int64_t)nt * NB;
  const int64_t per = (total + 7) / 8;
  const int64_t b = blockIdx.x;
  if (b >= 8 * per) return;
  const int64_t L = (b & 7) * per + (b >> 3);
  if (L >= total) return;
  const int rt = (int)(L / NB), nb = (int)(L % NB);
  const Tile tile = a.tiles[rt];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, q = lane >> 4;
  const int K = a.K, N = a.N;

  int64_t p = tile.row_begin + r;
  const bool row_ok = p < tile.row_end;
  if (!row_ok) p = tile.row_end - 1;
  const uint16_t* arow;
  if (GATEUP) {
    int64_t tok;
    if (p < a.routed_rows) {
      int64_t sl = a.perm[p];
      if (sl < 0 || sl >= a.routed_rows) sl = 0;
      tok = sl / a.k;
    } else {
      tok = p - a.routed_rows;
    }
    arow = a.A + tok * K;
  } else {
    arow = a.A + p * K;
  }
  arow += q * 8;

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
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int u = 0; u < KU; ++u) {
        b1v[f][u] = load16(w1p[f] + k0 + 32 * u);
        if (GATEUP) b3v[f][u] = load16(w3p[f] + k0 + 32 * u);
      }
#pragma unroll
    for (int u = 0; u < KU; ++u) av[u] = load16(arow + k0 + 32 * u);
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
  uint16_t* crow;
  if (GATEUP || p < a.routed_rows)
    crow = a.C + p * N;
  else
    crow = a.Cs + (p - a.routed_rows) * N;
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int nn = n0 + 16 * f + 4 * q;
    if (nn >= N) continue;
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = GATEUP ? silu_f32(acc1[f][i]) * acc3[f][i] : acc1[f][i];
    u32x2_t packed;
    packed[0] = f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
    packed[1] = f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16);
    *reinterpret_cast<u32x2_t*>(crow + nn) = packed;
  }
}

constexpr int kSkinnyBM = 16;

int64_t max_tiles_for(const FfnShape& sh, int BM) {
  // sum_e ceil(c_e / BM) <= (T*k) / BM + E, plus the shared expert's ceil(T / BM)
  return sh.T * sh.k / BM + sh.E + (sh.shared ? (sh.T + BM - 1) / BM : 0) + 1;
}

hipError_t tiles_launch(const FfnShape& sh, const int32_t* offsets, int BM, Tile* tiles,
                        int32_t* ntiles, hipStream_t s) {
  hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(1024), 0, s, offsets, sh.E, sh.T * sh.k,
                     sh.shared ? sh.T : (int64_t)0, BM, max_tiles_for(sh, BM), tiles, ntiles);
  return hipGetLastError();
}


template <int NF, int KU, bool GATEUP>
hipError_t skinny_launch(const FfnArgs& a, const FfnShape& sh, hipStream_t s) {
  constexpr int BN = 4 * 16 * NF;
  const int64_t NB = (a.N + BN - 1) / BN;
  const int64_t total = max_tiles_for(sh, kSkinnyBM) * NB;
  const int64_t grid = (total + 7) / 8 * 8;
  hipLaunchKernelGGL((ffn_skinny_kernel<NF, KU, GATEUP>), dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int64_t ffn_max_tiles(const FfnShape& sh) { return max_tiles_for(sh, kSkinnyBM); }

hipError_t launch_gate_up(const FfnShape& sh, const uint16_t* x, const int32_t* perm,
                          const int32_t* offsets, const uint16_t* w1, const uint16_t* w3,
                          const uint16_t* ws1, const uint16_t* ws3, uint16_t* h, Tile* tiles,
                          int32_t* ntiles, hipStream_t s) {
  hipError_t err = tiles_launch(sh, offsets, kSkinnyBM, tiles, ntiles, s);
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
  a.Cs = nullptr;
  a.tiles = tiles;
  a.ntiles = ntiles;
  a.k = sh.k;
  a.N = sh.I;
  a.K = sh.d;
  a.E = sh.E;
  return skinny_launch<2, 8, true>(a, sh, s);
}

hipError_t launch_down(const FfnShape& sh, const uint16_t* h, const int32_t* offsets,
                       const uint16_t* w2, const uint16_t* ws2, uint16_t* y_routed,
                       uint16_t* y_shared, Tile* tiles, int32_t* ntiles, hipStream_t s) {
  hipError_t err = tiles_launch(sh, offsets, kSkinnyBM, tiles, ntiles, s);
  if (err != hipSuccess) return err;
  FfnArgs a{};
  a.A = h;
  a.perm = nullptr;
  a.routed_rows = sh.T * sh.k;
  a.B1 = w2;
  a.B3 = nullptr;
  a.S1 = ws2;
  a.S3 = nullptr;
  a.C = y_routed;
  a.Cs = y_shared;
  a.tiles = tiles;
  a.ntiles = ntiles;
  a.k = sh.k;
  a.N = sh.d;
  a.K = sh.I;
  a.E = sh.E;
  return skinny_launch<2, 8, false>(a, sh, s);
}

}  // namespace moe
