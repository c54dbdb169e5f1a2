// Device helpers and launcher declarations shared by the HIP sources of libmoe.
// gfx950 (CDNA4) only: wave64, MFMA bf16 16x16x32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kWave = 64;
constexpr int kMaxTopK = 8;
constexpr int kMaxExperts = 1024;

__device__ __forceinline__ float bf16_to_f32(uint32_t v) { return __uint_as_float(v << 16); }

// fp32 -> bf16, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ u32x4_t load16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// Raw buffer resource over [base, base + bytes): loads take a 32-bit per-lane byte offset
// and a wave-uniform byte offset, so the address costs one VGPR; reads past `bytes`
// return zeros instead of faulting.  Word 3 is the gfx9-family raw-buffer format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ u32x4_t bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                           uint32_t soff) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// C(16x16, fp32) += A(16x32) * B(32x16), bf16 operands.
// Lane l supplies row (l & 15) of A and column (l & 15) of B, each with the 8
// consecutive k values 8*(l >> 4) .. +7; it receives C rows 4*(l >> 4) .. +3 of column
// (l & 15).  Any k assignment works as long as A and B use the same one.
__device__ __forceinline__ f32x4_t mfma16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// C(32x32, fp32) += A(32x16) * B(16x32), bf16 operands.
// Lane l supplies row (l & 31) of A and column (l & 31) of B, each with the 8 consecutive
// k values 8*(l >> 5) .. +7; it receives column (l & 31) of C, rows
// 8*(j >> 2) + 4*(l >> 5) + (j & 3) in register j (four runs of 4 consecutive rows).
__device__ __forceinline__ f32x16_t mfma32x32x16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// 16 bytes per lane from a raw buffer straight into LDS: lane l's bytes land at
// lds + 16 l (the wave writes 1 KiB contiguous); `lds` must be wave-uniform.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff,
                                      uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, voff, soff, 0, 0);
}

// SwiGLU of one output, silu(g) u = g u / (1 + e^-g).  e^-g is 2^(-g log2 e) on the
// hardware exp2 and the quotient one hardware reciprocal, each within about an fp32 ulp:
// far inside the bf16 rounding that h gets next.  Large negative g: the exp2 overflows to
// inf, the reciprocal gives 0 and the result is 0, the limit; large positive g: g u.
__device__ __forceinline__ float swiglu_f32(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(g * -1.4426950408889634f);
  return (g * u) * __builtin_amdgcn_rcpf(1.0f + e);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two fp32 values -> packed bf16 (lo in bits 0..15) with the hardware conversion
// (v_cvt_pk_bf16_f32): round to nearest even, NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Expert output rows inside the layer: 24-bit floats, the upper three bytes of an fp32
// (its mantissa cut to 15 bits, rounding toward zero: 16 significant bits, fp32's exponent
// range).  Four consecutive values pack little-endian into 12 bytes, so a row of N (a
// multiple of 4) takes 3N bytes and each group of four starts on a 4-byte boundary (one
// dwordx3 access).  Packing is three byte permutes per four values.
struct __attribute__((aligned(4))) F24x4 {
  uint32_t w[3];
};

__device__ __forceinline__ F24x4 pack_f24x4(f32x4_t v) {
  const uint32_t a = __float_as_uint(v[0]), b = __float_as_uint(v[1]),
                 c = __float_as_uint(v[2]), d = __float_as_uint(v[3]);
  F24x4 r;
  // v_perm_b32: byte selector i picks byte i of {hi:lo} (0-3 lo, 4-7 hi)
  r.w[0] = __builtin_amdgcn_perm(b, a, 0x05030201u);  // a1 a2 a3 b1
  r.w[1] = __builtin_amdgcn_perm(c, b, 0x06050302u);  // b2 b3 c1 c2
  r.w[2] = __builtin_amdgcn_perm(d, c, 0x07060503u);  // c3 d1 d2 d3
  return r;
}

__device__ __forceinline__ f32x4_t unpack_f24x4(F24x4 r) {
  f32x4_t v;
  v[0] = __uint_as_float(r.w[0] << 8);
  v[1] = __uint_as_float(((r.w[0] >> 24) | (r.w[1] << 8)) << 8);
  v[2] = __uint_as_float(((r.w[1] >> 16) | (r.w[2] << 16)) << 8);
  v[3] = __uint_as_float(r.w[2] & 0xffffff00u);
  return v;
}

// Workgroup barrier for LDS hand-offs: waits for this wave's LDS operations, then meets
// the other waves.  Unlike __syncthreads() it does not drain the wave's outstanding
// global loads (on CDNA a release fence waits for vmcnt(0)), so register prefetches of
// later k-steps stay in flight across it.  Only for kernels whose waves share data
// through LDS alone.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace moe

// ---------------------------------------------------------------- launchers (host)
// Each returns hipSuccess or the launch error; arguments are pre-validated by moe_abi.
namespace moe {

struct Tile {
  int32_t group;      // expert index, or E for the shared expert
  int32_t row_begin;  // first row (grouped order; shared rows start at T*k)
  int32_t row_end;    // one past the last row
  int32_t first;      // index of the group's first tile in the list
  int32_t count;      // number of tiles of the group
  int32_t pad[3];
};

// How a grouped launch cuts its groups into row tiles; passed by value to the kernels that
// build the list.
struct TileSpec {
  int32_t E;            // routed groups, rows given by the offsets
  int32_t BM;           // rows per tile
  int32_t parts;        // the shared expert's tiles are cut into this many parts
  int64_t routed_rows;  // T*k
  int64_t shared_rows;  // T with a shared expert, else 0
  int64_t capacity;     // entries the list has room for
};

// Router.  Up to kRouterSmallT tokens, one kernel computes each (16 tokens x 16 experts)
// tile of z over the whole K with the sigmoid and the bias in its epilogue, and takes each
// token's top-k and gates: from LDS with at most 16 experts, else from the biased scores
// and the sigmoids, [T, E] fp32 each (router_zpart_floats holds both), in the last
// workgroup of each token block to finish.  Above kRouterSmallT, the bf16 (hi, mid,
// lo) copy of W_r (w_split, [3 router_part_rows(E), d]) feeds the 256-row GEMM kernel,
// whose partial logits (z_part) the selection kernel adds in fp64.  logits may be null.
constexpr int64_t kRouterSmallT = 512;
// Rows per part (hi, mid, lo) of the split router weights and of the partial logits the
// 256-row kernel writes: E rounded up to a multiple of 4 (the padding rows are zero).
inline int router_part_rows(int E) { return (E + 3) / 4 * 4; }
// Above kRouterSmallT tokens the logits GEMM runs on the 256-row kernel, one workgroup per
// 256 tokens x 256 outputs: 160 workgroups at 8,192 tokens and E = 384, 80 at 4,096, for
// 256 CUs.  K is then cut into S slices, each writing its own partial logits, with S the
// smallest that minimises (rounds of workgroups) / S + S / 20: the second term stands
// for each slice's fixed cost (its pipeline fill and its partial output).  S = 3 for
// 8,192 and 4,096 tokens at K2 width.
inline int router_ksplit(int64_t T, int E, int d) {
  if (T <= kRouterSmallT) return 1;
  const int64_t wgs = ((T + 255) / 256) * ((3 * (int64_t)router_part_rows(E) + 255) / 256);
  const int chunks = d / 64;
  int best = 1;
  double best_cost = 1e30;
  for (int sl = 1; sl <= 8 && sl <= chunks; ++sl) {
    const double rounds = (double)((wgs * sl + 255) / 256);
    const double cost = rounds / sl + sl / 20.0;
    if (cost < best_cost - 1e-12) {
      best_cost = cost;
      best = sl;
    }
  }
  return best;
}
inline int64_t router_zpart_floats(int64_t T, int E, int d) {
  return T <= kRouterSmallT ? 2 * T * E
                            : T * 3 * router_part_rows(E) * router_ksplit(T, E, d);
}

// The pre-MoE RMSNorm done inside the small-batch router's pass over the residual stream:
// x_ffn[t] = bf16(x'[t] / sqrt(mean(x'[t]^2) + eps) * gain), written to x_ffn.
struct RouterNorm {
  const float* gain;
  float eps;
  uint16_t* x_ffn;
};

// The routing up to kRouterSmallT tokens, one launch: the scores (score = fl32(sigmoid(z) +
// b), NaN -> -inf; above 16 experts score and sig, [T, E] fp32 each, carry them from the
// workgroups of a token block to its last one), then the top-k into idx and the gates into
// w.  ws identifies the call's workspace: the launch counts arrivals in that workspace's
// slot of the library's counters.  With norm non-null, x is the residual stream and the
// router reads its normalised rows (and writes them to norm->x_ffn).
hipError_t launch_router_small(const uint16_t* x, const RouterNorm* norm, const float* w_r,
                               const float* bias, int64_t T, int d, int E, int k, float alpha,
                               float* score, float* sig, float* logits, int32_t* idx, float* w,
                               const void* ws, hipStream_t s);

// The whole routing: launch_router_small up to kRouterSmallT tokens, else the split, GEMM
// and selection launches.
hipError_t launch_router(const uint16_t* x, const float* w_r, const float* bias, int64_t T, int d,
                         int E, int k, float alpha, uint16_t* w_split, float* z_part,
                         Tile* tiles, int32_t* ntiles, float* logits, int32_t* topk_idx,
                         float* topk_w, const void* ws, hipStream_t s);


// ts (or null): also build the tile list of a grouped launch for the new offsets into
// tiles / ntiles, so that the launch can skip building it.
hipError_t launch_permute(const int32_t* topk_idx, int64_t T, int E, int k, int32_t* hist,
                          int32_t* base, int32_t* counts, int32_t* offsets, int32_t* perm,
                          int32_t* inv, hipStream_t s, const TileSpec* ts = nullptr,
                          Tile* tiles = nullptr, int32_t* ntiles = nullptr);
int64_t permute_blocks(int64_t T);

struct FfnShape {
  int64_t T;    // tokens
  int d;        // model width
  int E;        // routed experts
  int k;        // slots per token
  int I;        // expert intermediate width
  bool shared;  // shared expert present (Is == I)
  // h in two bf16 parts (hi = bf16(h), lo = bf16(h - hi)), rows [hi | lo] of 2I: the down
  // GEMM then runs over K = 2I with each weight used twice (bf16 kernels only)
  bool hsplit = false;
};

// The two-part form of h is used when a token has at most this many slots: with so few
// gate-weighted expert rows in a token's sum, the bf16 rounding of h alone takes most of
// the output's error budget.
constexpr int kHsplitMaxTopK = MOE_HSPLIT_MAX_TOP_K;

int64_t ffn_max_tiles(const FfnShape& sh);
// The tiles of the bf16 and of the FP8 gate/up and down launches at this shape (both
// projections use the same list).
TileSpec ffn_tile_spec(const FfnShape& sh);
TileSpec ffn_tile_spec_fp8(const FfnShape& sh);

// Dense C[rows, N] = A[rows, K] . W[N, K]^T with the grouped-GEMM kernels (one group):
// fp32 into Cf; bf16 into Cb; or bf16(C + R) into Cb with R [rows, N] fp32.
// ksplit > 1 (fp32 output, more than 512 rows only): K is cut into ksplit slices of whole
// 64-k chunks, and slice j writes its partial product to columns j N .. j N + N - 1 of
// Cf [rows, ksplit N].
enum class DenseOut { kF32, kBF16, kAddBF16 };
// wk > 0: A is in two bf16 parts, rows [hi | lo] of K = 2 wk, and W is [N, wk] (no K
// slices then).
hipError_t launch_dense(const uint16_t* A, int64_t rows, int K, const uint16_t* W, int N,
                        DenseOut mode, float* Cf, uint16_t* Cb, const float* R, Tile* tiles,
                        int32_t* ntiles, hipStream_t s, int ksplit = 1, int wk = 0);

hipError_t launch_gate_up(const FfnShape& sh, const uint16_t* x, const int32_t* perm,
                          const int32_t* offsets, const uint16_t* w1, const uint16_t* w3,
                          const uint16_t* ws1, const uint16_t* ws3, uint16_t* h, Tile* tiles,
                          int32_t* ntiles, hipStream_t s, bool tiles_ready = false);

// tiles_ready: the tile list already holds this shape's tiles for the same offsets (built
// by the permutation or by the gate/up launch just before), so the launch skips building it.
// y24: y_routed / y_shared hold rows of packed 24-bit floats (3 d bytes each, F24x4 groups)
// instead of fp32 rows.
hipError_t launch_down(const FfnShape& sh, const uint16_t* h, const int32_t* offsets,
                       const uint16_t* w2, const uint16_t* ws2, void* y_routed, void* y_shared,
                       Tile* tiles, int32_t* ntiles, hipStream_t s, bool tiles_ready = false,
                       bool y24 = false);

// FP8 (E4M3) expert weights with one fp32 scale per 128 x 128 block; device pointers.
struct Fp8Weights {
  const uint8_t* w1;       // [E, I, d]
  const uint8_t* w3;       // [E, I, d]
  const uint8_t* w2;       // [E, d, I]
  const float* w1_scale;   // [E, I/128, d/128]
  const float* w3_scale;   // [E, I/128, d/128]
  const float* w2_scale;   // [E, d/128, I/128]
  const uint8_t* ws1;      // [Is, d]   (shared expert; null without one)
  const uint8_t* ws3;      // [Is, d]
  const uint8_t* ws2;      // [d, Is]
  const float* ws1_scale;  // [Is/128, d/128]
  const float* ws3_scale;  // [Is/128, d/128]
  const float* ws2_scale;  // [d/128, Is/128]
};
constexpr int kFp8Block = 128;
constexpr int kFp8MaxK = 16384;  // the FP8 kernels keep a row of K/128 scales in LDS

hipError_t launch_gate_up_fp8(const FfnShape& sh, const uint16_t* x, const int32_t* perm,
                              const int32_t* offsets, const Fp8Weights& w, uint16_t* h,
                              Tile* tiles, int32_t* ntiles, hipStream_t s,
                              bool tiles_ready = false);

hipError_t launch_down_fp8(const FfnShape& sh, const uint16_t* h, const int32_t* offsets,
                           const Fp8Weights& w, void* y_routed, void* y_shared, Tile* tiles,
                           int32_t* ntiles, hipStream_t s, bool tiles_ready = false,
                           bool y24 = false);

// residual (bf16 [T, d]) may be null; when given it is added before the bf16 rounding.
// y24: the expert rows are packed 24-bit floats (as launch_down writes them with y24).
hipError_t launch_combine(const void* y_routed, const int32_t* inv, const float* topk_w,
                          const void* y_shared, const uint16_t* residual, uint16_t* out,
                          int64_t T, int d, int k, hipStream_t s, bool y24 = false);

// out[t] = bf16(x[t] / sqrt(mean(x[t]^2) + eps) * gain), fp64 arithmetic.
hipError_t launch_rmsnorm(const uint16_t* x, const float* gain, uint16_t* out, int64_t T, int d,
                          float eps, hipStream_t s);

// u = RMSNorm(sum_slot topk_w * y_routed[inv]) over L features (L <= 8192): out[t] =
// bf16(u) (rows of L), or with two_part [bf16(u) | bf16(u - bf16(u))] (rows of 2L).
// y_routed rows are packed 24-bit floats (3 L bytes each), as launch_down writes them with y24.
hipError_t launch_combine_rmsnorm(const void* y_routed, const int32_t* inv, const float* topk_w,
                                  uint16_t* out, int64_t T, int L, int k, float eps,
                                  bool two_part, hipStream_t s);
constexpr int kMaxLatent = 8192;
// The latent variant feeds its normalised row to the up-projection in two bf16 parts up to
// this latent width.  Narrow latents sum few terms per output, and one rounding of the row
// then takes a visible share of the error bar (L = 128-256: 2.2-2.3% of RMS with one part,
// 1.9% with two); at L = 3584 the error is the same either way and the second part would
// cost 170 us of up-projection at 4,096 tokens.
constexpr int kLatentTwoPartMaxL = 1024;

}  // namespace moe
