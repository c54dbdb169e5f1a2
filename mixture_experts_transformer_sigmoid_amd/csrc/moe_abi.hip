// C ABI of libmoe: argument checks, workspace layout and the launch sequence.
// Every check runs on the host before the first launch; nothing here synchronises.
#include <math.h>

#include <mutex>

#include "../../include/moe.h"
#include "arrival_slots.h"
#include "common.h"

// Fixed device scratch of moe_forward_noalloc: each GPU the library runs on holds its own
// copy from the module's load until the process ends.  Host code never passes this name to
// a kernel or a copy: the name is a host-side stand-in, and its device address comes from
// hipGetSymbolAddress (noalloc_scratch below).
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

using moe::FfnShape;
using moe::Tile;

constexpr size_t kWsAlign = 256;

size_t align_up(size_t v) { return (v + kWsAlign - 1) / kWsAlign * kWsAlign; }

bool aligned(const void* p, size_t a) { return p != nullptr && ((uintptr_t)p % a) == 0; }

bool has_shared(const moe_dims& d) { return d.d_shared > 0; }

constexpr uint64_t kMaxBuffer = (uint64_t)1 << 31;

// An [N, K] bf16 weight matrix the GEMM kernels can address (with 256 rows of slack).
bool matrix_ok(int64_t N, int64_t K) { return (uint64_t)(N + 256) * K * 2 < kMaxBuffer; }

moe_status check_dims(const moe_dims* dp) {
  if (dp == nullptr) return MOE_EINVAL;
  const moe_dims& d = *dp;
  if (d.tokens < 0 || d.d_model <= 0 || d.n_experts <= 0 || d.top_k <= 0 || d.d_expert <= 0 ||
      d.d_shared < 0)
    return MOE_EINVAL;
  if (d.top_k > d.n_experts) return MOE_EINVAL;
  if (!isfinite(d.routed_scale)) return MOE_EINVAL;
  if (d.top_k > moe::kMaxTopK || d.n_experts > moe::kMaxExperts) return MOE_EUNSUPPORTED;
  if (d.d_model % 64 != 0 || d.d_expert % 64 != 0) return MOE_EUNSUPPORTED;
  if (d.d_shared != 0 && d.d_shared != d.d_expert) return MOE_EUNSUPPORTED;
  // grouped rows (T*k routed + T shared) are indexed with int32
  if (d.tokens > (int64_t)(INT32_MAX / 2) / (d.top_k + 1)) return MOE_EUNSUPPORTED;
  // per-token launches (combine, norm) must stay below 2^32 work-items per grid
  if (d.tokens > ((int64_t)1 << 23)) return MOE_EUNSUPPORTED;
  // the GEMM kernels address x, one expert's weight matrix and the split router matrix
  // through 32-bit byte offsets, and the wide kernel adds a buffer's size to an offset
  // (up to 256 rows past the matrix) to make a load read nothing: each stays below 2 GiB
  if ((uint64_t)d.tokens * d.d_model * 2 >= kMaxBuffer) return MOE_EUNSUPPORTED;
  if (!matrix_ok(d.d_expert, d.d_model) || !matrix_ok(d.d_model, d.d_expert))
    return MOE_EUNSUPPORTED;
  if (!matrix_ok(3 * moe::router_part_rows(d.n_experts), d.d_model)) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

// The bf16 (hi, mid, lo) copy of the router matrix, used only above kRouterSmallT tokens
// (the small-batch router splits W_r in registers).
size_t router_wsplit_bytes(const moe_dims& d) {
  if (d.tokens <= moe::kRouterSmallT) return 0;
  return 3 * (size_t)moe::router_part_rows(d.n_experts) * d.d_model * 2;
}

bool hsplit(const moe_dims& d) {
  return d.top_k <= moe::kHsplitMaxTopK || d.d_expert <= MOE_HSPLIT_MAX_D_EXPERT;
}

// Columns of h per row: I, or 2I when h is kept in two bf16 parts (bf16 weights, few slots
// per token or narrow experts).
size_t h_width(const moe_dims& d) { return (hsplit(d) ? 2 : 1) * (size_t)d.d_expert; }

struct Layout {
  size_t zpart, wsplit, idx, w, counts, offsets, perm, inv, hist, base, tiles, ntiles, h, y,
      total;
};

Layout layout(const moe_dims& d) {
  const size_t T = (size_t)d.tokens, E = (size_t)d.n_experts, k = (size_t)d.top_k;
  const size_t slots = T * k;
  const size_t rows = slots + (has_shared(d) ? T : 0);
  const size_t nb = (size_t)moe::permute_blocks(d.tokens);
  FfnShape sh{d.tokens, d.d_model, d.n_experts, d.top_k, d.d_expert, has_shared(d)};
  const size_t max_tiles = (size_t)moe::ffn_max_tiles(sh);
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align_up(bytes);
    return o;
  };
  // the routing and the permutation first, in the order the header documents
  L.idx = take(slots * 4);
  L.w = take(slots * 4);
  L.counts = take(E * 4);
  L.offsets = take((E + 1) * 4);
  L.perm = take(slots * 4);
  L.inv = take(slots * 4);
  L.zpart = take((size_t)moe::router_zpart_floats(d.tokens, d.n_experts, d.d_model) * 4);
  L.wsplit = take(router_wsplit_bytes(d));
  L.hist = take(nb * E * 4);
  L.base = take(nb * E * 4);
  L.tiles = take(max_tiles * sizeof(Tile));
  L.ntiles = take(4);
  L.h = take(rows * h_width(d) * 2);
  // the layer's expert outputs, routed rows then the shared expert's, as packed 24-bit
  // floats (3 bytes per value)
  L.y = take(rows * (size_t)d.d_model * 3);
  L.total = off;
  return L;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

moe_status check_ws(const moe_dims& d, const void* ws, size_t ws_bytes) {
  if (!aligned(ws, kWsAlign)) return MOE_EINVAL;
  if (ws_bytes < layout(d).total) return MOE_EWORKSPACE;
  return MOE_OK;
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

FfnShape ffn_shape(const moe_dims& d) {
  return FfnShape{d.tokens, d.d_model, d.n_experts, d.top_k, d.d_expert, has_shared(d),
                  hsplit(d)};
}

// The FP8 kernels keep h in one bf16 part.
FfnShape ffn_shape_fp8(const moe_dims& d) {
  return FfnShape{d.tokens, d.d_model, d.n_experts, d.top_k, d.d_expert, has_shared(d), false};
}

#define MOE_TRY(expr)                 \
  do {                                \
    const moe_status st_ = (expr);    \
    if (st_ != MOE_OK) return st_;    \
  } while (0)

#define MOE_NEED(cond)                  \
  do {                                  \
    if (!(cond)) return MOE_EINVAL;     \
  } while (0)

moe_status route_impl(const moe_dims& d, const uint16_t* x, const float* w_r, const float* b,
                      int32_t* idx, float* w, float* logits, void* ws, hipStream_t s) {
  const Layout L = layout(d);
  return hip_status(moe::launch_router(x, w_r, b, d.tokens, d.d_model, d.n_experts, d.top_k,
                                       d.routed_scale, at<uint16_t>(ws, L.wsplit),
                                       at<float>(ws, L.zpart), at<Tile>(ws, L.tiles),
                                       at<int32_t>(ws, L.ntiles), logits, idx, w, ws, s));
}

// ts (or null): the permutation also builds this tile list in the workspace, for the
// grouped launches that follow on the same offsets
moe_status permute_impl(const moe_dims& d, const int32_t* idx, int32_t* counts, int32_t* offsets,
                        int32_t* perm, int32_t* inv, void* ws, hipStream_t s,
                        const moe::TileSpec* ts = nullptr) {
  const Layout L = layout(d);
  return hip_status(moe::launch_permute(idx, d.tokens, d.n_experts, d.top_k,
                                        at<int32_t>(ws, L.hist), at<int32_t>(ws, L.base), counts,
                                        offsets, perm, inv, s, ts, at<Tile>(ws, L.tiles),
                                        at<int32_t>(ws, L.ntiles)));
}

// tiles_ready: the workspace already holds this launch's tile list for these offsets
// (built by the permutation, or by the gate/up launch just before; both GEMMs share it)
moe_status gate_up_impl(const moe_dims& d, const uint16_t* x, const int32_t* perm,
                        const int32_t* offsets, const uint16_t* w1, const uint16_t* w3,
                        const uint16_t* ws1, const uint16_t* ws3, uint16_t* h, void* ws,
                        hipStream_t s, bool tiles_ready = false) {
  const Layout L = layout(d);
  return hip_status(moe::launch_gate_up(ffn_shape(d), x, perm, offsets, w1, w3, ws1, ws3, h,
                                        at<Tile>(ws, L.tiles), at<int32_t>(ws, L.ntiles), s,
                                        tiles_ready));
}

// y24: y_routed / y_shared are the layer's packed 24-bit rows (the workspace's y region),
// else the caller's fp32 rows.
moe_status down_impl(const moe_dims& d, const uint16_t* h, const int32_t* offsets,
                     const uint16_t* w2, const uint16_t* ws2, void* y_routed, void* y_shared,
                     void* ws, hipStream_t s, bool tiles_ready = false, bool y24 = false) {
  const Layout L = layout(d);
  return hip_status(moe::launch_down(ffn_shape(d), h, offsets, w2, ws2, y_routed, y_shared,
                                     at<Tile>(ws, L.tiles), at<int32_t>(ws, L.ntiles), s,
                                     tiles_ready, y24));
}

moe_status combine_impl(const moe_dims& d, const void* y_routed, const int32_t* inv,
                        const float* w, const void* y_shared, uint16_t* out, hipStream_t s,
                        bool y24 = false) {
  return hip_status(moe::launch_combine(y_routed, inv, w, y_shared, nullptr, out, d.tokens,
                                        d.d_model, d.top_k, s, y24));
}

bool shared_ptrs_ok(const moe_dims& d, const void* a, const void* b) {
  return has_shared(d) ? (aligned(a, 16) && aligned(b, 16)) : true;
}

// ------------------------------------------------------------------- latent variant
moe_status check_latent(const moe_dims* dims, int32_t L) {
  MOE_TRY(check_dims(dims));
  if (L <= 0) return MOE_EINVAL;
  if (L % 64 != 0 || L > moe::kMaxLatent) return MOE_EUNSUPPORTED;
  // the same 2 GiB bound as check_dims, for the latent rows, the experts on width L and
  // both projections
  if ((uint64_t)dims->tokens * L * 2 >= kMaxBuffer) return MOE_EUNSUPPORTED;
  if (!matrix_ok(dims->d_expert, L) || !matrix_ok(L, dims->d_expert)) return MOE_EUNSUPPORTED;
  if (!matrix_ok(L, dims->d_model) || !matrix_ok(dims->d_model, L)) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

struct LatentLayout {
  size_t zpart, wsplit, idx, w, counts, offsets, perm, inv, hist, base, tiles, ntiles, lat, h, hs,
      y, uhat, ys, total;
};

LatentLayout latent_layout(const moe_dims& d, int32_t L) {
  const size_t T = (size_t)d.tokens, E = (size_t)d.n_experts, k = (size_t)d.top_k;
  const size_t slots = T * k;
  const size_t nb = (size_t)moe::permute_blocks(d.tokens);
  // the largest tile list of the launches below: routed experts plus a T-row group
  FfnShape sh{d.tokens, L, d.n_experts, d.top_k, d.d_expert, true};
  const size_t max_tiles = (size_t)moe::ffn_max_tiles(sh);
  LatentLayout P{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align_up(bytes);
    return o;
  };
  // the routing and the permutation first, in the order the header documents
  P.idx = take(slots * 4);
  P.w = take(slots * 4);
  P.counts = take(E * 4);
  P.offsets = take((E + 1) * 4);
  P.perm = take(slots * 4);
  P.inv = take(slots * 4);
  P.zpart = take((size_t)moe::router_zpart_floats(d.tokens, d.n_experts, d.d_model) * 4);
  P.wsplit = take(router_wsplit_bytes(d));
  P.hist = take(nb * E * 4);
  P.base = take(nb * E * 4);
  P.tiles = take(max_tiles * sizeof(Tile));
  P.ntiles = take(4);
  P.lat = take(T * (size_t)L * 2);
  P.h = take(slots * h_width(d) * 2);
  P.hs = take(has_shared(d) ? T * h_width(d) * 2 : 0);
  P.y = take(slots * (size_t)L * 3);  // the routed experts' rows, packed 24-bit floats
  P.uhat = take(T * (size_t)L * 2 * (L <= moe::kLatentTwoPartMaxL ? 2 : 1));  // one or two parts
  P.ys = take(has_shared(d) ? T * (size_t)d.d_model * 4 : 0);
  P.total = off;
  return P;
}

// Routing and permutation of a layer entry point, into the workspace arrays at the given
// offsets (and the tile list of ts when ts is non-null).  Up to kRouterSmallT tokens one
// router kernel computes the scores and takes the top-k and the gates.  With norm non-null, x is the residual stream x' and the experts'
// input x_ffn = RMSNorm(x') goes to norm->x_ffn: written by the router kernel up to
// kRouterSmallT tokens, else by the norm kernel before the router.  The experts' input (x,
// or norm->x_ffn) is returned through x_in.
struct RouteBufs {
  size_t zpart, wsplit, idx, w, counts, offsets, perm, inv, hist, base, tiles, ntiles;
};

template <typename LayoutT>
RouteBufs route_bufs(const LayoutT& L) {
  return RouteBufs{L.zpart, L.wsplit, L.idx, L.w, L.counts, L.offsets,
                   L.perm,  L.inv,    L.hist, L.base, L.tiles, L.ntiles};
}

moe_status route_permute(const moe_dims& d, const uint16_t* x, const moe::RouterNorm* norm,
                         const float* w_router, const float* bias, void* ws, const RouteBufs& B,
                         const moe::TileSpec* ts, hipStream_t s, const uint16_t** x_in) {
  const int64_t T = d.tokens;
  const int E = d.n_experts;
  int32_t* idx = at<int32_t>(ws, B.idx);
  float* w = at<float>(ws, B.w);
  moe::Tile* tiles = at<Tile>(ws, B.tiles);
  int32_t* ntiles = at<int32_t>(ws, B.ntiles);
  int32_t* hist = at<int32_t>(ws, B.hist);
  int32_t* base = at<int32_t>(ws, B.base);
  int32_t* counts = at<int32_t>(ws, B.counts);
  int32_t* offsets = at<int32_t>(ws, B.offsets);
  int32_t* perm = at<int32_t>(ws, B.perm);
  int32_t* inv = at<int32_t>(ws, B.inv);
  if (T <= moe::kRouterSmallT) {
    float* score = at<float>(ws, B.zpart);
    MOE_TRY(hip_status(moe::launch_router_small(x, norm, w_router, bias, T, d.d_model, E, d.top_k,
                                                d.routed_scale, score, score + T * E, nullptr,
                                                idx, w, ws, s)));
    *x_in = norm != nullptr ? norm->x_ffn : x;
    return hip_status(moe::launch_permute(idx, T, E, d.top_k, hist, base, counts, offsets, perm,
                                          inv, s, ts, tiles, ntiles));
  }
  if (norm != nullptr) {
    MOE_TRY(hip_status(
        moe::launch_rmsnorm(x, norm->gain, norm->x_ffn, T, d.d_model, norm->eps, s)));
    x = norm->x_ffn;
  }
  *x_in = x;
  MOE_TRY(hip_status(moe::launch_router(x, w_router, bias, T, d.d_model, E, d.top_k,
                                        d.routed_scale, at<uint16_t>(ws, B.wsplit),
                                        at<float>(ws, B.zpart), tiles, ntiles, nullptr, idx, w,
                                        ws, s)));
  return hip_status(moe::launch_permute(idx, T, E, d.top_k, hist, base, counts, offsets, perm,
                                        inv, s, ts, tiles, ntiles));
}

// The layer; with norm non-null, x is the residual stream and the layer runs on its
// RMSNorm (moe_forward_block).  residual (or null) is added to the output before its
// rounding.  Arguments checked by the callers.
moe_status forward_impl(const moe_dims& d, const uint16_t* x, const moe::RouterNorm* norm,
                        const float* w_router, const float* bias, const uint16_t* w1,
                        const uint16_t* w3, const uint16_t* w2, const uint16_t* ws1,
                        const uint16_t* ws3, const uint16_t* ws2, const uint16_t* residual,
                        uint16_t* out, void* ws, hipStream_t s) {
  const Layout L = layout(d);
  float* w = at<float>(ws, L.w);
  int32_t* offsets = at<int32_t>(ws, L.offsets);
  int32_t* perm = at<int32_t>(ws, L.perm);
  int32_t* inv = at<int32_t>(ws, L.inv);
  uint16_t* h = at<uint16_t>(ws, L.h);
  uint8_t* y_routed = at<uint8_t>(ws, L.y);
  uint8_t* y_shared =
      has_shared(d) ? y_routed + (size_t)d.tokens * d.top_k * d.d_model * 3 : nullptr;
  const moe::TileSpec ts = moe::ffn_tile_spec(ffn_shape(d));
  const uint16_t* x_in = nullptr;
  MOE_TRY(route_permute(d, x, norm, w_router, bias, ws, route_bufs(L), &ts, s, &x_in));
  MOE_TRY(gate_up_impl(d, x_in, perm, offsets, w1, w3, ws1, ws3, h, ws, s, true));
  MOE_TRY(down_impl(d, h, offsets, w2, ws2, y_routed, y_shared, ws, s, true, true));
  return hip_status(moe::launch_combine(y_routed, inv, w, y_shared, residual, out, d.tokens,
                                        d.d_model, d.top_k, s, true));
}

// ---------------------------------------------------------------------- FP8 weights
moe_status check_fp8(const moe_dims& d, const moe_fp8_weights* w, bool gate_up, bool down) {
  if (w == nullptr) return MOE_EINVAL;
  const int B = moe::kFp8Block;
  if (d.d_model % B != 0 || d.d_expert % B != 0) return MOE_EUNSUPPORTED;
  if (d.d_model > moe::kFp8MaxK || d.d_expert > moe::kFp8MaxK) return MOE_EUNSUPPORTED;
  if (gate_up) {
    MOE_NEED(aligned(w->w1, 16) && aligned(w->w3, 16));
    MOE_NEED(aligned(w->w1_scale, 4) && aligned(w->w3_scale, 4));
    if (has_shared(d)) {
      MOE_NEED(aligned(w->ws1, 16) && aligned(w->ws3, 16));
      MOE_NEED(aligned(w->ws1_scale, 4) && aligned(w->ws3_scale, 4));
    }
  }
  if (down) {
    MOE_NEED(aligned(w->w2, 16) && aligned(w->w2_scale, 4));
    if (has_shared(d)) MOE_NEED(aligned(w->ws2, 16) && aligned(w->ws2_scale, 4));
  }
  return MOE_OK;
}

moe::Fp8Weights fp8_of(const moe_fp8_weights& w) {
  return moe::Fp8Weights{w.w1, w.w3, w.w2, w.w1_scale, w.w3_scale, w.w2_scale,
                         w.ws1, w.ws3, w.ws2, w.ws1_scale, w.ws3_scale, w.ws2_scale};
}

moe_status check_forward_args(const moe_dims& d, const float* w_router, const float* bias,
                              const uint16_t* w1, const uint16_t* w3, const uint16_t* w2,
                              const uint16_t* ws1, const uint16_t* ws3, const uint16_t* ws2,
                              uint16_t* out, void* ws, size_t ws_bytes) {
  MOE_NEED(aligned(w_router, 16) && aligned(bias, 4));
  MOE_NEED(aligned(w1, 16) && aligned(w3, 16) && aligned(w2, 16) && aligned(out, 16));
  if (has_shared(d)) MOE_NEED(aligned(ws1, 16) && aligned(ws3, 16) && aligned(ws2, 16));
  return check_ws(d, ws, ws_bytes);
}

// Device address of `scratch` on the current device, looked up once per device (with that
// device current) and kept: each GPU holds its own copy of the array at its own address.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

moe_status noalloc_scratch(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return MOE_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_forward(const moe_dims* dims, const uint16_t* x, const float* w_router,
                       const float* bias, const uint16_t* w1, const uint16_t* w3,
                       const uint16_t* w2, const uint16_t* ws1, const uint16_t* ws3,
                       const uint16_t* ws2, uint16_t* out, void* ws, size_t ws_bytes,
                       void* stream) {
  MOE_TRY(check_dims(dims));
  const moe_dims& d = *dims;
  if (d.tokens == 0) return MOE_OK;
  MOE_NEED(aligned(x, 16));
  MOE_TRY(check_forward_args(d, w_router, bias, w1, w3, w2, ws1, ws3, ws2, out, ws, ws_bytes));
  (void)hipGetLastError();
  return forward_impl(d, x, nullptr, w_router, bias, w1, w3, w2, ws1, ws3, ws2, nullptr, out, ws,
                      (hipStream_t)stream);
}

moe_status moe_workspace_release(const void* ws) {
  if (ws != nullptr) moe::arrival_release(ws);
  return MOE_OK;
}

moe_status moe_forward_noalloc(const moe_dims* dims, const uint16_t* x, const float* w_router,
                               const float* bias, const uint16_t* w1, const uint16_t* w3,
                               const uint16_t* w2, const uint16_t* ws1, const uint16_t* ws3,
                               const uint16_t* ws2, uint16_t* out, void* stream) {
  MOE_TRY(check_dims(dims));
  const moe_dims& d = *dims;
  if (d.tokens == 0) return MOE_OK;
  MOE_NEED(aligned(x, 16) && aligned(w_router, 16) && aligned(bias, 4));
  MOE_NEED(aligned(w1, 16) && aligned(w3, 16) && aligned(w2, 16) && aligned(out, 16));
  if (has_shared(d)) MOE_NEED(aligned(ws1, 16) && aligned(ws3, 16) && aligned(ws2, 16));
  if (layout(d).total > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ESCRATCH;
  void* ws = nullptr;
  MOE_TRY(noalloc_scratch(&ws));
  (void)hipGetLastError();
  return forward_impl(d, x, nullptr, w_router, bias, w1, w3, w2, ws1, ws3, ws2, nullptr, out, ws,
                      (hipStream_t)stream);
}

moe_status moe_expert_gate_up_fp8(const moe_dims* dims, const uint16_t* x,
                                  const int32_t* perm_rows, const int32_t* offsets,
                                  const moe_fp8_weights* w, uint16_t* h, void* ws,
                                  size_t ws_bytes, void* stream) {
  MOE_TRY(check_dims(dims));
  const moe_dims& d = *dims;
  MOE_TRY(check_fp8(d, w, true, false));
  if (d.tokens == 0) return MOE_OK;
  MOE_NEED(aligned(x, 16) && aligned(perm_rows, 4) && aligned(offsets, 4) && aligned(h, 16));
  MOE_TRY(check_ws(d, ws, ws_bytes));
  (void)hipGetLastError();
  const Layout L = layout(d);
  return hip_status(moe::launch_gate_up_fp8(ffn_shape_fp8(d), x, perm_rows, offsets, fp8_of(*w), h,
                                            at<Tile>(ws, L.tiles), at<int32_t>(ws, L.ntiles),
                                            (hipStream_t)stream));
}

moe_status moe_expert_down_fp8(const moe_dims* dims, const uint16_t* h, const int32_t* offsets,
                               const moe_fp8_weights* w, float* y_routed, float* y_shared,
                               void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_dims(dims));
  const moe_dims& d = *dims;
  MOE_TRY(check_fp8(d, w, false, true));
  if (d.tokens == 0) return MOE_OK;
  MOE_NEED(aligned(h, 16) && aligned(offsets, 4) && aligned(y_routed, 16));
  if (has_shared(d)) MOE_NEED(aligned(y_shared, 16));
  MOE_TRY(check_ws(d, ws, ws_bytes));
  (void)hipGetLastError();
  const Layout L = layout(d);
  return hip_status(moe::launch_down_fp8(ffn_shape_fp8(d), h, offsets, fp8_of(*w), y_routed,
                                         has_shared(d) ? y_shared : nullptr,
                                         at<Tile>(ws, L.tiles), at<int32_t>(ws, L.ntiles),
                                         (hipStream_t)stream));
}

moe_status moe_forward_fp8(const moe_dims* dims, const uint16_t* x, const float* w_router,
                           const float* bias, const moe_fp8_weights* w, uint16_t* out,
                           void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_dims(dims));
  const moe_dims& d = *dims;
  MOE_TRY(check_fp8(d, w, true, true));
  if (d.tokens == 0) return MOE_OK;
  MOE_NEED(aligned(x, 16) && aligned(w_router, 16) && aligned(bias, 4) && aligned(out, 16));
  MOE_TRY(check_ws(d, ws, ws_bytes));
  (void)hipGetLastError();
  const hipStream_t s = (hipStream_t)stream;
  const Layout L = layout(d);
  float* gw = at<float>(ws, L.w);
  int32_t* offsets = at<int32_t>(ws, L.offsets);
  int32_t* perm = at<int32_t>(ws, L.perm);
  int32_t* inv = at<int32_t>(ws, L.inv);
  uint16_t* h = at<uint16_t>(ws, L.h);
  uint8_t* y_routed = at<uint8_t>(ws, L.y);
  uint8_t* y_shared =
      has_shared(d) ? y_routed + (size_t)d.tokens * d.top_k * d.d_model * 3 : nullptr;
  const moe::Fp8Weights fw = fp8_of(*w);
  const moe::TileSpec ts = moe::ffn_tile_spec_fp8(ffn_shape_fp8(d));
  const uint16_t* x_in = nullptr;
  MOE_TRY(route_permute(d, x, nullptr, w_router, bias, ws, route_bufs(L), &ts, s, &x_in));
  MOE_TRY(hip_status(moe::launch_gate_up_fp8(ffn_shape_fp8(d), x, perm, offsets, fw, h,
                                             at<Tile>(ws, L.tiles), at<int32_t>(ws, L.ntiles),
                                             s, true)));
  MOE_TRY(hip_status(moe::launch_down_fp8(ffn_shape_fp8(d), h, offsets, fw, y_routed, y_shared,
                                          at<Tile>(ws, L.tiles), at<int32_t>(ws, L.ntiles),
                                          s, true, true)));
  return combine_impl(d, y_routed, inv, gw, y_shared, out, s, true);
}

moe_status moe_block_workspace_bytes(const moe_dims* dims, size_t* bytes) {
  MOE_TRY(check_dims(dims));
  MOE_NEED(bytes != nullptr);
  *bytes = layout(*dims).total + align_up((size_t)dims->tokens * dims->d_model * 2);
  return MOE_OK;
}

moe_status moe_forward_block(const moe_dims* dims, const uint16_t* x_res, const float* norm_w,
                             float norm_eps, const float* w_router, const float* bias,
                             const uint16_t* w1, const uint16_t* w3, const uint16_t* w2,
                             const uint16_t* ws1, const uint16_t* ws3, const uint16_t* ws2,
                             uint16_t* out, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_dims(dims));
  const moe_dims& d = *dims;
  if (d.tokens == 0) return MOE_OK;
  MOE_NEED(aligned(x_res, 16) && aligned(norm_w, 4));
  {
    // out and x_res must not share any byte (both [T, d] bf16)
    const uintptr_t a = (uintptr_t)x_res, o = (uintptr_t)out;
    const uintptr_t n = (uintptr_t)d.tokens * (uintptr_t)d.d_model * 2u;
    MOE_NEED(o + n <= a || a + n <= o);
  }
  if (!(norm_eps >= 0.0f) || !isfinite(norm_eps)) return MOE_EINVAL;
  MOE_TRY(check_forward_args(d, w_router, bias, w1, w3, w2, ws1, ws3, ws2, out, ws, ws_bytes));
  const size_t base = layout(d).total;
  if (ws_bytes < base + align_up((size_t)d.tokens * d.d_model * 2)) return MOE_EWORKSPACE;
  (void)hipGetLastError();
  const hipStream_t s = (hipStream_t)stream;
  // x_ffn = RMSNorm(x_res) goes to the end of the workspace, made by the router kernel's
  // own pass over x_res up to kRouterSmallT tokens (else by the norm kernel)
  const moe::RouterNorm norm{norm_w, norm_eps, at<uint16_t>(ws, base)};
  return forward_impl(d, x_res, &norm, w_router, bias, w1, w3, w2, ws1, ws3, ws2, x_res, out, ws,
                      s);
}

const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_EINVAL: return "MOE_EINVAL: invalid argument (null or misaligned pointer, bad dims)";
    case MOE_EUNSUPPORTED: return "MOE_EUNSUPPORTED: dims this library does not handle";
    case MOE_EWORKSPACE: return "MOE_EWORKSPACE: workspace smaller than moe_workspace_bytes()";
    case MOE_EHIP: return "MOE_EHIP: HIP launch error";
    case MOE_ESCRATCH:
      return "MOE_ESCRATCH: moe_forward_noalloc needs moe_workspace_bytes(dims) <= "
             "MOE_NOALLOC_SCRATCH_BYTES (its fixed device scratch)";
    default: return "unknown moe_status";
  }
}

moe_status moe_workspace_bytes(const moe_dims* dims, size_t* bytes) {
  MOE_TRY(check_dims(dims));
  MOE_NEED(bytes != nullptr);
  *bytes = layout(*dims).total;
  return MOE_OK;
}

moe_status moe_route(const moe_dims* dims, const uint16_t* x, const float* w_router,
                     const float* bias, int32_t* topk_idx, float* topk_w, float* logits, void* ws,
                     size_t ws_bytes, void* stream) {
  MOE_TRY(check_dims(dims));
  const moe_dims& d = *dims;
  if (d.tokens == 0) return MOE_OK;
  MOE_NEED(aligned(x, 16) && aligned(w_router, 16) && aligned(bias, 4));
  MOE_NEED(aligned(topk_idx, 4) && aligned(topk_w, 4));
  if (logits != nullptr) MOE_NEED(aligned(logits, 4));
  MOE_TRY(check_ws(d, ws, ws_bytes));
  (void)hipGetLastError();
  return route_impl(d, x, w_router, bias, topk_idx, topk_w, logits, ws, (hipStream_t)stream);
}

moe_status moe_permute(const moe_dims* dims, const int32_t* topk_idx, int32_t* counts,
                       int32_t* offsets, int32_t* perm_rows, int32_t* inv_perm, void* ws,
                       size_t ws_bytes, void* stream) {
  MOE_TRY(check_dims(dims));
  const moe_dims& d = *dims;
  MOE_NEED(aligned(counts, 4) && aligned(offsets, 4));
  if (d.tokens > 0) MOE_NEED(aligned(topk_idx, 4) && aligned(perm_rows, 4) && aligned(inv_perm, 4));
  MOE_TRY(check_ws(d, ws, ws_bytes));
  (void)hipGetLastError();
  return permute_impl(d, topk_idx, counts, offsets, perm_rows, inv_perm, ws, (hipStream_t)stream);
}

moe_status moe_expert_gate_up(const moe_dims* dims, const uint16_t* x, const int32_t* perm_rows,
                              const int32_t* offsets, const uint16_t* w1, const uint16_t* w3,
                              const uint16_t* ws1, const uint16_t* ws3, uint16_t* h, void* ws,
                              size_t ws_bytes, void* stream) {
  MOE_TRY(check_dims(dims));
  const moe_dims& d = *dims;
  if (d.tokens == 0) return MOE_OK;
  MOE_NEED(aligned(x, 16) && aligned(perm_rows, 4) && aligned(offsets, 4));
  MOE_NEED(aligned(w1, 16) && aligned(w3, 16) && aligned(h, 16));
  MOE_NEED(shared_ptrs_ok(d, ws1, ws3));
  MOE_TRY(check_ws(d, ws, ws_bytes));
  (void)hipGetLastError();
  return gate_up_impl(d, x, perm_rows, offsets, w1, w3, ws1, ws3, h, ws, (hipStream_t)stream);
}

moe_status moe_expert_down(const moe_dims* dims, const uint16_t* h, const int32_t* offsets,
                           const uint16_t* w2, const uint16_t* ws2, float* y_routed,
                           float* y_shared, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_dims(dims));
  const moe_dims& d = *dims;
  if (d.tokens == 0) return MOE_OK;
  MOE_NEED(aligned(h, 16) && aligned(offsets, 4) && aligned(w2, 16) && aligned(y_routed, 16));
  MOE_NEED(shared_ptrs_ok(d, ws2, y_shared));
  MOE_TRY(check_ws(d, ws, ws_bytes));
  (void)hipGetLastError();
  return down_impl(d, h, offsets, w2, ws2, y_routed, y_shared, ws, (hipStream_t)stream);
}

moe_status moe_expert_ffn(const moe_dims* dims, const uint16_t* x, const int32_t* perm_rows,
                          const int32_t* offsets, const uint16_t* w1, const uint16_t* w3,
                          const uint16_t* w2, const uint16_t* ws1, const uint16_t* ws3,
                          const uint16_t* ws2, float* y_routed, float* y_shared, void* ws,
                          size_t ws_bytes, void* stream) {
  MOE_TRY(check_dims(dims));
  const moe_dims& d = *dims;
  if (d.tokens == 0) return MOE_OK;
  MOE_NEED(aligned(x, 16) && aligned(perm_rows, 4) && aligned(offsets, 4));
  MOE_NEED(aligned(w1, 16) && aligned(w3, 16) && aligned(w2, 16) && aligned(y_routed, 16));
  MOE_NEED(shared_ptrs_ok(d, ws1, ws3) && shared_ptrs_ok(d, ws2, y_shared));
  MOE_TRY(check_ws(d, ws, ws_bytes));
  (void)hipGetLastError();
  const hipStream_t s = (hipStream_t)stream;
  uint16_t* h = at<uint16_t>(ws, layout(d).h);
  MOE_TRY(gate_up_impl(d, x, perm_rows, offsets, w1, w3, ws1, ws3, h, ws, s));
  return down_impl(d, h, offsets, w2, ws2, y_routed, y_shared, ws, s, true);
}

moe_status moe_combine(const moe_dims* dims, const float* y_routed, const int32_t* inv_perm,
                       const float* topk_w, const float* y_shared, uint16_t* out,
                       void* stream) {
  MOE_TRY(check_dims(dims));
  const moe_dims& d = *dims;
  if (d.tokens == 0) return MOE_OK;
  MOE_NEED(aligned(y_routed, 16) && aligned(inv_perm, 4) && aligned(topk_w, 4) && aligned(out, 16));
  if (y_shared != nullptr) MOE_NEED(aligned(y_shared, 16));
  (void)hipGetLastError();
  return combine_impl(d, y_routed, inv_perm, topk_w, y_shared, out, (hipStream_t)stream);
}

}  // extern "C"

extern "C" {

moe_status moe_latent_workspace_bytes(const moe_dims* dims, int32_t d_latent, size_t* bytes) {
  MOE_TRY(check_latent(dims, d_latent));
  MOE_NEED(bytes != nullptr);
  *bytes = latent_layout(*dims, d_latent).total;
  return MOE_OK;
}

moe_status moe_forward_latent(const moe_dims* dims, int32_t d_latent, const uint16_t* x,
                              const float* w_router, const float* bias, const uint16_t* w_down,
                              const uint16_t* w1, const uint16_t* w3, const uint16_t* w2,
                              const uint16_t* w_up, const uint16_t* ws1, const uint16_t* ws3,
                              const uint16_t* ws2, uint16_t* out, void* ws, size_t ws_bytes,
                              void* stream) {
  MOE_TRY(check_latent(dims, d_latent));
  const moe_dims& d = *dims;
  const int32_t L = d_latent;
  if (d.tokens == 0) return MOE_OK;
  MOE_NEED(aligned(x, 16) && aligned(w_router, 16) && aligned(bias, 4) && aligned(w_down, 16));
  MOE_NEED(aligned(w1, 16) && aligned(w3, 16) && aligned(w2, 16) && aligned(w_up, 16));
  MOE_NEED(aligned(out, 16));
  if (has_shared(d)) MOE_NEED(aligned(ws1, 16) && aligned(ws3, 16) && aligned(ws2, 16));
  const LatentLayout P = latent_layout(d, L);
  MOE_NEED(aligned(ws, kWsAlign));
  if (ws_bytes < P.total) return MOE_EWORKSPACE;
  (void)hipGetLastError();
  const hipStream_t s = (hipStream_t)stream;
  const int64_t T = d.tokens;
  float* w = at<float>(ws, P.w);
  int32_t* offsets = at<int32_t>(ws, P.offsets);
  int32_t* perm = at<int32_t>(ws, P.perm);
  int32_t* inv = at<int32_t>(ws, P.inv);
  Tile* tiles = at<Tile>(ws, P.tiles);
  int32_t* ntiles = at<int32_t>(ws, P.ntiles);
  uint16_t* lat = at<uint16_t>(ws, P.lat);
  uint16_t* h = at<uint16_t>(ws, P.h);
  uint8_t* y = at<uint8_t>(ws, P.y);
  uint16_t* uhat = at<uint16_t>(ws, P.uhat);
  // router on the full-width input ("Kimi K3 · Latent up-projection": the gate scores
  // hidden_states before the down-projection), and the permutation
  const uint16_t* x_in = nullptr;
  MOE_TRY(route_permute(d, x, nullptr, w_router, bias, ws, route_bufs(P), nullptr, s, &x_in));
  (void)x_in;
  // down-projection to the latent width (bf16: the experts' MFMA operand)
  MOE_TRY(hip_status(moe::launch_dense(x, T, d.d_model, w_down, L, moe::DenseOut::kBF16, nullptr,
                                       lat, nullptr, tiles, ntiles, s)));
  // routed experts on the latent
  const FfnShape rsh{T, L, d.n_experts, d.top_k, d.d_expert, false, hsplit(d)};
  MOE_TRY(hip_status(moe::launch_gate_up(rsh, lat, perm, offsets, w1, w3, nullptr, nullptr, h,
                                         tiles, ntiles, s)));
  MOE_TRY(hip_status(
      moe::launch_down(rsh, h, offsets, w2, nullptr, y, nullptr, tiles, ntiles, s, true, true)));
  // gate-weighted sum over the slots, RMSNorm (eps from the config), bf16
  const bool uhat2 = L <= moe::kLatentTwoPartMaxL;
  MOE_TRY(hip_status(
      moe::launch_combine_rmsnorm(y, inv, w, uhat, T, L, d.top_k, 1e-6f, uhat2, s)));
  const int KU = uhat2 ? 2 * L : L, WK = uhat2 ? L : 0;
  if (has_shared(d)) {
    // shared expert on the full-width input: a T-row group with no routed experts
    const FfnShape ssh{T, d.d_model, 0, 0, d.d_shared, true, hsplit(d)};
    uint16_t* hs = at<uint16_t>(ws, P.hs);
    float* ys = at<float>(ws, P.ys);
    MOE_TRY(hip_status(moe::launch_gate_up(ssh, x, nullptr, nullptr, nullptr, nullptr, ws1, ws3,
                                           hs, tiles, ntiles, s)));
    MOE_TRY(hip_status(moe::launch_down(ssh, hs, nullptr, nullptr, ws2, nullptr, ys, tiles, ntiles,
                                        s, true)));
    // up-projection (u_hat in one or two bf16 parts) with the shared output added before the
    // one bf16 rounding
    return hip_status(moe::launch_dense(uhat, T, KU, w_up, d.d_model, moe::DenseOut::kAddBF16,
                                        nullptr, out, ys, tiles, ntiles, s, 1, WK));
  }
  return hip_status(moe::launch_dense(uhat, T, KU, w_up, d.d_model, moe::DenseOut::kBF16,
                                      nullptr, out, nullptr, tiles, ntiles, s, 1, WK));
}

}  // extern "C"
