// Host side of the C ABI declared in include/moe.h: argument validation,
// workspace carving and launch sequencing.  Nothing here allocates device
// memory or synchronises.  Every kernel goes onto the caller's stream,
// except that moe_forward runs a weight-streaming shared expert on a second
// stream of its own, forked from and joined back into the caller's stream.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "../../include/moe.h"
#include "kernels.h"

namespace {

thread_local std::string g_last_error;

moe_status fail(moe_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

moe_status ok() {
  g_last_error.clear();
  return MOE_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQUIRE_PTR(ptr)                                                           \
  do {                                                                             \
    if ((ptr) == nullptr) return fail(MOE_ERR_INVALID_ARG, "%s is NULL", #ptr);    \
    if (!aligned16(ptr))                                                           \
      return fail(MOE_ERR_UNSUPPORTED, "%s is not 16-byte aligned", #ptr);         \
  } while (0)

#define OPTIONAL_PTR(ptr)                                                          \
  do {                                                                             \
    if ((ptr) != nullptr && !aligned16(ptr))                                       \
      return fail(MOE_ERR_UNSUPPORTED, "%s is not 16-byte aligned", #ptr);         \
  } while (0)

constexpr int64_t kMaxPairs = (int64_t)1 << 31;
constexpr int kMaxNormH = 8192;  // ScMoE norms hold one row per workgroup in registers

moe_status check_params(const moe_params* p) {
  if (!p) return fail(MOE_ERR_INVALID_ARG, "params is NULL");
  if (p->T < 0) return fail(MOE_ERR_INVALID_ARG, "T = %lld < 0", (long long)p->T);
  if (p->E < 1) return fail(MOE_ERR_INVALID_ARG, "E = %d < 1", p->E);
  if (p->k < 1 || p->k > MOE_MAX_TOP_K)
    return fail(MOE_ERR_INVALID_ARG, "k = %d outside 1..%d", p->k, MOE_MAX_TOP_K);
  if (p->k > p->E) return fail(MOE_ERR_INVALID_ARG, "k = %d > E = %d", p->k, p->E);
  if (p->H < 1) return fail(MOE_ERR_INVALID_ARG, "H = %d < 1", p->H);
  if (p->I < 1) return fail(MOE_ERR_INVALID_ARG, "I = %d < 1", p->I);
  if (p->I_shared < 0) return fail(MOE_ERR_INVALID_ARG, "I_shared = %d < 0", p->I_shared);
  if (!std::isfinite(p->swiglu_limit) || !(p->swiglu_limit > 0.0f))
    return fail(MOE_ERR_INVALID_ARG, "swiglu_limit must be finite and > 0 (no default)");
  if (!std::isfinite(p->routed_scaling_factor))
    return fail(MOE_ERR_INVALID_ARG, "routed_scaling_factor is not finite");
  if (p->scmoe != 0 && p->scmoe != 1)
    return fail(MOE_ERR_INVALID_ARG, "scmoe = %d is not 0 or 1", p->scmoe);
  if (p->scmoe && !(std::isfinite(p->norm_eps) && p->norm_eps > 0.0f))
    return fail(MOE_ERR_INVALID_ARG, "norm_eps must be finite and > 0 with scmoe");
  if (p->E > MOE_MAX_EXPERTS)
    return fail(MOE_ERR_UNSUPPORTED, "E = %d > %d", p->E, MOE_MAX_EXPERTS);
  if (p->H % 8 || p->I % 8 || p->I_shared % 8)
    return fail(MOE_ERR_UNSUPPORTED, "H, I, I_shared must be multiples of 8 (%d, %d, %d)", p->H,
                p->I, p->I_shared);
  if (p->T * (int64_t)p->k >= kMaxPairs)
    return fail(MOE_ERR_UNSUPPORTED, "T*k = %lld >= 2^31", (long long)(p->T * p->k));
  if (p->scmoe && p->H > kMaxNormH)
    return fail(MOE_ERR_UNSUPPORTED, "scmoe with H = %d > %d", p->H, kMaxNormH);
  if (p->w4 != 0 && p->w4 != 1)
    return fail(MOE_ERR_INVALID_ARG, "w4 = %d is not 0 or 1", p->w4);
  if (p->w4 && (p->H % 128 != 0 || p->I % 128 != 0))
    return fail(MOE_ERR_UNSUPPORTED, "W4A16 experts need H and I multiples of 128 (H=%d I=%d)",
                p->H, p->I);
  return MOE_OK;
}

// Workspace carving: 256-byte aligned slots in a fixed order.
struct Carver {
  size_t off = 0;
  char* base = nullptr;
  template <class T>
  T* take(size_t n) {
    off = (off + 255) & ~size_t(255);
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += n * sizeof(T);
    return p;
  }
};

// Tile variant by the mean rows per group: about one short row tile or less
// (decode) -> persistent weight streaming; several 256-row tiles -> the
// pipelined 256-row tiles (eight wavefronts); in between the 128-row tiles.
// MOE_GEMM_VARIANT=wstream | tile32 | tile128 | pipe256w8 | pingpong forces
// one (a tuning lever; results are identical up to fp32 summation order).
GemmVariant pick_variant_raw(int64_t rows, int64_t groups) {
  if (const char* env = std::getenv("MOE_GEMM_VARIANT")) {
    if (!std::strcmp(env, "tile32")) return GemmVariant::kTile32;
    if (!std::strcmp(env, "tile128")) return GemmVariant::kTile128;
    if (!std::strcmp(env, "wstream")) return GemmVariant::kWStream;
    if (!std::strcmp(env, "pipe256w8")) return GemmVariant::kPipe256W8;
    if (!std::strcmp(env, "pingpong")) return GemmVariant::kPingPong;
  }
  if (rows <= 64 * groups) return GemmVariant::kWStream;
  if (rows >= 512 * groups) return GemmVariant::kPingPong;
  return GemmVariant::kTile128;
}

// The pipelined and streaming variants address A rows and one group's
// weights with 32-bit element offsets and step K in 32-wide units, and the
// pipelined tiles address a tile's output with 32-bit byte offsets (output
// widths up to 2^20); other operands fall back to the LDS-staged tiles.
GemmVariant pick_variant(int64_t rows, int64_t groups, int64_t a_elems, int64_t w_group_elems,
                         bool k_multiple_of_32, int64_t max_width) {
  GemmVariant v = pick_variant_raw(rows, groups);
  const int64_t lim = (int64_t)1 << 31;
  if (v == GemmVariant::kWStream && (a_elems >= lim || w_group_elems >= lim || !k_multiple_of_32))
    v = GemmVariant::kTile32;
  const bool pipe = v == GemmVariant::kPipe256W8 || v == GemmVariant::kPingPong;
  if (pipe && (a_elems >= lim || w_group_elems >= lim || !k_multiple_of_32 ||
               max_width > ((int64_t)1 << 20)))
    v = GemmVariant::kTile128;
  return v;
}

struct Layout {
  float* logits;
  float* partial;
  int32_t* ids;
  float* w;
  int32_t* counts;
  int32_t* starts;
  int32_t* offsets;
  int32_t* sorted_token;
  int32_t* inv_pos;
  int32_t* mstart;
  uint16_t* h;
  float* y;
  uint16_t* hs;
  float* ys;
  uint16_t* xr;
  uint16_t* deq_gu;  // W4A16 experts dequantised to bf16 (batches beyond weight streaming)
  uint16_t* deq_dn;
  size_t bytes;
};

// The tile variant of the layer's expert GEMMs (routed and shared).
GemmVariant layer_variant(const moe_params& p) {
  const int64_t N = p.T * p.k;
  return pick_variant(N, p.E, std::max<int64_t>(N, p.T) * std::max(p.H, std::max(p.I, p.I_shared)),
                      (int64_t)2 * std::max(p.I, p.I_shared) * p.H,
                      p.H % 32 == 0 && p.I % 32 == 0 && p.I_shared % 32 == 0,
                      std::max(p.H, std::max(p.I, p.I_shared)));
}

// W4A16 routed experts are read as codes by the weight-streaming and
// ping-pong kernels (the latter for K >= 256 in both projections: H, I >=
// 256); the other tile variants (forced by MOE_GEMM_VARIANT, or the 128-row
// tiles of mid-sized batches) read them dequantised to bf16 in the
// workspace.
bool w4_codes_variant(const moe_params& p, GemmVariant v) {
  return v == GemmVariant::kWStream ||
         (v == GemmVariant::kPingPong && p.H >= 256 && p.I >= 256);
}
bool w4_dequant_batch(const moe_params& p) {
  return p.w4 && !w4_codes_variant(p, layer_variant(p));
}

Layout carve(const moe_params& p, void* ws) {
  Carver c;
  c.base = static_cast<char*>(ws);
  const int64_t T = p.T, N = p.T * p.k;
  const int tiles = permute_tiles(N);
  Layout L;
  const int splits = router_splits(T, p.H, p.E);
  L.logits = c.take<float>(T * p.E);
  L.partial = c.take<float>(splits > 1 ? (size_t)splits * T * p.E : 0);
  L.ids = c.take<int32_t>(N);
  L.w = c.take<float>(N);
  L.counts = c.take<int32_t>((size_t)tiles * p.E);
  L.starts = c.take<int32_t>((size_t)tiles * p.E);
  L.offsets = c.take<int32_t>(p.E + 1);
  L.sorted_token = c.take<int32_t>(N);
  L.inv_pos = c.take<int32_t>(N);
  L.mstart = c.take<int32_t>(p.E + 1);
  L.h = c.take<uint16_t>((size_t)N * p.I);
  L.y = c.take<float>((size_t)N * p.H);
  L.hs = c.take<uint16_t>((size_t)T * p.I_shared);
  L.ys = c.take<float>(p.I_shared ? (size_t)T * p.H : 0);
  L.xr = c.take<uint16_t>(p.scmoe ? (size_t)T * p.H : 0);
  const bool deq = w4_dequant_batch(p);
  L.deq_gu = deq ? c.take<uint16_t>((size_t)p.E * 2 * p.I * p.H) : nullptr;
  L.deq_dn = deq ? c.take<uint16_t>((size_t)p.E * p.H * p.I) : nullptr;
  L.bytes = (c.off + 255) & ~size_t(255);
  return L;
}

// Router-only and permute-only entry points use the front of the workspace
// (router: the logits first, then the K-slice partials).
size_t router_ws_bytes(const moe_params& p) {
  Carver c;
  const int splits = router_splits(p.T, p.H, p.E);
  c.take<float>((size_t)p.T * p.E);
  c.take<float>(splits > 1 ? (size_t)splits * p.T * p.E : 0);
  return c.off;
}
size_t permute_ws_bytes(const moe_params& p) {
  Carver c;
  const int tiles = permute_tiles(p.T * p.k);
  c.take<int32_t>((size_t)tiles * p.E);
  c.take<int32_t>((size_t)tiles * p.E);
  return c.off;
}

// A second stream and two events per thread and device.  moe_forward runs
// the shared expert on it beside the routing kernels when the grouped GEMMs
// stream weights (a few rows per expert): the routing launches are
// latency-bound and occupy few CUs while the shared weights are a fixed
// share of the bytes.  Created on first use (so not during a graph capture
// that starts with the first call), default priority, kept until the
// process ends.
struct SideStream {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr, join2 = nullptr;
};
constexpr int kMaxDevices = 64;

moe_status side_stream(SideStream** out) {
  thread_local SideStream per_device[kMaxDevices];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(MOE_ERR_DEVICE, "no usable current device (%d)", dev);
  SideStream& S = per_device[dev];
  if (S.stream == nullptr) {
    SideStream n;
    if (hipStreamCreateWithFlags(&n.stream, hipStreamNonBlocking) != hipSuccess)
      return fail(MOE_ERR_DEVICE, "second stream: %s", hipGetErrorString(hipGetLastError()));
    // the events only order work of one device: a device-scope release
    // (the default system-scope one writes back and invalidates caches for
    // the host's sake and stalls the queue for microseconds)
    const unsigned flags = hipEventDisableTiming | hipEventReleaseToDevice;
    if (hipEventCreateWithFlags(&n.fork, flags) != hipSuccess ||
        hipEventCreateWithFlags(&n.join, flags) != hipSuccess ||
        hipEventCreateWithFlags(&n.join2, flags) != hipSuccess)
      return fail(MOE_ERR_DEVICE, "stream events: %s", hipGetErrorString(hipGetLastError()));
    S = n;
  }
  *out = &S;
  return MOE_OK;
}

moe_status device_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
  return MOE_OK;
}

GemmProblem make_problem(const uint16_t* A, const int32_t* row_index, const int32_t* offsets,
                         const int32_t* mstart, const uint16_t* W, int64_t w_stride, void* out,
                         int64_t M, int G, int N, int K, GemmVariant v, bool gateup) {
  GemmProblem P;
  const int bm = gemm_tile_m(v), bn = gemm_tile_n(v, gateup);
  P.A = A;
  P.row_index = row_index;
  P.group_offsets = offsets;
  P.mtile_start = mstart;
  P.W = W;
  P.w_stride = w_stride;
  P.S = nullptr;
  P.s_stride = 0;
  P.tscale = nullptr;
  P.out = out;
  P.M = M;
  P.G = G;
  P.N = N;
  P.K = K;
  P.ntiles = (N + bn - 1) / bn;
  P.max_mtiles = (int32_t)((M + bm - 1) / bm + (offsets ? G : 0));
  P.packed = 0;
  P.hblk = 0;
  return P;
}

bool tiles_fit(const GemmProblem& a, const GemmProblem* b) {
  // every variant's tile index (at most m-tiles x n-tiles, counted here with
  // n-tiles rounded up to 8) stays a positive int
  auto n = [](const GemmProblem& p) { return (int64_t)p.max_mtiles * ((p.ntiles + 7) / 8 * 8); };
  const int64_t t = n(a) + (b ? n(*b) : 0);
  return t < ((int64_t)1 << 31);
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_DEVICE: return "MOE_ERR_DEVICE";
  }
  return "MOE_ERR_UNKNOWN";
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

moe_status moe_workspace_size(const moe_params* p, size_t* bytes) {
  moe_status s = check_params(p);
  if (s != MOE_OK) return s;
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = carve(*p, nullptr).bytes;
  return ok();
}

moe_status moe_router_topk(const moe_params* p, const moe_bf16* x, const float* w_router,
                           const float* corr_bias, int32_t* topk_ids, float* topk_w, void* ws,
                           size_t ws_bytes, hipStream_t stream) {
  moe_status s = check_params(p);
  if (s != MOE_OK) return s;
  if (p->T == 0) return ok();
  REQUIRE_PTR(x);
  REQUIRE_PTR(w_router);
  OPTIONAL_PTR(corr_bias);
  REQUIRE_PTR(topk_ids);
  REQUIRE_PTR(topk_w);
  REQUIRE_PTR(ws);
  if (ws_bytes < router_ws_bytes(*p))
    return fail(MOE_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, router_ws_bytes(*p));
  Carver c;
  c.base = static_cast<char*>(ws);
  const int splits = router_splits(p->T, p->H, p->E);
  float* logits = c.take<float>((size_t)p->T * p->E);
  float* partial = c.take<float>(splits > 1 ? (size_t)splits * p->T * p->E : 0);
  if ((s = device_status(launch_router(x, w_router, corr_bias, logits, partial, topk_ids, topk_w,
                                       p->T, p->H, p->E, p->k, p->routed_scaling_factor, stream),
                         "router")) != MOE_OK)
    return s;
  return ok();
}

moe_status moe_permute(const moe_params* p, const int32_t* topk_ids, const moe_bf16* x,
                       int32_t* expert_offsets, int32_t* sorted_token, int32_t* inv_pos,
                       moe_bf16* x_perm, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status s = check_params(p);
  if (s != MOE_OK) return s;
  if (x_perm && !x) return fail(MOE_ERR_INVALID_ARG, "x_perm needs x (the rows to gather)");
  REQUIRE_PTR(expert_offsets);
  const int64_t N = p->T * p->k;
  if (N > 0) {
    REQUIRE_PTR(topk_ids);
    REQUIRE_PTR(sorted_token);
    REQUIRE_PTR(inv_pos);
    OPTIONAL_PTR(x);
    OPTIONAL_PTR(x_perm);
    REQUIRE_PTR(ws);
    if (ws_bytes < permute_ws_bytes(*p))
      return fail(MOE_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, permute_ws_bytes(*p));
  }
  Carver c;
  c.base = static_cast<char*>(ws);
  const int tiles = permute_tiles(N);
  int32_t* counts = c.take<int32_t>((size_t)tiles * p->E);
  int32_t* starts = c.take<int32_t>((size_t)tiles * p->E);
  if ((s = device_status(launch_permute(topk_ids, counts, starts, expert_offsets, sorted_token,
                                        inv_pos, N, p->E, p->k, 0, nullptr, stream),
                         "permute")) != MOE_OK)
    return s;
  if (x_perm && N > 0 &&
      (s = device_status(launch_gather_rows(x, sorted_token, x_perm, N, p->H, stream),
                         "gather")) != MOE_OK)
    return s;
  return ok();
}

moe_status moe_grouped_gemm_workspace_size(int32_t n_groups, int64_t M_total, int32_t H,
                                           int32_t I, size_t* bytes) {
  if (n_groups < 1 || n_groups > MOE_MAX_EXPERTS)
    return fail(n_groups < 1 ? MOE_ERR_INVALID_ARG : MOE_ERR_UNSUPPORTED,
                "n_groups = %d outside 1..%d", n_groups, MOE_MAX_EXPERTS);
  if (M_total < 0 || H < 1 || I < 1) return fail(MOE_ERR_INVALID_ARG, "bad M_total/H/I");
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = ((size_t)(n_groups + 1) * sizeof(int32_t) + 255) & ~size_t(255);
  return ok();
}

moe_status moe_grouped_swiglu_gemm(int32_t n_groups, int64_t M_total, int32_t H, int32_t I,
                                   float swiglu_limit, const moe_bf16* a,
                                   const int32_t* row_index, const int32_t* group_offsets,
                                   const moe_bf16* w_gate_up, const moe_bf16* w_down, moe_bf16* h,
                                   float* y, void* ws, size_t ws_bytes, hipStream_t stream) {
  size_t need = 0;
  moe_status s = moe_grouped_gemm_workspace_size(n_groups, M_total, H, I, &need);
  if (s != MOE_OK) return s;
  if (!std::isfinite(swiglu_limit) || !(swiglu_limit > 0.0f))
    return fail(MOE_ERR_INVALID_ARG, "swiglu_limit must be finite and > 0 (no default)");
  if (H % 8 || I % 8) return fail(MOE_ERR_UNSUPPORTED, "H, I must be multiples of 8");
  if (M_total >= kMaxPairs) return fail(MOE_ERR_UNSUPPORTED, "M_total >= 2^31");
  if (M_total == 0) return ok();
  REQUIRE_PTR(a);
  OPTIONAL_PTR(row_index);
  REQUIRE_PTR(group_offsets);
  REQUIRE_PTR(w_gate_up);
  REQUIRE_PTR(w_down);
  REQUIRE_PTR(h);
  REQUIRE_PTR(y);
  REQUIRE_PTR(ws);
  if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  // A is addressed up to the largest row it can hold; the gate_up A is the
  // caller's [rows_a, H] input (rows_a unknown here: bound it by M_total when
  // gathered rows can repeat, the routed case), the down A is h [M_total, I].
  const GemmVariant v =
      pick_variant(M_total, n_groups, std::max<int64_t>(M_total, 1) * std::max(H, I),
                   (int64_t)2 * I * H, H % 32 == 0 && I % 32 == 0, std::max(H, I));
  int32_t* mstart = static_cast<int32_t*>(ws);
  GemmProblem gu = make_problem(a, row_index, group_offsets, mstart, w_gate_up,
                                (int64_t)2 * I * H, h, M_total, n_groups, I, H, v, true);
  GemmProblem dn = make_problem(h, nullptr, group_offsets, mstart, w_down, (int64_t)H * I, y,
                                M_total, n_groups, H, I, v, false);
  if (!tiles_fit(gu, nullptr) || !tiles_fit(dn, nullptr))
    return fail(MOE_ERR_UNSUPPORTED, "too many tiles for one launch");
  const int bm = gemm_tile_m(v);
  if ((s = device_status(
           launch_gemm_schedule(group_offsets, n_groups, bm, bm, mstart, nullptr, stream),
           "gemm schedule")) != MOE_OK)
    return s;
  if ((s = device_status(launch_grouped_gemm(v, true, gu, nullptr, swiglu_limit, stream),
                         "gate_up")) != MOE_OK)
    return s;
  if ((s = device_status(launch_grouped_gemm(v, false, dn, nullptr, swiglu_limit, stream),
                         "down")) != MOE_OK)
    return s;
  return ok();
}

}  // extern "C"

namespace {

// The finish (NULL = none): residual pointer, finite scales, post-norm flag
// and, for a plain layer's post-norm, the norm's own limits.
moe_status check_finish(const moe_params* p, const moe_finish* fin) {
  if (!fin) return MOE_OK;
  REQUIRE_PTR(fin->residual);
  if (!std::isfinite(fin->out_scale) || !std::isfinite(fin->residual_scale))
    return fail(MOE_ERR_INVALID_ARG, "finish scales must be finite");
  if (fin->post_norm != 0 && fin->post_norm != 1)
    return fail(MOE_ERR_INVALID_ARG, "finish post_norm = %d is not 0 or 1", fin->post_norm);
  if (fin->post_norm && !p->scmoe) {
    if (!(std::isfinite(p->norm_eps) && p->norm_eps > 0.0f))
      return fail(MOE_ERR_INVALID_ARG, "norm_eps must be finite and > 0 with a post-norm");
    if (p->H > kMaxNormH)
      return fail(MOE_ERR_UNSUPPORTED, "post-norm with H = %d > %d", p->H, kMaxNormH);
  }
  return MOE_OK;
}

moe_status combine_impl(const moe_params* p, const float* y_perm, const float* topk_w,
                        const int32_t* inv_pos, const float* y_shared, const float* gamma_post,
                        const moe_finish* fin, moe_bf16* out, hipStream_t stream) {
  moe_status s = check_params(p);
  if (s != MOE_OK) return s;
  if (p->T == 0) return ok();
  if ((s = check_finish(p, fin)) != MOE_OK) return s;
  REQUIRE_PTR(y_perm);
  REQUIRE_PTR(topk_w);
  REQUIRE_PTR(inv_pos);
  OPTIONAL_PTR(y_shared);
  OPTIONAL_PTR(gamma_post);
  REQUIRE_PTR(out);
  const int post = p->scmoe || (fin && fin->post_norm);
  if ((s = device_status(launch_combine(y_perm, topk_w, inv_pos, y_shared, gamma_post,
                                        fin ? fin->residual : nullptr, fin ? fin->out_scale : 1.f,
                                        fin ? fin->residual_scale : 1.f, out, p->T, p->H, p->k,
                                        post, p->norm_eps, stream),
                         "combine")) != MOE_OK)
    return s;
  return ok();
}

// one_stream: everything on `stream` (no second stream: the shared expert
// shares the routed experts' launches, W4A16 dequantisation runs in line).
moe_status forward_impl(const moe_params* p, const moe_bf16* x_routed, const moe_bf16* x_shared,
                        const moe_weights* w, const moe_finish* fin, moe_bf16* out,
                        const moe_probes* probes, void* ws, size_t ws_bytes, hipStream_t stream,
                        bool one_stream = false) {
  moe_status s = check_params(p);
  if (s != MOE_OK) return s;
  if (!w) return fail(MOE_ERR_INVALID_ARG, "weights is NULL");
  if (p->T == 0) return ok();
  if ((s = check_finish(p, fin)) != MOE_OK) return s;
  REQUIRE_PTR(x_routed);
  if (p->scmoe && !x_shared)
    return fail(MOE_ERR_INVALID_ARG, "scmoe needs x_shared (the current layer's input)");
  OPTIONAL_PTR(x_shared);
  REQUIRE_PTR(w->w_router);
  OPTIONAL_PTR(w->corr_bias);
  const bool w4 = p->w4 != 0;
  if (w4) {
    REQUIRE_PTR(w->w_gate_up_q);
    REQUIRE_PTR(w->w_gate_up_scale);
    REQUIRE_PTR(w->w_down_q);
    REQUIRE_PTR(w->w_down_scale);
    OPTIONAL_PTR(w->w_gate_up_tscale);
    OPTIONAL_PTR(w->w_down_tscale);
  } else {
    REQUIRE_PTR(w->w_gate_up);
    REQUIRE_PTR(w->w_down);
  }
  const bool packed = w->w_gate_up_packed != nullptr;
  const bool packed_s = w->ws_gate_up_packed != nullptr;
  if ((w->w_down_packed != nullptr) != packed)
    return fail(MOE_ERR_INVALID_ARG, "w_gate_up_packed and w_down_packed go together");
  if ((w->ws_down_packed != nullptr) != packed_s)
    return fail(MOE_ERR_INVALID_ARG, "ws_gate_up_packed and ws_down_packed go together");
  if (packed && w4)
    return fail(MOE_ERR_INVALID_ARG, "packed routed experts are bf16 (params.w4 = 0)");
  if ((packed || packed_s) && (p->H % 32 || p->I_shared % 32 || (packed && p->I % 32)))
    return fail(MOE_ERR_UNSUPPORTED, "packed experts need H, I and I_shared multiples of 32");
  if (!w4 && p->I_shared > 0 && packed != packed_s)  // the 256-row tiles run both in one launch
    return fail(MOE_ERR_INVALID_ARG,
                "bf16 routed and shared experts: both packed pairs or neither");
  OPTIONAL_PTR(w->w_gate_up_packed);
  OPTIONAL_PTR(w->w_down_packed);
  OPTIONAL_PTR(w->ws_gate_up_packed);
  OPTIONAL_PTR(w->ws_down_packed);
  if (p->I_shared > 0) {
    REQUIRE_PTR(w->ws_gate_up);
    REQUIRE_PTR(w->ws_down);
  }
  OPTIONAL_PTR(w->gamma_pre);
  OPTIONAL_PTR(w->gamma_post);
  REQUIRE_PTR(out);
  REQUIRE_PTR(ws);
  if (probes) {
    OPTIONAL_PTR(probes->topk_ids);
    OPTIONAL_PTR(probes->topk_w);
    OPTIONAL_PTR(probes->expert_offsets);
    OPTIONAL_PTR(probes->sorted_token);
    OPTIONAL_PTR(probes->inv_pos);
    OPTIONAL_PTR(probes->xr);
    OPTIONAL_PTR(probes->logits);
    OPTIONAL_PTR(probes->h);
    OPTIONAL_PTR(probes->y);
    OPTIONAL_PTR(probes->h_shared);
    OPTIONAL_PTR(probes->y_shared);
  }
  const int64_t T = p->T, N = T * p->k;
  const GemmVariant v = layer_variant(*p);
  // W4A16: weight streaming and the ping-pong tile unpack the codes in their
  // kernels; the other tiles read the experts dequantised into the workspace
  const bool w4_codes = w4 && w4_codes_variant(*p, v);
  const bool w4_deq = w4 && !w4_codes;
  Layout L = carve(*p, ws);
  if (ws_bytes < L.bytes) return fail(MOE_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, L.bytes);
  if (probes) {
    if (probes->topk_ids) L.ids = probes->topk_ids;
    if (probes->topk_w) L.w = probes->topk_w;
    if (probes->expert_offsets) L.offsets = probes->expert_offsets;
    if (probes->sorted_token) L.sorted_token = probes->sorted_token;
    if (probes->inv_pos) L.inv_pos = probes->inv_pos;
    if (probes->xr && p->scmoe) L.xr = probes->xr;
    if (probes->logits) L.logits = probes->logits;
    if (probes->h) L.h = probes->h;
    if (probes->y) L.y = probes->y;
    if (probes->h_shared && p->I_shared > 0) L.hs = probes->h_shared;
    if (probes->y_shared && p->I_shared > 0) L.ys = probes->y_shared;
  }
  const uint16_t* xr = x_routed;
  const uint16_t* xs = x_shared ? x_shared : x_routed;
  const bool shared = p->I_shared > 0;

  GemmProblem gu = make_problem(xr, L.sorted_token, L.offsets, L.mstart, w->w_gate_up,
                                (int64_t)2 * p->I * p->H, L.h, N, p->E, p->I, p->H, v, true);
  GemmProblem dn = make_problem(L.h, nullptr, L.offsets, L.mstart, w->w_down,
                                (int64_t)p->H * p->I, L.y, N, p->E, p->H, p->I, v, false);
  if (w4) {  // the tensor scales multiply the fp32 sums in the epilogues
    gu.tscale = w->w_gate_up_tscale;
    dn.tscale = w->w_down_tscale;
  }
  if (w4_deq) {  // bf16 copies [E, 2I, H] and [E, H, I] in the workspace
    gu.W = L.deq_gu;
    dn.W = L.deq_dn;
  }
  if (w4_codes) {  // packed codes (uint16 units between experts) and group-major scales
    gu.W = reinterpret_cast<const uint16_t*>(w->w_gate_up_q);
    gu.w_stride = (int64_t)2 * p->I * p->H / 4;
    gu.S = w->w_gate_up_scale;
    gu.s_stride = (int64_t)(p->H / 128) * 2 * p->I;
    dn.W = reinterpret_cast<const uint16_t*>(w->w_down_q);
    dn.w_stride = (int64_t)p->H * p->I / 4;
    dn.S = w->w_down_scale;
    dn.s_stride = (int64_t)(p->I / 128) * p->H;
    if (v == GemmVariant::kWStream) {  // its own tile width; the ping-pong tile keeps the bf16 one
      gu.ntiles = (p->I + gemm_w4_tile_n(true) - 1) / gemm_w4_tile_n(true);
      dn.ntiles = (p->H + gemm_w4_tile_n(false) - 1) / gemm_w4_tile_n(false);
    }
  }
  GemmProblem sgu = make_problem(xs, nullptr, nullptr, nullptr, w->ws_gate_up, 0, L.hs, T, 1,
                                 p->I_shared, p->H, v, true);
  GemmProblem sdn = make_problem(L.hs, nullptr, nullptr, nullptr, w->ws_down, 0, L.ys, T, 1, p->H,
                                 p->I_shared, v, false);
  // tile-blocked copies of the bf16 experts, for the 256-row tiles (their
  // K stages then are contiguous 16 KB blocks, byte offsets within 4 GiB
  // per expert); other tiles read the rows.  The problems of one launch
  // share their layout: bf16 routed and shared experts take theirs
  // together, a shared expert after the W4A16 code tiles alone
  const bool pipe_tiles = v == GemmVariant::kPingPong || v == GemmVariant::kPipe256W8;
  const bool routed_fits = 2 * pack_experts_elems(1, p->I, p->H, true) <= UINT32_MAX &&
                           2 * pack_experts_elems(1, p->H, p->I, false) <= UINT32_MAX;
  const bool shared_fits = 2 * pack_experts_elems(1, p->I_shared, p->H, true) <= UINT32_MAX &&
                           2 * pack_experts_elems(1, p->H, p->I_shared, false) <= UINT32_MAX;
  const bool shared_alone = shared && w4_codes && v == GemmVariant::kPingPong;
  const bool use_packed = pipe_tiles && packed && routed_fits && shared_fits;
  if (use_packed) {
    gu.W = w->w_gate_up_packed;
    gu.w_stride = pack_experts_elems(1, p->I, p->H, true);
    gu.packed = 1;
    dn.W = w->w_down_packed;
    dn.w_stride = pack_experts_elems(1, p->H, p->I, false);
    dn.packed = 1;
  }
  if (pipe_tiles && packed_s && shared_fits && (use_packed || shared_alone)) {
    sgu.W = w->ws_gate_up_packed;
    sgu.packed = 1;
    sdn.W = w->ws_down_packed;
    sdn.packed = 1;
  }
  // the 256-row tiles pass h (and the shared expert's) from gate_up to down
  // stage-blocked within each tile, so that down reads a K stage of a tile as
  // one contiguous block (the W4A16 code tiles keep h in rows); a caller who
  // reads h or h_shared gets them in rows
  if (pipe_tiles && !(probes && (probes->h || probes->h_shared))) {
    if (!w4_codes) gu.hblk = dn.hblk = 1;
    sgu.hblk = sdn.hblk = 1;
  }
  if (p->scmoe) gu.A = L.xr;
  if (!tiles_fit(gu, shared ? &sgu : nullptr) || !tiles_fit(dn, shared ? &sdn : nullptr))
    return fail(MOE_ERR_UNSUPPORTED, "too many tiles for one launch");

  // Weight streaming (decode-sized batches): the shared expert's two GEMMs
  // run on the second stream, forked at the start, on half of the CUs, while
  // the routing kernels run on the rest; the combine waits for them.
  // MOE_SHARED_BESIDE=0 keeps the shared expert in the routed launches (a
  // tuning lever; the results are the same)
  const char* beside_env = std::getenv("MOE_SHARED_BESIDE");
  const bool beside = shared && v == GemmVariant::kWStream && !one_stream &&
                      !(beside_env && !std::strcmp(beside_env, "0"));
  const bool deq_side = w4_deq && !one_stream;
  SideStream* side = nullptr;
  if ((beside || deq_side) && (s = side_stream(&side)) != MOE_OK) return s;

  auto mark = [&](int ev) -> moe_status {
    if (probes && probes->events[ev])
      return device_status(hipEventRecord(probes->events[ev], stream), "event record");
    return MOE_OK;
  };
  if ((s = mark(MOE_EV_BEGIN)) != MOE_OK) return s;
  if (beside) {
    const int wgs = std::max(8, gemm_cu_count() / 2 / 8 * 8);
    if ((s = device_status(hipEventRecord(side->fork, stream), "fork")) != MOE_OK ||
        (s = device_status(hipStreamWaitEvent(side->stream, side->fork, 0), "fork")) != MOE_OK ||
        (s = device_status(launch_grouped_gemm(v, true, sgu, nullptr, p->swiglu_limit,
                                               side->stream, wgs),
                           "shared gate_up")) != MOE_OK ||
        (s = device_status(launch_grouped_gemm(v, false, sdn, nullptr, p->swiglu_limit,
                                               side->stream, wgs),
                           "shared down")) != MOE_OK ||
        (s = device_status(hipEventRecord(side->join, side->stream), "join")) != MOE_OK)
      return s;
  }
  // W4A16 beyond weight streaming: the experts are dequantised on the
  // second stream, gate_up's while the routing kernels run, down's while the
  // gate_up GEMM runs; each GEMM waits for its own weights
  if (w4_deq && !deq_side &&
      ((s = device_status(launch_w4_dequant(w->w_gate_up_q, w->w_gate_up_scale, nullptr, L.deq_gu, p->E,
                                            (int64_t)2 * p->I, p->H, stream),
                          "dequantise gate_up")) != MOE_OK ||
       (s = device_status(launch_w4_dequant(w->w_down_q, w->w_down_scale, nullptr, L.deq_dn, p->E, p->H,
                                            p->I, stream),
                          "dequantise down")) != MOE_OK))
    return s;
  if (deq_side) {
    if ((s = device_status(hipEventRecord(side->fork, stream), "fork")) != MOE_OK ||
        (s = device_status(hipStreamWaitEvent(side->stream, side->fork, 0), "fork")) != MOE_OK ||
        (s = device_status(launch_w4_dequant(w->w_gate_up_q, w->w_gate_up_scale, nullptr, L.deq_gu, p->E,
                                             (int64_t)2 * p->I, p->H, side->stream),
                           "dequantise gate_up")) != MOE_OK ||
        (s = device_status(hipEventRecord(side->join, side->stream), "join")) != MOE_OK ||
        (s = device_status(launch_w4_dequant(w->w_down_q, w->w_down_scale, nullptr, L.deq_dn, p->E, p->H,
                                             p->I, side->stream),
                           "dequantise down")) != MOE_OK ||
        (s = device_status(hipEventRecord(side->join2, side->stream), "join")) != MOE_OK)
      return s;
  }
  if (p->scmoe) {
    if ((s = device_status(launch_rmsnorm_bf16(x_routed, w->gamma_pre, L.xr, T, p->H, p->norm_eps,
                                               stream),
                           "pre-norm")) != MOE_OK)
      return s;
    xr = L.xr;
  }
  if ((s = mark(MOE_EV_PRENORM)) != MOE_OK) return s;
  if (route_small_fits(T, p->E, p->k)) {
    // decode-sized: the router GEMM, then top-k, permutation and the GEMM's
    // m-tile prefix in one launch (the router event follows both)
    if ((s = device_status(launch_route_small(xr, w->w_router, w->corr_bias, L.logits, L.partial,
                                              L.ids, L.w, T, p->H, p->E, p->k,
                                              p->routed_scaling_factor, L.offsets,
                                              L.sorted_token, L.inv_pos, gemm_tile_m(v), L.mstart,
                                              stream),
                           "routing")) != MOE_OK)
      return s;
    if ((s = mark(MOE_EV_ROUTER)) != MOE_OK) return s;
  } else {
    if ((s = device_status(launch_router(xr, w->w_router, w->corr_bias, L.logits, L.partial,
                                         L.ids, L.w, T, p->H, p->E, p->k,
                                         p->routed_scaling_factor, stream),
                           "router")) != MOE_OK)
      return s;
    if ((s = mark(MOE_EV_ROUTER)) != MOE_OK) return s;
    // the permutation and the grouped GEMM's m-tile prefix (one launch for a
    // batch of at most 4096 pairs)
    if ((s = device_status(launch_permute(L.ids, L.counts, L.starts, L.offsets, L.sorted_token,
                                          L.inv_pos, N, p->E, p->k, gemm_tile_m(v), L.mstart,
                                          stream),
                           "permute")) != MOE_OK)
      return s;
  }
  // (the gate_up weights' dequantisation ends inside the permute step, so
  // the gate_up step times the GEMM alone)
  if (deq_side &&
      (s = device_status(hipStreamWaitEvent(stream, side->join, 0), "join")) != MOE_OK)
    return s;
  if ((s = mark(MOE_EV_PERMUTE)) != MOE_OK) return s;
  // routed and shared problems in one launch; W4A16 routed experts read as
  // codes take a launch of their own, and the bf16 shared expert follows
  const bool one_launch = shared && !beside && !w4_codes;
  const bool after = shared && !beside && w4_codes;
  if ((s = device_status(launch_grouped_gemm(v, true, gu, one_launch ? &sgu : nullptr,
                                             p->swiglu_limit, stream),
                         "gate_up")) != MOE_OK)
    return s;
  if (after && (s = device_status(launch_grouped_gemm(v, true, sgu, nullptr, p->swiglu_limit,
                                                      stream),
                                  "shared gate_up")) != MOE_OK)
    return s;
  if ((s = mark(MOE_EV_GATE_UP)) != MOE_OK) return s;
  if (deq_side &&
      (s = device_status(hipStreamWaitEvent(stream, side->join2, 0), "join")) != MOE_OK)
    return s;
  if ((s = device_status(launch_grouped_gemm(v, false, dn, one_launch ? &sdn : nullptr,
                                             p->swiglu_limit, stream),
                         "down")) != MOE_OK)
    return s;
  if (after && (s = device_status(launch_grouped_gemm(v, false, sdn, nullptr, p->swiglu_limit,
                                                      stream),
                                  "shared down")) != MOE_OK)
    return s;
  if ((s = mark(MOE_EV_DOWN)) != MOE_OK) return s;
  if (beside &&
      (s = device_status(hipStreamWaitEvent(stream, side->join, 0), "join")) != MOE_OK)
    return s;
  const int post = p->scmoe || (fin && fin->post_norm);
  if ((s = device_status(launch_combine(L.y, L.w, L.inv_pos, shared ? L.ys : nullptr,
                                        w->gamma_post, fin ? fin->residual : nullptr,
                                        fin ? fin->out_scale : 1.f,
                                        fin ? fin->residual_scale : 1.f, out, T, p->H, p->k,
                                        post, p->norm_eps, stream),
                         "combine")) != MOE_OK)
    return s;
  if ((s = mark(MOE_EV_COMBINE)) != MOE_OK) return s;
  return ok();
}

}  // namespace

extern "C" {

moe_status moe_combine(const moe_params* p, const float* y_perm, const float* topk_w,
                       const int32_t* inv_pos, const float* y_shared, const float* gamma_post,
                       moe_bf16* out, hipStream_t stream) {
  return combine_impl(p, y_perm, topk_w, inv_pos, y_shared, gamma_post, nullptr, out, stream);
}

moe_status moe_combine_finish(const moe_params* p, const float* y_perm, const float* topk_w,
                              const int32_t* inv_pos, const float* y_shared,
                              const float* gamma_post, const moe_finish* fin, moe_bf16* out,
                              hipStream_t stream) {
  if (!fin) return fail(MOE_ERR_INVALID_ARG, "fin is NULL");
  return combine_impl(p, y_perm, topk_w, inv_pos, y_shared, gamma_post, fin, out, stream);
}

moe_status moe_router_backward_workspace_size(const moe_params* p, size_t* bytes) {
  moe_status s = check_params(p);
  if (s != MOE_OK) return s;
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = router_backward_workspace_bytes(p->T, p->H, p->E);
  return ok();
}

moe_status moe_router_backward(const moe_params* p, const float* grad_logits,
                               int64_t g_row_stride, int64_t g_col_stride, const moe_bf16* x,
                               const float* w_router, moe_bf16* grad_x, float* grad_w,
                               float* grad_b, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status s = check_params(p);
  if (s != MOE_OK) return s;
  if (g_row_stride < 0 || g_col_stride < 0)
    return fail(MOE_ERR_INVALID_ARG, "gradient strides must be >= 0 (%lld, %lld)",
                (long long)g_row_stride, (long long)g_col_stride);
  OPTIONAL_PTR(grad_x);
  OPTIONAL_PTR(grad_w);
  OPTIONAL_PTR(grad_b);
  if (p->T > 0) {
    if (!grad_logits) return fail(MOE_ERR_INVALID_ARG, "grad_logits is NULL");
    if (reinterpret_cast<uintptr_t>(grad_logits) & 3u)
      return fail(MOE_ERR_UNSUPPORTED, "grad_logits is not 4-byte aligned");
    if (grad_x) REQUIRE_PTR(w_router);
    if (grad_w) REQUIRE_PTR(x);
    const size_t need = router_backward_workspace_bytes(p->T, p->H, p->E);
    if (grad_w && need > 0) {
      REQUIRE_PTR(ws);
      if (ws_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
    }
  }
  if (!grad_x && !grad_w && !grad_b) return ok();  // nothing asked for
  if ((s = device_status(launch_router_backward(grad_logits, g_row_stride, g_col_stride, x,
                                                w_router, grad_x, grad_w, grad_b, p->T, p->H,
                                                p->E, ws, stream),
                         "router backward")) != MOE_OK)
    return s;
  return ok();
}

moe_status moe_w4_dequantize(const uint8_t* q, const uint8_t* scale, const float* tscale,
                             int32_t n_groups, int64_t rows, int32_t K, moe_bf16* out,
                             hipStream_t stream) {
  if (n_groups < 0 || rows < 0 || K < 0)
    return fail(MOE_ERR_INVALID_ARG, "negative size (n_groups %d, rows %lld, K %d)", n_groups,
                (long long)rows, K);
  if (K % 128 != 0) return fail(MOE_ERR_UNSUPPORTED, "K = %d is not a multiple of 128", K);
  if ((int64_t)n_groups * rows >= kMaxPairs)
    return fail(MOE_ERR_UNSUPPORTED, "n_groups * rows = %lld >= 2^31",
                (long long)((int64_t)n_groups * rows));
  if (n_groups == 0 || rows == 0 || K == 0) return ok();
  REQUIRE_PTR(q);
  REQUIRE_PTR(scale);
  REQUIRE_PTR(out);
  if (reinterpret_cast<uintptr_t>(tscale) & 3u)
    return fail(MOE_ERR_UNSUPPORTED, "tscale is not 4-byte aligned");
  moe_status s;
  if ((s = device_status(launch_w4_dequant(q, scale, tscale, out, n_groups, rows, K, stream),
                         "dequantise")) != MOE_OK)
    return s;
  return ok();
}

moe_status moe_packed_experts_size(const moe_params* p, int64_t* gate_up_elems,
                                   int64_t* down_elems) {
  moe_status s = check_params(p);
  if (s != MOE_OK) return s;
  if (!gate_up_elems || !down_elems) return fail(MOE_ERR_INVALID_ARG, "output pointer is NULL");
  if (p->H % 32 || p->I % 32)
    return fail(MOE_ERR_UNSUPPORTED, "packed experts need H and I multiples of 32");
  *gate_up_elems = pack_experts_elems(p->E, p->I, p->H, true);
  *down_elems = pack_experts_elems(p->E, p->H, p->I, false);
  return ok();
}

moe_status moe_pack_experts(const moe_params* p, const moe_bf16* w_gate_up, const moe_bf16* w_down,
                            moe_bf16* gate_up_packed, moe_bf16* down_packed, hipStream_t stream) {
  int64_t gu = 0, dn = 0;
  moe_status s = moe_packed_experts_size(p, &gu, &dn);
  if (s != MOE_OK) return s;
  REQUIRE_PTR(w_gate_up);
  REQUIRE_PTR(w_down);
  REQUIRE_PTR(gate_up_packed);
  REQUIRE_PTR(down_packed);
  // one workgroup per 256 x 32 block: the grid's x dimension bounds the count
  if (gu / (256 * 32) > INT32_MAX || dn / (256 * 32) > INT32_MAX)
    return fail(MOE_ERR_UNSUPPORTED, "experts too large to pack in one launch");
  if ((s = device_status(launch_pack_experts(w_gate_up, gate_up_packed, p->E, p->I, p->H, true,
                                             stream),
                         "pack gate_up")) != MOE_OK ||
      (s = device_status(launch_pack_experts(w_down, down_packed, p->E, p->H, p->I, false,
                                             stream),
                         "pack down")) != MOE_OK)
    return s;
  return ok();
}

moe_status moe_probe_mfma_bf16(int32_t workgroups, int32_t iters, float* sink, double* flops,
                               hipStream_t stream) {
  if (workgroups < 1 || iters < 1)
    return fail(MOE_ERR_INVALID_ARG, "workgroups = %d, iters = %d must be >= 1", workgroups,
                iters);
  REQUIRE_PTR(sink);
  if (!flops) return fail(MOE_ERR_INVALID_ARG, "flops is NULL");
  moe_status s;
  if ((s = device_status(launch_probe_mfma(workgroups, iters, sink, stream), "mfma probe")) !=
      MOE_OK)
    return s;
  *flops = probe_mfma_flops(workgroups, iters);
  return ok();
}

moe_status moe_probe_hbm_read(const void* src, int64_t bytes, int32_t workgroups,
                              uint32_t* sink, hipStream_t stream) {
  if (workgroups < 1 || bytes < 16 || bytes % 16)
    return fail(MOE_ERR_INVALID_ARG, "bytes = %lld must be a positive multiple of 16, "
                "workgroups = %d >= 1", (long long)bytes, workgroups);
  REQUIRE_PTR(src);
  REQUIRE_PTR(sink);
  moe_status s;
  if ((s = device_status(launch_probe_read(src, bytes, workgroups, sink, stream), "read probe")) !=
      MOE_OK)
    return s;
  return ok();
}

moe_status moe_forward(const moe_params* p, const moe_bf16* x_routed, const moe_bf16* x_shared,
                       const moe_weights* w, moe_bf16* out, const moe_probes* probes, void* ws,
                       size_t ws_bytes, hipStream_t stream) {
  return forward_impl(p, x_routed, x_shared, w, nullptr, out, probes, ws, ws_bytes, stream);
}

moe_status moe_forward_finish(const moe_params* p, const moe_bf16* x_routed,
                              const moe_bf16* x_shared, const moe_weights* w,
                              const moe_finish* fin, moe_bf16* out, const moe_probes* probes,
                              void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!fin) return fail(MOE_ERR_INVALID_ARG, "fin is NULL");
  return forward_impl(p, x_routed, x_shared, w, fin, out, probes, ws, ws_bytes, stream);
}

static_assert(MOE_NOALLOC_SCRATCH_BYTES == MOE_NOALLOC_SCRATCH_BYTES_DEV, "scratch size");

moe_status moe_forward_noalloc(const moe_params* p, const moe_bf16* x_routed,
                               const moe_bf16* x_shared, const moe_weights* w, moe_bf16* out,
                               const moe_probes* probes, hipStream_t stream) {
  moe_status s = check_params(p);
  if (s != MOE_OK) return s;
  const size_t need = carve(*p, nullptr).bytes;
  if (need > MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_ERR_WORKSPACE,
                "this call needs %zu bytes of scratch; the fixed scratch holds %zu "
                "(moe_forward takes a workspace of any size)",
                need, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
  void* scratch = nullptr;
  size_t bytes = 0;
  if ((s = device_status(noalloc_scratch(&scratch, &bytes), "fixed scratch address")) != MOE_OK)
    return s;
  return forward_impl(p, x_routed, x_shared, w, nullptr, out, probes, scratch, bytes, stream,
                      /*one_stream=*/true);
}

}  // extern "C"
