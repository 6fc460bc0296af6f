// Router of the routed-MoE layer on gfx950: fp32 logits, sigmoid scores, a
// selection-only correction bias, and a wavefront top-k.
//
// Logits.  The router runs in fp32 with fp32 weights against bf16
// activations ("bridge.models.beam.modeling_beam", beam_router_gating_linear
// and BeamTopKRouter).  A bf16 activation times an fp32 weight is computed
// exactly on bf16 matrix cores by splitting each fp32 weight w into three
// bf16 pieces w = hi + mid + lo (8 + 8 + 8 significant bits, each piece the
// truncation of what is left, so the split is exact); each bf16 x bf16
// product is exact in fp32 and the MFMA sums them with fp32 accumulation.
// The logits therefore equal an fp32 GEMM up to summation order, at the
// rate of three bf16 MFMAs instead of one fp32 MFMA of a quarter the K.
//
// Top-k (topk.h).  s = sigmoid(l) (evaluated in fp64, rounded once to
// fp32), s' = s + b in fp32, and the k largest s' over all E experts are
// chosen, ties to the lower expert id, NaN below every number; the ids are
// written in ascending order with weight rsf * s ("Module glm5next_mlp",
// section "Numerics the kernels rely on"; Constants, KERNEL_MAX_TOP_K).  One
// wavefront ranks one token: each lane holds up to 16 experts as 64-bit
// keys (orderable score bits, inverted id) and k wave-wide arg-max rounds
// pick the winners.
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "permute_small.h"
#include "topk.h"

namespace {

constexpr int RT_BT = 64;       // tokens per workgroup tile
constexpr int RT_BE = 64;       // experts per workgroup tile
constexpr int RT_BK = 64;       // K per LDS stage
constexpr int RT_LD = RT_BK + 8;  // padded LDS row (bf16 elements): 144 bytes
constexpr int RT_MAX_SPLITS = 16; // K slices of the router GEMM at most
constexpr int RT_DEPTH = 2;       // K steps in flight per workgroup

__device__ __forceinline__ void split3(float w, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  uint32_t u = __float_as_uint(w);
  uint32_t h = u & 0xffff0000u;
  float r1 = w - __uint_as_float(h);          // exact: the 16 bits below hi
  uint32_t m = __float_as_uint(r1) & 0xffff0000u;
  float r2 = r1 - __uint_as_float(m);         // exact: at most 8 bits left
  hi = h >> 16;
  mid = m >> 16;
  lo = __float_as_uint(r2) >> 16;             // exact in bf16
}

// partial[s][T, E] = fp32(x[T, K_s] @ w[E, K_s]^T) over the s-th K slice of
// k_slice columns.  Grid: (ceil(T/64), ceil(E/64), splits).  With one split
// the partial is the logit itself.
__global__ __launch_bounds__(256) void router_logits_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ w, float* __restrict__ partial,
    int64_t T, int H, int E, int k_slice) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[RT_BT * RT_LD];
  __shared__ __attribute__((aligned(16))) uint16_t wsp[3][RT_BE * RT_LD];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t t0 = (int64_t)blockIdx.x * RT_BT;
  const int e0 = blockIdx.y * RT_BE;

  f32x16_t acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;

  // x tile: 64 rows x 64 k = 512 chunks of 8 bf16, two per thread
  constexpr int XQ = RT_BT * RT_BK / 8 / 256, WQ = RT_BE * RT_BK / 4 / 256;
  int xr_[XQ], xc_[XQ];
#pragma unroll
  for (int q = 0; q < XQ; ++q) {
    const int idx = tid + q * 256;
    xr_[q] = idx / (RT_BK / 8);
    xc_[q] = (idx % (RT_BK / 8)) * 8;
  }
  // w tile: 64 rows x 64 k = 1024 float4, four per thread
  int wr_[WQ], wc_[WQ];
#pragma unroll
  for (int q = 0; q < WQ; ++q) {
    const int idx = tid + q * 256;
    wr_[q] = idx / (RT_BK / 4);
    wc_[q] = (idx % (RT_BK / 4)) * 4;
  }
  const int k_begin = blockIdx.z * k_slice;
  const int k_end = min(H, k_begin + k_slice);
  const int nit = k_end > k_begin ? (k_end - k_begin + RT_BK - 1) / RT_BK : 0;
  float* __restrict__ logits = partial + (int64_t)blockIdx.z * T * E;

  // K steps go through a ring of RT_DEPTH register buffers: the loads of
  // step it + RT_DEPTH are issued as soon as step it is in LDS, so a slice
  // pays about one memory round trip instead of one per step
  uint4 xv[RT_DEPTH][XQ];
  float4 wv[RT_DEPTH][WQ];
  auto load = [&](int it, auto d_c) __attribute__((always_inline)) {
    constexpr int d = decltype(d_c)::value;
    const int k0 = k_begin + it * RT_BK;
#pragma unroll
    for (int q = 0; q < XQ; ++q) {
      xv[d][q] = make_uint4(0, 0, 0, 0);
      if (t0 + xr_[q] < T && k0 + xc_[q] < k_end)
        xv[d][q] = *reinterpret_cast<const uint4*>(x + (t0 + xr_[q]) * (int64_t)H + k0 + xc_[q]);
    }
#pragma unroll
    for (int q = 0; q < WQ; ++q) {
      wv[d][q] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (e0 + wr_[q] < E && k0 + wc_[q] < k_end)
        wv[d][q] = *reinterpret_cast<const float4*>(w + (int64_t)(e0 + wr_[q]) * H + k0 + wc_[q]);
    }
  };
  auto step = [&](int it, auto d_c) __attribute__((always_inline)) {
    constexpr int d = decltype(d_c)::value;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < XQ; ++q) *reinterpret_cast<uint4*>(&xs[xr_[q] * RT_LD + xc_[q]]) = xv[d][q];
#pragma unroll
    for (int q = 0; q < WQ; ++q) {
      uint32_t h[4], m[4], l[4];
      split3(wv[d][q].x, h[0], m[0], l[0]);
      split3(wv[d][q].y, h[1], m[1], l[1]);
      split3(wv[d][q].z, h[2], m[2], l[2]);
      split3(wv[d][q].w, h[3], m[3], l[3]);
      const int o = wr_[q] * RT_LD + wc_[q];
      *reinterpret_cast<uint2*>(&wsp[0][o]) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
      *reinterpret_cast<uint2*>(&wsp[1][o]) = make_uint2(m[0] | (m[1] << 16), m[2] | (m[3] << 16));
      *reinterpret_cast<uint2*>(&wsp[2][o]) = make_uint2(l[0] | (l[1] << 16), l[2] | (l[3] << 16));
    }
    __syncthreads();
    if (it + RT_DEPTH < nit) load(it + RT_DEPTH, d_c);
#pragma unroll
    for (int ks = 0; ks < RT_BK / 16; ++ks) {
      const int kk = ks * 16 + (lane >> 5) * 8;
      bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(&xs[(wm * 32 + (lane & 31)) * RT_LD + kk]);
      const int bo = (wn * 32 + (lane & 31)) * RT_LD + kk;
      bf16x8_t b2 = *reinterpret_cast<const bf16x8_t*>(&wsp[2][bo]);
      bf16x8_t b1 = *reinterpret_cast<const bf16x8_t*>(&wsp[1][bo]);
      bf16x8_t b0 = *reinterpret_cast<const bf16x8_t*>(&wsp[0][bo]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b2, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b1, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b0, acc, 0, 0, 0);
    }
  };
  using D0 = std::integral_constant<int, 0>;
  using D1 = std::integral_constant<int, 1>;
  static_assert(RT_DEPTH == 2, "the ring below is unrolled for two buffers");
  if (0 < nit) load(0, D0{});
  if (1 < nit) load(1, D1{});
  for (int it0 = 0; it0 < nit; it0 += RT_DEPTH) {
    step(it0, D0{});
    if (it0 + 1 < nit) step(it0 + 1, D1{});
  }
  // 32x32 accumulator: lane holds column (lane & 31), rows 8*(r/4) + 4*(lane/32) + r%4
  const int col = e0 + wn * 32 + (lane & 31);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    int64_t row = t0 + wm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    if (row < T && col < E) logits[row * E + col] = acc[r];
  }
}

// One wavefront per token.  Grid: ceil(T/4) workgroups of 256.
template <int TK_PER_LANE>
__global__ __launch_bounds__(256) void router_topk_kernel(
    const float* __restrict__ partial, int splits, float* __restrict__ logits,
    const float* __restrict__ bias, int32_t* __restrict__ ids, float* __restrict__ wts,
    int64_t T, int E, int k, float rsf) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  topk_token<TK_PER_LANE>(partial, splits, logits, bias, ids, wts, t, T, E, k, rsf, lane);
}

// Routing of a batch small enough for one workgroup (decode): the logits'
// K-slice partials are summed (in slice order, as the top-k kernel sums
// them) into LDS, each wavefront ranks tokens from those LDS-staged logits,
// the picks go to LDS as well, and the same workgroup then permutes the
// pairs and writes the grouped GEMM's m-tile prefix -- one launch after the
// router GEMM instead of two.  The LDS of the logits is reused for the
// permute's histograms.
constexpr int RS_MAX_LOGITS = 16384;  // T * E staged in LDS
constexpr int RS_LDS_WORDS =
    RS_MAX_LOGITS > PM_WAVES * MOE_MAX_EXPERTS_DEV ? RS_MAX_LOGITS : PM_WAVES * MOE_MAX_EXPERTS_DEV;

// Workgroup barrier without a memory fence: LDS visibility comes from the
// lgkmcnt(0) wait before it, and global stores still in flight are not
// waited for (nothing in the workgroup reads them back).
__device__ __forceinline__ void rs_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int TK_PER_LANE>
__global__ __launch_bounds__(PM_THREADS) void route_small_kernel(
    const float* __restrict__ partial, int splits, float* __restrict__ logits,
    const float* __restrict__ bias, int32_t* __restrict__ ids, float* __restrict__ wts, int T,
    int E, int k, float rsf, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_token,
    int32_t* __restrict__ inv_pos, int bm, int32_t* __restrict__ mstart) {
  __shared__ __attribute__((aligned(16))) int32_t lds[RS_LDS_WORDS];
  __shared__ int32_t ids_lds[PM_TILE];
  __shared__ int32_t wsum[2 * PM_WAVES];
  float* lg_lds = reinterpret_cast<float*>(lds);
  const int TE = T * E;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // the biases of this lane's experts, loaded once (in flight with the
  // partials) for every token the wave ranks
  float bv[TK_PER_LANE];
  topk_bias<TK_PER_LANE>(bias, E, lane, bv);
  // logits: slice partials summed in slice order; two elements per thread
  // and pass, their 2 x RT_MAX_SPLITS loads in flight together.  The loads
  // are unconditional (indices past the slices or past T*E are clamped to
  // valid ones and their values dropped), so they issue back to back.
  static_assert(RT_MAX_SPLITS == 16, "one pass over the slices");
  for (int i0 = threadIdx.x; i0 < TE; i0 += 2 * PM_THREADS) {
    const int i1 = i0 + PM_THREADS < TE ? i0 + PM_THREADS : i0;
    float p0[RT_MAX_SPLITS], p1[RT_MAX_SPLITS];
#pragma unroll
    for (int u = 0; u < RT_MAX_SPLITS; ++u) {
      const int64_t su = u < splits ? u : splits - 1;
      p0[u] = partial[su * TE + i0];
      p1[u] = partial[su * TE + i1];
    }
    float l0 = p0[0], l1 = p1[0];
#pragma unroll
    for (int u = 1; u < RT_MAX_SPLITS; ++u) {
      if (u < splits) {
        l0 += p0[u];
        l1 += p1[u];
      }
    }
    lg_lds[i0] = l0;
    if (splits > 1) logits[i0] = l0;
    if (i0 + PM_THREADS < TE) {
      lg_lds[i1] = l1;
      if (splits > 1) logits[i1] = l1;
    }
  }
  // the logits in LDS everywhere (the global copies need not have landed)
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  rs_barrier();
  for (int t = wave; t < T; t += PM_WAVES) {
    float lg[TK_PER_LANE];
#pragma unroll
    for (int i = 0; i < TK_PER_LANE; ++i) {
      const int e = lane + 64 * i;
      lg[i] = e < E ? lg_lds[t * E + e] : 0.f;
    }
    topk_select<TK_PER_LANE>(lg, bv, ids, wts, ids_lds, t, E, k, rsf, lane);
  }
  // the picks in LDS everywhere (their global copies need not have landed)
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  rs_barrier();
  permute_small_body(ids_lds, offsets, sorted_token, inv_pos, (int64_t)T * k, E, k, bm, mstart,
                     lds, wsum);
}

}  // namespace

int router_splits(int64_t T, int H, int E) {
  // enough workgroups to cover the chip (about two per CU), each slice a
  // multiple of the 64-wide K step
  const int64_t tiles = ((T + RT_BT - 1) / RT_BT) * ((E + RT_BE - 1) / RT_BE);
  if (tiles == 0) return 1;
  int64_t s = (512 + tiles - 1) / tiles;
  const int64_t max_s = (H + 63) / 64;
  if (s > max_s) s = max_s;
  if (s > RT_MAX_SPLITS) s = RT_MAX_SPLITS;
  return s < 1 ? 1 : (int)s;
}

static hipError_t launch_router_logits(const uint16_t* x, const float* w, float* logits,
                                       float* partial, int64_t T, int H, int E,
                                       hipStream_t stream) {
  const int splits = router_splits(T, H, E);
  int k_slice = (H + splits - 1) / splits;
  k_slice = (k_slice + RT_BK - 1) / RT_BK * RT_BK;
  float* part = splits > 1 ? partial : logits;
  dim3 grid((unsigned)((T + RT_BT - 1) / RT_BT), (unsigned)((E + RT_BE - 1) / RT_BE), splits);
  hipLaunchKernelGGL(router_logits_kernel, grid, dim3(256), 0, stream, x, w, part, T, H, E,
                     k_slice);
  return hipGetLastError();
}

hipError_t launch_router(const uint16_t* x, const float* w, const float* bias, float* logits,
                         float* partial, int32_t* ids, float* wts, int64_t T, int H, int E, int k,
                         float rsf, hipStream_t stream) {
  hipError_t e = launch_router_logits(x, w, logits, partial, T, H, E, stream);
  if (e != hipSuccess) return e;
  const int splits = router_splits(T, H, E);
  float* part = splits > 1 ? partial : logits;
  const dim3 g((unsigned)((T + 3) / 4)), b(256);
  if (E <= 64)
    hipLaunchKernelGGL(router_topk_kernel<1>, g, b, 0, stream, part, splits, logits, bias, ids, wts, T, E, k, rsf);
  else if (E <= 128)
    hipLaunchKernelGGL(router_topk_kernel<2>, g, b, 0, stream, part, splits, logits, bias, ids, wts, T, E, k, rsf);
  else if (E <= 256)
    hipLaunchKernelGGL(router_topk_kernel<4>, g, b, 0, stream, part, splits, logits, bias, ids, wts, T, E, k, rsf);
  else if (E <= 512)
    hipLaunchKernelGGL(router_topk_kernel<8>, g, b, 0, stream, part, splits, logits, bias, ids, wts, T, E, k, rsf);
  else
    hipLaunchKernelGGL(router_topk_kernel<16>, g, b, 0, stream, part, splits, logits, bias, ids, wts, T, E, k, rsf);
  return hipGetLastError();
}

bool route_small_fits(int64_t T, int E, int k) {
  return T * k <= PM_TILE && T * E <= RS_MAX_LOGITS;
}

hipError_t launch_route_small(const uint16_t* x, const float* w, const float* bias, float* logits,
                              float* partial, int32_t* ids, float* wts, int64_t T, int H, int E,
                              int k, float rsf, int32_t* offsets, int32_t* sorted_token,
                              int32_t* inv_pos, int bm, int32_t* mstart, hipStream_t stream) {
  hipError_t e = launch_router_logits(x, w, logits, partial, T, H, E, stream);
  if (e != hipSuccess) return e;
  const int splits = router_splits(T, H, E);
  float* part = splits > 1 ? partial : logits;
  const int bmv = bm > 0 ? bm : 1;
  const int Ti = (int)T;
#define MOE_ROUTE_SMALL(TK)                                                                      \
  hipLaunchKernelGGL(route_small_kernel<TK>, dim3(1), dim3(PM_THREADS), 0, stream, part, splits, \
                     logits, bias, ids, wts, Ti, E, k, rsf, offsets, sorted_token, inv_pos, bmv,  \
                     mstart)
  if (E <= 64)
    MOE_ROUTE_SMALL(1);
  else if (E <= 128)
    MOE_ROUTE_SMALL(2);
  else if (E <= 256)
    MOE_ROUTE_SMALL(4);
  else if (E <= 512)
    MOE_ROUTE_SMALL(8);
  else
    MOE_ROUTE_SMALL(16);
#undef MOE_ROUTE_SMALL
  return hipGetLastError();
}
