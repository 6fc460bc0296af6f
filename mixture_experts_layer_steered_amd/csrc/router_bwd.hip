// Backward of the router gating GEMM on gfx950 (training path).
//
// Forward: l = x @ W_r^T (+ b) in the router dtype, fp32, with fp32 router
// weights and bf16 activations whose saved copy keeps its bf16 dtype
// ("bridge.models.beam.modeling_beam", _BeamRouterGatingLinear).  Its
// backward for an upstream gradient dL [T, E]:
//   grad_x = bf16(fp32(dL @ W_r))      [T, H]  (the input's dtype)
//   grad_W = fp32(dL^T @ x)            [E, H]
//   grad_b = fp32(sum_t dL[t, :])      [E]
// Both GEMMs run on fp32 matrix cores (v_mfma_f32_32x32x2_f32): every
// product is exact in fp32 (a bf16 x widens exactly), so the results equal
// fp32 GEMMs up to summation order.  The page's second concern -- an
// expanded, stride-0 gradient (e.g. of logits.sum()) read as raw storage by
// a GEMM that ignores strides -- does not arise: dL is read through its row
// and column strides (in elements, 0 allowed) as it comes.
//
// grad_x: 64 x 128 output tiles, K = E in steps of 32.  grad_W: 64 x 128
// tiles of [E, H], the token dimension split into slices whose partial sums
// go to a workspace and are added in slice order by a second kernel (no
// atomics: reruns repeat bit for bit).  grad_b comes with grad_W: the
// workgroups of the first hidden tile also sum their slice's dL columns as
// they load them (each thread a fixed quarter of a column's tokens, the four
// quarters added in order at the end), and the same reduction adds the
// slices; alone it is one workgroup per expert with a fixed-order sum.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int RB_BM = 64;   // output rows per tile (tokens for grad_x, experts for grad_W)
constexpr int RB_BN = 128;  // output columns per tile (hidden)
constexpr int RB_BK = 32;   // K per LDS step
constexpr int RB_LDA = RB_BM + 1;   // padded LDS rows
constexpr int RB_LDB = RB_BN + 4;

// 64 x 128 tile = 2 x 2 wavefronts of 32 x 64 (two 32 x 32 MFMA blocks).
// A is held in LDS as As[k][m] (m = output row), B as Bs[k][n]; lane l of a
// v_mfma_f32_32x32x2_f32 supplies A[m = l % 32][k = l / 32] and B[k = l / 32]
// [n = l % 32]; the accumulator element r of lane l is row
// 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32 of the block.
__device__ __forceinline__ void rb_mfma_step(const float* As, const float* Bs, int wm, int wn,
                                             int lane, f32x16_t (&acc)[2]) {
#pragma unroll
  for (int kk = 0; kk < RB_BK; kk += 2) {
    const int k = kk + (lane >> 5);
    const float a = As[k * RB_LDA + wm * 32 + (lane & 31)];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const float bv = Bs[k * RB_LDB + wn * 64 + b * 32 + (lane & 31)];
      acc[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, bv, acc[b], 0, 0, 0);
    }
  }
}

// grad_x[t, h] = bf16(sum_e dL[t, e] W[e, h]).  Grid (ceil(T/64), ceil(H/128)):
// token tiles on x (no 65535 bound), neighbours share a W column block.
__global__ __launch_bounds__(256) void router_bwd_dx_kernel(
    const float* __restrict__ dl, int64_t rs, int64_t cs, const float* __restrict__ w,
    uint16_t* __restrict__ gx, int64_t T, int H, int E) {
  __shared__ float As[RB_BK * RB_LDA];  // As[e][t]
  __shared__ float Bs[RB_BK * RB_LDB];  // Bs[e][h]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t t0 = (int64_t)blockIdx.x * RB_BM;
  const int h0 = blockIdx.y * RB_BN;
  f32x16_t acc[2];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[b][r] = 0.f;

  for (int e0 = 0; e0 < E; e0 += RB_BK) {
    float av[8];
#pragma unroll
    for (int n = 0; n < 8; ++n) {  // dL tile: 64 tokens x 32 experts
      const int q = tid + 256 * n, tt = q >> 5, ee = q & 31;
      const int64_t t = t0 + tt;
      av[n] = (t < T && e0 + ee < E) ? dl[t * rs + (int64_t)(e0 + ee) * cs] : 0.f;
    }
    float4 bv[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) {  // W tile: 32 experts x 128 hidden
      const int q = tid + 256 * n, kk = q >> 5, c4 = q & 31;
      const int h = h0 + 4 * c4;
      bv[n] = (e0 + kk < E && h < H)
                  ? *reinterpret_cast<const float4*>(w + (int64_t)(e0 + kk) * H + h)
                  : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __syncthreads();
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const int q = tid + 256 * n;
      As[(q & 31) * RB_LDA + (q >> 5)] = av[n];
    }
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int q = tid + 256 * n;
      *reinterpret_cast<float4*>(&Bs[(q >> 5) * RB_LDB + 4 * (q & 31)]) = bv[n];
    }
    __syncthreads();
    rb_mfma_step(As, Bs, wm, wn, lane, acc);
  }
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int h = h0 + wn * 64 + b * 32 + (lane & 31);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t t = t0 + wm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (t < T && h < H) gx[t * H + h] = (uint16_t)f32_to_bf16_bits(acc[b][r]);
    }
  }
}

// part[s][e, h] = sum over the tokens of slice s of dL[t, e] x[t, h], and,
// with part_b, part_b[s][e] = sum over the slice of dL[t, e].
// Grid (ceil(H/128), ceil(E/64), slices); with one slice the outputs are
// grad_W and grad_b themselves.
__global__ __launch_bounds__(256) void router_bwd_dw_kernel(
    const float* __restrict__ dl, int64_t rs, int64_t cs, const uint16_t* __restrict__ x,
    float* __restrict__ part, float* __restrict__ part_b, int64_t T, int H, int E,
    int64_t slice) {
  __shared__ float As[RB_BK * RB_LDA];  // As[t][e]
  __shared__ float Bs[RB_BK * RB_LDB];  // Bs[t][h]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int e0 = blockIdx.y * RB_BM;
  const int h0 = blockIdx.x * RB_BN;
  const int64_t tb = (int64_t)blockIdx.z * slice;
  const int64_t te = tb + slice < T ? tb + slice : T;
  f32x16_t acc[2];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[b][r] = 0.f;
  const bool bias = part_b != nullptr && blockIdx.x == 0;  // uniform
  // thread tid's dL loads all fall in expert column e0 + (tid & 63): it sums
  // them (tokens t = tid / 64 mod 4 of each step, in order)
  float bsum = 0.f;

  for (int64_t t0 = tb; t0 < te; t0 += RB_BK) {
    float av[8];
#pragma unroll
    for (int n = 0; n < 8; ++n) {  // dL tile: 32 tokens x 64 experts
      const int q = tid + 256 * n, tt = q >> 6, ee = q & 63;
      const int64_t t = t0 + tt;
      av[n] = (t < te && e0 + ee < E) ? dl[t * rs + (int64_t)(e0 + ee) * cs] : 0.f;
    }
    if (bias)
#pragma unroll
      for (int n = 0; n < 8; ++n) bsum += av[n];
    uint4 xv[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) {  // x tile: 32 tokens x 128 hidden, 8 bf16 per load
      const int q = tid + 256 * n, tt = q >> 4, c8 = q & 15;
      const int64_t t = t0 + tt;
      const int h = h0 + 8 * c8;
      xv[n] = (t < te && h < H) ? *reinterpret_cast<const uint4*>(x + t * H + h)
                                : make_uint4(0, 0, 0, 0);
    }
    __syncthreads();
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const int q = tid + 256 * n;
      As[(q >> 6) * RB_LDA + (q & 63)] = av[n];
    }
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int q = tid + 256 * n, tt = q >> 4, c8 = q & 15;
      float* dst = &Bs[tt * RB_LDB + 8 * c8];
      const uint32_t u[4] = {xv[n].x, xv[n].y, xv[n].z, xv[n].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        dst[2 * j] = bf16_bits_to_f32(u[j] & 0xffffu);
        dst[2 * j + 1] = bf16_bits_to_f32(u[j] >> 16);
      }
    }
    __syncthreads();
    rb_mfma_step(As, Bs, wm, wn, lane, acc);
  }
  if (bias) {  // the four quarters of each column, in order
    __syncthreads();
    As[tid] = bsum;
    __syncthreads();
    if (tid < RB_BM && e0 + tid < E)
      part_b[(int64_t)blockIdx.z * E + e0 + tid] =
          ((As[tid] + As[tid + 64]) + As[tid + 128]) + As[tid + 192];
  }
  float* out = part + (int64_t)blockIdx.z * E * H;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int h = h0 + wn * 64 + b * 32 + (lane & 31);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int e = e0 + wm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (e < E && h < H) out[(int64_t)e * H + h] = acc[b][r];
    }
  }
}

// grad_W = sum of the slices' partials in slice order, four values a
// thread; with part_b, grad_b likewise (threads below E).
__global__ __launch_bounds__(256) void router_bwd_dw_reduce_kernel(
    const float* __restrict__ part, float* __restrict__ gw, const float* __restrict__ part_b,
    float* __restrict__ gb, int E, int64_t n4, int64_t stride4, int slices) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (part_b != nullptr && i < E) {
    float sb = part_b[i];
#pragma unroll 8
    for (int k = 1; k < slices; ++k) sb += part_b[(int64_t)k * E + i];
    gb[i] = sb;
  }
  if (i >= n4) return;
  const float4* p = reinterpret_cast<const float4*>(part);
  float4 s = p[i];
#pragma unroll 8
  for (int k = 1; k < slices; ++k) {
    const float4 v = p[i + k * stride4];
    s.x += v.x;
    s.y += v.y;
    s.z += v.z;
    s.w += v.w;
  }
  reinterpret_cast<float4*>(gw)[i] = s;
}

// grad_b[e] = sum_t dL[t, e]: one workgroup per expert; thread j sums the
// tokens t = j (mod 256) in order, then a fixed tree over the threads.
__global__ __launch_bounds__(256) void router_bwd_db_kernel(
    const float* __restrict__ dl, int64_t rs, int64_t cs, float* __restrict__ gb, int64_t T) {
  __shared__ float red[256];
  const int e = blockIdx.x;
  float s = 0.f;
  for (int64_t t = threadIdx.x; t < T; t += 256) s += dl[t * rs + (int64_t)e * cs];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) gb[e] = red[0];
}

// zero n floats (an empty batch's grad_W and grad_b)
__global__ __launch_bounds__(256) void router_bwd_zero_kernel(float* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

// token slices for grad_W: enough workgroups to cover the device about four
// times over, each slice a whole number of K steps
int dw_slices(int64_t T, int H, int E, int64_t* slice) {
  const int64_t tiles = (int64_t)((E + RB_BM - 1) / RB_BM) * ((H + RB_BN - 1) / RB_BN);
  const int64_t steps = (T + RB_BK - 1) / RB_BK;
  int64_t s = (1024 + tiles - 1) / tiles;
  if (s > steps) s = steps;
  if (s > 64) s = 64;
  if (s < 1) s = 1;
  const int64_t per = (steps + s - 1) / s;
  *slice = per * RB_BK;
  return (int)((steps + per - 1) / per);
}

}  // namespace

// workspace: the slices' grad_W partials, then their grad_b partials
size_t dw_part_bytes(int s, int H, int E) {
  return ((size_t)s * E * H * sizeof(float) + 255) / 256 * 256;
}

size_t router_backward_workspace_bytes(int64_t T, int H, int E) {
  int64_t slice = 0;
  const int s = dw_slices(T, H, E, &slice);
  return s > 1 ? dw_part_bytes(s, H, E) + (size_t)s * E * sizeof(float) : 0;
}

hipError_t launch_router_backward(const float* dl, int64_t rs, int64_t cs, const uint16_t* x,
                                  const float* w, uint16_t* gx, float* gw, float* gb, int64_t T,
                                  int H, int E, void* ws, hipStream_t stream) {
  if (T == 0) {
    // an empty batch still defines grad_W = 0 and grad_b = 0 (a fill kernel:
    // the call may be captured in a graph)
    const int64_t nw = (int64_t)E * H;
    if (gw)
      hipLaunchKernelGGL(router_bwd_zero_kernel, dim3((unsigned)((nw + 255) / 256)), dim3(256), 0,
                         stream, gw, nw);
    if (gb)
      hipLaunchKernelGGL(router_bwd_zero_kernel, dim3((unsigned)((E + 255) / 256)), dim3(256), 0,
                         stream, gb, (int64_t)E);
    return hipGetLastError();
  }
  if (gx)
    hipLaunchKernelGGL(router_bwd_dx_kernel,
                       dim3((unsigned)((T + RB_BM - 1) / RB_BM), (unsigned)((H + RB_BN - 1) / RB_BN)),
                       dim3(256), 0, stream, dl, rs, cs, w, gx, T, H, E);
  if (gw) {
    int64_t slice = 0;
    const int s = dw_slices(T, H, E, &slice);
    float* part = s > 1 ? static_cast<float*>(ws) : gw;
    float* part_b =
        gb ? (s > 1 ? reinterpret_cast<float*>(static_cast<char*>(ws) + dw_part_bytes(s, H, E)) : gb)
           : nullptr;
    hipLaunchKernelGGL(router_bwd_dw_kernel,
                       dim3((unsigned)((H + RB_BN - 1) / RB_BN), (unsigned)((E + RB_BM - 1) / RB_BM),
                            (unsigned)s),
                       dim3(256), 0, stream, dl, rs, cs, x, part, part_b, T, H, E, slice);
    if (s > 1) {
      const int64_t n4 = (int64_t)E * H / 4;
      hipLaunchKernelGGL(router_bwd_dw_reduce_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256),
                         0, stream, part, gw, part_b, gb, E, n4, n4, s);
    }
  } else if (gb) {
    hipLaunchKernelGGL(router_bwd_db_kernel, dim3((unsigned)E), dim3(256), 0, stream, dl, rs, cs,
                       gb, T);
  }
  return hipGetLastError();
}
