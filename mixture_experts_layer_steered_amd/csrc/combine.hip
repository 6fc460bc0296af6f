// Weighted unpermute-combine and the ScMoE RMSNorms of the routed-MoE layer
// on gfx950.  Both are HBM-bound row kernels: one workgroup per token row,
// 16-byte loads along H, fp32 (combine) / fp64 (norm statistics) arithmetic
// in a fixed order, so reruns repeat bit for bit.
//
// Combine ("Module glm5next_mlp", section "One all-reduce for both EP and
// TP": the shared output and the routed slots are summed in one kernel):
//   z[t] = ys[t] + sum_{j<k} w[t,j] * y[inv_pos[t*k+j]]      (fp32, j ascending)
//   out[t] = bf16(z[t])  or, for the ScMoE pairing,
//   out[t] = bf16(z[t] * gamma_post / sqrt(mean(z[t]^2) + eps))
// ("core.models.hybrid.shortcut_block", ShortcutMoEBlock._postprocess: the
// merged routed and shared result is normalised; a plain layer may ask for
// the same norm: Beam's sandwich norm on the MLP output).
//
// Optional finish, fused into the same pass ("bridge.models.beam.
// modeling_beam", _beam_bda and scaled_residual_add: output * coefs[0] +
// residual * coefs[1] in the residual's dtype; ShortcutMoEBlock._postprocess:
// the residual/BDA, coefficients 1):
//   out[t] = bf16(bf16(o * c0) + bf16(res[t] * c1))     (fp32 products, sum)
// with o the bf16 layer output above.  out may be the residual buffer itself:
// each element's residual is read by the thread that writes it, before it
// writes it.
//
// Pre-norm ("core.models.hybrid.shortcut_block", module doc and
// _moe_router_preprocess: the shortcut input is normalised before routing):
//   xr[t] = bf16(fp32((x[t] * r) * gamma)),  r = 1 / sqrt(sum(x^2)/H + eps),
// with the sum of squares and r in fp64: bf16 squares are exact in fp64 and
// IEEE sqrt/div make r reproducible, so xr rarely differs in any bit from an
// fp64 reference that rounds the same products.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int CB_THREADS = 512;  // per token row (226 -> 221 us at T = 8192, H = 4096 against 256)

// Loads of data read exactly once (the routed slot rows, the shared expert's
// row, the residual row, the pre-norm's input row): non-temporal, so the
// stream does not displace other lines in the caches (12 % faster combine at
// T = 8192, H = 4096, k = 8).
__device__ __forceinline__ float4 load_stream(const float4* p) {
  const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
  return make_float4(v[0], v[1], v[2], v[3]);
}
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 load_stream(const uint2* p) {
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(v[0], v[1]);
}
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
constexpr int CB_MAXV = 4;  // float4 groups held per thread with the post-norm (H <= 8192)

template <int THREADS>
__device__ __forceinline__ double block_sum_f64(double v, double* red) {
  v = wave_sum_f64(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  double s = 0.0;
#pragma unroll
  for (int w = 0; w < THREADS / 64; ++w) s += red[w];
  return s;
}

__device__ __forceinline__ uint2 pack_bf16x4(float a, float b, float c, float d) {
  return make_uint2(f32_to_bf16_bits(a) | (f32_to_bf16_bits(b) << 16),
                    f32_to_bf16_bits(c) | (f32_to_bf16_bits(d) << 16));
}

// bf16(bf16(o * c0) + bf16(r * c1)) for one bf16 value each (bits)
__device__ __forceinline__ uint32_t finish_bf16(uint32_t o, uint32_t r, float c0, float c1) {
  const uint32_t a = f32_to_bf16_bits(bf16_bits_to_f32(o) * c0);
  const uint32_t b = f32_to_bf16_bits(bf16_bits_to_f32(r) * c1);
  return f32_to_bf16_bits(bf16_bits_to_f32(a) + bf16_bits_to_f32(b));
}

// four bf16 outputs (packed) through the finish with four residual values
__device__ __forceinline__ uint2 finish_bf16x4(uint2 o, uint2 r, float c0, float c1) {
  return make_uint2(finish_bf16(o.x & 0xffffu, r.x & 0xffffu, c0, c1) |
                        (finish_bf16(o.x >> 16, r.x >> 16, c0, c1) << 16),
                    finish_bf16(o.y & 0xffffu, r.y & 0xffffu, c0, c1) |
                        (finish_bf16(o.y >> 16, r.y >> 16, c0, c1) << 16));
}

// out and residual may be one buffer (no __restrict__ on either)
template <bool POST, bool RES>
__global__ __launch_bounds__(CB_THREADS) void combine_kernel(
    const float* __restrict__ y_perm, const float* __restrict__ w,
    const int32_t* __restrict__ inv_pos, const float* __restrict__ y_shared,
    const float* __restrict__ gamma, const uint16_t* residual, float c0, float c1,
    uint16_t* out, int H, int k, float eps) {
  __shared__ float ws[MOE_MAX_TOP_K_DEV];
  __shared__ int64_t rows[MOE_MAX_TOP_K_DEV];
  __shared__ double red[CB_THREADS / 64];
  const int64_t t = blockIdx.x;
  if (threadIdx.x < k) {
    ws[threadIdx.x] = w[t * k + threadIdx.x];
    rows[threadIdx.x] = (int64_t)inv_pos[t * k + threadIdx.x] * H;
  }
  __syncthreads();
  const int H4 = H >> 2;
  const float4* ys4 = y_shared ? reinterpret_cast<const float4*>(y_shared + t * H) : nullptr;
  uint2* o2 = reinterpret_cast<uint2*>(out + t * H);
  const uint2* r2 = RES ? reinterpret_cast<const uint2*>(residual + t * H) : nullptr;
  auto put = [&](int c4, uint2 v) {
    if (RES) v = finish_bf16x4(v, load_stream(r2 + c4), c0, c1);
    o2[c4] = v;
  };

  auto zval = [&](int c4) {
    float4 z = ys4 ? load_stream(ys4 + c4) : make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
      const float4 y = load_stream(reinterpret_cast<const float4*>(y_perm + rows[j]) + c4);
      const float wj = ws[j];
      z.x = fmaf(wj, y.x, z.x);
      z.y = fmaf(wj, y.y, z.y);
      z.z = fmaf(wj, y.z, z.z);
      z.w = fmaf(wj, y.w, z.w);
    }
    return z;
  };

  if (!POST) {
    for (int c4 = threadIdx.x; c4 < H4; c4 += CB_THREADS) {
      const float4 z = zval(c4);
      put(c4, pack_bf16x4(z.x, z.y, z.z, z.w));
    }
    return;
  }
  float4 zs[CB_MAXV];
  double ss = 0.0;
#pragma unroll
  for (int i = 0; i < CB_MAXV; ++i) {
    const int c4 = threadIdx.x + i * CB_THREADS;
    if (c4 < H4) {
      zs[i] = zval(c4);
      ss += (double)zs[i].x * zs[i].x + (double)zs[i].y * zs[i].y +
            (double)zs[i].z * zs[i].z + (double)zs[i].w * zs[i].w;
    }
  }
  const double sum = block_sum_f64<CB_THREADS>(ss, red);
  const double r = 1.0 / sqrt(sum / (double)H + (double)eps);
  const float4* g4 = reinterpret_cast<const float4*>(gamma);
#pragma unroll
  for (int i = 0; i < CB_MAXV; ++i) {
    const int c4 = threadIdx.x + i * CB_THREADS;
    if (c4 < H4) {
      const float4 g = gamma ? g4[c4] : make_float4(1.f, 1.f, 1.f, 1.f);
      put(c4, pack_bf16x4((float)((double)zs[i].x * r * (double)g.x),
                          (float)((double)zs[i].y * r * (double)g.y),
                          (float)((double)zs[i].z * r * (double)g.z),
                          (float)((double)zs[i].w * r * (double)g.w)));
    }
  }
}

constexpr int RN_THREADS = 256;  // per row (512 measured slower here)
constexpr int RN_MAXV = 4;       // 8-element groups per thread (H <= 8192)

__global__ __launch_bounds__(RN_THREADS) void rmsnorm_bf16_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ gamma, uint16_t* __restrict__ out,
    int H, float eps) {
  __shared__ double red[RN_THREADS / 64];
  const int64_t t = blockIdx.x;
  const uint4* x8 = reinterpret_cast<const uint4*>(x + t * H);
  const int H8 = H >> 3;
  uint4 v[RN_MAXV];
  double ss = 0.0;
#pragma unroll
  for (int i = 0; i < RN_MAXV; ++i) {
    const int c = threadIdx.x + i * RN_THREADS;
    if (c < H8) {
      v[i] = load_stream(x8 + c);
      const uint32_t u[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const double a = bf16_bits_to_f32(u[q] & 0xffffu), b = bf16_bits_to_f32(u[q] >> 16);
        ss += a * a + b * b;
      }
    }
  }
  const double sum = block_sum_f64<RN_THREADS>(ss, red);
  const double r = 1.0 / sqrt(sum / (double)H + (double)eps);
  uint4* o8 = reinterpret_cast<uint4*>(out + t * H);
  const float4* g4 = reinterpret_cast<const float4*>(gamma);
#pragma unroll
  for (int i = 0; i < RN_MAXV; ++i) {
    const int c = threadIdx.x + i * RN_THREADS;
    if (c < H8) {
      const uint32_t u[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
      float g[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
      if (gamma) {  // the row's 8 gains in two 16-byte loads
        const float4 g0 = g4[2 * c], g1 = g4[2 * c + 1];
        g[0] = g0.x; g[1] = g0.y; g[2] = g0.z; g[3] = g0.w;
        g[4] = g1.x; g[5] = g1.y; g[6] = g1.z; g[7] = g1.w;
      }
      uint32_t o[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        double a = (double)bf16_bits_to_f32(u[q] & 0xffffu) * r;
        double b = (double)bf16_bits_to_f32(u[q] >> 16) * r;
        if (gamma) {
          a *= (double)g[2 * q];
          b *= (double)g[2 * q + 1];
        }
        o[q] = f32_to_bf16_bits((float)a) | (f32_to_bf16_bits((float)b) << 16);
      }
      o8[c] = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
}

}  // namespace

hipError_t launch_combine(const float* y_perm, const float* w, const int32_t* inv_pos,
                          const float* y_shared, const float* gamma_post, const uint16_t* residual,
                          float c0, float c1, uint16_t* out, int64_t T, int H, int k,
                          int post_norm, float eps, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  void (*kern)(const float*, const float*, const int32_t*, const float*, const float*,
               const uint16_t*, float, float, uint16_t*, int, int, float);
  if (post_norm)
    kern = residual ? combine_kernel<true, true> : combine_kernel<true, false>;
  else
    kern = residual ? combine_kernel<false, true> : combine_kernel<false, false>;
  hipLaunchKernelGGL(kern, dim3((unsigned)T), dim3(CB_THREADS), 0, stream, y_perm, w, inv_pos,
                     y_shared, gamma_post, residual, c0, c1, out, H, k, eps);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_bf16(const uint16_t* x, const float* gamma, uint16_t* out, int64_t T,
                               int H, float eps, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(rmsnorm_bf16_kernel, dim3((unsigned)T), dim3(RN_THREADS), 0, stream, x,
                     gamma, out, H, eps);
  return hipGetLastError();
}
