// Measured peaks of the part the layer runs on, for reporting the layer's
// rates against what this GPU delivers as well as against its published
// figures: a bf16 matrix-core throughput probe and an HBM read-stream
// probe.  Neither is on the layer's path.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int PB_CHAINS = 4;  // independent accumulators per wavefront
typedef uint32_t pb_u32x4 __attribute__((ext_vector_type(4)));

// Each wavefront runs `iters` rounds of PB_CHAINS independent
// v_mfma_f32_32x32x16_bf16 on operands derived from `seed` (non-zero,
// varied bits: the part draws more power -- and may clock lower -- on
// random operands than on zeros), then folds its accumulators into one
// float per lane so the work cannot be dropped.
__global__ __launch_bounds__(256) void probe_mfma_kernel(int iters, uint32_t seed,
                                                         float* __restrict__ sink) {
  const uint32_t tid = blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t h = seed ^ (tid * 0x9E3779B9u);
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  u32x4_t av, bv;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h = h * 1664525u + 1013904223u;
    // two bf16 values in [1, 2) with random mantissas and signs
    av[i] = 0x3F803F80u | (h & 0x807F807Fu);
    h = h * 1664525u + 1013904223u;
    bv[i] = 0x3F803F80u | (h & 0x807F807Fu);
  }
  const bf16x8_t a = __builtin_bit_cast(bf16x8_t, av);
  const bf16x8_t b = __builtin_bit_cast(bf16x8_t, bv);
  f32x16_t acc[PB_CHAINS];
#pragma unroll
  for (int c = 0; c < PB_CHAINS; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < PB_CHAINS; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < PB_CHAINS; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  sink[tid] = s;
}

// Workgroup b reads its own contiguous block of src (the blocks tile the
// buffer in order), 16 KB per step: four non-temporal 16-byte loads per
// thread, each load of the workgroup covering 4 KB contiguously, and folds
// them into one word per thread.
__global__ __launch_bounds__(256) void probe_read_kernel(const pb_u32x4* __restrict__ src,
                                                         int64_t n16, uint32_t* __restrict__ sink) {
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;  // 16-byte pieces per workgroup
  const int64_t begin = (int64_t)blockIdx.x * per;
  const int64_t end = begin + per < n16 ? begin + per : n16;
  uint32_t x = 0;
  int64_t i = begin + threadIdx.x;
  for (; i + 768 < end; i += 1024) {
    const pb_u32x4 v0 = __builtin_nontemporal_load(src + i);
    const pb_u32x4 v1 = __builtin_nontemporal_load(src + i + 256);
    const pb_u32x4 v2 = __builtin_nontemporal_load(src + i + 512);
    const pb_u32x4 v3 = __builtin_nontemporal_load(src + i + 768);
    x ^= v0.x ^ v0.y ^ v0.z ^ v0.w ^ v1.x ^ v1.y ^ v1.z ^ v1.w;
    x ^= v2.x ^ v2.y ^ v2.z ^ v2.w ^ v3.x ^ v3.y ^ v3.z ^ v3.w;
  }
  for (; i < end; i += 256) {
    const pb_u32x4 v = __builtin_nontemporal_load(src + i);
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = x;
}

}  // namespace

hipError_t launch_probe_mfma(int wgs, int iters, float* sink, hipStream_t stream) {
  hipLaunchKernelGGL(probe_mfma_kernel, dim3(wgs), dim3(256), 0, stream, iters, 0x2545F491u,
                     sink);
  return hipGetLastError();
}

double probe_mfma_flops(int wgs, int iters) {
  // 4 wavefronts per workgroup, PB_CHAINS MFMAs of 32 x 32 x 16 per round
  return (double)wgs * 4 * iters * PB_CHAINS * 2.0 * 32 * 32 * 16;
}

hipError_t launch_probe_read(const void* src, int64_t bytes, int wgs, uint32_t* sink,
                             hipStream_t stream) {
  hipLaunchKernelGGL(probe_read_kernel, dim3(wgs), dim3(256), 0, stream,
                     static_cast<const pb_u32x4*>(src), bytes / 16, sink);
  return hipGetLastError();
}
