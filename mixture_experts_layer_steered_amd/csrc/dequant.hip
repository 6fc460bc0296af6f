// W4A16 expert weights -> bf16, for batches whose grouped GEMMs run on the
// tiled bf16 matrix-core kernels (more than 64 rows per expert, bound by
// the MFMAs, where the weight bytes no longer decide the time), and for
// callers who expand fixed weights once.
//
// Format (the grouped W4A16 expert GEMM of "Module glm5next_mlp", with the
// two scale levels of the NVFP4 routed experts its module doc names, in
// this library's layout): a weight is (u - 8) * e4m3(scale) * tensor_scale,
// u a 4-bit code; codes run along K in 4-byte words of 8 columns whose byte
// j holds columns j and j + 4 in its low and high nibble; one E4M3 scale
// byte per row and 128 columns, stored group-major [K/128, rows]; one fp32
// tensor scale per group (expert).  (u - 8) has at most 3 significant bits
// and an E4M3 value at most 4, so (u - 8) * e4m3(scale) is exact in bf16
// (8 significant bits, and far inside its exponent range): without a
// tensor scale this expansion is exact.  With one, the product is scaled
// in fp32 and rounded once to bf16 (to nearest, ties to even) -- exact
// again when the tensor scale is a power of two.  The forward itself never
// folds the tensor scale in here: its GEMMs apply it to their fp32
// accumulators.
//
// One workgroup per weight row (of all groups): its threads walk the row's
// code words, 4 bytes in and 16 bytes (8 bf16) out each.
#include "common.h"
#include "kernels.h"

namespace {

__global__ __launch_bounds__(256) void w4_dequant_kernel(const uint32_t* __restrict__ q,
                                                         const uint8_t* __restrict__ scale,
                                                         const float* __restrict__ tscale,
                                                         uint16_t* __restrict__ out, int rows,
                                                         int K) {
  const int64_t row_all = blockIdx.x;  // row over all groups
  const int g = (int)(row_all / rows), r = (int)(row_all - (int64_t)g * rows);  // uniform
  const int wpr = K / 8, groups = K / 128;
  const uint32_t* qr = q + row_all * wpr;
  uint4* orow = reinterpret_cast<uint4*>(out + row_all * K);
  const uint8_t* sr = scale + (int64_t)g * groups * rows + r;  // group-major scales
  const float ts = tscale ? tscale[g] : 1.0f;
  for (int c8 = threadIdx.x; c8 < wpr; c8 += 256) {
    const float sc = e4m3_to_f32(sr[(int64_t)(c8 >> 4) * rows]);
    const float m = -136.0f * sc;  // exact: 136 has 5 significant bits, sc at most 4
    const uint32_t d = __builtin_nontemporal_load(qr + c8);  // read once
    // bytes u of columns 0..3 (low nibbles) and 4..7 (high nibbles), then
    // bf16 pairs 128 + u (bits 0x43 over each byte); (128 + u) * sc - 136 sc
    // = (u - 8) * sc is exact in one fma; times the tensor scale (exact for
    // 1), then one rounding to bf16
    const uint32_t lo = d & 0x0F0F0F0Fu, hi = (d >> 4) & 0x0F0F0F0Fu;
    const uint32_t pr[4] = {__builtin_amdgcn_perm(0x43434343u, lo, 0x04010400u),
                            __builtin_amdgcn_perm(0x43434343u, lo, 0x04030402u),
                            __builtin_amdgcn_perm(0x43434343u, hi, 0x04010400u),
                            __builtin_amdgcn_perm(0x43434343u, hi, 0x04030402u)};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a = fmaf(__uint_as_float(pr[j] << 16), sc, m) * ts;
      const float b = fmaf(__uint_as_float(pr[j] & 0xffff0000u), sc, m) * ts;
      o[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(float2_t{a, b}, bf16x2_t));
    }
    orow[c8] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

}  // namespace

hipError_t launch_w4_dequant(const uint8_t* q, const uint8_t* scale, const float* tscale,
                             uint16_t* out, int G, int64_t rows, int K, hipStream_t stream) {
  const int64_t all_rows = (int64_t)G * rows;
  if (all_rows == 0) return hipSuccess;
  hipLaunchKernelGGL(w4_dequant_kernel, dim3((unsigned)all_rows), dim3(256), 0, stream,
                     reinterpret_cast<const uint32_t*>(q), scale, tscale, out, (int)rows, K);
  return hipGetLastError();
}
