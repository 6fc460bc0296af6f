// Grouped expert GEMMs of the routed-MoE layer on gfx950 (CDNA4) bf16 MFMA.
//
// One launch per projection covers every expert (and the shared expert in
// the same launch) -- "Module glm5next_mlp", Modules forward_prefill_gemm:
// one grouped launch per projection for all experts, with tile variants.
//
//   gate_up: per group g and row r of its segment,
//            [g_r, u_r] = A[row(r)] @ W_gu[g]^T (fp32 accumulators), and the
//            epilogue writes h[r] = bf16(silu(min(g_r, L)) * clamp(u_r, -L, L))
//            -- the clamp of "Numerics the kernels rely on", applied to the
//            fp32 accumulators.  A workgroup owns BN gate columns and the
//            matching BN up columns (rows n and I + n of the fused weight,
//            "mstar.model.components.distributed.mlp", ParallelGatedMLP), so
//            each lane holds g and u of the same (row, column) in the same
//            accumulator slot.
//   down:    y[r] = h[r] @ W_d[g]^T, fp32 out.
//
// Operands are K-contiguous on both sides ([rows, K] activations, [out, in]
// weights), so every lane feeds the MFMA with one 16-byte LDS read per
// operand fragment.  Tiles are staged through LDS (BK = 64, 16-byte chunks
// XOR-swizzled by row to spread banks) with a register prefetch of the next
// K step in flight during the MFMAs.  Rows of a routed tile are gathered
// through row_index (the permutation), so no permuted copy of x is made.
//
// Schedule: expert segment sizes live on the device.  A one-workgroup
// kernel turns group_offsets into the prefix of m-tiles per group; each GEMM
// workgroup maps its tile id to (group, m-tile, n-tile) by binary search and
// exits when past the end.  Workgroup ids are remapped so each of the 8 XCDs
// works a contiguous range of tiles, m-tiles fastest: consecutive tiles on an
// XCD share one weight n-tile in that XCD's L2.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int BK = 64;
constexpr int CH = BK / 8;  // 16-byte chunks per LDS row

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ (row & 7); }

__device__ __forceinline__ int xcd_remap(int bid, int nb) {
  const int xcd = bid & 7, local = bid >> 3;
  const int per = nb >> 3, rem = nb & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + local;
}

template <int BM, int BN, int WAVES_M, int WAVES_N, bool GATEUP>
__device__ __forceinline__ void gemm_tile(const GemmProblem& P, int tile, float limit) {
  constexpr int THREADS = WAVES_M * WAVES_N * 64;
  constexpr int NB = GATEUP ? 2 * BN : BN;  // weight rows per tile
  constexpr int WM = BM / WAVES_M;          // rows per wave
  constexpr int WN = BN / WAVES_N;          // output columns per wave
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int NMAT = GATEUP ? 2 : 1;
  constexpr int A_CHUNKS = BM * CH / THREADS;
  constexpr int B_CHUNKS = NB * CH / THREADS;
  static_assert(A_CHUNKS >= 1 && B_CHUNKS >= 1, "tile too small for the workgroup");
  static_assert(BM * CH % THREADS == 0 && NB * CH % THREADS == 0, "uneven load split");

  __shared__ __attribute__((aligned(16))) uint16_t As[BM * BK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[NB * BK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;

  const int mt_global = tile % P.max_mtiles;
  const int nt = tile / P.max_mtiles;

  // tile -> group, first row, end row
  int g = 0;
  int64_t row0, row_end;
  if (P.group_offsets == nullptr) {
    row0 = (int64_t)mt_global * BM;
    row_end = P.M;
    if (row0 >= row_end) return;
  } else {
    if (mt_global >= P.mtile_start[P.G]) return;
    int lo = 0, hi = P.G - 1;  // last g with mtile_start[g] <= mt_global
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (P.mtile_start[mid] <= mt_global) lo = mid; else hi = mid - 1;
    }
    g = lo;
    row0 = P.group_offsets[g] + (int64_t)(mt_global - P.mtile_start[g]) * BM;
    row_end = P.group_offsets[g + 1];
  }
  const int n0 = nt * BN;
  const int K = P.K, N = P.N;
  const uint16_t* __restrict__ Wg = P.W + (int64_t)g * P.w_stride;

  // per-thread source rows of the A and B chunks it loads (fixed over K)
  const uint16_t* a_src[A_CHUNKS];
  int a_dst[A_CHUNKS];
  int a_cc[A_CHUNKS];
#pragma unroll
  for (int i = 0; i < A_CHUNKS; ++i) {
    const int c = tid + i * THREADS;
    const int r = c / CH, cc = c % CH;
    const int64_t gr = row0 + r;
    a_src[i] = nullptr;
    if (gr < row_end) {
      const int64_t src = P.row_index ? (int64_t)P.row_index[gr] : gr;
      a_src[i] = P.A + src * K + cc * 8;
    }
    a_dst[i] = r * BK + swz(r, cc) * 8;
    a_cc[i] = cc;
  }
  const uint16_t* b_src[B_CHUNKS];
  int b_dst[B_CHUNKS];
  int b_cc[B_CHUNKS];
#pragma unroll
  for (int i = 0; i < B_CHUNKS; ++i) {
    const int c = tid + i * THREADS;
    const int r = c / CH, cc = c % CH;
    int n, wrow;
    if (GATEUP) {
      n = n0 + (r < BN ? r : r - BN);
      wrow = r < BN ? n : N + n;  // gate rows [0, N), up rows [N, 2N)
    } else {
      n = n0 + r;
      wrow = n;
    }
    b_src[i] = (n < N) ? Wg + (int64_t)wrow * K + cc * 8 : nullptr;
    b_dst[i] = r * BK + swz(r, cc) * 8;
    b_cc[i] = cc;
  }

  f32x16_t acc[NMAT][TM][TN];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[m][i][j][r] = 0.f;

  uint4 a_reg[A_CHUNKS], b_reg[B_CHUNKS];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) {
      a_reg[i] = make_uint4(0, 0, 0, 0);
      if (a_src[i] && k0 + a_cc[i] * 8 < K) a_reg[i] = *reinterpret_cast<const uint4*>(a_src[i] + k0);
    }
#pragma unroll
    for (int i = 0; i < B_CHUNKS; ++i) {
      b_reg[i] = make_uint4(0, 0, 0, 0);
      if (b_src[i] && k0 + b_cc[i] * 8 < K) b_reg[i] = *reinterpret_cast<const uint4*>(b_src[i] + k0);
    }
  };

  load(0);
  for (int k0 = 0; k0 < K; k0 += BK) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) *reinterpret_cast<uint4*>(&As[a_dst[i]]) = a_reg[i];
#pragma unroll
    for (int i = 0; i < B_CHUNKS; ++i) *reinterpret_cast<uint4*>(&Bs[b_dst[i]]) = b_reg[i];
    __syncthreads();
    if (k0 + BK < K) load(k0 + BK);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int chunk = ks * 2 + (lane >> 5);
      bf16x8_t af[TM];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = wm * WM + i * 32 + (lane & 31);
        af[i] = *reinterpret_cast<const bf16x8_t*>(&As[r * BK + swz(r, chunk) * 8]);
      }
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int r = m * BN + wn * WN + j * 32 + (lane & 31);
          const bf16x8_t bfrag = *reinterpret_cast<const bf16x8_t*>(&Bs[r * BK + swz(r, chunk) * 8]);
#pragma unroll
          for (int i = 0; i < TM; ++i)
            acc[m][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfrag, acc[m][i][j], 0, 0, 0);
        }
      }
    }
  }

  // epilogue: 32x32 accumulator, lane holds column (lane & 31) and rows
  // 8*(r/4) + 4*(lane/32) + r%4
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = n0 + wn * WN + j * 32 + (lane & 31);
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = row0 + wm * WM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row >= row_end) continue;
        if (GATEUP) {
          const float hv = swiglu_clamped(acc[0][i][j][r], acc[NMAT - 1][i][j][r], limit);
          static_cast<uint16_t*>(P.out)[row * N + col] = (uint16_t)f32_to_bf16_bits(hv);
        } else {
          static_cast<float*>(P.out)[row * N + col] = acc[0][i][j][r];
        }
      }
    }
  }
}

template <int BM, int BN, int WAVES_M, int WAVES_N, bool GATEUP>
__global__ __launch_bounds__(WAVES_M * WAVES_N * 64) void grouped_gemm_kernel(
    GemmProblem p0, GemmProblem p1, int tiles0, float limit) {
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  if (tile < tiles0)
    gemm_tile<BM, BN, WAVES_M, WAVES_N, GATEUP>(p0, tile, limit);
  else
    gemm_tile<BM, BN, WAVES_M, WAVES_N, GATEUP>(p1, tile - tiles0, limit);
}

// m-tile prefix of up to two tile heights over one set of group offsets.
__global__ __launch_bounds__(1024) void gemm_schedule_kernel(const int32_t* __restrict__ offsets,
                                                             int G, int bm0, int bm1,
                                                             int32_t* __restrict__ start0,
                                                             int32_t* __restrict__ start1) {
  __shared__ int32_t wsum[2][16];
  const int g = threadIdx.x, lane = g & 63, wave = g >> 6;
  int32_t n = (g < G) ? offsets[g + 1] - offsets[g] : 0;
  int32_t v[2] = {(n + bm0 - 1) / bm0, (n + bm1 - 1) / bm1};
  int32_t incl[2] = {v[0], v[1]};
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      int32_t o = __shfl_up(incl[q], off, 64);
      if (lane >= off) incl[q] += o;
    }
  }
  if (lane == 63) { wsum[0][wave] = incl[0]; wsum[1][wave] = incl[1]; }
  __syncthreads();
  int32_t before[2] = {0, 0};
  for (int w = 0; w < wave; ++w) { before[0] += wsum[0][w]; before[1] += wsum[1][w]; }
  if (g < G) {
    start0[g] = before[0] + incl[0] - v[0];
    if (start1) start1[g] = before[1] + incl[1] - v[1];
  }
  if (g == G - 1) {
    start0[G] = before[0] + incl[0];
    if (start1) start1[G] = before[1] + incl[1];
  }
}

template <int BM, int BN, int WM_, int WN_>
hipError_t launch_pair(const GemmProblem& a, const GemmProblem* b, float limit, bool gateup,
                       hipStream_t stream) {
  const int tiles0 = a.max_mtiles * a.ntiles;
  const int tiles1 = b ? b->max_mtiles * b->ntiles : 0;
  const int total = tiles0 + tiles1;
  if (total == 0) return hipSuccess;
  GemmProblem pb = b ? *b : a;
  dim3 grid(total), block(WM_ * WN_ * 64);
  if (gateup)
    hipLaunchKernelGGL((grouped_gemm_kernel<BM, BN, WM_, WN_, true>), grid, block, 0, stream, a,
                       pb, tiles0, limit);
  else
    hipLaunchKernelGGL((grouped_gemm_kernel<BM, BN, WM_, WN_, false>), grid, block, 0, stream, a,
                       pb, tiles0, limit);
  return hipGetLastError();
}

}  // namespace

int gemm_tile_m(GemmVariant v) { return v == GemmVariant::kStream ? 32 : 128; }
int gemm_tile_n(GemmVariant) { return 128; }

hipError_t launch_gemm_schedule(const int32_t* group_offsets, int G, int bm0, int bm1,
                                int32_t* start0, int32_t* start1, hipStream_t stream) {
  hipLaunchKernelGGL(gemm_schedule_kernel, dim3(1), dim3(1024), 0, stream, group_offsets, G, bm0,
                     bm1, start0, start1);
  return hipGetLastError();
}

hipError_t launch_grouped_gemm(GemmVariant v, bool gateup, const GemmProblem& a,
                               const GemmProblem* b, float limit, hipStream_t stream) {
  if (v == GemmVariant::kStream) return launch_pair<32, 128, 1, 4>(a, b, limit, gateup, stream);
  return launch_pair<128, 128, 2, 2>(a, b, limit, gateup, stream);
}
