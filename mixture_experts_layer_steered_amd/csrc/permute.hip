// Token permutation of the routed-MoE layer on gfx950: a stable counting
// sort of the T*k (token, slot) pairs by expert id ("Module glm5next_mlp",
// Constants, MOE_MODULE: token sort / permute / unpermute kernels).
//
// Deterministic and exact, with no global atomics:
//   1. permute_hist:    one workgroup per tile of 4096 pairs counts the ids
//                       of its tile in LDS and writes counts[tile][E].
//   2. permute_scan:    one workgroup turns the counts into the exclusive
//                       start of every (expert, tile) run in expert-major
//                       order, and the expert offsets.
//   3. permute_scatter: one workgroup per tile again; each wavefront owns 256
//                       consecutive pairs, gets its start per expert from an
//                       LDS prefix over the waves, and ranks equal ids inside
//                       a 64-pair step with ballot match masks, so every
//                       expert's rows keep the pairs' order.
// With a single tile (decode) one workgroup does all three, and the grouped
// GEMM's m-tile prefix, in one launch.
// The LDS atomics of steps 1 and 3 only count; the order of the increments
// never shows in a result.
#include "common.h"
#include "kernels.h"
#include "permute_small.h"

namespace {

__global__ __launch_bounds__(PM_THREADS) void permute_hist_kernel(
    const int32_t* __restrict__ ids, int32_t* __restrict__ counts, int64_t N, int E) {
  __shared__ int32_t hist[MOE_MAX_EXPERTS_DEV];
  for (int e = threadIdx.x; e < E; e += PM_THREADS) hist[e] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * PM_TILE;
  for (int i = threadIdx.x; i < PM_TILE; i += PM_THREADS) {
    int64_t p = base + i;
    if (p < N) atomicAdd(&hist[ids[p]], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += PM_THREADS) counts[(int64_t)blockIdx.x * E + e] = hist[e];
}

// Single workgroup.  counts[tiles][E] -> starts[tiles][E] (exclusive start of
// each (expert, tile) run in expert-major order) and offsets[E+1]; with
// mstart, also the grouped GEMM's m-tile prefix for tiles of bm rows
// (mstart[e] = sum over e' < e of ceil(n_e' / bm), mstart[E] the total).
__global__ __launch_bounds__(PM_THREADS) void permute_scan_kernel(
    const int32_t* __restrict__ counts, int32_t* __restrict__ starts,
    int32_t* __restrict__ offsets, int tiles, int E, int64_t N, int bm,
    int32_t* __restrict__ mstart) {
  __shared__ int32_t tot[MOE_MAX_EXPERTS_DEV];
  __shared__ int32_t wsum[PM_WAVES];
  __shared__ int32_t msum[PM_WAVES];
  const int e = threadIdx.x;
  int32_t run = 0;
  if (e < E) {
    for (int t = 0; t < tiles; ++t) {
      int32_t c = counts[(int64_t)t * E + e];
      starts[(int64_t)t * E + e] = run;
      run += c;
    }
  }
  // exclusive scan of run over experts (block scan: wave prefix + wave totals)
  const int lane = e & 63, wave = e >> 6;
  int32_t v = (e < E) ? run : 0;
  int32_t incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int32_t o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int32_t before = 0;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  const int32_t excl = before + incl - v;
  if (e < E) {
    offsets[e] = excl;
    tot[e] = excl;
  }
  if (e == 0) offsets[E] = (int32_t)N;
  if (mstart != nullptr) {  // the same block scan over the experts' m-tile counts
    const int32_t mv = (v + bm - 1) / bm;
    int32_t mincl = mv;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      int32_t o = __shfl_up(mincl, off, 64);
      if (lane >= off) mincl += o;
    }
    if (lane == 63) msum[wave] = mincl;
    __syncthreads();
    int32_t mbefore = 0;
    for (int w = 0; w < wave; ++w) mbefore += msum[w];
    if (e < E) mstart[e] = mbefore + mincl - mv;
    if (e == E - 1) mstart[E] = mbefore + mincl;
  }
  __syncthreads();
  if (e < E) {
    for (int t = 0; t < tiles; ++t) starts[(int64_t)t * E + e] += tot[e];
  }
}

__global__ __launch_bounds__(PM_THREADS) void permute_scatter_kernel(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ starts,
    int32_t* __restrict__ sorted_token, int32_t* __restrict__ inv_pos, int64_t N, int E, int k) {
  __shared__ int32_t whist[PM_WAVES][MOE_MAX_EXPERTS_DEV];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < PM_WAVES * E; i += PM_THREADS) whist[i / E][i % E] = 0;
  __syncthreads();
  const int64_t wbase = (int64_t)blockIdx.x * PM_TILE + (int64_t)wave * PM_PER_WAVE;
  int my_e[PM_STEPS];
#pragma unroll
  for (int s = 0; s < PM_STEPS; ++s) {
    int64_t p = wbase + s * 64 + lane;
    my_e[s] = (p < N) ? ids[p] : MOE_MAX_EXPERTS_DEV;  // sentinel: matches no expert
    if (p < N) atomicAdd(&whist[wave][my_e[s]], 1);
  }
  __syncthreads();
  // per expert: exclusive prefix over the waves, offset by the tile's start
  for (int e = threadIdx.x; e < E; e += PM_THREADS) {
    int32_t run = starts[(int64_t)blockIdx.x * E + e];
    for (int w = 0; w < PM_WAVES; ++w) {
      int32_t c = whist[w][e];
      whist[w][e] = run;
      run += c;
    }
  }
  __syncthreads();
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int s = 0; s < PM_STEPS; ++s) {
    const int e = my_e[s];
    // lanes holding the same id: intersect ballots over the id's 11 bits
    uint64_t same = ~0ull;
#pragma unroll
    for (int b = 0; b < 11; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bal = __ballot(bit);
      same &= bit ? bal : ~bal;
    }
    const int rank = __popcll(same & lt_mask);
    const int cnt = __popcll(same);
    if (e < E) {
      const int64_t p = wbase + s * 64 + lane;
      const int32_t pos = whist[wave][e] + rank;
      sorted_token[pos] = (int32_t)(p / k);
      inv_pos[p] = pos;
      if (rank == 0) whist[wave][e] += cnt;
    }
  }
}

// All pairs in one tile (N <= 4096, decode-sized batches): the three passes
// in one workgroup, plus the m-tile prefix of the grouped GEMM over the
// expert counts (the schedule the GEMM launches read), in one launch.
__global__ __launch_bounds__(PM_THREADS) void permute_small_kernel(
    const int32_t* __restrict__ ids, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_token, int32_t* __restrict__ inv_pos, int64_t N, int E, int k,
    int bm, int32_t* __restrict__ mstart) {
  __shared__ int32_t whist[PM_WAVES * MOE_MAX_EXPERTS_DEV];
  __shared__ int32_t wsum[2 * PM_WAVES];
  permute_small_body(ids, offsets, sorted_token, inv_pos, N, E, k, bm, mstart, whist, wsum);
}

// Optional materialised gather of the permuted activations: 16 bytes per
// thread, consecutive threads along a row (coalesced reads of the source row
// and writes of the destination row); grid-stride over (row, chunk).
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint4* __restrict__ x,
                                                          const int32_t* __restrict__ sorted_token,
                                                          uint4* __restrict__ x_perm, int64_t N,
                                                          int chunks) {
  const int64_t total = N * chunks;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / chunks;
    const int c = (int)(i - r * chunks);
    x_perm[i] = x[(int64_t)sorted_token[r] * chunks + c];
  }
}

}  // namespace

int permute_tiles(int64_t N) { return (int)((N + PM_TILE - 1) / PM_TILE); }

hipError_t launch_gather_rows(const uint16_t* x, const int32_t* sorted_token, uint16_t* x_perm,
                              int64_t N, int H, hipStream_t stream) {
  const int chunks = H / 8;
  const int64_t total = N * chunks;
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256;
  const unsigned grid = (unsigned)(blocks < 8192 ? blocks : 8192);
  hipLaunchKernelGGL(gather_rows_kernel, dim3(grid), dim3(256), 0, stream,
                     reinterpret_cast<const uint4*>(x), sorted_token,
                     reinterpret_cast<uint4*>(x_perm), N, chunks);
  return hipGetLastError();
}

hipError_t launch_permute(const int32_t* ids, int32_t* counts, int32_t* starts, int32_t* offsets,
                          int32_t* sorted_token, int32_t* inv_pos, int64_t N, int E, int k,
                          int bm, int32_t* mstart, hipStream_t stream) {
  const int tiles = permute_tiles(N);
  if (tiles == 1) {
    hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(PM_THREADS), 0, stream, ids, offsets,
                       sorted_token, inv_pos, N, E, k, bm > 0 ? bm : 1, mstart);
    return hipGetLastError();
  }
  if (tiles == 0) {
    // no pairs: offsets are all zero
    hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(PM_THREADS), 0, stream, counts, starts,
                       offsets, 0, E, (int64_t)0, bm > 0 ? bm : 1, mstart);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(permute_hist_kernel, dim3(tiles), dim3(PM_THREADS), 0, stream, ids, counts,
                     N, E);
  hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(PM_THREADS), 0, stream, counts, starts,
                     offsets, tiles, E, N, bm > 0 ? bm : 1, mstart);
  hipLaunchKernelGGL(permute_scatter_kernel, dim3(tiles), dim3(PM_THREADS), 0, stream, ids,
                     starts, sorted_token, inv_pos, N, E, k);
  return hipGetLastError();
}
