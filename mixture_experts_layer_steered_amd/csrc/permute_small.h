// Stable counting sort of at most 4096 (token, slot) pairs by expert id in
// one workgroup of 1024 threads ("Module glm5next_mlp", Constants,
// MOE_MODULE: token sort / permute / unpermute): the per-wave histograms,
// the scans over experts (expert offsets, and the grouped GEMM's m-tile
// prefix over the counts for tiles of bm rows), and a scatter that ranks
// equal ids inside a 64-pair step with ballot match masks, so every
// expert's rows keep the pairs' order.  Used by the permute's one-launch
// path and by the fused routing of decode-sized batches.  The LDS atomics
// only count; the order of the increments never shows in a result.
#pragma once

#include "common.h"
#include "kernels.h"

constexpr int PM_THREADS = 1024;
constexpr int PM_WAVES = PM_THREADS / 64;
constexpr int PM_PER_WAVE = 256;
constexpr int PM_TILE = PM_WAVES * PM_PER_WAVE;  // 4096 pairs
constexpr int PM_STEPS = PM_PER_WAVE / 64;

// Workgroup barrier for LDS only: this thread's LDS operations have completed
// (lgkmcnt(0)), and global stores still in flight are not waited for (the
// results go to later launches).
__device__ __forceinline__ void pm_lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Every thread of the workgroup calls it (it synchronises the workgroup).
// ids: the N <= PM_TILE expert ids (global or LDS memory); whist: LDS of
// PM_WAVES * MOE_MAX_EXPERTS_DEV ints; wsum: LDS of 2 * PM_WAVES ints.
__device__ __forceinline__ void permute_small_body(const int32_t* ids, int32_t* offsets,
                                                   int32_t* sorted_token, int32_t* inv_pos,
                                                   int64_t N, int E, int k, int bm,
                                                   int32_t* mstart, int32_t* whist,
                                                   int32_t* wsum) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  constexpr int MX = MOE_MAX_EXPERTS_DEV;
  for (int i = threadIdx.x; i < PM_WAVES * E; i += PM_THREADS) whist[(i / E) * MX + i % E] = 0;
  pm_lds_barrier();
  // each wave takes a contiguous run of the pairs in order, as few 64-pair
  // steps as spread the batch over all the waves (one step each up to 1024
  // pairs); the order of the runs is the order of the waves
  const int steps = (int)((N + PM_WAVES * 64 - 1) / (PM_WAVES * 64));
  const int64_t wbase = (int64_t)wave * steps * 64;
  int my_e[PM_STEPS];
#pragma unroll
  for (int s = 0; s < PM_STEPS; ++s) {
    const int64_t p = wbase + s * 64 + lane;
    const bool in = s < steps && p < N;
    my_e[s] = in ? ids[p] : MX;  // sentinel: matches no expert
    if (in) atomicAdd(&whist[wave * MX + my_e[s]], 1);
  }
  pm_lds_barrier();
  // thread e: expert e's count, then exclusive scans over experts of the
  // counts (offsets) and of the m-tiles ceil(count / bm) (GEMM schedule)
  const int e = threadIdx.x;
  int32_t cnt = 0;
  if (e < E)
    for (int w = 0; w < PM_WAVES; ++w) cnt += whist[w * MX + e];
  int32_t v[2] = {cnt, (cnt + bm - 1) / bm};
  int32_t incl[2] = {v[0], v[1]};
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int32_t o = __shfl_up(incl[q], off, 64);
      if (lane >= off) incl[q] += o;
    }
  }
  if (lane == 63) {
    wsum[wave] = incl[0];
    wsum[PM_WAVES + wave] = incl[1];
  }
  pm_lds_barrier();
  int32_t before[2] = {0, 0};
  for (int w = 0; w < wave; ++w) {
    before[0] += wsum[w];
    before[1] += wsum[PM_WAVES + w];
  }
  const int32_t start = before[0] + incl[0] - v[0];
  if (e < E) {
    offsets[e] = start;
    if (mstart) mstart[e] = before[1] + incl[1] - v[1];
    // each wave's run of expert e starts after the earlier waves' pairs
    int32_t run = start;
    for (int w = 0; w < PM_WAVES; ++w) {
      const int32_t c = whist[w * MX + e];
      whist[w * MX + e] = run;
      run += c;
    }
  }
  if (e == E - 1) {
    offsets[E] = (int32_t)N;
    if (mstart) mstart[E] = before[1] + incl[1];
  }
  pm_lds_barrier();
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int s = 0; s < PM_STEPS; ++s) {
    if (s >= steps) break;  // uniform
    const int ee = my_e[s];
    uint64_t same = ~0ull;
#pragma unroll
    for (int b = 0; b < 11; ++b) {
      const bool bit = (ee >> b) & 1;
      const uint64_t bal = __ballot(bit);
      same &= bit ? bal : ~bal;
    }
    const int rank = __popcll(same & lt_mask);
    const int n_same = __popcll(same);
    if (ee < E) {
      const int64_t p = wbase + s * 64 + lane;
      const int32_t pos = whist[wave * MX + ee] + rank;
      sorted_token[pos] = (int32_t)(p / k);
      inv_pos[p] = pos;
      if (rank == 0) whist[wave * MX + ee] += n_same;
    }
  }
}
