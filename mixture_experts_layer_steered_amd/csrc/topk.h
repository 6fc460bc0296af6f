// Per-token expert selection of the router's top-k kernel ("Module
// glm5next_mlp", section
// "Numerics the kernels rely on"; Constants, KERNEL_MAX_TOP_K):
// s = sigmoid(l) (evaluated in fp64, rounded once to fp32), s' = s + b in
// fp32, the k largest s' over all E experts, ties to the lower expert id,
// NaN below every number; ids in ascending order with weight rsf * s (the
// bias never enters a weight).
#pragma once

#include "common.h"

__device__ __forceinline__ float topk_sigmoid(float l) {
  return (float)(1.0 / (1.0 + exp(-(double)l)));
}

// Total order key: larger = ranks first.  High word: the biased score's bits
// made unsigned-orderable (NaN -> 0, below everything); low word: ~id, so on
// equal scores the lower id wins.
__device__ __forceinline__ uint64_t topk_key(float sb, int e) {
  uint32_t u;
  if (sb != sb) {
    u = 0u;
  } else {
    u = __float_as_uint(sb + 0.0f);  // -0 -> +0
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  }
  return ((uint64_t)u << 32) | (uint32_t)(~(uint32_t)e);
}

// One wavefront ranks token t.  The logit of expert e is the sum of the
// `splits` K-slice partials partial[s][t][e] in slice order (fixed, so
// reruns repeat); with splits > 1 it is also written to logits[t][e].
// TK_PER_LANE = ceil(E/64) experts per lane, as 64-bit keys; k wave-wide
// arg-max rounds pick the winners.  TK_SLICES partial loads are in flight
// per expert (registers against round trips).  Lanes j < k write pick j's rank-ordered
// id and weight; the function returns the id (lane < k) and its slot.
template <int TK_PER_LANE, int TK_SLICES = (TK_PER_LANE <= 4 ? 16 : 64 / TK_PER_LANE)>
__device__ __forceinline__ void topk_token(const float* __restrict__ partial, int splits,
                                           float* __restrict__ logits,
                                           const float* __restrict__ bias,
                                           int32_t* __restrict__ ids, float* __restrict__ wts,
                                           int64_t t, int64_t T, int E, int k, float rsf,
                                           int lane, int& out_id, int& out_slot) {
  const int64_t TE = T * E;
  uint64_t key[TK_PER_LANE];
  float lg[TK_PER_LANE];
#pragma unroll
  for (int i = 0; i < TK_PER_LANE; ++i) {
    const int e = lane + 64 * i;
    key[i] = 0;
    lg[i] = 0.f;
    if (e < E) {
      // the K-slice partials, TK_SLICES loads in flight (one round trip for
      // the usual slice counts), summed in slice order
      float l = 0.f;
      for (int sp0 = 0; sp0 < splits; sp0 += TK_SLICES) {
        float pv[TK_SLICES];
#pragma unroll
        for (int u = 0; u < TK_SLICES; ++u)
          pv[u] = sp0 + u < splits ? partial[(sp0 + u) * TE + t * E + e] : 0.f;
#pragma unroll
        for (int u = 0; u < TK_SLICES; ++u)
          if (sp0 + u < splits) l = sp0 + u == 0 ? pv[u] : l + pv[u];
      }
      if (splits > 1) logits[t * E + e] = l;
      lg[i] = l;
      const float s = topk_sigmoid(l);
      const float b = bias ? bias[e] : 0.0f;
      key[i] = topk_key(s + b, e);
    }
  }
  int mine = -1;       // lane j < k ends up holding the j-th pick
  float mine_l = 0.f;  // and its logit
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < TK_PER_LANE; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_u64(best);
    const int e = (int)(~(uint32_t)best);
    float le = 0.f;
#pragma unroll
    for (int i = 0; i < TK_PER_LANE; ++i) {
      if (key[i] == best) {
        key[i] = 0;  // taken: 0 is below every real key
        le = lg[i];
      }
    }
    le = __shfl(le, e & 63, MOE_WAVE);  // the owner lane of expert e holds its logit
    if (lane == j) {
      mine = e;
      mine_l = le;
    }
  }
  // ascending order: rank of each pick among the k picks
  int rank = 0;
  for (int i = 0; i < k; ++i) {
    const int other = __shfl(mine, i, MOE_WAVE);
    rank += (lane < k && other < mine) ? 1 : 0;
  }
  if (lane < k) {
    ids[t * k + rank] = mine;
    wts[t * k + rank] = rsf * topk_sigmoid(mine_l);
  }
  out_id = mine;
  out_slot = rank;
}
