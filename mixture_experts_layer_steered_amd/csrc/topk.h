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

// The correction bias of lane L's experts L + 64 i (0 past E or without a
// bias), loaded once and kept in registers across tokens.
template <int TK_PER_LANE>
__device__ __forceinline__ void topk_bias(const float* __restrict__ bias, int E, int lane,
                                          float (&bv)[TK_PER_LANE]) {
#pragma unroll
  for (int i = 0; i < TK_PER_LANE; ++i) {
    const int e = lane + 64 * i;
    bv[i] = (bias && e < E) ? bias[e] : 0.0f;
  }
}

// The selection of one token by one wavefront from its logits in
// registers: lane L holds experts L + 64 i (i < TK_PER_LANE) as lg[i] (lanes
// past E hold anything; only e < E ranks) and their biases as bv[i].  k wave-wide arg-max rounds over
// 64-bit keys pick the winners; the picks' ids and weights go to ids / wts
// of token t in ascending id order, the ids also to ids_copy when it is
// not null (the same layout, e.g. in LDS).
//
// With at most two experts per lane (E <= 128) the selection is a
// threshold search instead: the k-th largest score is found bit by bit with
// one ballot per bit (and per half), the experts above it are picked, and
// ties at it go to the lowest ids; a pick's slot is the number of picks
// with a lower id (one ballot per half).  The keys order scores first and
// ids second, so both forms pick the same experts.
template <int TK_PER_LANE>
__device__ __forceinline__ void topk_select(const float (&lg)[TK_PER_LANE],
                                            const float (&bv)[TK_PER_LANE],
                                            int32_t* __restrict__ ids, float* __restrict__ wts,
                                            int32_t* ids_copy, int64_t t, int E, int k, float rsf,
                                            int lane) {
  uint64_t key[TK_PER_LANE];
  float sg[TK_PER_LANE];  // the unbiased scores: the emitted weights reuse them
#pragma unroll
  for (int i = 0; i < TK_PER_LANE; ++i) {
    const int e = lane + 64 * i;
    key[i] = 0;
    sg[i] = 0.f;
    if (e < E) {
      sg[i] = topk_sigmoid(lg[i]);
      key[i] = topk_key(sg[i] + bv[i], e);
    }
  }
  if constexpr (TK_PER_LANE <= 2) {
    // the high words of the keys (the orderable scores; 0 for NaN), lanes
    // past E excluded: the k-th largest score thr is the largest value with
    // at least k scores >= it, found bit by bit from the top with one ballot
    // per bit; the picks are every score above thr and, of those equal to
    // it, the lowest ids (the order of the full keys)
    uint32_t kv[TK_PER_LANE];
    bool valid[TK_PER_LANE];
#pragma unroll
    for (int i = 0; i < TK_PER_LANE; ++i) {
      valid[i] = lane + 64 * i < E;
      kv[i] = (uint32_t)(key[i] >> 32);
    }
    uint32_t thr = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = thr | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int i = 0; i < TK_PER_LANE; ++i) cnt += __popcll(__ballot(valid[i] && kv[i] >= cand));
      if (cnt >= k) thr = cand;
    }
    uint64_t above[TK_PER_LANE], eq[TK_PER_LANE];
    int need = k;  // picks still to make among the scores equal to thr
#pragma unroll
    for (int i = 0; i < TK_PER_LANE; ++i) {
      above[i] = __ballot(valid[i] && kv[i] > thr);
      eq[i] = __ballot(valid[i] && kv[i] == thr);
      need -= __popcll(above[i]);
    }
    const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int before = 0, eq_before = 0;  // picks and ties in the halves of lower ids
#pragma unroll
    for (int i = 0; i < TK_PER_LANE; ++i) {
      const int e = lane + 64 * i;
      const bool is_above = (above[i] >> lane) & 1ull;
      const bool is_eq = (eq[i] >> lane) & 1ull;
      const bool pick = is_above || (is_eq && eq_before + __popcll(eq[i] & lower) < need);
      const uint64_t picks = __ballot(pick);
      if (pick) {
        const int slot = before + __popcll(picks & lower);
        ids[t * k + slot] = e;
        wts[t * k + slot] = rsf * sg[i];
        if (ids_copy) ids_copy[t * k + slot] = e;
      }
      before += __popcll(picks);
      eq_before += __popcll(eq[i]);
    }
    return;
  }
  int mine = -1;       // lane j < k ends up holding the j-th pick
  float mine_s = 0.f;  // and its unbiased score
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < TK_PER_LANE; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_u64(best);
    const int e = (int)(~(uint32_t)best);
    float se = 0.f;
#pragma unroll
    for (int i = 0; i < TK_PER_LANE; ++i) {
      if (key[i] == best) {
        key[i] = 0;  // taken: 0 is below every real key
        se = sg[i];
      }
    }
    se = __shfl(se, e & 63, MOE_WAVE);  // the owner lane of expert e holds its score
    if (lane == j) {
      mine = e;
      mine_s = se;
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
    wts[t * k + rank] = rsf * mine_s;
    if (ids_copy) ids_copy[t * k + rank] = mine;
  }
}

// One wavefront ranks token t from the router GEMM's K-slice partials: the
// logit of expert e is the sum of the `splits` partials partial[s][t][e] in
// slice order (fixed, so reruns repeat); with splits > 1 it is also written
// to logits[t][e].  TK_SLICES partial loads are in flight per expert
// (registers against round trips).
template <int TK_PER_LANE, int TK_SLICES = (TK_PER_LANE <= 4 ? 16 : 64 / TK_PER_LANE)>
__device__ __forceinline__ void topk_token(const float* __restrict__ partial, int splits,
                                           float* __restrict__ logits,
                                           const float* __restrict__ bias,
                                           int32_t* __restrict__ ids, float* __restrict__ wts,
                                           int64_t t, int64_t T, int E, int k, float rsf,
                                           int lane) {
  const int64_t TE = T * E;
  float bv[TK_PER_LANE];
  topk_bias<TK_PER_LANE>(bias, E, lane, bv);  // in flight with the partials
  float lg[TK_PER_LANE];
#pragma unroll
  for (int i = 0; i < TK_PER_LANE; ++i) {
    const int e = lane + 64 * i;
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
    }
  }
  topk_select<TK_PER_LANE>(lg, bv, ids, wts, nullptr, t, E, k, rsf, lane);
}
