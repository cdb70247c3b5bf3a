// Workgroup-wide temperature / top-k sampling of one logit row.
//
// "PersonaPlex native LM audit", section 7 'One exact generator step' and the sampling
// defaults after it: the generator samples text over the 25 largest logits at
// temperature 0.7 and audio over the 250 largest at temperature 0.8. The page gives the
// parameters, not the procedure; this file implements the plain reading:
//   candidates = the top_k logits ordered by value, larger first, equal values by lower
//   index; weights w_i = exp((l_i - l_0) / temperature) in float64; the draw u in [0, 1)
//   returns the first candidate whose running sum w_0 + .. + w_i (added left to right)
//   exceeds u * (w_0 + .. + w_{k-1}).
// top_k <= 1 or temperature <= 0 selects the largest logit (lowest index on ties).
//
// Steps, all inside one workgroup of NT threads, thread t holding the logits
// i = j*NT + t, j < PER (coalesced loads):
//   1. map each float to an unsigned key with the same order (-0 and +0 share one key);
//   2. find the k-th largest key T two bits at a time from the top: the next two bits of
//      T are the largest d in 0..3 for which at least k keys are >= (T's higher bits, d,
//      zeros) -- per-wave counts, one workgroup total of three thresholds per step;
//   3. take every key > T; among the keys == T keep the lowest indices still needed,
//      found (only when there are more ties than needed) as the smallest index I with
//      enough ties at or below it, by the same bitwise search over index bits;
//   4. gather the k taken (key, index) pairs into LDS in any order as one 64-bit word
//      (key, then the complemented index: a larger word comes first) and rank-sort them;
//   5. float64 weights in parallel, running sums by one thread in candidate order (the
//      fixed left-to-right order of the definition), the first crossing found in parallel.
#pragma once

#include "device.h"
#include "internal.h"

namespace pp {

struct SampleLds {
  uint64_t comp[kMaxTopK]; // taken (key << 32 | ~index), gathered in any order, zero-padded
  float val[kMaxTopK];     // candidates in sampling order
  int32_t sidx[kMaxTopK];
  double w[kMaxTopK];      // weights, zero-padded to a multiple of 16
  double cs[kMaxTopK];     // running sums
  uint32_t red[2][3][16];
  int32_t cnt;
  int32_t pick;
};

// Order-preserving map of float32 onto uint32: a larger float gives a larger key.
__device__ __forceinline__ uint32_t order_key(float v) {
  const uint32_t u = __float_as_uint(v == 0.f ? 0.f : v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Integer sum over the 64 lanes, returned wave-uniform: DPP sums within each row of 16
// lanes, then the four row sums read into scalar registers.
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);   // lane ^ 1
  v += (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);   // lane ^ 2
  v += (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false);  // mirror within 8
  v += (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false);  // mirror within 16
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 0) + (uint32_t)__builtin_amdgcn_readlane((int)v, 16) +
         (uint32_t)__builtin_amdgcn_readlane((int)v, 32) + (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
}

// Per-wave counting of predicates over a thread's elements. With few waves the ballot
// masks' population counts on the scalar unit are the cheapest; with 16 waves the scalar
// unit is shared too widely, and per-lane sums reduced once per wave win.
template <int NT>
struct WaveCounter {
  uint32_t v = 0;
  __device__ __forceinline__ void add(bool pred) {
    if constexpr (NT <= 256) v += (uint32_t)__popcll(__ballot(pred));
    else v += pred ? 1u : 0u;
  }
  __device__ __forceinline__ uint32_t total() const {
    if constexpr (NT <= 256) return v;
    else return wave_sum_u32(v);
  }
};

// Workgroup totals of three wave-uniform counters with one barrier; `red` alternates
// between two halves so that consecutive calls need no second barrier.
template <int NT>
__device__ __forceinline__ void block_count3(uint32_t a, uint32_t b, uint32_t c, uint32_t (*red)[3][16],
                                             int parity, uint32_t& ta, uint32_t& tb, uint32_t& tc) {
  if ((threadIdx.x & 63) == 0) {
    red[parity][0][threadIdx.x >> 6] = a;
    red[parity][1][threadIdx.x >> 6] = b;
    red[parity][2][threadIdx.x >> 6] = c;
  }
  __syncthreads();
  ta = tb = tc = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    ta += red[parity][0][i];
    tb += red[parity][1][i];
    tc += red[parity][2][i];
  }
}

// Returns the selected index in every thread. Requires 1 <= n <= NT * PER <= 32768,
// finite logits, top_k <= kMaxTopK; u in [0, 1). Every thread of the workgroup must call it.
template <int NT, int PER>
__device__ __forceinline__ int block_sample_top_k(const float* __restrict__ lg, int n, float temperature,
                                                  int top_k, double u, SampleLds& s) {
  static_assert(NT % 64 == 0 && NT <= 1024 && NT * PER <= 32768, "workgroup size");
  const int tid = threadIdx.x;
  const bool greedy = top_k <= 1 || !(temperature > 0.f);
  const int k = greedy ? 1 : min(top_k, n);

  // Every logit load is issued before the first is used: indices past n read the last
  // logit (no branch around a load, which would make each wait for the one before) and
  // take key 0, below every finite or infinite key.
  float lv[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = j * NT + tid;
    lv[j] = lg[i < n ? i : n - 1];
  }
  uint32_t key[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) key[j] = j * NT + tid < n ? order_key(lv[j]) : 0u;
  if (tid == 0) s.cnt = 0;

  // 2. T = the k-th largest key; each wave counts with ballots.
  uint32_t T = 0;
  int parity = 0;
  for (int b = 30; b >= 0; b -= 2, parity ^= 1) {
    const uint32_t c1 = T | (1u << b), c2 = T | (2u << b), c3 = T | (3u << b);
    WaveCounter<NT> n1, n2, n3;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      n1.add(key[j] >= c1);
      n2.add(key[j] >= c2);
      n3.add(key[j] >= c3);
    }
    uint32_t t1, t2, t3;
    block_count3<NT>(n1.total(), n2.total(), n3.total(), s.red, parity, t1, t2, t3);
    const uint32_t kk = (uint32_t)k;
    T = t3 >= kk ? c3 : t2 >= kk ? c2 : t1 >= kk ? c1 : T;
  }

  // 3. keys > T all taken; ties at T by lowest index.
  WaveCounter<NT> gt, eq;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    gt.add(key[j] > T);
    eq.add(key[j] == T);
  }
  uint32_t G, E, unused;
  block_count3<NT>(gt.total(), eq.total(), 0u, s.red, parity, G, E, unused);
  parity ^= 1;
  const uint32_t need = (uint32_t)k - G;   // 1 <= need <= E
  int last = 0x7fffffff;                   // ties with index <= last are taken
  if (E > need) {
    // smallest X with #(ties with index <= X) >= need: grow X from the top bit, keeping
    // #(ties with index < X) < need
    uint32_t X = 0;
    for (int b = 14; b >= 0; --b, parity ^= 1) {
      const uint32_t cand = X | (1u << b);
      WaveCounter<NT> c;
#pragma unroll
      for (int j = 0; j < PER; ++j) c.add(key[j] == T && (uint32_t)(j * NT + tid) < cand);
      uint32_t tc, u1, u2;
      block_count3<NT>(c.total(), 0u, 0u, s.red, parity, tc, u1, u2);
      if (tc < need) X = cand;
    }
    last = (int)X;
  }

  // 4. gather, then rank sort: larger words first (key desc, index asc).
  const int k8 = (k + 7) & ~7;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = j * NT + tid;
    if (key[j] > T || (key[j] == T && i <= last)) {
      const int p = atomicAdd(&s.cnt, 1);
      s.comp[p] = ((uint64_t)key[j] << 32) | (uint64_t)(~(uint32_t)i);
    }
  }
  if (tid < k8 - k) s.comp[k + tid] = 0;   // never ahead of a taken word (keys are > 0)
  __syncthreads();
  for (int i = tid; i < k; i += NT) {
    const uint64_t ci = s.comp[i];
    int r = 0;
    for (int j0 = 0; j0 < k8; j0 += 8) {
      uint64_t cj[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) cj[e] = s.comp[j0 + e];
#pragma unroll
      for (int e = 0; e < 8; ++e) r += cj[e] > ci ? 1 : 0;
    }
    s.val[r] = key_float((uint32_t)(ci >> 32));
    s.sidx[r] = (int)(~(uint32_t)ci);
  }
  __syncthreads();
  if (greedy) return s.sidx[0];

  // 5. weights, running sums, draw.
  constexpr int CH = 16;   // weights read ahead of the dependent additions
  const int k16 = (k + CH - 1) & ~(CH - 1);
  const double top = (double)s.val[0], t = (double)temperature;
  for (int i = tid; i < k16; i += NT) s.w[i] = i < k ? exp(((double)s.val[i] - top) / t) : 0.0;
  __syncthreads();
  if (tid == 0) {
    double acc = 0.0;
    for (int i0 = 0; i0 < k16; i0 += CH) {
      double wv[CH];
#pragma unroll
      for (int e = 0; e < CH; ++e) wv[e] = s.w[i0 + e];
#pragma unroll
      for (int e = 0; e < CH; ++e) {
        acc += wv[e];   // the zero padding leaves the sums past k at the total
        s.cs[i0 + e] = acc;
      }
    }
    s.pick = s.sidx[k - 1];   // only kept if u * total rounds up to the total
  }
  __syncthreads();
  const double r = u * s.cs[k - 1];
  for (int i = tid; i < k; i += NT)
    if (s.cs[i] > r && (i == 0 || !(s.cs[i - 1] > r))) s.pick = s.sidx[i];
  __syncthreads();
  return s.pick;
}

}  // namespace pp
