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
// Steps, all inside one workgroup of NT threads, thread t owning the PER consecutive
// logits [t*PER, t*PER+PER):
//   1. map each float to an unsigned key with the same order (-0 and +0 share one key);
//   2. find the k-th largest key T bit by bit from the top: bit b of T is set when at
//      least k keys are >= (T's higher bits, 1, zeros) -- one workgroup count per bit;
//   3. one exclusive scan of (count > T, count == T) in index order places every key > T
//      and the lowest-index keys == T that are still needed into an LDS list of k entries,
//      in index order;
//   4. a rank sort of that list by (key desc, list position asc);
//   5. float64 weights in parallel, running sums by one thread in candidate order (the
//      fixed left-to-right order of the definition), the first crossing found in parallel.
#pragma once

#include "device.h"
#include "internal.h"

namespace pp {

struct SampleLds {
  uint32_t key[kMaxTopK];  // selected keys, in index order
  int32_t idx[kMaxTopK];
  float val[kMaxTopK];     // candidates in sampling order
  int32_t sidx[kMaxTopK];
  double c[kMaxTopK];      // weights, then running sums
  float red[2][16];
  uint32_t scan[16];
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

// Workgroup sum of small integer counts (exact in float32 below 2^24) with one barrier;
// `red` alternates between two halves so that consecutive calls need no second barrier.
template <int NT>
__device__ __forceinline__ uint32_t block_count(uint32_t v, float (*red)[16], int parity) {
  const float w = wave_sum((float)v);
  if ((threadIdx.x & 63) == 0) red[parity][threadIdx.x >> 6] = w;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) t += red[parity][i];
  return (uint32_t)t;
}

// Exclusive prefix sum over threads in thread order; *total receives the workgroup sum.
// The caller synchronises before `scan` is used again.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* scan, uint32_t* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  if (lane == 63) scan[w] = x;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    const uint32_t s = scan[i];
    before += i < w ? s : 0u;
    tot += s;
  }
  *total = tot;
  return before + x - v;
}

// Returns the selected index in every thread. Requires 1 <= n <= NT * PER, finite
// logits, top_k <= kMaxTopK; u in [0, 1). Every thread of the workgroup must call it.
template <int NT, int PER>
__device__ __forceinline__ int block_sample_top_k(const float* __restrict__ lg, int n, float temperature, int top_k, double u,
                                  SampleLds& s) {
  static_assert(NT % 64 == 0 && NT <= 1024, "workgroup size");
  const int tid = threadIdx.x;
  const bool greedy = top_k <= 1 || !(temperature > 0.f);
  const int k = greedy ? 1 : min(top_k, n);

  uint32_t key[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = tid * PER + j;
    key[j] = i < n ? order_key(lg[i]) : 0u;   // 0 is below every finite or infinite key
  }

  // 2. T = the k-th largest key.
  uint32_t T = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = T | (1u << b);
    uint32_t cnt = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) cnt += key[j] >= cand ? 1u : 0u;
    if (block_count<NT>(cnt, s.red, b & 1) >= (uint32_t)k) T = cand;
  }

  // 3. compaction in index order: all keys > T, then the lowest-index ties still needed.
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    gt += key[j] > T ? 1u : 0u;
    eq += key[j] == T ? 1u : 0u;
  }
  uint32_t tot;
  const uint32_t before = block_excl_scan<NT>((gt << 16) | eq, s.scan, &tot);
  const int need_eq = k - (int)(tot >> 16);
  int g0 = (int)(before >> 16), e0 = (int)(before & 0xffffu);
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const uint32_t kj = key[j];
    if (kj > T) {
      const int p = g0 + min(e0, need_eq);
      s.key[p] = kj;
      s.idx[p] = tid * PER + j;
      ++g0;
    } else if (kj == T) {
      if (e0 < need_eq) {
        const int p = g0 + e0;
        s.key[p] = kj;
        s.idx[p] = tid * PER + j;
      }
      ++e0;
    }
  }
  __syncthreads();

  // 4. rank sort: larger keys first; equal keys keep list (= index) order.
  for (int i = tid; i < k; i += NT) {
    const uint32_t ki = s.key[i];
    int r = 0;
    for (int j = 0; j < k; ++j) {
      const uint32_t kj = s.key[j];
      r += (kj > ki || (kj == ki && j < i)) ? 1 : 0;
    }
    s.val[r] = key_float(ki);
    s.sidx[r] = s.idx[i];
  }
  __syncthreads();
  if (greedy) return s.sidx[0];

  // 5. weights, running sums, draw.
  const double top = (double)s.val[0], t = (double)temperature;
  for (int i = tid; i < k; i += NT) s.c[i] = exp(((double)s.val[i] - top) / t);
  __syncthreads();
  if (tid == 0) {
    double acc = 0.0;
    for (int i = 0; i < k; ++i) {
      acc += s.c[i];
      s.c[i] = acc;
    }
    s.pick = s.sidx[k - 1];   // only reached if u * total rounds up to the total
  }
  __syncthreads();
  const double r = u * s.c[k - 1];
  for (int i = tid; i < k; i += NT)
    if (s.c[i] > r && (i == 0 || !(s.c[i - 1] > r))) s.pick = s.sidx[i];
  __syncthreads();
  return s.pick;
}

}  // namespace pp
