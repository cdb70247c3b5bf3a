// Layout of the float16 activation operands of the skinny matrix products (batched decode).
#pragma once

#include <hip/hip_runtime.h>

#include <stddef.h>

namespace pp {

// The activations are kept in the order the products' MFMA fragments read them: 16-session
// tiles, then 32-element k-steps, then 64 lanes of 8 values, lane = session % 16 +
// 16 * ((k % 32) / 8). Element (b, k) of a [B][K] matrix (K a multiple of 32) sits at this
// index; a wave's load of one tile and step is 1 KB of contiguous memory.
__device__ __forceinline__ size_t frag_act_index(int b, int k, int K) {
  return ((((size_t)(b >> 4) * (size_t)(K >> 5) + (size_t)(k >> 5)) * 64 + (size_t)((b & 15) + 16 * ((k & 31) >> 3))) << 3) +
         (size_t)(k & 7);
}

}  // namespace pp
