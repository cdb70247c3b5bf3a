// Keys and values of the memory bank for the memory readers ("Current sequence memory:
// one writer, four readers", section 6: K = M W_K^T + b_K, V = M W_V^T + b_V over the
// visible memory rows). They depend on the memory only, so they are formed once when rows
// are written and stored like the temporal ring ([heads][slots][d_head]); every decode step
// then reads them with the ring attention kernel.
#include "device.h"
#include "internal.h"

namespace pp {

// 64 slots x 64 outputs per workgroup, 256 threads, 4 x 4 per thread, float32 FMA over
// 16-wide slices of the row staged in LDS.
template <typename WT>
__global__ __launch_bounds__(kBlock) void k_reader_kv(ReaderKvArgs a) {
  __shared__ float Ms[64][17], Ws[64][17];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int n_to = a.D / 64;
  const int ts = blockIdx.x / n_to, to = blockIdx.x % n_to;
  const WT* M = static_cast<const WT*>(a.mem);
  const WT* W = static_cast<const WT*>(a.W);
  float acc[4][4] = {};
  for (int j0 = 0; j0 < a.mem_dim; j0 += 16) {
    for (int i = tid; i < 64 * 16; i += kBlock) {
      const int r = i >> 4, kk = i & 15;
      const int sl = ts * 64 + r;
      Ms[r][kk] = sl < a.n ? Elem<WT>::load1(M + (size_t)sl * a.mem_dim + j0 + kk) : 0.f;
      Ws[r][kk] = Elem<WT>::load1(W + (size_t)(to * 64 + r) * a.mem_dim + j0 + kk);
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] += Ms[4 * ty + r][kk] * Ws[4 * tx + c][kk];
    __syncthreads();
  }
  WT* out = static_cast<WT*>(a.out);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int sl = ts * 64 + 4 * ty + r;
    if (sl >= a.n) continue;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int o = to * 64 + 4 * tx + c;
      const int h = o / a.dh, d = o - h * a.dh;
      Elem<WT>::store1(out + ((size_t)h * a.max_slots + a.slot0 + sl) * a.dh + d, acc[r][c] + a.bias[o]);
    }
  }
}

hipError_t launch_reader_kv(const ReaderKvArgs& a, bool bf16, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  if (a.D % 64 || a.mem_dim % 16 || a.slot0 < 0 || a.slot0 + a.n > a.max_slots || a.D % a.dh) return hipErrorInvalidValue;
  const dim3 grid(((a.n + 63) / 64) * (a.D / 64));
  if (bf16) hipLaunchKernelGGL(k_reader_kv<bf16_t>, grid, dim3(kBlock), 0, s, a);
  else hipLaunchKernelGGL(k_reader_kv<float>, grid, dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

}  // namespace pp
