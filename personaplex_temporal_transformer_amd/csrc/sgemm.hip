// Skinny matrix products for batched decode: B sessions (B <= 64) at one position share
// every weight byte the step streams ("PersonaPlex native LM audit", section 3: the
// per-block linears of the temporal step, with the batch as the tensors' leading axis).
//
// out[b][n] = sum_k act[b][k] W[n][k]. A workgroup owns 16 output columns (for SiLU-gated
// rows: 8 g rows and their 8 z rows) over all of K; its 8 waves split K into equal runs of
// 32-element steps, taken in groups of U steps with the next group's loads in flight
// while the current one is multiplied. Per step a lane takes 8 weights of one row (bf16,
// widened to float16 in registers) and 8 activations of one session per 16-session tile,
// and issues one v_mfma_f32_16x16x32_f16 per tile: A = activations (row = session
// lane % 16, k = 8 * (lane / 16) + e), B = weights (column = lane % 16, same k), so the
// lane holds D[session 4 * (lane / 16) + i][column lane % 16]. The weights are read from a
// copy packed once per model in exactly that fragment order -- tile, 32-element step,
// lane, 8 elements -- so each load instruction of a wave reads 1 KB of contiguous memory
// (the row-major matrix would give 16 rows x 64 bytes per instruction). The float16
// activations are written in the same order by their producers (the row RMSNorm, the
// attention combine and this file's SiLU-product epilogue; frag_act_index), so their loads
// are 1 KB contiguous as well (row-major [B][K] they were 16 rows x 64 bytes, and the
// batched step took 3-16 % longer at B = 16-64); up to 8 sessions, the products that
// follow a row norm form it themselves into LDS (NORM below). The waves' partial tiles
// are summed in LDS in wave order (fixed order: reproducible), then the epilogue applies
// RoPE / ring append, the residual add, the SiLU product or a plain store.
#include <cmath>

#include "device.h"
#include "frag_layout.h"
#include "internal.h"

namespace pp {

constexpr int kSgWaves = 8;

// BAL: the grid has one workgroup per CU (at most), and workgroup b owns the contiguous
// column tiles [b * tiles / grid, (b + 1) * tiles / grid) -- at most NT of them, nt at run
// time -- so every CU streams an equal share; otherwise workgroup b owns tiles b*NT ..
// b*NT + NT-1.
// NORM (one session tile, B <= kSgemmNormMaxBatch, K <= kSgemmNormMaxK): the activations
// are the RMSNorm of the float32 rows a.xin ("PersonaPlex native LM audit", section 3: the
// pre-norm of the block's attention and gated-MLP halves), formed by every workgroup: the
// rows are loaded ahead of the first weights, each session's sum of squares is reduced
// (per thread, then per wave, then over the waves in wave order) while those weights are in
// flight, and the normalised rows are written to LDS as float16 fragments, which the
// product then reads in place of a.act. This replaces a separate row-norm launch per
// product; at small B re-reading B rows per workgroup (served by the L2) costs less than
// the launch.
template <int EPI, int NBT, int NT, bool BAL, bool NORM>
__global__ __launch_bounds__(kSgWaves * 64) void k_sgemm(SgemmArgs a) {
  static_assert(!NORM || (NBT == 1 && BAL), "the RMSNorm prologue serves one session tile");
  constexpr int BN = kSgemmNormMaxBatch;
  __shared__ float red[kSgWaves][NT * NBT][64][4];
  __shared__ float tile[NBT * 16][NT * 16 + 1];
  // NORM: float16 fragments of the normalised rows, [32-element step][k group][session][8]
  __shared__ u32x4 act_lds[NORM ? kSgemmNormMaxK / 32 * 4 * BN : 1];
  __shared__ float red_n[NORM ? kSgWaves : 1][BN];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;
  const int nsteps = a.K / 32;
  const int tiles = EPI == SEPI_SWIGLU ? a.F / 8 : a.N / 16;
  const int tile0 = BAL ? (int)((long long)blockIdx.x * tiles / gridDim.x) : (int)blockIdx.x * NT;
  const int nt = BAL ? (int)((long long)(blockIdx.x + 1) * tiles / gridDim.x) - tile0 : NT;   // <= NT
  // packed fragments of this workgroup's tiles: [tile][step][lane][8]
  const uint16_t* Wr = static_cast<const uint16_t*>(a.W) + ((size_t)tile0 * nsteps * 64 + lane) * 8;
  const size_t tstride = (size_t)nsteps * 512;
  const int s0 = w * nsteps / kSgWaves, s1 = (w + 1) * nsteps / kSgWaves;
  // this lane's activation fragments in each session tile (fragment order: tile, step,
  // lane, 8 values -- frag_act_index); lanes of sessions past B read zeros
  bool live[NBT];
#pragma unroll
  for (int t = 0; t < NBT; ++t) live[t] = t * 16 + n < a.B;
  // No load below sits under a branch, so the compiler waits for each group of loads alone
  // (a load under a branch makes it wait for all outstanding loads, which would drain the
  // next group's prefetch): lanes of sessions past B read their activations through a
  // buffer resource at an offset past its end, which returns zeros without memory traffic
  // (in LDS: a slot of a live session, then zeroed); column tiles past nt re-read tile
  // nt - 1 and their products are dropped.
  const auto act_rs = make_rsrc(NORM ? nullptr : a.act, (uint32_t)(NBT * nsteps * 1024));
  const int dead_off = 1 << 30;   // past any activation buffer (at most 4 x 352 x 1 KB)
  // this lane's activation fragment of step st in session tile t
  auto load_act = [&](int t, int st) -> u32x4 {
    if constexpr (NORM) {
      const u32x4 v = act_lds[(st * 4 + (lane >> 4)) * BN + (n < BN ? n : BN - 1)];
      return live[0] ? v : u32x4{0u, 0u, 0u, 0u};
    } else {
      const int off = ((t * nsteps + st) * 64 + lane) * 16 + (live[t] ? 0 : dead_off);
      return __builtin_amdgcn_raw_buffer_load_b128(act_rs, off, 0, 0);
    }
  };
  // this lane's weight fragment of step st in column tile j of the workgroup
  auto wptr = [&](int j, int st) { return Wr + (j < nt ? j : nt - 1) * tstride + (size_t)st * 512; };
  f32x4 acc[NT][NBT];
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int t = 0; t < NBT; ++t) acc[j][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // groups of U steps, the next group's loads issued before the current group is
  // multiplied (loads complete in issue order, so the wait for a group is exact)
  constexpr int U = NT * NBT == 1 ? 8 : (NT * NBT == 2 ? 4 : 2);
  u32x4 wv[2][U][NT], av[2][U][NBT];
  auto load_w = [&](int buf, int st0) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < NT; ++j) wv[buf][u][j] = load_stream(wptr(j, st0 + u));
  };
  auto load_a = [&](int buf, int st0) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < NBT; ++t) av[buf][u][t] = load_act(t, st0 + u);
  };
  auto load_group = [&](int buf, int st0) {
    if constexpr (NORM) {
      load_w(buf, st0);
      load_a(buf, st0);
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int j = 0; j < NT; ++j) wv[buf][u][j] = load_stream(wptr(j, st0 + u));
#pragma unroll
        for (int t = 0; t < NBT; ++t) av[buf][u][t] = load_act(t, st0 + u);
      }
    }
  };
  auto mul_group = [&](int buf) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const f16x8 wf = bf16x8_to_f16(wv[buf][u][j]);
#pragma unroll
        for (int t = 0; t < NBT; ++t)
          acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, av[buf][u][t]), wf, acc[j][t], 0, 0, 0);
      }
  };
  const int ng = (s1 - s0) / U;
  int gi0 = 0;   // first group of the main loop
  if constexpr (NORM) {
    // rows and scales first, then the first weights, so the reductions below wait for the
    // rows alone. The rows are buffer loads bounded by the B rows: the loads of rows past B
    // (and of k past K) return zeros without memory traffic, and none sits under a branch.
    constexpr int NX = kSgemmNormMaxK / (kSgWaves * 64 * 4);   // float4 per thread and row
    const int K = a.K;
    const auto xr = make_rsrc(a.xin, (uint32_t)((size_t)a.B * K * 4));
    const auto ar = make_rsrc(a.alpha, (uint32_t)K * 4);
    f32x4 xv[BN][NX], al[NX];
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      const int k = (i * kSgWaves * 64 + tid) * 4;
      const int kk = k < K ? k : 1 << 24;   // k past K: past every row, a zero read
      al[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ar, kk * 4, 0, 0));
#pragma unroll
      for (int b = 0; b < BN; ++b)
        xv[b][i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, (b * K + kk) * 4, 0, 0));
    }
    // the first two groups' weights, both buffers (with no branch around them, so that
    // the reductions below wait for the rows alone; steps past the wave's run load its
    // last step again and are never used): they stream while the norm is formed
#pragma unroll
    for (int g2 = 0; g2 < 2; ++g2)
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const int st = s0 + g2 * U + u;
          wv[g2][u][j] = load_stream(wptr(j, st < nsteps ? st : nsteps - 1));
        }
    float ss[BN];
#pragma unroll
    for (int b = 0; b < BN; ++b) {
      ss[b] = 0.f;
#pragma unroll
      for (int i = 0; i < NX; ++i) {
        const f32x4 v = xv[b][i];
        const float q = v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
        ss[b] += (i * kSgWaves * 64 + tid) * 4 < K ? q : 0.f;
      }
      ss[b] = wave_sum(ss[b]);
    }
    if (lane == 0) {
#pragma unroll
      for (int b = 0; b < BN; ++b) red_n[w][b] = ss[b];
    }
    lds_barrier();
    const float osc = ldexpf(1.0f, -a.act_exp);   // the float16 operand's scale (a power of two)
    uint2* al2 = reinterpret_cast<uint2*>(act_lds);
#pragma unroll
    for (int b = 0; b < BN; ++b) {
      float tot = 0.f;
#pragma unroll
      for (int ww = 0; ww < kSgWaves; ++ww) tot += red_n[ww][b];
      const float r = 1.0f / sqrtf(tot / (float)K + a.eps);
#pragma unroll
      for (int i = 0; i < NX; ++i) {
        const int k = (i * kSgWaves * 64 + tid) * 4;   // four consecutive k: one half fragment
        if (b < a.B && k < K) {
          const f32x4 y = ((xv[b][i] * r) * al[i]) * osc;
          const uint32_t lo = (uint32_t)f32_to_f16(y.x) | ((uint32_t)f32_to_f16(y.y) << 16);
          const uint32_t hi = (uint32_t)f32_to_f16(y.z) | ((uint32_t)f32_to_f16(y.w) << 16);
          al2[(((k >> 5) * 4 + ((k & 31) >> 3)) * BN + b) * 2 + ((k & 7) >> 2)] = make_uint2(lo, hi);
        }
      }
    }
    lds_barrier();
    // the first iteration of the loop below, with both groups' weights already loaded
    if (ng > 0) {
      load_a(0, s0);
      if (ng > 1) load_a(1, s0 + U);
      mul_group(0);
      if (ng > 1) {
        if (ng > 2) load_group(0, s0 + 2 * U);
        mul_group(1);
      }
    }
    gi0 = 2;
  } else {
    if (ng > 0) load_group(0, s0);
  }
  for (int gi = gi0; gi < ng; gi += 2) {
    if (gi + 1 < ng) load_group(1, s0 + (gi + 1) * U);
    mul_group(0);
    if (gi + 1 < ng) {
      if (gi + 2 < ng) load_group(0, s0 + (gi + 2) * U);
      mul_group(1);
    }
  }
  for (int st = s0 + ng * U; st < s1; ++st) {
    u32x4 a1[NBT];
#pragma unroll
    for (int t = 0; t < NBT; ++t) a1[t] = load_act(t, st);
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const f16x8 wf = bf16x8_to_f16(load_stream(wptr(j, st)));
#pragma unroll
      for (int t = 0; t < NBT; ++t)
        acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a1[t]), wf, acc[j][t], 0, 0, 0);
    }
  }
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int t = 0; t < NBT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[w][j * NBT + t][lane][i] = acc[j][t][i];
  __syncthreads();
  for (int o = tid; o < nt * NBT * 256; o += kSgWaves * 64) {
    const int jt = o >> 8, l = (o >> 2) & 63, i = o & 3;
    const int j = jt / NBT, t = jt - j * NBT;
    float v = 0.f;
#pragma unroll
    for (int ww = 0; ww < kSgWaves; ++ww) v += red[ww][jt][l][i];
    tile[t * 16 + 4 * (l >> 4) + i][j * 16 + (l & 15)] = v;
  }
  __syncthreads();

  // epilogue: thread -> (session b, column c of the workgroup's NT * 16)
  for (int o = tid; o < NBT * 16 * nt * 16; o += kSgWaves * 64) {
    const int b = o / (nt * 16), cc = o - b * (nt * 16);
    if (b >= a.B) continue;
    const int j = cc >> 4, c = cc & 15;
    const int tl = tile0 + j;     // this column's 16-column tile
    const float am = ldexpf(1.0f, a.acc_exp);   // undoes the float16 operand scales (exact)
    const float v = tile[b][cc] * am;
    if constexpr (EPI == SEPI_STORE) {
      a.out[(size_t)b * a.N + tl * 16 + c] = v;
    } else if constexpr (EPI == SEPI_RESID) {
      a.x[(size_t)b * a.N + tl * 16 + c] += v;
    } else if constexpr (EPI == SEPI_SWIGLU) {
      if (c < 8) a.s_out[frag_act_index(b, tl * 8 + c, a.F)] = f32_to_f16(silu(v) * (tile[b][cc + 8] * am) * ldexpf(1.0f, -a.s16_exp));
    } else {
      const int col = tl * 16 + c;
      const int sec = col / a.D, wcol = col - sec * a.D;
      const int head = wcol / a.dh, d = wcol - head * a.dh;
      float y = v;
      if (sec < 2) {
        const float partner = tile[b][cc ^ 1] * am;
        const float cs = a.rope[d & ~1], sn = a.rope[d | 1];
        y = (d & 1) ? partner * sn + v * cs : v * cs - partner * sn;
      }
      if (sec == 0) {
        a.q_out[(size_t)b * a.D + wcol] = y;
      } else {
        const long long pos = a.pos >= 0 ? a.pos : a.state[0];
        uint16_t* ring = static_cast<uint16_t*>(sec == 1 ? a.kc : a.vc) + (size_t)b * a.kv_bstride;
        ring[((size_t)head * a.C + (size_t)(pos % a.C)) * a.dh + d] = f32_to_bf16(y);
      }
    }
  }
}

// Packs W [rows][K] (row-major bf16) into the fragment order above: tile t (16 output
// columns; SiLU-gated: g rows 8t.. and z rows F+8t..), step s, lane l, element e holds
// W[row(t, l % 16)][32 s + 8 (l / 16) + e]. One thread per 16-byte fragment.
__global__ __launch_bounds__(kBlock) void k_sgemm_pack(const uint16_t* __restrict__ W, uint16_t* __restrict__ P,
                                                       int tiles, int K, int F, int swiglu, float scale) {
  const int nsteps = K / 32;
  const long long i = (long long)blockIdx.x * kBlock + threadIdx.x;
  if (i >= (long long)tiles * nsteps * 64) return;
  const int l = (int)(i % 64);
  const long long ts = i / 64;
  const int st = (int)(ts % nsteps), t = (int)(ts / nsteps);
  const int n = l & 15, g = l >> 4;
  const int row = swiglu ? (n < 8 ? t * 8 + n : F + t * 8 + (n - 8)) : t * 16 + n;
  const u32x4 v = *reinterpret_cast<const u32x4*>(W + (size_t)row * K + st * 32 + 8 * g);
  u32x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e)   // w * 2^-w_exp: exact in bfloat16 (same significand)
    o[e] = (uint32_t)f32_to_bf16(bf16_lo(v[e]) * scale) | ((uint32_t)f32_to_bf16(bf16_hi(v[e]) * scale) << 16);
  *reinterpret_cast<u32x4*>(P + (size_t)i * 8) = o;
}

hipError_t launch_sgemm_pack(const void* W, void* packed, int rows_out, int K, int F, bool swiglu, int w_exp,
                             hipStream_t s) {
  if (K % 32 || (swiglu ? F % 8 : rows_out % 16)) return hipErrorInvalidValue;
  const int tiles = swiglu ? F / 8 : rows_out / 16;
  const long long n = (long long)tiles * (K / 32) * 64;
  hipLaunchKernelGGL(k_sgemm_pack, dim3((unsigned)((n + kBlock - 1) / kBlock)), dim3(kBlock), 0, s,
                     static_cast<const uint16_t*>(W), static_cast<uint16_t*>(packed), tiles, K, F, swiglu ? 1 : 0,
                     std::ldexp(1.0f, -w_exp));
  return hipGetLastError();
}

template <int EPI, int NT, bool NORM>
static void launch_bal(const SgemmArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((k_sgemm<EPI, 1, NT, true, NORM>), dim3(grid), dim3(kSgWaves * 64), 0, s, a);
}

// One session tile: one workgroup per CU, each with an equal run of column tiles.
template <int EPI, bool NORM>
static void launch_one_tile(const SgemmArgs& a, int tiles, hipStream_t s) {
  const int n_cu = a.n_cu > 0 ? a.n_cu : 256;
  const int grid = tiles < n_cu ? tiles : n_cu;
  const int per = (tiles + grid - 1) / grid;   // tiles of the busiest workgroup
  if (per <= 1) launch_bal<EPI, 1, NORM>(a, grid, s);
  else if (per <= 2) launch_bal<EPI, 2, NORM>(a, grid, s);
  else if (per <= 3) launch_bal<EPI, 3, NORM>(a, grid, s);
  else if (per <= 4) launch_bal<EPI, 4, NORM>(a, grid, s);
  else if (per <= 6) launch_bal<EPI, 6, NORM>(a, grid, s);
  else if (per <= 8) launch_bal<EPI, 8, NORM>(a, grid, s);
  else launch_bal<EPI, 8, NORM>(a, (tiles + 7) / 8, s);
}

template <int EPI>
static hipError_t launch_epi(const SgemmArgs& a, hipStream_t s) {
  const int tiles = EPI == SEPI_SWIGLU ? a.F / 8 : a.N / 16;
  const dim3 block(kSgWaves * 64);
  const int nbt = (a.B + 15) / 16;
  if (a.xin) {
    if constexpr (EPI == SEPI_QKV || EPI == SEPI_SWIGLU) {
      launch_one_tile<EPI, true>(a, tiles, s);
      return hipGetLastError();
    }
    return hipErrorInvalidValue;
  }
  if (nbt == 1) {
    launch_one_tile<EPI, false>(a, tiles, s);
    return hipGetLastError();
  }
  // two column tiles per workgroup (each activation fragment feeds two products) when
  // there are enough tiles to keep every CU busy
  const bool two = tiles % 2 == 0 && tiles >= 512;
  if (two) {
    const dim3 grid(tiles / 2);
    if (nbt == 2) hipLaunchKernelGGL((k_sgemm<EPI, 2, 2, false, false>), grid, block, 0, s, a);
    else if (nbt == 3) hipLaunchKernelGGL((k_sgemm<EPI, 3, 2, false, false>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_sgemm<EPI, 4, 2, false, false>), grid, block, 0, s, a);
    return hipGetLastError();
  }
  const dim3 grid(tiles);
  if (nbt == 2) hipLaunchKernelGGL((k_sgemm<EPI, 2, 1, false, false>), grid, block, 0, s, a);
  else if (nbt == 3) hipLaunchKernelGGL((k_sgemm<EPI, 3, 1, false, false>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((k_sgemm<EPI, 4, 1, false, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_sgemm(int epi, const SgemmArgs& a, hipStream_t s) {
  if (a.B < 1 || a.B > kSgemmMaxBatch || a.K % 32 || a.K <= 0) return hipErrorInvalidValue;
  if (epi == SEPI_SWIGLU ? (a.F <= 0 || a.F % 8) : (a.N <= 0 || a.N % 16)) return hipErrorInvalidValue;
  if (epi == SEPI_QKV && (a.N != 3 * a.D || a.dh % 2 || a.D % a.dh)) return hipErrorInvalidValue;
  if (a.xin && (a.B > kSgemmNormMaxBatch || a.K > kSgemmNormMaxK || a.K % 4 || !a.alpha)) return hipErrorInvalidValue;
  switch (epi) {
    case SEPI_STORE: return launch_epi<SEPI_STORE>(a, s);
    case SEPI_RESID: return launch_epi<SEPI_RESID>(a, s);
    case SEPI_QKV: return launch_epi<SEPI_QKV>(a, s);
    case SEPI_SWIGLU: return launch_epi<SEPI_SWIGLU>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace pp
