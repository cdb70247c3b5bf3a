// Full-sequence (prefill) kernels: T frames at positions p0 .. p0+T-1 at once.
//
// "PersonaPlex native LM audit", section 3: the same block as in decode, applied to all
// frames -- RMSNorm -> X W_QKV^T -> RoPE on Q and K -> causal attention (0 <= q - k < C)
// -> W_O + residual -> RMSNorm -> W_in -> SiLU(g) * z -> W_out + residual.
//
// bf16 path: the matrix products are dense, so they run on the CDNA4 matrix cores
// (v_mfma_f32_32x32x16_bf16, fp32 accumulation); operands are bf16 (activations are
// rounded to bf16 once per product), statistics and the residual stream stay fp32.
// float32 path (small shapes, fp32 parity): plain FMA kernels with the same epilogues.
#include "device.h"
#include "internal.h"

namespace pp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- RoPE table

__global__ __launch_bounds__(kBlock) void k_rope_rows(float* rope, int T, int p0, int dh, double log_theta) {
  const int i = blockIdx.x * kBlock + threadIdx.x;   // (t, j)
  const int half = dh / 2;
  if (i >= T * half) return;
  const int t = i / half, j = i - t * half;
  const double ang = (double)(p0 + t) * exp(-log_theta * (double)(2 * j) / (double)dh);
  double sn, cs;
  sincos(ang, &sn, &cs);
  rope[(size_t)t * dh + 2 * j] = (float)cs;
  rope[(size_t)t * dh + 2 * j + 1] = (float)sn;
}

hipError_t launch_rope_rows(float* rope, int T, int p0, int dh, double log_theta, hipStream_t s) {
  const int n = T * (dh / 2);
  hipLaunchKernelGGL(k_rope_rows, dim3((n + kBlock - 1) / kBlock), dim3(kBlock), 0, s, rope, T, p0, dh, log_theta);
  return hipGetLastError();
}

// ---------------------------------------------------------------- epilogue (one element)

// Output element (row, col) of the product with value v; `partner` is the value at column
// col ^ 1 of the same row (the RoPE pair partner). Writes through the epilogue kind.
template <typename OT, int EPI>
__device__ __forceinline__ void gemm_store(const GemmArgs& g, int row, int col, float v, float partner) {
  if (EPI == GEPI_QKV) {
    const int sec = col / g.D;
    const int w = col - sec * g.D;
    const int head = w / g.dh, d = w - head * g.dh;
    float y = v;
    if (sec < 2) {
      const float c = g.rope[(size_t)row * g.dh + (d & ~1)], s = g.rope[(size_t)row * g.dh + (d | 1)];
      y = (d & 1) ? partner * s + v * c : v * c - partner * s;
    }
    if (sec == 0) {
      Elem<OT>::store1(static_cast<OT*>(g.q_out) + ((size_t)head * g.M + row) * g.dh + d, y);
    } else {
      const int slot = (g.p0 + row) % g.C;
      OT* base = static_cast<OT*>(sec == 1 ? g.kc : g.vc);
      Elem<OT>::store1(base + ((size_t)head * g.C + slot) * g.dh + d, y);
    }
  } else if (EPI == GEPI_RESID) {
    g.x[(size_t)row * g.N + col] += v;
  }
}

// ---------------------------------------------------------------- bf16 MFMA GEMM

constexpr int GBM = 128, GBN = 128, GBK = 64, GLD = GBK + 8;  // LDS rows padded by 16 bytes

// C[M][N] = A[M][K] B[N][K]^T for one 128 x 128 tile per workgroup (4 waves, each 64 x 64 as
// 2 x 2 tiles of 32 x 32 x 16 MFMAs). The next k-tile is prefetched into registers while
// the current one is multiplied from LDS. GEPI_SWIGLU: the B tile holds W_in rows
// j0..j0+63 (g) and F+j0..F+j0+63 (z), and wave (wm, wn) multiplies g rows wn*32.. and z
// rows 64+wn*32.., so g and z of the same output land in the same lane.
template <int EPI>
__global__ __launch_bounds__(256) void k_gemm_bf16(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint16_t As[GBM * GLD];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[GBN * GLD];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w & 1, wn = w >> 1;
  const int n_tm = (g.M + GBM - 1) / GBM;
  const int n_tn = EPI == GEPI_SWIGLU ? g.F / 64 : g.N / GBN;
  const int tiles = n_tm * n_tn;

  // Tile order: workgroup b runs on XCD b mod 8; give each XCD a contiguous range of tiles,
  // walked in groups of 8 M-tiles per N-tile so concurrent workgroups of an XCD share the
  // weight tile (and a few activation tiles) in that XCD's L2.
  int b = blockIdx.x;
  if (tiles % 8 == 0) b = (b % 8) * (tiles / 8) + b / 8;
  constexpr int GROUP = 8;
  const int group = b / (GROUP * n_tn);
  const int first_m = group * GROUP;
  const int gsize = n_tm - first_m < GROUP ? n_tm - first_m : GROUP;
  const int tm = first_m + (b % (GROUP * n_tn)) % gsize;
  const int tn = (b % (GROUP * n_tn)) / gsize;

  const int m0 = tm * GBM;
  const uint16_t* A = static_cast<const uint16_t*>(g.A);
  const uint16_t* B = static_cast<const uint16_t*>(g.B);
  const int K = g.K;
  auto brow = [&](int r) -> int {
    if (EPI == GEPI_SWIGLU) return r < 64 ? tn * 64 + r : g.F + tn * 64 + (r - 64);
    return tn * GBN + r;
  };

  u32x4 ra[4], rb[4];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + 256 * i, r = id >> 3, kc = id & 7;
      const int am = m0 + r < g.M ? m0 + r : g.M - 1;
      ra[i] = *reinterpret_cast<const u32x4*>(A + (size_t)am * K + kt * GBK + kc * 8);
      rb[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(B + (size_t)brow(r) * K + kt * GBK + kc * 8));
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + 256 * i, r = id >> 3, kc = id & 7;
      *reinterpret_cast<u32x4*>(As + r * GLD + kc * 8) = ra[i];
      *reinterpret_cast<u32x4*>(Bs + r * GLD + kc * 8) = rb[i];
    }
  };
  auto bcol0 = [&](int j) -> int { return EPI == GEPI_SWIGLU ? j * 64 + wn * 32 : wn * 64 + j * 32; };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int nk = K / GBK;
  gload(0);
  sstore();
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int ks = 0; ks < GBK / 16; ++ks) {
      bf16x8 av[2], bv[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        av[i] = *reinterpret_cast<const bf16x8*>(As + (wm * 64 + i * 32 + (lane & 31)) * GLD + ks * 16 + 8 * (lane >> 5));
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bv[j] = *reinterpret_cast<const bf16x8*>(Bs + (bcol0(j) + (lane & 31)) * GLD + ks * 16 + 8 * (lane >> 5));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
    if (kt + 1 < nk) {
      sstore();
      __syncthreads();
    }
  }

  // ---- epilogue: acc[i][j][4*jj + ii] is (row 8*jj + 4*(lane/32) + ii, col lane%32) of tile (i, j)
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int row = m0 + wm * 64 + i * 32 + 8 * jj + 4 * (lane >> 5) + ii;
        if (EPI == GEPI_SWIGLU) {
          const float gv = acc[i][0][4 * jj + ii], zv = acc[i][1][4 * jj + ii];
          if (row < g.M) {
            const int col = tn * 64 + wn * 32 + (lane & 31);
            static_cast<uint16_t*>(g.s_out)[(size_t)row * g.F + col] = f32_to_bf16(silu(gv) * zv);
          }
        } else {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const float v = acc[i][j][4 * jj + ii];
            const float partner = dpp_xor1(v);  // column col ^ 1 of the same row
            const int col = tn * GBN + wn * 64 + j * 32 + (lane & 31);
            if (row < g.M) gemm_store<bf16_t, EPI>(g, row, col, v, partner);
          }
        }
      }
}

// ---------------------------------------------------------------- float32 GEMM (FMA)

// 64 x 64 tile (B rows), 256 threads; thread (tx, ty) owns rows 4ty..4ty+3 and tile
// columns {2tx, 2tx+1, 32+2tx, 33+2tx}, so a RoPE pair and (for SwiGLU: B rows 0..31 are
// g rows j0.., rows 32..63 the z rows) a g/z pair sit in one thread.
template <int EPI>
__global__ __launch_bounds__(256) void k_gemm_f32(GemmArgs g) {
  __shared__ float As[64][17], Bs[64][17];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int n_tn = EPI == GEPI_SWIGLU ? (g.F + 31) / 32 : (g.N + 63) / 64;
  const int tm = blockIdx.x / n_tn, tn = blockIdx.x % n_tn;
  const int m0 = tm * 64;
  const float* A = static_cast<const float*>(g.A);
  const float* B = static_cast<const float*>(g.B);
  auto brow = [&](int r) -> int {
    if (EPI == GEPI_SWIGLU) {
      const int j = tn * 32 + (r & 31);
      return j < g.F ? (r < 32 ? j : g.F + j) : -1;
    }
    const int n = tn * 64 + r;
    return n < g.N ? n : -1;
  };
  float acc[4][4] = {};
  for (int k0 = 0; k0 < g.K; k0 += 16) {
    for (int i = tid; i < 64 * 16; i += 256) {
      const int r = i >> 4, kk = i & 15, k = k0 + kk;
      const int am = m0 + r;
      As[r][kk] = (am < g.M && k < g.K) ? A[(size_t)am * g.K + k] : 0.f;
      const int br = brow(r);
      Bs[r][kk] = (br >= 0 && k < g.K) ? B[(size_t)br * g.K + k] : 0.f;
    }
    __syncthreads();
    const int cols[4] = {2 * tx, 2 * tx + 1, 32 + 2 * tx, 33 + 2 * tx};
#pragma unroll
    for (int kk = 0; kk < 16; ++kk)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] += As[4 * ty + r][kk] * Bs[cols[c]][kk];
    __syncthreads();
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = m0 + 4 * ty + r;
    if (row >= g.M) continue;
    if (EPI == GEPI_SWIGLU) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int j = tn * 32 + 2 * tx + c;
        if (j < g.F) static_cast<float*>(g.s_out)[(size_t)row * g.F + j] = silu(acc[r][c]) * acc[r][2 + c];
      }
    } else {
      const int cols[4] = {2 * tx, 2 * tx + 1, 32 + 2 * tx, 33 + 2 * tx};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int col = tn * 64 + cols[c];
        if (col < g.N) gemm_store<float, EPI>(g, row, col, acc[r][c], acc[r][c ^ 1]);
      }
    }
  }
}

template <int EPI>
static hipError_t gemm_dispatch(bool bf16, const GemmArgs& g, hipStream_t s) {
  if (bf16) {
    const int n_tm = (g.M + GBM - 1) / GBM;
    const int n_tn = EPI == GEPI_SWIGLU ? g.F / 64 : g.N / GBN;
    hipLaunchKernelGGL(k_gemm_bf16<EPI>, dim3(n_tm * n_tn), dim3(256), 0, s, g);
  } else {
    const int n_tm = (g.M + 63) / 64;
    const int n_tn = EPI == GEPI_SWIGLU ? (g.F + 31) / 32 : (g.N + 63) / 64;
    hipLaunchKernelGGL(k_gemm_f32<EPI>, dim3(n_tm * n_tn), dim3(256), 0, s, g);
  }
  return hipGetLastError();
}

hipError_t launch_gemm(int epi, bool bf16, const GemmArgs& g, int n_cu, hipStream_t s) {
  (void)n_cu;
  if (g.M <= 0) return hipSuccess;
  if (bf16) {
    // MFMA tiles: K in steps of 64, N in tiles of 128 (SwiGLU: F in tiles of 64)
    if (g.K % GBK) return hipErrorInvalidValue;
    if (epi == GEPI_SWIGLU ? g.F % 64 : g.N % GBN) return hipErrorInvalidValue;
  } else if (epi == GEPI_QKV && (g.dh % 2)) {
    return hipErrorInvalidValue;
  }
  switch (epi) {
    case GEPI_QKV: return gemm_dispatch<GEPI_QKV>(bf16, g, s);
    case GEPI_RESID: return gemm_dispatch<GEPI_RESID>(bf16, g, s);
    case GEPI_SWIGLU: return gemm_dispatch<GEPI_SWIGLU>(bf16, g, s);
  }
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------- bf16 flash attention

// Workgroup (query block qb of 128 frames, head h); wave w owns queries qb*128 + 32w ..+31,
// one per lane column (lane % 32). For each block of 64 keys (up to the causal limit):
//   S^T = K Q^T   (A = K rows from LDS, B = Q^T kept in registers) -> lane holds the 32
//                 scores of its query for 32 of the 64 keys; its partner lane (lane ^ 32)
//                 holds the other 32, so the softmax max/sum need one exchange;
//   O^T += V^T P^T (A = V^T from LDS, staged transposed; B = P^T straight from the S^T
//                 registers -- the k index of the product is a fixed permutation of the
//                 keys, applied identically to V^T).
// The running max/sum rescale O^T in registers. Causal + window mask per element.
template <int DH>
__global__ __launch_bounds__(256) void k_attn_prefill_bf16(AttnPrefillArgs a) {
  constexpr int BQ = 128, BKV = 64;
  constexpr int KLD = DH + 8;    // K tile row pitch (bf16 elements)
  constexpr int VLD = BKV + 8;   // V^T row pitch (keys)
  __shared__ __attribute__((aligned(16))) uint16_t Ks[BKV * KLD];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[DH * VLD];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = blockIdx.y;
  const int n_qb = (a.T + BQ - 1) / BQ;
  const int qb = n_qb - 1 - blockIdx.x;      // longest (latest) query blocks first
  const int hi = lane >> 5, ql = lane & 31;
  const int qi = qb * BQ + w * 32 + ql;      // this lane's query (frame index)
  const int qrow = qi < a.T ? qi : a.T - 1;
  const uint16_t* Q = static_cast<const uint16_t*>(a.q);
  const uint16_t* Kg = static_cast<const uint16_t*>(a.k);
  const uint16_t* Vg = static_cast<const uint16_t*>(a.v);

  bf16x8 qr[DH / 16];
#pragma unroll
  for (int ks = 0; ks < DH / 16; ++ks)
    qr[ks] = *reinterpret_cast<const bf16x8*>(Q + ((size_t)h * a.T + qrow) * DH + ks * 16 + 8 * hi);

  float m = -INFINITY, l = 0.f;
  f32x16 o[DH / 32];
#pragma unroll
  for (int dt = 0; dt < DH / 32; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[dt][e] = 0.f;

  const int qlast = (qb + 1) * BQ < a.T ? (qb + 1) * BQ - 1 : a.T - 1;
  const int qfirst = qb * BQ;
  int kfirst = qfirst - a.C + 1;
  kfirst = kfirst > 0 ? kfirst / BKV * BKV : 0;
  constexpr int CH = DH / 8;  // 16-byte chunks per key row

  for (int k0 = kfirst; k0 <= qlast; k0 += BKV) {
    // ---- stage K (as is) and V (transposed) of keys k0 .. k0+63
#pragma unroll
    for (int i = 0; i < BKV * CH / 256; ++i) {
      const int id = tid + 256 * i, r = id / CH, c8 = id % CH;
      const int key = k0 + r;
      u32x4 kv4 = {0u, 0u, 0u, 0u}, vv4 = {0u, 0u, 0u, 0u};
      if (key < a.T) {
        const size_t off = ((size_t)h * a.C + (a.p0 + key) % a.C) * DH + c8 * 8;
        kv4 = *reinterpret_cast<const u32x4*>(Kg + off);
        vv4 = *reinterpret_cast<const u32x4*>(Vg + off);
      }
      *reinterpret_cast<u32x4*>(Ks + r * KLD + c8 * 8) = kv4;
      const uint32_t vw[4] = {vv4.x, vv4.y, vv4.z, vv4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Vt[(c8 * 8 + 2 * e) * VLD + r] = (uint16_t)(vw[e] & 0xffffu);
        Vt[(c8 * 8 + 2 * e + 1) * VLD + r] = (uint16_t)(vw[e] >> 16);
      }
    }
    __syncthreads();

    // ---- S^T for the 64 keys: s[kt][4*jj + ii] is key k0 + 32*kt + 8*jj + 4*hi + ii
    f32x16 s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s[kt][e] = 0.f;
#pragma unroll
      for (int ks = 0; ks < DH / 16; ++ks) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(Ks + (kt * 32 + ql) * KLD + ks * 16 + 8 * hi);
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qr[ks], s[kt], 0, 0, 0);
      }
    }
    float mb = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = k0 + 32 * kt + 8 * (e >> 2) + 4 * hi + (e & 3);
        const bool ok = key <= qi && qi - key < a.C && key < a.T;
        const float v = ok ? s[kt][e] * a.scale : -INFINITY;
        s[kt][e] = v;
        mb = fmaxf(mb, v);
      }
    mb = fmaxf(mb, __shfl_xor(mb, 32, kWave));
    const float mn = fmaxf(m, mb);
    const float sc = mn == -INFINITY ? 1.f : expf(m - mn);
    l *= sc;
#pragma unroll
    for (int dt = 0; dt < DH / 32; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[dt][e] *= sc;
    m = mn;

    // ---- P^T (bf16) and O^T += V^T P^T over 4 steps of 16 keys
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int kt = t >> 1, j8 = 8 * (t & 1);
      bf16x8 pb;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p = s[kt][j8 + i] == -INFINITY ? 0.f : expf(s[kt][j8 + i] - mn);
        l += p;
        pb[i] = (__bf16)p;
      }
      const int kbase = kt * 32 + 16 * (t & 1) + 4 * hi;
#pragma unroll
      for (int dt = 0; dt < DH / 32; ++dt) {
        const uint16_t* vrow = Vt + (dt * 32 + ql) * VLD;
        const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow + kbase);
        const u32x2 hi8 = *reinterpret_cast<const u32x2*>(vrow + kbase + 8);
        const u32x4 packed = {lo.x, lo.y, hi8.x, hi8.y};
        const bf16x8 va = __builtin_bit_cast(bf16x8, packed);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, o[dt], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // ---- normalise and write: o[dt][4*jj + ii] is dim dt*32 + 8*jj + 4*hi + ii of query qi
  const float lt = l + __shfl_xor(l, 32, kWave);
  const float inv = 1.0f / lt;
  if (qi < a.T) {
    uint16_t* out = static_cast<uint16_t*>(a.out) + (size_t)qi * (a.H * DH) + h * DH;
#pragma unroll
    for (int dt = 0; dt < DH / 32; ++dt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d = dt * 32 + 8 * jj + 4 * hi;
        const uint32_t w0 = (uint32_t)f32_to_bf16(o[dt][4 * jj] * inv) | ((uint32_t)f32_to_bf16(o[dt][4 * jj + 1] * inv) << 16);
        const uint32_t w1 = (uint32_t)f32_to_bf16(o[dt][4 * jj + 2] * inv) | ((uint32_t)f32_to_bf16(o[dt][4 * jj + 3] * inv) << 16);
        *reinterpret_cast<u32x2*>(out + d) = u32x2{w0, w1};
      }
  }
}

// ---------------------------------------------------------------- float32 attention

// One workgroup of d_head threads per (query, head): online softmax over the visible keys,
// one key at a time (scores reduced through LDS). For the small fp32 shapes only.
template <int DH>
__global__ __launch_bounds__(DH) void k_attn_prefill_f32(AttnPrefillArgs a) {
  __shared__ float red[DH / 64 > 0 ? DH / 64 : 1];
  const int t = blockIdx.x, h = blockIdx.y, d = threadIdx.x;
  const float* Q = static_cast<const float*>(a.q);
  const float* Kg = static_cast<const float*>(a.k);
  const float* Vg = static_cast<const float*>(a.v);
  const float qd = Q[((size_t)h * a.T + t) * DH + d] * a.scale;
  float m = -INFINITY, l = 0.f, o = 0.f;
  const int kfirst = t - a.C + 1 > 0 ? t - a.C + 1 : 0;
  for (int key = kfirst; key <= t; ++key) {
    const size_t off = ((size_t)h * a.C + (a.p0 + key) % a.C) * DH + d;
    float part = wave_sum(qd * Kg[off]);
    if ((d & 63) == 0) red[d >> 6] = part;
    __syncthreads();
    float sc = 0.f;
    for (int i = 0; i < DH / 64; ++i) sc += red[i];
    __syncthreads();
    const float mn = fmaxf(m, sc);
    const float r = expf(m - mn), p = expf(sc - mn);
    l = l * r + p;
    o = o * r + p * Vg[off];
    m = mn;
  }
  static_cast<float*>(a.out)[(size_t)t * (a.H * DH) + h * DH + d] = o / l;
}

hipError_t launch_attn_prefill(const AttnPrefillArgs& a, bool bf16, int dh, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  if (bf16) {
    const dim3 grid((a.T + 127) / 128, a.H);
    if (dh == 128) hipLaunchKernelGGL(k_attn_prefill_bf16<128>, grid, dim3(256), 0, s, a);
    else if (dh == 64) hipLaunchKernelGGL(k_attn_prefill_bf16<64>, grid, dim3(256), 0, s, a);
    else return hipErrorInvalidValue;
  } else {
    const dim3 grid(a.T, a.H);
    if (dh == 128) hipLaunchKernelGGL(k_attn_prefill_f32<128>, grid, dim3(128), 0, s, a);
    else if (dh == 64) hipLaunchKernelGGL(k_attn_prefill_f32<64>, grid, dim3(64), 0, s, a);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pp
