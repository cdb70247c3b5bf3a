// Full-sequence (prefill) kernels: T frames at positions p0 .. p0+T-1 at once.
//
// "PersonaPlex native LM audit", section 3: the same block as in decode, applied to all
// frames -- RMSNorm -> X W_QKV^T -> RoPE on Q and K -> causal attention (0 <= q - k < C)
// -> W_O + residual -> RMSNorm -> W_in -> SiLU(g) * z -> W_out + residual.
//
// bf16 path: the matrix products are dense, so they run on the CDNA4 matrix cores
// (fp32 accumulation). The activations of the four projections enter as float16 (11-bit
// significand: eight times less rounding than bfloat16, at the same matrix-core rate;
// v_mfma_f32_32x32x16_f16), and so do the weights, from a float16 copy of every bfloat16
// matrix made once at model creation -- exact for bfloat16 values in float16's normal
// range, which covers weights of this scale. In attention, Q K^T is a bfloat16 product (keys
// are bfloat16 in the ring, shared with decode) and P V a float16 one (P and the transposed
// V copy in float16). Statistics and the residual stream stay fp32.
// float32 path (small shapes, fp32 parity): plain FMA kernels with the same epilogues.
#include <cmath>

#include <type_traits>

#include "device.h"
#include "internal.h"

namespace pp {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- RoPE table

__global__ __launch_bounds__(kBlock) void k_rope_rows(float* rope, int T, long long p0, int dh, double log_theta) {
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

hipError_t launch_rope_rows(float* rope, int T, long long p0, int dh, double log_theta, hipStream_t s) {
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
      OT* xb = static_cast<OT*>(sec == 1 ? g.kx : g.vx);
      if (xb) Elem<OT>::store1(xb + ((size_t)head * g.x_pitch + g.xoff + row) * g.dh + d, y);
    }
  } else if (EPI == GEPI_RESID) {
    g.x[(size_t)row * g.N + col] += v;
  }
}

// ---------------------------------------------------------------- bf16 MFMA GEMM

constexpr int GBK = 64;

// LDS tiles are rows of 64 bf16 (8 chunks of 16 bytes = 128 B) without padding. The LDS
// serves a 16-byte-per-lane read for 16 lanes at a time from a 256-byte bank window, i.e.
// from two consecutive 128-byte rows; chunk kc of row r therefore sits at slot
// kc ^ ((r >> 1) & 7), so 16 consecutive rows read at one chunk index hit 16 distinct
// 16-byte bank groups (rows r and r+1 share a slot but sit in different halves).
__device__ __forceinline__ int swz_slot(int r, int kc) { return kc ^ ((r >> 1) & 7); }
__device__ __forceinline__ int swz(int r, int kc) { return r * 8 + swz_slot(r, kc); }

// Column of key t in the transposed V copy: bits 2 and 3 of t swapped, so that within
// each group of 16 keys the order is 0-3, 8-11, 4-7, 12-15 -- the order in which one
// lane holds probabilities after the S^T product (see k_attn_prefill_f16).
__device__ __forceinline__ int vt_perm(int t) { return (t & ~12) | ((t & 4) << 1) | ((t & 8) >> 1); }

// Wait until at most N vector-memory operations of this wave are outstanding and all its
// LDS operations are done, then synchronise the workgroup. Loads into LDS complete in
// issue order, so N = the loads issued after the ones that must have landed.
template <int N>
__device__ __forceinline__ void vm_wait_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// GEMM stage rows hold KB/8 chunks of 16 bytes. Rows of 8 chunks (KB = 64) use swz_slot;
// rows of 4 chunks (KB = 32) XOR the chunk index with bits 2..3 of the row, so that 16
// consecutive rows read at one chunk index again fall into 16 distinct 16-byte bank groups
// of a 256-byte window (bits 2..3 of the row pick the 64-byte quarter, the XOR the chunk).
template <int CPRL>
__device__ __forceinline__ int gswz_slot(int r, int kc) {
  static_assert(CPRL == 4 || CPRL == 8, "row width");
  return CPRL == 8 ? kc ^ ((r >> 1) & 7) : kc ^ ((r >> 2) & 3);
}

template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Wait until at most a * L loads of this wave are outstanding (0 <= a; a above A counts as A).
template <int L, int A>
__device__ __forceinline__ void vm_wait_tiles(int a) {
  if constexpr (A == 0) {
    vm_wait<0>();
  } else {
    if (a >= A) vm_wait<A * L>();
    else vm_wait_tiles<L, A - 1>(a);
  }
}
__device__ __forceinline__ void lds_wait_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// C[M][N] = A[M][K] B[N][K]^T with float16 A (activations) and B (the model's float16
// weight copy, converted once from bf16, scaled by a power of two that the epilogue
// undoes: g.acc_exp). Workgroup = WM x WN waves, tile BM x BN with BM = WM*32*MI,
// BN = WN*32*NI; wave (wm, wn) owns rows wm*32*MI.. and 32*NI columns as MI x NI tiles of
// 32 x 32 (v_mfma_f32_32x32x16_f16, fp32 accumulation).
// k-tiles of KB columns go from global memory straight into LDS (buffer loads with the LDS
// flag: no registers, no LDS write instructions). Stage st holds one k-tile: rows 0..BM-1
// of A, then rows BM..BM+BN-1 of B. One barrier per k-tile, in one of two schedules:
//   early (LATE = false): NS-1 tiles ahead; the barrier opens tile kt, whose first
//     fragments are read before the stage of tile kt-1 is refilled with tile kt+NS-1;
//   late (LATE = true): all NS stages in use; the barrier sits before tile kt's last
//     k-step: once every wave has read all of tile kt's fragments its stage is refilled
//     with tile kt+NS, and tile kt+1's first fragments are read under the last k-step's
//     matrix products.
// Rows of A past M read as zeros (out of the buffer's range) and are not stored.
// Split-K (gridDim.y > 1): workgroup row y takes its share of the k-tiles and writes
// float32 partial sums part[y][row][B row] in place of the epilogue (k_splitk_resid /
// k_splitk_swiglu add the splits in order and apply it).
// GEPI_SWIGLU: the B tile holds W_in rows j0..j0+BN/2-1 (g) and F+j0.. (z); wave (wm, wn)
// multiplies g rows wn*16*NI.. (NI/2 tiles) and the z rows BN/2 + wn*16*NI.., so g and z
// of one output share a lane.
// TAG only names the instantiation (the W_out product's residual launches are TAG 1, so a
// kernel profile lists them apart from W_O's); the code does not depend on it.
template <int EPI, int WM, int WN, int MI, int NI, int NS, int KB, bool LATE, int TAG>
__global__ __launch_bounds__(WM * WN * 64) void k_gemm_f16(GemmArgs g) {
  constexpr int NW = WM * WN;
  constexpr int BM = WM * 32 * MI, BN = WN * 32 * NI;
  constexpr int CPRL = KB / 8;            // 16-byte chunks per LDS row
  constexpr int RPI = 64 / CPRL;          // LDS rows one load instruction fills (1 KB)
  constexpr int NQ = (BM + BN) / RPI;     // load instructions per k-tile
  constexpr int LW = (NQ + NW - 1) / NW;  // per wave: LW for waves w < NQ - NW*(LW-1), else LW-1
  constexpr int KS = KB / 16;             // k-steps (of 16) per tile
  static_assert(KB == 32 || KB == 64, "k-tile width");
  static_assert(BM % RPI == 0 && NQ >= NW, "load instructions cover whole A / B rows");
  static_assert(KS % 2 == 0, "the two fragment register sets alternate per k-step");
  static_assert(NS >= 2 && (NS - 1) * LW < 64, "stages");
  static_assert(EPI != GEPI_SWIGLU || NI % 2 == 0, "SwiGLU pairs g and z tiles");
  // GEPI_QKV reuses the LDS for half of its output tile (fp32, row pitch TPF floats)
  constexpr int TPF = BN / 2 + 4;
  constexpr int STAGE = (BM + BN) * CPRL;
  constexpr int STAGE_CH = NS * STAGE, TILE_CH = EPI == GEPI_QKV ? BM * TPF * 4 / 16 : 0;
  __shared__ u32x4 lds[STAGE_CH > TILE_CH ? STAGE_CH : TILE_CH];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w % WM, wn = w / WM;
  const int n_tm = (g.M + BM - 1) / BM;
  const int n_tn = EPI == GEPI_SWIGLU ? g.F / (BN / 2) : g.N / BN;
  const int tiles = n_tm * n_tn;

  // Tile order: workgroup b runs on XCD b mod 8; give each XCD a contiguous range of tiles,
  // walked in groups of 8 M-tiles per N-tile so concurrent workgroups of an XCD share
  // weight and activation k-slices in that XCD's L2.
  int b = blockIdx.x;
  if (tiles % 8 == 0) b = (b % 8) * (tiles / 8) + b / 8;
  constexpr int GROUP = 8;
  const int group = b / (GROUP * n_tn);
  const int first_m = group * GROUP;
  const int gsize = n_tm - first_m < GROUP ? n_tm - first_m : GROUP;
  const int tm = first_m + (b % (GROUP * n_tn)) % gsize;
  const int tn = (b % (GROUP * n_tn)) / gsize;

  const int m0 = tm * BM;
  const int K = g.K;
  // split-K: workgroup row blockIdx.y of gridDim.y takes k-tiles kt0 .. kt0+nk-1
  const int n_split = gridDim.y, split = blockIdx.y;
  const int kt0 = split * (K / KB) / n_split;
  const int nk = (split + 1) * (K / KB) / n_split - kt0;
  auto brow = [&](int r) -> int {
    if (EPI == GEPI_SWIGLU) return r < BN / 2 ? tn * (BN / 2) + r : g.F + tn * (BN / 2) + (r - BN / 2);
    return tn * BN + r;
  };
  const u32x4 ar = rsrc_words(g.A, (uint32_t)((size_t)g.M * K * 2));
  const u32x4 br = rsrc_words(g.B, (uint32_t)((size_t)(EPI == GEPI_SWIGLU ? 2 * g.F : g.N) * K * 2));
  // Instruction q = w + NW*j fills stage rows q*RPI .. q*RPI + RPI-1 (1 KB, lane i at chunk
  // position q*64 + i): lane i fetches row q*RPI + i/CPRL and the k-chunk that gswz_slot
  // puts at slot i%CPRL of that row (the XOR is its own inverse).
  const bool full = w + NW * (LW - 1) < NQ;  // this wave issues LW loads per k-tile
  uint32_t voff[LW];
#pragma unroll
  for (int j = 0; j < LW; ++j) {
    const int q = w + NW * j;
    const int r = q * RPI + lane / CPRL;
    const int chunk = gswz_slot<CPRL>(r, lane % CPRL);
    const size_t grow = r < BM ? (size_t)(m0 + r) : (size_t)brow(r - BM);
    voff[j] = (uint32_t)((grow * K + chunk * 8) * 2);
  }
  auto issue_one = [&](int kt, int st, int j) {
    const int q = w + NW * j;
    if (j < LW - 1 || full)
      lds_dma16(q * RPI < BM ? ar : br, voff[j], (uint32_t)((kt0 + kt) * KB * 2), lds_addr(lds + st * STAGE + q * 64));
  };
  auto issue = [&](int kt, int st) {
#pragma unroll
    for (int j = 0; j < LW; ++j) issue_one(kt, st, j);
  };
  auto wait_tiles = [&](int a, auto amax) {  // at most a of this wave's k-tiles still loading
    if (full) vm_wait_tiles<LW, decltype(amax)::value>(a);
    else vm_wait_tiles<LW - 1, decltype(amax)::value>(a);
  };
  // first stage row (B part) of the wave's column tile j
  auto bcol0 = [&](int j) -> int {
    if (EPI == GEPI_SWIGLU) return BM + (j < NI / 2 ? 0 : BN / 2) + wn * 16 * NI + (j % (NI / 2)) * 32;
    return BM + wn * 32 * NI + j * 32;
  };

  f32x16 acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // One fragment: stage row r, k-chunk kc.
  auto frag = [&](int st, int r, int kc) -> f16x8 {
    return __builtin_bit_cast(f16x8, lds[st * STAGE + r * CPRL + gswz_slot<CPRL>(r, kc)]);
  };
  // Fragments of k-step ks of stage st (lane: row/col lane%32, k-chunk 2*ks + lane/32).
  auto load_frags = [&](int st, int ks, f16x8 (&av)[MI], f16x8 (&bv)[NI]) {
    const int kc = ks * 2 + (lane >> 5);
#pragma unroll
    for (int j = 0; j < NI; ++j) bv[j] = frag(st, bcol0(j) + (lane & 31), kc);
#pragma unroll
    for (int i = 0; i < MI; ++i) av[i] = frag(st, wm * 32 * MI + i * 32 + (lane & 31), kc);
  };
  auto mfmas = [&](const f16x8 (&av)[MI], const f16x8 (&bv)[NI]) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
  };
  // Pin the schedule of n k-steps whose MFMAs each alternate with the next k-step's
  // fragment reads (masks: 0x008 MFMA, 0x100 LDS read), so LDS latency hides under the
  // matrix-core work of the same wave.
  constexpr int NF = MI + NI, NM = MI * NI;
  auto interleave = [&](auto n) {
#pragma unroll
    for (int ks = 0; ks < decltype(n)::value; ++ks)
#pragma unroll
      for (int i = 0; i < NM; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i < NF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
  };

  f16x8 a0[MI], b0[NI], a1[MI], b1[NI];
  if constexpr (LATE) {
    // All NS stages in use; the barrier sits before each tile's last k-step.
#pragma unroll
    for (int s = 0; s < NS; ++s)
      if (s < nk) issue(s, s);
    wait_tiles(nk - 1, std::integral_constant<int, NS - 1>{});  // tile 0 has landed
    lds_wait_barrier();
    load_frags(0, 0, a0, b0);
    int st = 0;
    for (int kt = 0; kt < nk; ++kt) {
      // k-steps 0 .. KS-2, each with the next k-step's fragment reads
#pragma unroll
      for (int ks = 0; ks + 1 < KS; ++ks) {
        if (ks % 2 == 0) {
          load_frags(st, ks + 1, a1, b1);
          mfmas(a0, b0);
        } else {
          load_frags(st, ks + 1, a0, b0);
          mfmas(a1, b1);
        }
      }
      interleave(std::integral_constant<int, KS - 1>{});
      // The last k-step's fragments are in set 1. Tile kt+1 landed (tiles kt+2 .. kt+NS-1
      // may still be loading) and every wave is done reading tile kt. After the last tile
      // the wait, the barrier and the reads of the next stage are harmless (in-bounds LDS,
      // nothing loading), which keeps the loop body free of branches around the MFMAs.
      wait_tiles(nk - 2 - kt, std::integral_constant<int, NS - 2>{});
      lds_wait_barrier();
      // The last k-step's MFMAs, the next stage's first fragment reads and this wave's
      // loads of tile kt+NS, interleaved in program order (each load is an asm statement
      // the scheduler does not move anything across): a burst of loads would hold up
      // the in-order issue of the MFMAs behind it.
      const int sn = st + 1 == NS ? 0 : st + 1;
      const bool more = kt + NS < nk;
#pragma unroll
      for (int t = 0; t < NM; ++t) {
        const int i = t / NI, j = t % NI;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1[i], b1[j], acc[i][j], 0, 0, 0);
        if (t < NI) b0[t] = frag(sn, bcol0(t) + (lane & 31), lane >> 5);
        else if (t < NF) a0[t - NI] = frag(sn, wm * 32 * MI + (t - NI) * 32 + (lane & 31), lane >> 5);
#pragma unroll
        for (int r = t * LW / NM; r < (t + 1) * LW / NM; ++r)
          if (more) issue_one(kt + NS, st, r);
      }
      if constexpr (NM < NF) {
#pragma unroll
        for (int t = NM; t < NF; ++t) {
          if (t < NI) b0[t] = frag(sn, bcol0(t) + (lane & 31), lane >> 5);
          else a0[t - NI] = frag(sn, wm * 32 * MI + (t - NI) * 32 + (lane & 31), lane >> 5);
        }
      }
      st = sn;
    }
  } else {
    // NS-1 tiles ahead; the barrier opens each tile, the stage read by the previous tile is
    // refilled once this tile's first fragments are read.
#pragma unroll
    for (int s = 0; s + 1 < NS; ++s)
      if (s < nk) issue(s, s);
    int st = 0;
    for (int kt = 0; kt < nk; ++kt) {
      // tile kt landed; tiles kt+1 .. kt+NS-2 may still be loading
      wait_tiles(nk - 1 - kt, std::integral_constant<int, NS - 2>{});
      lds_wait_barrier();
      const int nst = st == 0 ? NS - 1 : st - 1;
      load_frags(st, 0, a0, b0);
      if (kt + NS - 1 < nk) issue(kt + NS - 1, nst);
#pragma unroll
      for (int ks = 0; ks + 1 < KS; ++ks) {
        if (ks % 2 == 0) {
          load_frags(st, ks + 1, a1, b1);
          mfmas(a0, b0);
        } else {
          load_frags(st, ks + 1, a0, b0);
          mfmas(a1, b1);
        }
      }
      mfmas(a1, b1);
      interleave(std::integral_constant<int, KS - 1>{});
      __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
      st = st + 1 == NS ? 0 : st + 1;
    }
  }

  // ---- epilogue: acc[i][j][4*jj + ii] is (row 8*jj + 4*(lane/32) + ii, col lane%32) of tile (i, j)
  if (n_split > 1) {
    // split-K: float32 partial sums part[split][row][B row]; a separate pass adds the
    // splits in order and applies the epilogue
    const int ncol = EPI == GEPI_SWIGLU ? 2 * g.F : g.N;
    float* pbase = g.part + (size_t)split * g.M * ncol;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int row = m0 + wm * 32 * MI + i * 32 + 8 * jj + 4 * (lane >> 5) + ii;
          if (row >= g.M) continue;
#pragma unroll
          for (int j = 0; j < NI; ++j) pbase[(size_t)row * ncol + brow(bcol0(j) - BM + (lane & 31))] = acc[i][j][4 * jj + ii];
        }
    return;
  }
  // the float16 operands are scaled copies (power-of-two exponents): undo them, exactly
  if (g.acc_exp != 0) {
    const float am = ldexpf(1.0f, g.acc_exp);
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] *= am;
  }
  if constexpr (EPI == GEPI_QKV) {
    // Half a tile at a time (128-byte-aligned column halves): the waves holding those
    // columns write their fp32 values into LDS, then every thread takes 8 consecutive
    // columns of a row -- 4 RoPE pairs, whose cos/sin are 8 consecutive floats of the
    // table (two 16-byte loads) -- rotates them, and stores them as one 16-byte bf16 word:
    // Q rows to q_out, K / V rows to their ring slots; V tiles also fill the transposed
    // copy along keys. The tile lies in one of the Q / K / V sections.
    const int sec = tn * BN / g.D;
    float* T = reinterpret_cast<float*>(lds);
    constexpr int HALF = BN / 2, CPR = HALF / 8;  // columns per half, 8-column chunks per row
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      __syncthreads();  // the pipeline stages (first half) / the previous half are no longer read
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const int rl = wm * 32 * MI + i * 32 + 8 * jj + 4 * (lane >> 5) + ii;
#pragma unroll
            for (int j = 0; j < NI; ++j) {
              const int cl = wn * 32 * NI + j * 32 + (lane & 31) - half * HALF;
              if (cl >= 0 && cl < HALF) T[rl * TPF + cl] = acc[i][j][4 * jj + ii];
            }
          }
      // thread tid takes items idx = tid + it*NW*64 (row idx / CPR, 8-column chunk idx % CPR);
      // the RoPE table values of all its items are loaded before the first store (loads
      // interleaved with the stores would wait one memory round trip per item)
      constexpr int NIT = (BM * CPR + NW * 64 - 1) / (NW * 64);
      f32x4 rc0[NIT], rc1[NIT];
      if (sec < 2) {
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
          const int idx = tid + it * NW * 64;
          const int rl = idx / CPR, c = idx - rl * CPR;
          const int row = m0 + rl < g.M ? m0 + rl : g.M - 1;  // clamped: in-bounds, unused
          const int wcol = tn * BN + half * HALF + c * 8 - sec * g.D;
          const int d = wcol % g.dh;
          const float* rp = g.rope + (size_t)row * g.dh + d;
          rc0[it] = idx < BM * CPR ? *reinterpret_cast<const f32x4*>(rp) : f32x4{0.f, 0.f, 0.f, 0.f};
          rc1[it] = idx < BM * CPR ? *reinterpret_cast<const f32x4*>(rp + 4) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
      __syncthreads();
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int idx = tid + it * NW * 64;
        if (idx >= BM * CPR) continue;
        const int rl = idx / CPR, c = idx - rl * CPR;
        const int row = m0 + rl;
        if (row >= g.M) continue;
        const int wcol = tn * BN + half * HALF + c * 8 - sec * g.D;
        const int head = wcol / g.dh, d = wcol - head * g.dh;
        const f32x4 lo = *reinterpret_cast<const f32x4*>(T + rl * TPF + c * 8);
        const f32x4 hi = *reinterpret_cast<const f32x4*>(T + rl * TPF + c * 8 + 4);
        float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        if (sec < 2) {
          const f32x4 c0 = rc0[it], c1 = rc1[it];
          const float cs[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const float e = v[2 * k], o = v[2 * k + 1], cc = cs[2 * k], sn = cs[2 * k + 1];
            v[2 * k] = e * cc - o * sn;
            v[2 * k + 1] = e * sn + o * cc;
          }
        }
        // K and V go to the ring as bfloat16 (the cache type, read by decode). The chunk's
        // own attention takes Q and K as float16 (Q here, K in the key space): an 8-bit
        // significand on both sides of Q.K^T costs about as much accuracy per block as the
        // ring's rounding itself.
        uint32_t pk[4], ph[4];
        const float hs = ldexpf(1.0f, -(sec == 0 ? g.q16_exp : g.k16_exp));   // float16 copy scale
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          pk[k] = (uint32_t)f32_to_bf16(v[2 * k]) | ((uint32_t)f32_to_bf16(v[2 * k + 1]) << 16);
          ph[k] = (uint32_t)f32_to_f16(v[2 * k] * hs) | ((uint32_t)f32_to_f16(v[2 * k + 1] * hs) << 16);
        }
        if (sec == 0) {
          *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(g.q_out) + ((size_t)head * g.M + row) * g.dh + d) =
              u32x4{ph[0], ph[1], ph[2], ph[3]};
        } else {
          *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(sec == 1 ? g.kc : g.vc) +
                                    ((size_t)head * g.C + (g.p0 + row) % g.C) * g.dh + d) = u32x4{pk[0], pk[1], pk[2], pk[3]};
          if (sec == 1 && g.kx)
            *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(g.kx) + ((size_t)head * g.x_pitch + g.xoff + row) * g.dh + d) =
                u32x4{ph[0], ph[1], ph[2], ph[3]};
        }
      }
      if (sec == 2 && g.vt) {
        // key t of the tile sits in column xoff + vt_perm(t) (xoff is a multiple of 16);
        // 8 consecutive columns from 8 rows
        const int pend = m0 + BM < g.vt_pitch - g.xoff ? m0 + BM : g.vt_pitch - g.xoff;
        for (int idx = tid; idx < HALF * (BM / 8); idx += NW * 64) {
          const int cl = idx / (BM / 8), pg = idx - cl * (BM / 8);
          const int p = m0 + pg * 8;
          if (p >= pend) continue;
          const int wcol = tn * BN + half * HALF + cl - 2 * g.D;
          const int head = wcol / g.dh, d = wcol - head * g.dh;
          uint32_t wv[4];
          const float vs = ldexpf(1.0f, -g.vt_exp);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r0 = vt_perm(p + 2 * e) - m0, r1 = vt_perm(p + 2 * e + 1) - m0;
            wv[e] = (uint32_t)f32_to_f16(T[r0 * TPF + cl] * vs) | ((uint32_t)f32_to_f16(T[r1 * TPF + cl] * vs) << 16);
          }
          *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(g.vt) + ((size_t)head * g.dh + d) * g.vt_pitch + g.xoff + p) =
              u32x4{wv[0], wv[1], wv[2], wv[3]};
        }
      }
    }
  } else if constexpr (EPI == GEPI_RESID) {
    // x += C, one row of 32 x 32 tiles (i) at a time: its NI*16 residual values per lane are
    // all loaded before the first of its stores (the loads are independent; interleaved with
    // stores to the same array they would wait one memory round trip per pair), then added
    // and stored. Lanes 0-31 / 32-63 cover 32 consecutive columns of one row (128-byte runs).
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      float xv[NI][16];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int row = m0 + wm * 32 * MI + i * 32 + 8 * jj + 4 * (lane >> 5) + ii;
          const int rc = row < g.M ? row : g.M - 1;  // clamped: the loads are unconditional
#pragma unroll
          for (int j = 0; j < NI; ++j) {
            const int col = tn * BN + wn * 32 * NI + j * 32 + (lane & 31);
            xv[j][4 * jj + ii] = g.x[(size_t)rc * g.N + col];
          }
        }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int row = m0 + wm * 32 * MI + i * 32 + 8 * jj + 4 * (lane >> 5) + ii;
          if (row >= g.M) continue;
#pragma unroll
          for (int j = 0; j < NI; ++j) {
            const int col = tn * BN + wn * 32 * NI + j * 32 + (lane & 31);
            g.x[(size_t)row * g.N + col] = xv[j][4 * jj + ii] + acc[i][j][4 * jj + ii];
          }
        }
    }
  } else {
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int row = m0 + wm * 32 * MI + i * 32 + 8 * jj + 4 * (lane >> 5) + ii;
        if (EPI == GEPI_SWIGLU) {
#pragma unroll
          for (int j = 0; j < NI / 2; ++j) {
            const float gv = acc[i][j][4 * jj + ii], zv = acc[i][j + NI / 2][4 * jj + ii];
            if (row < g.M) {
              const int col = tn * (BN / 2) + wn * 16 * NI + j * 32 + (lane & 31);
              static_cast<uint16_t*>(g.s_out)[(size_t)row * g.F + col] = f32_to_f16(silu(gv) * zv * ldexpf(1.0f, -g.s16_exp));
            }
          }
        } else {
#pragma unroll
          for (int j = 0; j < NI; ++j) {
            const int col = tn * BN + wn * 32 * NI + j * 32 + (lane & 31);
            if (row < g.M) gemm_store<bf16_t, EPI>(g, row, col, acc[i][j][4 * jj + ii], 0.f);
          }
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

// MFMA tile configurations (waves WM x WN, MI x NI 32 x 32 tiles per wave, LDS stages,
// k-tile width).
struct GemmCfg {
  int wm, wn, mi, ni, ns, kb, late;
  int bm() const { return wm * 32 * mi; }
  int bn() const { return wn * 32 * ni; }
};
#define PP_GEMM_CFGS(X)         \
  X(0, 2, 4, 3, 2, 2, 64, 1)    \
  X(1, 2, 4, 2, 2, 3, 64, 0)    \
  X(2, 2, 2, 3, 2, 3, 64, 0)    \
  X(3, 2, 2, 2, 2, 4, 64, 0)    \
  X(4, 2, 4, 3, 2, 2, 64, 0)    \
  X(5, 2, 2, 3, 4, 2, 64, 1)    \
  X(6, 2, 2, 2, 2, 4, 64, 1)    \
  X(7, 2, 4, 2, 2, 3, 64, 1)    \
  X(8, 2, 2, 3, 2, 3, 64, 1)    \
  X(9, 1, 4, 7, 2, 2, 64, 1)    \
  X(10, 1, 4, 7, 2, 2, 64, 0)
static const GemmCfg kGemmCfgs[] = {
#define PP_CFG_ROW(id, wm, wn, mi, ni, ns, kb, late) {wm, wn, mi, ni, ns, kb, late},
    PP_GEMM_CFGS(PP_CFG_ROW)
#undef PP_CFG_ROW
};
constexpr int kNumGemmCfgs = sizeof(kGemmCfgs) / sizeof(kGemmCfgs[0]);
// Per-configuration efficiency, from whole-prefill timings with one configuration forced:
// the late-barrier 192 x 256 tile is the fastest at T = 3000 (the early one 4 % slower, the
// four-wave 96 x 128-per-wave variant 3 %); smaller tiles re-read more weight and activation
// k-slices per product.
static const double kGemmEff[kNumGemmCfgs] = {1.0, 0.95, 0.85, 0.8, 0.96, 0.97, 0.8, 0.9, 0.85, 1.0, 0.96};

static bool cfg_fits(const GemmCfg& c, const GemmArgs& g, int epi) {
  if (epi == GEPI_SWIGLU) return c.ni % 2 == 0 && g.F % (c.bn() / 2) == 0;
  // QKV tiles must not straddle the Q / K / V sections (their 16-byte stores stay in one head)
  if (epi == GEPI_QKV) return g.N % c.bn() == 0 && g.D % c.bn() == 0 && g.dh % 8 == 0;
  return g.N % c.bn() == 0;
}

// The configuration with the least work on the busiest CU, ceil(tiles / n_cu) * tile
// area, scaled by its efficiency.
static int pick_cfg(const GemmArgs& g, int epi, int n_cu) {
  int best = -1;
  double best_cost = 0;
  for (int i = 0; i < kNumGemmCfgs; ++i) {
    const GemmCfg& c = kGemmCfgs[i];
    if (!cfg_fits(c, g, epi)) continue;
    const long n_tn = epi == GEPI_SWIGLU ? g.F / (c.bn() / 2) : g.N / c.bn();
    const long tiles = (long)((g.M + c.bm() - 1) / c.bm()) * n_tn;
    const double cost = (double)((tiles + n_cu - 1) / n_cu) * c.bm() * c.bn() / kGemmEff[i];
    if (best < 0 || cost < best_cost) {
      best = i;
      best_cost = cost;
    }
  }
  return best;
}

// Split-K sums, added in split order: x[r][c] += part[0][r][c] + part[1][r][c] + ...
__global__ __launch_bounds__(kBlock) void k_splitk_resid(const float* __restrict__ part, float* __restrict__ x,
                                                         long long mn, int n_split, int acc_exp) {
  const long long i = ((long long)blockIdx.x * kBlock + threadIdx.x) * 4;
  if (i >= mn) return;
  f32x4 acc = *reinterpret_cast<const f32x4*>(part + i);
  for (int s = 1; s < n_split; ++s) acc += *reinterpret_cast<const f32x4*>(part + (size_t)s * mn + i);
  f32x4* xp = reinterpret_cast<f32x4*>(x + i);
  *xp = *xp + acc * ldexpf(1.0f, acc_exp);
}
// s_out[r][j] = SiLU(g) * z as float16, g = the split sums of B row j, z of B row F + j.
__global__ __launch_bounds__(kBlock) void k_splitk_swiglu(const float* __restrict__ part, uint16_t* __restrict__ s_out,
                                                          int M, int F, int n_split, int acc_exp, int s16_exp) {
  const long long i = ((long long)blockIdx.x * kBlock + threadIdx.x) * 4;  // (r, j), j % 4 == 0
  if (i >= (long long)M * F) return;
  const long long r = i / F, j = i - r * F;
  const size_t ms = (size_t)M * 2 * F;
  const float* p = part + (size_t)r * 2 * F + j;
  f32x4 gs = *reinterpret_cast<const f32x4*>(p), zs = *reinterpret_cast<const f32x4*>(p + F);
  for (int s = 1; s < n_split; ++s) {
    gs += *reinterpret_cast<const f32x4*>(p + s * ms);
    zs += *reinterpret_cast<const f32x4*>(p + s * ms + F);
  }
  const float am = ldexpf(1.0f, acc_exp), ss = ldexpf(1.0f, -s16_exp);
  gs *= am;
  zs *= am;
  const uint32_t lo = (uint32_t)f32_to_f16(silu(gs.x) * zs.x * ss) | ((uint32_t)f32_to_f16(silu(gs.y) * zs.y * ss) << 16);
  const uint32_t hi = (uint32_t)f32_to_f16(silu(gs.z) * zs.z * ss) | ((uint32_t)f32_to_f16(silu(gs.w) * zs.w * ss) << 16);
  *reinterpret_cast<u32x2*>(s_out + i) = u32x2{lo, hi};
}

// Splits of K for a product with `tiles` output tiles: enough workgroups for every CU, at
// least 4 k-tiles per split, partial sums within the workspace; 1 = no split (also for the
// QKV epilogue, which stays fused).
static int pick_split(int epi, const GemmArgs& g, int tiles, int n_cu) {
  if (!g.part || epi == GEPI_QKV || tiles * 2 > n_cu) return 1;
  const size_t ncol = epi == GEPI_SWIGLU ? 2 * (size_t)g.F : (size_t)g.N;
  const size_t per_split = (size_t)g.M * ncol * sizeof(float);
  int sp = n_cu / tiles;
  sp = sp < 8 ? sp : 8;
  const int nk = g.K / GBK;
  while (sp > 1 && (nk / sp < 4 || per_split * sp > g.part_bytes)) --sp;
  return sp;
}

template <int EPI, int WM, int WN, int MI, int NI, int NS, int KB, bool LATE>
static hipError_t launch_cfg(const GemmArgs& g, int n_cu, hipStream_t s) {
  constexpr int BM = WM * 32 * MI, BN = WN * 32 * NI;
  const int n_tn = EPI == GEPI_SWIGLU ? g.F / (BN / 2) : g.N / BN;
  const int n_tm = (g.M + BM - 1) / BM;
  const int sp = pick_split(EPI, g, n_tm * n_tn, n_cu);
  if (EPI == GEPI_RESID && g.tag == 1)
    hipLaunchKernelGGL((k_gemm_f16<EPI, WM, WN, MI, NI, NS, KB, LATE, 1>), dim3(n_tm * n_tn, sp), dim3(WM * WN * 64), 0, s, g);
  else
    hipLaunchKernelGGL((k_gemm_f16<EPI, WM, WN, MI, NI, NS, KB, LATE, 0>), dim3(n_tm * n_tn, sp), dim3(WM * WN * 64), 0, s, g);
  if (sp > 1) {
    if (EPI == GEPI_RESID) {
      const long long mn = (long long)g.M * g.N;
      hipLaunchKernelGGL(k_splitk_resid, dim3((unsigned)((mn / 4 + kBlock - 1) / kBlock)), dim3(kBlock), 0, s, g.part, g.x,
                         mn, sp, g.acc_exp);
    } else if (EPI == GEPI_SWIGLU) {
      const long long mf = (long long)g.M * g.F;
      hipLaunchKernelGGL(k_splitk_swiglu, dim3((unsigned)((mf / 4 + kBlock - 1) / kBlock)), dim3(kBlock), 0, s, g.part,
                         static_cast<uint16_t*>(g.s_out), g.M, g.F, sp, g.acc_exp, g.s16_exp);
    }
  }
  return hipGetLastError();
}

template <int EPI>
static hipError_t gemm_dispatch(bool bf16, const GemmArgs& g, int n_cu, hipStream_t s) {
  if (bf16) {
    const int c = pick_cfg(g, EPI, n_cu > 0 ? n_cu : 256);
    switch (c) {
#define PP_CFG_CASE(id, wm, wn, mi, ni, ns, kb, late) \
  case id:                                            \
    if constexpr (EPI != GEPI_SWIGLU || ni % 2 == 0) return launch_cfg<EPI, wm, wn, mi, ni, ns, kb, late != 0>(g, n_cu > 0 ? n_cu : 256, s); \
    break;
      PP_GEMM_CFGS(PP_CFG_CASE)
#undef PP_CFG_CASE
      default: return hipErrorInvalidValue;
    }
  } else {
    const int n_tm = (g.M + 63) / 64;
    const int n_tn = EPI == GEPI_SWIGLU ? (g.F + 31) / 32 : (g.N + 63) / 64;
    hipLaunchKernelGGL(k_gemm_f32<EPI>, dim3(n_tm * n_tn), dim3(256), 0, s, g);
  }
  return hipGetLastError();
}

// The prefill's float16 copy of a bf16 matrix, w * 2^-w_exp: one 16-byte word (8 values)
// per thread. The exponent is chosen per matrix so its largest |w| lands in [2^14, 2^15);
// bfloat16's significand is the shorter, so values inside float16's normal range convert
// exactly, and the rest (below 2^-14 after scaling) round to nearest even.
__global__ __launch_bounds__(kBlock) void k_bf16_to_f16(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                        long long n16, float scale) {
  const long long i = (long long)blockIdx.x * kBlock + threadIdx.x;
  if (i >= n16) return;
  const u32x4 v = src[i];
  u32x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    o[e] = (uint32_t)f32_to_f16(bf16_lo(v[e]) * scale) | ((uint32_t)f32_to_f16(bf16_hi(v[e]) * scale) << 16);
  dst[i] = o;
}

hipError_t launch_bf16_to_f16(const void* src, void* dst, size_t n_elems, int w_exp, hipStream_t s) {
  if (n_elems % 8) return hipErrorInvalidValue;
  const long long n16 = (long long)(n_elems / 8);
  hipLaunchKernelGGL(k_bf16_to_f16, dim3((unsigned)((n16 + kBlock - 1) / kBlock)), dim3(kBlock), 0, s,
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n16, std::ldexp(1.0f, -w_exp));
  return hipGetLastError();
}

hipError_t launch_gemm(int epi, bool bf16, const GemmArgs& g, int n_cu, hipStream_t s) {
  if (g.M <= 0) return hipSuccess;
  if (bf16) {
    // MFMA tiles: K in steps of 64, and N (SwiGLU: F) must split into some configuration's tiles
    if (g.K % GBK) return hipErrorInvalidValue;
    bool any = false;
    for (int i = 0; i < kNumGemmCfgs; ++i) any = any || cfg_fits(kGemmCfgs[i], g, epi);
    if (!any) return hipErrorInvalidValue;
    // buffer loads address A and B with 32-bit byte offsets
    const size_t b_rows = epi == GEPI_SWIGLU ? 2 * (size_t)g.F : (size_t)g.N;
    // (rows of the last A tile past M included: they are read as zeros)
    if (((size_t)g.M + 256) * g.K * 2 > 0xffffffffull || b_rows * g.K * 2 > 0xffffffffull) return hipErrorInvalidValue;
  } else if (epi == GEPI_QKV && (g.dh % 2)) {
    return hipErrorInvalidValue;
  }
  switch (epi) {
    case GEPI_QKV: return gemm_dispatch<GEPI_QKV>(bf16, g, n_cu, s);
    case GEPI_RESID: return gemm_dispatch<GEPI_RESID>(bf16, g, n_cu, s);
    case GEPI_SWIGLU: return gemm_dispatch<GEPI_SWIGLU>(bf16, g, n_cu, s);
  }
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------- flash attention (bf16-weight path)

// Workgroup = 128 queries of one head, 4 waves; wave w owns queries qb*128 + 32w .. +31,
// one per lane column (lane % 32). Keys go by blocks of 64 through two LDS stages, loaded
// straight from global memory: float16 K rows of the chunk's key space and the matching 64
// columns of the transposed float16 V copy; Q is float16 as well. Query i is key index
// koff + i. Per key block:
//   S^T = K Q^T   (A = K rows from LDS, B = Q^T kept in registers): lane (q, half) holds
//                 q's scores for 32 of the 64 keys, its partner lane (lane ^ 32) the other
//                 32, so the row max and sum need one exchange;
//   O^T += V^T P^T (A = V^T from LDS, B = P^T straight from the S^T registers: the k index
//                 of this product runs over the keys in the order the lane holds them,
//                 which is the column order of the transposed V copy).
// Softmax in base 2 with the 1/sqrt(d) scale folded into one FMA; the running max/sum
// rescale O^T in registers only when some lane's block max exceeds the reference max by
// more than 8 (base-2 exponent units), so most key blocks skip it. Masks (causal, window, end of
// sequence) are applied only on key blocks that need them; key blocks entirely in a
// wave's future are skipped by that wave.
// Key split (gridDim.y > 1): workgroup row y takes its share of the query block's key
// blocks and writes the unnormalised O, the running max and the sum, float32, for
// k_attn_prefill_combine.
template <int DH>
__global__ __launch_bounds__(256, 2) void k_attn_prefill_f16(AttnPrefillArgs a) {
  constexpr int BQ = 128, BKV = 64;
  constexpr int KCH = DH / 8;                  // 16-byte chunks per K row
  // slot of chunk c of K row r: 256-byte rows (d_head 128) span the bank window, so XOR
  // with r & 15 spreads 16 rows; 128-byte rows (d_head 64) use the GEMM tiles' swizzle
  auto kslot = [](int r, int c) { return KCH == 16 ? c ^ (r & 15) : swz_slot(r, c); };
  constexpr int KRPI = 64 / KCH;               // K rows per LDS-load instruction
  constexpr int KL = BKV * KCH / 256;          // K loads per wave per key block
  constexpr int VL = DH * 8 / 256;             // V^T loads per wave per key block
  __shared__ u32x4 Ks[2][BKV * KCH];
  __shared__ u32x4 Vs[2][DH * 8];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n_qb = (a.T + BQ - 1) / BQ;
  // longest query blocks first over all heads; head h lands on XCD h mod 8 (H % 8 == 0
  // keeps a head's keys in one L2)
  const int qb = n_qb - 1 - (int)blockIdx.x / a.H;
  const int h = (int)blockIdx.x % a.H;
  const int hi = lane >> 5, ql = lane & 31;
  const int qw0 = qb * BQ + w * 32;            // first query of this wave
  const int qi = qw0 + ql;                     // this lane's query
  const int qrow = qi < a.T ? qi : a.T - 1;

  f16x8 qr[DH / 16];
  const uint16_t* Q = static_cast<const uint16_t*>(a.q) + ((size_t)h * a.T + qrow) * DH;
#pragma unroll
  for (int ks = 0; ks < DH / 16; ++ks) qr[ks] = *reinterpret_cast<const f16x8*>(Q + ks * 16 + 8 * hi);

  const int ko = a.koff, nk = a.koff + a.T;
  const u32x4 krs = rsrc_words(static_cast<const uint16_t*>(a.k) + (size_t)h * a.k_pitch * DH, (uint32_t)((size_t)nk * DH * 2));
  const u32x4 vrs = rsrc_words(static_cast<const uint16_t*>(a.vt) + (size_t)h * DH * a.vt_pitch,
                               (uint32_t)((size_t)DH * a.vt_pitch * 2));
  uint32_t koff[KL], voff[VL];
#pragma unroll
  for (int j = 0; j < KL; ++j) {
    const int r = (w + 4 * j) * KRPI + lane / KCH, slot = lane % KCH;
    koff[j] = (uint32_t)(r * DH * 2 + (kslot(r, slot) * 16));
  }
#pragma unroll
  for (int j = 0; j < VL; ++j) {
    const int d = (w + 4 * j) * 8 + lane / 8, slot = lane % 8;
    voff[j] = (uint32_t)((size_t)d * a.vt_pitch * 2 + (swz_slot(d, slot) * 16));
  }
  auto issue = [&](int k0, int st) {
#pragma unroll
    for (int j = 0; j < KL; ++j) lds_dma16(krs, koff[j], (uint32_t)(k0 * DH * 2), lds_addr(&Ks[st][(w + 4 * j) * 64]));
#pragma unroll
    for (int j = 0; j < VL; ++j) lds_dma16(vrs, voff[j], (uint32_t)(k0 * 2), lds_addr(&Vs[st][(w + 4 * j) * 64]));
  };

  const float c = a.scale * 1.4426950408889634f;  // scores -> base-2 exponent units
  float m = -INFINITY, l = 0.f;
  f32x16 o[DH / 32];
#pragma unroll
  for (int dt = 0; dt < DH / 32; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[dt][e] = 0.f;

  const int qlast = (qb + 1) * BQ < a.T ? (qb + 1) * BQ - 1 : a.T - 1;
  int kfirst = ko + qb * BQ - a.C + 1;
  kfirst = (kfirst > a.jlo ? kfirst : a.jlo) / BKV * BKV;
  const int nkb_all = (ko + qlast - kfirst) / BKV + 1;
  const int n_split = gridDim.y, split = blockIdx.y;
  const int kb_lo = split * nkb_all / n_split;
  const int nkb = (split + 1) * nkb_all / n_split - kb_lo;
  kfirst += kb_lo * BKV;

  if (nkb > 0) issue(kfirst, 0);
  // Q is waited for here, once (together with the first K / V block, issued just above):
  // passed through an empty asm statement, its registers are no longer pending loads to the
  // compiler, which would otherwise wait on the vector-memory counter before the score
  // products of every key block -- a counter the K / V prefetch (issued by asm, invisible to
  // the compiler) also counts, so those waits would drain the prefetch every block.
#pragma unroll
  for (int ks = 0; ks < DH / 16; ++ks) asm volatile("" : "+v"(qr[ks]));
  for (int kb = 0; kb < nkb; ++kb) {
    const int st = kb & 1, k0 = kfirst + kb * BKV;
    vm_wait_barrier<0>();
    if (kb + 1 < nkb) issue(k0 + BKV, st ^ 1);
    if (k0 > ko + qw0 + 31) continue;  // the whole block is in this wave's future

    // ---- S^T: s[kt][4*jj + ii] is key k0 + 32*kt + 8*jj + 4*hi + ii
    f32x16 s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s[kt][e] = 0.f;
#pragma unroll
      for (int ks = 0; ks < DH / 16; ++ks) {
        const int r = kt * 32 + ql, ch = ks * 2 + hi;
        const f16x8 ka = __builtin_bit_cast(f16x8, Ks[st][r * KCH + kslot(r, ch)]);
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka, qr[ks], s[kt], 0, 0, 0);
      }
    }
    // masking only where the block needs it (causal, window, end of keys, first visible
    // key); the compiler flattens this branch into selects (one range test per score)
    const bool masked = k0 + BKV - 1 > ko + qw0 || k0 < ko + qw0 + 31 - a.C + 1 || k0 + BKV > nk || k0 < a.jlo;
    if (masked) {
      // this lane's visible keys form one range [lo, hi]: one unsigned compare per score
      const int lo = max(a.jlo, ko + qi - a.C + 1), hi_k = min(ko + qi, nk - 1);
      const uint32_t span = (uint32_t)(hi_k - lo);  // huge (wrapped) when the range is empty
      const int base = k0 + 4 * hi - lo;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const uint32_t off = (uint32_t)(base + 32 * kt + 8 * (e >> 2) + (e & 3));
          s[kt][e] = (hi_k >= lo && off <= span) ? s[kt][e] : -INFINITY;
        }
    }
    float mb = s[0][0];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 16; ++e) mb = fmaxf(mb, s[kt][e]);
    mb = fmaxf(mb, __shfl_xor(mb, 32, kWave));
    const float mn = fmaxf(m, mb);
    // Lazy rescaling: the reference max m moves (and O, l are rescaled) only when some
    // lane's block max exceeds it by more than 2^8 in probability terms, so p <= 256
    // (exact in float16 to the same relative precision) and the final O / l is unchanged.
    // Also taken while m is -inf (the comparison with NaN fails).
    if (__ballot(!((mn - m) * c <= 8.f))) {
      const float mref = mn == -INFINITY ? 0.f : mn;  // rows with nothing visible yet
      const float sc = __builtin_amdgcn_exp2f((m - mref) * c);
      l *= sc;
#pragma unroll
      for (int dt = 0; dt < DH / 32; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[dt][e] *= sc;
      m = mn;
    }
    const float moff = -(m == -INFINITY ? 0.f : m) * c;

    // ---- P^T (bf16) and O^T += V^T P^T, 16 keys per step
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int kt = t >> 1, j8 = 8 * (t & 1);
      f16x8 pb;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[kt][j8 + i], c, moff));
        l += p;
        pb[i] = (_Float16)p;
      }
      const int vch = kt * 4 + 2 * (t & 1) + hi;
#pragma unroll
      for (int dt = 0; dt < DH / 32; ++dt) {
        const int d = dt * 32 + ql;
        const f16x8 va = __builtin_bit_cast(f16x8, Vs[st][swz(d, vch)]);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pb, o[dt], 0, 0, 0);
      }
    }
  }

  // ---- normalise and write: o[dt][4*jj + ii] is dim dt*32 + 8*jj + 4*hi + ii of query qi
  const float lt = l + __shfl_xor(l, 32, kWave);
  if (n_split > 1) {
    // partials: O [split][h][t][DH], then (max, sum) [split][h][t][2] after all the O
    if (qi < a.T) {
      const size_t row = ((size_t)split * a.H + h) * a.T + qi;
      float* po = a.part + row * DH;
#pragma unroll
      for (int dt = 0; dt < DH / 32; ++dt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          *reinterpret_cast<f32x4*>(po + dt * 32 + 8 * jj + 4 * hi) =
              f32x4{o[dt][4 * jj], o[dt][4 * jj + 1], o[dt][4 * jj + 2], o[dt][4 * jj + 3]};
      if (hi == 0) {
        float* pml = a.part + (size_t)n_split * a.H * a.T * DH + row * 2;
        pml[0] = m;
        pml[1] = lt;
      }
    }
    return;
  }
  const float inv = 1.0f / lt;
  if (qi < a.T) {
    uint16_t* out = static_cast<uint16_t*>(a.out) + (size_t)qi * (a.H * DH) + h * DH;
#pragma unroll
    for (int dt = 0; dt < DH / 32; ++dt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d = dt * 32 + 8 * jj + 4 * hi;
        const uint32_t w0 = (uint32_t)f32_to_f16(o[dt][4 * jj] * inv) | ((uint32_t)f32_to_f16(o[dt][4 * jj + 1] * inv) << 16);
        const uint32_t w1 = (uint32_t)f32_to_f16(o[dt][4 * jj + 2] * inv) | ((uint32_t)f32_to_f16(o[dt][4 * jj + 3] * inv) << 16);
        *reinterpret_cast<u32x2*>(out + d) = u32x2{w0, w1};
      }
  }
}

// Combines the key splits of query t, head h: with M the largest split max, weights
// w_s = 2^((m_s - M) * c), out = sum w_s O_s / sum w_s l_s. DH/4 threads per (head, query)
// row, 4 dimensions each (16-byte loads); the rows h*T + t of a workgroup are consecutive.
template <int DH>
__global__ __launch_bounds__(256) void k_attn_prefill_combine(AttnPrefillArgs a, int n_split) {
  constexpr int TPR = DH / 4, RPB = 256 / TPR, SM = 8;
  const int row = blockIdx.x * RPB + (int)threadIdx.x / TPR, d = ((int)threadIdx.x % TPR) * 4;
  const size_t plane = (size_t)a.H * a.T;
  if ((size_t)row >= plane) return;
  const float c = a.scale * 1.4426950408889634f;
  const float* pml = a.part + (size_t)n_split * plane * DH;
  float ms[SM], ls[SM];
  f32x4 os[SM];
#pragma unroll
  for (int s = 0; s < SM; ++s) {
    const int sc = s < n_split ? s : n_split - 1;  // clamped: every load is unconditional
    const size_t r = sc * plane + row;
    ms[s] = pml[r * 2];
    ls[s] = pml[r * 2 + 1];
    os[s] = *reinterpret_cast<const f32x4*>(a.part + r * DH + d);
  }
  float mx = -INFINITY;
#pragma unroll
  for (int s = 0; s < SM; ++s) mx = s < n_split ? fmaxf(mx, ms[s]) : mx;
  float den = 0.f;
  f32x4 num = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < SM; ++s) {
    if (s >= n_split || ms[s] == -INFINITY) continue;  // no visible key in this split
    const float w = __builtin_amdgcn_exp2f((ms[s] - mx) * c);
    num += w * os[s];
    den += w * ls[s];
  }
  const float inv = 1.0f / den;
  const int h = row / a.T, t = row - h * a.T;
  const uint32_t lo = (uint32_t)f32_to_f16(num.x * inv) | ((uint32_t)f32_to_f16(num.y * inv) << 16);
  const uint32_t hi = (uint32_t)f32_to_f16(num.z * inv) | ((uint32_t)f32_to_f16(num.w * inv) << 16);
  *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + (size_t)t * (a.H * DH) + h * DH + d) = u32x2{lo, hi};
}

// ---------------------------------------------------------------- float32 attention

// One workgroup of d_head threads per (query, head): online softmax over the visible keys
// of the chunk's key space, one key at a time (scores reduced through LDS). For the small
// fp32 shapes only.
template <int DH>
__global__ __launch_bounds__(DH) void k_attn_prefill_f32(AttnPrefillArgs a) {
  __shared__ float red[DH / 64 > 0 ? DH / 64 : 1];
  const int t = blockIdx.x, h = blockIdx.y, d = threadIdx.x;
  const float* Q = static_cast<const float*>(a.q);
  const float* Kg = static_cast<const float*>(a.k);
  const float* Vg = static_cast<const float*>(a.v);
  const float qd = Q[((size_t)h * a.T + t) * DH + d] * a.scale;
  float m = -INFINITY, l = 0.f, o = 0.f;
  const int qk = a.koff + t;
  const int kfirst = qk - a.C + 1 > a.jlo ? qk - a.C + 1 : a.jlo;
  for (int key = kfirst; key <= qk; ++key) {
    const size_t off = ((size_t)h * a.k_pitch + key) * DH + d;
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
    // K rows of the key space and V from its transposed copy; 64-key blocks of V^T
    if (!a.vt || a.T > a.C || a.koff % 16 || a.jlo < 0 || a.jlo > a.koff || a.k_pitch < a.koff + a.T ||
        a.vt_pitch < (a.koff + a.T + 63) / 64 * 64)
      return hipErrorInvalidValue;
    if (dh != 128 && dh != 64) return hipErrorInvalidValue;
    // key splits: enough workgroups for every CU (two per CU fit), at least 4 key blocks
    // (of 64) per split for the shortest query block, partials within the workspace
    const int wgs = (a.T + 127) / 128 * a.H;
    const int n_cu = a.n_cu > 0 ? a.n_cu : 256;
    int sp = 1;
    if (a.part && wgs * 2 <= n_cu) {
      sp = n_cu / wgs < 8 ? n_cu / wgs : 8;
      const int keys_min = a.koff - a.jlo + (a.T < 128 ? a.T : 128);  // keys of query block 0 (at most)
      const size_t per_split = (size_t)a.H * a.T * (dh + 2) * sizeof(float);
      while (sp > 1 && (keys_min / 64 / sp < 4 || per_split * sp > a.part_bytes)) --sp;
    }
    const dim3 grid(wgs, sp);
    if (dh == 128) hipLaunchKernelGGL(k_attn_prefill_f16<128>, grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(k_attn_prefill_f16<64>, grid, dim3(256), 0, s, a);
    if (sp > 1) {
      const long long rows = (long long)a.T * a.H;  // 8 (d_head 128) or 16 (64) rows per workgroup
      if (dh == 128) hipLaunchKernelGGL(k_attn_prefill_combine<128>, dim3((unsigned)((rows + 7) / 8)), dim3(256), 0, s, a, sp);
      else hipLaunchKernelGGL(k_attn_prefill_combine<64>, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, s, a, sp);
    }
  } else {
    if (a.T > a.C || a.jlo < 0 || a.jlo > a.koff || a.k_pitch < a.koff + a.T || !a.v) return hipErrorInvalidValue;
    const dim3 grid(a.T, a.H);
    if (dh == 128) hipLaunchKernelGGL(k_attn_prefill_f32<128>, grid, dim3(128), 0, s, a);
    else if (dh == 64) hipLaunchKernelGGL(k_attn_prefill_f32<64>, grid, dim3(64), 0, s, a);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- chunk history

// K rows (and float32 V rows): one thread per 16-byte chunk of a row.
template <typename T>
__global__ __launch_bounds__(kBlock) void k_gather_rows(GatherArgs a, const void* ring, void* dst) {
  constexpr int EPC = 16 / sizeof(T);
  const int cpr = a.dh / EPC;
  const long long n = (long long)a.H * a.jhi * cpr;
  const long long i = (long long)blockIdx.x * kBlock + threadIdx.x;
  if (i >= n) return;
  const int c = (int)(i % cpr);
  const long long hj = i / cpr;
  const int j = (int)(hj % a.jhi), h = (int)(hj / a.jhi);
  u32x4 v = u32x4{0u, 0u, 0u, 0u};
  if (j >= a.jlo) {
    const long long pos = a.q0 + j;   // >= 0 for j >= jlo
    v = *reinterpret_cast<const u32x4*>(static_cast<const T*>(ring) + ((size_t)h * a.C + pos % a.C) * a.dh + c * EPC);
  }
  *reinterpret_cast<u32x4*>(static_cast<T*>(dst) + ((size_t)h * a.x_pitch + j) * a.dh + c * EPC) = v;
}

// bf16 path, one workgroup per (64 keys, head): the K rows widened to float16 (the prefill
// attention's key operand; bfloat16 -> float16 is exact inside float16's normal range) and
// V transposed to float16 through LDS. Every K and V load of a thread is issued before the
// first conversion. The 64 x d_head V tile is read as whole key rows (16-byte loads, 16
// lanes per 256-byte row) and written as whole 128-byte runs of a transposed row (8
// columns per thread); column c of the tile holds key vt_perm(c). Keys below jlo are zero;
// so are the V columns past jhi up to the tile end, which the chunk's own V (written later
// by the QKV epilogue) covers. K rows are written below jhi only.
__global__ __launch_bounds__(256) void k_gather_kv16(GatherArgs a) {
  constexpr int P = 66;                      // LDS row pitch in halves (bank spread)
  constexpr int NQ = 64 * (128 / 8) / 256;   // 16-byte chunks per thread and tile, d_head <= 128
  __shared__ uint16_t tile[128 * P];         // [d][key], d_head <= 128
  const int j0 = blockIdx.x * 64, h = blockIdx.y, dh = a.dh, cpr = dh / 8;
  const uint16_t* K = static_cast<const uint16_t*>(a.kring) + (size_t)h * a.C * dh;
  const uint16_t* V = static_cast<const uint16_t*>(a.vring) + (size_t)h * a.C * dh;
  u32x4 kv[NQ], vv[NQ];
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const int q = threadIdx.x + 256 * i, jr = q / cpr, c = q - jr * cpr, j = j0 + jr;
    kv[i] = vv[i] = u32x4{0u, 0u, 0u, 0u};
    if (q < 64 * cpr && j >= a.jlo && j < a.jhi) {
      const size_t off = (size_t)((a.q0 + j) % a.C) * dh + c * 8;
      kv[i] = *reinterpret_cast<const u32x4*>(K + off);
      vv[i] = *reinterpret_cast<const u32x4*>(V + off);
    }
  }
  const float ks = ldexpf(1.0f, -a.k16_exp), vs = ldexpf(1.0f, -a.vt_exp);
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const int q = threadIdx.x + 256 * i, jr = q / cpr, c = q - jr * cpr, j = j0 + jr;
    if (q >= 64 * cpr) continue;
    if (j < a.jhi) {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w[e] = (uint32_t)f32_to_f16_sat(bf16_lo(kv[i][e]) * ks) | ((uint32_t)f32_to_f16_sat(bf16_hi(kv[i][e]) * ks) << 16);
      *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.kx) + ((size_t)h * a.x_pitch + j) * dh + c * 8) =
          u32x4{w[0], w[1], w[2], w[3]};
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tile[(c * 8 + 2 * e) * P + jr] = f32_to_f16_sat(bf16_lo(vv[i][e]) * vs);
      tile[(c * 8 + 2 * e + 1) * P + jr] = f32_to_f16_sat(bf16_hi(vv[i][e]) * vs);
    }
  }
  __syncthreads();
  for (int q = threadIdx.x; q < dh * 8; q += 256) {
    const int d = q >> 3, cg = q & 7;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = (uint32_t)tile[d * P + vt_perm(cg * 8 + 2 * e)] | ((uint32_t)tile[d * P + vt_perm(cg * 8 + 2 * e + 1)] << 16);
    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.vt) + ((size_t)h * dh + d) * a.vt_pitch + j0 + cg * 8) =
        u32x4{w[0], w[1], w[2], w[3]};
  }
}

hipError_t launch_gather_history(const GatherArgs& a, bool bf16, hipStream_t s) {
  if (a.jhi <= 0) return hipSuccess;
  if (a.jhi % 16 || a.jlo < 0 || a.jlo > a.jhi || a.q0 + a.jlo < 0 || a.x_pitch < a.jhi || a.dh % 8)
    return hipErrorInvalidValue;
  const int epc = bf16 ? 8 : 4;
  const long long nr = (long long)a.H * a.jhi * (a.dh / epc);
  const dim3 gr((unsigned)((nr + kBlock - 1) / kBlock));
  if (bf16) {
    // V^T tiles of 64 columns (the last one up to a multiple of 64) inside the V^T rows
    if (!a.vt || a.dh > 128 || (a.jhi + 63) / 64 * 64 > a.vt_pitch) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_gather_kv16, dim3((unsigned)((a.jhi + 63) / 64), (unsigned)a.H), dim3(256), 0, s, a);
  } else {
    if (!a.vx) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_gather_rows<float>, gr, dim3(kBlock), 0, s, a, a.kring, a.kx);
    hipLaunchKernelGGL(k_gather_rows<float>, gr, dim3(kBlock), 0, s, a, a.vring, a.vx);
  }
  return hipGetLastError();
}

}  // namespace pp
