// Internal interfaces between the C ABI (api.cpp) and the kernel files (*.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pp {

constexpr int kMaxStreams = 32;   // text + audio streams of the embedding sum
constexpr int kBlock = 256;       // threads per workgroup (4 waves) for every kernel here
constexpr int kMaxAttnSplits = 64;  // split-K factor of the decode attention, at most

// ---------------------------------------------------------------- embedding sum
struct EmbedArgs {
  const void* tables[kMaxStreams];  // stream k -> table [vocab_k][D]
  int32_t ids_arg[kMaxStreams];     // one frame's IDs when ids_dev == nullptr
  const int32_t* ids_dev;           // [rows][n_streams] device IDs (prefill) or nullptr
  float* out;                       // [rows][D]
  long long* state;                 // if non-null, state[0] := pos
  long long pos;
  int n_streams, D, rows;
  // RoPE table of this position (decode), computed on the host in float64 and rounded:
  // rope_cs[2j] = cos(pos * omega_j), rope_cs[2j+1] = sin(pos * omega_j), with
  // omega_j = theta^(-2j/d_head); the kernel copies it to `rope` (device) for the step.
  float* rope;
  int dh;
  float rope_cs[128];
};
hipError_t launch_embed(const EmbedArgs& a, bool bf16, hipStream_t s);

// ---------------------------------------------------------------- GEMV family (decode)
enum GemvPro {
  PRO_COPY = 0,        // x as given
  PRO_RMSNORM = 1,     // alpha * x / sqrt(mean(x^2) + eps)
  PRO_DEPTH_ATTN = 2,  // x = depth attention output computed from q and the depth cache
  PRO_ATTN_MERGE = 3,  // x = merge of the decode-attention split partials (<= 8 splits)
  PRO_LAYERNORM = 4,   // alpha * (x - mean(x)) / sqrt(var(x) + eps) + beta
};
enum GemvEpi {
  EPI_STORE = 0,   // out[row] = W x
  EPI_RESID = 1,   // out[row] += W x                       (residual stream, fp32)
  EPI_QKV = 2,     // RoPE on Q and K, q -> out, K and V -> ring slot
  EPI_SWIGLU = 3,  // rows i (g) and F + i (z): out[i] = SiLU(g) * z
  EPI_DEPTH_QKV = 4,  // depth QKV: q -> out, K and V -> depth cache row (fp32), no RoPE
};

struct GemvArgs {
  const void* W;        // [rows][K] row-major
  const float* x;       // [K] input vector
  const float* alpha;   // [K] RMSNorm / LayerNorm scale (PRO_RMSNORM, PRO_LAYERNORM)
  const float* beta;    // [K] LayerNorm shift (PRO_LAYERNORM)
  float eps;
  int K;
  int n_groups;         // row groups; a group is rows_per_group rows
  float* out;
  // EPI_QKV / EPI_DEPTH_QKV
  int D, dh, C;         // model width, head width, ring capacity (slots)
  void* kc;             // K ring of this layer, batch 0: [H][C][dh]   (depth: [H][C][dh] fp32)
  void* vc;
  const long long* state;  // state[0] = position of this frame (slot = pos mod C)
  long long pos;           // >= 0: the position itself (direct launches); -1: read state[0]
  const float* rope;       // [dh] cos/sin pairs of this frame's position
  int slot_override;    // depth: >= 0 gives the cache row directly
  // EPI_SWIGLU
  int F;
  // a second input added to the output (EPI_STORE, EPI_RESID: a bias), or null
  const float* add;
  // rows spread over several matrices: row r is row (r % rows_per_mat) of mats[r / rows_per_mat]
  // (rows_per_mat = 0: one matrix W)
  const void* mats[32];
  int rows_per_mat;
  // PRO_DEPTH_ATTN: position aq_pos of this frame's depth loop attends to the depth
  // positions p with 0 <= aq_pos - p < awin; cache [aH][acap][adh] float32
  const float* aq;
  const float* ak;
  const float* av;
  int aH, adh, acap, aq_pos, awin;
  float ascale;
  // PRO_ATTN_MERGE: partial outputs [H][S][dh] and (max, sum) pairs [H][S][2]
  const float* po;
  const float* pml;
  int pS;
};
// rows_per_group: 2 or 4; blocks: workgroups of 8 waves (normally one per CU).
hipError_t launch_gemv(int pro, int epi, bool bf16, int rows_per_group, const GemvArgs& a,
                       int blocks, hipStream_t s);

// ---------------------------------------------------------------- attention (decode)
struct AttnDecodeArgs {
  const float* q;       // [H][dh], after RoPE
  const void* k;        // ring of this layer, batch 0: [H][C][dh]
  const void* v;
  const long long* state;
  long long pos;        // >= 0: the position itself (direct launches); -1: read state[0]
  int C, H, S;          // S = splits of the key range per head
  float scale;
  float* part_o;        // [H][S][dh] partial outputs (unnormalised)
  float* part_ml;       // [H][S][2] partial (max in base-2 units, sum)
  float* out;           // [H * dh], written by the combine kernel
  int combine;          // 1: launch the combine kernel; 0: the consumer merges
  // several sessions at one position (batched decode): session b's query, ring and
  // partials follow at b * H*dh floats, b * kv_bstride elements and b * H*S*(dh | 2)
  // floats; the combine kernel writes session b's output at b * H*dh (float16 to out16
  // when it is set, in the skinny products' fragment order: frag_act_index(b, h*dh + d, H*dh))
  int batch;
  long long kv_bstride;
  uint16_t* out16;
  int o16_exp;          // out16 holds o * 2^-o16_exp
};
hipError_t launch_attn_decode(const AttnDecodeArgs& a, bool bf16, int dh, hipStream_t s);

// ---------------------------------------------------------------- row RMSNorm
// rows x D; float32 and/or float16 outputs (either may be null); f16_frag: the float16 rows in
// the skinny products' fragment order (frag_act_index, D % 32 == 0) instead of row-major
// the float16 rows are written as y * 2^-f16_exp
hipError_t launch_rmsnorm_rows(const float* x, const float* alpha, float eps, int D, int rows,
                               float* out_f32, void* out_f16, bool f16_frag, hipStream_t s, int f16_exp = 0);

// Per row of a bf16 matrix [rows][K] (K % 8 == 0): sum of squares and largest |w|.
hipError_t launch_row_stats(const void* W, int rows, int K, float* ss, float* amax, hipStream_t s);

}  // namespace pp

namespace pp {
// ---------------------------------------------------------------- depth transformer
// Per-frame control words of the depth loop, in device memory so that a captured graph
// reads them at replay time.
struct DepthCtrl {
  int32_t text;          // text token that conditions position 0
  int32_t forced[32];    // forced[q] >= 0: the code of position q; -1: selected by the model
  float temperature;     // selection rule: top_k <= 1 or temperature <= 0 -> argmax,
  int32_t top_k;         //   else temperature / top-k sampling with draw u[q]
  int32_t pad;
  double u[32];
};

struct DepthSetupArgs {
  const float* h_src;   // caller's temporal hidden [d_temporal]
  float* h_dst;         // library copy
  int d_temporal;
  DepthCtrl* ctrl;
  int32_t text_token;
  int32_t forced[32];
  int n_steps;
};
hipError_t launch_depth_setup(const DepthSetupArgs& a, hipStream_t s);

struct DepthSelectArgs {
  const float* c_all;        // [n_steps][D] temporal-to-depth projections
  const void* text_emb;      // [text_vocab][D]
  const void* audio_emb[32]; // position q > 0 reads table q-1
  const DepthCtrl* ctrl;
  const float* logits;       // [n_steps][n_out]
  int32_t* codes;            // [n_steps]
  float* z;                  // [D] residual of position q
  int q, D, n_out, n_steps;
};
constexpr int kDepthSampleMaxOut = 2048;   // sampled depth selection: n_out <= this
hipError_t launch_depth_select(const DepthSelectArgs& a, bool bf16, hipStream_t s);
}  // namespace pp

namespace pp {
// ---------------------------------------------------------------- prefill
enum GemmEpi { GEPI_QKV = 0, GEPI_RESID = 1, GEPI_SWIGLU = 2 };

struct GemmArgs {
  const void* A;        // [M][K] activations, row-major (float16 on the bf16-weight path, or float32)
  const void* B;        // weights, row-major [rows][K] (float16 copy on the bf16-weight path, or float32)
  int M, N, K;          // N = output columns (GEPI_SWIGLU: N = F, B has 2F rows)
  // GEPI_QKV: columns Q|K|V; RoPE on Q and K with rope[row][d] (cos, sin pairs);
  // Q -> q_out [H][M][dh]; K, V -> ring slots (p0 + row) mod C of [H][C][dh]
  void* q_out;
  void* kc;
  void* vc;
  const float* rope;
  int D, dh, C, p0;
  float* x;             // GEPI_RESID: x[row][col] += (A W^T)[row][col], float32 [M][N]
  void* s_out;          // GEPI_SWIGLU: [M][F] = SiLU(g) * z (float16 on the bf16-weight path)
  int F;
  // GEPI_QKV, bf16 only: Q goes to q_out as float16; if non-null, V is also written
  // transposed as float16, vt[H][dh][vt_pitch]: key index j in column vt_perm(j) (bits 2
  // and 3 of j swapped), for the prefill attention; row `row` is key index xoff + row
  void* vt;
  int vt_pitch;
  // GEPI_QKV: K (and on the float32 path V) are also written to the chunk's contiguous key
  // space kx / vx [H][x_pitch][dh] at key index xoff + row (xoff a multiple of 16), where
  // the attention reads them -- always on the bf16 path (K as float16), on the float32 path
  // for a chunk that starts past position 0
  void* kx;
  void* vx;
  int x_pitch, xoff;
  // bf16-weight path, GEPI_RESID / GEPI_SWIGLU: workspace for float32 split-K partial sums
  // (part_bytes bytes); when the product has too few output tiles to fill the GPU, K is
  // split over several workgroups per tile and the splits are added in order afterwards.
  // NULL: never split.
  float* part;
  size_t part_bytes;
  // bf16-weight path: the epilogue multiplies the products by 2^acc_exp (undoing the
  // scales of the float16 operands); the float16 outputs it writes are Q * 2^-q16_exp, the
  // K copy * 2^-k16_exp, V^T * 2^-vt_exp, SiLU(g) * z * 2^-s16_exp. Zero: no scaling.
  int acc_exp, q16_exp, k16_exp, vt_exp, s16_exp;
  int tag;   // 1: the W_out product (a separate kernel name in profiles; same code)
};
hipError_t launch_gemm(int epi, bool bf16, const GemmArgs& g, int n_cu, hipStream_t s);
// float16 copy w * 2^-w_exp of n_elems bfloat16 values (n_elems % 8 == 0), round to nearest
// even: exact unless the scaled value falls below float16's normal range (2^-14)
hipError_t launch_bf16_to_f16(const void* src, void* dst, size_t n_elems, int w_exp, hipStream_t s);

// The attention of a chunk of T frames at positions p0..p0+T-1 runs in a contiguous key
// space: key index j is position p0 - koff + j, query i is key index koff + i. Keys
// [jlo, koff) are the history gathered from the ring, [koff, koff + T) the chunk's own.
struct AttnPrefillArgs {
  const void* q;        // [H][T][dh] rotated queries (float16 on the bf16 path)
  const void* k;        // keys [H][k_pitch][dh]: the key space (float16 on the bf16 path), or on
                        // the float32 path for koff == 0 the ring itself
  const void* v;        // float32 path: values, same layout as k
  const void* vt;       // bf16 path: V transposed, float16 [H][dh][vt_pitch], key j in column vt_perm(j)
  int vt_pitch, k_pitch;
  void* out;            // [T][H*dh] (float16 on the bf16 path)
  int T, H, C;
  int koff;             // key index of query 0, a multiple of 16
  int jlo;              // first key index that exists and is inside some query's window
  float scale;
  // bf16 path: workspace for key-split partials (part_bytes bytes). When the query blocks
  // x heads cannot fill the GPU (a short chunk over a long history), each query block's
  // keys are split over several workgroups and a second pass combines them. NULL: never.
  float* part;
  size_t part_bytes;
  int n_cu;
};
hipError_t launch_attn_prefill(const AttnPrefillArgs& a, bool bf16, int dh, hipStream_t s);

// History of a chunk at p0 > 0: keys [jlo, jhi) of its key space (positions q0 + j) are
// copied from their ring slots (q0 + j) mod C -- K to kx (float16 on the bf16 path), V to vt
// (bf16 path, transposed float16) or vx (float32 path) -- and keys [0, jlo) are zero-filled.
// jhi is a multiple of 16.
struct GatherArgs {
  const void* kring;
  const void* vring;    // this layer's ring [H][C][dh]
  void* kx;
  void* vx;
  void* vt;
  int x_pitch, vt_pitch, C, H, dh;
  int k16_exp, vt_exp;  // the float16 copies hold K * 2^-k16_exp, V * 2^-vt_exp (saturated)
  long long q0;
  int jlo, jhi;
};
hipError_t launch_gather_history(const GatherArgs& a, bool bf16, hipStream_t s);

// rope[t][2j] = cos((p0 + t) * omega_j), rope[t][2j+1] = sin(...), angles in float64
hipError_t launch_rope_rows(float* rope, int T, long long p0, int dh, double log_theta, hipStream_t s);
}  // namespace pp

namespace pp {
// ---------------------------------------------------------------- generator frame
constexpr int kGenMaxRing = 8;   // code-ring slots (maximum delay + 3)
constexpr int kMaxTopK = 1024;   // sampling candidates at most

// The generator's device state: the delayed-code ring with its provided flags, and the
// current frame's temporal input, selections and text control.
struct GenState {
  int32_t tok[kMaxStreams][kGenMaxRing];
  int32_t prov[kMaxStreams][kGenMaxRing];
  int32_t ids[kMaxStreams];      // temporal input of the frame (ring slot s-1)
  int32_t chosen[kMaxStreams];   // the frame's selection per stream (supplied or sampled)
  int32_t text_forced;           // supplied text of the target slot, -1 if none
  int32_t pad;
  double u_text;                 // the text draw
};

struct GenPrepArgs {
  GenState* g;
  DepthCtrl* dctrl;
  int32_t provided[kMaxStreams];   // -1: not supplied
  int32_t delays[kMaxStreams];
  int32_t initial[kMaxStreams];
  double u[kMaxStreams];           // [0] text, [1 + q] depth position q
  long long s;                     // cursor at entry
  int n, C;
  float audio_temperature;
  int audio_top_k;
};
struct GenTextArgs {
  GenState* g;
  DepthCtrl* dctrl;
  const float* logits;   // [n] text logits of the frame
  int n;
  float temperature;
  int top_k;
};
struct GenFinishArgs {
  GenState* g;
  const int32_t* codes;   // [n_streams - 1] depth selections
  int32_t* out;           // [n_streams] aligned output, or nullptr
  int32_t delays[kMaxStreams];
  long long s;
  int n, C, max_delay;
};
constexpr int kGenTextThreads = 1024, kGenTextPer = 32;   // text rows up to 32768 logits
hipError_t launch_gen_prepare(const GenPrepArgs& a, hipStream_t s);
hipError_t launch_gen_text(const GenTextArgs& a, hipStream_t s);
hipError_t launch_gen_finish(const GenFinishArgs& a, hipStream_t s);

// rows independent draws: out[r] = sample of logits[r*n .. r*n+n) with u[r]; n <= 32768
hipError_t launch_sample_rows(const float* logits, int rows, int n, float temperature, int top_k,
                              const double* u, int32_t* out, hipStream_t s);
}  // namespace pp

namespace pp {
// ---------------------------------------------------------------- batched decode (skinny products)
enum SgemmEpi { SEPI_STORE = 0, SEPI_RESID = 1, SEPI_QKV = 2, SEPI_SWIGLU = 3 };

// out[b][n] = sum_k act[b][k] W[n][k] for the B sessions of a batched decode step:
// float16 activations, bf16 weights widened to float16, float32 accumulation.
struct SgemmArgs {
  const uint16_t* act;   // [B][K] float16 in fragment order (frag_act_index; K % 32 == 0;
                         // the buffer holds whole 16-row tiles, rows >= B are not read)
  const void* W;         // bfloat16 weights packed by launch_sgemm_pack (rows = N, or 2F g|z rows)
  int B, K, N;           // N = output columns (SEPI_SWIGLU: F)
  float* out;            // SEPI_STORE: [B][N] float32
  float* x;              // SEPI_RESID: [B][N] float32, += product
  uint16_t* s_out;       // SEPI_SWIGLU: [B][F] float16 SiLU(g) * z, in fragment order
  int F;
  // SEPI_QKV: columns Q | K | V of width D; RoPE on Q and K with rope[dh] (cos, sin pairs of
  // this position); Q -> q_out [B][D] float32; K, V -> slot pos mod C of session b's ring
  // (kc / vc + b * kv_bstride elements, [H][C][dh] bfloat16)
  float* q_out;
  void* kc;
  void* vc;
  long long kv_bstride;
  const float* rope;
  const long long* state;
  long long pos;         // >= 0: the position; -1: read state[0]
  int D, dh, C;
  // the products are multiplied by 2^acc_exp (undoing the float16 operand scales); the
  // SiLU products are written as SiLU(g) * z * 2^-s16_exp
  int acc_exp, s16_exp;
  int n_cu;              // compute units (0: 256); one session tile runs one workgroup per CU
  // RMSNorm prologue (B <= kSgemmNormMaxBatch, K <= kSgemmNormMaxK; act is then unused):
  // the activations are alpha * x / sqrt(mean(x^2) + eps) of the float32 rows xin [B][K],
  // formed by every workgroup and written to its LDS as float16 * 2^-act_exp
  const float* xin;
  const float* alpha;
  float eps;
  int act_exp;
};
constexpr int kSgemmMaxBatch = 64;
constexpr int kSgemmNormMaxBatch = 8;
constexpr int kSgemmNormMaxK = 4096;
hipError_t launch_sgemm(int epi, const SgemmArgs& a, hipStream_t s);
// Copy of a row-major [rows][K] bf16 matrix in the fragment order the skinny products
// read (same byte count); rows_out = N (or F for the SiLU-gated W_in with 2F rows).
// The packed copy holds w * 2^-w_exp (exact in bfloat16 for the exponents used).
hipError_t launch_sgemm_pack(const void* W, void* packed, int rows_out, int K, int F, bool swiglu, int w_exp,
                             hipStream_t s);
}  // namespace pp

namespace pp {
// ---------------------------------------------------------------- memory readers
// Keys (or values) of memory rows for one reader: out[h][slot][d] = (W m_slot + b)[h*dh + d]
// for slots slot0 .. slot0+n-1, stored in the weight type (float32 products).
struct ReaderKvArgs {
  const void* mem;      // [n][mem_dim] rows (weight type)
  const void* W;        // [D][mem_dim]
  const float* bias;    // [D]
  void* out;            // [H][max_slots][dh]
  int n, slot0, mem_dim, D, dh, max_slots;
};
hipError_t launch_reader_kv(const ReaderKvArgs& a, bool bf16, hipStream_t s);
}  // namespace pp

