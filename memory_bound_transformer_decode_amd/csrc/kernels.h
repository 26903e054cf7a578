// Host-side launchers of the decode-step kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dec {

// Record the message dec_last_error() returns on this thread.
void set_last_error(const char* msg);

// Weight storage formats of the matrix kernels: bf16, or one byte per weight with an
// fp32 scale per row -- OCP E4M3 codes or two's-complement int8 codes.
enum WFmt : int { W_BF16 = 0, W_E4M3 = 1, W_I8 = 2 };

// Counters that many work groups update or poll sit 256 bytes apart: accesses to one
// address, or to one line, are served one after another.
constexpr int COUNTER_STRIDE = 64;

// What the matrix kernels do with the fp32 row sums y[b][n] = scale[n] * sum_k W[n][k] x[b][k].
enum Epilogue : int {
  EPI_LOGITS = 0,  // out[b][n] = y                                   (LM head)
  EPI_RESID = 1,   // out[b][n] += y                                  (O and down: residual add)
  EPI_SILU = 2,    // act[b][i] = bf16(silu(y_gate[i]) * y_up[i])     (gate+up rows i, d_ff + i)
  EPI_QKV = 3      // RoPE on q/k rows, q -> fp32 buffer, k/v -> paged KV cache (QKV rows)
};

struct MatmulParams {
  const void* W;         // [N][K] bf16, E4M3 or int8
  const float* scale;    // [N] or nullptr (bf16)
  int N, K;              // weight rows, columns
  int d_ff;              // EPI_SILU: up rows start at d_ff (N = 2 d_ff)
  const uint16_t* x;     // bf16 activations [Bp][ldx]
  int ldx;
  // The QKV product's input keeps more than bf16's 8 significant bits: q and k feed a
  // softmax whose logits can be large, which turns a relative error of q or k into a
  // larger one of the attention weights.  On the matrix-vector kernels it comes as two
  // bf16 parts, x + xl (xl = bf16(v - x) of the fp32 value v, about 16 significant
  // bits; xl: [Bp][ldx], or the norm-fused kernels form both parts in LDS).  On the
  // matrix cores it comes as fp16 codes in x (x_f16 set: 11 significant bits, one
  // operand instead of two), and the weights enter the products as fp16 too.
  const uint16_t* xl;
  int x_f16;
  int Bp;                // padded batch (bucket)
  float* out;            // EPI_LOGITS / EPI_RESID: [Bp][ldo]
  int ldo;
  uint16_t* act;         // EPI_SILU: bf16 [Bp][ldact]
  int ldact;
  // EPI_QKV
  float* q;              // [Bp][Hq][dh]
  void* pool;            // KV pool (bf16 or E4M3 elements)
  int layer;
  const int32_t* seq_lens;  // [Bp]; < 0 marks a padded row (no cache write)
  const int32_t* bt;        // [Bp][bps]
  const float2* rope;       // [max_seq_len][dh / 2] (cos, sin)
  int Hq, Hkv, dh, num_blocks, bps;
  // RMSNorm fused into the matrix kernel (Bp <= 8, matrix-vector path): when nh is set,
  // x = bf16(RMSNorm(nh) ng) is computed by each work group into LDS and p.x is unused
  const float* nh;        // [Bp][K] fp32 residual stream
  const float* ng;        // [K] gain
  float eps;
  // MFMA products that split K over work groups: partial tiles and per-row-block
  // arrival counters (COUNTER_STRIDE apart, zero between launches)
  float* gpart;
  unsigned* gcnt;
  size_t gpart_floats;   // capacity of gpart
  int gcnt_n;            // counters at gcnt
  // RMSNorm folded into the MFMA products (the norm's 1 / rms is one factor per batch
  // row, so it can be applied to the products' sums).  A residual-add product (O, down)
  // with xout set also writes xout[b][r] = bf16(h_new[b][r] xg[r]) -- the next norm's
  // input times its gain; fp16 when xout_f16 (the next product is QKV) -- and, for its
  // row block rb, ssq_out[rb GEMM_SSQ_STRIDE + b] =
  // the sum of h_new[b][r]^2 over the block's rows.  A product with ssq_n > 0 multiplies
  // its sums for batch row b by 1 / sqrt(sum_{i < ssq_n} ssq_in[i GEMM_SSQ_STRIDE + b] / K
  // + eps).
  uint16_t* xout;
  int xout_f16;
  int ldxo;
  const float* xg;
  float* ssq_out;
  const float* ssq_in;
  int ssq_n;
};

// MFMA products (Bp up to 64): row blocks of GEMM_WAVES waves of 16-row tiles, K split over
// ks work groups where the row blocks alone leave the chip under-filled.
constexpr int GEMM_WAVES = 4;
// gate+up's alternative row block: 7 waves, so that d_ff = 14336 or 28672 splits into one
// row block per CU (1792 wave tiles = 256 x 7) instead of 448 of 4 waves (1.75 per CU)
constexpr int GEMM_WAVES_WIDE = 7;
constexpr int GEMM_MAX_SPLIT = 16;
constexpr int GEMM_TARGET_GROUPS = 256;  // one per CU of MI355X
struct GemmPlan {
  int n_rb;            // row blocks
  int ks;              // work groups per row block (K split)
  int waves;           // waves per work group (tiles per row block / tpw)
  int tpw;             // 16-row tiles per wave
  size_t part_floats;  // partial-tile floats the launch needs (0 when ks == 1)
};
// rows: per group (d_ff for gate+up, whose groups are 2); K; padded batch; one-byte weights
GemmPlan gemm_plan(int rows, int n_groups, int K, int Bp, bool byte_weights);
// row-block sums of squares of the folded RMSNorm: at most GEMM_SSQ_MAX row blocks of
// the residual products (d_model <= 8192), GEMM_SSQ_STRIDE batch rows apart
constexpr int GEMM_SSQ_MAX = 128;
constexpr int GEMM_SSQ_STRIDE = 64;
hipError_t launch_gemm_mfma(const MatmulParams& p, int epi, WFmt wq, bool kv_fp8, hipStream_t s);

// y = matrix x for one of the epilogues: MFMA tiles when mfma, else the matrix-vector
// kernels (batches above 8 rows in slices of 8).
hipError_t launch_matmul(const MatmulParams& p, int epi, WFmt wq, bool kv_fp8, bool mfma, hipStream_t s);

struct NormParams {
  const float* h;       // [Bp][d] fp32 (input, or output for the embedding kernel)
  float* h_out;         // embed: h written here
  const float* gain;    // [d]
  uint16_t* x;          // [Bp][d] bf16 out (fp16 when x_f16)
  uint16_t* x_lo;       // [Bp][d] bf16(x_fp32 - x) out, or nullptr (the next product is QKV
                        // on the matrix-vector kernels)
  int x_f16;            // x as fp16 codes (the next product is QKV on the matrix cores)
  int d, Bp;
  float eps;
  // embedding
  const void* E; const float* E_scale; const int32_t* ids;
  unsigned* pend;       // embedding kernel: n_pend words set to ATTN_O_PENDING2 (the step's first
  int n_pend;           // kernel marks the first layer's attention output as not yet written)
};

// h = E[ids[b]] (dequantized), x = RMSNorm(h) g
hipError_t launch_embed_norm(const NormParams& p, WFmt wq, hipStream_t s);
// x = RMSNorm(h) g
hipError_t launch_rmsnorm(const NormParams& p, hipStream_t s);

struct AttnParams {
  const float* q;         // [Bp][Hq][dh] fp32 (RoPE applied)
  const void* pool;
  int layer;
  const int32_t* seq_lens;  // [Bp]; the row's position p (attends to 0..p); < 0: no positions
  const int32_t* bt;        // [Bp][bps]
  float* part_o;          // [Bp][Hq][n_split][dh]
  float* part_ml;         // [Bp][Hq][n_split][2]
  uint16_t* o;            // [Bp][Hq * dh] bf16 out
  unsigned* cnt;          // [Bp][Hkv] split arrival counters, zero between launches
  int Bp, Hq, Hkv, dh, num_blocks, bps, n_split;
  int mfma;               // the MFMA form of the blocks' arithmetic (k_attn_mfma)
};

// Context splits per (sequence, kv head) of the attention kernel: a function of the
// shape and the padded batch only (workspaces are sized with it).
constexpr int ATTN_MAX_SPLIT = 64;
constexpr int ATTN_WAVES = 8;  // waves per attention work group
struct AttnShape {
  int Hq, Hkv, dh;
  int bps;  // block-table entries per sequence
};
int attn_splits(const AttnShape& s, int Bp);
// Workspace of one attention launch: partial outputs, partial max / sum, counters.
struct AttnScratch {
  size_t part_o, part_ml, cnt, total;  // byte offsets (256-byte aligned) and size
};
AttnScratch attn_scratch(const AttnShape& s, int Bp);

// split-K paged GQA decode attention; the last split of each (sequence, kv head)
// combines (one kernel)
hipError_t launch_attention(const AttnParams& p, bool kv_fp8, hipStream_t s);
// zero n 32-bit counters with a kernel (safe inside a captured graph)
hipError_t launch_zero_u32(unsigned* p, int n, hipStream_t s);

// Attention and the O projection of one layer in one launch (a single sequence on the
// matrix-vector path, attn_o.hip): attention's n_attn work groups first, then work
// groups that hold `rows` rows of W_o per wave in registers and wait for attention.
constexpr int ATTN_O_RMAX = 6;  // rows of W_o per wave
constexpr int ATTN_O_VMAX = 8;  // 16-byte vectors of a row per lane
constexpr int ATTN_O_WREGS = 48;  // 16-byte weight vectors a lane may hold (192 VGPRs)
// The attention output's "not yet written" value in the fused launch: a bf16 NaN pattern
// that the attention kernels never store (they store 0xFFBF in its place)
constexpr uint16_t ATTN_O_PENDING = 0xFFFFu;
constexpr unsigned ATTN_O_PENDING2 = 0xFFFFFFFFu;  // two of them
struct AttnOParams {
  AttnParams a;       // Bp = 1, MFMA form; a.o holds ATTN_O_PENDING in every element at launch
  MatmulParams m;     // the O product: x = a.o, out = h (EPI_RESID), Bp = 1
  uint16_t* next;     // the next layer's attention output (a.Hq a.dh bf16, not a.o): set to
                      // ATTN_O_PENDING by this launch
  int* abort;         // set by a wait that gave up (the launch's values are then wrong)
  int spin;           // polls before a wait gives up
  int n_attn;         // attention work groups: a.n_split a.Hkv a.Bp
  int rows;           // rows of W_o per wave, 1 .. ATTN_O_RMAX
};
// The fused launch's shape: rows of W_o per wave and attention splits such that every O
// work group is resident beside the attention work groups (one work group per CU), the
// most splits (up to attn_splits) that allow it; rows = 0 when the shape does not fit.
struct AttnOPlan {
  int rows, n_split;
};
AttnOPlan attn_o_plan(const AttnShape& s, int Bp, int N, WFmt wq, int n_cu);
// The head shapes the fused launch is built for (d_head 64 or 128, 4, 5 or 8 query heads
// per kv head).
bool attn_o_supported(int Hq, int Hkv, int dh);
hipError_t launch_attn_o(const AttnOParams& p, WFmt wq, bool kv_fp8, hipStream_t s);

// The unfused form for the unfused step (measurement only): scores S = q K^T / sqrt(dh)
// written to HBM (scores [Bp][Hq][ld_s] fp32, ld_s >= the longest context), a softmax
// kernel over each row in place, then o = P V.
hipError_t launch_attention_unfused(const AttnParams& p, float* scores, int ld_s, bool kv_fp8, hipStream_t s);

// Elementwise kernels of the unfused step (measurement only): RoPE + KV-cache write of
// the fp32 QKV rows qkv [Bp][N] (p: the QKV product's parameters), SiLU x mul of the
// fp32 gate+up rows gu [Bp][2 d_ff] into a, and h += delta over n elements.
hipError_t launch_rope_kv(const MatmulParams& p, const float* qkv, bool kv_fp8, hipStream_t s);
hipError_t launch_silu_mul(const float* gu, int d_ff, int Bp, uint16_t* a, int lda, hipStream_t s);
hipError_t launch_add(float* h, const float* delta, int n, hipStream_t s);

// top-k / top-p sampling of rows r < n with the draws uniforms[r] in [0, 1) (see
// sample.hip); 1 <= top_k <= SAMPLE_MAX_K, temperature > 0, 0 < top_p <= 1
constexpr int SAMPLE_MAX_K = 64;
hipError_t launch_sample_topkp(const float* logits, int ldl, int V, int n, const float* uniforms, float temperature,
                               int top_k, float top_p, int32_t* out, hipStream_t s);

// out[r] = argmax over v < V of logits[r][v] (first index of the largest value), r < n
hipError_t launch_argmax(const float* logits, int ldl, int V, int n, int32_t* out, hipStream_t s);

// (cos, sin)(p * theta^(-2i/dh)) for p < max_seq, i < dh/2, evaluated in double
hipError_t launch_rope_table(float2* rope, int max_seq, int dh, double theta, hipStream_t s);

// streaming read used to measure the device's HBM read bandwidth
hipError_t launch_bw_probe(const void* buf, size_t bytes, float* sink, hipStream_t s);

}  // namespace dec
