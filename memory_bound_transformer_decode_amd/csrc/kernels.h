// Host-side launchers of the decode-step kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dec {

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
  const void* W;         // [N][K] bf16 or E4M3
  const float* scale;    // [N] or nullptr (bf16)
  int N, K;              // weight rows, columns
  int d_ff;              // EPI_SILU: up rows start at d_ff (N = 2 d_ff)
  const uint16_t* x;     // bf16 activations [Bp][ldx]
  int ldx;
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
  // matrix-vector kernels (k_gemv): work group 0 zeroes rearm[i COUNTER_STRIDE], i <
  // n_rearm, at its start (the counters of the QKV + attention kernel before it)
  unsigned* rearm;
  int n_rearm;
  // MFMA products that split K over work groups: partial tiles and per-row-block
  // arrival counters (COUNTER_STRIDE apart, zero between launches)
  float* gpart;
  unsigned* gcnt;
  size_t gpart_floats;   // capacity of gpart
  int gcnt_n;            // counters at gcnt
  // RMSNorm folded into the MFMA products (the norm's 1 / rms is one factor per batch
  // row, so it can be applied to the products' sums).  A residual-add product (O, down)
  // with xout set also writes xout[b][r] = bf16(h_new[b][r] xg[r]) -- the next norm's
  // input times its gain -- and, for its row block rb, ssq_out[rb GEMM_SSQ_STRIDE + b] =
  // the sum of h_new[b][r]^2 over the block's rows.  A product with ssq_n > 0 multiplies
  // its sums for batch row b by 1 / sqrt(sum_{i < ssq_n} ssq_in[i GEMM_SSQ_STRIDE + b] / K
  // + eps).
  uint16_t* xout;
  int ldxo;
  const float* xg;
  float* ssq_out;
  const float* ssq_in;
  int ssq_n;
};

// MFMA products (Bp up to 64): row blocks of GEMM_WAVES waves of 16-row tiles, K split over
// ks work groups where the row blocks alone leave the chip under-filled.
constexpr int GEMM_WAVES = 4;
constexpr int GEMM_MAX_SPLIT = 16;
constexpr int GEMM_TARGET_GROUPS = 256;  // one per CU of MI355X
struct GemmPlan {
  int n_rb;            // row blocks
  int ks;              // work groups per row block (K split)
  int tpw;             // 16-row tiles per wave
  size_t part_floats;  // partial-tile floats the launch needs (0 when ks == 1)
};
// rows: per group (d_ff for gate+up, whose groups are 2); K; padded batch; E4M3 weights
GemmPlan gemm_plan(int rows, int n_groups, int K, int Bp, bool fp8);
// row-block sums of squares of the folded RMSNorm: at most GEMM_SSQ_MAX row blocks of
// the residual products (d_model <= 8192), GEMM_SSQ_STRIDE batch rows apart
constexpr int GEMM_SSQ_MAX = 128;
constexpr int GEMM_SSQ_STRIDE = 64;
hipError_t launch_gemm_mfma(const MatmulParams& p, int epi, bool w_fp8, bool kv_fp8, hipStream_t s);

// y = matrix x for one of the epilogues: MFMA tiles when mfma, else the matrix-vector
// kernels (batches above 8 rows in slices of 8).
hipError_t launch_matmul(const MatmulParams& p, int epi, bool w_fp8, bool kv_fp8, bool mfma,
                         hipStream_t s);

struct NormParams {
  const float* h;       // [Bp][d] fp32 (input, or output for the embedding kernel)
  float* h_out;         // embed: h written here
  const float* gain;    // [d]
  uint16_t* x;          // [Bp][d] bf16 out
  int d, Bp;
  float eps;
  // embedding
  const void* E; const float* E_scale; const int32_t* ids;
};

// h = E[ids[b]] (dequantized), x = RMSNorm(h) g
hipError_t launch_embed_norm(const NormParams& p, bool w_fp8, hipStream_t s);
// x = RMSNorm(h) g
hipError_t launch_rmsnorm(const NormParams& p, hipStream_t s);

struct AttnParams {
  const float* q;         // [Bp][Hq][dh] fp32 (RoPE applied)
  const void* pool;
  int layer;
  const int32_t* seq_lens;  // [Bp]
  const int32_t* bt;        // [Bp][bps]
  float* part_o;          // [Bp][Hq][n_split][dh]
  float* part_ml;         // [Bp][Hq][n_split][2]
  uint16_t* o;            // [Bp][Hq * dh] bf16 out
  unsigned* cnt;          // [Bp][Hkv] split arrival counters, zero between launches
  int Bp, Hq, Hkv, dh, num_blocks, bps, n_split;
  int mfma;               // the MFMA form of the blocks' arithmetic (k_attn_mfma)
  // QKV + attention kernel only: per kv head c, work groups that wrote its q/k/v rows
  // (ready[c COUNTER_STRIDE], complete at ready_target); zero at the launch (the
  // O-projection kernel that follows clears them: MatmulParams::rearm)
  unsigned* ready;
  unsigned ready_target;
  unsigned* err_dev;      // wait timeout flag, device copy
  unsigned* err_host;     // wait timeout flag, pinned host copy
  uint64_t timeout_ticks; // bound on one wait, in s_memrealtime ticks
};

// split-K paged GQA decode attention; the last split of each (sequence, kv head)
// combines (one kernel)
hipError_t launch_attention(const AttnParams& p, bool kv_fp8, hipStream_t s);

// The norm-fused QKV product (mp, Bp <= 8) and attention (ap) in one kernel: the
// attention work groups follow the product's and start once the product work groups of
// their kv head are done.  Needs d_head % (2 QKV_ATTN_IPW) == 0 and
// qkv_attn_lds_bytes(...) <= 160 KB; returns hipErrorInvalidValue otherwise.
constexpr int QKV_ATTN_IPW = 8;  // row pairs (waves) per product work group
// Query heads per kv head up to which the kernel is built: the attention state of wider
// groups does not fit the 128 registers per lane that keep two product work groups per
// CU (one work group's 8 waves at up to 4 waves per SIMD).
constexpr int QKV_ATTN_MAX_GROUP = 4;
hipError_t launch_qkv_attn(const MatmulParams& mp, const AttnParams& ap, bool w_fp8, bool kv_fp8, hipStream_t s);
// work groups of the product part; the attention part's ready_target
int qkv_attn_groups(const MatmulParams& mp);
unsigned qkv_attn_ready_target(int Hq, int Hkv, int dh);
size_t qkv_attn_lds_bytes(int Bp, int K, int Hq, int Hkv, int dh);

// ---------------------------------------------------------------- persistent step (Bp <= 8)

struct DevMat {
  const void* w;
  const float* scale;
};

struct StepParams {
  int L, d, Hq, Hkv, dh, dff, V, Bp, num_blocks, bps, n_split;
  float eps;
  int split[5];           // waves sharing one row pair's K range: QKV, O, gate+up, down, LM head
  int xs_bytes;           // LDS bytes for the activation block
  const DevMat* w_qkv;    // device arrays [L]
  const DevMat* w_o;
  const DevMat* w_gu;
  const DevMat* w_down;
  DevMat embed, lm;
  const float* attn_norm;
  const float* mlp_norm;
  const float* final_norm;
  const int32_t* ids;
  const int32_t* lens;
  const int32_t* bt;
  float* h;
  float* q;
  float* part_o;
  float* part_ml;
  uint16_t* o;
  uint16_t* a;
  const float2* rope;
  void* pool;
  float* logits;
  unsigned* bar;          // [count, generation] of the grid barrier
  unsigned* attn_cnt;     // [Bp][Hq] splits finished per head (self-resetting)
  unsigned* err_dev;      // barrier timeout flag, device copy
  unsigned* err_host;     // barrier timeout flag, pinned host copy
  uint64_t timeout_ticks; // bound on one barrier wait, in s_memrealtime ticks
};

// One launch of the whole step: grid = one work group per CU, all resident.
hipError_t launch_step(const StepParams& p, bool w_fp8, bool kv_fp8, int grid, hipStream_t s);
size_t step_lds_bytes(const StepParams& p);
int step_max_rounds();
int step_waves_per_group();

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
