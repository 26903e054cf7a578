/*
 * dec.h -- C ABI of the MI355X (gfx950) decode-step library.
 *
 * One call, dec_step, runs one autoregressive decode step of a dense pre-norm
 * decoder-only transformer for a batch of sequences: every weight is streamed
 * from HBM once to produce one new token's logits per sequence ("GPU Inference
 * Internals", section Roofline: Why Decode Is Memory-Bound; kernel-fusion
 * architecture study, section 5 Benchmark environment).  The step is
 *
 *   h = E[id]
 *   per layer: x = RMSNorm(h) g_attn; [q;k;v] = W_qkv x; RoPE(q, k) at position p;
 *              K/V of the new token -> paged cache; o = GQA attention over positions 0..p;
 *              h += W_o o; x = RMSNorm(h) g_mlp; h += W_down (silu(W_gate x) * (W_up x))
 *   logits = W_lm (RMSNorm(h) g_final)
 *
 * (layer op sequence: "Kernels, Fusion & CUDA Graphs", opening section, and
 * "CUDA graphs & kernel fusion", Direct answer; the fused kernels follow the
 * fused-kernel table in "Kernels, Fusion & CUDA Graphs", Fix 1: kernel fusion;
 * the per-batch-size graph replay follows Fix 2: CUDA graphs).
 *
 * Conventions
 *   - Matrices are row-major [rows][cols], row = output channel, columns (the
 *     reduction axis) contiguous.  Storage is bf16, or OCP E4M3 ("e4m3fn":
 *     bias 7, max 448, no infinities) with one fp32 scale per row:
 *     W[n][k] = scale[n] * e4m3(code[n][k]).
 *   - Norm gains are fp32.  Activations inside the step: residual stream fp32,
 *     matrix operands bf16, accumulation fp32, logits fp32.
 *   - RMSNorm: g_i v_i / sqrt(mean(v^2) + eps).  RoPE: adjacent pairs
 *     (2i, 2i+1) rotated by p * theta^(-2i/dh), p = 0-based token position.
 *     Query head j reads KV head j / (n_q_heads / n_kv_heads).  Attention
 *     scale 1/sqrt(d_head); the new token attends to itself.
 *   - KV pool (caller-owned, kv_dtype elements), layout
 *       [n_layers][2 (K, V)][num_blocks][n_kv_heads][16 slots][d_head];
 *     position p of a sequence lives in block block_table[p / 16], slot p % 16.
 *   - All device pointers are device memory of the current HIP device; every
 *     pointer must be 16-byte aligned.  Every call is host-thread-safe only per
 *     context: one context is used by one thread at a time.
 *
 * Errors: every function returns a dec_status (0 = ok).  Validation happens
 * before anything is enqueued, so a failing call has no side effects; the
 * message is in dec_last_error() (thread-local).  A HIP runtime failure
 * returns DEC_E_HIP and leaves the context failed: later calls on it return
 * DEC_E_STATE until dec_destroy.
 */
#ifndef DEC_H
#define DEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct dec_ctx dec_ctx; /* opaque; created and owned by the library */

typedef enum {
  DEC_OK = 0,
  DEC_E_INVALID = -1,     /* a null pointer, a shape rule or an argument out of range */
  DEC_E_STATE = -2,       /* step before weights are loaded, or the context has failed */
  DEC_E_CAPACITY = -3,    /* n_seqs > max_batch, position >= max_seq_len, block id >= num_blocks */
  DEC_E_UNSUPPORTED = -4, /* a configuration this build does not implement */
  DEC_E_HIP = -5          /* the HIP runtime reported an error */
} dec_status;

typedef enum { DEC_BF16 = 0, DEC_FP8_E4M3 = 1 } dec_dtype;

enum {
  DEC_FLAG_EAGER = 1u,       /* launch kernels one by one instead of replaying a captured graph */
  DEC_FLAG_UNFUSED = 2u,     /* one kernel per op, intermediates through HBM (measurement only):
                                RMSNorm kernels, the matrix kernels with fp32 outputs, then RoPE +
                                KV write, SiLU x mul and residual adds as kernels of their own */
  DEC_FLAG_NO_MFMA = 4u,     /* matrix-vector kernels and vector attention at every batch size (no MFMA) */
  DEC_FLAG_CAPTURE_ALL = 8u, /* capture every batch bucket at the first step instead of lazily */
  DEC_FLAG_PERSISTENT = 16u, /* a padded batch of <= 8 whose layer input fits in LDS runs the
                                whole step as one persistent kernel with grid barriers; without
                                it (the default) every batch runs one kernel per fused op */
  DEC_FLAG_FUSED_QKV_ATTN = 32u /* batches of <= 8 with <= 4 query heads per kv head: QKV
                                projection and attention in one kernel, its attention work groups
                                waiting (bounded) for their kv head's q/k/v rows; measured slower
                                than the two kernels of the default plan */
};

typedef struct dec_config {
  int32_t n_layers;     /* >= 0 (0: embedding -> final norm -> LM head)              */
  int32_t d_model;      /* multiple of 16                                            */
  int32_t n_q_heads;    /* multiple of n_kv_heads; n_q_heads / n_kv_heads <= 8       */
  int32_t n_kv_heads;
  int32_t d_head;       /* 64 or 128                                                 */
  int32_t d_ff;         /* multiple of 16                                            */
  int32_t vocab;        /* even                                                       */
  float rms_eps;        /* > 0                                                        */
  float rope_theta;     /* > 1                                                        */
  int32_t weight_dtype; /* dec_dtype                                                  */
  int32_t kv_dtype;     /* dec_dtype                                                  */
  int32_t block_size;   /* must be 16                                                 */
  int32_t num_blocks;   /* physical blocks in the KV pool                             */
  int32_t max_batch;    /* a batch bucket: 1, 2, 4, 8, 16, 24, ..., 64; steps take up
                           to max_batch sequences, padded up to the next bucket       */
  int32_t max_seq_len;  /* positions per sequence; block tables have
                           ceil(max_seq_len / 16) entries per sequence                */
  uint32_t flags;       /* DEC_FLAG_*                                                 */
} dec_config;

typedef struct dec_mat {
  const void* w;      /* device [rows][cols] bf16 or E4M3 codes                        */
  const float* scale; /* device fp32 [rows] for E4M3 storage; must be NULL for bf16    */
} dec_mat;

typedef struct dec_weights {
  dec_mat embed;           /* [vocab][d_model]                                          */
  const float* attn_norm;  /* device [n_layers][d_model]                                */
  const dec_mat* qkv;      /* host array of n_layers: [(Hq + 2 Hkv) d_head][d_model];
                              rows: all Q heads, then K heads, then V heads; head j
                              occupies d_head consecutive rows                        */
  const dec_mat* o;        /* host array of n_layers: [d_model][Hq d_head]             */
  const float* mlp_norm;   /* device [n_layers][d_model]                                */
  const dec_mat* gate_up;  /* host array of n_layers: [2 d_ff][d_model]; rows [0, d_ff)
                              gate, rows [d_ff, 2 d_ff) up                           */
  const dec_mat* down;     /* host array of n_layers: [d_model][d_ff]                  */
  const float* final_norm; /* device [d_model]                                          */
  dec_mat lm_head;         /* [vocab][d_model] (untied from the embedding)              */
} dec_weights;

typedef struct dec_step_args {
  int32_t n_seqs;              /* 1 .. max_batch live sequences                          */
  const int32_t* token_ids;    /* host [n_seqs], each in [0, vocab)                      */
  const int32_t* seq_lens;     /* host [n_seqs]: tokens already cached = 0-based position
                                  of the new token, in [0, max_seq_len)                  */
  const int32_t* block_tables; /* host [n_seqs][ceil(max_seq_len / 16)] physical block ids;
                                  entries 0 .. seq_len / 16 must be in [0, num_blocks)    */
} dec_step_args;

typedef struct dec_info {
  int32_t kernels_per_step;  /* kernels the last step launched (graph nodes when replayed) */
  int32_t bucket;            /* padded batch of the last step                             */
  int32_t attn_splits;       /* context splits per (sequence, KV head) in the last step   */
  int32_t used_mfma;         /* 1 if the last step used the MFMA matrix kernels           */
  int32_t used_graph;        /* 1 if the last step replayed a captured graph              */
  int32_t graphs_captured;   /* buckets with a live captured graph                        */
  uint32_t flags;            /* current DEC_FLAG_* set                                    */
  int32_t persistent;        /* 1 if the last step ran as one persistent kernel            */
} dec_info;

/* Bytes of device workspace a context with this config needs (0 on an invalid
 * config; see dec_last_error).  Pure host computation. */
size_t dec_workspace_bytes(const dec_config* cfg);

/* Create a context.  hip_stream: the hipStream_t all device work goes on (NULL =
 * the default stream; graphs are captured on a private stream and replayed on
 * this one).  kv_pool: device pool laid out as above (caller-owned).
 * workspace: device buffer of at least dec_workspace_bytes(cfg) bytes,
 * 256-byte aligned (caller-owned).  logits: device fp32 [max_batch][vocab]
 * (caller-owned); rows [0, n_seqs) hold the step's logits.  The library keeps
 * the pointers and never frees them; the context must not outlive them. */
int dec_create(const dec_config* cfg, void* hip_stream, void* kv_pool, void* workspace,
               size_t workspace_bytes, float* logits, dec_ctx** out);

/* Record weight pointers (the arrays in `w` are copied; the device memory they
 * point to is not).  May be called again; any captured graphs are dropped. */
int dec_load_weights(dec_ctx* ctx, const dec_weights* w);

/* Enqueue one decode step on the context's stream and return without waiting.
 * The host arrays are copied before the call returns.  After the stream
 * reaches the end of the step, logits rows [0, n_seqs) are valid and every
 * live sequence's K and V of its new token are in the pool (at position
 * seq_len).  The caller then advances seq_lens and extends block tables. */
int dec_step(dec_ctx* ctx, const dec_step_args* args);

/* Change DEC_FLAG_EAGER / DEC_FLAG_UNFUSED / DEC_FLAG_NO_MFMA between steps
 * (captured graphs of the other mode are kept). */
int dec_set_flags(dec_ctx* ctx, uint32_t flags);

/* Matrix kernels of the step, for dec_launch_matmul. */
typedef enum {
  DEC_MAT_QKV = 0,     /* fused QKV + RoPE + KV-cache write (not launchable alone) */
  DEC_MAT_O = 1,       /* O projection + residual add                            */
  DEC_MAT_GATE_UP = 2, /* gate+up projection + SiLU x mul                        */
  DEC_MAT_DOWN = 3,    /* down projection + residual add                         */
  DEC_MAT_LM_HEAD = 4  /* LM head -> logits                                      */
} dec_matrix;

/* Enqueue one matrix kernel of the step -- `which` of layer `layer` (ignored for
 * the LM head) -- exactly as dec_step runs it, for the padded batch of the last
 * step, on the context's stream.  For measuring one kernel in isolation (weight
 * streaming is the step's dominant cost: "GPU Inference Internals", Roofline:
 * Why Decode Is Memory-Bound).  It overwrites step intermediates and, for the LM
 * head, the logits; DEC_MAT_QKV is refused because it would write the KV cache.
 * Needs a previous dec_step; DEC_E_INVALID for a bad `which` or `layer`. */
int dec_launch_matmul(dec_ctx* ctx, int which, int layer);

/* Greedy sampling after the last step: token_ids[s] = the index of the largest logit of
 * sequence s (the first one on ties; NaN never wins), for s < n_seqs of that step,
 * enqueued on the context's stream.  token_ids: device memory, int32 [n_seqs], 4-byte
 * aligned, owned by the caller.  The sampling kernel that turns the logits into token
 * ids on the GPU, so that only the ids need to be copied back ("Kernels, Fusion & CUDA
 * Graphs", Fix 1 table: sampling; "The serving engine's kernel stack").  Needs a
 * previous dec_step (DEC_E_STATE otherwise); DEC_E_INVALID for a NULL or misaligned
 * token_ids. */
int dec_sample_greedy(dec_ctx* ctx, int32_t* token_ids);

/* Top-k / top-p sampling after the last step, enqueued on the context's stream: for each
 * sequence s < n_seqs of that step, the candidates are its top_k largest logits (the
 * lower index first on equal logits; NaN ranks as -inf), weighted exp((z - z_max) /
 * temperature) in that order; the nucleus is the shortest prefix of them whose weight
 * reaches top_p of the candidates' total; token_ids[s] = the first nucleus candidate
 * whose running weight exceeds uniforms[s] times the nucleus weight.  The random draws
 * are inputs: uniforms, device float32 [n_seqs] in [0, 1), 4-byte aligned, owned by the
 * caller; token_ids: device int32 [n_seqs], 4-byte aligned, owned by the caller.  The
 * sampling step after the LM head, on the GPU ("Kernels, Fusion & CUDA Graphs", Fix 1
 * table: sampling; "The serving engine's kernel stack").  1 <= top_k <= 64, temperature
 * > 0, 0 < top_p <= 1 (DEC_E_INVALID otherwise, and for NULL or misaligned pointers);
 * needs a previous dec_step (DEC_E_STATE otherwise).  top_k = 1 is greedy sampling. */
int dec_sample(dec_ctx* ctx, const float* uniforms, float temperature, int32_t top_k, float top_p,
               int32_t* token_ids);

/* Describe the last step (kernels, bucket, path). */
int dec_get_info(const dec_ctx* ctx, dec_info* out);

/* Wait for the context's stream, release graphs and host staging, free ctx. */
int dec_destroy(dec_ctx* ctx);

/* Message of the last failing call on this thread ("" if none). */
const char* dec_last_error(void);

/* Streaming read of `bytes` of device memory at `buf` (16-byte aligned, a
 * multiple of 16), `reps` times, on `hip_stream`; returns the best observed
 * read bandwidth in bytes/s through *out.  Measures the HBM read rate the
 * kernels above can expect on this device ("GPU Inference Internals", The
 * Hardware Ledger: record the sustained bandwidth, not only the datasheet). */
int dec_bw_probe(const void* buf, size_t bytes, int reps, void* hip_stream, double* out);

#ifdef __cplusplus
}
#endif

#endif /* DEC_H */
