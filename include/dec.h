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
 * Two calls run the same plan over several tokens of a sequence at once: the
 * k-token verify step of speculative decoding (dec_verify) and chunked prefill of
 * a prompt into the paged cache (dec_prefill).
 *
 * Conventions
 *   - Matrices are row-major [rows][cols], row = output channel, columns (the
 *     reduction axis) contiguous.  Storage is bf16, or one byte per weight with
 *     one fp32 scale per row: OCP E4M3 codes ("e4m3fn": bias 7, max 448, no
 *     infinities), W[n][k] = scale[n] * e4m3(code[n][k]), or two's-complement
 *     int8 codes, W[n][k] = scale[n] * code[n][k].
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
  DEC_E_CAPACITY = -3,    /* rows > max_batch, position >= max_seq_len, block id >= num_blocks */
  DEC_E_UNSUPPORTED = -4, /* a configuration this build does not implement */
  DEC_E_HIP = -5          /* the HIP runtime reported an error */
} dec_status;

/* Storage formats.  DEC_INT8 is for weights only (weight-only quantization; the
 * KV cache is bf16 or E4M3). */
typedef enum { DEC_BF16 = 0, DEC_FP8_E4M3 = 1, DEC_INT8 = 2 } dec_dtype;

enum {
  DEC_FLAG_EAGER = 1u,       /* launch kernels one by one instead of replaying a captured graph */
  DEC_FLAG_UNFUSED = 2u,     /* one kernel per op, intermediates through HBM (measurement only):
                                RMSNorm kernels, the matrix kernels with fp32 outputs, then RoPE +
                                KV write, attention as scores -> softmax -> P V with the scores in
                                HBM, SiLU x mul and residual adds as kernels of their own */
  DEC_FLAG_NO_MFMA = 4u,     /* matrix-vector kernels and vector attention at every batch size (no MFMA) */
  DEC_FLAG_CAPTURE_ALL = 8u, /* capture every batch bucket at the first step instead of lazily */
  DEC_FLAG_NO_ATTN_O = 16u   /* attention and the O projection as separate launches at batch 1 */
};

/* Bits of dec_get_info's path_flags: how the last call ran. */
enum {
  DEC_PATH_GRAPH = 1,           /* replayed a captured hipGraph (else eager launches) */
  DEC_PATH_MFMA_PRODUCTS = 2,   /* the matrix products ran on MFMA tiles (else matrix-vector kernels) */
  DEC_PATH_MFMA_ATTENTION = 4,  /* attention's arithmetic ran on MFMA */
  DEC_PATH_FOLDED_NORM = 8,     /* RMSNorm folded into the MFMA products (no norm kernels) */
  DEC_PATH_UNFUSED = 16,        /* the unfused plan (DEC_FLAG_UNFUSED) */
  DEC_PATH_ATTN_O = 32          /* attention and the O projection ran as one launch per layer */
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
  int32_t kv_dtype;     /* DEC_BF16 or DEC_FP8_E4M3                                   */
  int32_t block_size;   /* must be 16                                                 */
  int32_t num_blocks;   /* physical blocks in the KV pool                             */
  int32_t max_batch;    /* a batch bucket: 1, 2, 4, 8, 16, 24, ..., 64; calls take up
                           to max_batch rows (tokens), padded up to the next bucket;
                           it is also dec_prefill's chunk length                      */
  int32_t max_seq_len;  /* positions per sequence, <= 524288; block tables have
                           ceil(max_seq_len / 16) entries per sequence                */
  uint32_t flags;       /* DEC_FLAG_*                                                 */
} dec_config;

typedef struct dec_mat {
  const void* w;      /* device [rows][cols] bf16, E4M3 or int8 codes                  */
  const float* scale; /* device fp32 [rows] for one-byte storage; must be NULL for bf16 */
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

typedef struct dec_verify_args {
  int32_t n_seqs;              /* >= 1, with n_seqs * k <= max_batch                      */
  int32_t k;                   /* tokens per sequence, 1 .. 8                             */
  const int32_t* token_ids;    /* host [n_seqs][k], each in [0, vocab)                   */
  const int32_t* seq_lens;     /* host [n_seqs]: tokens already cached = position of the
                                  sequence's first token; seq_len + k <= max_seq_len     */
  const int32_t* block_tables; /* host [n_seqs][ceil(max_seq_len / 16)]; entries
                                  0 .. (seq_len + k - 1) / 16 in [0, num_blocks)          */
} dec_verify_args;

typedef struct dec_prefill_args {
  int32_t n_tokens;            /* >= 1 prompt tokens                                     */
  const int32_t* token_ids;    /* host [n_tokens], each in [0, vocab)                    */
  int32_t start_pos;           /* tokens already cached (0 for a new sequence)           */
  const int32_t* block_table;  /* host [ceil(max_seq_len / 16)]; entries
                                  0 .. (start_pos + n_tokens - 1) / 16 in [0, num_blocks) */
} dec_prefill_args;

typedef struct dec_info {
  int32_t kernels_per_step;  /* kernels one plan of the last call launched (graph nodes when replayed) */
  int32_t bucket;            /* padded rows of the last plan                              */
  int32_t attn_splits;       /* context splits per (sequence, KV head) in the last plan   */
  int32_t used_mfma;         /* 1 if the last plan ran the products on MFMA tiles         */
  int32_t used_graph;        /* 1 if the last plan replayed a captured graph              */
  int32_t graphs_captured;   /* (bucket, plan) pairs with a live captured graph           */
  uint32_t flags;            /* current DEC_FLAG_* set                                    */
  int32_t rows;              /* tokens the last call processed                            */
  int32_t launches;          /* plans the last call ran (dec_prefill: one per chunk)      */
} dec_info;

/* Bytes of device workspace a context with this config needs (0 on an invalid
 * config; see dec_last_error).  Pure host computation. */
size_t dec_workspace_bytes(const dec_config* cfg);

/* Create a context: the engine-side state of the decode loop -- static device
 * buffers the per-step inputs are copied into, pinned host staging, and the
 * per-batch-bucket graphs captured later ("Kernels, Fusion & CUDA Graphs", Fix 2:
 * CUDA graphs; "The serving engine's kernel stack").  hip_stream: the hipStream_t
 * all device work goes on (NULL = the default stream; graphs are captured on a
 * private stream and replayed on this one).  kv_pool: device pool laid out as
 * above (caller-owned).  workspace: device buffer of at least
 * dec_workspace_bytes(cfg) bytes, 256-byte aligned (caller-owned).  logits: device
 * fp32 [max_batch][vocab] (caller-owned); rows [0, n) hold the last call's logits.
 * The library keeps the pointers and never frees them; the context must not
 * outlive them.  On success *out holds the context; on failure *out is NULL. */
int dec_create(const dec_config* cfg, void* hip_stream, void* kv_pool, void* workspace,
               size_t workspace_bytes, float* logits, dec_ctx** out);

/* Record weight pointers: the stored model whose every matrix one step streams
 * once ("GPU Inference Internals", Roofline: Why Decode Is Memory-Bound; one-byte
 * formats with per-channel scales dequantized inside the product kernels:
 * kernel-fusion architecture study, section 11).  The arrays in `w` are copied;
 * the device memory they point to is not, and must outlive the context.  May be
 * called again; any captured graphs are dropped.  DEC_E_INVALID for a NULL or
 * misaligned pointer, or a scale present (bf16) or missing (one-byte) where the
 * format says otherwise. */
int dec_load_weights(dec_ctx* ctx, const dec_weights* w);

/* Enqueue one decode step on the context's stream and return without waiting:
 * copy the batch's ids, positions and block tables into the static buffers, then
 * replay the graph of the batch's bucket, padded rows being inert ("Kernels,
 * Fusion & CUDA Graphs", Fix 2: CUDA graphs and The serving engine's kernel stack).
 * The host arrays are copied before the call returns.  After the stream reaches
 * the end of the step, logits rows [0, n_seqs) are valid and every live sequence's
 * K and V of its new token are in the pool (at position seq_len).  The caller then
 * advances seq_lens and extends block tables.  DEC_E_CAPACITY for n_seqs above
 * max_batch, a position at or above max_seq_len or a block id outside the pool. */
int dec_step(dec_ctx* ctx, const dec_step_args* args);

/* The verification step of speculative decoding: for each sequence s, k proposed
 * tokens at positions seq_lens[s] .. seq_lens[s] + k - 1 run through the model in
 * one pass, each weight read once for all n_seqs * k tokens, each token attending
 * causally to the cache and to the tokens before it ("GPU Inference Internals",
 * Roofline: Why Decode Is Memory-Bound, the speculative-decoding paragraph).
 * Enqueued like dec_step; afterwards logits row s * k + j holds the logits after
 * token j of sequence s (the distribution of the token at position seq_lens[s] +
 * j + 1), and the pool holds the K/V of all k tokens.  Tokens the caller rejects
 * are simply overwritten by later steps at the same positions. */
int dec_verify(dec_ctx* ctx, const dec_verify_args* args);

/* Chunked prefill of one sequence's prompt into the paged cache: the prompt runs
 * through the model max_batch tokens at a time (each chunk one plan, weights read
 * once per chunk; tokens attend causally to the cache and to the chunk's earlier
 * tokens), writing the K/V of every position start_pos .. start_pos + n_tokens - 1
 * ("GPU Inference Internals", Roofline: Why Decode Is Memory-Bound, the Prefill
 * paragraph; kernel-fusion architecture study, sections 10 and 14: prefill and
 * chunked prefill).  Only the last chunk runs the LM head: afterwards logits row
 * *logits_row holds the logits after the prompt's last token (the distribution of
 * the first generated token).  Enqueued on the context's stream; returns after
 * enqueueing every chunk. */
int dec_prefill(dec_ctx* ctx, const dec_prefill_args* args, int32_t* logits_row);

/* Change DEC_FLAG_EAGER / DEC_FLAG_UNFUSED / DEC_FLAG_NO_MFMA / DEC_FLAG_NO_ATTN_O
 * between steps (captured graphs of the other mode are kept). */
int dec_set_flags(dec_ctx* ctx, uint32_t flags);

/* Wait for the context's stream, then report whether every device-side wait of the
 * calls so far ended normally.  At batch 1, attention and the O projection run as one
 * launch (DEC_PATH_ATTN_O; "Kernels, Fusion & CUDA Graphs", Fix 1, the fused-kernel
 * table) whose O work groups poll attention's output until every element is written; that wait
 * is bounded, and one that gives up sets a device flag instead of hanging: the launch
 * ends with wrong values.  Returns DEC_OK, or DEC_E_HIP when a wait gave up (the
 * context is then failed: destroy it) or the stream reported an error. */
int dec_check(dec_ctx* ctx);

/* Polls a device-side wait makes before it gives up (default 32768, each about a
 * memory round trip: tens of milliseconds; 0 gives up at once).  For exercising the
 * failure path of dec_check; captured graphs are dropped (they hold the limit).
 * DEC_E_INVALID for a NULL ctx or a negative limit. */
int dec_set_wait_limit(dec_ctx* ctx, int32_t polls);

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
 * row s (the first one on ties; NaN never wins), for the rows with logits of the last
 * call, enqueued on the context's stream.  token_ids: device memory, int32 [rows],
 * 4-byte aligned, owned by the caller.  The sampling kernel that turns the logits into
 * token ids on the GPU, so that only the ids need to be copied back ("Kernels, Fusion &
 * CUDA Graphs", Fix 1 table: sampling; "The serving engine's kernel stack").  Needs a
 * previous call with logits (DEC_E_STATE otherwise); DEC_E_INVALID for a NULL or
 * misaligned token_ids. */
int dec_sample_greedy(dec_ctx* ctx, int32_t* token_ids);

/* Top-k / top-p sampling after the last step, enqueued on the context's stream: for each
 * row s with logits, the candidates are its top_k largest logits (the lower index first
 * on equal logits; NaN ranks as -inf), weighted exp((z - z_max) / temperature) in that
 * order; the nucleus is the shortest prefix of them whose weight reaches top_p of the
 * candidates' total; token_ids[s] = the first nucleus candidate whose running weight
 * exceeds uniforms[s] times the nucleus weight.  The random draws are inputs: uniforms,
 * device float32 [rows] in [0, 1), 4-byte aligned, owned by the caller; token_ids:
 * device int32 [rows], 4-byte aligned, owned by the caller.  The sampling step after the
 * LM head, on the GPU ("Kernels, Fusion & CUDA Graphs", Fix 1 table: sampling; "The
 * serving engine's kernel stack").  1 <= top_k <= 64, temperature > 0, 0 < top_p <= 1
 * (DEC_E_INVALID otherwise, and for NULL or misaligned pointers); needs a previous call
 * with logits (DEC_E_STATE otherwise).  top_k = 1 is greedy sampling. */
int dec_sample(dec_ctx* ctx, const float* uniforms, float temperature, int32_t top_k, float top_p,
               int32_t* token_ids);

/* How the last call ran: the kernels one plan launched -- the launch count the
 * pages' launch-tax model multiplies by the per-launch cost ("CUDA graphs & kernel
 * fusion", Direct answer; "Kernels, Fusion & CUDA Graphs", When the CPU becomes
 * the bottleneck) -- and DEC_PATH_* bits.  Both are 0 before the first call.
 * DEC_E_INVALID for a NULL argument. */
int dec_get_info(const dec_ctx* ctx, int32_t* kernels_per_step, int32_t* path_flags);

/* The same, and more, as a struct (bucket, splits, graphs, rows, launches). */
int dec_get_step_info(const dec_ctx* ctx, dec_info* out);

/* Wait for the context's stream, release graphs and host staging, free ctx.  The
 * caller's buffers are not freed.  NULL is accepted (DEC_OK). */
int dec_destroy(dec_ctx* ctx);

/* Message of the last failing call on this thread ("" if none). */
const char* dec_last_error(void);

/* ---------------------------------------------------------------- attention alone */

/* The attention step of decode as a call of its own (the same kernels as dec_step's):
 * each query row attends to positions 0 .. seq_lens[r] of its sequence's paged cache,
 * exact softmax attention computed block by block with a running max and sum, the
 * context split over work groups and the splits' partials combined by the last to
 * finish ("GPU Inference Internals", Kernels: FlashAttention and the Memory
 * Hierarchy; the KV read the batch does not amortize: Batching Economics). */
#define DEC_ATTN_MAX_ROWS 64

typedef struct dec_attn_desc {
  int32_t n_rows;             /* query rows, 1 .. DEC_ATTN_MAX_ROWS                      */
  int32_t n_q_heads;          /* multiple of n_kv_heads, at most 8 per KV head            */
  int32_t n_kv_heads;
  int32_t d_head;             /* 64 or 128                                               */
  int32_t kv_dtype;           /* DEC_BF16 or DEC_FP8_E4M3                                */
  int32_t n_layers;           /* layers in the pool                                      */
  int32_t layer;              /* the layer whose K/V are read, 0 .. n_layers - 1          */
  int32_t num_blocks;         /* physical blocks in the pool                             */
  int32_t max_blocks_per_seq; /* block-table row length, 1 .. 32768                      */
} dec_attn_desc;

/* Workspace bytes dec_attention needs for this descriptor (0 if it is invalid). */
size_t dec_attention_workspace_bytes(const dec_attn_desc* desc);

/* Enqueue attention on hip_stream (NULL = the default stream).  All pointers are device
 * memory owned by the caller:
 *   q            fp32 [n_rows][n_q_heads][d_head], RoPE already applied (16-byte aligned)
 *   kv_pool      the pool in the layout above, kv_dtype elements (16-byte aligned)
 *   seq_lens     int32 [n_rows]: row r attends to positions 0 .. seq_lens[r] (a negative
 *                value: no positions, the row's output is 0)
 *   block_tables int32 [n_rows][max_blocks_per_seq]
 *   o            bf16 [n_rows][n_q_heads * d_head] out (16-byte aligned)
 *   workspace    at least dec_attention_workspace_bytes(desc) bytes, 256-byte aligned
 * Query head j reads KV head j / (n_q_heads / n_kv_heads); scale 1 / sqrt(d_head).
 * Device metadata is not read on the host: positions are clamped below
 * max_blocks_per_seq * 16 and block ids into [0, num_blocks), so any metadata keeps the
 * reads inside the table and the pool (wrong metadata gives wrong results, no fault).
 * Calls that share a workspace on one stream run one after another; calls on two
 * streams need two workspaces.  DEC_E_INVALID / DEC_E_UNSUPPORTED for a bad descriptor,
 * a NULL or misaligned pointer or a small workspace. */
int dec_attention(const dec_attn_desc* desc, const float* q, const void* kv_pool, const int32_t* seq_lens,
                  const int32_t* block_tables, uint16_t* o, void* workspace, size_t workspace_bytes,
                  void* hip_stream);

/* dec_attention for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same kernels and
 * arguments without the workspace, which comes from a static scratch area of the
 * library -- DEC_ATTN_NOALLOC_SCRATCH_BYTES per GPU, held until the process ends.  The
 * call allocates nothing (its first call on a GPU looks up that GPU's scratch address);
 * it clears the split counters it uses with a kernel on hip_stream.  Shapes whose
 * workspace (dec_attention_workspace_bytes) exceeds the scratch are refused with
 * DEC_E_CAPACITY.  Calls on one GPU share its scratch: calls that can overlap (other
 * streams, other threads) race and must be serialized by the caller. */
#define DEC_ATTN_NOALLOC_SCRATCH_BYTES (8u << 20)
int dec_attention_noalloc(const dec_attn_desc* desc, const float* q, const void* kv_pool,
                          const int32_t* seq_lens, const int32_t* block_tables, uint16_t* o,
                          void* hip_stream);

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
