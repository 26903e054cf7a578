// Host runtime behind include/dec.h: validation, workspace layout, pinned staging
// of the per-step inputs, the kernel plan of one step, and one captured hipGraph
// per batch-size bucket.
//
// The engine step the pages describe has the CPU prepare the batch, block tables
// and metadata, copy them into static device buffers, and replay a graph captured
// once per batch size, padding the live batch up to the nearest captured size
// (ladder 1, 2, 4, then every 8); eager launches stay available for debugging and
// measurement ("Kernels, Fusion & CUDA Graphs", Fix 2: CUDA graphs and The serving
// engine's kernel stack; "CUDA graphs & kernel fusion", Direct answer and Deep
// dive).  Everything that varies per step is read by the kernels from device
// buffers, so one graph per bucket serves every step.
//
// A plan runs over rows.  A row is one token of one sequence: its id, its 0-based
// position and its sequence's block table.  A decode step has one row per sequence;
// the k-token verify step has k rows per sequence at consecutive positions; a prefill
// chunk has one row per prompt token.  The QKV kernel writes the K/V of every row
// before the attention kernel starts, so a row at position p attends to the rows of
// its own sequence at positions below p in the same launch: the causal mask of a
// multi-token step comes from the per-row positions alone.

#include <hip/hip_runtime.h>
#include <rocprofiler-sdk-roctx/roctx.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "dec.h"
#include "kernels.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

constexpr int LADDER[] = {1, 2, 4, 8, 16, 24, 32, 40, 48, 56, 64};
constexpr int N_BUCKETS = sizeof(LADDER) / sizeof(LADDER[0]);
constexpr uint32_t KNOWN_FLAGS =
    DEC_FLAG_EAGER | DEC_FLAG_UNFUSED | DEC_FLAG_NO_MFMA | DEC_FLAG_CAPTURE_ALL | DEC_FLAG_NO_ATTN_O;
// Plans: the flags that change the kernels (UNFUSED, NO_MFMA, NO_ATTN_O) and whether the
// LM head runs (prefill chunks before the last skip it).
constexpr int MODE_SKIP_LM = 4;
constexpr int MODE_NO_ATTN_O = 8;
constexpr int N_MODES = 16;
constexpr int MAX_VERIFY_K = 8;
// Polls before a fused attention + O launch's wait gives up (each poll is a memory round
// trip of about a microsecond plus a short sleep: tens of milliseconds, against
// microseconds for the attention it waits for).
constexpr int ATTN_O_SPIN = 1 << 15;

int mode_of(uint32_t flags, bool skip_lm) {
  return ((flags & DEC_FLAG_UNFUSED) ? 1 : 0) | ((flags & DEC_FLAG_NO_MFMA) ? 2 : 0) | (skip_lm ? MODE_SKIP_LM : 0) |
         ((flags & DEC_FLAG_NO_ATTN_O) ? MODE_NO_ATTN_O : 0);
}

int bucket_index(int n) {
  for (int i = 0; i < N_BUCKETS; ++i)
    if (LADDER[i] >= n) return i;
  return -1;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int blocks_per_seq(const dec_config& c) { return (c.max_seq_len + 15) / 16; }

dec::AttnShape attn_shape(const dec_config& c) {
  return dec::AttnShape{c.n_q_heads, c.n_kv_heads, c.d_head, blocks_per_seq(c)};
}

struct Layout {
  size_t ids, lens, bt, static_bytes;  // static region: ids | lens | block tables
  size_t h, x, xl, q, part_o, part_ml, o, a, rope;  // xl: the QKV input's second bf16 part
  size_t uf;                           // unfused step: fp32 product rows [MB][max(N)]
  size_t us;                           // unfused step: attention scores [MB][Hq][max_seq_len]
  size_t attn_cnt;                     // attention split arrival counters
  size_t attn_o_buf, attn_o_abort;     // fused attention + O launches: o of even and odd layers; abort flag
  size_t ssq;                          // folded RMSNorm: row-block sums of squares
  size_t gpart, gcnt;                  // MFMA products split over K: partial tiles, row-block counters
  size_t gpart_floats, gcnt_n;
  size_t total;
};

Layout layout_of(const dec_config& c) {
  Layout L{};
  const size_t MB = (size_t)c.max_batch;
  const size_t bps = (size_t)blocks_per_seq(c);
  size_t off = 0;
  L.ids = off;
  off += MB * 4;
  L.lens = off;
  off += MB * 4;
  L.bt = off;
  off += MB * bps * 4;
  L.static_bytes = off;
  off = align256(off);
  L.h = off;
  off = align256(off + MB * c.d_model * 4);
  L.x = off;
  off = align256(off + MB * c.d_model * 2);
  L.xl = off;
  off = align256(off + MB * c.d_model * 2);
  L.q = off;
  off = align256(off + MB * c.n_q_heads * c.d_head * 4);
  size_t rows_split = 0;  // max over buckets of Bp * n_split
  for (int i = 0; i < N_BUCKETS && LADDER[i] <= c.max_batch; ++i) {
    const size_t r = (size_t)LADDER[i] * dec::attn_splits(attn_shape(c), LADDER[i]);
    if (r > rows_split) rows_split = r;
  }
  L.part_o = off;
  off = align256(off + rows_split * c.n_q_heads * c.d_head * 4);
  L.part_ml = off;
  off = align256(off + rows_split * c.n_q_heads * 2 * 4);
  L.o = off;
  off = align256(off + MB * c.n_q_heads * c.d_head * 2);
  L.a = off;
  off = align256(off + MB * c.d_ff * 2);
  L.rope = off;
  off = align256(off + (size_t)c.max_seq_len * (c.d_head / 2) * 8);
  L.uf = off;  // largest product row: QKV, gate+up or d_model
  {
    size_t n = (size_t)(c.n_q_heads + 2 * c.n_kv_heads) * c.d_head;
    if ((size_t)2 * c.d_ff > n) n = (size_t)2 * c.d_ff;
    if ((size_t)c.d_model > n) n = c.d_model;
    off = align256(off + MB * n * 4);
  }
  L.us = off;
  off = align256(off + MB * c.n_q_heads * (size_t)c.max_seq_len * 4);
  // MFMA products: the largest partial-tile buffer and row-block count over the step's
  // matrices (gate+up also as one plain matrix, as the unfused step runs it) and the
  // buckets (every bucket, so that the size does not depend on which run on MFMA)
  size_t part_floats = 0, n_rb = 0;
  for (int i = 0; i < N_BUCKETS && LADDER[i] <= c.max_batch; ++i) {
    const int Bp = LADDER[i];
    const int qkv_rows = (c.n_q_heads + 2 * c.n_kv_heads) * c.d_head;
    const int shapes[6][3] = {{qkv_rows, 1, c.d_model}, {c.d_model, 1, c.n_q_heads * c.d_head},
                              {c.d_ff, 2, c.d_model},   {2 * c.d_ff, 1, c.d_model},
                              {c.d_model, 1, c.d_ff},   {c.vocab, 1, c.d_model}};
    for (const auto& sh : shapes) {
      const dec::GemmPlan gp = dec::gemm_plan(sh[0], sh[1], sh[2], Bp, c.weight_dtype != DEC_BF16);
      if (gp.part_floats > part_floats) part_floats = gp.part_floats;
      if (gp.ks > 1 && (size_t)gp.n_rb > n_rb) n_rb = gp.n_rb;
    }
  }
  L.gpart = off;
  L.gpart_floats = part_floats;
  L.gcnt_n = n_rb;
  off = align256(off + part_floats * 4);
  L.attn_cnt = off;
  off = align256(off + MB * c.n_kv_heads * 4);
  L.attn_o_buf = off;  // two buffers of Hq d_head bf16 (one sequence)
  off = align256(off + 2 * align256((size_t)c.n_q_heads * c.d_head * 2));
  L.attn_o_abort = off;
  off = align256(off + 4);
  L.ssq = off;
  off = align256(off + (size_t)dec::GEMM_SSQ_MAX * dec::GEMM_SSQ_STRIDE * 4);
  L.gcnt = off;
  off = align256(off + n_rb * dec::COUNTER_STRIDE * 4);
  L.total = off;
  return L;
}

int validate_config(const dec_config* c) {
  if (!c) return fail(DEC_E_INVALID, "config is NULL");
  if (c->n_layers < 0) return fail(DEC_E_INVALID, "n_layers must be >= 0 (got %d)", c->n_layers);
  if (c->d_model <= 0 || c->d_model % 16) return fail(DEC_E_INVALID, "d_model must be a positive multiple of 16 (got %d)", c->d_model);
  if (c->d_ff <= 0 || c->d_ff % 16) return fail(DEC_E_INVALID, "d_ff must be a positive multiple of 16 (got %d)", c->d_ff);
  if (c->n_kv_heads <= 0 || c->n_q_heads <= 0 || c->n_q_heads % c->n_kv_heads)
    return fail(DEC_E_INVALID, "n_q_heads (%d) must be a positive multiple of n_kv_heads (%d)", c->n_q_heads, c->n_kv_heads);
  if (c->n_q_heads / c->n_kv_heads > 8)
    return fail(DEC_E_UNSUPPORTED, "query heads per KV head must be <= 8 (got %d)", c->n_q_heads / c->n_kv_heads);
  if (c->d_head != 64 && c->d_head != 128) return fail(DEC_E_UNSUPPORTED, "d_head must be 64 or 128 (got %d)", c->d_head);
  if (c->vocab <= 0 || c->vocab % 2) return fail(DEC_E_INVALID, "vocab must be positive and even (got %d)", c->vocab);
  if (!(c->rms_eps > 0.f) || !std::isfinite(c->rms_eps)) return fail(DEC_E_INVALID, "rms_eps must be a positive finite number");
  if (!(c->rope_theta > 1.f) || !std::isfinite(c->rope_theta)) return fail(DEC_E_INVALID, "rope_theta must be finite and > 1");
  if ((c->weight_dtype != DEC_BF16 && c->weight_dtype != DEC_FP8_E4M3 && c->weight_dtype != DEC_INT8) ||
      (c->kv_dtype != DEC_BF16 && c->kv_dtype != DEC_FP8_E4M3))
    return fail(DEC_E_INVALID, "weight_dtype must be DEC_BF16, DEC_FP8_E4M3 or DEC_INT8; kv_dtype DEC_BF16 or DEC_FP8_E4M3");
  if (c->block_size != 16) return fail(DEC_E_UNSUPPORTED, "block_size must be 16 (got %d)", c->block_size);
  if (c->num_blocks <= 0) return fail(DEC_E_INVALID, "num_blocks must be positive (got %d)", c->num_blocks);
  if (bucket_index(c->max_batch) < 0 || LADDER[bucket_index(c->max_batch)] != c->max_batch)
    return fail(DEC_E_INVALID, "max_batch must be one of 1, 2, 4, 8, 16, 24, ..., 64 (got %d)", c->max_batch);
  if (c->max_seq_len <= 0) return fail(DEC_E_INVALID, "max_seq_len must be positive (got %d)", c->max_seq_len);
  // attention keeps a wave's block ids in its 64 lanes: at most 64 splits x 8 waves x 64
  // blocks of 16 positions
  if (c->max_seq_len > dec::ATTN_MAX_SPLIT * dec::ATTN_WAVES * 64 * 16)
    return fail(DEC_E_UNSUPPORTED, "max_seq_len must be <= %d (got %d)", dec::ATTN_MAX_SPLIT * dec::ATTN_WAVES * 64 * 16,
                c->max_seq_len);
  if (c->flags & ~KNOWN_FLAGS) return fail(DEC_E_INVALID, "unknown flag bits 0x%x", c->flags & ~KNOWN_FLAGS);
  return DEC_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

dec::WFmt wfmt_of(int weight_dtype) {
  return weight_dtype == DEC_FP8_E4M3 ? dec::W_E4M3 : weight_dtype == DEC_INT8 ? dec::W_I8 : dec::W_BF16;
}

}  // namespace

namespace dec {
void set_last_error(const char* msg) { g_err = msg; }
}  // namespace dec

struct dec_ctx {
  dec_config cfg{};
  hipStream_t stream = nullptr;
  hipStream_t cap_stream = nullptr;
  int device = 0;
  void* pool = nullptr;
  uint8_t* ws = nullptr;
  float* logits = nullptr;
  Layout L{};
  bool loaded = false;
  bool failed = false;
  int last_n = 0;  // rows with logits after the last call (0: none yet)
  int wait_limit = ATTN_O_SPIN;  // polls of a device-side wait before it gives up
  // weights
  dec_mat embed{}, lm{};
  std::vector<dec_mat> qkv, o, gu, down;
  const float* attn_norm = nullptr;
  const float* mlp_norm = nullptr;
  const float* final_norm = nullptr;
  // host staging of the per-step inputs (double-buffered, pinned)
  uint8_t* pinned[2] = {nullptr, nullptr};
  hipEvent_t slot_ev[2] = {nullptr, nullptr};
  bool slot_pending[2] = {false, false};
  int slot = 0;
  // graphs per (bucket, plan)
  hipGraphExec_t graphs[N_BUCKETS][N_MODES] = {};
  dec_info info{};
};

namespace {

template <typename T>
T* ws_ptr(dec_ctx* c, size_t off) {
  return reinterpret_cast<T*>(c->ws + off);
}

int hip_fail(dec_ctx* c, hipError_t e, const char* what) {
  if (c) c->failed = true;
  return fail(DEC_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define HIPCHK(ctx, call, what)                       \
  do {                                                \
    hipError_t e_ = (call);                           \
    if (e_ != hipSuccess) return hip_fail(ctx, e_, what); \
  } while (0)

// Buckets from 4 rows up run the products on the matrix cores (unless
// DEC_FLAG_NO_MFMA); smaller ones run the matrix-vector kernels.  Measured on the 8B and
// 32B shapes: the vector kernels' activation reads from LDS (Bp per weight vector) and,
// for one-byte codes, the widening of every weight once per batch row make them slower
// than the MFMA tiles from 4 rows on (8B bf16, batch 4: 3.73 against 4.09 ms per step);
// the MFMA tiles pad the batch to 16 columns at no extra HBM traffic.
constexpr int MFMA_MIN_BATCH_BF16 = 4;
constexpr int MFMA_MIN_BATCH_BYTE = 4;
bool use_mfma(const dec_config& g, int Bp) {
  return !(g.flags & DEC_FLAG_NO_MFMA) &&
         Bp >= (g.weight_dtype != DEC_BF16 ? MFMA_MIN_BATCH_BYTE : MFMA_MIN_BATCH_BF16);
}

// Parameters of the matrix kernel `which` (dec_matrix) of layer l for a padded batch Bp.
dec::MatmulParams matmul_params(dec_ctx* c, int which, int l, int Bp, int* epi) {
  const dec_config& g = c->cfg;
  const int d = g.d_model, dh = g.d_head, Hq = g.n_q_heads, Hkv = g.n_kv_heads;
  dec::MatmulParams p{};
  p.Bp = Bp;
  p.seq_lens = ws_ptr<int32_t>(c, c->L.lens);
  p.bt = ws_ptr<int32_t>(c, c->L.bt);
  p.rope = ws_ptr<float2>(c, c->L.rope);
  p.pool = c->pool;
  p.q = ws_ptr<float>(c, c->L.q);
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.dh = dh;
  p.num_blocks = g.num_blocks;
  p.bps = blocks_per_seq(g);
  p.d_ff = g.d_ff;
  p.layer = l;
  p.gpart = ws_ptr<float>(c, c->L.gpart);
  p.gcnt = ws_ptr<unsigned>(c, c->L.gcnt);
  p.gpart_floats = c->L.gpart_floats;
  p.gcnt_n = (int)c->L.gcnt_n;
  uint16_t* x = ws_ptr<uint16_t>(c, c->L.x);
  float* h = ws_ptr<float>(c, c->L.h);
  switch (which) {
    case DEC_MAT_QKV:  // [q; k; v] = W_qkv x, RoPE, K/V -> cache (x: fp16, or x + xl)
      p.W = c->qkv[l].w;
      p.scale = c->qkv[l].scale;
      p.N = (Hq + 2 * Hkv) * dh;
      p.K = d;
      p.x = x;
      if (use_mfma(g, Bp)) p.x_f16 = 1;
      else p.xl = ws_ptr<uint16_t>(c, c->L.xl);
      p.ldx = d;
      *epi = dec::EPI_QKV;
      break;
    case DEC_MAT_O:  // h += W_o o
      p.W = c->o[l].w;
      p.scale = c->o[l].scale;
      p.N = d;
      p.K = Hq * dh;
      p.x = ws_ptr<uint16_t>(c, c->L.o);
      p.ldx = Hq * dh;
      p.out = h;
      p.ldo = d;
      *epi = dec::EPI_RESID;
      break;
    case DEC_MAT_GATE_UP:  // a = silu(W_gate x) * (W_up x)
      p.W = c->gu[l].w;
      p.scale = c->gu[l].scale;
      p.N = 2 * g.d_ff;
      p.K = d;
      p.x = x;
      p.ldx = d;
      p.act = ws_ptr<uint16_t>(c, c->L.a);
      p.ldact = g.d_ff;
      *epi = dec::EPI_SILU;
      break;
    case DEC_MAT_DOWN:  // h += W_down a
      p.W = c->down[l].w;
      p.scale = c->down[l].scale;
      p.N = d;
      p.K = g.d_ff;
      p.x = ws_ptr<uint16_t>(c, c->L.a);
      p.ldx = g.d_ff;
      p.out = h;
      p.ldo = d;
      *epi = dec::EPI_RESID;
      break;
    default:  // logits = W_lm x
      p.W = c->lm.w;
      p.scale = c->lm.scale;
      p.N = g.vocab;
      p.K = d;
      p.x = x;
      p.ldx = d;
      p.out = c->logits;
      p.ldo = g.vocab;
      *epi = dec::EPI_LOGITS;
      break;
  }
  return p;
}

// Row blocks of a residual product on the MFMA tiles -- O (K = Hq dh) or down (K = d_ff)
// -- : the number of row-block sums of squares it writes for the folded RMSNorm that
// follows it.
int residual_row_blocks(const dec_config& g, int Bp, int which) {
  const int K = which == DEC_MAT_O ? g.n_q_heads * g.d_head : g.d_ff;
  return dec::gemm_plan(g.d_model, 1, K, Bp, g.weight_dtype != DEC_BF16).n_rb;
}

// The MFMA plan folds the two RMSNorms of a layer and the final one into the products:
// O and down write the next norm's input times its gain (x) and their row blocks' sums of
// squares of h; QKV (past layer 0, whose x the embedding kernel normalizes), gate+up and
// the LM head scale their sums by 1 / rms.  Up to GEMM_SSQ_MAX row blocks; not in the
// unfused step, which runs the norms as kernels of their own.
bool fold_norm(const dec_config& g, int Bp) {
  return use_mfma(g, Bp) && !(g.flags & DEC_FLAG_UNFUSED) &&
         residual_row_blocks(g, Bp, DEC_MAT_O) <= dec::GEMM_SSQ_MAX &&
         residual_row_blocks(g, Bp, DEC_MAT_DOWN) <= dec::GEMM_SSQ_MAX;
}

void set_fold_norm(dec_ctx* c, int which, int l, int Bp, dec::MatmulParams& p) {
  const dec_config& g = c->cfg;
  const int d = g.d_model;
  float* ssq = ws_ptr<float>(c, c->L.ssq);
  p.eps = g.rms_eps;
  if (which == DEC_MAT_O || which == DEC_MAT_DOWN) {
    p.xout = ws_ptr<uint16_t>(c, c->L.x);
    // down before the next layer's QKV (on the matrix cores, as all products of a folded
    // plan) writes its input as fp16
    if (which == DEC_MAT_DOWN && l + 1 < g.n_layers) p.xout_f16 = 1;
    p.ldxo = d;
    p.xg = which == DEC_MAT_O ? c->mlp_norm + (size_t)l * d
           : l + 1 < g.n_layers ? c->attn_norm + (size_t)(l + 1) * d : c->final_norm;
    p.ssq_out = ssq;
  } else if (which == DEC_MAT_GATE_UP || (which == DEC_MAT_QKV && l > 0) ||
             (which == DEC_MAT_LM_HEAD && g.n_layers > 0)) {
    // the sums of the residual product before it: O before gate+up, down before the
    // next layer's QKV and before the LM head
    p.ssq_in = ssq;
    p.ssq_n = residual_row_blocks(g, Bp, which == DEC_MAT_GATE_UP ? DEC_MAT_O : DEC_MAT_DOWN);
  }
}

// Attention's arithmetic on the matrix cores (k_attn_mfma) at every batch unless
// DEC_FLAG_NO_MFMA.  Measured, with q and P split into bf16 parts by the hardware
// conversion: as fast or faster than the vector form from one row (8B batch 1 2.82
// against 2.86 ms per step, 32B 6.38 against 6.50), as the vector form's per-position
// arithmetic sits on each wave's chain of blocks.
bool attn_mfma(const dec_config& g) { return !(g.flags & DEC_FLAG_NO_MFMA); }

int device_cus() {
  static int n_cu = 0;
  if (n_cu == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      v = 256;
    n_cu = v > 0 ? v : 256;
  }
  return n_cu;
}


// norm_gain: when set, the kernel computes x = RMSNorm(h) norm_gain itself (fused_norm)
hipError_t run_matmul(dec_ctx* c, int which, int l, int Bp, hipStream_t s, const float* norm_gain = nullptr) {
  const dec_config& g = c->cfg;
  int epi = 0;
  dec::MatmulParams p = matmul_params(c, which, l, Bp, &epi);
  if (norm_gain) {
    p.nh = ws_ptr<float>(c, c->L.h);
    p.ng = norm_gain;
    p.eps = g.rms_eps;
  }
  if (fold_norm(g, Bp)) set_fold_norm(c, which, l, Bp, p);
  return dec::launch_matmul(p, epi, wfmt_of(g.weight_dtype), g.kv_dtype == DEC_FP8_E4M3, use_mfma(g, Bp), s);
}

// Batches of <= 8 rows on the matrix-vector kernels normalize their own input in LDS
// ([Bp][d] bf16 in two parts for QKV must fit in 128 KB)
bool fused_norm(const dec_config& g, int Bp) {
  return !use_mfma(g, Bp) && Bp <= 8 && (size_t)Bp * g.d_model * 4 <= 128 * 1024;
}

// The fused attention + O launch's shape (attn_o.hip): rows of W_o per wave (0 where the
// two run as separate launches) and attention splits.  A single sequence on the
// matrix-vector kernels, MFMA attention, and O work groups that fit beside attention's.
dec::AttnOPlan attn_o_plan(const dec_config& g, int Bp) {
  if (Bp != 1 || g.n_layers == 0 || use_mfma(g, Bp) || !attn_mfma(g) || !fused_norm(g, Bp) ||
      (g.flags & (DEC_FLAG_UNFUSED | DEC_FLAG_NO_ATTN_O)))
    return dec::AttnOPlan{0, 0};
  return dec::attn_o_plan(attn_shape(g), Bp, g.d_model, wfmt_of(g.weight_dtype), device_cus());
}
int attn_o_rows(const dec_config& g, int Bp) { return attn_o_plan(g, Bp).rows; }

// The fused attention + O launch's attention output for layer l (buffers alternate by layer)
uint16_t* attn_o_buf(dec_ctx* c, int l) {
  const size_t n = align256((size_t)c->cfg.n_q_heads * c->cfg.d_head * 2);
  return reinterpret_cast<uint16_t*>(c->ws + c->L.attn_o_buf + (size_t)(l & 1) * n);
}

dec::AttnParams attn_params(dec_ctx* c, int Bp, int layer) {
  const dec_config& g = c->cfg;
  dec::AttnParams ap{};
  ap.q = ws_ptr<float>(c, c->L.q);
  ap.pool = c->pool;
  ap.seq_lens = ws_ptr<int32_t>(c, c->L.lens);
  ap.bt = ws_ptr<int32_t>(c, c->L.bt);
  ap.part_o = ws_ptr<float>(c, c->L.part_o);
  ap.part_ml = ws_ptr<float>(c, c->L.part_ml);
  ap.o = ws_ptr<uint16_t>(c, c->L.o);
  ap.cnt = ws_ptr<unsigned>(c, c->L.attn_cnt);
  ap.Bp = Bp;
  ap.Hq = g.n_q_heads;
  ap.Hkv = g.n_kv_heads;
  ap.dh = g.d_head;
  ap.num_blocks = g.num_blocks;
  ap.bps = blocks_per_seq(g);
  ap.n_split = dec::attn_splits(attn_shape(g), Bp);
  ap.mfma = attn_mfma(g) ? 1 : 0;
  ap.layer = layer;
  return ap;
}

// The unfused step (DEC_FLAG_UNFUSED, measurement only): RMSNorm kernels, the matrix
// kernels with a plain fp32 output, attention as scores -> softmax -> P V through HBM,
// and the elementwise work as kernels of its own.
hipError_t enqueue_unfused(dec_ctx* c, int Bp, bool skip_lm, hipStream_t s) {
  const dec_config& g = c->cfg;
  const dec::WFmt wq = wfmt_of(g.weight_dtype);
  const bool kvfp8 = g.kv_dtype == DEC_FP8_E4M3;
  const bool mfma = use_mfma(g, Bp);
  const int d = g.d_model;
  float* h = ws_ptr<float>(c, c->L.h);
  float* uf = ws_ptr<float>(c, c->L.uf);
  hipError_t e;
  dec::NormParams np{};
  np.h = h;
  np.h_out = h;
  np.x = ws_ptr<uint16_t>(c, c->L.x);
  np.d = d;
  np.Bp = Bp;
  np.eps = g.rms_eps;
  np.E = c->embed.w;
  np.E_scale = c->embed.scale;
  np.ids = ws_ptr<int32_t>(c, c->L.ids);
  np.gain = g.n_layers > 0 ? c->attn_norm : c->final_norm;
  // layer 0's QKV input: fp16 for the matrix cores, else two bf16 parts
  uint16_t* xl = ws_ptr<uint16_t>(c, c->L.xl);
  auto qkv_input = [&](bool on) {
    np.x_f16 = on && mfma;
    np.x_lo = on && !mfma ? xl : nullptr;
  };
  qkv_input(g.n_layers > 0);
  if ((e = dec::launch_embed_norm(np, wq, s)) != hipSuccess) return e;
  // the product of `which` with its rows written plainly to uf [Bp][N]
  auto plain = [&](int which, int l, dec::MatmulParams* keep) -> hipError_t {
    int epi = 0;
    dec::MatmulParams p = matmul_params(c, which, l, Bp, &epi);
    if (keep) *keep = p;
    p.out = uf;
    p.ldo = p.N;
    return dec::launch_matmul(p, dec::EPI_LOGITS, wq, kvfp8, mfma, s);
  };
  for (int l = 0; l < g.n_layers; ++l) {
    if (l > 0) {
      np.gain = c->attn_norm + (size_t)l * d;
      qkv_input(true);
      if ((e = dec::launch_rmsnorm(np, s)) != hipSuccess) return e;
    }
    dec::MatmulParams qp{};
    if ((e = plain(DEC_MAT_QKV, l, &qp)) != hipSuccess) return e;
    if ((e = dec::launch_rope_kv(qp, uf, kvfp8, s)) != hipSuccess) return e;
    dec::AttnParams ap = attn_params(c, Bp, l);
    if ((e = dec::launch_attention_unfused(ap, ws_ptr<float>(c, c->L.us), g.max_seq_len, kvfp8, s)) != hipSuccess)
      return e;
    if ((e = plain(DEC_MAT_O, l, nullptr)) != hipSuccess) return e;
    if ((e = dec::launch_add(h, uf, Bp * d, s)) != hipSuccess) return e;
    np.gain = c->mlp_norm + (size_t)l * d;
    qkv_input(false);
    if ((e = dec::launch_rmsnorm(np, s)) != hipSuccess) return e;
    if ((e = plain(DEC_MAT_GATE_UP, l, nullptr)) != hipSuccess) return e;
    if ((e = dec::launch_silu_mul(uf, g.d_ff, Bp, ws_ptr<uint16_t>(c, c->L.a), g.d_ff, s)) != hipSuccess) return e;
    if ((e = plain(DEC_MAT_DOWN, l, nullptr)) != hipSuccess) return e;
    if ((e = dec::launch_add(h, uf, Bp * d, s)) != hipSuccess) return e;
  }
  if (skip_lm) return hipSuccess;
  if (g.n_layers > 0) {
    np.gain = c->final_norm;
    qkv_input(false);
    if ((e = dec::launch_rmsnorm(np, s)) != hipSuccess) return e;
  }
  return run_matmul(c, DEC_MAT_LM_HEAD, 0, Bp, s);
}

// Enqueue the plan of one step for a padded batch of Bp rows on stream s (without the
// LM head when skip_lm).
hipError_t enqueue_step(dec_ctx* c, int Bp, bool skip_lm, hipStream_t s) {
  if (c->cfg.flags & DEC_FLAG_UNFUSED) return enqueue_unfused(c, Bp, skip_lm, s);
  const dec_config& g = c->cfg;
  const dec::WFmt wq = wfmt_of(g.weight_dtype);
  const bool kvfp8 = g.kv_dtype == DEC_FP8_E4M3;
  float* h = ws_ptr<float>(c, c->L.h);
  uint16_t* x = ws_ptr<uint16_t>(c, c->L.x);
  const int d = g.d_model;
  hipError_t e;

  dec::NormParams np{};
  np.h = h;
  np.h_out = h;
  np.x = x;
  np.d = d;
  np.Bp = Bp;
  np.eps = g.rms_eps;
  np.E = c->embed.w;
  np.E_scale = c->embed.scale;
  np.ids = ws_ptr<int32_t>(c, c->L.ids);
  np.gain = g.n_layers > 0 ? c->attn_norm : c->final_norm;
  // layer 0's QKV input: fp16 for the matrix cores, else two bf16 parts
  const bool mfma = use_mfma(g, Bp);
  uint16_t* xl = ws_ptr<uint16_t>(c, c->L.xl);
  auto qkv_input = [&](bool on) {
    np.x_f16 = on && mfma;
    np.x_lo = on && !mfma ? xl : nullptr;
  };
  qkv_input(g.n_layers > 0);
  // the fused attention + O launches: the first layer's attention output starts the
  // step marked as not yet written (each launch marks the next layer's)
  const dec::AttnOPlan ao = attn_o_plan(g, Bp);
  const int ao_rows = ao.rows;
  if (ao_rows > 0) {
    np.pend = reinterpret_cast<unsigned*>(attn_o_buf(c, 0));
    np.n_pend = g.n_q_heads * g.d_head / 2;
  }
  if ((e = dec::launch_embed_norm(np, wq, s)) != hipSuccess) return e;
  np.pend = nullptr;
  np.n_pend = 0;

  // no RMSNorm kernels: the matrix-vector kernels normalize their own input (fn), or the
  // MFMA products fold the norms
  const bool fn = fused_norm(g, Bp);
  const bool nk = !fn && !fold_norm(g, Bp);
  for (int l = 0; l < g.n_layers; ++l) {
    const float* an = c->attn_norm + (size_t)l * d;
    if (l > 0 && nk) {
      np.gain = an;
      qkv_input(true);
      if ((e = dec::launch_rmsnorm(np, s)) != hipSuccess) return e;
    }
    if ((e = run_matmul(c, DEC_MAT_QKV, l, Bp, s, fn ? an : nullptr)) != hipSuccess) return e;
    // attention over positions 0..p, then h += W_o o
    if (ao_rows > 0) {
      dec::AttnOParams P{};
      P.a = attn_params(c, Bp, l);
      P.a.n_split = ao.n_split;  // no more than attn_splits: the workspace holds the partials
      P.a.o = attn_o_buf(c, l);
      int epi = 0;
      P.m = matmul_params(c, DEC_MAT_O, l, Bp, &epi);
      P.m.x = P.a.o;
      P.next = attn_o_buf(c, l + 1);
      P.abort = ws_ptr<int>(c, c->L.attn_o_abort);
      P.spin = c->wait_limit;
      P.n_attn = P.a.n_split * P.a.Hkv * Bp;
      P.rows = ao_rows;
      if ((e = dec::launch_attn_o(P, wq, kvfp8, s)) != hipSuccess) return e;
    } else {
      if ((e = dec::launch_attention(attn_params(c, Bp, l), kvfp8, s)) != hipSuccess) return e;
      if ((e = run_matmul(c, DEC_MAT_O, l, Bp, s)) != hipSuccess) return e;
    }
    // x = RMSNorm(h) g_mlp
    const float* mn = c->mlp_norm + (size_t)l * d;
    if (nk) {
      np.gain = mn;
      qkv_input(false);
      if ((e = dec::launch_rmsnorm(np, s)) != hipSuccess) return e;
    }
    if ((e = run_matmul(c, DEC_MAT_GATE_UP, l, Bp, s, fn ? mn : nullptr)) != hipSuccess) return e;
    if ((e = run_matmul(c, DEC_MAT_DOWN, l, Bp, s)) != hipSuccess) return e;
  }
  if (skip_lm) return hipSuccess;
  if (g.n_layers > 0 && nk) {
    np.gain = c->final_norm;
    qkv_input(false);
    if ((e = dec::launch_rmsnorm(np, s)) != hipSuccess) return e;
  }
  if ((e = run_matmul(c, DEC_MAT_LM_HEAD, 0, Bp, s, fn ? c->final_norm : nullptr)) != hipSuccess) return e;
  return hipSuccess;
}

// Kernels one plan launches (graph nodes when replayed).
int kernels_of_plan(const dec_config& g, int Bp, bool skip_lm) {
  const bool mfma = use_mfma(g, Bp);
  const int slices = (!mfma && Bp > 8) ? Bp / 8 : 1;  // the matrix-vector kernels take 8 rows
  const int L = g.n_layers;
  if (g.flags & DEC_FLAG_UNFUSED) {
    // embedding; per layer two norms (one in layer 0), QKV, RoPE + KV write, scores,
    // softmax, P V, O, add, gate+up, SiLU x mul, down, add; final norm and LM head
    const int per_layer = 13 + 4 * (slices - 1);
    int n = 1 + per_layer * L - (L > 0 ? 1 : 0);
    if (!skip_lm) n += (L > 0 ? 1 : 0) + slices;
    return n;
  }
  // per layer: QKV, attention, O (one launch with attention at batch 1 where it fits),
  // gate+up, down, and two RMSNorm kernels unless the matrix-vector kernels fuse them or
  // the MFMA products fold them
  const bool norms = !fused_norm(g, Bp) && !fold_norm(g, Bp);
  const int per_layer = (attn_o_rows(g, Bp) > 0 ? 4 : 5) + (norms ? 2 : 0) + 4 * (slices - 1);
  int n = 1 + per_layer * L - (norms && L > 0 ? 1 : 0);
  if (!skip_lm) n += slices + (norms && L > 0 ? 1 : 0);
  return n;
}

void drop_graphs(dec_ctx* c) {
  for (auto& row : c->graphs)
    for (auto& ge : row)
      if (ge) {
        (void)hipGraphExecDestroy(ge);
        ge = nullptr;
      }
}

int capture(dec_ctx* c, int bi, int mode) {
  hipGraph_t graph = nullptr;
  HIPCHK(c, hipStreamBeginCapture(c->cap_stream, hipStreamCaptureModeThreadLocal), "hipStreamBeginCapture");
  hipError_t e = enqueue_step(c, LADDER[bi], (mode & MODE_SKIP_LM) != 0, c->cap_stream);
  hipError_t e2 = hipStreamEndCapture(c->cap_stream, &graph);
  if (e != hipSuccess) {
    if (graph) (void)hipGraphDestroy(graph);
    return hip_fail(c, e, "kernel launch during capture");
  }
  if (e2 != hipSuccess) return hip_fail(c, e2, "hipStreamEndCapture");
  hipGraphExec_t exec = nullptr;
  e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  (void)hipGraphDestroy(graph);
  if (e != hipSuccess) return hip_fail(c, e, "hipGraphInstantiate");
  c->graphs[bi][mode] = exec;
  return DEC_OK;
}

int check_mat(const dec_mat& m, bool scaled, const char* name, int layer) {
  if (!m.w) return fail(DEC_E_INVALID, "%s[%d].w is NULL", name, layer);
  if (!aligned16(m.w)) return fail(DEC_E_INVALID, "%s[%d].w is not 16-byte aligned", name, layer);
  if (scaled && !m.scale) return fail(DEC_E_INVALID, "%s[%d].scale is NULL for one-byte weights", name, layer);
  if (!scaled && m.scale) return fail(DEC_E_INVALID, "%s[%d].scale must be NULL for bf16 weights", name, layer);
  return DEC_OK;
}

// The checks every call that runs the plan makes before anything is enqueued.
int check_ready(dec_ctx* c) {
  if (c->failed) return fail(DEC_E_STATE, "context has failed; destroy it");
  if (!c->loaded) return fail(DEC_E_STATE, "no weights loaded (dec_load_weights)");
  return DEC_OK;
}

// Token id, positions [p0, p1] and the block-table entries they need, for one sequence.
int check_tokens(const dec_config& g, const char* what, int s, const int32_t* ids, int n_ids, int p0, int p1,
                 const int32_t* bt_row) {
  for (int j = 0; j < n_ids; ++j)
    if (ids[j] < 0 || ids[j] >= g.vocab)
      return fail(DEC_E_INVALID, "%s: token id %d of sequence %d is %d, outside [0, %d)", what, j, s, ids[j], g.vocab);
  if (p0 < 0) return fail(DEC_E_INVALID, "%s: seq_lens[%d] = %d is negative", what, s, p0);
  if (p1 >= g.max_seq_len)
    return fail(DEC_E_CAPACITY, "%s: sequence %d reaches position %d; positions must be < max_seq_len %d", what, s,
                p1, g.max_seq_len);
  for (int k = 0; k <= p1 / 16; ++k) {
    const int blk = bt_row[k];
    if (blk < 0 || blk >= g.num_blocks)
      return fail(DEC_E_CAPACITY, "%s: block_tables[%d][%d] = %d outside [0, %d)", what, s, k, blk, g.num_blocks);
  }
  return DEC_OK;
}

// Staging of `rows` rows padded to Bp: fill(ids, lens, bt) writes the live rows into the
// pinned slot, the padded rows get token 0 and position -1 (no cache write, no
// attention), and one copy moves the static region to the device.
template <typename Fill>
int stage(dec_ctx* c, int rows, int Bp, const Fill& fill) {
  const int bps = blocks_per_seq(c->cfg);
  const int s = c->slot;
  c->slot ^= 1;
  // wait until the copy that last used this slot has finished
  if (c->slot_pending[s]) HIPCHK(c, hipEventSynchronize(c->slot_ev[s]), "waiting for a staging slot");
  uint8_t* st = c->pinned[s];
  int32_t* ids = reinterpret_cast<int32_t*>(st + c->L.ids);
  int32_t* lens = reinterpret_cast<int32_t*>(st + c->L.lens);
  int32_t* bt = reinterpret_cast<int32_t*>(st + c->L.bt);
  fill(ids, lens, bt);
  for (int b = rows; b < Bp; ++b) {
    ids[b] = 0;
    lens[b] = -1;
    std::memset(bt + (size_t)b * bps, 0, (size_t)bps * 4);
  }
  HIPCHK(c, hipMemcpyAsync(c->ws, st, c->L.static_bytes, hipMemcpyHostToDevice, c->stream), "staging copy");
  HIPCHK(c, hipEventRecord(c->slot_ev[s], c->stream), "hipEventRecord");
  c->slot_pending[s] = true;
  return DEC_OK;
}

// Run the plan for Bp padded rows already staged: replay the bucket's graph (captured
// on first use) or launch eagerly.
int run_plan(dec_ctx* c, int Bp, bool skip_lm) {
  const dec_config& g = c->cfg;
  const int bi = bucket_index(Bp);
  const int mode = mode_of(g.flags, skip_lm);
  if (g.flags & DEC_FLAG_EAGER) {
    hipError_t e = enqueue_step(c, Bp, skip_lm, c->stream);
    if (e != hipSuccess) return hip_fail(c, e, "kernel launch");
    c->info.used_graph = 0;
  } else {
    if (g.flags & DEC_FLAG_CAPTURE_ALL) {
      for (int i = 0; i < N_BUCKETS && LADDER[i] <= g.max_batch; ++i)
        if (!c->graphs[i][mode]) {
          int rc = capture(c, i, mode);
          if (rc != DEC_OK) return rc;
        }
    }
    if (!c->graphs[bi][mode]) {
      int rc = capture(c, bi, mode);
      if (rc != DEC_OK) return rc;
    }
    HIPCHK(c, hipGraphLaunch(c->graphs[bi][mode], c->stream), "hipGraphLaunch");
    c->info.used_graph = 1;
  }
  int ncap = 0;
  for (auto& row : c->graphs)
    for (auto& ge : row) ncap += ge != nullptr;
  c->info.kernels_per_step = kernels_of_plan(g, Bp, skip_lm);
  c->info.bucket = Bp;
  const dec::AttnOPlan aop = attn_o_plan(g, Bp);
  c->info.attn_splits = aop.rows > 0 ? aop.n_split : dec::attn_splits(attn_shape(g), Bp);
  c->info.used_mfma = use_mfma(g, Bp) ? 1 : 0;
  c->info.graphs_captured = ncap;
  c->info.flags = g.flags;
  return DEC_OK;
}

}  // namespace

extern "C" {

const char* dec_last_error(void) { return g_err.c_str(); }

size_t dec_workspace_bytes(const dec_config* cfg) {
  if (validate_config(cfg) != DEC_OK) return 0;
  return layout_of(*cfg).total;
}

int dec_create(const dec_config* cfg, void* hip_stream, void* kv_pool, void* workspace, size_t workspace_bytes,
               float* logits, dec_ctx** out) {
  if (!out) return fail(DEC_E_INVALID, "out is NULL");
  *out = nullptr;
  int rc = validate_config(cfg);
  if (rc != DEC_OK) return rc;
  if (!kv_pool || !workspace || !logits) return fail(DEC_E_INVALID, "kv_pool, workspace and logits must be non-NULL");
  if (!aligned16(kv_pool) || !aligned16(logits)) return fail(DEC_E_INVALID, "kv_pool and logits must be 16-byte aligned");
  if (((uintptr_t)workspace & 255u) != 0) return fail(DEC_E_INVALID, "workspace must be 256-byte aligned");
  const Layout L = layout_of(*cfg);
  if (workspace_bytes < L.total)
    return fail(DEC_E_INVALID, "workspace has %zu bytes, needs %zu", workspace_bytes, L.total);

  dec_ctx* c = new dec_ctx();
  c->cfg = *cfg;
  c->stream = static_cast<hipStream_t>(hip_stream);
  c->pool = kv_pool;
  c->ws = static_cast<uint8_t*>(workspace);
  c->logits = logits;
  c->L = L;
  hipError_t e;
  if ((e = hipGetDevice(&c->device)) != hipSuccess || (e = hipStreamCreateWithFlags(&c->cap_stream, hipStreamNonBlocking)) != hipSuccess) {
    rc = hip_fail(nullptr, e, "dec_create: device / capture stream");
    delete c;
    return rc;
  }
  for (int i = 0; i < 2; ++i) {
    if ((e = hipHostMalloc(reinterpret_cast<void**>(&c->pinned[i]), L.static_bytes, hipHostMallocDefault)) != hipSuccess ||
        (e = hipEventCreateWithFlags(&c->slot_ev[i], hipEventDisableTiming)) != hipSuccess) {
      rc = hip_fail(nullptr, e, "dec_create: pinned staging");
      dec_destroy(c);
      return rc;
    }
    std::memset(c->pinned[i], 0, L.static_bytes);
  }
  // RoPE table once; the static region starts zeroed (ids 0, every row padded until
  // set) and so do the arrival counters
  if ((e = dec::launch_rope_table(ws_ptr<float2>(c, L.rope), cfg->max_seq_len, cfg->d_head, (double)cfg->rope_theta,
                                  c->stream)) != hipSuccess ||
      (e = hipMemsetAsync(c->ws, 0, L.static_bytes, c->stream)) != hipSuccess ||
      (e = hipMemsetAsync(c->ws + L.attn_cnt, 0, L.total - L.attn_cnt, c->stream)) != hipSuccess ||
      (e = hipStreamSynchronize(c->stream)) != hipSuccess) {
    rc = hip_fail(nullptr, e, "dec_create: initialising the workspace");
    dec_destroy(c);
    return rc;
  }
  c->info.flags = cfg->flags;
  *out = c;
  return DEC_OK;
}

int dec_load_weights(dec_ctx* c, const dec_weights* w) {
  if (!c || !w) return fail(DEC_E_INVALID, "ctx or weights is NULL");
  if (c->failed) return fail(DEC_E_STATE, "context has failed; destroy it");
  const dec_config& g = c->cfg;
  const bool scaled = g.weight_dtype != DEC_BF16;
  int rc;
  if ((rc = check_mat(w->embed, scaled, "embed", 0)) != DEC_OK) return rc;
  if ((rc = check_mat(w->lm_head, scaled, "lm_head", 0)) != DEC_OK) return rc;
  if (!w->final_norm) return fail(DEC_E_INVALID, "final_norm is NULL");
  if (g.n_layers > 0) {
    if (!w->attn_norm || !w->mlp_norm || !w->qkv || !w->o || !w->gate_up || !w->down)
      return fail(DEC_E_INVALID, "per-layer weight arrays must be non-NULL");
    for (int l = 0; l < g.n_layers; ++l) {
      if ((rc = check_mat(w->qkv[l], scaled, "qkv", l)) != DEC_OK || (rc = check_mat(w->o[l], scaled, "o", l)) != DEC_OK ||
          (rc = check_mat(w->gate_up[l], scaled, "gate_up", l)) != DEC_OK ||
          (rc = check_mat(w->down[l], scaled, "down", l)) != DEC_OK)
        return rc;
    }
  }
  drop_graphs(c);
  c->embed = w->embed;
  c->lm = w->lm_head;
  c->attn_norm = w->attn_norm;
  c->mlp_norm = w->mlp_norm;
  c->final_norm = w->final_norm;
  c->qkv.assign(w->qkv, w->qkv + g.n_layers);
  c->o.assign(w->o, w->o + g.n_layers);
  c->gu.assign(w->gate_up, w->gate_up + g.n_layers);
  c->down.assign(w->down, w->down + g.n_layers);
  c->loaded = true;
  c->info.graphs_captured = 0;
  return DEC_OK;
}

int dec_set_flags(dec_ctx* c, uint32_t flags) {
  if (!c) return fail(DEC_E_INVALID, "ctx is NULL");
  if (flags & ~KNOWN_FLAGS) return fail(DEC_E_INVALID, "unknown flag bits 0x%x", flags & ~KNOWN_FLAGS);
  c->cfg.flags = flags;
  c->info.flags = flags;
  return DEC_OK;
}

int dec_check(dec_ctx* c) {
  if (!c) return fail(DEC_E_INVALID, "ctx is NULL");
  if (c->failed) return fail(DEC_E_STATE, "context has failed; destroy it");
  HIPCHK(c, hipStreamSynchronize(c->stream), "hipStreamSynchronize");
  int gave_up = 0;
  HIPCHK(c, hipMemcpy(&gave_up, c->ws + c->L.attn_o_abort, sizeof gave_up, hipMemcpyDeviceToHost),
         "reading the device wait flag");
  if (gave_up) {
    c->failed = true;
    return fail(DEC_E_HIP,
                "a fused attention + O launch gave up waiting for attention's output after %d polls; "
                "its results are wrong",
                c->wait_limit);
  }
  return DEC_OK;
}

int dec_set_wait_limit(dec_ctx* c, int32_t polls) {
  if (!c) return fail(DEC_E_INVALID, "ctx is NULL");
  if (polls < 0) return fail(DEC_E_INVALID, "the wait limit must be >= 0 (got %d)", polls);
  c->wait_limit = polls;
  drop_graphs(c);
  return DEC_OK;
}

// A named range around each call that enqueues work, for profilers that record roctx
// markers (rocprofv3 --marker-trace); without one attached the calls do nothing.
struct TraceRange {
  explicit TraceRange(const char* name) { roctxRangePushA(name); }
  ~TraceRange() { roctxRangePop(); }
  TraceRange(const TraceRange&) = delete;
  TraceRange& operator=(const TraceRange&) = delete;
};

int dec_step(dec_ctx* c, const dec_step_args* a) {
  TraceRange tr("dec_step");
  if (!c || !a) return fail(DEC_E_INVALID, "ctx or args is NULL");
  int rc = check_ready(c);
  if (rc != DEC_OK) return rc;
  const dec_config& g = c->cfg;
  const int n = a->n_seqs;
  if (n < 1) return fail(DEC_E_INVALID, "n_seqs must be >= 1 (got %d)", n);
  if (n > g.max_batch) return fail(DEC_E_CAPACITY, "n_seqs %d exceeds max_batch %d", n, g.max_batch);
  if (!a->token_ids || !a->seq_lens || !a->block_tables)
    return fail(DEC_E_INVALID, "token_ids, seq_lens and block_tables must be non-NULL");
  const int bps = blocks_per_seq(g);
  for (int b = 0; b < n; ++b) {
    const int p = a->seq_lens[b];
    if ((rc = check_tokens(g, "dec_step", b, a->token_ids + b, 1, p, p, a->block_tables + (size_t)b * bps)) != DEC_OK)
      return rc;
  }
  const int Bp = LADDER[bucket_index(n)];
  rc = stage(c, n, Bp, [&](int32_t* ids, int32_t* lens, int32_t* bt) {
    std::memcpy(ids, a->token_ids, (size_t)n * 4);
    std::memcpy(lens, a->seq_lens, (size_t)n * 4);
    std::memcpy(bt, a->block_tables, (size_t)n * bps * 4);
  });
  if (rc != DEC_OK) return rc;
  if ((rc = run_plan(c, Bp, false)) != DEC_OK) return rc;
  c->last_n = n;
  c->info.rows = n;
  c->info.launches = 1;
  return DEC_OK;
}

int dec_verify(dec_ctx* c, const dec_verify_args* a) {
  TraceRange tr("dec_verify");
  if (!c || !a) return fail(DEC_E_INVALID, "ctx or args is NULL");
  int rc = check_ready(c);
  if (rc != DEC_OK) return rc;
  const dec_config& g = c->cfg;
  const int n = a->n_seqs, k = a->k;
  if (n < 1) return fail(DEC_E_INVALID, "n_seqs must be >= 1 (got %d)", n);
  if (k < 1 || k > MAX_VERIFY_K) return fail(DEC_E_INVALID, "k must be in [1, %d] (got %d)", MAX_VERIFY_K, k);
  if ((int64_t)n * k > g.max_batch)
    return fail(DEC_E_CAPACITY, "n_seqs x k = %d rows exceed max_batch %d", n * k, g.max_batch);
  if (!a->token_ids || !a->seq_lens || !a->block_tables)
    return fail(DEC_E_INVALID, "token_ids, seq_lens and block_tables must be non-NULL");
  const int bps = blocks_per_seq(g);
  for (int s = 0; s < n; ++s) {
    const int p = a->seq_lens[s];
    if ((rc = check_tokens(g, "dec_verify", s, a->token_ids + (size_t)s * k, k, p, p + k - 1,
                           a->block_tables + (size_t)s * bps)) != DEC_OK)
      return rc;
  }
  const int rows = n * k;
  const int Bp = LADDER[bucket_index(rows)];
  // row s k + j: token j of sequence s at position seq_lens[s] + j, with s's block table
  rc = stage(c, rows, Bp, [&](int32_t* ids, int32_t* lens, int32_t* bt) {
    std::memcpy(ids, a->token_ids, (size_t)rows * 4);
    for (int s = 0; s < n; ++s)
      for (int j = 0; j < k; ++j) {
        lens[s * k + j] = a->seq_lens[s] + j;
        std::memcpy(bt + (size_t)(s * k + j) * bps, a->block_tables + (size_t)s * bps, (size_t)bps * 4);
      }
  });
  if (rc != DEC_OK) return rc;
  if ((rc = run_plan(c, Bp, false)) != DEC_OK) return rc;
  c->last_n = rows;
  c->info.rows = rows;
  c->info.launches = 1;
  return DEC_OK;
}

int dec_prefill(dec_ctx* c, const dec_prefill_args* a, int32_t* logits_row) {
  TraceRange tr("dec_prefill");
  if (!c || !a || !logits_row) return fail(DEC_E_INVALID, "ctx, args or logits_row is NULL");
  int rc = check_ready(c);
  if (rc != DEC_OK) return rc;
  const dec_config& g = c->cfg;
  const int n = a->n_tokens, p0 = a->start_pos;
  if (n < 1) return fail(DEC_E_INVALID, "n_tokens must be >= 1 (got %d)", n);
  if (!a->token_ids || !a->block_table) return fail(DEC_E_INVALID, "token_ids and block_table must be non-NULL");
  if ((int64_t)p0 + n - 1 > INT32_MAX) return fail(DEC_E_CAPACITY, "start_pos + n_tokens overflows");
  if ((rc = check_tokens(g, "dec_prefill", 0, a->token_ids, n, p0, p0 + n - 1, a->block_table)) != DEC_OK) return rc;
  const int bps = blocks_per_seq(g);
  const int chunk = g.max_batch;
  int launches = 0, last_rows = 0;
  for (int t0 = 0; t0 < n; t0 += chunk) {
    const int rows = n - t0 < chunk ? n - t0 : chunk;
    const bool last = t0 + rows >= n;
    const int Bp = LADDER[bucket_index(rows)];
    rc = stage(c, rows, Bp, [&](int32_t* ids, int32_t* lens, int32_t* bt) {
      std::memcpy(ids, a->token_ids + t0, (size_t)rows * 4);
      for (int j = 0; j < rows; ++j) {
        lens[j] = p0 + t0 + j;
        std::memcpy(bt + (size_t)j * bps, a->block_table, (size_t)bps * 4);
      }
    });
    if (rc != DEC_OK) return rc;
    // only the chunk that holds the prompt's last token needs logits
    if ((rc = run_plan(c, Bp, !last)) != DEC_OK) return rc;
    ++launches;
    last_rows = rows;
  }
  c->last_n = last_rows;
  c->info.rows = n;
  c->info.launches = launches;
  *logits_row = last_rows - 1;
  return DEC_OK;
}

int dec_launch_matmul(dec_ctx* c, int which, int layer) {
  if (!c) return fail(DEC_E_INVALID, "ctx is NULL");
  if (c->failed) return fail(DEC_E_STATE, "context has failed; destroy it");
  if (!c->loaded || c->info.bucket == 0) return fail(DEC_E_STATE, "dec_launch_matmul needs a previous dec_step");
  if (which < DEC_MAT_O || which > DEC_MAT_LM_HEAD)
    return fail(DEC_E_INVALID, "which must be DEC_MAT_O, DEC_MAT_GATE_UP, DEC_MAT_DOWN or DEC_MAT_LM_HEAD");
  if (which != DEC_MAT_LM_HEAD && (layer < 0 || layer >= c->cfg.n_layers))
    return fail(DEC_E_INVALID, "layer %d outside [0, %d)", layer, c->cfg.n_layers);
  // the same kernel as in the step: a fused RMSNorm where the step fuses it
  const float* ng = nullptr;
  if (fused_norm(c->cfg, c->info.bucket)) {
    if (which == DEC_MAT_GATE_UP) ng = c->mlp_norm + (size_t)layer * c->cfg.d_model;
    if (which == DEC_MAT_LM_HEAD) ng = c->final_norm;
  }
  hipError_t e = run_matmul(c, which, which == DEC_MAT_LM_HEAD ? 0 : layer, c->info.bucket, c->stream, ng);
  if (e != hipSuccess) return hip_fail(c, e, "kernel launch");
  return DEC_OK;
}

int dec_sample_greedy(dec_ctx* c, int32_t* token_ids) {
  if (!c || !token_ids) return fail(DEC_E_INVALID, "ctx or token_ids is NULL");
  if (((uintptr_t)token_ids & 3u) != 0) return fail(DEC_E_INVALID, "token_ids is not 4-byte aligned");
  if (c->failed) return fail(DEC_E_STATE, "context has failed; destroy it");
  if (!c->loaded || c->last_n <= 0) return fail(DEC_E_STATE, "dec_sample_greedy needs a previous dec_step");
  hipError_t e = dec::launch_argmax(c->logits, c->cfg.vocab, c->cfg.vocab, c->last_n, token_ids, c->stream);
  if (e != hipSuccess) return hip_fail(c, e, "kernel launch");
  return DEC_OK;
}

int dec_sample(dec_ctx* c, const float* uniforms, float temperature, int32_t top_k, float top_p,
               int32_t* token_ids) {
  if (!c || !token_ids || !uniforms) return fail(DEC_E_INVALID, "ctx, uniforms or token_ids is NULL");
  if (((uintptr_t)token_ids & 3u) != 0 || ((uintptr_t)uniforms & 3u) != 0)
    return fail(DEC_E_INVALID, "token_ids or uniforms is not 4-byte aligned");
  if (!(temperature > 0.f) || !std::isfinite(temperature))
    return fail(DEC_E_INVALID, "temperature must be positive and finite");
  if (top_k < 1 || top_k > dec::SAMPLE_MAX_K)
    return fail(DEC_E_INVALID, "top_k must be in [1, %d] (got %d)", dec::SAMPLE_MAX_K, top_k);
  if (!(top_p > 0.f) || top_p > 1.f) return fail(DEC_E_INVALID, "top_p must be in (0, 1]");
  if (c->failed) return fail(DEC_E_STATE, "context has failed; destroy it");
  if (!c->loaded || c->last_n <= 0) return fail(DEC_E_STATE, "dec_sample needs a previous dec_step");
  hipError_t e = dec::launch_sample_topkp(c->logits, c->cfg.vocab, c->cfg.vocab, c->last_n, uniforms, temperature,
                                          top_k, top_p, token_ids, c->stream);
  if (e != hipSuccess) return hip_fail(c, e, "kernel launch");
  return DEC_OK;
}

int dec_get_info(const dec_ctx* c, int32_t* kernels_per_step, int32_t* path_flags) {
  if (!c || !kernels_per_step || !path_flags) return fail(DEC_E_INVALID, "ctx, kernels_per_step or path_flags is NULL");
  const dec_info& i = c->info;
  *kernels_per_step = i.kernels_per_step;
  int32_t f = 0;
  if (i.used_graph) f |= DEC_PATH_GRAPH;
  if (i.used_mfma) f |= DEC_PATH_MFMA_PRODUCTS;
  if (i.bucket > 0 && !(i.flags & DEC_FLAG_NO_MFMA)) f |= DEC_PATH_MFMA_ATTENTION;
  if (i.flags & DEC_FLAG_UNFUSED) f |= DEC_PATH_UNFUSED;
  else if (i.bucket > 0 && fold_norm(c->cfg, i.bucket)) f |= DEC_PATH_FOLDED_NORM;
  if (i.bucket > 0 && attn_o_rows(c->cfg, i.bucket) > 0) f |= DEC_PATH_ATTN_O;
  *path_flags = f;
  return DEC_OK;
}

int dec_get_step_info(const dec_ctx* c, dec_info* out) {
  if (!c || !out) return fail(DEC_E_INVALID, "ctx or out is NULL");
  *out = c->info;
  return DEC_OK;
}

int dec_destroy(dec_ctx* c) {
  if (!c) return DEC_OK;
  int rc = DEC_OK;
  if (c->stream || c->cap_stream) {
    hipError_t e = hipStreamSynchronize(c->stream);
    if (e != hipSuccess) rc = fail(DEC_E_HIP, "dec_destroy: %s", hipGetErrorString(e));
  }
  drop_graphs(c);
  for (int i = 0; i < 2; ++i) {
    if (c->slot_ev[i]) (void)hipEventDestroy(c->slot_ev[i]);
    if (c->pinned[i]) (void)hipHostFree(c->pinned[i]);
  }
  if (c->cap_stream) (void)hipStreamDestroy(c->cap_stream);
  delete c;
  return rc;
}

int dec_bw_probe(const void* buf, size_t bytes, int reps, void* hip_stream, double* out) {
  if (!buf || !out || reps < 1 || bytes < 16 || bytes % 16 || !aligned16(buf))
    return fail(DEC_E_INVALID, "dec_bw_probe: need a 16-byte aligned buffer, bytes a positive multiple of 16, reps >= 1");
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t e;
  double best = 0.0;
  if ((e = hipEventCreate(&e0)) != hipSuccess || (e = hipEventCreate(&e1)) != hipSuccess) goto done;
  for (int r = 0; r < reps + 1; ++r) {
    if ((e = hipEventRecord(e0, s)) != hipSuccess) goto done;
    if ((e = dec::launch_bw_probe(buf, bytes, nullptr, s)) != hipSuccess) goto done;
    if ((e = hipEventRecord(e1, s)) != hipSuccess) goto done;
    if ((e = hipEventSynchronize(e1)) != hipSuccess) goto done;
    float ms = 0.f;
    if ((e = hipEventElapsedTime(&ms, e0, e1)) != hipSuccess) goto done;
    if (r > 0 && ms > 0.f && bytes / (ms * 1e-3) > best) best = bytes / (ms * 1e-3);  // first run warms up
  }
done:
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (e != hipSuccess) return fail(DEC_E_HIP, "dec_bw_probe: %s", hipGetErrorString(e));
  *out = best;
  return DEC_OK;
}

}  // extern "C"
